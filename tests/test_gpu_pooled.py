"""GPU parity of the overlapping compression and the max-pooled selection
(InfLLM-V2's inference setting, kernel 32 / stride 16, and other shapes)
against the CPU oracle, through the C ABI.

Compressed keys must match the oracle bit for bit (bulk and token by token);
block sets bit for bit on rows whose pooled top-k cut has a gap of at least
1e-4 (float32 decision scores); pooled block scores within 1e-5.
"""
import dataclasses
import os
import sys

import numpy as np
import pytest
import torch

import block_sparse_attention_pool_amd as sda
import oracle as O
import synth
from synth import inputs
from tests.parity_util import DELTA, DEV, bits, f64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    sda.lib()          # raises if libsda.so is missing: there is no fallback path


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _strided_gpu(K, T, window, stride, NC_cap=None, lens=None):
    B, H, Tc, d = K.shape
    NC_cap = NC_cap or -(-Tc // stride)
    kt = torch.zeros((B, H, NC_cap, d), dtype=torch.bfloat16, device=K.device)
    lo = torch.zeros(B, dtype=torch.int32, device=K.device)
    hi = torch.as_tensor(lens if lens is not None else [T] * B, dtype=torch.int32, device=K.device)
    sda.sda_update_compressed_keys_strided(K, kt, lo, hi, int(hi.max().item()), window, stride)
    return kt


def _oracle_strided(K, b, g, T, window, stride):
    return O.store_bf16(O.compressed_keys_strided(f64(K[b, g, :T]), T, window, stride))


def _tie_free_pooled(cfg, ktc, lens, window, stride, rows, delta=DELTA, max_iter=200):
    """bf16 F whose listed rows have a pooled top-k cut gap >= delta."""
    attempts = np.zeros((cfg.B, cfg.NQ, cfg.H_kv), dtype=np.int64)
    for _ in range(max_iter):
        F = inputs.to_bf16(inputs.indexer_vectors(cfg, 0, attempts))
        Fd = O.bf16_to_f64(bits(F))
        bad = []
        for (b, q, g) in rows:
            T = lens[b]
            _, s = O.select_row_pooled(Fd[b, q, g], ktc[(b, g)], T, window, stride, cfg.n_init, cfg.n_local,
                                       cfg.top_k)
            cand = O.candidates(O.num_blocks(T), cfg.n_init, cfg.n_local)
            if O.cut_gap(s, cand, cfg.top_k) < delta:
                bad.append((b, q, g))
        if not bad:
            return F
        for r in bad:
            attempts[r] += 1
    raise RuntimeError("could not draw tie-free indexer vectors")


def _check_rows(bi, ns, want, rows):
    bi, ns = bi.cpu().numpy(), ns.cpu().numpy()
    for r in rows:
        n = int(ns[r])
        assert n == len(want[r]), (r, n, want[r])
        assert np.array_equal(bi[r][:n], want[r]), (r, bi[r][:n], want[r])
        assert np.all(bi[r][n:] == -1)


# ---------------------------------------------------------------------------
# compressed keys
# ---------------------------------------------------------------------------

KEY_CASES = [
    # (B, H_kv, d, lengths, window, stride)
    (1, 2, 64, [4096], 32, 16),
    (1, 2, 64, [4096], 64, 32),
    (1, 2, 64, [4096], 48, 16),
    (1, 2, 64, [4096], 16, 8),
    (2, 2, 128, [3001, 130], 32, 16),
    (2, 2, 128, [1, 77], 64, 8),
]


@pytest.mark.parametrize("case", KEY_CASES)
def test_strided_keys_bulk_and_incremental(case):
    B, H, d, lens, window, stride = case
    _say("strided keys", case)
    cfg = dataclasses.replace(synth.get_config(1), B=B, H_kv=H, H_q=H * 4, d=d, T=max(lens))
    K, _, _ = inputs.kv_layer(cfg, 0, device="cpu")
    Kg = K.to(DEV)
    kt = _strided_gpu(Kg, None, window, stride, lens=lens)
    for b in range(B):
        for g in range(H):
            want = _oracle_strided(K, b, g, lens[b], window, stride)
            got = kt[b, g, :want.shape[0]].double().cpu().numpy()
            assert np.array_equal(got, want), (b, g)
    # token by token (and in uneven runs) from a shorter bulk build
    T0 = [max(1, t - 70) for t in lens]
    kt2 = _strided_gpu(Kg, None, window, stride, lens=T0)
    cur = list(T0)
    for step in [1, 1, 3, 17, 1, 64, 200]:
        lo = torch.as_tensor(cur, dtype=torch.int32, device=DEV)
        nxt = [min(c + step, t) for c, t in zip(cur, lens)]
        hi = torch.as_tensor(nxt, dtype=torch.int32, device=DEV)
        sda.sda_update_compressed_keys_strided(Kg, kt2, lo, hi, step, window, stride)
        cur = nxt
    assert cur == list(lens)
    for b in range(B):
        ne = O.num_entries(lens[b], stride)
        assert torch.equal(kt2[b, :, :ne], kt[b, :, :ne]), b


# ---------------------------------------------------------------------------
# pooled selection
# ---------------------------------------------------------------------------

SELECT_CASES = [
    # (B, H_kv, d, lengths, window, stride, n_init, n_local, top_k)
    (1, 2, 64, [4096], 32, 16, 1, 2, 8),
    (3, 2, 64, [4096, 3001, 130], 32, 16, 1, 2, 8),
    (2, 4, 128, [32768, 20000], 32, 16, 1, 2, 16),
    (2, 2, 128, [8192, 5000], 64, 32, 2, 1, 5),
    (1, 2, 64, [4096], 16, 8, 0, 0, 12),
    (3, 2, 64, [20, 1, 70], 32, 16, 1, 2, 8),      # fewer blocks than the budget: every block
    (1, 2, 64, [16384], 32, 16, 1, 2, 80),         # top_k past the in-launch selection's 64
]


@pytest.mark.parametrize("case", SELECT_CASES)
def test_pooled_select_matches_oracle(case):
    # top_k <= 64: selection inside the scoring launch; top_k = 80: the
    # separate selection launch
    B, H, d, lens, window, stride, n_init, n_local, top_k = case
    _say("pooled select", case, "in-launch selection" if top_k <= 64 else "two launches")
    cfg = dataclasses.replace(synth.get_config(2), B=B, H_kv=H, H_q=H * 4, d=d, T=max(lens), n_init=n_init,
                              n_local=n_local, top_k=top_k, bias_frac=0.0, bias_beta=0.0)
    K, _, _ = inputs.kv_layer(cfg, 0, device="cpu")
    Kg = K.to(DEV)
    kt = _strided_gpu(Kg, None, window, stride, lens=lens)
    ktc = {(b, g): _oracle_strided(K, b, g, lens[b], window, stride) for b in range(B) for g in range(H)}
    rows = [(b, 0, g) for b in range(B) for g in range(H)]
    F = _tie_free_pooled(cfg, ktc, lens, window, stride, rows)
    Fd = O.bf16_to_f64(bits(F))
    seq = torch.as_tensor(lens, dtype=torch.int32, device=DEV)
    NB_cap = -(-kt.shape[2] * stride // 64)
    scores = torch.full((B, 1, H, NB_cap), float("nan"), dtype=torch.float32, device=DEV)
    bi, ns = sda.sda_score_select_pooled(F.to(DEV), kt, seq, window, stride, n_init, n_local, top_k,
                                         scores=scores)
    torch.cuda.synchronize()
    want, worst = {}, 0.0
    for (b, q, g) in rows:
        sel, s = O.select_row_pooled(Fd[b, q, g], ktc[(b, g)], lens[b], window, stride, n_init, n_local, top_k)
        want[(b, q, g)] = sel
        got = scores[b, q, g, :s.size].double().cpu().numpy()
        worst = max(worst, float(np.abs(got - s).max()))
    _say("  max |pooled score - oracle|", worst)
    assert worst < 1e-5
    _check_rows(bi, ns, want, rows)


def test_pooled_64_64_equals_plain_select():
    cfg = synth.get_config(1)
    K, _, _ = inputs.kv_layer(cfg, 0, device="cpu")
    Kg = K.to(DEV)
    kt_plain = torch.zeros((cfg.B, cfg.H_kv, cfg.NB, cfg.d), dtype=torch.bfloat16, device=DEV)
    z = torch.zeros(cfg.B, dtype=torch.int32, device=DEV)
    seq = torch.full((cfg.B,), cfg.T, dtype=torch.int32, device=DEV)
    sda.sda_update_compressed_keys(Kg, kt_plain, z, seq, cfg.T)
    kt = _strided_gpu(Kg, cfg.T, 64, 64)
    assert torch.equal(kt, kt_plain)
    F = inputs.to_bf16(inputs.indexer_vectors(cfg, 0)).to(DEV)
    s1 = torch.empty((cfg.B, 1, cfg.H_kv, cfg.NB), dtype=torch.float32, device=DEV)
    s2 = torch.empty_like(s1)
    a = sda.sda_score_select(F, kt_plain, seq, cfg.n_init, cfg.n_local, cfg.top_k, scores=s1)
    b = sda.sda_score_select_pooled(F, kt, seq, 64, 64, cfg.n_init, cfg.n_local, cfg.top_k, scores=s2)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    assert torch.equal(s1, s2)


@pytest.mark.parametrize("spike,top_k,want", [
    (10 * 64 + 60, 1, [0, 10, 62, 63]),         # windows 42 and 43 hold it: blocks 10 and 11 tie, 10 wins
    (10 * 64 + 60, 2, [0, 10, 11, 62, 63]),
    (10 * 64 + 5, 1, [0, 9, 62, 63]),           # window 39 reaches back into block 9: 9 and 10 tie
    (10 * 64 + 20, 1, [0, 10, 62, 63]),         # only windows inside block 10 hold it
])
def test_pooled_spike_and_shared_window_tie(spike, top_k, want):
    # keys are zero except one token along f: the blocks that overlap a window
    # holding it score f.k/32, every other block 0; equal scores from one
    # shared window go to the lower block index
    T, d = 4096, 64
    K = torch.zeros((1, 1, T, d), dtype=torch.bfloat16)
    f = torch.zeros((1, 1, 1, d), dtype=torch.bfloat16)
    f[0, 0, 0, :8] = 0.5
    K[0, 0, spike, :8] = 2.0
    Kg = K.to(DEV)
    kt = _strided_gpu(Kg, T, 32, 16)
    seq = torch.full((1,), T, dtype=torch.int32, device=DEV)
    bi, ns = sda.sda_score_select_pooled(f.to(DEV), kt, seq, 32, 16, 1, 2, top_k)
    got = bi[0, 0, 0, :ns[0, 0, 0].item()].cpu().tolist()
    assert got == want
    ktc = O.store_bf16(O.compressed_keys_strided(f64(K[0, 0]), T, 32, 16))
    assert list(O.select_row_pooled(f64(f[0, 0, 0]), ktc, T, 32, 16, 1, 2, top_k)[0]) == want


def test_c3_pooled_128k_sampled_rows():
    # the 128K, 8-sequence layer with InfLLM-V2's inference compression
    # (8192 compressed keys per row): every row's selection is checked for
    # the top-k certificate on the GPU's own pooled scores, sampled rows
    # against the oracle bit for bit (keys and blocks)
    cfg = synth.get_config(3)
    window, stride = 32, 16
    _say("c3 pooled: draw K on the GPU")
    K, V, _ = inputs.kv_layer(cfg, 1, device=DEV)
    del V
    kt = _strided_gpu(K, cfg.T, window, stride)
    sample = [(0, 0), (3, 5), (7, 7)]
    ktc = {}
    for (b, g) in sample:
        ktc[(b, g)] = _oracle_strided(K[b:b + 1, g:g + 1].cpu(), 0, 0, cfg.T, window, stride)
        assert np.array_equal(kt[b, g].double().cpu().numpy(), ktc[(b, g)]), (b, g)
    _say("c3 pooled: keys of the sampled rows match")
    rows = [(b, 0, g) for (b, g) in sample]
    F = _tie_free_pooled(cfg, ktc, [cfg.T] * cfg.B, window, stride, rows)
    Fd = O.bf16_to_f64(bits(F))
    seq = torch.full((cfg.B,), cfg.T, dtype=torch.int32, device=DEV)
    scores = torch.empty((cfg.B, 1, cfg.H_kv, cfg.NB), dtype=torch.float32, device=DEV)
    bi, ns = sda.sda_score_select_pooled(F.to(DEV), kt, seq, window, stride, cfg.n_init, cfg.n_local,
                                         cfg.top_k, scores=scores)
    torch.cuda.synchronize()
    want = {r: O.select_row_pooled(Fd[r], ktc[(r[0], r[2])], cfg.T, window, stride, cfg.n_init, cfg.n_local,
                                   cfg.top_k)[0] for r in rows}
    _check_rows(bi, ns, want, rows)
    # certificate on every row: chosen candidates score >= every other candidate
    sc = scores.cpu().numpy()
    bi_h, ns_h = bi.cpu().numpy(), ns.cpu().numpy()
    cand = O.candidates(cfg.NB, cfg.n_init, cfg.n_local)
    for b in range(cfg.B):
        for g in range(cfg.H_kv):
            chosen = set(int(j) for j in bi_h[b, 0, g, :ns_h[b, 0, g]])
            assert len(chosen) == cfg.n_sel
            top = [j for j in cand if j in chosen]
            rest = [j for j in cand if j not in chosen]
            assert len(top) == cfg.top_k
            assert sc[b, 0, g, top].min() >= sc[b, 0, g, rest].max()


# ---------------------------------------------------------------------------
# InfLLM-V2's G-head selector on overlapping compressed keys
# ---------------------------------------------------------------------------

MH_CASES = [
    # (B, H_kv, G, d, lengths, window, stride, n_init, n_local, top_k)
    (2, 2, 8, 128, [16384, 9000], 32, 16, 1, 2, 16),
    (1, 2, 4, 64, [4096], 32, 16, 1, 2, 8),
    (2, 1, 8, 128, [20, 4000], 64, 32, 0, 1, 5),
    (1, 2, 8, 128, [16384], 32, 16, 1, 2, 80),        # top_k past the in-launch selection
]


@pytest.mark.parametrize("case", MH_CASES)
def test_multihead_pooled_select_matches_oracle(case):
    import math
    B, H, G, d, lens, window, stride, n_init, n_local, k = case
    _say("multihead pooled", case)
    T_cap = max(lens)
    cfg = dataclasses.replace(synth.get_config(2), B=B, H_kv=H, H_q=H * G, d=d, T=T_cap, n_init=n_init,
                              n_local=n_local, top_k=k, bias_frac=0.0, bias_beta=0.0)
    K, _, _ = inputs.kv_layer(cfg, 0, device="cpu")
    kt = _strided_gpu(K.to(DEV), None, window, stride, lens=lens)
    ktc = {(b, g): _oracle_strided(K, b, g, lens[b], window, stride) for b in range(B) for g in range(H)}
    tau = math.sqrt(d)
    rng = np.random.default_rng(len(lens) * 7 + k)
    Qf = rng.standard_normal((B, 1, H * G, d)).astype(np.float32)
    for _ in range(100):          # re-draw the heads of rows whose top-k cut is a near-tie
        Q = inputs.to_bf16(Qf)
        Qd = O.bf16_to_f64(bits(Q))
        bad = []
        for b in range(B):
            for g in range(H):
                _, s = O.select_row_multihead_pooled(Qd[b, 0, g * G:(g + 1) * G], ktc[(b, g)], lens[b], window,
                                                     stride, n_init, n_local, k, tau)
                cand = O.candidates(O.num_blocks(lens[b]), n_init, n_local)
                if k < cand.size and O.cut_gap(s, cand, k) < 1e-4 * abs(np.sort(s[cand])[::-1][k - 1]):
                    bad.append((b, g))
        if not bad:
            break
        for (b, g) in bad:
            Qf[b, 0, g * G:(g + 1) * G] = rng.standard_normal((G, d))
    seq = torch.as_tensor(lens, dtype=torch.int32, device=DEV)
    NB_cap = -(-kt.shape[2] * stride // 64)
    scores = torch.full((B, 1, H, NB_cap), float("nan"), dtype=torch.float32, device=DEV)
    bi, ns = sda.sda_score_select_multihead_pooled(Q.to(DEV), kt, seq, window, stride, n_init, n_local, k, tau,
                                                   scores=scores)
    torch.cuda.synchronize()
    rows, want, worst, skipped = [], {}, 0.0, 0
    for b in range(B):
        for g in range(H):
            T = lens[b]
            sel, s = O.select_row_multihead_pooled(Qd[b, 0, g * G:(g + 1) * G], ktc[(b, g)], T, window, stride,
                                                   n_init, n_local, k, tau)
            got = scores[b, 0, g, :s.size].double().cpu().numpy()
            worst = max(worst, float(np.abs(got - s).max() / max(1e-30, np.abs(s).max())))
            cand = O.candidates(O.num_blocks(T), n_init, n_local)
            if k < cand.size:
                top = np.sort(s[cand])[::-1][k - 1]
                if O.cut_gap(s, cand, k) < 1e-4 * abs(top):
                    skipped += 1
                    continue
            rows.append((b, 0, g))
            want[(b, 0, g)] = sel
    _say(f"  max relative |block score - oracle| {worst:.2e}; {len(rows)} rows compared, {skipped} near-ties")
    assert worst < 1e-4
    assert skipped == 0
    _check_rows(bi, ns, want, rows)
