"""GPU parity of prefill: per-token block selection (sda_prefill_select) and
causal block-sparse attention (sda_prefill_attention) against the oracle's
prefill_select_rows / prefill_rows.

Selection is compared bit for bit on every query whose top-k cut gap (in
float32 decision scores) is at least 1e-4, the bound on the float32 score
error; queries inside that gap could go either way and are counted, not
compared (they are few: the inputs are continuous draws).  Attention is
compared on every query within 2e-3 over the lists the GPU chose, which the
selection check validates.
"""
import dataclasses
import sys

import numpy as np
import pytest
import torch

import block_sparse_attention_pool_amd as sda
import oracle as O
import synth
from synth import inputs
from tests.parity_util import DELTA, DEV, TOL, bits

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    sda.lib()


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _f64(t):
    return O.bf16_to_f64(bits(t))


def _ktilde_gpu(K, lens):
    B, H, Tc, d = K.shape
    kt = torch.zeros((B, H, -(-Tc // 64), d), dtype=torch.bfloat16, device=DEV)
    sda.sda_update_compressed_keys(K, kt, torch.zeros(B, dtype=torch.int32, device=DEV),
                                   torch.as_tensor(lens, dtype=torch.int32, device=DEV), Tc)
    return kt


def _expected_counts(lens, pos0, nq, n_init, n_local, k):
    """n_sel of every query from its position alone."""
    out = np.zeros((len(lens), nq), dtype=np.int64)
    for b, T in enumerate(lens):
        p = pos0 + np.arange(nq)
        nb = np.where(p < T, p // 64 + 1, 0)
        lo = np.minimum(n_init, nb)
        hi = np.maximum(lo, nb - n_local)
        out[b] = lo + (nb - hi) + np.minimum(k, hi - lo)
    return out


def _check_rows(Fd, kt_rows, bi, ns, lens, pos0, n_init, n_local, k, rows):
    """Selection of the listed (b, r, g) rows against the oracle; returns the
    number of rows left out for a near-tie."""
    bi = bi.cpu().numpy()
    ns = ns.cpu().numpy()
    skipped = 0
    for (b, r, g) in rows:
        p = pos0 + r
        if p >= lens[b]:
            assert ns[b, r, g] == 0 and np.all(bi[b, r, g] == -1)
            continue
        nb = p // 64 + 1
        kt = kt_rows[(b, g)][:nb]
        want, s = O.select_row(Fd[b, r, g], kt, n_init, n_local, k)
        if O.cut_gap(s, O.candidates(nb, n_init, n_local), k) < DELTA:
            skipped += 1
            continue
        n = int(ns[b, r, g])
        assert n == len(want) and list(bi[b, r, g, :n]) == list(want), (b, r, g)
        assert np.all(bi[b, r, g, n:] == -1)
    return skipped


CASES = [
    # (B, H_kv, G, d, lens, pos0, nq, n_init, n_local, top_k)
    (2, 2, 4, 64, [1000, 600], 0, 1000, 1, 2, 4),
    (1, 2, 8, 128, [2000], 700, 900, 2, 1, 8),
    (2, 1, 4, 128, [777, 777], 0, 777, 0, 1, 3),
    (1, 1, 4, 64, [500], 0, 500, 1, 1, 50),          # top-k past every candidate: dense causal
]


@pytest.mark.parametrize("case", CASES)
def test_prefill_small_every_query(case):
    B, H, G, d, lens, pos0, nq, n_init, n_local, k = case
    _say("prefill", case)
    T_cap = max(lens)
    cfg = dataclasses.replace(synth.get_config(1), B=B, H_kv=H, H_q=H * G, d=d, T=T_cap)
    gen = torch.Generator().manual_seed(d + k)
    K = torch.randn((B, H, T_cap, d), generator=gen).to(torch.bfloat16)
    V = torch.randn((B, H, T_cap, d), generator=gen).to(torch.bfloat16)
    Q = torch.randn((B, nq, H * G, d), generator=gen).to(torch.bfloat16)
    F = inputs.to_bf16(inputs.prefill_indexer_vectors(cfg, 0, nq, pos0=pos0))
    Kg, Vg = K.to(DEV), V.to(DEV)
    seq = torch.as_tensor(lens, dtype=torch.int32, device=DEV)
    ktg = _ktilde_gpu(Kg, lens)
    bi, ns = sda.sda_prefill_select(F.to(DEV), ktg, seq, pos0, n_init, n_local, k)
    out, lse = sda.sda_prefill_attention(Q.to(DEV), Kg, Vg, seq, bi, ns, pos0)
    torch.cuda.synchronize()
    assert np.array_equal(ns.cpu().numpy()[:, :, 0], _expected_counts(lens, pos0, nq, n_init, n_local, k))
    Kd, Vd, Qd, Fd = _f64(K), _f64(V), _f64(Q), _f64(F)
    kt_rows = {(b, g): O.store_bf16(O.compressed_keys(Kd[b, g], lens[b])) for b in range(B) for g in range(H)}
    rows = [(b, r, g) for b in range(B) for r in range(nq) for g in range(H)]
    skipped = _check_rows(Fd, kt_rows, bi, ns, lens, pos0, n_init, n_local, k, rows)
    _say(f"  selection: {len(rows) - skipped} of {len(rows)} rows compared, {skipped} near-ties left out")
    assert skipped <= 0.02 * len(rows)
    bi_h, ns_h = bi.cpu().numpy(), ns.cpu().numpy()
    o, l = out.double().cpu().numpy(), lse.double().cpu().numpy()
    err = lerr = 0.0
    scale = d ** -0.5
    for b in range(B):
        for g in range(H):
            lists = [bi_h[b, r, g, :ns_h[b, r, g]] for r in range(nq)]
            live = [r for r in range(nq) if pos0 + r < lens[b]]
            want, wl = O.prefill_rows(Qd[b, live, g * G:(g + 1) * G], Kd[b, g], Vd[b, g], [lists[r] for r in live],
                                      pos0, scale)
            err = max(err, float(np.abs(o[b, live, g * G:(g + 1) * G] - want).max()))
            lerr = max(lerr, float(np.abs(l[b, live, g * G:(g + 1) * G] - wl).max()))
            dead = [r for r in range(nq) if pos0 + r >= lens[b]]
            if dead:
                assert np.all(o[b, dead, g * G:(g + 1) * G] == 0)
                assert np.all(np.isneginf(l[b, dead, g * G:(g + 1) * G]))
    _say(f"  attention: max abs err {err:.2e}, lse {lerr:.2e}")
    assert err <= TOL and lerr <= 1e-3


def test_prefill_32k_llama8b_shaped_sampled():
    # the 8B-shaped layer (B 8, H_q 32, H_kv 8, d 128) prefilling 32K tokens:
    # every query's block count from its position, list format on every row,
    # selection and attention of sampled queries against the oracle
    cfg = dataclasses.replace(synth.get_config(2), bias_frac=0.0, bias_beta=0.0)
    T, G = cfg.T, cfg.G
    _say("prefill 32K: draw")
    K, V, _ = inputs.kv_layer(cfg, 0, device=DEV)
    F = inputs.to_bf16(inputs.prefill_indexer_vectors(cfg, 0, T))
    Q = inputs.prefill_queries(cfg, 0, T, device=DEV)
    seq = torch.full((cfg.B,), T, dtype=torch.int32, device=DEV)
    ktg = _ktilde_gpu(K, [T] * cfg.B)
    sel = (cfg.n_init, cfg.n_local, cfg.top_k)
    bi, ns = sda.sda_prefill_select(F.to(DEV), ktg, seq, 0, *sel)
    out, lse = sda.sda_prefill_attention(Q, K, V, seq, bi, ns, 0)
    torch.cuda.synchronize()
    exp = _expected_counts([T] * cfg.B, 0, T, *sel)
    assert np.array_equal(ns.cpu().numpy(), np.repeat(exp[:, :, None], cfg.H_kv, axis=2))
    bi_h = bi.cpu().numpy()
    valid = bi_h >= 0
    assert np.all((np.diff(bi_h, axis=-1) > 0) | ~valid[..., 1:])
    rng = np.random.default_rng(7)
    pos = sorted(set([0, 1, 63, 64, 65, 191, 192, 1000, 4095, 4096, 16383, 32767] +
                     list(rng.integers(0, T, 12))))
    rows = [(int(rng.integers(cfg.B)), p, int(rng.integers(cfg.H_kv))) for p in pos]
    kv_rows = sorted(set((b, g) for (b, _, g) in rows))
    Kd = {(b, g): _f64(K[b, g]) for (b, g) in kv_rows}
    Vd = {(b, g): _f64(V[b, g]) for (b, g) in kv_rows}
    kt_rows = {bg: O.store_bf16(O.compressed_keys(Kd[bg], T)) for bg in kv_rows}
    Fd = {(b, r, g): _f64(F[b, r, g]) for (b, r, g) in rows}
    skipped = _check_rows(Fd, kt_rows, bi, ns, [T] * cfg.B, 0, *sel, rows)
    _say(f"prefill 32K: {len(rows) - skipped} of {len(rows)} sampled selections compared")
    assert skipped <= 2
    err = lerr = 0.0
    ns_h = ns.cpu().numpy()
    for (b, r, g) in rows:
        qd = _f64(Q[b, r, g * G:(g + 1) * G])
        o, l = O.decode_row(qd, Kd[(b, g)], Vd[(b, g)], bi_h[b, r, g, :ns_h[b, r, g]], r + 1, cfg.d ** -0.5)
        err = max(err, float(np.abs(out[b, r, g * G:(g + 1) * G].double().cpu().numpy() - o).max()))
        lerr = max(lerr, float(np.abs(lse[b, r, g * G:(g + 1) * G].double().cpu().numpy() - l).max()))
    _say(f"prefill 32K: max abs err {err:.2e}, lse {lerr:.2e}")
    assert err <= TOL and lerr <= 1e-3


def test_prefill_select_refuses_positions_past_its_register_budget():
    cfg = synth.get_config(1)
    f = torch.zeros((1, 64, 2, 64), dtype=torch.bfloat16, device=DEV)
    kt = torch.zeros((1, 2, 600, 64), dtype=torch.bfloat16, device=DEV)
    seq = torch.full((1,), 600 * 64, dtype=torch.int32, device=DEV)
    with pytest.raises(sda.SdaError, match="registers"):
        sda.sda_prefill_select(f, kt, seq, 32768 - 63, 1, 2, 8)
    assert cfg.d == 64


ATT_CASES = [
    # (B, H_kv, G, d, lens, pos0, nq, n_sel_max): the row-tiled engine at every
    # wave count (G = 1: 2 waves, 2: 4, 3: 8 with idle padding rows, 4, 16 and
    # 32: 8), ragged lengths, a chunk offset, lists holding blocks past the
    # query's position (masked by causality) and empty lists
    (2, 2, 1, 64, [300, 700], 0, 700, 7),
    (1, 1, 2, 128, [400], 129, 200, 9),
    (2, 2, 3, 64, [520, 260], 0, 520, 6),
    (1, 2, 4, 128, [3000], 0, 3000, 12),
    (1, 1, 16, 128, [450], 10, 300, 8),
    (1, 1, 32, 64, [333], 0, 333, 5),
]


@pytest.mark.parametrize("case", ATT_CASES)
def test_prefill_attention_on_drawn_lists(case):
    B, H, G, d, lens, pos0, nq, nsm = case
    _say("prefill attention", case)
    T_cap = max(lens)
    gen = torch.Generator().manual_seed(1000 + G * 7 + d)
    K = torch.randn((B, H, T_cap, d), generator=gen).to(torch.bfloat16)
    V = torch.randn((B, H, T_cap, d), generator=gen).to(torch.bfloat16)
    Q = torch.randn((B, nq, H * G, d), generator=gen).to(torch.bfloat16)
    rng = np.random.default_rng(G * 100 + d)
    bi = np.full((B, nq, H, nsm), -1, dtype=np.int32)
    ns = np.zeros((B, nq, H), dtype=np.int32)
    nb_all = -(-T_cap // 64)
    for b in range(B):
        for r in range(nq):
            p = pos0 + r
            for g in range(H):
                if rng.random() < 0.03:
                    continue                                   # an empty list
                top = min(nb_all, p // 64 + 2)                 # may reach one block past the position
                n = int(rng.integers(1, min(nsm, top) + 1))
                blocks = np.sort(rng.choice(top, size=n, replace=False))
                bi[b, r, g, :n] = blocks
                ns[b, r, g] = n
    seq = torch.as_tensor(lens, dtype=torch.int32, device=DEV)
    out, lse = sda.sda_prefill_attention(Q.to(DEV), K.to(DEV), V.to(DEV), seq, torch.as_tensor(bi, device=DEV),
                                         torch.as_tensor(ns, device=DEV), pos0)
    torch.cuda.synchronize()
    Kd, Vd, Qd = _f64(K), _f64(V), _f64(Q)
    o, l = out.double().cpu().numpy(), lse.double().cpu().numpy()
    err = lerr = 0.0
    for b in range(B):
        for g in range(H):
            # a query sees tokens below min(its position + 1, the cached length)
            for r in range(nq):
                T = min(pos0 + r + 1, lens[b])
                blocks = bi[b, r, g, :ns[b, r, g]]
                qh = Qd[b, r, g * G:(g + 1) * G]
                toks = O.block_tokens(blocks, T) if len(blocks) else np.zeros(0, dtype=np.int64)
                if len(toks) == 0:
                    assert np.all(o[b, r, g * G:(g + 1) * G] == 0), (b, r, g)
                    assert np.all(np.isneginf(l[b, r, g * G:(g + 1) * G])), (b, r, g)
                    continue
                want, wl = O.decode_row(qh, Kd[b, g], Vd[b, g], blocks, T, d ** -0.5)
                err = max(err, float(np.abs(o[b, r, g * G:(g + 1) * G] - want).max()))
                lerr = max(lerr, float(np.abs(l[b, r, g * G:(g + 1) * G] - wl).max()))
    _say(f"  max abs err {err:.2e}, lse {lerr:.2e}")
    assert err <= TOL and lerr <= 1e-3
