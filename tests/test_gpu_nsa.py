"""GPU parity of the NSA three-branch output (sda_nsa_decode) against the CPU
oracle, through the C ABI: compressed branch over the compressed keys and
values, selection branch over the listed blocks (plain or grouped, modes A
and B), window branch over the last w tokens, gated sum; max-abs 2e-3 on the
output, 1e-3 on each branch's log-sum-exp.
"""
import dataclasses
import math
import sys

import numpy as np
import pytest
import torch

import block_sparse_attention_pool_amd as sda
import oracle as O
import synth
from synth import inputs
from tests.parity_util import DEV, TOL, bits, f64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    sda.lib()          # raises if libsda.so is missing: there is no fallback path


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _compressed(X, lens, window, stride):
    """Compressed cache of X (keys or values) on the GPU, [B, H, ceil(T_cap/stride), d]."""
    B, H, Tc, d = X.shape
    out = torch.zeros((B, H, -(-Tc // stride), d), dtype=torch.bfloat16, device=DEV)
    lo = torch.zeros(B, dtype=torch.int32, device=DEV)
    hi = torch.as_tensor(lens, dtype=torch.int32, device=DEV)
    if window == stride == 64:
        sda.sda_update_compressed_keys(X, out, lo, hi, max(lens))
    else:
        sda.sda_update_compressed_keys_strided(X, out, lo, hi, max(lens), window, stride)
    return out


def _lists(rng, B, NQ, H, lens, n_sel_max, short_rows=True):
    bi = np.full((B, NQ, H, n_sel_max), -1, dtype=np.int32)
    ns = np.zeros((B, NQ, H), dtype=np.int32)
    for b in range(B):
        nb = -(-lens[b] // 64)
        if nb == 0:
            continue                                     # an empty sequence lists nothing
        for q in range(NQ):
            for g in range(H):
                n = min(n_sel_max, nb)
                if short_rows and (q + g) % 3 == 2:
                    n = max(1, n - 2)                    # a shorter list, -1 padded
                lst = np.sort(rng.choice(nb, size=n, replace=False))
                bi[b, q, g, :n] = lst
                ns[b, q, g] = n
    return bi, ns


def _run_case(B, NQ, H_q, H, d, lens, n_sel_max, cw, cs, window, C, mode, seed):
    cfg = dataclasses.replace(synth.get_config(2), B=B, H_q=H_q, H_kv=H, d=d, T=max(lens), NQ=NQ,
                              bias_frac=0.0, bias_beta=0.0)
    K, V, _ = inputs.kv_layer(cfg, 0, device="cpu")
    Kg, Vg = K.to(DEV), V.to(DEV)
    kc, vc = _compressed(Kg, lens, cw, cs), _compressed(Vg, lens, cw, cs)
    rng = np.random.default_rng(seed)
    Q = inputs.to_bf16(rng.standard_normal((B, NQ, H_q, d)).astype(np.float32))
    gates = torch.from_numpy(rng.uniform(0.0, 1.0, (B, NQ, H_q, 3)).astype(np.float32))
    bi, ns = _lists(rng, B, NQ, H, lens, n_sel_max)
    seq = torch.as_tensor(lens, dtype=torch.int32, device=DEV)
    out, lse, uc = sda.sda_nsa_decode(Q.to(DEV), Kg, Vg, kc, vc, seq, torch.from_numpy(bi).to(DEV),
                                      torch.from_numpy(ns).to(DEV), gates.to(DEV), cs, window, group_C=C, mode=mode)
    torch.cuda.synchronize()
    G = H_q // H
    scale = 1.0 / math.sqrt(d)
    Qd = O.bf16_to_f64(bits(Q))
    gd = gates.double().numpy()
    out_h, lse_h = out.double().cpu().numpy(), lse.double().cpu().numpy()
    err, lerr = 0.0, 0.0
    for b in range(B):
        T = lens[b]
        n_cmp = O.num_entries(T, cs)
        for g in range(H):
            kk, vv = f64(K[b, g, :T]), f64(V[b, g, :T])
            kcd = O.store_bf16(O.compressed_keys_strided(kk, T, cw, cs))
            vcd = O.store_bf16(O.compressed_keys_strided(vv, T, cw, cs))
            assert np.array_equal(kc[b, g, :n_cmp].double().cpu().numpy(), kcd)
            assert np.array_equal(vc[b, g, :n_cmp].double().cpu().numpy(), vcd)
            for q0 in range(0, NQ, C):
                qs = list(range(q0, min(q0 + C, NQ)))
                lists = [bi[b, q, g, :ns[b, q, g]] for q in qs]
                active = lists if mode == O.MODE_EXACT else [lists[0]] * len(qs)
                for c, q in enumerate(qs):
                    hs = slice(g * G, (g + 1) * G)
                    o, _, l = O.nsa_row(Qd[b, q, hs], kk, vv, kcd, vcd, active[c], T, n_cmp, window, gd[b, q, hs],
                                        scale)
                    err = max(err, float(np.abs(out_h[b, q, hs] - o).max()))
                    fin = np.isfinite(l.T)
                    assert np.array_equal(np.isfinite(lse_h[b, q, hs]), fin)
                    if fin.any():
                        lerr = max(lerr, float(np.abs(lse_h[b, q, hs][fin] - l.T[fin]).max()))
                if C > 1 and uc is not None:
                    want_u = len(O.union_blocks(lists if mode == O.MODE_EXACT else [lists[0]]))
                    assert int(uc[b, q0 // C, g].item()) == want_u
    _say("  max |out - oracle|", err, " max |lse - oracle|", lerr)
    assert err <= TOL
    assert lerr <= 1e-3


CASES = [
    # (B, NQ, H_q, H_kv, d, lengths, n_sel_max, cmp window, cmp stride, window, C, mode)
    (1, 1, 8, 2, 64, [4096], 11, 64, 64, 512, 1, 0),
    (2, 1, 8, 2, 64, [4096, 3001], 11, 32, 16, 100, 1, 0),
    (2, 1, 16, 2, 128, [8192, 777], 19, 64, 64, 0, 1, 0),
    (1, 1, 8, 2, 64, [300], 5, 32, 16, 5000, 1, 0),            # window wider than the sequence
    (2, 8, 16, 4, 128, [8192, 6000], 16, 64, 64, 256, 4, 0),    # grouped, exact merge
    (2, 8, 16, 4, 128, [8192, 6000], 16, 32, 16, 200, 4, 1),    # grouped, shared representative
    (1, 6, 8, 2, 64, [2048], 8, 64, 64, 130, 4, 0),             # last group smaller
    (3, 2, 8, 2, 64, [20, 1, 70], 2, 32, 16, 16, 2, 0),         # shorter than a block: one partial block
    # exact mode with two or more queries per (batch, KV head) runs on row tiles that hold every group
    (2, 8, 32, 4, 128, [8192, 6000], 16, 64, 64, 256, 8, 0),    # 8 queries x G = 8: 64 rows in one group
    (1, 4, 8, 2, 64, [4096], 11, 32, 16, 300, 1, 0),            # one query per group, four share a tile
    (2, 6, 8, 2, 64, [4096, 3001], 11, 32, 16, 100, 2, 0),      # unaligned window, 4x more compressed entries
    (1, 32, 32, 8, 64, [2048], 8, 64, 64, 130, 4, 0),           # 32 queries x G = 4: a 128-row tile
    (1, 40, 16, 4, 64, [3000], 9, 32, 16, 64, 4, 0),            # two tiles per KV head, the second of 8 queries
    (1, 4, 8, 2, 128, [5000], 8, 64, 64, 0, 2, 0),              # no window
    (2, 4, 8, 2, 64, [0, 100], 4, 32, 16, 50, 2, 0),            # an empty sequence: every branch empty
    (2, 8, 32, 4, 128, [8192, 6000], 16, 64, 64, 256, 8, 1),    # shared mode, 64 rows per group
    (1, 12, 16, 4, 64, [3000], 9, 32, 16, 100, 3, 1),           # shared mode, four groups of 3 in a tile
]


@pytest.mark.parametrize("i", range(len(CASES)))
def test_nsa_matches_oracle(i):
    _say("nsa", CASES[i])
    _run_case(*CASES[i], seed=100 + i)


def test_nsa_gate_reductions_match_existing_calls():
    # gates (0, 1, 0) give the selection branch alone: sda_grouped_decode's
    # output; gates (0, 0, 1) with a window of every token give dense
    # attention (torch SDPA on the CPU); gates (1, 0, 0) with kernel =
    # stride = 64 give decode over the compressed cache as if it were a KV cache
    B, NQ, H_q, H, d, T = 1, 4, 8, 2, 64, 4096
    cfg = dataclasses.replace(synth.get_config(1), NQ=NQ)
    K, V, _ = inputs.kv_layer(cfg, 0, device="cpu")
    Kg, Vg = K.to(DEV), V.to(DEV)
    kc, vc = _compressed(Kg, [T], 64, 64), _compressed(Vg, [T], 64, 64)
    rng = np.random.default_rng(7)
    Q = inputs.to_bf16(rng.standard_normal((B, NQ, H_q, d)).astype(np.float32)).to(DEV)
    bi, ns = _lists(rng, B, NQ, H, [T], 11, short_rows=False)
    bi, ns = torch.from_numpy(bi).to(DEV), torch.from_numpy(ns).to(DEV)
    seq = torch.full((B,), T, dtype=torch.int32, device=DEV)

    def gates(gc, gs, gw):
        return torch.tensor([gc, gs, gw], dtype=torch.float32, device=DEV).expand(B, NQ, H_q, 3).contiguous()
    o_s, _, _ = sda.sda_nsa_decode(Q, Kg, Vg, kc, vc, seq, bi, ns, gates(0, 1, 0), 64, 256, group_C=2)
    ref, _, _ = sda.sda_grouped_decode(Q, Kg, Vg, seq, bi, ns, 2)
    assert (o_s - ref).abs().max().item() < 1e-5
    o_w, _, _ = sda.sda_nsa_decode(Q, Kg, Vg, kc, vc, seq, bi, ns, gates(0, 0, 1), 64, T + 64, group_C=2)
    for g in range(H):
        for q in range(NQ):
            qq = Q[0, q, g * 4:(g + 1) * 4].double().cpu()[None]
            dense = torch.nn.functional.scaled_dot_product_attention(qq, K[0, g].double()[None, None],
                                                                     V[0, g].double()[None, None])[0]
            assert (o_w[0, q, g * 4:(g + 1) * 4].double().cpu() - dense).abs().max().item() <= TOL
    o_c, _, _ = sda.sda_nsa_decode(Q, Kg, Vg, kc, vc, seq, bi, ns, gates(1, 0, 0), 64, 256, group_C=2)
    nb = T // 64
    all_blocks = torch.arange(1, dtype=torch.int32, device=DEV).expand(B, NQ, H, 1).contiguous()
    ones = torch.ones((B, NQ, H), dtype=torch.int32, device=DEV)
    ref_c, _ = sda.sda_sparse_decode(Q, kc, vc, torch.full((B,), nb, dtype=torch.int32, device=DEV), all_blocks, ones)
    assert (o_c - ref_c).abs().max().item() < 1e-5


def test_nsa_c4_full_size_sampled_rows():
    # the verification workload as the bench runs it (T = 64K, B 4, 16 draft
    # queries in groups of 4, H_q 32, H_kv 8, a 512-token window, 64/64
    # compressed keys and values, exact merge): every output of three
    # sampled (batch, group, KV head) tasks against the oracle
    cfg = synth.get_config(4)
    C, n, window = cfg.group_C, cfg.top_k, 512
    _say("nsa c4: draw K/V on the GPU")
    K, V, _ = inputs.kv_layer(cfg, 0, device=DEV)
    seq = torch.full((cfg.B,), cfg.T, dtype=torch.int32, device=DEV)
    zero = torch.zeros(cfg.B, dtype=torch.int32, device=DEV)
    kc = torch.zeros((cfg.B, cfg.H_kv, cfg.NB, cfg.d), dtype=torch.bfloat16, device=DEV)
    vc = torch.zeros_like(kc)
    sda.sda_update_compressed_keys(K, kc, zero, seq, cfg.T)
    sda.sda_update_compressed_keys(V, vc, zero, seq, cfg.T)
    rng = np.random.default_rng(44)
    Q = inputs.to_bf16(inputs.attention_queries(cfg, 0, sigma=0.5))
    gates = torch.from_numpy(rng.uniform(0.0, 1.0, (cfg.B, cfg.NQ, cfg.H_q, 3)).astype(np.float32))
    bi, ns = _lists(rng, cfg.B, cfg.NQ, cfg.H_kv, [cfg.T] * cfg.B, n, short_rows=False)
    out, lse, uc = sda.sda_nsa_decode(Q.to(DEV), K, V, kc, vc, seq, torch.from_numpy(bi).to(DEV),
                                      torch.from_numpy(ns).to(DEV), gates.to(DEV), 64, window, group_C=C)
    torch.cuda.synchronize()
    G = cfg.G
    Qd = O.bf16_to_f64(bits(Q))
    gd = gates.double().numpy()
    out_h = out.double().cpu().numpy()
    err = 0.0
    for (b, grp, g) in [(0, 0, 0), (1, 2, 5), (3, 3, 7)]:
        kk, vv = f64(K[b, g].cpu()), f64(V[b, g].cpu())
        kcd = O.store_bf16(O.compressed_keys(kk, cfg.T))
        vcd = O.store_bf16(O.compressed_keys(vv, cfg.T))
        assert np.array_equal(kc[b, g].double().cpu().numpy(), kcd)
        qs = list(range(grp * C, grp * C + C))
        lists = [bi[b, q, g, :ns[b, q, g]] for q in qs]
        assert int(uc[b, grp, g].item()) == len(O.union_blocks(lists))
        hs = slice(g * G, (g + 1) * G)
        for c, q in enumerate(qs):
            o, _, _ = O.nsa_row(Qd[b, q, hs], kk, vv, kcd, vcd, lists[c], cfg.T, cfg.NB, window, gd[b, q, hs],
                                1.0 / math.sqrt(cfg.d))
            err = max(err, float(np.abs(out_h[b, q, hs] - o).max()))
    _say("nsa c4: max |out - oracle|", err)
    assert err <= TOL


def test_nsa_tiles_repeat_bit_identically():
    # the row-tiled three-branch launch on one workspace: a call, a call of
    # another shape (its split counters must come back to zero), then the
    # first call again, whose output and lse must repeat bit for bit
    B, H_q, H, d, lens = 2, 16, 4, 128, [8192, 6000]
    cfg = dataclasses.replace(synth.get_config(2), B=B, H_q=H_q, H_kv=H, d=d, T=max(lens), NQ=8,
                              bias_frac=0.0, bias_beta=0.0)
    K, V, _ = inputs.kv_layer(cfg, 0, device=DEV)
    kc, vc = _compressed(K, lens, 64, 64), _compressed(V, lens, 64, 64)
    rng = np.random.default_rng(17)
    seq = torch.as_tensor(lens, dtype=torch.int32, device=DEV)

    def make(NQ):
        Q = inputs.to_bf16(rng.standard_normal((B, NQ, H_q, d)).astype(np.float32)).to(DEV)
        gates = torch.from_numpy(rng.uniform(0.0, 1.0, (B, NQ, H_q, 3)).astype(np.float32)).to(DEV)
        bi, ns = _lists(rng, B, NQ, H, lens, 16)
        return Q, gates, torch.from_numpy(bi).to(DEV), torch.from_numpy(ns).to(DEV)
    a, b = make(8), make(6)
    need = max(sda.lib().sda_nsa_decode_workspace(B, nq, H_q, H, 16, d, max(lens), kc.shape[2], w, 4, 0)
               for nq, w in ((8, 256), (6, 130)))
    ws = torch.zeros(need, dtype=torch.uint8, device=DEV)
    o1, l1, u1 = sda.sda_nsa_decode(a[0], K, V, kc, vc, seq, a[2], a[3], a[1], 64, 256, group_C=4, ws=ws)
    o1, l1, u1 = o1.clone(), l1.clone(), u1.clone()
    sda.sda_nsa_decode(b[0], K, V, kc, vc, seq, b[2], b[3], b[1], 64, 130, group_C=4, ws=ws)
    o2, l2, u2 = sda.sda_nsa_decode(a[0], K, V, kc, vc, seq, a[2], a[3], a[1], 64, 256, group_C=4, ws=ws)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(u1, u2)
    assert torch.equal(torch.nan_to_num(l1, neginf=-1e30), torch.nan_to_num(l2, neginf=-1e30))
