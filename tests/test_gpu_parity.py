"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on
the same seeded inputs.  Block indices must match bit for bit; outputs must
lie within 2e-3 max-abs.  Small cases run whole; the full-size workloads
compare every row that the oracle can afford and sample the rest.
"""
import math
import sys

import numpy as np
import pytest
import torch

import block_sparse_attention_pool_amd as sda
import oracle as O
import synth
from synth import inputs
from tests.parity_util import (DELTA, DELTA_REL_MH, DEV, TOL, SparseRows, bits, f64, gpu_ktilde, oracle_decode,
                               oracle_kt, oracle_select, rows_of, scale_of, seq, tie_free_indexer)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    sda.lib()          # raises if libsda.so is missing: there is no fallback path


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _check_selection(cfg, bi, ns, want, rows):
    bi = bi.cpu().numpy()
    ns = ns.cpu().numpy()
    bad = 0
    for r in rows:
        w = want[r]
        n = int(ns[r])
        if n != len(w) or not np.array_equal(bi[r][:n], w) or not np.all(bi[r][n:] == -1):
            bad += 1
    return bad


# ---------------------------------------------------------------------------
# config 1: the whole path on the tiny decode step
# ---------------------------------------------------------------------------

def test_c1_full_path():
    cfg = synth.get_config(1)
    _say("c1: draw")
    K, V, _ = inputs.kv_layer(cfg, 0, device="cpu")
    Kg, Vg = K.to(DEV), V.to(DEV)
    kv_rows = [(b, g) for b in range(cfg.B) for g in range(cfg.H_kv)]
    kt = oracle_kt(K, cfg.T, kv_rows)
    _say("c1: compressed keys")
    ktg = gpu_ktilde(Kg, cfg.T)
    for (b, g) in kv_rows:
        assert np.array_equal(ktg[b, g].double().cpu().numpy(), kt[(b, g)])      # bit for bit
    rows = rows_of(cfg)
    F, _ = tie_free_indexer(cfg, 0, kt, rows)
    want = oracle_select(cfg, O.bf16_to_f64(bits(F)), kt, rows)
    _say("c1: select")
    scores = torch.empty((cfg.B, cfg.NQ, cfg.H_kv, ktg.shape[2]), dtype=torch.float32, device=DEV)
    bi, ns = sda.sda_score_select(F.to(DEV), ktg, seq(cfg), cfg.n_init, cfg.n_local, cfg.top_k, scores=scores)
    assert _check_selection(cfg, bi, ns, want, rows) == 0
    Fd = O.bf16_to_f64(bits(F))
    for (b, q, g) in rows:
        s = O.indexer_scores(Fd[b, q, g], kt[(b, g)])
        assert np.abs(scores[b, q, g, :cfg.NB].double().cpu().numpy() - s).max() < 1e-5
    _say("c1: decode")
    Q = inputs.to_bf16(inputs.attention_queries(cfg, 0))
    out, lse = sda.sda_sparse_decode(Q.to(DEV), Kg, Vg, seq(cfg), bi, ns)
    torch.cuda.synchronize()
    Qd = O.bf16_to_f64(bits(Q))
    rk = SparseRows(K, V, cfg.T)
    G = cfg.G
    err = 0.0
    for (b, q, g) in rows:
        o, l = oracle_decode(Qd, rk, b, q, g, G, want[(b, q, g)], cfg.T, scale_of(cfg))
        err = max(err, np.abs(out[b, q, g * G:(g + 1) * G].double().cpu().numpy() - o).max())
        assert np.abs(lse[b, q, g * G:(g + 1) * G].double().cpu().numpy() - l).max() < 1e-3
    _say("c1: max abs err", err)
    assert err <= TOL


def test_c1_dense_special_case_matches_sdpa():
    # k >= every candidate: the block set is all blocks, so the result is
    # dense attention over the T tokens (torch SDPA on the CPU, float64)
    cfg = synth.get_config(1)
    K, V, _ = inputs.kv_layer(cfg, 0, device="cpu")
    Kg, Vg = K.to(DEV), V.to(DEV)
    ktg = gpu_ktilde(Kg, cfg.T)
    F = inputs.to_bf16(inputs.indexer_vectors(cfg, 0)).to(DEV)
    bi, ns = sda.sda_score_select(F, ktg, seq(cfg), 1, 2, cfg.NB)
    assert ns.min().item() == cfg.NB == ns.max().item()
    for g in range(cfg.H_kv):
        assert torch.equal(bi[0, 0, g, :cfg.NB].cpu(), torch.arange(cfg.NB, dtype=torch.int32))
        assert torch.all(bi[0, 0, g, cfg.NB:] == -1)
    Q = inputs.to_bf16(inputs.attention_queries(cfg, 0))
    out, _ = sda.sda_sparse_decode(Q.to(DEV), Kg, Vg, seq(cfg), bi, ns)
    G = cfg.G
    for g in range(cfg.H_kv):
        q = Q[0, 0, g * G:(g + 1) * G].double()[None]
        ref = torch.nn.functional.scaled_dot_product_attention(q, K[0, g].double()[None, None],
                                                               V[0, g].double()[None, None])[0]
        assert (out[0, 0, g * G:(g + 1) * G].double().cpu() - ref).abs().max().item() <= TOL


# ---------------------------------------------------------------------------
# compressed keys: partial blocks and incremental updates
# ---------------------------------------------------------------------------

def test_ktilde_partial_block_and_incremental_update():
    cfg = synth.get_config(1)
    K, _, _ = inputs.kv_layer(cfg, 0, device="cpu")
    Kg = K.to(DEV)
    T0, T1 = 3000, 3131
    kt0 = oracle_kt(K, T1, [(0, 0), (0, 1)])
    bulk = gpu_ktilde(Kg, T1)
    nb = O.num_blocks(T1)
    for g in range(2):
        assert np.array_equal(bulk[0, g, :nb].double().cpu().numpy(), kt0[(0, g)])   # bit for bit
    # token-by-token on the GPU equals the bulk build bit for bit
    inc = gpu_ktilde(Kg, T0)
    for t in range(T0, T1):
        lo = torch.tensor([t], dtype=torch.int32, device=DEV)
        hi = torch.tensor([t + 1], dtype=torch.int32, device=DEV)
        sda.sda_update_compressed_keys(Kg, inc, lo, hi, 1)
    assert torch.equal(inc[:, :, :nb], bulk[:, :, :nb])
    # and is the bf16 rounding of the oracle's running-mean update: within half
    # a bf16 ulp of it (plus the running mean's own fp64 noise)
    kk = f64(K[0, 0, :T1])
    run = O.compressed_keys(kk, T0)
    for t in range(T0, T1):
        run = O.append_token(run, t, kk[t])
    got = inc[0, 0, :nb].double().cpu().numpy()
    half_ulp = np.ldexp(1.0, np.frexp(np.abs(got) + 2.0 ** -133)[1] - 9)
    assert np.all(np.abs(got - run) <= half_ulp * (1 + 1e-9) + 1e-12)


# ---------------------------------------------------------------------------
# selection edge cases
# ---------------------------------------------------------------------------

def _select_direct(kt_np, F_np, T, n_init, n_local, k):
    """Run score_select on a hand-made K~ and F (both rounded to bf16)."""
    B, H, NB, d = kt_np.shape
    ktg = torch.from_numpy(O.store_bf16(kt_np)).to(torch.bfloat16).to(DEV)
    Fb = inputs.to_bf16(F_np)
    bi, ns = sda.sda_score_select(Fb.to(DEV), ktg, torch.full((B,), T, dtype=torch.int32, device=DEV),
                                  n_init, n_local, k)
    return bi.cpu().numpy(), ns.cpu().numpy(), O.bf16_to_f64(bits(Fb))


@pytest.mark.parametrize("T,k", [(1, 8), (64, 8), (65, 8), (128, 8), (192, 8), (640, 0), (640, 7),
                                 (640, 100), (4000, 5)])
def test_select_small_and_degenerate(T, k):
    rng = np.random.default_rng(T * 31 + k)
    NB, d = 70, 64
    kt = rng.standard_normal((1, 2, NB, d)) / 8
    F = rng.standard_normal((1, 1, 2, d)) / 8
    bi, ns, Fd = _select_direct(kt, F, T, 1, 2, k)
    nb = O.num_blocks(T)
    for g in range(2):
        want, _ = O.select_row(Fd[0, 0, g], O.store_bf16(kt[0, g, :nb]), 1, 2, k)
        n = int(ns[0, 0, g])
        assert n == len(want)
        assert list(bi[0, 0, g, :n]) == list(want)
        assert np.all(bi[0, 0, g, n:] == -1)


@pytest.mark.parametrize("NB,T,n_init,n_local,k", [
    (4096, 4096 * 64, 1, 2, 40),        # 16 chunk lists: the longest the in-launch merge takes
    (5000, 5000 * 64 - 10, 1, 2, 40),   # past it the selection runs as a second launch
    (1000, 301 * 64 - 5, 3, 5, 64),     # chunks past the sequence end, longest lists
    (600, 600 * 64, 0, 0, 1),
    (2048, 2048 * 64, 1, 2, 65)])       # lists too long for the merge: second launch
def test_select_long_rows(NB, T, n_init, n_local, k):
    rng = np.random.default_rng(NB + k)
    kt = rng.standard_normal((1, 2, NB, 64)) / 8
    F = rng.standard_normal((1, 1, 2, 64)) / 8
    bi, ns, Fd = _select_direct(kt, F, T, n_init, n_local, k)
    nb = O.num_blocks(T)
    for g in range(2):
        want, _ = O.select_row(Fd[0, 0, g], O.store_bf16(kt[0, g, :nb]), n_init, n_local, k)
        n = int(ns[0, 0, g])
        assert list(bi[0, 0, g, :n]) == list(want)
        assert np.all(bi[0, 0, g, n:] == -1)


def _gapped_rows(cand, top_k, scores_by_row, gap):
    """Rows whose top-k cut gap is at least `gap` (selection decided without near-ties)."""
    return [r for r, s in scores_by_row.items() if O.cut_gap(s, cand, top_k) >= gap]


@pytest.mark.parametrize("NQ,top_k", [(1, 16), (20, 16), (7, 16), (64, 16), (1, 80), (3, 80)])
def test_select_paths_match_oracle(NQ, top_k):
    # top_k <= 64: the selection runs inside the scoring launch (the last
    # arriving chunk workgroup merges per-chunk lists); top_k = 80: the
    # separate radix-select launch.  Both against the oracle on every row
    # whose cut gap exceeds the float32 score error, call after call, with
    # the in-launch path's arrival counters back at zero after each call.
    cfg = synth.get_config(2)
    K, _, _ = inputs.kv_layer(cfg, 0, device=DEV)
    ktg = gpu_ktilde(K, cfg.T)
    kv_rows = [(b, g) for b in range(cfg.B) for g in range(cfg.H_kv)]
    kt = oracle_kt(K, cfg.T, kv_rows)
    rng = np.random.default_rng(NQ + top_k)
    F = inputs.to_bf16(rng.standard_normal((cfg.B, NQ, cfg.H_kv, cfg.d)) / 8)
    Fd = O.bf16_to_f64(bits(F))
    nb = O.num_blocks(cfg.T)
    cand = O.candidates(nb, cfg.n_init, cfg.n_local)
    sc = {(b, q, g): O.decision_scores(O.indexer_scores(Fd[b, q, g], kt[(b, g)]))
          for b in range(cfg.B) for q in range(NQ) for g in range(cfg.H_kv)}
    rows = _gapped_rows(cand, top_k, sc, DELTA)
    _say(f"select NQ={NQ} top_k={top_k}: {len(rows)} of {len(sc)} rows tie-free")
    assert len(rows) >= 0.8 * len(sc)
    want = {r: O.block_set(nb, cfg.n_init, cfg.n_local, O.top_k(sc[r], cand, top_k)) for r in rows}
    nbytes = sda.lib().sda_score_select_workspace(cfg.B, NQ, cfg.H_kv, ktg.shape[2], top_k)
    ws = torch.zeros(nbytes, dtype=torch.uint8, device=DEV)
    # one arrival counter per (b, KV head, vector tile); tiles of up to 16
    # vectors, halved while the grid holds fewer than 512 workgroups
    chunks = -(-ktg.shape[2] // 256)
    nv = 1
    while nv < NQ and nv < 16:
        nv *= 2
    while nv > 1 and chunks * cfg.B * cfg.H_kv * -(-NQ // nv) < 512:
        nv //= 2
    n_cnt = cfg.B * cfg.H_kv * -(-NQ // nv)
    first = None
    for it in range(6):
        bi, ns = sda.sda_score_select(F.to(DEV), ktg, seq(cfg), cfg.n_init, cfg.n_local, top_k, ws=ws)
        torch.cuda.synchronize()
        if first is None:
            first = (bi.clone(), ns.clone())
            _check_selection(cfg, bi, ns, want, rows)
        assert torch.equal(bi, first[0]) and torch.equal(ns, first[1]), it
        if top_k <= 64:
            assert int(ws[nbytes - 4 * n_cnt:].count_nonzero()) == 0, it


@pytest.mark.parametrize("NQ,top_k", [(1, 16), (3, 16), (1, 80)])
def test_comparator_select_paths_match_oracle(NQ, top_k):
    # the comparator's in-launch selection (top_k <= 64) and its selection
    # launch (top_k = 80) against the oracle's summed softmax on every row
    # with a clear relative cut gap; counters back at zero after each call
    cfg = synth.get_config(2)
    K, _, _ = inputs.kv_layer(cfg, 0, device=DEV)
    ktg = gpu_ktilde(K, cfg.T)
    kv_rows = [(b, g) for b in range(cfg.B) for g in range(cfg.H_kv)]
    kt = oracle_kt(K, cfg.T, kv_rows)
    rng = np.random.default_rng(40 + NQ + top_k)
    Q = inputs.to_bf16(rng.standard_normal((cfg.B, NQ, cfg.H_q, cfg.d)))
    Qd = O.bf16_to_f64(bits(Q))
    G = cfg.G
    tau = math.sqrt(cfg.d)
    nb = O.num_blocks(cfg.T)
    cand = O.candidates(nb, cfg.n_init, cfg.n_local)
    rows, want = [], {}
    for b in range(cfg.B):
        for q in range(NQ):
            for g in range(cfg.H_kv):
                s = O.decision_scores(O.multihead_scores(Qd[b, q, g * G:(g + 1) * G], kt[(b, g)], tau))
                top = np.sort(s[cand])[::-1][top_k - 1]
                if O.cut_gap(s, cand, top_k) >= DELTA_REL_MH * abs(top):
                    rows.append((b, q, g))
                    want[(b, q, g)] = O.block_set(nb, cfg.n_init, cfg.n_local, O.top_k(s, cand, top_k))
    _say(f"comparator NQ={NQ} top_k={top_k}: {len(rows)} of {cfg.B * NQ * cfg.H_kv} rows tie-free")
    assert len(rows) >= 0.8 * cfg.B * NQ * cfg.H_kv
    nbytes = sda.lib().sda_score_select_multihead_workspace(cfg.B, NQ, cfg.H_q, cfg.H_kv, ktg.shape[2], top_k)
    ws = torch.zeros(nbytes, dtype=torch.uint8, device=DEV)
    first = None
    for it in range(4):
        bi, ns = sda.sda_score_select_multihead(Q.to(DEV), ktg, seq(cfg), cfg.n_init, cfg.n_local, top_k, tau,
                                                ws=ws)
        torch.cuda.synchronize()
        if first is None:
            first = (bi.clone(), ns.clone())
            _check_selection(cfg, bi, ns, want, rows)
        assert torch.equal(bi, first[0]) and torch.equal(ns, first[1]), it
        if top_k <= 64:
            assert int(ws[nbytes - 4 * cfg.B * cfg.H_kv * NQ:].count_nonzero()) == 0, it


# exact: both launches run the same split plan.  At one split the plain decode
# takes 10 waves (all of the LDS); the step needs LDS for the merge and takes 9.
@pytest.mark.parametrize("cid,split_k,exact", [(2, 0, False), (2, 5, True), (3, 0, False), (3, 7, True),
                                               (3, 1, False)])
def test_decode_step_matches_separate_calls(cid, split_k, exact):
    # the step entry point (the next layer's selection finished inside this
    # layer's decode launch) against
    # sda_score_select for the next layer and sda_sparse_decode for this one:
    # identical block lists; identical outputs when both run the same split
    # plan, else equal up to the order of the split merge
    cfg = synth.get_config(cid)
    _say(f"decode step: config {cid}, split_k {split_k}")
    K0, V0, _ = inputs.kv_layer(cfg, 0, device=DEV)
    K1, _, _ = inputs.kv_layer(cfg, 1, device=DEV)
    kt1 = gpu_ktilde(K1, cfg.T)
    del K1
    kt0 = gpu_ktilde(K0, cfg.T)
    F0 = inputs.to_bf16(inputs.indexer_vectors(cfg, 0)).to(DEV)
    F1 = inputs.to_bf16(inputs.indexer_vectors(cfg, 1)).to(DEV)
    Q0 = inputs.to_bf16(inputs.attention_queries(cfg, 0)).to(DEV)
    sel = (cfg.n_init, cfg.n_local, cfg.top_k)
    bi0, ns0 = sda.sda_score_select(F0, kt0, seq(cfg), *sel)
    ref_bi1, ref_ns1 = sda.sda_score_select(F1, kt1, seq(cfg), *sel)
    ref_out, ref_lse = sda.sda_sparse_decode(Q0, K0, V0, seq(cfg), bi0, ns0, split_k=split_k)
    nbytes = sda.lib().sda_decode_step_workspace(cfg.B, cfg.H_q, cfg.H_kv, cfg.d, bi0.shape[-1], split_k,
                                                 kt1.shape[2], cfg.top_k)
    ws = torch.zeros(nbytes, dtype=torch.uint8, device=DEV)
    for it in range(6):
        out, lse, bi1, ns1 = sda.sda_decode_step(Q0, K0, V0, seq(cfg), bi0, ns0, F1, kt1, seq(cfg), *sel,
                                                 split_k=split_k, ws=ws)
        torch.cuda.synchronize()
        assert torch.equal(bi1, ref_bi1) and torch.equal(ns1, ref_ns1), it
        if exact:
            assert torch.equal(out, ref_out) and torch.equal(lse, ref_lse), it
        else:
            assert (out - ref_out).abs().max().item() <= 1e-5, it
            assert (lse - ref_lse).abs().max().item() <= 1e-5, it
        if split_k != 1:      # split arrival counters (the workspace's first ints) back at zero
            assert int(ws[:4 * cfg.B * cfg.H_kv].count_nonzero()) == 0, it


@pytest.mark.parametrize("d,top_k,n_init,n_local,split_k", [(128, 32, 1, 2, 0), (64, 8, 0, 3, 0),
                                                       (128, 64, 2, 0, 3), (128, 5, 3, 1, 2), (64, 16, 1, 2, 1),
                                                       (128, 80, 1, 2, 0)])
def test_decode_step_ragged(d, top_k, n_init, n_local, split_k):
    # ragged lengths in both layers, the next layer's capacity not a multiple
    # of a chunk, sequences shorter than init + local, one-block sequences:
    # the step's block sets equal sda_score_select's, its outputs
    # sda_sparse_decode's (bit for bit with the same explicit split count).
    # top_k = 80 is past the in-launch selection: the step runs the calls.
    B, H_kv, G = 3, 2, 4
    H_q = H_kv * G
    T_cap, NBn = 5000, 300
    gen = torch.Generator(device=DEV).manual_seed(7 * d + top_k)
    def rnd(*shape, scale=1.0):
        return (torch.randn(*shape, generator=gen, device=DEV) * scale).to(torch.bfloat16)
    K, V = rnd(B, H_kv, T_cap, d), rnd(B, H_kv, T_cap, d)
    Kn = rnd(B, H_kv, NBn * 64, d)
    Q, F0, F1 = rnd(B, 1, H_q, d), rnd(B, 1, H_kv, d, scale=d ** -0.5), rnd(B, 1, H_kv, d, scale=d ** -0.5)
    seq0 = torch.tensor([5000, 3000, 65], dtype=torch.int32, device=DEV)
    seq1 = torch.tensor([NBn * 64 - 5, 64 * 3, 1], dtype=torch.int32, device=DEV)
    zero = torch.zeros(B, dtype=torch.int32, device=DEV)
    kt0 = torch.zeros((B, H_kv, -(-T_cap // 64), d), dtype=torch.bfloat16, device=DEV)
    kt1 = torch.zeros((B, H_kv, NBn, d), dtype=torch.bfloat16, device=DEV)
    sda.sda_update_compressed_keys(K, kt0, zero, seq0, T_cap)
    sda.sda_update_compressed_keys(Kn, kt1, zero, seq1, NBn * 64)
    sel = (n_init, n_local, top_k)
    bi0, ns0 = sda.sda_score_select(F0, kt0, seq0, *sel)
    ref_bi1, ref_ns1 = sda.sda_score_select(F1, kt1, seq1, *sel)
    ref_out, ref_lse = sda.sda_sparse_decode(Q, K, V, seq0, bi0, ns0, split_k=split_k)
    nsm = bi0.shape[-1]
    fused = sda.lib().sda_decode_step_is_fused(B, H_q, H_kv, d, nsm, split_k, NBn, top_k)
    _say(f"ragged step d={d} top_k={top_k} split_k={split_k}: one launch = {fused}")
    assert fused == (1 if top_k <= 64 else 0)
    # this layer's compressed keys, pooled up to a shorter length: the step
    # refreshes the blocks the remaining tokens touch (1 to 70 per sequence)
    old0 = seq0 - torch.tensor([70, 1, 1], dtype=torch.int32, device=DEV)
    kt0r = torch.zeros_like(kt0)
    sda.sda_update_compressed_keys(K, kt0r, zero, old0, T_cap)
    for it in range(4):
        out, lse, bi1, ns1 = sda.sda_decode_step(Q, K, V, seq0, bi0, ns0, F1, kt1, seq1, *sel, split_k=split_k,
                                                 k_tilde_cur=kt0r, len_old_cur=old0, max_new_tokens_cur=70)
        torch.cuda.synchronize()
        assert torch.equal(kt0r, kt0), it
        assert torch.equal(ns1, ref_ns1) and torch.equal(bi1, ref_bi1), it
        if split_k > 0:
            assert torch.equal(out, ref_out) and torch.equal(lse, ref_lse), it
        else:
            assert (out - ref_out).abs().max().item() <= 1e-5, it
            assert ((lse - ref_lse).abs().nan_to_num(0.0)).max().item() <= 1e-5, it
    # the one-block sequence selects its only block; the three-block one all of its blocks
    assert int(ns1[2, 0, 0]) == 1 and int(bi1[2, 0, 0, 0]) == 0
    assert int(ns1[1, 0, 0]) == 3 and list(bi1[1, 0, 0, :3].tolist()) == [0, 1, 2]


def test_select_ties_go_to_lower_index():
    rng = np.random.default_rng(5)
    NB, d = 300, 128
    kt = rng.standard_normal((1, 1, NB, d)) / 64
    kt[0, 0, [40, 90, 91, 150, 260]] = kt[0, 0, 7]       # six identical pooled keys
    F = np.zeros((1, 1, 1, d))
    F[0, 0, 0] = kt[0, 0, 7] * 50                          # they score highest
    bi, ns, Fd = _select_direct(kt, F, NB * 64, 1, 2, 4)
    assert list(bi[0, 0, 0, :ns[0, 0, 0]]) == [0, 7, 40, 90, 91, 298, 299]
    want, _ = O.select_row(Fd[0, 0, 0], O.store_bf16(kt[0, 0]), 1, 2, 4)
    assert list(want) == [0, 7, 40, 90, 91, 298, 299]


# ---------------------------------------------------------------------------
# decode invariants
# ---------------------------------------------------------------------------

def _c1_decode_inputs(T=None):
    cfg = synth.get_config(1)
    T = cfg.T if T is None else T
    K, V, _ = inputs.kv_layer(cfg, 0, device="cpu")
    Kg, Vg = K.to(DEV), V.to(DEV)
    ktg = gpu_ktilde(Kg, T)
    F = inputs.to_bf16(inputs.indexer_vectors(cfg, 0)).to(DEV)
    bi, ns = sda.sda_score_select(F, ktg, seq(cfg, T), cfg.n_init, cfg.n_local, cfg.top_k)
    Q = inputs.to_bf16(inputs.attention_queries(cfg, 0))
    return cfg, K, V, Kg, Vg, bi, ns, Q, T


def test_decode_split_invariance_and_determinism():
    cfg, K, V, Kg, Vg, bi, ns, Q, T = _c1_decode_inputs()
    Qg = Q.to(DEV)
    ref, lref = sda.sda_sparse_decode(Qg, Kg, Vg, seq(cfg), bi, ns, split_k=1)
    for sk in (2, 3, 5, 11, 0):
        o, l = sda.sda_sparse_decode(Qg, Kg, Vg, seq(cfg), bi, ns, split_k=sk)
        assert (o - ref).abs().max().item() < 1e-5
        assert (l - lref).abs().max().item() < 1e-5
        o2, _ = sda.sda_sparse_decode(Qg, Kg, Vg, seq(cfg), bi, ns, split_k=sk)
        assert torch.equal(o, o2)


def test_decode_partial_last_block():
    cfg, K, V, Kg, Vg, bi, ns, Q, T = _c1_decode_inputs(T=4000)
    out, lse = sda.sda_sparse_decode(Q.to(DEV), Kg, Vg, seq(cfg, T), bi, ns)
    bi_h, ns_h = bi.cpu().numpy(), ns.cpu().numpy()
    Qd = O.bf16_to_f64(bits(Q))
    rk = SparseRows(K, V, T)
    G = cfg.G
    for g in range(cfg.H_kv):
        blocks = bi_h[0, 0, g, :ns_h[0, 0, g]]
        assert O.num_blocks(T) - 1 in blocks                # the partial block is local
        o, l = oracle_decode(Qd, rk, 0, 0, g, G, blocks, T, scale_of(cfg))
        assert np.abs(out[0, 0, g * G:(g + 1) * G].double().cpu().numpy() - o).max() <= TOL


def test_decode_empty_and_invalid_entries():
    cfg, K, V, Kg, Vg, bi, ns, Q, T = _c1_decode_inputs()
    bi2 = bi.clone()
    ns2 = ns.clone()
    ns2[0, 0, 1] = 0                                          # empty row
    bi2[0, 0, 0, 3] = 10_000                                  # out-of-range ids are skipped
    bi2[0, 0, 0, 4] = -5
    out, lse = sda.sda_sparse_decode(Q.to(DEV), Kg, Vg, seq(cfg), bi2, ns2)
    G = cfg.G
    assert torch.all(out[0, 0, G:2 * G] == 0)
    assert torch.all(torch.isneginf(lse[0, 0, G:2 * G]))
    keep = [int(j) for i, j in enumerate(bi.cpu().numpy()[0, 0, 0, :ns[0, 0, 0]]) if i not in (3, 4)]
    o, _ = oracle_decode(O.bf16_to_f64(bits(Q)), SparseRows(K, V, T), 0, 0, 0, G, keep, T, scale_of(cfg))
    assert np.abs(out[0, 0, :G].double().cpu().numpy() - o).max() <= TOL


def test_multi_query_plain_decode_each_query_own_list():
    cfg = synth.get_config(1)
    import dataclasses
    cfg = dataclasses.replace(cfg, NQ=3)
    K, V, _ = inputs.kv_layer(cfg, 0, device="cpu")
    Kg, Vg = K.to(DEV), V.to(DEV)
    ktg = gpu_ktilde(Kg, cfg.T)
    F = inputs.to_bf16(inputs.indexer_vectors(cfg, 0)).to(DEV)
    bi, ns = sda.sda_score_select(F, ktg, seq(cfg), 1, 2, 8)
    Q = inputs.to_bf16(inputs.attention_queries(cfg, 0))
    out, _ = sda.sda_sparse_decode(Q.to(DEV), Kg, Vg, seq(cfg), bi, ns)
    Qd = O.bf16_to_f64(bits(Q))
    rk = SparseRows(K, V, cfg.T)
    for (b, q, g) in rows_of(cfg):
        blocks = bi.cpu().numpy()[b, q, g, :ns[b, q, g].item()]
        o, _ = oracle_decode(Qd, rk, b, q, g, cfg.G, blocks, cfg.T, scale_of(cfg))
        assert np.abs(out[b, q, g * cfg.G:(g + 1) * cfg.G].double().cpu().numpy() - o).max() <= TOL


def test_graph_replay_matches_eager():
    # the decode step captured as a HIP graph; every replay, with eager work and
    # synchronisations in between, reproduces the eager result bit for bit
    cfg = synth.get_config(1)
    K, V, _ = inputs.kv_layer(cfg, 0, device=DEV)
    ktg = gpu_ktilde(K, cfg.T)
    F = inputs.to_bf16(inputs.indexer_vectors(cfg, 0)).to(DEV)
    Q = inputs.to_bf16(inputs.attention_queries(cfg, 0)).to(DEV)
    s = seq(cfg)
    sc, (bi, ns) = sda.prepare(sda.sda_score_select, F, ktg, s, 1, 2, 8)
    dc, (out, lse) = sda.prepare(sda.sda_sparse_decode, Q, K, V, s, bi, ns, split_k=3)
    sc.run()
    dc.run()
    torch.cuda.synchronize()
    ref_bi, ref_out, ref_lse = bi.clone(), out.clone(), lse.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        sc.run()
        dc.run()
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        sc.run()
        dc.run()
    for r in range(4):
        out.zero_()
        bi.fill_(-7)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(bi, ref_bi) and torch.equal(out, ref_out) and torch.equal(lse, ref_lse), r
        # eager work between replays, on other buffers
        sda.sda_sparse_decode(Q, K, V, s, ref_bi, ns, split_k=2)
        torch.cuda.synchronize()


def _gpu_lists_of(bi, ns, rows):
    bi = bi.cpu().numpy()
    ns = ns.cpu().numpy()
    return {r: bi[r][:ns[r]] for r in rows}


def test_split_merge_matches_oracle_and_repeats():
    # the last-arriving workgroup's log-sum-exp merge of the splits: every
    # split plan within tolerance of the oracle on sampled rows and of each
    # other; the default plan bit for bit the same call after call (the
    # arrival counters reset each time)
    cfg = synth.get_config(2)
    K, V, _ = inputs.kv_layer(cfg, 0, device=DEV)
    ktg = gpu_ktilde(K, cfg.T)
    F = inputs.to_bf16(inputs.indexer_vectors(cfg, 0)).to(DEV)
    Q = inputs.to_bf16(inputs.attention_queries(cfg, 0))
    bi, ns = sda.sda_score_select(F, ktg, seq(cfg), cfg.n_init, cfg.n_local, cfg.top_k)
    lists = _gpu_lists_of(bi, ns, [(b, 0, (b + 3) % cfg.H_kv) for b in range(cfg.B)])
    Qd = O.bf16_to_f64(bits(Q))
    rk = SparseRows(K, V, cfg.T)
    Qg = Q.to(DEV)
    ws = torch.zeros(sda.lib().sda_sparse_decode_workspace(cfg.B, 1, cfg.H_q, cfg.H_kv, bi.shape[-1], cfg.d, 0),
                     dtype=torch.uint8, device=DEV)
    ref, lref = sda.sda_sparse_decode(Qg, K, V, seq(cfg), bi, ns, ws=ws)
    for (b, q, g), blocks in lists.items():
        o, l = oracle_decode(Qd, rk, b, q, g, cfg.G, blocks, cfg.T, scale_of(cfg))
        assert np.abs(ref[b, q, g * cfg.G:(g + 1) * cfg.G].double().cpu().numpy() - o).max() <= TOL
        assert np.abs(lref[b, q, g * cfg.G:(g + 1) * cfg.G].double().cpu().numpy() - l).max() <= 1e-3
    for it in range(20):
        out, lse = sda.sda_sparse_decode(Qg, K, V, seq(cfg), bi, ns, ws=ws)
        torch.cuda.synchronize()
        assert torch.equal(out, ref) and torch.equal(lse, lref), it
        assert int(ws[:4 * cfg.B * cfg.H_kv].count_nonzero()) == 0, it
    for sk in (1, 2, 3, 7, 19):
        o2, l2 = sda.sda_sparse_decode(Qg, K, V, seq(cfg), bi, ns, split_k=sk)
        assert (o2 - ref).abs().max().item() <= 1e-5, sk
        assert (l2 - lref).abs().max().item() <= 1e-5, sk


def _replays_match(g, outs, refs, eager_between):
    for r in range(4):
        for o in outs:
            o.fill_(-7) if o.dtype == torch.int32 else o.zero_()
        g.replay()
        torch.cuda.synchronize()
        for o, ref in zip(outs, refs):
            assert torch.equal(o, ref), r
        eager_between()
        torch.cuda.synchronize()


def _capture(fn):
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    return g


def test_graph_replay_of_decode_step_and_tiled_calls():
    # the one-launch decode step (as the benchmark captures it), the row-tiled
    # prefill attention and the tiled exact grouped decode with split-K (its
    # arrival counters must be back at zero after every replay): every
    # replay, with eager work and synchronisations in between, equals the
    # eager result bit for bit
    cfg = synth.get_config(1)
    K, V, _ = inputs.kv_layer(cfg, 0, device=DEV)
    ktg = gpu_ktilde(K, cfg.T)
    F = inputs.to_bf16(inputs.indexer_vectors(cfg, 0)).to(DEV)
    Q = inputs.to_bf16(inputs.attention_queries(cfg, 0)).to(DEV)
    s = seq(cfg)
    bi, ns = sda.sda_score_select(F, ktg, s, 1, 2, 8)
    step, souts = sda.prepare(sda.sda_decode_step, Q, K, V, s, bi, ns, F, ktg, s, 1, 2, 8)
    step.run()
    torch.cuda.synchronize()
    refs = [o.clone() for o in souts]
    g = _capture(step.run)
    _replays_match(g, list(souts), refs, lambda: sda.sda_sparse_decode(Q, K, V, s, bi, ns, split_k=2))

    # prefill attention over a 2048-token chunk of the same cache
    NQ = 2048
    Qp = torch.randn((cfg.B, NQ, cfg.H_q, cfg.d), generator=torch.Generator(device=DEV).manual_seed(3),
                     device=DEV).to(torch.bfloat16)
    Fp = torch.randn((cfg.B, NQ, cfg.H_kv, cfg.d), generator=torch.Generator(device=DEV).manual_seed(4),
                     device=DEV).to(torch.bfloat16)
    pbi, pns = sda.sda_prefill_select(Fp, ktg, s, 1000, 1, 2, 8)
    pout = torch.empty((cfg.B, NQ, cfg.H_q, cfg.d), dtype=torch.float32, device=DEV)
    plse = torch.empty((cfg.B, NQ, cfg.H_q), dtype=torch.float32, device=DEV)

    def prefill():
        sda.sda_prefill_attention(Qp, K, V, s, pbi, pns, 1000, out=pout, lse=plse)
    prefill()
    torch.cuda.synchronize()
    prefs = [pout.clone(), plse.clone()]
    g = _capture(prefill)
    _replays_match(g, [pout, plse], prefs, lambda: sda.sda_sparse_decode(Q, K, V, s, bi, ns))

    # exact grouped decode with all 16 queries of a sequence in one group (G = 4:
    # 64 rows, the tiled engine) and three splits
    NQg = 16
    Qg = torch.randn((cfg.B, NQg, cfg.H_q, cfg.d), generator=torch.Generator(device=DEV).manual_seed(5),
                     device=DEV).to(torch.bfloat16)
    Fg = torch.randn((cfg.B, NQg, cfg.H_kv, cfg.d), generator=torch.Generator(device=DEV).manual_seed(6),
                     device=DEV).to(torch.bfloat16)
    gbi, gns = sda.sda_score_select(Fg, ktg, s, 1, 2, 8)
    nbytes = sda.lib().sda_grouped_decode_workspace(cfg.B, NQg, cfg.H_q, cfg.H_kv, gbi.shape[-1], cfg.d, cfg.NB,
                                                    NQg, sda.SDA_GROUP_EXACT, 3)
    assert nbytes > 0
    gws = torch.zeros(nbytes, dtype=torch.uint8, device=DEV)
    gout = torch.empty((cfg.B, NQg, cfg.H_q, cfg.d), dtype=torch.float32, device=DEV)
    glse = torch.empty((cfg.B, NQg, cfg.H_q), dtype=torch.float32, device=DEV)
    guc = torch.empty((cfg.B, 1, cfg.H_kv), dtype=torch.int32, device=DEV)

    def grouped():
        sda.sda_grouped_decode(Qg, K, V, s, gbi, gns, NQg, sda.SDA_GROUP_EXACT, out=gout, lse=glse,
                               union_count=guc, split_k=3, ws=gws)
    grouped()
    torch.cuda.synchronize()
    grefs = [gout.clone(), glse.clone(), guc.clone()]
    g = _capture(grouped)
    _replays_match(g, [gout, glse, guc], grefs, lambda: sda.sda_sparse_decode(Q, K, V, s, bi, ns))
    # the per-query decode of the same lists agrees
    pq, _ = sda.sda_sparse_decode(Qg, K, V, s, gbi, gns)
    assert (gout - pq).abs().max().item() < 1e-4
