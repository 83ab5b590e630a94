"""Pins for the CPU oracle: closed forms, brute force, library routines and
the pages' printed values.  None of these re-types the oracle's formula; each
would fail on a plausible slip in it (dropped term, wrong sign or index,
transposed operand).  CPU only.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle as O

HERE = os.path.dirname(os.path.abspath(__file__))


def rng(seed):
    return np.random.default_rng(seed)


# ---------------------------------------------------------------------------
# compressed keys
# ---------------------------------------------------------------------------

def test_bf16_decode_exact():
    # bit patterns with known values: 1.0, -2.0, 0.5, smallest normal, 1 + 2^-7
    bits = np.array([0x3F80, 0xC000, 0x3F00, 0x0080, 0x3F81], dtype=np.uint16)
    want = [1.0, -2.0, 0.5, 2.0 ** -126, 1.0 + 2.0 ** -7]
    assert list(O.bf16_to_f64(bits)) == want
    # agrees with torch's own bf16 -> float conversion
    t = torch.randn(1000).to(torch.bfloat16)
    b = t.view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(O.bf16_to_f64(b), t.to(torch.float64).numpy())


def test_store_bf16_hand_cases():
    # grid points stay; halfway cases go to the even neighbour; the ulp of
    # [1, 2) is 2^-7 and of [2^-126, 2^-125) is 2^-133 (as of the subnormals)
    u = 2.0 ** -7
    x = np.array([1.0, 1.0 + u, 1.0 + u / 2, 1.0 + 3 * u / 2, 1.0 + u / 2 + 2.0 ** -40,
                  -1.0 - u / 2, 3.0, 2.0 ** -126, 2.0 ** -133, 2.0 ** -134, 3 * 2.0 ** -134,
                  0.0, -0.0, 65504.0])
    want = [1.0, 1.0 + u, 1.0, 1.0 + 2 * u, 1.0 + u, -1.0, 3.0, 2.0 ** -126, 2.0 ** -133, 0.0,
            2 * 2.0 ** -133, 0.0, -0.0, 65536.0]
    got = O.store_bf16(x)
    assert list(got) == want
    assert np.signbit(got[12])
    big = (2.0 - 2.0 ** -8) * 2.0 ** 127                    # halfway to 2^128: rounds up, overflows
    assert O.store_bf16(np.array([big, -big, (2.0 - 2.0 ** -7) * 2.0 ** 127])).tolist() == \
        [np.inf, -np.inf, (2.0 - 2.0 ** -7) * 2.0 ** 127]


def test_store_bf16_matches_torch_on_float32_values():
    # on values that are exactly float32, one rounding float32 -> bf16 is the
    # same as float64 -> bf16; torch's conversion rounds to nearest even
    v = (rng(3).standard_normal(20000) * np.exp(rng(4).uniform(-30, 30, 20000))).astype(np.float32)
    v[:8] = np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8), 2 ** -130, 0.0, 7.0, 1e-40, 3e38],
                     dtype=np.float32)
    t = torch.from_numpy(v).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(O.store_bf16(v.astype(np.float64)), t)


def test_store_bf16_nearest_brute_force():
    # every result is the nearest of the two neighbouring bf16 values (the
    # even one on a tie), found here by walking the bf16 bit patterns
    x = rng(5).standard_normal(3000) * 10.0 ** rng(6).integers(-20, 20, 3000)
    r = O.store_bf16(x)
    for xi, ri in zip(x, r):
        b = int(np.array([ri], dtype=np.float32).view(np.uint32)[0]) >> 16
        assert np.float32(ri).view(np.uint32) & 0xFFFF == 0          # a bf16 value
        lo, hi = sorted([O.bf16_to_f64(np.array([b - 1], np.uint16))[0] if b & 0x7FFF else ri,
                         O.bf16_to_f64(np.array([b + 1], np.uint16))[0]])
        assert abs(xi - ri) <= min(abs(xi - lo), abs(xi - hi))


def test_compressed_keys_constant_block():
    k = np.zeros((256, 8))
    for j in range(4):
        k[j * 64:(j + 1) * 64] = j + 0.25
    kt = O.compressed_keys(k, 256)
    assert kt.shape == (4, 8)
    assert np.all(kt == (np.arange(4) + 0.25)[:, None])


def test_compressed_keys_permutation_invariant_and_block_local():
    r = rng(1)
    k = r.standard_normal((200, 16))
    kt = O.compressed_keys(k, 200)
    kp = k.copy()
    for j in range(4):
        lo, hi = 64 * j, min(64 * j + 64, 200)
        kp[lo:hi] = kp[lo:hi][r.permutation(hi - lo)]
    assert np.allclose(O.compressed_keys(kp, 200), kt, rtol=0, atol=1e-14)
    # changing one token changes only its own block
    k2 = k.copy()
    k2[130] += 5.0
    d = np.abs(O.compressed_keys(k2, 200) - kt).max(axis=1)
    assert d[2] > 0 and d[0] == d[1] == d[3] == 0


def test_compressed_keys_linearity_per_token_dot():
    # f . K~_j equals the average over the block's tokens of f . k_t,
    # evaluated here token by token with plain Python sums
    r = rng(2)
    T, d = 150, 6
    k = r.standard_normal((T, d))
    f = r.standard_normal(d)
    kt = O.compressed_keys(k, T)
    for j in range(3):
        toks = range(64 * j, min(64 * j + 64, T))
        want = sum(sum(f[i] * k[t][i] for i in range(d)) for t in toks) / len(toks)
        assert abs(float(kt[j] @ f) - want) < 1e-12


def test_compressed_keys_partial_last_block():
    r = rng(3)
    k = r.standard_normal((300, 4))
    kt = O.compressed_keys(k, 65)          # tokens 0..64: block 1 holds token 64 only
    assert kt.shape == (2, 4)
    assert np.array_equal(kt[1], k[64])
    kt = O.compressed_keys(k, 100)         # block 1 = tokens 64..99, tokens >= T ignored
    assert np.allclose(kt[1], k[64:100].sum(0) / 36, atol=1e-14)


def test_incremental_update_matches_bulk():
    r = rng(4)
    d = 5
    k = r.standard_normal((300, d))
    kt = np.zeros((0, d))
    for T in range(0, 300):
        kt = O.append_token(kt, T, k[T])
        if T + 1 in (1, 2, 63, 64, 65, 128, 129, 200, 300):
            bulk = O.compressed_keys(k, T + 1)
            assert kt.shape == bulk.shape
            assert np.allclose(kt, bulk, rtol=0, atol=1e-12)


# ---------------------------------------------------------------------------
# selection
# ---------------------------------------------------------------------------

def test_init_local_hand_cases():
    # nb = 1, 2, 3 with one initial and two local blocks: they overlap and
    # every block is fixed, so nothing is left to score
    assert O.init_local(1, 1, 2) == ({0}, {0})
    assert O.init_local(2, 1, 2) == ({0}, {0, 1})
    assert O.init_local(3, 1, 2) == ({0}, {1, 2})
    for nb in (1, 2, 3):
        assert O.candidates(nb, 1, 2).size == 0
        assert list(O.block_set(nb, 1, 2, [])) == list(range(nb))
    assert list(O.candidates(6, 1, 2)) == [1, 2, 3]
    assert list(O.candidates(6, 0, 0)) == list(range(6))


def test_top_k_brute_force_small():
    # exhaustive: the chosen set is the k-subset of candidates with the
    # largest total score (scores distinct), for every k
    r = rng(5)
    for trial in range(30):
        nb = int(r.integers(4, 12))
        n_init, n_local = int(r.integers(0, 3)), int(r.integers(0, 3))
        s = r.standard_normal(nb)
        cand = O.candidates(nb, n_init, n_local)
        for k in range(0, len(cand) + 2):
            got = set(O.top_k(s, cand, k).tolist())
            kk = min(k, len(cand))
            best = max(itertools.combinations(cand.tolist(), kk),
                       key=lambda sub: sum(s[j] for j in sub)) if kk else ()
            assert got == set(best), (trial, k)
            bs = O.block_set(nb, n_init, n_local, list(got))
            assert list(bs) == sorted(set(bs))       # ascending, no repeats
            fixed = set(range(min(n_init, nb))) | set(range(max(0, nb - n_local), nb))
            assert set(bs) == fixed | set(best)


def test_top_k_certificate_and_counts():
    r = rng(6)
    nb, k = 2048, 32
    s = r.standard_normal(nb)
    cand = O.candidates(nb, 1, 2)
    chosen = O.top_k(s, cand, k)
    rest = np.setdiff1d(cand, chosen)
    assert len(chosen) == k
    assert s[chosen].min() > s[rest].max()
    assert len(O.block_set(nb, 1, 2, chosen)) == 35


def test_top_k_ties_go_to_lower_index():
    s = np.zeros(10)
    s[[7, 8]] = 1.0                          # two clear winners, then a flat tie
    cand = O.candidates(10, 1, 2)            # 1..7
    got = O.top_k(s, cand, 4)
    assert list(got) == [7, 1, 2, 3]
    assert list(O.top_k(np.zeros(10), cand, 3)) == [1, 2, 3]


def test_select_all_and_none():
    r = rng(7)
    kt = r.standard_normal((20, 8))
    f = r.standard_normal(8)
    blocks, _ = O.select_row(f, kt, 1, 2, 100)       # k >= |Cand|: every block
    assert list(blocks) == list(range(20))
    blocks, _ = O.select_row(f, kt, 1, 2, 0)         # k = 0: fixed blocks only
    assert list(blocks) == [0, 18, 19]


def test_indexer_scores_orientation():
    # a block whose pooled key points along f must win; one pointing against
    # it must lose (catches a sign flip or a transposed product)
    r = rng(8)
    d, nb = 16, 40
    kt = r.standard_normal((nb, d)) * 0.01
    f = r.standard_normal(d)
    kt[17] = f
    kt[23] = -f
    blocks, s = O.select_row(f, kt, 0, 0, 1)
    assert list(blocks) == [17]
    assert int(np.argmin(s)) == 23


def test_cut_gap():
    s = np.array([0.0, 5.0, 4.0, 3.0, 1.0])
    cand = np.array([1, 2, 3, 4])
    assert O.cut_gap(s, cand, 2) == 1.0
    assert O.cut_gap(s, cand, 4) == np.inf


# ---------------------------------------------------------------------------
# attention over the selected blocks
# ---------------------------------------------------------------------------

def _sdpa(q, k, v, scale):
    # torch's reference attention on the CPU in float64
    qt = torch.from_numpy(q)[None, None, None, :]
    kt = torch.from_numpy(k)[None, None]
    vt = torch.from_numpy(v)[None, None]
    return torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=scale)[0, 0, 0].numpy()


def test_attend_all_blocks_equals_dense_sdpa():
    r = rng(9)
    for T in (64, 100, 640, 1000):
        d = 32
        k = r.standard_normal((T + 7, d))
        v = r.standard_normal((T + 7, d))
        q = r.standard_normal(d)
        nb = O.num_blocks(T)
        o, lse = O.attend(q, k, v, list(range(nb)), T, 1 / math.sqrt(d))
        want = _sdpa(q, k[:T], v[:T], 1 / math.sqrt(d))
        assert np.allclose(o, want, rtol=0, atol=1e-12)
        z = (k[:T] @ q) / math.sqrt(d)
        assert abs(lse - float(torch.logsumexp(torch.from_numpy(z), 0))) < 1e-10


def test_attend_selected_blocks_equals_sdpa_on_gathered_tokens():
    r = rng(10)
    T, d = 1000, 16
    k = r.standard_normal((T, d))
    v = r.standard_normal((T, d))
    q = r.standard_normal(d)
    blocks = [0, 3, 9, 15]                   # block 15 is the partial last one
    toks = [t for j in blocks for t in range(64 * j, min(64 * j + 64, T))]
    o, _ = O.attend(q, k, v, blocks, T, 0.3)
    assert np.allclose(o, _sdpa(q, k[toks], v[toks], 0.3), rtol=0, atol=1e-12)


def test_attend_closed_forms():
    r = rng(11)
    T, d = 300, 8
    k = r.standard_normal((T, d))
    v = r.standard_normal((T, d))
    # q = 0: uniform weights, the output is the mean of V over the selected tokens
    o, lse = O.attend(np.zeros(d), k, v, [1, 4], T, 0.125)
    toks = list(range(64, 128)) + list(range(256, 300))
    assert np.allclose(o, v[toks].mean(0), atol=1e-13)
    assert abs(lse - math.log(len(toks))) < 1e-12
    # a single token: the output is that token's value
    o, lse = O.attend(r.standard_normal(d), k, v, [0], 1, 1.0)
    assert np.array_equal(o, v[0])


def test_attend_single_block_plain_python_softmax():
    r = rng(12)
    d = 4
    k = r.standard_normal((64, d))
    v = r.standard_normal((64, d))
    q = r.standard_normal(d)
    scale = 0.7
    z = [scale * sum(q[i] * k[t][i] for i in range(d)) for t in range(64)]
    w = [math.exp(x) for x in z]
    tot = sum(w)
    want = [sum(w[t] * v[t][i] for t in range(64)) / tot for i in range(d)]
    o, _ = O.attend(q, k, v, [0], 64, scale)
    assert np.allclose(o, want, rtol=0, atol=1e-13)


def test_decode_row_heads_independent():
    r = rng(13)
    T, d, G = 256, 8, 4
    k = r.standard_normal((T, d))
    v = r.standard_normal((T, d))
    qh = r.standard_normal((G, d))
    out, _ = O.decode_row(qh, k, v, [0, 2], T, 0.5)
    for h in range(G):
        toks = list(range(0, 64)) + list(range(128, 192))
        assert np.allclose(out[h], _sdpa(qh[h], k[toks], v[toks], 0.5), atol=1e-12)


# ---------------------------------------------------------------------------
# grouped verification (SSV)
# ---------------------------------------------------------------------------

def test_ssv_worked_example_union():
    g = json.load(open(os.path.join(HERE, "golden", "ssv_worked_example.json")))
    lists = g["queries"]
    counts = O.load_counts(lists)
    for blk, n in g["printed_load_counts"].items():
        assert counts[int(blk)] == n
    u = O.union_blocks(lists)
    assert list(u) == [3, 4, 7, 8, 12, 13, 19, 20, 21, 22]
    assert sum(counts.values()) == 16 and len(u) == 10


def test_union_formula_printed_values():
    g = json.load(open(os.path.join(HERE, "golden", "ssv_worked_example.json")))
    for case in g["printed_saving"]:
        s = O.saving_formula(case["C"], case["gamma"])
        assert abs(s - case["saving"]) < 1e-12
        assert abs(1 - s - case["remaining"]) < 1e-12
        # the saving is 1 - |merged| / (n C)
        n = 16
        assert abs(1 - O.union_size_formula(n, case["C"], case["gamma"]) / (n * case["C"]) - s) < 1e-12


@pytest.mark.parametrize("gamma,want", [(0.5, 40), (0.75, 28), (0.875, 22)])
def test_union_size_on_chain_constructed_sets(gamma, want):
    # query c+1 keeps gamma*n of query c's blocks and adds (1-gamma)*n blocks
    # new to the group: the merged size is exactly n(1 + (C-1)(1-gamma))
    n, C = 16, 4
    keep = int(round(gamma * n))
    r = rng(14)
    fresh = iter(r.permutation(1000)[:200].tolist())
    lists = [sorted(next(fresh) for _ in range(n))]
    for c in range(1, C):
        kept = r.choice(lists[-1], size=keep, replace=False).tolist()
        lists.append(sorted(kept + [next(fresh) for _ in range(n - keep)]))
    assert len(O.union_blocks(lists)) == want == O.union_size_formula(n, C, gamma)


def test_grouped_modes():
    r = rng(15)
    T, d, G, C = 640, 8, 2, 3
    k = r.standard_normal((T, d))
    v = r.standard_normal((T, d))
    q = r.standard_normal((C, G, d))
    lists = [[0, 3, 7], [0, 4, 7, 9], [2, 3]]
    out_a, _, ua = O.grouped_row(q, k, v, lists, T, 0.4, O.MODE_EXACT)
    assert ua == len({0, 2, 3, 4, 7, 9})
    for c in range(C):                       # mode A is per-query attention
        for h in range(G):
            toks = [t for j in lists[c] for t in range(64 * j, 64 * j + 64)]
            assert np.allclose(out_a[c, h], _sdpa(q[c, h], k[toks], v[toks], 0.4), atol=1e-12)
    out_b, _, ub = O.grouped_row(q, k, v, lists, T, 0.4, O.MODE_SHARED_REP)
    assert ub == 3
    toks = [t for j in lists[0] for t in range(64 * j, 64 * j + 64)]
    for c in range(C):                       # mode B: everyone uses the first query's list
        assert np.allclose(out_b[c, 0], _sdpa(q[c, 0], k[toks], v[toks], 0.4), atol=1e-12)
    same = [lists[1]] * C                    # identical lists: the two modes agree
    a, _, _ = O.grouped_row(q, k, v, same, T, 0.4, O.MODE_EXACT)
    b, _, _ = O.grouped_row(q, k, v, same, T, 0.4, O.MODE_SHARED_REP)
    assert np.array_equal(a, b)
    assert O.groups(10, 4) == [[0, 1, 2, 3], [4, 5, 6, 7], [8, 9]]


# ---------------------------------------------------------------------------
# G-head comparator
# ---------------------------------------------------------------------------

def test_multihead_one_head_ranks_like_the_indexer():
    # softmax over blocks is monotone, so with one head the ranking (and the
    # chosen set) equals that of the raw dot product
    r = rng(16)
    nb, d = 300, 32
    kt = r.standard_normal((nb, d)) / 8
    f = r.standard_normal(d)
    a, _ = O.select_row(f, kt, 1, 2, 20)
    b, _ = O.select_row_multihead(f[None, :], kt, 1, 2, 20, math.sqrt(d))
    assert np.array_equal(a, b)


def test_multihead_scores_sum_and_symmetry():
    r = rng(17)
    nb, d, G = 50, 16, 4
    kt = r.standard_normal((nb, d))
    q = r.standard_normal((G, d))
    s = O.multihead_scores(q, kt, 4.0)
    assert abs(s.sum() - G) < 1e-12                      # each head's softmax sums to 1
    assert np.allclose(O.multihead_scores(q[::-1], kt, 4.0), s, atol=1e-15)
    # against torch's softmax, head by head
    want = torch.softmax(torch.from_numpy(q @ kt.T / 4.0), dim=1).sum(0).numpy()
    assert np.allclose(s, want, atol=1e-14)
