"""Pins of the oracle's overlapping compression and block max-pool (CPU).

The pages give the compression of eq. (4) with a general kernel l and stride
s, the inference setting l = 32, s = 16 ([SparDA] §4.4), and a max-pool of
the compressed scores onto the block grid ([SparDA] §4.3, fig. 3).  These
tests check the oracle against formulations written differently from it:
windows collected token by token, hand-derived spike cases, plain Python
sums, and brute-force subset search.
"""
import itertools

import numpy as np
import pytest

import oracle as O

SHAPES = [(32, 16), (64, 64), (16, 16), (64, 32), (32, 32), (48, 16)]


def _windows_by_token_scan(T, window, stride):
    """Member tokens of every window, found by asking of each token which
    windows hold it (a window starts at a multiple of the stride before T)."""
    members = {}
    for t in range(T):
        for j in range(0, T // stride + 2):
            if j * stride < T and j * stride <= t < j * stride + window:
                members.setdefault(j, []).append(t)
    return members


@pytest.mark.parametrize("window,stride", SHAPES)
@pytest.mark.parametrize("T", [1, 15, 16, 17, 63, 64, 100, 130, 200])
def test_strided_keys_match_token_scan(window, stride, T):
    rng = np.random.default_rng(T * 131 + window + stride)
    k = rng.standard_normal((T, 3))
    got = O.compressed_keys_strided(k, T, window, stride)
    members = _windows_by_token_scan(T, window, stride)
    assert got.shape[0] == len(members) == O.num_entries(T, stride)
    for j, toks in members.items():
        want = [sum(k[t, c] for t in toks) / len(toks) for c in range(3)]
        assert np.allclose(got[j], want, rtol=0, atol=1e-12)


def test_strided_keys_64_64_is_block_mean():
    rng = np.random.default_rng(5)
    k = rng.standard_normal((300, 8))
    assert np.array_equal(O.compressed_keys_strided(k, 300, 64, 64), O.compressed_keys(k, 300))


@pytest.mark.parametrize("window,stride", SHAPES)
@pytest.mark.parametrize("T", [1, 40, 64, 65, 128, 200, 320])
def test_pool_range_matches_token_scan(window, stride, T):
    members = _windows_by_token_scan(T, window, stride)
    n = len(members)
    for J in range(O.num_blocks(T)):
        block_toks = set(range(J * 64, min(J * 64 + 64, T)))
        want = sorted(j for j, toks in members.items() if block_toks & set(toks))
        lo, hi = O.pool_range(J, window, stride, n)
        assert list(range(lo, hi + 1)) == want


def _lifted_blocks(T, t_spike, window=32, stride=16):
    """Blocks whose pooled score rises when one key points along f."""
    k = np.zeros((T, 4))
    k[t_spike, 0] = 10.0
    f = np.array([1.0, 0.0, 0.0, 0.0])
    kt = O.compressed_keys_strided(k, T, window, stride)
    s = O.max_pool_blocks(O.indexer_scores(f, kt), T, window, stride)
    return sorted(int(j) for j in np.nonzero(s > 0)[0])


def test_pool_spike_cases_32_16():
    T = 640                                   # ten blocks of 64
    # windows are [16j, 16j + 32): a token in the middle of a block is held
    # only by windows inside that block
    assert _lifted_blocks(T, 3 * 64 + 20) == [3]
    assert _lifted_blocks(T, 3 * 64 + 40) == [3]
    # the last 16 tokens of block 3 are also in the window [240, 272), which
    # overlaps block 4; the first 16 tokens are also in [176, 208)
    assert _lifted_blocks(T, 3 * 64 + 60) == [3, 4]
    assert _lifted_blocks(T, 3 * 64 + 5) == [2, 3]
    assert _lifted_blocks(T, 0) == [0]
    assert _lifted_blocks(T, T - 1) == [9]
    # 64/64: a block's own window only
    assert _lifted_blocks(T, 3 * 64 + 60, 64, 64) == [3]
    assert _lifted_blocks(T, 3 * 64 + 5, 64, 64) == [3]


def test_pool_straddling_window_lifts_both_blocks_equally():
    T = 640
    k = np.zeros((T, 2))
    k[3 * 64 + 60, 0] = 8.0
    f = np.array([1.0, 0.0])
    kt = O.compressed_keys_strided(k, T, 32, 16)
    s = O.max_pool_blocks(O.indexer_scores(f, kt), T, 32, 16)
    # window 15 = [240, 272) holds the spike with 31 other zero keys: 8/32;
    # window 14 = [224, 256) too: block 3 sees max(8/32, 8/32), block 4 sees 8/32
    assert s[3] == s[4] == 8.0 / 32


def test_pooled_scores_are_window_means_of_token_dots():
    # f . K~_j = mean over the window's tokens of f . k_t (linearity), by
    # plain Python sums; the block score is the largest such mean over the
    # windows that share a token with the block
    rng = np.random.default_rng(11)
    T, d = 290, 5
    k = rng.standard_normal((T, d))
    f = rng.standard_normal(d)
    for window, stride in [(32, 16), (64, 32), (48, 16)]:
        s = O.max_pool_blocks(O.indexer_scores(f, O.compressed_keys_strided(k, T, window, stride)), T, window,
                              stride)
        members = _windows_by_token_scan(T, window, stride)
        for J in range(O.num_blocks(T)):
            bt = set(range(J * 64, min(J * 64 + 64, T)))
            best = None
            for toks in members.values():
                if bt & set(toks):
                    m = sum(sum(f[c] * k[t, c] for c in range(d)) for t in toks) / len(toks)
                    best = m if best is None else max(best, m)
            assert abs(s[J] - best) < 1e-12


def test_pooled_64_64_selection_equals_plain_selection():
    rng = np.random.default_rng(3)
    T, d = 64 * 40 - 17, 16
    k = rng.standard_normal((T, d))
    kt = O.store_bf16(O.compressed_keys(k, T))
    for seed in range(5):
        f = np.random.default_rng(seed).standard_normal(d)
        a, sa = O.select_row(f, kt, 1, 2, 6)
        b, sb = O.select_row_pooled(f, kt, T, 64, 64, 1, 2, 6)
        assert np.array_equal(a, b) and np.array_equal(sa, sb)


def test_pooled_selection_brute_force_small():
    # best-sum k-subset of the candidates under block scores built by the
    # token scan: the unique answer whenever the pooled scores have no ties
    rng = np.random.default_rng(17)
    T, d, window, stride = 64 * 9 + 23, 4, 32, 16
    k = rng.standard_normal((T, d))
    members = _windows_by_token_scan(T, window, stride)
    nb = O.num_blocks(T)
    for trial in range(4):
        f = rng.standard_normal(d)
        kt = O.compressed_keys_strided(k, T, window, stride)
        wmean = {j: float(np.mean([f @ k[t] for t in toks])) for j, toks in members.items()}
        bs = []
        for J in range(nb):
            bt = set(range(J * 64, min(J * 64 + 64, T)))
            bs.append(max(v for j, v in wmean.items() if bt & set(members[j])))
        bs = O.decision_scores(np.array(bs))
        for n_init, n_local, kk in [(1, 2, 3), (0, 0, 4), (2, 1, 2), (1, 1, 0)]:
            cand = [j for j in range(nb) if j >= n_init and j < nb - n_local]
            if len(set(bs[cand])) < len(cand):
                continue
            best = max(itertools.combinations(cand, min(kk, len(cand))), key=lambda c: sum(bs[list(c)]))
            want = sorted(set(range(min(n_init, nb))) | set(range(max(0, nb - n_local), nb)) | set(best))
            got, _ = O.select_row_pooled(f, kt, T, window, stride, n_init, n_local, kk)
            assert list(got) == want


# ---------------------------------------------------------------------------
# InfLLM-V2's G-head selector on overlapping compressed keys
# ---------------------------------------------------------------------------

def test_multihead_pooled_64_64_is_the_plain_comparator():
    rng = np.random.default_rng(21)
    T = 64 * 40 + 9
    k = rng.standard_normal((T, 16))
    kt = O.compressed_keys_strided(k, T, 64, 64)
    qh = rng.standard_normal((4, 16))
    a, sa = O.select_row_multihead_pooled(qh, kt, T, 64, 64, 1, 2, 5, 4.0)
    b, sb = O.select_row_multihead(qh, kt, 1, 2, 5, 4.0)
    assert list(a) == list(b) and np.array_equal(sa, sb)


def test_multihead_pooled_one_head_ranks_like_the_pooled_indexer():
    # one head: the entry softmax is a monotone map of the raw scores, and a
    # max commutes with a monotone map, so the block ranking is the indexer's
    rng = np.random.default_rng(22)
    T = 64 * 50
    k = rng.standard_normal((T, 16))
    kt = O.compressed_keys_strided(k, T, 32, 16)
    f = rng.standard_normal(16)
    a, _ = O.select_row_multihead_pooled(f[None], kt, T, 32, 16, 1, 2, 7, 3.0)
    b, _ = O.select_row_pooled(f, kt, T, 32, 16, 1, 2, 7)
    assert list(a) == list(b)


def test_multihead_pooled_block_scores_by_token_scan():
    # block score = the largest summed softmax weight among the windows that
    # hold one of the block's tokens; softmax written out with plain exp
    rng = np.random.default_rng(23)
    T, window, stride, d, G, tau = 64 * 6 + 30, 32, 16, 8, 3, 2.0
    k = rng.standard_normal((T, d))
    kt = O.compressed_keys_strided(k, T, window, stride)
    qh = rng.standard_normal((G, d))
    members = _windows_by_token_scan(T, window, stride)
    ssum = {}
    for h in range(G):
        z = {j: float(qh[h] @ kt[j]) / tau for j in members}
        zmax = max(z.values())
        tot = sum(np.exp(v - zmax) for v in z.values())
        for j in members:
            ssum[j] = ssum.get(j, 0.0) + np.exp(z[j] - zmax) / tot
    _, got = O.select_row_multihead_pooled(qh, kt, T, window, stride, 0, 1, 2, tau)
    for J in range(O.num_blocks(T)):
        toks = set(range(J * 64, min(J * 64 + 64, T)))
        want = max(ssum[j] for j, ts in members.items() if toks & set(ts))
        assert abs(got[J] - want) <= 1e-7 * max(1.0, want)
