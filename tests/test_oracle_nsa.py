"""Pins of the oracle's NSA three-branch output (CPU).

[SSV]'s NSA derivation gives the three branches (compressed keys and values,
the selected blocks, the last w tokens) and their gated sum; the verification
kernel outputs that sum per draft query.  The pins reduce each branch to a
case with an independent answer: torch SDPA on gathered tokens, the dense
result when a branch covers every token, kernel = stride = 1 compression
(the compressed cache is the cache itself), closed forms at q = 0, and a
plain-Python softmax on a tiny case.
"""
import math

import numpy as np
import pytest
import torch

import oracle as O


def _sdpa(q, k, v, scale=None):
    qt = torch.as_tensor(q, dtype=torch.float64)[None, None, None]
    kt = torch.as_tensor(k, dtype=torch.float64)[None, None]
    vt = torch.as_tensor(v, dtype=torch.float64)[None, None]
    return torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=scale)[0, 0, 0].numpy()


def _data(T, d, G=2, seed=0):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((G, d)), rng.standard_normal((T, d)), rng.standard_normal((T, d)))


def test_window_tokens_hand_cases():
    assert list(O.window_tokens(100, 64)) == list(range(36, 100))
    assert list(O.window_tokens(10, 64)) == list(range(10))
    assert list(O.window_tokens(128, 128)) == list(range(128))
    assert O.window_tokens(50, 0).size == 0


def test_attend_tokens_matches_sdpa_on_gathered_tokens():
    q, k, v = _data(300, 16)
    tok = np.array([3, 17, 64, 65, 199, 250, 299])
    o, lse = O.attend_tokens(q[0], k, v, tok, 0.25)
    assert np.allclose(o, _sdpa(q[0], k[tok], v[tok], scale=0.25), atol=1e-12)
    z = (k[tok] @ q[0]) * 0.25
    assert abs(lse - float(torch.logsumexp(torch.as_tensor(z), 0))) < 1e-12
    o0, l0 = O.attend_tokens(q[0], k, v, [], 0.25)
    assert np.all(o0 == 0) and l0 == -np.inf


def test_selection_only_gates_equal_block_decode():
    q, k, v = _data(640, 16)
    blocks = [0, 3, 7, 9]
    gates = np.tile([0.0, 1.0, 0.0], (2, 1))
    kc = O.compressed_keys(k, 640)
    vc = O.compressed_keys(v, 640)
    out, _, _ = O.nsa_row(q, k, v, kc, vc, blocks, 640, 10, 128, gates, 0.25)
    want, _ = O.decode_row(q, k, v, blocks, 640, 0.25)
    assert np.allclose(out, want, atol=1e-12)


@pytest.mark.parametrize("T", [640, 601, 37])
def test_window_branch_covering_everything_is_dense_attention(T):
    q, k, v = _data(T, 16, seed=T)
    gates = np.tile([0.0, 0.0, 1.0], (2, 1))
    kc = O.compressed_keys(k, T)
    out, _, _ = O.nsa_row(q, k, v, kc, kc, [0], T, kc.shape[0], 4096, gates, 1 / math.sqrt(16))
    for h in range(2):
        assert np.allclose(out[h], _sdpa(q[h], k[:T], v[:T]), atol=1e-12)


def test_aligned_window_equals_decode_over_last_blocks():
    q, k, v = _data(640, 16, seed=3)
    gates = np.tile([0.0, 0.0, 1.0], (2, 1))
    kc = O.compressed_keys(k, 640)
    out, _, _ = O.nsa_row(q, k, v, kc, kc, [0], 640, 10, 192, gates, 0.25)
    want, _ = O.decode_row(q, k, v, [7, 8, 9], 640, 0.25)
    assert np.allclose(out, want, atol=1e-12)


def test_compressed_branch_with_unit_windows_is_dense_attention():
    # kernel = stride = 1: every compressed entry is one token, so the
    # compressed branch attends to the whole cache
    T = 333
    q, k, v = _data(T, 16, seed=5)
    kc = O.compressed_keys_strided(k, T, 1, 1)
    vc = O.compressed_keys_strided(v, T, 1, 1)
    assert np.array_equal(kc, k) and np.array_equal(vc, v)
    gates = np.tile([1.0, 0.0, 0.0], (2, 1))
    out, _, _ = O.nsa_row(q, k, v, kc, vc, [0], T, T, 64, gates, 0.2)
    for h in range(2):
        assert np.allclose(out[h], _sdpa(q[h], k, v, scale=0.2), atol=1e-12)


def test_zero_query_closed_forms():
    # q = 0: every branch is the plain mean of its values
    T, d = 700, 8
    _, k, v = _data(T, d, seed=9)
    q = np.zeros((1, d))
    kc = O.compressed_keys_strided(k, T, 32, 16)
    vc = O.compressed_keys_strided(v, T, 32, 16)
    n_cmp = O.num_entries(T, 16)
    blocks = [0, 4, 10]
    gates = np.array([[0.5, 0.25, 0.125]])
    out, br, _ = O.nsa_row(q, k, v, kc, vc, blocks, T, n_cmp, 100, gates, 0.3)
    sel = np.concatenate([np.arange(0, 64), np.arange(256, 320), np.arange(640, 700)])
    assert np.allclose(br[0, 0], vc.mean(axis=0), atol=1e-12)
    assert np.allclose(br[1, 0], v[sel].mean(axis=0), atol=1e-12)
    assert np.allclose(br[2, 0], v[600:700].mean(axis=0), atol=1e-12)
    assert np.allclose(out[0], 0.5 * vc.mean(0) + 0.25 * v[sel].mean(0) + 0.125 * v[600:700].mean(0), atol=1e-12)


def test_tiny_case_plain_python():
    # one head, d = 2, five tokens, explicit exponentials
    k = np.array([[1.0, 0.0], [0.0, 1.0], [1.0, 1.0], [-1.0, 0.5], [0.25, -2.0]])
    v = np.array([[1.0, 2.0], [3.0, -1.0], [0.0, 0.5], [2.0, 2.0], [-1.0, 4.0]])
    q = np.array([[0.5, -1.0]])
    kc = np.array([[0.5, 0.5], [0.0, 0.75]])          # any compressed cache of two entries
    vc = np.array([[2.0, 0.5], [1.0, 1.0]])
    s = 0.7

    def soft(qv, ks, vs):
        w = [math.exp(s * (qv[0] * kk[0] + qv[1] * kk[1])) for kk in ks]
        tot = sum(w)
        return [sum(w[i] * vs[i][c] for i in range(len(ks))) / tot for c in range(2)]
    # the selection branch sees block 0 = all five tokens; window of 2 = tokens 3, 4
    oc = soft(q[0], kc, vc)
    os_ = soft(q[0], k, v)
    ow = soft(q[0], k[3:], v[3:])
    g = np.array([[0.2, 0.3, 0.5]])
    out, _, _ = O.nsa_row(q, k, v, kc, vc, [0], 5, 2, 2, g, s)
    want = [0.2 * oc[c] + 0.3 * os_[c] + 0.5 * ow[c] for c in range(2)]
    assert np.allclose(out[0], want, atol=1e-12)


def test_grouped_nsa_modes():
    T, d, C = 1024, 8, 3
    rng = np.random.default_rng(21)
    k, v = rng.standard_normal((T, d)), rng.standard_normal((T, d))
    q = rng.standard_normal((C, 2, d))
    g = rng.uniform(0, 1, (C, 2, 3))
    kc, vc = O.compressed_keys(k, T), O.compressed_keys(v, T)
    lists = [[0, 2, 5, 15], [0, 3, 5, 15], [1, 2, 14, 15]]
    outA, uA = O.grouped_nsa_row(q, k, v, kc, vc, lists, T, 16, 100, g, 0.3, O.MODE_EXACT)
    outB, uB = O.grouped_nsa_row(q, k, v, kc, vc, lists, T, 16, 100, g, 0.3, O.MODE_SHARED_REP)
    assert uA == 7 and uB == 4
    for c in range(C):
        assert np.allclose(outA[c], O.nsa_row(q[c], k, v, kc, vc, lists[c], T, 16, 100, g[c], 0.3)[0])
        assert np.allclose(outB[c], O.nsa_row(q[c], k, v, kc, vc, lists[0], T, 16, 100, g[c], 0.3)[0])
    same = [lists[0]] * C
    a, _ = O.grouped_nsa_row(q, k, v, kc, vc, same, T, 16, 100, g, 0.3, O.MODE_EXACT)
    b, _ = O.grouped_nsa_row(q, k, v, kc, vc, same, T, 16, 100, g, 0.3, O.MODE_SHARED_REP)
    assert np.array_equal(a, b)
