"""Pins of the oracle's prefill (CPU).

[SparDA] eq. (3) makes the block set a function of the query position i
(init blocks, the local window next to i, top-k), and the complexity
section's eq. (13), (15), (16) count one selection and one top-k attention
per query token.  The pins reduce prefill to cases with an independent
answer: dense causal attention when top-k covers every block (torch SDPA
with a causal mask), torch SDPA on each query's gathered causal tokens,
brute force over all k-subsets of the complete blocks found by scanning
tokens, the first query attending only to token 0, invariance to everything
after a query's position, and a chunked prefill equal to the whole one.
"""
import itertools

import numpy as np
import pytest
import torch

import oracle as O

BLOCK = 64


def _data(T, d=16, G=2, seed=0):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((T, G, d)), rng.standard_normal((T, d)), rng.standard_normal((T, d)),
            rng.standard_normal((T, d)) / 4)


def test_prefill_lengths_hand_cases():
    assert list(O.prefill_lengths(0, 4)) == [1, 2, 3, 4]
    assert list(O.prefill_lengths(100, 3)) == [101, 102, 103]
    assert O.prefill_lengths(5, 0).size == 0


def test_dense_selection_is_causal_attention():
    # top-k larger than any query's candidate count: every query attends to
    # every token up to its position; torch SDPA with a causal mask
    T, scale = 330, 0.3
    q, k, v, f = _data(T)
    kt = O.compressed_keys(k, T)
    lists = O.prefill_select_rows(f, kt, 0, 1, 1, 100)
    out, lse = O.prefill_rows(q, k, v, lists, 0, scale)
    mask = torch.ones(T, T, dtype=torch.bool).tril()
    for h in range(q.shape[1]):
        qt = torch.as_tensor(q[:, h])[None, None]
        want = torch.nn.functional.scaled_dot_product_attention(
            qt, torch.as_tensor(k)[None, None], torch.as_tensor(v)[None, None], attn_mask=mask,
            scale=scale)[0, 0].numpy()
        assert np.allclose(out[:, h], want, atol=1e-12)
        z = (torch.as_tensor(q[:, h]) @ torch.as_tensor(k).T) * scale
        z = z.masked_fill(~mask, float("-inf"))
        assert np.allclose(lse[:, h], torch.logsumexp(z, 1).numpy(), atol=1e-12)


def test_first_query_sees_only_token_zero():
    q, k, v, f = _data(200)
    kt = O.compressed_keys(k, 200)
    lists = O.prefill_select_rows(f[:1], kt, 0, 1, 2, 4)
    assert list(lists[0]) == [0]
    out, _ = O.prefill_rows(q[:1], k, v, lists, 0, 0.5)
    assert np.allclose(out[0], v[0][None].repeat(q.shape[1], 0), atol=1e-14)


def _brute_select(f, kt, p, n_init, n_local, k):
    """Token scan: a block competes when all 64 of its tokens are at or
    before p, it is not one of the first n_init blocks and it is not among
    the n_local blocks ending with the one that holds p; the chosen set is
    the k-subset of largest score sum."""
    cur = p // BLOCK
    fixed = set(range(0, min(n_init, cur + 1))) | set(range(max(0, cur - n_local + 1), cur + 1))
    comp = [j for j in range(cur + 1) if all(t <= p for t in range(j * BLOCK, j * BLOCK + BLOCK))]
    cand = [j for j in comp if j not in fixed]
    s = {j: float(np.float32(kt[j] @ f)) for j in cand}
    kk = min(k, len(cand))
    best = max(itertools.combinations(cand, kk), key=lambda c: sum(s[j] for j in c)) if kk else ()
    return sorted(fixed | set(best))


@pytest.mark.parametrize("n_init,n_local,k", [(1, 1, 2), (1, 2, 3), (0, 1, 4), (2, 3, 1), (1, 1, 0)])
def test_selection_brute_force_every_position(n_init, n_local, k):
    T = 11 * BLOCK + 17
    _, kk, _, f = _data(T, seed=3 + k)
    kt = O.compressed_keys(kk, T)
    for pos0, nq in ((0, T), (300, 50)):
        lists = O.prefill_select_rows(f[pos0:pos0 + nq], kt, pos0, n_init, n_local, k)
        for r in range(0, nq, 7):
            assert list(lists[r]) == _brute_select(f[pos0 + r], kt, pos0 + r, n_init, n_local, k), (pos0, r)


def test_each_query_matches_sdpa_on_its_gathered_causal_tokens():
    T, scale = 700, 0.25
    q, k, v, f = _data(T, seed=9)
    kt = O.compressed_keys(k, T)
    lists = O.prefill_select_rows(f, kt, 0, 1, 2, 3)
    out, _ = O.prefill_rows(q, k, v, lists, 0, scale)
    for r in range(0, T, 37):
        tok = np.array([t for j in lists[r] for t in range(j * BLOCK, j * BLOCK + BLOCK) if t <= r])
        for h in range(q.shape[1]):
            want = torch.nn.functional.scaled_dot_product_attention(
                torch.as_tensor(q[r, h])[None, None, None], torch.as_tensor(k[tok])[None, None],
                torch.as_tensor(v[tok])[None, None], scale=scale)[0, 0, 0].numpy()
            assert np.allclose(out[r, h], want, atol=1e-12)


def test_nothing_after_a_query_matters():
    T = 500
    q, k, v, f = _data(T, seed=4)
    kt = O.compressed_keys(k, T)
    lists = O.prefill_select_rows(f, kt, 0, 1, 2, 3)
    out, _ = O.prefill_rows(q, k, v, lists, 0, 0.3)
    p = 321
    k2, v2, f2 = k.copy(), v.copy(), f.copy()
    k2[p + 1:] += 5.0
    v2[p + 1:] -= 3.0
    f2[:p] *= -1.0
    kt2 = O.compressed_keys(k2, T)
    lists2 = O.prefill_select_rows(f2, kt2, 0, 1, 2, 3)
    out2, _ = O.prefill_rows(q, k2, v2, lists2, 0, 0.3)
    assert list(lists2[p]) == list(lists[p])
    assert np.allclose(out2[p], out[p], atol=1e-14)


def test_chunked_prefill_equals_whole():
    T, a = 450, 193
    q, k, v, f = _data(T, seed=5)
    kt = O.compressed_keys(k, T)
    whole = O.prefill_select_rows(f, kt, 0, 1, 2, 2)
    parts = O.prefill_select_rows(f[:a], kt, 0, 1, 2, 2) + O.prefill_select_rows(f[a:], kt, a, 1, 2, 2)
    assert all(list(x) == list(y) for x, y in zip(whole, parts))
    o_w, _ = O.prefill_rows(q, k, v, whole, 0, 0.4)
    o_p = np.concatenate([O.prefill_rows(q[:a], k, v, whole[:a], 0, 0.4)[0],
                          O.prefill_rows(q[a:], k, v, whole[a:], a, 0.4)[0]])
    assert np.allclose(o_w, o_p, atol=1e-14)


def test_prefill_needs_a_local_block():
    _, k, _, f = _data(128)
    with pytest.raises(ValueError):
        O.prefill_select_rows(f, O.compressed_keys(k, 128), 0, 1, 0, 2)
