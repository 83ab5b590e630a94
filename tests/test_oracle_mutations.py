"""Planted mistakes: each test swaps one oracle function for a plausibly wrong
version (on the CPU, in this process only) and checks that at least one pin
in test_oracle_pins.py then fails.  This is how the pins are shown to bind.
"""
import numpy as np
import pytest

import oracle
import oracle.sda_oracle as impl
from tests import test_oracle_pins as pins


def _patch(monkeypatch, name, fn):
    monkeypatch.setattr(impl, name, fn)
    monkeypatch.setattr(oracle, name, fn)


def _fails(*pin_fns):
    for fn in pin_fns:
        try:
            fn()
        except (AssertionError, IndexError, ValueError):
            return True
    return False


def _param_pin(fn, *args):
    return lambda: fn(*args)


@pytest.mark.parametrize("kind", ["truncate", "half_up", "via_float32", "seven_bits"])
def test_mutant_store_bf16(monkeypatch, kind):
    real = impl.store_bf16

    def bad(x):
        x = np.asarray(x, dtype=np.float64)
        _, e = np.frexp(x)
        e = np.maximum(e, -125)
        y = np.ldexp(x, 8 - e)
        if kind == "truncate":
            return np.ldexp(np.trunc(y), e - 8)
        if kind == "half_up":
            return np.ldexp(np.floor(np.abs(y) + 0.5) * np.sign(y), e - 8)
        if kind == "via_float32":          # double rounding through float32
            return real(x.astype(np.float32).astype(np.float64))
        return np.ldexp(np.rint(np.ldexp(x, 7 - e)), e - 7)
    _patch(monkeypatch, "store_bf16", bad)
    assert _fails(pins.test_store_bf16_hand_cases, pins.test_store_bf16_matches_torch_on_float32_values,
                  pins.test_store_bf16_nearest_brute_force)


def test_mutant_pool_divides_by_full_block(monkeypatch):
    def bad(k, T, block=64):
        nb = impl.num_blocks(T, block)
        return np.stack([k[j * block:min(j * block + block, T)].sum(0) / block for j in range(nb)])
    _patch(monkeypatch, "compressed_keys", bad)
    assert _fails(pins.test_compressed_keys_partial_last_block)


def test_mutant_pool_shifted_window(monkeypatch):
    def bad(k, T, block=64):
        nb = impl.num_blocks(T, block)
        return np.stack([k[j * block + 1:min(j * block + block + 1, T)].mean(0) for j in range(nb)])
    _patch(monkeypatch, "compressed_keys", bad)
    assert _fails(pins.test_compressed_keys_constant_block)


def test_mutant_incremental_wrong_count(monkeypatch):
    def bad(kt, T_old, k_new, block=64):
        nb_old = impl.num_blocks(T_old, block)
        if T_old % block == 0:
            out = np.zeros((nb_old + 1, k_new.shape[-1]))
            out[:nb_old] = kt[:nb_old]
            out[nb_old] = k_new
            return out
        n = T_old - (nb_old - 1) * block
        out = np.array(kt[:nb_old], copy=True)
        out[nb_old - 1] += (k_new - out[nb_old - 1]) / n          # should be n + 1
        return out
    _patch(monkeypatch, "append_token", bad)
    assert _fails(pins.test_incremental_update_matches_bulk)


def test_mutant_score_sign(monkeypatch):
    _patch(monkeypatch, "indexer_scores", lambda f, kt: -(kt @ f))
    assert _fails(pins.test_indexer_scores_orientation)


def test_mutant_top_k_smallest(monkeypatch):
    def bad(scores, cand, k):
        cand = np.asarray(cand)
        if k <= 0 or cand.size == 0:
            return np.zeros(0, dtype=np.int64)
        order = np.lexsort((cand, np.asarray(scores)[cand]))
        return cand[order[:k]]
    _patch(monkeypatch, "top_k", bad)
    assert _fails(pins.test_top_k_brute_force_small, pins.test_top_k_certificate_and_counts)


def test_mutant_tie_to_higher_index(monkeypatch):
    def bad(scores, cand, k):
        cand = np.asarray(cand)
        if k <= 0 or cand.size == 0:
            return np.zeros(0, dtype=np.int64)
        order = np.lexsort((-cand, -np.asarray(scores)[cand]))
        return cand[order[:k]]
    _patch(monkeypatch, "top_k", bad)
    assert _fails(pins.test_top_k_ties_go_to_lower_index)


def test_mutant_local_window_off_by_one(monkeypatch):
    def bad(nb, n_init, n_local):
        return set(range(min(n_init, nb))), set(range(max(0, nb - n_local - 1), nb - 1))
    _patch(monkeypatch, "init_local", bad)
    assert _fails(pins.test_init_local_hand_cases, pins.test_select_all_and_none)


def test_mutant_attention_without_scale(monkeypatch):
    real = impl.attend
    _patch(monkeypatch, "attend", lambda q, k, v, b, T, scale: real(q, k, v, b, T, 1.0))
    assert _fails(pins.test_attend_all_blocks_equals_dense_sdpa)


def test_mutant_attention_ignores_length(monkeypatch):
    def bad(blocks, T, block=64):
        return np.concatenate([np.arange(j * block, j * block + block) for j in blocks])
    _patch(monkeypatch, "block_tokens", bad)
    assert _fails(pins.test_attend_selected_blocks_equals_sdpa_on_gathered_tokens,
                  pins.test_attend_all_blocks_equals_dense_sdpa)


def test_mutant_attention_transposed_value(monkeypatch):
    def bad(q, k, v, blocks, T, scale):
        tok = impl.block_tokens(blocks, T)
        z = (k[tok] @ q) * scale
        p = np.exp(z - z.max())
        return (p @ k[tok]) / p.sum(), float(z.max() + np.log(p.sum()))     # K used as V
    _patch(monkeypatch, "attend", bad)
    assert _fails(pins.test_attend_closed_forms)


def test_mutant_softmax_over_heads(monkeypatch):
    def bad(q_heads, kt, tau):
        z = (q_heads @ kt.T) / tau
        e = np.exp(z - z.max(axis=0, keepdims=True))
        return (e / e.sum(axis=0, keepdims=True)).sum(0)             # normalised over heads
    _patch(monkeypatch, "multihead_scores", bad)
    assert _fails(pins.test_multihead_scores_sum_and_symmetry)


def test_mutant_mode_b_uses_last_query(monkeypatch):
    real = impl.grouped_row

    def bad(q_rows, k, v, lists, T, scale, mode):
        if mode == impl.MODE_SHARED_REP:
            lists = [lists[-1]] + list(lists[1:])
        return real(q_rows, k, v, lists, T, scale, mode)
    _patch(monkeypatch, "grouped_row", bad)
    assert _fails(pins.test_grouped_modes)


@pytest.mark.parametrize("gamma,want", [(0.75, 28)])
def test_mutant_union_formula_sign(monkeypatch, gamma, want):
    _patch(monkeypatch, "union_size_formula", lambda n, C, g: n * (1 + (C - 1) * g))
    assert _fails(pins.test_union_formula_printed_values,
                  _param_pin(pins.test_union_size_on_chain_constructed_sets, gamma, want))


# ---- overlapping compression and block max-pool -------------------------------
from tests import test_oracle_pooled as pooled  # noqa: E402


def _pool_pins():
    return [_param_pin(pooled.test_pool_range_matches_token_scan, w, s, T)
            for (w, s) in pooled.SHAPES for T in (40, 200, 320)] + \
           [pooled.test_pool_spike_cases_32_16, pooled.test_pooled_scores_are_window_means_of_token_dots,
            pooled.test_pool_straddling_window_lifts_both_blocks_equally]


@pytest.mark.parametrize("kind", ["contained", "starts_inside", "one_short", "no_clip"])
def test_mutant_pool_range(monkeypatch, kind):
    def bad(J, window, stride, n_entries, block=64):
        if kind == "contained":            # only windows inside the block
            lo, hi = -(-(J * block) // stride), ((J + 1) * block - window) // stride
        elif kind == "starts_inside":      # windows that start inside the block
            lo, hi = -(-(J * block) // stride), ((J + 1) * block - 1) // stride
        elif kind == "one_short":          # drops the last overlapping window
            lo, hi = max(0, -(-(J * block - window + 1) // stride)), ((J + 1) * block - 1) // stride - 1
        else:                              # windows past the sequence end kept
            lo, hi = max(0, -(-(J * block - window + 1) // stride)), ((J + 1) * block - 1) // stride
        return max(lo, 0), min(hi, n_entries + 3) if kind == "no_clip" else min(hi, n_entries - 1)
    _patch(monkeypatch, "pool_range", bad)
    assert _fails(*_pool_pins())


def test_mutant_pool_mean_not_max(monkeypatch):
    def bad(entry_scores, T, window, stride, block=64):
        e = np.asarray(entry_scores, dtype=np.float64)
        out = []
        for J in range(impl.num_blocks(T, block)):
            lo, hi = impl.pool_range(J, window, stride, e.size, block)
            out.append(e[lo:hi + 1].mean())
        return np.array(out)
    _patch(monkeypatch, "max_pool_blocks", bad)
    assert _fails(pooled.test_pool_straddling_window_lifts_both_blocks_equally,
                  pooled.test_pooled_scores_are_window_means_of_token_dots)


@pytest.mark.parametrize("kind", ["full_divisor", "floor_count", "stride_as_window"])
def test_mutant_strided_keys(monkeypatch, kind):
    def bad(k, T, window, stride):
        n = T // stride if kind == "floor_count" else -(-T // stride)
        w = stride if kind == "stride_as_window" else window
        out = []
        for j in range(n):
            lo, hi = j * stride, min(j * stride + w, T)
            out.append(k[lo:hi].sum(0) / (w if kind == "full_divisor" else hi - lo))
        return np.stack(out)
    _patch(monkeypatch, "compressed_keys_strided", bad)
    pins_ = [_param_pin(pooled.test_strided_keys_match_token_scan, w, s, T)
             for (w, s) in pooled.SHAPES for T in (17, 100, 130)]
    assert _fails(*pins_)


# ---- NSA three branches ----------------------------------------------------------
from tests import test_oracle_nsa as nsa  # noqa: E402


def _nsa_pins():
    return [nsa.test_window_tokens_hand_cases, nsa.test_selection_only_gates_equal_block_decode,
            _param_pin(nsa.test_window_branch_covering_everything_is_dense_attention, 601),
            nsa.test_aligned_window_equals_decode_over_last_blocks,
            nsa.test_compressed_branch_with_unit_windows_is_dense_attention, nsa.test_zero_query_closed_forms,
            nsa.test_tiny_case_plain_python]


@pytest.mark.parametrize("kind", ["one_short", "one_long"])
def test_mutant_window_tokens(monkeypatch, kind):
    def bad(T, window):
        lo = max(0, int(T) - int(window) + (1 if kind == "one_short" else -1))
        return np.arange(lo, int(T), dtype=np.int64)
    _patch(monkeypatch, "window_tokens", bad)
    assert _fails(*_nsa_pins())


@pytest.mark.parametrize("kind", ["gates_swapped", "cmp_one_short", "selection_on_window", "no_scale_cmp"])
def test_mutant_nsa_row(monkeypatch, kind):
    real_attend = impl.attend_tokens

    def bad(q_heads, k, v, kc, vc, blocks, T, n_cmp, window, gates, scale):
        G = q_heads.shape[0]
        sel_tok = impl.block_tokens(blocks, T)
        win_tok = impl.window_tokens(T, window)
        cmp_tok = np.arange(int(n_cmp) - (1 if kind == "cmp_one_short" else 0))
        if kind == "selection_on_window":
            sel_tok = win_tok
        out = np.zeros((G, k.shape[-1]))
        br = np.zeros((3, G, k.shape[-1]))
        lse = np.zeros((3, G))
        for h in range(G):
            for b, (kk, vv, tok) in enumerate(((kc, vc, cmp_tok), (k, v, sel_tok), (k, v, win_tok))):
                sc = 1.0 if (kind == "no_scale_cmp" and b == 0) else scale
                br[b, h], lse[b, h] = real_attend(q_heads[h], kk, vv, tok, sc)
            g = gates[h][::-1] if kind == "gates_swapped" else gates[h]
            out[h] = g[0] * br[0, h] + g[1] * br[1, h] + g[2] * br[2, h]
        return out, br, lse
    _patch(monkeypatch, "nsa_row", bad)
    assert _fails(*_nsa_pins())


# --- prefill -------------------------------------------------------------------
def _prefill_pins():
    from tests import test_oracle_prefill as pf
    return [pf.test_prefill_lengths_hand_cases, pf.test_dense_selection_is_causal_attention,
            pf.test_first_query_sees_only_token_zero,
            _param_pin(pf.test_selection_brute_force_every_position, 1, 2, 3),
            pf.test_each_query_matches_sdpa_on_its_gathered_causal_tokens, pf.test_nothing_after_a_query_matters,
            pf.test_chunked_prefill_equals_whole]


@pytest.mark.parametrize("shift", [-1, 1])
def test_mutant_prefill_lengths_off_by_one(monkeypatch, shift):
    def bad(pos0, nq):
        return np.arange(int(pos0) + 1 + shift, int(pos0) + int(nq) + 1 + shift, dtype=np.int64)
    _patch(monkeypatch, "prefill_lengths", bad)
    assert _fails(*_prefill_pins())


@pytest.mark.parametrize("kind", ["local_at_sequence_end", "all_blocks_scored", "pos0_ignored"])
def test_mutant_prefill_select(monkeypatch, kind):
    def bad(f_rows, kt_stored, pos0, n_init, n_local, k):
        out = []
        n_all = kt_stored.shape[0]
        for r in range(len(f_rows)):
            p = (0 if kind == "pos0_ignored" else pos0) + r
            nb = p // 64 + 1
            if kind == "local_at_sequence_end":
                blocks, _ = impl.select_row(f_rows[r], kt_stored, n_init, n_local, k)
                blocks = blocks[blocks < nb]
            elif kind == "all_blocks_scored":
                blocks, _ = impl.select_row(f_rows[r], kt_stored[:nb], n_init, 0, k)
                blocks = np.array(sorted(set(blocks) | set(range(max(0, nb - n_local), nb))))
            else:
                blocks, _ = impl.select_row(f_rows[r], kt_stored[:nb], n_init, n_local, k)
            assert n_all >= nb
            out.append(blocks)
        return out
    _patch(monkeypatch, "prefill_select_rows", bad)
    assert _fails(*_prefill_pins())


def test_mutant_prefill_not_causal(monkeypatch):
    def bad(q_rows, k, v, lists, pos0, scale):
        T = k.shape[0]
        outs, lses = [], []
        for r in range(len(q_rows)):
            o, l = impl.decode_row(q_rows[r], k, v, lists[r], T, scale)
            outs.append(o)
            lses.append(l)
        return np.stack(outs), np.stack(lses)
    _patch(monkeypatch, "prefill_rows", bad)
    assert _fails(*_prefill_pins())


@pytest.mark.parametrize("kind", ["sum_then_softmax", "mean_pool", "softmax_after_pool"])
def test_mutant_multihead_pooled(monkeypatch, kind):
    from tests import test_oracle_pooled as pp

    def bad(q_heads, kt_stored, T, window, stride, n_init, n_local, k, tau):
        if kind == "sum_then_softmax":             # raw head scores summed, one softmax
            z = (np.asarray(q_heads) @ kt_stored.T).sum(0) / tau
            e = np.exp(z - z.max())
            s_e = impl.decision_scores(e / e.sum())
            s = impl.max_pool_blocks(s_e, T, window, stride)
        elif kind == "mean_pool":
            s_e = impl.decision_scores(impl.multihead_scores(q_heads, kt_stored, tau))
            nb = impl.num_blocks(T)
            s = np.array([s_e[impl.pool_range(J, window, stride, s_e.size)[0]:
                              impl.pool_range(J, window, stride, s_e.size)[1] + 1].mean() for J in range(nb)])
        else:                                      # pool raw scores, softmax over blocks
            z = (np.asarray(q_heads) @ kt_stored.T) / tau
            pooled = np.stack([impl.max_pool_blocks(zh, T, window, stride) for zh in z])
            pooled = pooled - pooled.max(axis=1, keepdims=True)
            e = np.exp(pooled)
            s = impl.decision_scores((e / e.sum(axis=1, keepdims=True)).sum(0))
        nb = impl.num_blocks(T)
        cand = impl.candidates(nb, n_init, n_local)
        return impl.block_set(nb, n_init, n_local, impl.top_k(s, cand, k)), s
    _patch(monkeypatch, "select_row_multihead_pooled", bad)
    assert _fails(pp.test_multihead_pooled_64_64_is_the_plain_comparator,
                  pp.test_multihead_pooled_block_scores_by_token_scan)
