"""Seeded inputs: determinism and the stated distributions (CPU)."""
import dataclasses

import numpy as np

import synth
from synth import inputs


def test_draws_are_reproducible_and_distinct():
    c = synth.get_config(1)
    K1, V1, _ = inputs.kv_layer(c, 0)
    K2, V2, _ = inputs.kv_layer(c, 0)
    assert K1.equal(K2) and V1.equal(V2)
    assert not K1.equal(V1)
    K3, _, _ = inputs.kv_layer(c, 1)
    assert not K1.equal(K3)
    F1 = inputs.indexer_vectors(c, 0)
    assert np.array_equal(F1, inputs.indexer_vectors(c, 0))
    assert abs(float(K1.float().std()) - 1.0) < 0.02


def test_redraw_changes_only_that_row():
    c = dataclasses.replace(synth.get_config(2), B=2, H_kv=3)
    att = np.zeros((2, 1, 3), dtype=int)
    F0 = inputs.indexer_vectors(c, 0, att)
    att[1, 0, 2] = 1
    F1 = inputs.indexer_vectors(c, 0, att)
    diff = np.abs(F1 - F0).reshape(6, -1).max(1)
    assert diff[5] > 0 and np.all(diff[:5] == 0)


def test_bias_blocks_count_and_range():
    c = dataclasses.replace(synth.get_config(2), B=2, H_kv=2, T=64 * 100)
    m = inputs.biased_block_mask(c, 0)
    assert m.shape == (2, 2, 100)
    assert np.all(m.sum(-1) == 5)
    assert not m[..., 0].any() and not m[..., -2:].any()


def test_config_byte_counts():
    c3 = synth.get_config(3)
    assert c3.n_sel == 35 and c3.NB == 2048
    assert c3.selected_kv_bytes() == 73_400_320
    assert c3.ktilde_bytes() == 33_554_432
    assert synth.get_config(1).selected_kv_bytes() == 360_448


def test_prefill_indexer_vectors_are_a_stationary_correlated_sequence():
    import synth
    from synth import inputs
    cfg = synth.get_config(1)
    F = inputs.prefill_indexer_vectors(cfg, 0, 4000)
    assert F.shape == (1, 4000, 2, 64)
    assert abs(F.std() * np.sqrt(cfg.d) - 1.0) < 0.05
    r = np.mean([np.corrcoef(F[0, :-1, g, i], F[0, 1:, g, i])[0, 1] for g in range(2) for i in range(64)])
    assert abs(r - inputs.PREFILL_RHO) < 0.01
    tail = inputs.prefill_indexer_vectors(cfg, 0, 500, pos0=3500)
    assert np.array_equal(tail, F[:, 3500:])
