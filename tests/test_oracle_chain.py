"""Pins of the oracle's refresh/reuse layer chain (CPU).

[SSV] core mechanism 2: a refresh layer routes (selects blocks) and caches
the selection; a reuse layer skips routing and inherits the cache of the
latest refresh layer; the chain's time is R T_refresh + (L - R) T_reuse.
Pins: hand schedules, r = 1 routing every layer itself, each reuse layer
holding exactly its latest refresh layer's lists (found by scanning back),
a chain whose first layer reuses refused, and the time formula against its
own saving form (L T_refresh minus (L - R)(T_refresh - T_reuse)).
"""
import numpy as np
import pytest

import oracle as O


def test_refresh_schedule_hand_cases():
    assert O.refresh_schedule(5, 1) == [True] * 5
    assert O.refresh_schedule(7, 3) == [True, False, False, True, False, False, True]
    assert O.refresh_schedule(4, 5) == [True, False, False, False]


def _route(j):
    return [np.array([j, 10 + j]), np.array([20 + j])]


@pytest.mark.parametrize("L,r", [(6, 1), (7, 3), (10, 5), (4, 4)])
def test_each_layer_holds_its_latest_refresh(L, r):
    sched = O.refresh_schedule(L, r)
    lists = O.chain_lists(sched, _route)
    for j in range(L):
        last = max(i for i in range(j + 1) if sched[i])
        assert all(np.array_equal(a, b) for a, b in zip(lists[j], _route(last)))
    if r == 1:
        assert all(all(np.array_equal(a, b) for a, b in zip(lists[j], _route(j))) for j in range(L))


def test_chain_must_start_with_a_refresh():
    with pytest.raises(ValueError):
        O.chain_lists([False, True], _route)


@pytest.mark.parametrize("L,r,tr,tu", [(15, 1, 60.0, 50.0), (15, 3, 60.0, 50.0), (15, 5, 71.5, 54.25)])
def test_chain_time_formula(L, r, tr, tu):
    sched = O.refresh_schedule(L, r)
    R = -(-L // r)
    assert sum(sched) == R
    assert O.chain_time(sched, tr, tu) == pytest.approx(L * tr - (L - R) * (tr - tu))
