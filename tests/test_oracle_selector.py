"""Pins of the DFlash 2 path-selector oracle (oracle/dflash2.py): the reduction
to per-position argmax, the greedy walk checked by enumeration (and shown to
differ from the best whole path), the roles of the two embedding tables, the
gate, the anchor as the first predecessor, and tie order."""
import itertools

import numpy as np
import pytest

from oracle import dflash2 as ds

R, V, K, T = 8, 40, 4, 5


def _inputs(seed=0):
    rng = np.random.default_rng(seed)
    cand = np.stack([rng.permutation(V)[:K] for _ in range(T)])
    u = rng.standard_normal((T, K))
    A = rng.standard_normal((V, R))
    Bt = rng.standard_normal((V, R))
    g = ds.gate(rng.standard_normal((R, 6)), rng.standard_normal((T, 6)))
    return cand, u, A, Bt, g


def test_zero_pair_table_gives_per_position_argmax():
    cand, u, A, Bt, g = _inputs()
    path, _, _ = ds.select_path(3, cand, u, np.zeros_like(A), Bt, g)
    assert list(path) == [cand[t][int(np.argmax(u[t]))] for t in range(T)]


def test_walk_is_stepwise_argmax_by_enumeration():
    rng = np.random.default_rng(1)
    for _ in range(20):
        first = rng.standard_normal(K)
        tabs = [rng.standard_normal((K, K)) for _ in range(T - 1)]
        locally_greedy = []
        for p in itertools.product(range(K), repeat=T):
            ok = first[p[0]] == first.max() and all(
                tabs[t][p[t], p[t + 1]] == tabs[t][p[t]].max() for t in range(T - 1))
            if ok:
                locally_greedy.append(list(p))
        assert locally_greedy == [ds.walk(first, tabs)]


def test_walk_is_not_the_best_whole_path():
    first = np.array([1.0, 0.9])
    tabs = [np.array([[0.0, 0.0], [5.0, 0.0]])]
    assert ds.walk(first, tabs) == [0, 0]                       # greedy takes 1.0 then 0.0
    best = max(itertools.product(range(2), repeat=2), key=lambda p: first[p[0]] + tabs[0][p[0], p[1]])
    assert list(best) == [1, 0]                                 # the best sum is 0.9 + 5.0


def test_previous_token_reads_A_and_next_token_reads_B():
    cand, u, _, _, g = _inputs()
    x, y = int(cand[1][0]), int(cand[2][1])
    A = np.zeros((V, R))
    Bt = np.zeros((V, R))
    A[x] = 1.0
    Bt[y] = 1.0
    s = ds.pair_scores(u[2], cand[1], cand[2], A, Bt, g[2]) - u[2][None]
    assert s[0, 1] > 0                          # a = x (previous), b = y (next)
    assert np.count_nonzero(s) == 1
    s_rev = ds.pair_scores(u[2], np.array([y]), np.array([x]), A, Bt, g[2]) - u[2][:1][None]
    assert s_rev[0, 0] == 0                     # roles are not symmetric


def test_gate_range_and_closed_form_at_zero():
    h = np.random.default_rng(3).standard_normal((4, 6))
    g = ds.gate(np.random.default_rng(4).standard_normal((R, 6)), h)
    assert np.all((g > 0) & (g < 1))
    assert np.allclose(ds.gate(np.zeros((R, 6)), h), 0.5)


def test_closed_gate_channels_drop_out():
    cand, u, A, Bt, g = _inputs()
    g2 = g.copy()
    g2[2, :] = 0.0
    s = ds.pair_scores(u[2], cand[1], cand[2], A, Bt, g2[2])
    assert np.allclose(s, np.repeat(u[2][None], K, 0))


def test_first_position_scores_against_the_anchor():
    cand, u, _, _, g = _inputs()
    A = np.zeros((V, R))
    Bt = np.random.default_rng(5).standard_normal((V, R))
    anchor = int(np.setdiff1d(np.arange(V), cand.ravel())[0])
    A[anchor] = 3.0
    _, f_anchor, _ = ds.select_path(anchor, cand, u, A, Bt, g)
    other = int(np.setdiff1d(np.arange(V), np.concatenate([cand.ravel(), [anchor]]))[0])
    _, f_other, _ = ds.select_path(other, cand, u, A, Bt, g)
    assert np.allclose(f_other, u[0])
    assert not np.allclose(f_anchor, u[0])


def test_logit_shift_per_position_leaves_the_path():
    cand, u, A, Bt, g = _inputs()
    a, _, _ = ds.select_path(2, cand, u, A, Bt, g)
    b, _, _ = ds.select_path(2, cand, u + np.arange(T)[:, None] * 3.7, A, Bt, g)
    assert np.array_equal(a, b)


def test_ties_go_to_the_lower_rank():
    assert ds.walk(np.array([0.5, 0.5, 0.1]), [np.array([[1, 1, 0], [0, 2, 2], [0, 0, 0.0]])]) == [0, 0]
