"""Planted mistakes in the selector oracle (CPU, monkeypatch) must each fail a
selector pin: swapped embedding roles, the gate ignored, the walk started
without the anchor, the best whole path instead of the greedy walk, the wrong
position's logits, and ties to the higher rank."""
import itertools

import numpy as np

import oracle.dflash2 as ds
from tests import test_oracle_selector as pins

_orig_pair = ds.pair_scores
_orig_walk = ds.walk
_orig_select = ds.select_path


def _fails(fn):
    try:
        fn()
    except AssertionError:
        return True
    return False


ALL = [getattr(pins, n) for n in dir(pins) if n.startswith("test_")]


def _any_fails():
    return any(_fails(t) for t in ALL)


def test_unmutated_pins_pass():
    assert not _any_fails()


def test_swapped_tables_caught(monkeypatch):
    monkeypatch.setattr(ds, "pair_scores", lambda u, p, i, A, Bt, g: _orig_pair(u, p, i, Bt, A, g))
    assert _fails(pins.test_previous_token_reads_A_and_next_token_reads_B)


def test_ignored_gate_caught(monkeypatch):
    monkeypatch.setattr(ds, "pair_scores", lambda u, p, i, A, Bt, g: _orig_pair(u, p, i, A, Bt, np.ones_like(g)))
    assert _fails(pins.test_closed_gate_channels_drop_out)


def test_walk_without_anchor_caught(monkeypatch):
    def no_anchor(anchor, cand, u, A, Bt, gates):
        return _orig_select(int(cand[0][0]), cand, u, A, Bt, gates)
    monkeypatch.setattr(ds, "select_path", no_anchor)
    assert _fails(pins.test_first_position_scores_against_the_anchor)


def test_global_best_path_caught(monkeypatch):
    def best(first, tabs):
        k, T = len(first), len(tabs) + 1
        return list(max(itertools.product(range(k), repeat=T),
                        key=lambda p: first[p[0]] + sum(tabs[t][p[t], p[t + 1]] for t in range(T - 1))))
    monkeypatch.setattr(ds, "walk", best)
    assert _fails(pins.test_walk_is_not_the_best_whole_path)


def test_previous_positions_logits_caught(monkeypatch):
    def shifted(anchor, cand, u, A, Bt, gates):
        return _orig_select(anchor, cand, np.roll(u, 1, axis=0), A, Bt, gates)
    monkeypatch.setattr(ds, "select_path", shifted)
    assert _fails(pins.test_zero_pair_table_gives_per_position_argmax)


def test_ties_to_higher_rank_caught(monkeypatch):
    def hi(first, tabs):
        path = [len(first) - 1 - int(np.argmax(first[::-1]))]
        for tab in tabs:
            row = tab[path[-1]]
            path.append(len(row) - 1 - int(np.argmax(row[::-1])))
        return path
    monkeypatch.setattr(ds, "walk", hi)
    assert _fails(pins.test_ties_go_to_the_lower_rank)
