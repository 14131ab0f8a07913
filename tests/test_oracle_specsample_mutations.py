"""Planted mistakes in the speculative-sampling oracle (CPU, monkeypatch) must
each fail a pin: the acceptance ratio inverted, the replacement drawn from the
verifier's row instead of the residual, the verifier row shifted by one
offset, the Gumbel draw taken with the wrong sign, and the block of the
two-stage draw chosen without regard to the block masses."""
import numpy as np

import oracle.specsample as ss
from tests import test_oracle_specsample as pins


def _fails(fn, *args):
    try:
        fn(*args)
    except AssertionError:
        return True
    return False


def test_unmutated_pins_pass():
    assert not _fails(pins.test_first_token_distribution_equals_target, 5, 1)
    assert not _fails(pins.test_sampler_emits_the_verifier_distribution)


def test_inverted_ratio_caught(monkeypatch):
    monkeypatch.setattr(ss, "accepts", lambda r, q, p: r * p < q)
    assert _fails(pins.test_first_token_distribution_equals_target, 5, 1)


def test_replacement_from_verifier_row_caught(monkeypatch):
    monkeypatch.setattr(ss, "residual", lambda p, q: np.asarray(p, dtype=np.float64).copy())
    assert _fails(pins.test_first_token_distribution_equals_target, 5, 1)


def test_shifted_verifier_row_caught(monkeypatch):
    monkeypatch.setattr(ss, "verifier_row", lambda j: j)
    assert _fails(pins.test_sampler_emits_the_verifier_distribution)


def test_wrong_gumbel_sign_caught(monkeypatch):
    orig = ss.gumbel
    monkeypatch.setattr(ss, "gumbel", lambda u: -orig(u))
    assert _fails(pins.test_gumbel_draw_matches_softmax)


def test_block_choice_ignoring_masses_caught(monkeypatch):
    def uniform_block(w, u):
        nb = -(-len(w) // ss.BLOCK)
        return min(int(u * nb), nb - 1)
    monkeypatch.setattr(ss, "block_choice", uniform_block)
    assert _fails(pins.test_two_stage_draw_across_blocks)
