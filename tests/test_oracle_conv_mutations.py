"""Planted mistakes in the two-tap convolution oracle (CPU, monkeypatch) must
each fail a convolution pin: swapped taps, the correction indexed by c mod 16
instead of c // 16, a left tap that wraps around the block, the correction
computed from the previous row, and the sites permuted in the layer."""
import numpy as np

import oracle.dflash2 as ds
from tests import test_oracle_conv as pins

_orig = ds.two_tap_conv


def _fails(fn):
    try:
        fn()
    except AssertionError:
        return True
    return False


ALL = [getattr(pins, n) for n in dir(pins) if n.startswith("test_")]


def test_unmutated_pins_pass():
    assert not any(_fails(t) for t in ALL)


def _conv(x, w, kbase, *, swap=False, tile=False, wrap=False, prev_corr=False):
    x = np.asarray(x, np.float64)
    B, D = x.shape
    G = D // 16
    w = np.asarray(w, np.float64)
    kbase = np.asarray(kbase, np.float64)
    if swap:
        w = np.concatenate([w[G:], w[:G]])
        kbase = kbase[::-1]
    left = np.roll(x, 1, axis=0) if wrap else np.concatenate([np.zeros((1, D)), x[:-1]])
    z = (left if prev_corr else x) @ w.T
    rep = (lambda a: np.tile(a, (1, 16))) if tile else (lambda a: np.repeat(a, 16, axis=1))
    return (kbase[0][None] + rep(z[:, :G])) * x + (kbase[1][None] + rep(z[:, G:])) * left


def test_mutation_model_matches_the_oracle():
    rng = np.random.Generator(np.random.PCG64(9))
    x, w, kb = rng.standard_normal((5, 32)), rng.standard_normal((4, 32)), rng.standard_normal((2, 32))
    assert np.allclose(_conv(x, w, kb), _orig(x, w, kb), atol=1e-12)


def test_swapped_taps_caught(monkeypatch):
    monkeypatch.setattr(ds, "two_tap_conv", lambda x, w, k: _conv(x, w, k, swap=True))
    assert _fails(pins.test_correction_grouping_tap_roles_and_source_row)


def test_channel_mod_16_caught(monkeypatch):
    monkeypatch.setattr(ds, "two_tap_conv", lambda x, w, k: _conv(x, w, k, tile=True))
    assert _fails(pins.test_correction_grouping_tap_roles_and_source_row)


def test_wraparound_left_tap_caught(monkeypatch):
    monkeypatch.setattr(ds, "two_tap_conv", lambda x, w, k: _conv(x, w, k, wrap=True))
    assert _fails(pins.test_block_boundary_and_locality_by_brute_force)
    assert _fails(pins.test_static_taps_equal_numpy_convolve)


def test_correction_from_previous_row_caught(monkeypatch):
    monkeypatch.setattr(ds, "two_tap_conv", lambda x, w, k: _conv(x, w, k, prev_corr=True))
    assert _fails(pins.test_correction_grouping_tap_roles_and_source_row)


def test_permuted_sites_caught(monkeypatch):
    monkeypatch.setattr(ds, "CONV_SITES", ("attn_out", "attn_in", "ffn_out", "ffn_in"))
    assert _fails(pins.test_sites_sit_around_attention_and_ffn)
