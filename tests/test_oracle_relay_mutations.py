"""Planted mistakes in the relay oracle (on the CPU, via monkeypatch) must each
fail one of the relay pins: no shift, relaying the first rejection, swapped
beta/gamma halves, swapped token embeddings, LayerNorm dropped, RMSNorm of the
shared projection dropped."""
import numpy as np
import pytest

import oracle.dflow as ofl
import oracle.dflash as od
from tests import test_oracle_relay as pins

_orig_plan = ofl.relay_plan
_orig_inputs = ofl.relay_inputs
_orig_fuse = od.fuse_context


def _fails(fn):
    try:
        fn()
    except AssertionError:
        return True
    return False


def test_unmutated_pins_pass():
    for t in (pins.test_worked_example_shift, pins.test_gamma_is_additive_offset,
              pins.test_beta_scales_layer_normed_h, pins.test_bonus_and_first_rejection_enter_in_page_order,
              pins.test_layer_norm_moments_closed_form, pins.test_verifier_features_scale_invariant,
              pins.test_worked_example_next_round_start):
        t()
    pins.test_offsets_cover_next_block_from_two(16)


def test_missing_shift_caught(monkeypatch):
    def no_shift(anchor_pos, n, B):
        return [(o, t - 1, off - 1) for o, t, off in _orig_plan(anchor_pos, n, B)]
    monkeypatch.setattr(ofl, "relay_plan", no_shift)
    assert _fails(pins.test_worked_example_shift)


def test_relaying_first_rejection_caught(monkeypatch):
    def from_first_rejection(anchor_pos, n, B):
        nxt = anchor_pos + n + 1
        return [(o, anchor_pos + o + 1, anchor_pos + o + 1 - nxt) for o in range(n + 1, B)]
    monkeypatch.setattr(ofl, "relay_plan", from_first_rejection)
    assert _fails(lambda: pins.test_offsets_cover_next_block_from_two(16))


def _patched_inputs(swap_halves=False, swap_embed=False, no_ln=False):
    def f(w, d, rw, hidden, bonus, first_rejected):
        h = od.fuse_context(w["w_c"], w["g_c"], hidden, d.rms_eps)
        k = h.shape[0]
        a, b = (first_rejected, bonus) if swap_embed else (bonus, first_rejected)
        cond = np.concatenate([np.repeat(w["embed"][a][None], k, 0), np.repeat(w["embed"][b][None], k, 0), h], 1)
        bg = od.silu(cond @ rw["w1"].T) @ rw["w2"].T
        beta, gamma = bg[:, :d.D], bg[:, d.D:]
        if swap_halves:
            beta, gamma = gamma, beta
        ln = h if no_ln else ofl.layer_norm(h)
        return w["e_mask"][None] + beta * ln + gamma
    return f


def test_unpatched_rewrite_matches():
    d = pins._dims()
    w, rw = pins._weights(d)
    hid = pins._hidden(d, 3)
    assert np.allclose(_patched_inputs()(w, d, rw, hid, 3, 7), _orig_inputs(w, d, rw, hid, 3, 7), rtol=1e-12)


def test_swapped_beta_gamma_caught(monkeypatch):
    monkeypatch.setattr(ofl, "relay_inputs", _patched_inputs(swap_halves=True))
    assert _fails(pins.test_gamma_is_additive_offset) or _fails(pins.test_beta_scales_layer_normed_h)


def test_swapped_embeddings_caught(monkeypatch):
    monkeypatch.setattr(ofl, "relay_inputs", _patched_inputs(swap_embed=True))
    assert _fails(pins.test_bonus_and_first_rejection_enter_in_page_order)


def test_dropped_layer_norm_caught(monkeypatch):
    monkeypatch.setattr(ofl, "relay_inputs", _patched_inputs(no_ln=True))
    assert _fails(pins.test_beta_scales_layer_normed_h)


def test_dropped_rmsnorm_caught(monkeypatch):
    def no_rms(w_c, g_c, hidden, eps):
        return np.concatenate([np.asarray(h, np.float64) for h in hidden], 1) @ np.asarray(w_c, np.float64).T
    monkeypatch.setattr(od, "fuse_context", no_rms)
    monkeypatch.setattr(ofl, "fuse_context", no_rms)
    assert _fails(pins.test_verifier_features_scale_invariant) or _fails(pins.test_beta_scales_layer_normed_h)
