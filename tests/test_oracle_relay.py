"""Pins of the DFlow relay oracle (oracle/dflow.py) against what the DFlow page
and the mathematics fix: the page's two worked examples, closed forms of
LayerNorm, the reduction to the plain mask embedding, and structural facts of
the modulation (beta scales LN(h), gamma is an additive offset, the two token
embeddings enter in the page's order)."""
import json
import os
from dataclasses import replace

import numpy as np
import pytest

import oracle
from oracle import dflow as ofl

GOLD = os.path.join(os.path.dirname(__file__), "golden")
D = 32


def _dims(B=16):
    import synth
    return replace(synth.get_config("dflow_relay").dims, D=D, Dt=16, L=3, V=50, B=B, Hq=2, Hkv=2, hd=16, I=48)


def _weights(d, seed=0):
    rng = np.random.default_rng(seed)
    w = {"w_c": rng.standard_normal((d.D, d.L * d.Dt)) * 0.2,
         "g_c": 1 + 0.1 * rng.standard_normal(d.D),
         "embed": rng.standard_normal((d.V, d.D)),
         "e_mask": rng.standard_normal(d.D)}
    rw = {"w1": rng.standard_normal((d.D, 3 * d.D)) * 0.1, "w2": rng.standard_normal((2 * d.D, d.D)) * 0.1}
    return w, rw


def _hidden(d, k, seed=1):
    rng = np.random.default_rng(seed)
    return [rng.standard_normal((k, d.Dt)) for _ in range(d.L)]


# ------------------------------------------------------------ positions

def test_worked_example_next_round_start():
    g = json.load(open(os.path.join(GOLD, "accept_worked_example.json")))
    B = g["drafted"] + 1  # anchor + drafted candidates
    plan = ofl.relay_plan(0, g["accepted"], B)
    # next block anchor is the bonus, one past the accepted candidates; the first
    # drafted position of the next round follows it
    next_anchor = plan[0][1] - plan[0][2]
    assert next_anchor + 1 == g["next_round_first_drafted_position"]


def test_worked_example_shift():
    g = json.load(open(os.path.join(GOLD, "dflow_shift_example.json")))
    src = g["suffix_positions"]
    # choose a round whose reusable suffix is exactly those positions
    P, B = 0, src[-1] + 1
    n = src[0] - 2 - P
    plan = ofl.relay_plan(P, n, B)
    assert [P + o for o, _, _ in plan] == src
    assert [t for _, t, _ in plan] == g["served_positions"]


@pytest.mark.parametrize("B", [8, 16])
def test_offsets_cover_next_block_from_two(B):
    for n in range(B):
        plan = ofl.relay_plan(100, n, B)
        offs = [o for _, _, o in plan]
        assert offs == list(range(2, B - n))       # next-block offsets 2..B-1-n
        assert (len(plan) == 0) == (n >= B - 2)    # no reusable suffix when almost all accepted
        for o_src, tgt, o_next in plan:
            assert o_src >= n + 2                  # the first rejection is not relayed
            assert 100 + n + 1 + o_next == tgt     # lands inside the next block


def test_relay_plan_rejects_bad_counts():
    with pytest.raises(ValueError):
        ofl.relay_plan(0, 16, 16)
    with pytest.raises(ValueError):
        ofl.relay_plan(0, -1, 16)


# ------------------------------------------------------------ LayerNorm

def test_layer_norm_moments_closed_form():
    x = np.random.default_rng(2).standard_normal((5, 64)) * 3 + 7
    y = ofl.layer_norm(x)
    var = x.var(axis=1)
    assert np.allclose(y.mean(axis=1), 0, atol=1e-12)
    assert np.allclose((y * y).mean(axis=1), var / (var + ofl.LN_EPS), rtol=1e-12)


def test_layer_norm_affine_invariance():
    x = np.random.default_rng(3).standard_normal((3, 40))
    assert np.allclose(ofl.layer_norm(5.0 * x + 11.0), ofl.layer_norm(x), atol=1e-5)


# ------------------------------------------------------------ modulation

def test_zero_mlp_gives_plain_mask_embedding():
    d = _dims()
    w, rw = _weights(d)
    rw["w2"] = np.zeros_like(rw["w2"])
    x = ofl.relay_inputs(w, d, rw, _hidden(d, 4), 3, 7)
    assert np.array_equal(x, np.repeat(w["e_mask"][None], 4, 0))


def _cond_free_of_h(d, rw):
    rw = dict(rw)
    w1 = rw["w1"].copy()
    w1[:, 2 * d.D:] = 0.0   # MLP sees only the two token embeddings
    rw["w1"] = w1
    return rw


def test_gamma_is_additive_offset():
    d = _dims()
    w, rw = _weights(d)
    rw = _cond_free_of_h(d, rw)
    w2 = rw["w2"].copy()
    w2[:d.D] = 0.0          # beta = 0: only gamma remains
    rw["w2"] = w2
    x = ofl.relay_inputs(w, d, rw, _hidden(d, 5), 3, 7)
    off = x - w["e_mask"][None]
    assert np.abs(off).max() > 1e-3
    assert np.allclose(off, off[0][None], atol=1e-13)   # the same offset at every relay row


def test_beta_scales_layer_normed_h():
    d = _dims()
    w, rw = _weights(d)
    rw = _cond_free_of_h(d, rw)
    w2 = rw["w2"].copy()
    w2[d.D:] = 0.0          # gamma = 0: only beta * LN(h) remains
    rw["w2"] = w2
    hid = _hidden(d, 5)
    x = ofl.relay_inputs(w, d, rw, hid, 3, 7)
    h = oracle.fuse_context(w["w_c"], w["g_c"], hid, d.rms_eps)
    mu = h.mean(1, keepdims=True)
    ln = (h - mu) / np.sqrt(((h - mu) ** 2).mean(1, keepdims=True) + ofl.LN_EPS)
    beta = (x - w["e_mask"][None]) / ln
    assert np.abs(beta).max() > 1e-3
    assert np.allclose(beta, beta[0][None], rtol=1e-9, atol=1e-12)   # one scale vector per request


def test_bonus_and_first_rejection_enter_in_page_order():
    d = _dims()
    w, rw = _weights(d)
    hid = _hidden(d, 3)
    only_bonus = dict(rw, w1=rw["w1"].copy())
    only_bonus["w1"][:, d.D:2 * d.D] = 0.0     # columns of E(first rejection) off
    a = ofl.relay_inputs(w, d, only_bonus, hid, 3, 7)
    assert np.array_equal(a, ofl.relay_inputs(w, d, only_bonus, hid, 3, 9))
    assert not np.allclose(a, ofl.relay_inputs(w, d, only_bonus, hid, 4, 7))
    only_rej = dict(rw, w1=rw["w1"].copy())
    only_rej["w1"][:, :d.D] = 0.0              # columns of E(bonus) off
    b = ofl.relay_inputs(w, d, only_rej, hid, 3, 7)
    assert np.array_equal(b, ofl.relay_inputs(w, d, only_rej, hid, 4, 7))
    assert not np.allclose(b, ofl.relay_inputs(w, d, only_rej, hid, 3, 9))


def test_verifier_features_scale_invariant():
    # RMSNorm of the shared projection, then LN: rescaling the verifier
    # features changes nothing (up to eps)
    d = _dims()
    w, rw = _weights(d)
    hid = _hidden(d, 4)
    a = ofl.relay_inputs(w, d, rw, hid, 3, 7)
    b = ofl.relay_inputs(w, d, rw, [h * 40.0 for h in hid], 3, 7)
    assert np.allclose(a, b, rtol=1e-4, atol=1e-5)


def test_block_inputs_substitute_only_relay_offsets():
    d = _dims(B=8)
    w, rw = _weights(d)
    rows = {2: np.full(d.D, 5.0), 4: np.full(d.D, -1.0)}
    x = ofl.block_inputs(w, d, 11, rows)
    assert np.array_equal(x[0], w["embed"][11])
    for j in range(1, d.B):
        assert np.array_equal(x[j], rows[j] if j in rows else w["e_mask"])


def test_relay_state_is_per_request_and_cleared_on_take():
    st = ofl.RelayState()
    st.set(0, 3, 8, np.ones((3, 4)))
    st.set(5, 6, 8, np.ones((0, 4)))
    got = st.take(0)
    assert sorted(got) == [2, 3, 4]
    assert st.take(0) == {} and st.take(5) == {}
    with pytest.raises(ValueError):
        st.set(1, 2, 8, np.ones((2, 4)))   # B-2-n = 4 rows expected
