"""Pins of the DFlash 2 two-tap dynamic convolution oracle (CPU).

Source: "DFlash 2：正确 token 已在候选里，选一条连贯的路就好", second insight
section (Conv_k(x)_t = k_{t,0} * x_t + k_{t,1} * x_{t-1}; base kernel plus a
correction from the current hidden state, one correction per 16 channels; the
block's first position reads the last verified token; before and after the
attention and FFN sub-layers; 16.5M extra parameters).

Pins: the static special case equals numpy's convolution; a closed form fixes
the 16-channel grouping, the tap roles and which row the correction reads;
brute force fixes the block boundary and the locality; the parameter count
matches the page's figure; identity and scaling equivalences fix the four
sites in the layer."""
import copy
import dataclasses

import numpy as np

import oracle
import synth
from oracle import dflash2 as ds


def _rng(k):
    return np.random.Generator(np.random.PCG64(k))


def _tiny():
    wl = synth.get_config("dflash2_select")
    d = wl.dims
    w = synth.weights_as_f32(synth.make_weights(d, wl.seed))
    hid = synth.as_f32(synth.make_hidden(d, wl.seed, 0, 0, 24))
    cache = oracle.ContextCache.empty(d)
    cache.append(w, d, hid)
    return d, w, cache


def _identity_conv(d, overrides=None):
    G = d.D // 16
    site = {"w": np.zeros((2 * G, d.D)), "kbase": np.stack([np.ones(d.D), np.zeros(d.D)])}
    conv = [{s: copy.deepcopy(site) for s in ds.CONV_SITES} for _ in range(d.N)]
    for (l, s), v in (overrides or {}).items():
        conv[l][s] = v
    return conv


def test_static_taps_equal_numpy_convolve():
    # W = 0: every channel is the fixed 2-tap filter [k0, k1] along the block
    rng = _rng(1)
    B, D = 9, 64
    x = rng.standard_normal((B, D))
    kb = rng.standard_normal((2, D))
    y = ds.two_tap_conv(x, np.zeros((2 * D // 16, D)), kb)
    for c in range(D):
        ref = np.convolve(x[:, c], [kb[0, c], kb[1, c]])[:B]
        assert np.allclose(y[:, c], ref, rtol=0, atol=1e-13)


def test_correction_grouping_tap_roles_and_source_row():
    # x_0 = x_1 = ones, other rows zero; W_0 rows constant alpha_g / D, W_1 rows
    # beta_g / D, kbase = 0.  Then (W_j x_t)[g] is alpha_g (beta_g) on rows 0-1
    # and zero elsewhere, so y_0 = alpha_g (no left row), y_1 = alpha_g + beta_g
    # and y_2 = 0 (the correction reads the current row, which is zero).
    rng = _rng(2)
    B, D = 6, 128
    G = D // 16
    alpha, beta = rng.uniform(0.5, 2.0, G), rng.uniform(-2.0, -0.5, G)
    w = np.concatenate([np.repeat(alpha[:, None] / D, D, 1), np.repeat(beta[:, None] / D, D, 1)])
    x = np.zeros((B, D))
    x[0] = x[1] = 1.0
    y = ds.two_tap_conv(x, w, np.zeros((2, D)))
    g_of_c = np.arange(D) // 16
    assert np.allclose(y[0], alpha[g_of_c], atol=1e-12)
    assert np.allclose(y[1], alpha[g_of_c] + beta[g_of_c], atol=1e-12)
    assert np.allclose(y[2:], 0.0, atol=1e-12)


def test_block_boundary_and_locality_by_brute_force():
    rng = _rng(3)
    B, D = 8, 32
    x = rng.standard_normal((B, D))
    w = rng.standard_normal((2 * D // 16, D)) * 0.3
    kb = rng.standard_normal((2, D))
    y = ds.two_tap_conv(x, w, kb)
    # offset 0 has no left neighbour: its output is k_{0,0} * x_0 whatever the last row holds
    x2 = x.copy()
    x2[B - 1] += 5.0
    assert np.array_equal(ds.two_tap_conv(x2, w, kb)[0], y[0])
    k00 = kb[0] + np.repeat(w[: D // 16] @ x[0], 16)
    assert np.allclose(y[0], k00 * x[0], atol=1e-12)
    # a change at offset t reaches offsets t and t + 1 only
    for t in range(B):
        xp = x.copy()
        xp[t] += rng.standard_normal(D)
        changed = np.flatnonzero(np.any(ds.two_tap_conv(xp, w, kb) != y, axis=1))
        assert set(changed.tolist()) <= {t, t + 1} and t in changed.tolist()


def test_parameter_count_matches_the_page():
    # two [D/16, D] correction matrices and two base kernels per site, four
    # sites per layer: 16.5M at the 5-layer drafter of width 2560
    assert round(ds.conv_param_count(2560, 5) / 1e6, 1) == 16.5


def test_identity_conv_is_the_base_drafter():
    d, w, cache = _tiny()
    base = oracle.draft_block(w, d, cache, 7)
    conv = ds.draft_block_conv(w, d, cache, 7, _identity_conv(d))
    assert np.array_equal(base["logits"], conv["logits"])


def _scaled(w, l, keys, s):
    w2 = copy.deepcopy(w)
    for k in keys:
        w2["layers"][l][k] = np.asarray(w2["layers"][l][k], np.float64) * s
    return w2


def _static(d, s):
    return {"w": np.zeros((2 * (d.D // 16), d.D)), "kbase": np.stack([np.full(d.D, s), np.zeros(d.D)])}


def test_sites_sit_around_attention_and_ffn():
    # a static tap (s, 0) at one site equals scaling the weights that site feeds
    d, w, cache = _tiny()
    cases = [("attn_in", ("w_q", "w_kb", "w_vb"), 1.7), ("attn_out", ("w_o",), 2.0),
             ("ffn_in", ("w_gate", "w_up"), 1.3), ("ffn_out", ("w_down",), 2.0)]
    for site, keys, s in cases:
        for l in range(d.N):
            got = ds.draft_block_conv(w, d, cache, 11, _identity_conv(d, {(l, site): _static(d, s)}))
            ref = oracle.draft_block(_scaled(w, l, keys, s), d, cache, 11)
            err = np.abs(got["logits"] - ref["logits"]).max() / np.abs(ref["logits"]).max()
            assert err < 1e-12, (site, l, err)


def test_left_tap_mixes_the_previous_offset_in_the_drafter():
    # a pure left tap at the first site moves every offset's normed input one
    # offset down the block: offset 1 then sees the anchor's row
    d, w, cache = _tiny()
    d1 = dataclasses.replace(d, N=1)
    w1 = dict(w, layers=w["layers"][:1])
    site = {"w": np.zeros((2 * (d.D // 16), d.D)), "kbase": np.stack([np.zeros(d.D), np.ones(d.D)])}
    c1 = oracle.ContextCache.empty(d1)
    c1.K, c1.V = cache.K[:1], cache.V[:1]
    got = ds.draft_block_conv(w1, d1, c1, 5, _identity_conv(d1, {(0, "attn_in"): site}))
    # reference: the same forward with the attention input rows shifted by hand
    hooks = [(lambda v: np.concatenate([np.zeros((1, v.shape[1])), v[:-1]]),) + (lambda v: v,) * 3]
    ref = oracle.draft_block(w1, d1, c1, 5, conv=hooks)
    assert np.allclose(got["logits"], ref["logits"], rtol=0, atol=1e-12)
    base = oracle.draft_block(w1, d1, c1, 5)
    assert not np.allclose(got["logits"], base["logits"])
