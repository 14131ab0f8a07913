"""Pins for the float64 oracle: each test ties it to something other than
itself (library routines, closed forms, invariants, brute force, the pages'
worked examples).  CPU only."""
import dataclasses
import itertools
import json
import os

import numpy as np
import pytest
import torch

import oracle
import oracle.dflash as od
import synth
from synth.configs import Dims
from tests import _libforms as lf

GOLD = os.path.join(os.path.dirname(__file__), "golden")

MICRO = Dims("micro", "f32", D=64, L=2, Dt=48, N=2, Hq=4, Hkv=2, hd=16, I=96, V=50, B=6)


def _weights(d, seed=11):
    return synth.weights_as_f32(synth.make_weights(d, seed))


def _hidden(d, n, seed=11, req=0, start=0):
    return synth.make_hidden(d, seed, req, start, n)


# ---------------------------------------------------------------- fusion

def test_fusion_equals_blockwise_sum_and_library_rmsnorm():
    d = MICRO
    w = _weights(d)
    hid = _hidden(d, 9)
    got = oracle.fuse_context(w["w_c"], w["g_c"], hid, d.rms_eps)
    ref = lf.fuse(w, d, hid).numpy()
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


def test_wc_orientation_and_size_from_pages():
    g = json.load(open(os.path.join(GOLD, "wc_size.json")))
    D, L = g["D"], g["L"]
    nbytes = D * (L * D) * g["bytes_per_element"]
    assert abs(nbytes / 1e6 - g["approx_megabytes"]) < 0.5
    # The oracle consumes W_c as [D, L*D]: the concatenated features are the
    # input axis.  A [L*D, D] matrix must be rejected by the shapes.
    d = dataclasses.replace(MICRO, Dt=MICRO.D)
    w = _weights(d)
    assert w["w_c"].shape == (d.D, d.L * d.D)
    hid = _hidden(d, 3)
    assert oracle.fuse_context(w["w_c"], w["g_c"], hid, d.rms_eps).shape == (3, d.D)
    with pytest.raises(ValueError):
        oracle.fuse_context(np.ascontiguousarray(w["w_c"].T), w["g_c"], hid, d.rms_eps)


def test_rmsnorm_invariants():
    rng = np.random.default_rng(0)
    z = rng.standard_normal((5, 32)) * 3
    g = 1 + 0.1 * rng.standard_normal(32)
    eps = 1e-6
    y = oracle.rms_norm(z, g, eps)
    ms = np.mean(z * z, axis=1)
    np.testing.assert_allclose(np.mean((y / g) ** 2, axis=1), ms / (ms + eps), rtol=1e-12)
    # scaling the input by a rescales the output by sqrt((ms+eps)/(ms+eps/a^2))
    a = 37.5
    ratio = np.sqrt((ms + eps) / (ms + eps / a ** 2))[:, None]
    np.testing.assert_allclose(oracle.rms_norm(z * a, g, eps), y * ratio, rtol=1e-12)
    # eps matters: all-zero input maps to zero, not NaN
    assert np.all(oracle.rms_norm(np.zeros((1, 32)), g, eps) == 0)


def test_chunked_fuse_equals_one_shot():
    d = MICRO
    w = _weights(d)
    hid = _hidden(d, 20)
    a = oracle.ContextCache.empty(d)
    a.append(w, d, hid)
    b = oracle.ContextCache.empty(d)
    b.append(w, d, [h[:7] for h in hid])
    b.append(w, d, [h[7:] for h in hid])
    for l in range(d.N):
        np.testing.assert_allclose(a.K[l], b.K[l], rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(a.V[l], b.V[l], rtol=1e-10, atol=1e-12)
    b.truncate(11)
    assert b.length == 11
    np.testing.assert_allclose(b.K[1], a.K[1][:, :11], rtol=1e-10, atol=1e-12)


# ---------------------------------------------------------------- RoPE

def test_rope_equals_complex_rotation():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((3, 7, 16))
    pos = np.array([0, 1, 5, 100, 4095, 8200, 3])
    got = oracle.rope(x, pos, 10000.0)
    ref = lf.rope_complex(torch.tensor(x), torch.tensor(pos), 10000.0).numpy()
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


def test_rope_norm_preserving_and_identity_at_zero():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((2, 4, 64))
    y = oracle.rope(x, np.array([0, 9, 77, 1234]), 10000.0)
    half = 32
    np.testing.assert_allclose(x[..., :half] ** 2 + x[..., half:] ** 2,
                               y[..., :half] ** 2 + y[..., half:] ** 2, rtol=1e-12)
    np.testing.assert_array_equal(y[:, 0], x[:, 0])


def test_draft_invariant_under_position_shift():
    """RoPE makes attention depend on relative position only: drafting with
    the whole sequence shifted by a constant gives the same logits."""
    d = MICRO
    w = _weights(d)
    hid = _hidden(d, 12)
    a = oracle.ContextCache.empty(d)
    a.append(w, d, hid)
    la = oracle.draft_block(w, d, a, 3)["logits"]
    # shift: pretend 100 earlier positions existed by re-rotating keys
    b = oracle.ContextCache.empty(d)
    Hc = oracle.fuse_context(w["w_c"], w["g_c"], hid, d.rms_eps)
    for l, lw in enumerate(w["layers"]):
        k, v = oracle.project_context_kv(lw, Hc, np.arange(100, 112), d)
        b.K[l], b.V[l] = k, v

    class Shifted(oracle.ContextCache):
        @property
        def length(self):
            return 112
    s = Shifted(b.K, b.V)
    lb = oracle.draft_block(w, d, s, 3)["logits"]
    np.testing.assert_allclose(la, lb, rtol=1e-9, atol=1e-10)


# ---------------------------------------------------------------- attention

def test_attention_equals_sdpa_on_concatenated_kv():
    rng = np.random.default_rng(3)
    Hq, Hkv, B, T, hd = 8, 2, 5, 13, 16
    q = rng.standard_normal((Hq, B, hd))
    K = rng.standard_normal((Hkv, T, hd))
    V = rng.standard_normal((Hkv, T, hd))
    got = oracle.block_attention(q, K, V, Hq // Hkv)
    ref = lf.sdpa(torch.tensor(q), torch.tensor(K), torch.tensor(V), Hq // Hkv).numpy()
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


def test_empty_context_reduces_to_plain_bidirectional_attention():
    rng = np.random.default_rng(4)
    q = rng.standard_normal((4, 6, 16))
    kb = rng.standard_normal((4, 6, 16))
    vb = rng.standard_normal((4, 6, 16))
    got = oracle.block_attention(q, kb, vb, 1)
    qt, kt, vt = (torch.tensor(a) for a in (q, kb, vb))
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt).transpose(0, 1).reshape(6, -1)
    np.testing.assert_allclose(got, ref.numpy(), rtol=1e-12, atol=1e-12)


def test_identical_keys_give_mean_of_values():
    rng = np.random.default_rng(5)
    q = rng.standard_normal((2, 3, 8))
    K = np.repeat(rng.standard_normal((1, 1, 8)), 9, axis=1).repeat(2, axis=0)
    V = rng.standard_normal((2, 9, 8))
    got = oracle.block_attention(q, K, V, 1).reshape(3, 2, 8)
    for h in range(2):
        np.testing.assert_allclose(got[:, h], np.broadcast_to(V[h].mean(0), (3, 8)), rtol=1e-12)


def test_gqa_equals_mha_with_replicated_heads():
    rng = np.random.default_rng(6)
    q = rng.standard_normal((8, 4, 16))
    K = rng.standard_normal((2, 10, 16))
    V = rng.standard_normal((2, 10, 16))
    a = oracle.block_attention(q, K, V, 4)
    b = oracle.block_attention(q, np.repeat(K, 4, axis=0), np.repeat(V, 4, axis=0), 1)
    np.testing.assert_allclose(a, b, rtol=1e-13)


def test_no_rope_identical_masks_give_identical_outputs_and_context_order_free():
    d = dataclasses.replace(MICRO, use_rope=False)
    w = _weights(d)
    hid = _hidden(d, 10)
    c = oracle.ContextCache.empty(d)
    c.append(w, d, hid)
    r = oracle.draft_block(w, d, c, 7)
    lg = r["logits"]
    for j in range(1, lg.shape[0]):
        np.testing.assert_allclose(lg[j], lg[0], rtol=1e-12, atol=1e-12)
    perm = np.random.default_rng(7).permutation(10)
    c2 = oracle.ContextCache([k[:, perm] for k in c.K], [v[:, perm] for v in c.V])
    np.testing.assert_allclose(oracle.draft_block(w, d, c2, 7)["logits"], lg, rtol=1e-10, atol=1e-12)


def test_context_changes_the_draft():
    """KV injection: the context must influence every block position."""
    d = MICRO
    w = _weights(d)
    c0 = oracle.ContextCache.empty(d)
    c1 = oracle.ContextCache.empty(d)
    c1.append(w, d, _hidden(d, 8))
    a = oracle.draft_block(w, d, c0, 5)["logits"]
    b = oracle.draft_block(w, d, c1, 5)["logits"]
    assert np.all(np.abs(a - b).max(axis=1) > 1e-6)


# ---------------------------------------------------------------- FFN, LM head

def test_ffn_equals_library_form():
    d = MICRO
    w = _weights(d)
    u = np.random.default_rng(8).standard_normal((6, d.D))
    lw = w["layers"][0]
    got = oracle.swiglu_ffn(u, lw)
    F = torch.nn.functional
    ut = torch.tensor(u)
    ref = F.linear(F.silu(F.linear(ut, lf.t(lw["w_gate"]))) * F.linear(ut, lf.t(lw["w_up"])),
                   lf.t(lw["w_down"]))
    np.testing.assert_allclose(got, ref.numpy(), rtol=1e-10, atol=1e-12)
    z = dict(lw, w_down=np.zeros_like(lw["w_down"]))
    assert np.all(oracle.swiglu_ffn(u, z) == 0)


def test_topk_equals_stable_argsort_and_breaks_ties_low_id():
    rng = np.random.default_rng(9)
    lg = np.round(rng.standard_normal((4, 200)), 1)   # many exact ties
    ids, vals = oracle.topk(lg, 16)
    for r in range(4):
        order = np.argsort(-lg[r], kind="stable")[:16]
        np.testing.assert_array_equal(ids[r], order)
        np.testing.assert_array_equal(vals[r], lg[r, order])
    assert ids[0, 0] == int(np.argmax(lg[0]))


# ---------------------------------------------------------------- acceptance

def _naive_accept(cand, target):
    mism = [c != t for c, t in zip(cand, target[:-1])]
    n = mism.index(True) if True in mism else len(cand)
    return n + 1, target[n]


@pytest.mark.parametrize("B,V", [(2, 2), (3, 3), (4, 2), (5, 3)])
def test_accept_exhaustive(B, V):
    tb = json.load(open(os.path.join(GOLD, "tau_bounds.json")))
    for cand in itertools.product(range(V), repeat=B - 1):
        for tgt in itertools.product(range(V), repeat=B):
            tau, bonus = oracle.accept(cand, tgt)
            assert (tau, bonus) == _naive_accept(list(cand), list(tgt))
            assert tb["tau_min"] <= tau <= B


def test_accept_constructed_first_mismatch():
    rng = np.random.default_rng(10)
    B, V = 16, 1000
    cand = rng.integers(0, V, size=(64, B - 1)).astype(np.int32)
    m = synth.draw_first_mismatch("uniform", 64, B, 5)
    tgt = synth.make_targets(cand, m, V, 5)
    for r in range(64):
        tau, bonus = oracle.accept(cand[r], tgt[r])
        assert tau == m[r] + 1
        assert bonus == tgt[r, m[r]]


def test_accept_worked_example_from_pages():
    g = json.load(open(os.path.join(GOLD, "accept_worked_example.json")))
    K = g["drafted"]
    cand = list(range(100, 100 + K))
    tgt = cand[:g["accepted"]] + [7] + [0] * (K - g["accepted"])
    tau, bonus = oracle.accept(cand, tgt)
    assert tau == g["accepted"] + 1 and bonus == 7
    # drafted positions are numbered 1..K after the anchor; the tau committed
    # tokens occupy 1..tau, so the next round's first drafted token is tau + 1
    assert tau + 1 == g["next_round_first_drafted_position"]


# ---------------------------------------------------------------- whole forward

@pytest.mark.parametrize("ctx", [0, 5, 17])
def test_whole_forward_equals_library_form(ctx):
    d = MICRO
    w = _weights(d)
    hid = _hidden(d, ctx) if ctx else [np.zeros((0, d.Dt), np.float32)] * d.L
    c = oracle.ContextCache.empty(d)
    if ctx:
        c.append(w, d, hid)
    got = oracle.draft_block(w, d, c, 13)["logits"]
    ref = lf.forward(w, d, hid, 13)
    np.testing.assert_allclose(got, ref, rtol=1e-10, atol=1e-11)


def test_whole_forward_tiny_config_equals_library_form():
    wl = synth.get_config("tiny")
    d = wl.dims
    w = _weights(d, wl.seed)
    hid = _hidden(d, 64, wl.seed)
    o = oracle.OracleDrafter(w, d)
    o.fuse(0, hid)
    got = o.draft(0, 321)["logits"]
    ref = lf.forward(w, d, hid, 321)
    np.testing.assert_allclose(got, ref, rtol=1e-10, atol=1e-11)


# ---- storage precision (bf16 activations) for token-id decisions

def test_round_bf16_matches_torch_conversion():
    """oracle.round_bf16 equals torch's float32 -> bfloat16 conversion (round
    to nearest, ties to even) on random values, exact ties and tiny values."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(5)
    x = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.integers(-30, 30, 20000),
                        rng.standard_normal(1000) * 1e-39]).astype(np.float32)
    # exact ties: the 16 dropped bits are 0x8000, with odd and even kept bits
    ties = (np.arange(1000, dtype=np.uint32) << np.uint32(16)) | np.uint32(0x8000)
    x = np.concatenate([x, (ties + np.uint32(0x3F800000)).view(np.float32)])
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy().astype(np.float64)
    assert np.array_equal(oracle.round_bf16(x), ref)


def test_storage_hook_identity_is_the_plain_draft():
    """With an identity rounding the storage form equals the plain draft (up to
    float64 rounding of the regrouped RMSNorm)."""
    d = _tiny_dims()
    w = synth.weights_as_f32(synth.make_weights(d, 3))
    c = oracle.ContextCache.empty(d)
    c.append(w, d, synth.as_f32(synth.make_hidden(d, 3, 0, 0, 20)))
    a = oracle.draft_block(w, d, c, 9)["logits"]
    b = oracle.draft_block(w, d, c, 9, store=lambda v: v)["logits"]
    assert np.abs(a - b).max() <= 1e-12 * np.abs(a).max()
    assert np.allclose(oracle.normed_stored(a, np.ones(a.shape[1]), 1e-6, None),
                       oracle.rms_norm(a, np.ones(a.shape[1]), 1e-6))


def test_storage_rounding_touches_each_stored_activation():
    """The rounding applies to what a bf16 drafter stores between its
    projections, and to nothing else: per layer the context K and V, the
    rotated Q / K_b / V_b, the attention output, the gained attention and FFN
    operands and the SwiGLU product, then the final gained state."""
    d = _tiny_dims()
    w = synth.weights_as_f32(synth.make_weights(d, 4))
    c = oracle.ContextCache.empty(d)
    c.append(w, d, synth.as_f32(synth.make_hidden(d, 4, 0, 0, 12)))
    seen = []

    def rec(v):
        seen.append(tuple(np.shape(v)))
        return oracle.round_bf16(v)

    plain = oracle.draft_block(w, d, c, 2)["logits"]
    got = oracle.draft_block(w, d, c, 2, store=rec)["logits"]
    B, ctx = d.B, 12
    per_layer = [(B, d.D), (d.Hkv, ctx, d.hd), (d.Hkv, B, d.hd), (d.Hkv, ctx, d.hd), (d.Hkv, B, d.hd),
                 (d.Hq, B, d.hd), (B, d.Hq * d.hd), (B, d.D), (B, d.I)]
    assert seen == per_layer * d.N + [(B - 1, d.D)]
    # bf16 storage moves the logits by about the bf16 unit, not more
    rel = np.abs(got - plain).max() / np.abs(plain).max()
    assert 1e-5 < rel < 3e-2


def _tiny_dims():
    from synth.configs import _tiny
    return _tiny()
