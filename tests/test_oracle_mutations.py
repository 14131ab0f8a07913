"""Planted mistakes in the oracle (on the CPU, via monkeypatch) must each be
caught by one of the pins: shows the pins are sharp enough to notice a dropped
term, a wrong sign or index, or a transposed operand."""
import numpy as np
import pytest
import torch

import oracle
import oracle.dflash as od
import synth
from tests import _libforms as lf
from tests.test_oracle_pins import MICRO, _hidden, _weights

_orig_rope = od.rope
_orig_attn = od.block_attention
_orig_rms = od.rms_norm


def _forward_matches(d=MICRO, ctx=7):
    w = _weights(d)
    hid = _hidden(d, ctx)
    c = od.ContextCache.empty(d)
    c.append(w, d, hid)
    got = od.draft_block(w, d, c, 13)["logits"]
    ref = lf.forward(w, d, hid, 13)
    return np.allclose(got, ref, rtol=1e-8, atol=1e-9)


def _rope_matches():
    x = np.random.default_rng(1).standard_normal((2, 5, 16))
    pos = np.array([0, 3, 17, 900, 5])
    return np.allclose(od.rope(x, pos, 10000.0),
                       lf.rope_complex(torch.tensor(x), torch.tensor(pos), 10000.0).numpy(),
                       rtol=1e-10, atol=1e-12)


def _attn_matches():
    rng = np.random.default_rng(3)
    q = rng.standard_normal((8, 5, 16))
    K = rng.standard_normal((2, 11, 16))
    V = rng.standard_normal((2, 11, 16))
    return np.allclose(od.block_attention(q, K, V, 4),
                       lf.sdpa(torch.tensor(q), torch.tensor(K), torch.tensor(V), 4).numpy(),
                       rtol=1e-10, atol=1e-12)


def test_unmutated_baselines_pass():
    assert _forward_matches() and _rope_matches() and _attn_matches()


def test_rope_sign_flip_caught(monkeypatch):
    monkeypatch.setattr(od, "rope", lambda x, pos, base: _orig_rope(x, -np.asarray(pos), base))
    assert not _rope_matches()
    assert not _forward_matches()


def test_rope_interleaved_pairing_caught(monkeypatch):
    def interleaved(x, pos, base):
        hd = x.shape[-1]
        perm = np.concatenate([np.arange(0, hd, 2), np.arange(1, hd, 2)])
        inv = np.argsort(perm)
        return _orig_rope(x[..., perm], pos, base)[..., inv]
    monkeypatch.setattr(od, "rope", interleaved)
    assert not _rope_matches()


def test_gqa_head_mapping_caught(monkeypatch):
    def wrong(q, K, V, G):
        Hkv = K.shape[0]
        Kx = np.stack([K[h % Hkv] for h in range(q.shape[0])])
        Vx = np.stack([V[h % Hkv] for h in range(q.shape[0])])
        return _orig_attn(q, Kx, Vx, 1)
    monkeypatch.setattr(od, "block_attention", wrong)
    assert not _attn_matches()


def test_missing_softmax_scale_caught(monkeypatch):
    monkeypatch.setattr(od, "block_attention",
                        lambda q, K, V, G: _orig_attn(q * np.sqrt(q.shape[-1]), K, V, G))
    assert not _attn_matches()


def test_dropped_context_kv_caught(monkeypatch):
    def no_ctx(q, K, V, G):
        B = q.shape[1]
        return _orig_attn(q, K[:, -B:], V[:, -B:], G)
    monkeypatch.setattr(od, "block_attention", no_ctx)
    assert not _forward_matches()


def test_causal_mask_in_block_caught(monkeypatch):
    def causal(q, K, V, G):
        Hq, B, hd = q.shape
        T = K.shape[1]
        out = np.empty((B, Hq, hd))
        for h in range(Hq):
            s = q[h] @ K[h // G].T / np.sqrt(hd)
            s[:, T - B:] += np.triu(np.full((B, B), -np.inf), 1)
            p = np.exp(s - s.max(1, keepdims=True))
            out[:, h] = (p / p.sum(1, keepdims=True)) @ V[h // G]
        return out.reshape(B, -1)
    monkeypatch.setattr(od, "block_attention", causal)
    assert not _forward_matches()


def test_transposed_fusion_blocks_caught():
    d = MICRO
    w = _weights(d)
    hid = _hidden(d, 4)
    # wrong: interpret W_c's input axis as layer-interleaved instead of layer-blocked
    wc = w["w_c"].reshape(d.D, d.Dt, d.L).transpose(0, 2, 1).reshape(d.D, -1)
    bad = oracle.fuse_context(wc, w["g_c"], hid, d.rms_eps)
    assert not np.allclose(bad, lf.fuse(w, d, hid).numpy(), rtol=1e-6)


def test_missing_final_norm_caught(monkeypatch):
    calls = {"n": 0}

    def rms_skip_last(z, g, eps):
        if z.shape[0] == MICRO.B - 1:      # only the final norm sees B-1 rows
            return np.asarray(z, dtype=np.float64)
        return _orig_rms(z, g, eps)
    monkeypatch.setattr(od, "rms_norm", rms_skip_last)
    assert not _forward_matches()


def test_accept_without_bonus_caught():
    from tests.test_oracle_pins import _naive_accept
    cand, tgt = [1, 2, 3], [1, 2, 9, 4]
    tau, bonus = oracle.accept(cand, tgt)
    assert (tau, bonus) == _naive_accept(cand, tgt) == (3, 9)
    wrong = (tau - 1, bonus)
    assert wrong != _naive_accept(cand, tgt)


def test_topk_high_id_tiebreak_caught():
    lg = np.array([[0.5, 1.0, 1.0, 0.2]])
    ids, _ = oracle.topk(lg, 2)
    assert list(ids[0]) == list(np.argsort(-lg[0], kind="stable")[:2]) == [1, 2]
