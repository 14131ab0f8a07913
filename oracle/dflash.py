"""Float64 NumPy oracle of the DFlash draft step (test infrastructure only).

Notation: D drafter width, L tapped target layers of width Dt, N drafter
layers, Hq/Hkv query/KV heads of size hd (G = Hq/Hkv), I SwiGLU width,
V vocabulary, B block size (anchor + B-1 masks).  Matrices are [out, in].
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional, Sequence

import numpy as np

F = np.float64


def _f64(a) -> np.ndarray:
    a = np.asarray(a)
    if not np.issubdtype(a.dtype, np.floating):
        raise TypeError("oracle inputs must be floating point (decode bf16 bit patterns first)")
    return a.astype(F, copy=False)


# --------------------------------------------------------------------------
# Building blocks
# --------------------------------------------------------------------------

def rms_norm(z: np.ndarray, g: np.ndarray, eps: float) -> np.ndarray:
    """RMSNorm over the last axis with gain g: z / sqrt(mean(z^2) + eps) * g.

    The fusion equation of the DFlash page (section 三) and of the DFlow page
    (fusion equation in the recomputation-window section) normalises the
    projected target features with RMSNorm.  eps and the learnable gain are not
    on the pages (reading: eps = 1e-6, gain g)."""
    z = _f64(z)
    ms = np.mean(z * z, axis=-1, keepdims=True)
    return z / np.sqrt(ms + eps) * _f64(g)


def rope(x: np.ndarray, pos: np.ndarray, base: float) -> np.ndarray:
    """Rotary position embedding, rotate-half convention, on the last axis.

    Not on the pages (reading): channel i (i < hd/2) pairs with channel
    i + hd/2 and the pair rotates by angle pos * base**(-2i/hd).  x has shape
    [..., T, hd] and pos has T entries."""
    x = _f64(x)
    hd = x.shape[-1]
    half = hd // 2
    inv_freq = F(base) ** (-(np.arange(half, dtype=F) * 2.0) / hd)
    ang = np.asarray(pos, dtype=F)[:, None] * inv_freq[None, :]   # [T, half]
    c, s = np.cos(ang), np.sin(ang)
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def fuse_context(w_c, g_c, hidden: Sequence[np.ndarray], eps: float) -> np.ndarray:
    """Target-context fusion H_c = RMSNorm(W_c [H^(l1); ...; H^(lL)]).

    DFlash page, section 三 (fusion equation); DFlow page, recomputation-window
    section (same equation).  The L tapped layers are concatenated along the
    feature axis, so W_c is [D, L*Dt].  Returns [n, D]."""
    cat = np.concatenate([_f64(h) for h in hidden], axis=1)   # [n, L*Dt]
    z = cat @ _f64(w_c).T
    return rms_norm(z, g_c, eps)


def project_context_kv(layer: dict, H_c: np.ndarray, pos: np.ndarray, d) -> tuple:
    """Per-layer context keys and values K_c = W_c^K H_c, V_c = W_c^V H_c.

    DFlash page, section 二 "注意力模式" (K_c, V_c definitions).  Per the
    engineering note of section 四 and section 2 of the deployment notes, the
    projected K/V (not raw H_c) is what the drafter caches.  Keys are rotated
    at their absolute positions (reading: RoPE on keys of the context too).
    Returns K, V as [Hkv, n, hd]."""
    n = H_c.shape[0]
    k = (H_c @ _f64(layer["w_kc"]).T).reshape(n, d.Hkv, d.hd).transpose(1, 0, 2)
    v = (H_c @ _f64(layer["w_vc"]).T).reshape(n, d.Hkv, d.hd).transpose(1, 0, 2)
    if d.use_rope:
        k = rope(k, pos, d.rope_base)
    return k, v


def block_attention(q: np.ndarray, K: np.ndarray, V: np.ndarray, G: int) -> np.ndarray:
    """KV-injected bidirectional block attention.

    q [Hq, B, hd] comes from the block only; K, V [Hkv, T, hd] are the context
    entries followed by the block's own.  No mask of any kind (DFlash page,
    section 二 "注意力模式": queries only from the block, context only as extra
    K/V, bidirectional inside the block).  Query head h reads KV head h // G
    (reading: standard grouped-query attention).  Scale 1/sqrt(hd).
    Returns [B, Hq*hd]."""
    Hq, B, hd = q.shape
    out = np.empty((B, Hq, hd), dtype=F)
    scale = 1.0 / np.sqrt(F(hd))
    for h in range(Hq):
        g = h // G
        s = (q[h] @ K[g].T) * scale             # [B, T]
        s = s - s.max(axis=1, keepdims=True)
        p = np.exp(s)
        p = p / p.sum(axis=1, keepdims=True)
        out[:, h, :] = p @ V[g]
    return out.reshape(B, Hq * hd)


def round_bf16(a: np.ndarray) -> np.ndarray:
    """Round to the nearest bfloat16 value (ties to even), through float32,
    returned as float64: the storage precision of a bf16 drafter's activations
    (weights already hold bf16 values).  bfloat16 keeps the top 16 bits of the
    float32 pattern; adding 0x7FFF plus the lowest kept bit before truncation
    rounds to nearest, ties to even.  Finite inputs only."""
    b = np.ascontiguousarray(np.asarray(a, dtype=np.float32)).view(np.uint32).astype(np.uint64)
    b = (b + np.uint64(0x7FFF) + ((b >> np.uint64(16)) & np.uint64(1))) & np.uint64(0xFFFF0000)
    return b.astype(np.uint32).view(np.float32).astype(F)


def normed_stored(x: np.ndarray, g: np.ndarray, eps: float, store) -> np.ndarray:
    """RMSNorm with the normed operand held in storage precision: the gained
    row x * g is what is stored (rounded by `store`), and the per-row factor
    1 / sqrt(mean(x^2) + eps) applies to the stored values (a per-row scalar
    commutes with the projection that reads them).  store=None gives rms_norm."""
    if store is None:
        return rms_norm(x, g, eps)
    x = _f64(x)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return store(x * _f64(g)) / np.sqrt(ms + eps)


def silu(x: np.ndarray) -> np.ndarray:
    return x / (1.0 + np.exp(-x))


def swiglu_ffn(u: np.ndarray, layer: dict) -> np.ndarray:
    """SwiGLU feed-forward W_down(SiLU(W_gate u) * W_up u).

    The DFlash pseudocode (section 四) applies a per-layer FFN to the block
    states; its form (SwiGLU) is fixed by the model shape used here."""
    g = u @ _f64(layer["w_gate"]).T
    a = u @ _f64(layer["w_up"]).T
    return (silu(g) * a) @ _f64(layer["w_down"]).T


# --------------------------------------------------------------------------
# Context cache: projected K/V per request (append and rewind)
# --------------------------------------------------------------------------

@dataclass
class ContextCache:
    """Projected context K/V of one request, per drafter layer.

    DFlash page section 四: the drafter's cache stores projected K/V and is
    rolled back to the committed length after verification."""
    K: List[np.ndarray] = field(default_factory=list)   # per layer [Hkv, ctx, hd]
    V: List[np.ndarray] = field(default_factory=list)

    @classmethod
    def empty(cls, d) -> "ContextCache":
        z = np.zeros((d.Hkv, 0, d.hd), dtype=F)
        return cls([z.copy() for _ in range(d.N)], [z.copy() for _ in range(d.N)])

    @property
    def length(self) -> int:
        return self.K[0].shape[1]

    def append(self, w: dict, d, hidden: Sequence[np.ndarray]) -> np.ndarray:
        """Fuse n new verifier rows and append their K/V at positions
        length..length+n-1.  Returns the fused H_c rows."""
        n = hidden[0].shape[0]
        H_c = fuse_context(w["w_c"], w["g_c"], hidden, d.rms_eps)
        pos = np.arange(self.length, self.length + n)
        for l, layer in enumerate(w["layers"]):
            k, v = project_context_kv(layer, H_c, pos, d)
            self.K[l] = np.concatenate([self.K[l], k], axis=1)
            self.V[l] = np.concatenate([self.V[l], v], axis=1)
        return H_c

    def truncate(self, keep: int) -> None:
        self.K = [k[:, :keep] for k in self.K]
        self.V = [v[:, :keep] for v in self.V]


# --------------------------------------------------------------------------
# Draft step
# --------------------------------------------------------------------------

def draft_block(w: dict, d, cache: ContextCache, anchor: int,
                block_inputs: Optional[np.ndarray] = None, conv=None, store=None) -> dict:
    """One-pass block draft over the cached context.

    DFlash page, section 二 (block [anchor, mask x (B-1)]; one forward pass, no
    iterative denoising) and the `draft_forward` / `dflash_cycle` pseudocode of
    section 四: block embeddings are the anchor's token embedding followed by
    the shared mask embedding; every layer takes Q from the block and K/V from
    [context; block]; the shared LM head scores offsets 1..B-1.

    Readings: each layer is the sequential pre-norm residual form
    x += Attn(RMSNorm(x)); x += FFN(RMSNorm(x)) with an output projection W_o;
    a final RMSNorm precedes the shared LM head; block offset j sits at
    absolute position ctx + j.

    conv: None, or per layer four callables [B, D] -> [B, D] applied at the
    DFlash 2 convolution sites (normed attention input, attention output
    before the residual add, normed FFN input, FFN output before the residual
    add); see oracle.dflash2.draft_block_conv.

    store: None (every activation in float64), or a rounding function for
    the activations a bf16 drafter stores between its projections (the pages
    fix no precision; a bf16 drafter keeps its activations in bf16 with fp32
    sums): the context K/V, the rotated Q / K_b / V_b, the attention output,
    the gained normed operands (normed_stored), the SwiGLU product and the
    final normed state.  Token-id decisions on a bf16 drafter are compared in
    that precision; the residual stream and every sum stay float64.

    Returns dict with "logits" [B-1, V], "hidden" [B, D] (final residual
    stream) and "x0" [B, D] (block input)."""
    assert store is None or conv is None, "storage rounding is defined for the plain drafter"
    st = (lambda v: v) if store is None else store
    B = d.B
    if block_inputs is None:
        x = np.stack([_f64(w["embed"][anchor])] + [_f64(w["e_mask"])] * (B - 1))
    else:
        x = _f64(block_inputs).copy()
    x0 = x.copy()
    ctx = cache.length
    pos = np.arange(ctx, ctx + B)
    ident = (lambda v: v,) * 4
    for l, layer in enumerate(w["layers"]):
        c_attn_in, c_attn_out, c_ffn_in, c_ffn_out = ident if conv is None else conv[l]
        u = c_attn_in(normed_stored(x, layer["g_attn"], d.rms_eps, store))
        q = (u @ _f64(layer["w_q"]).T).reshape(B, d.Hq, d.hd).transpose(1, 0, 2)
        kb = (u @ _f64(layer["w_kb"]).T).reshape(B, d.Hkv, d.hd).transpose(1, 0, 2)
        vb = (u @ _f64(layer["w_vb"]).T).reshape(B, d.Hkv, d.hd).transpose(1, 0, 2)
        if d.use_rope:
            q = rope(q, pos, d.rope_base)
            kb = rope(kb, pos, d.rope_base)
        K = np.concatenate([st(cache.K[l]), st(kb)], axis=1)
        V = np.concatenate([st(cache.V[l]), st(vb)], axis=1)
        o = st(block_attention(st(q), K, V, d.G))
        x = x + c_attn_out(o @ _f64(layer["w_o"]).T)
        u = c_ffn_in(normed_stored(x, layer["g_ffn"], d.rms_eps, store))
        if store is None:
            x = x + c_ffn_out(swiglu_ffn(u, layer))
        else:
            hh = st(silu(u @ _f64(layer["w_gate"]).T) * (u @ _f64(layer["w_up"]).T))
            x = x + hh @ _f64(layer["w_down"]).T
    h = normed_stored(x[1:], w["g_final"], d.rms_eps, store)
    logits = h @ _f64(w["w_lm"]).T
    return {"logits": logits, "hidden": x, "x0": x0}


def topk(logits: np.ndarray, k: int) -> tuple:
    """Top-k per row ordered by (logit descending, id ascending).

    The DFlash pseudocode takes the argmax per position (section 四); the
    DFlash 2 selector keeps the top-16 per position.  Tie order is a reading.
    Returns ids [rows, k] (int32) and values [rows, k]."""
    logits = _f64(logits)
    rows, Vn = logits.shape
    ids = np.empty((rows, k), dtype=np.int32)
    vals = np.empty((rows, k), dtype=F)
    for r in range(rows):
        order = np.lexsort((np.arange(Vn), -logits[r]))[:k]
        ids[r] = order
        vals[r] = logits[r, order]
    return ids, vals


def accept(cand: Sequence[int], target: Sequence[int]) -> tuple:
    """Greedy acceptance: longest matching prefix plus the bonus token.

    cand holds the B-1 drafted tokens c_1..c_{B-1}; target holds the B
    verifier argmax tokens t_0..t_{B-1}, where t_j is the verifier's choice
    after block offset j.  n counts leading positions with c_{j+1} == t_j;
    tau = n + 1 (the bonus is counted, so 1 <= tau <= B) and the bonus token is
    t_n.  DFlash page section 四 (`dflash_cycle`: longest common prefix, then
    the token from the verifier at the first mismatch); DFlow page opening
    section (accepted prefix, first rejection replaced by the bonus token);
    DFlash page notation table (tau counts the bonus)."""
    Bm1 = len(cand)
    n = 0
    while n < Bm1 and int(cand[n]) == int(target[n]):
        n += 1
    return n + 1, int(target[n])


class OracleDrafter:
    """Float64 drafter holding per-request context caches."""

    def __init__(self, weights: dict, d):
        self.d = d
        self.w = weights
        self.caches = {}

    def cache(self, r: int) -> ContextCache:
        if r not in self.caches:
            self.caches[r] = ContextCache.empty(self.d)
        return self.caches[r]

    def fuse(self, r: int, hidden: Sequence[np.ndarray]) -> np.ndarray:
        return self.cache(r).append(self.w, self.d, hidden)

    def draft(self, r: int, anchor: int, store=None) -> dict:
        return draft_block(self.w, self.d, self.cache(r), anchor, store=store)

    def reset(self, r: int, keep: int) -> None:
        self.cache(r).truncate(keep)
