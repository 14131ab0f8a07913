"""Seeded generators: weights, verifier hidden states, anchors, target tokens.

Every tensor is filled in chunks of 2**20 elements; chunk c of tensor t draws
standard normals (float32) from PCG64(SeedSequence([seed, t, c])).  Chunks are
independent streams, so filling runs on a thread pool and the values do not
depend on the thread count.  Weights and the mask embedding are N(0, 0.02);
RMSNorm gains are 1 + N(0, 0.02); verifier features are N(0, 1).  bf16 storage
rounds each float32 draw to nearest-even.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from typing import Dict, List, Sequence

import numpy as np

from .configs import Dims, GEOM_P_MEAN_6_5

CHUNK = 1 << 20
_HIDDEN_ROWS_PER_BLOCK = 64
_POOL = None


def _pool() -> ThreadPoolExecutor:
    global _POOL
    if _POOL is None:
        n = min(16, os.cpu_count() or 1)
        _POOL = ThreadPoolExecutor(max_workers=n)
    return _POOL


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest-even), returned as uint16 bits."""
    v = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).copy()
    r = (v >> 16) & 1
    r += 0x7FFF
    v += r
    v >>= 16
    return v.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact upcast of bf16 bits to float32."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _fill(shape, keys: Sequence[int], scale: float, offset: float, dtype: str) -> np.ndarray:
    n = int(np.prod(shape))
    out = np.empty(n, np.uint16 if dtype == "bf16" else np.float32)

    def work(c):
        s = c * CHUNK
        e = min(n, s + CHUNK)
        rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(list(keys) + [c])))
        x = rng.standard_normal(e - s, dtype=np.float32)
        x *= np.float32(scale)
        if offset:
            x += np.float32(offset)
        if dtype == "bf16":
            v = x.view(np.uint32)
            r = (v >> 16) & 1
            r += 0x7FFF
            v += r
            v >>= 16
            out[s:e] = v
        else:
            out[s:e] = x

    nch = (n + CHUNK - 1) // CHUNK
    if nch <= 2:
        for c in range(nch):
            work(c)
    else:
        list(_pool().map(work, range(nch)))
    return out.reshape(shape)


LAYER_KEYS = ("g_attn", "w_q", "w_kb", "w_vb", "w_kc", "w_vc", "w_o",
              "g_ffn", "w_gate", "w_up", "w_down")


def layer_shapes(d: Dims) -> Dict[str, tuple]:
    return {
        "g_attn": (d.D,),
        "w_q": (d.Hq * d.hd, d.D),
        "w_kb": (d.Hkv * d.hd, d.D),
        "w_vb": (d.Hkv * d.hd, d.D),
        "w_kc": (d.Hkv * d.hd, d.D),
        "w_vc": (d.Hkv * d.hd, d.D),
        "w_o": (d.D, d.Hq * d.hd),
        "g_ffn": (d.D,),
        "w_gate": (d.I, d.D),
        "w_up": (d.I, d.D),
        "w_down": (d.D, d.I),
    }


def make_weights(d: Dims, seed: int) -> dict:
    """Synthetic drafter weights in storage dtype (fp32 arrays or bf16 bits).

    Tensor order (the tensor index t in the chunk seed): w_c, g_c, embed,
    e_mask, g_final, then for each layer the LAYER_KEYS order.  The LM head is
    tied to the embedding.
    """
    s = 1000 + seed
    t = [0]

    def nxt(shape, gain=False):
        a = _fill(shape, [s, t[0]], 0.02, 1.0 if gain else 0.0, d.dtype)
        t[0] += 1
        return a

    w = {}
    w["w_c"] = nxt((d.D, d.L * d.Dt))
    w["g_c"] = nxt((d.D,), gain=True)
    w["embed"] = nxt((d.V, d.D))
    w["e_mask"] = nxt((d.D,))
    w["g_final"] = nxt((d.D,), gain=True)
    w["w_lm"] = w["embed"]
    shapes = layer_shapes(d)
    layers = []
    for _ in range(d.N):
        lw = {}
        for k in LAYER_KEYS:
            lw[k] = nxt(shapes[k], gain=k.startswith("g_"))
        layers.append(lw)
    w["layers"] = layers
    return w


def make_relay_weights(d: Dims, seed: int) -> dict:
    """Relay MLP weights in storage dtype: w1 [D, 3D], w2 [2D, D], ~N(0, 0.02).
    Tensor indices start at 10000 so they never meet the drafter's."""
    s = 1000 + seed
    return {"w1": _fill((d.D, 3 * d.D), [s, 10000], 0.02, 0.0, d.dtype),
            "w2": _fill((2 * d.D, d.D), [s, 10001], 0.02, 0.0, d.dtype)}


def make_selector_weights(d: Dims, seed: int, rank: int = 256) -> dict:
    """Path-selector tables in storage dtype: a, b [V, rank] ~ N(0, 0.2) (so the
    pairwise term is on the scale of the logit gaps and the walk does not reduce
    to the per-position argmax), w_h [rank, D] ~ N(0, 1/sqrt(D)) (gate
    pre-activations of unit scale).  Tensor indices start at 20000."""
    s = 1000 + seed
    return {"a": _fill((d.V, rank), [s, 20000], 0.2, 0.0, d.dtype),
            "b": _fill((d.V, rank), [s, 20001], 0.2, 0.0, d.dtype),
            "w_h": _fill((rank, d.D), [s, 20002], float(1.0 / np.sqrt(d.D)), 0.0, d.dtype)}


def make_conv_weights(d: Dims, seed: int) -> list:
    """Two-tap convolution weights in storage dtype, per layer and site
    (attn_in, attn_out, ffn_in, ffn_out): w [2 * D/16, D] ~ N(0, 0.1/sqrt(D))
    (tap corrections of about 0.1 on unit-scale rows), kbase [2, D] with the
    current tap 1 + N(0, 0.05) and the left tap 0.25 + N(0, 0.05) (a clearly
    non-zero neighbour mix).  Tensor indices start at 21000."""
    s = 1000 + seed
    sites = ("attn_in", "attn_out", "ffn_in", "ffn_out")
    out = []
    for l in range(d.N):
        layer = {}
        for i, site in enumerate(sites):
            t = 21000 + 8 * (4 * l + i)
            k0 = _fill((1, d.D), [s, t + 1], 0.05, 1.0, d.dtype)
            k1 = _fill((1, d.D), [s, t + 2], 0.05, 0.25, d.dtype)
            layer[site] = {"w": _fill((2 * (d.D // 16), d.D), [s, t], float(0.1 / np.sqrt(d.D)), 0.0, d.dtype),
                           "kbase": np.ascontiguousarray(np.concatenate([k0, k1], axis=0))}
        out.append(layer)
    return out


def conv_weights_as_f32(cw: list) -> list:
    """Exact float32 view of make_conv_weights' output."""
    def cv(a):
        return bf16_bits_to_f32(a) if a.dtype == np.uint16 else a
    return [{site: {k: cv(v) for k, v in t.items()} for site, t in layer.items()} for layer in cw]


def weights_as_f32(w: dict) -> dict:
    """Exact float32 view of the stored weights (bf16 bits are upcast)."""
    def cv(a):
        return bf16_bits_to_f32(a) if a.dtype == np.uint16 else a
    out = {k: cv(v) for k, v in w.items() if k not in ("layers", "w_lm")}
    out["w_lm"] = out["embed"] if w["w_lm"] is w["embed"] else cv(w["w_lm"])
    out["layers"] = [{k: cv(v) for k, v in lw.items()} for lw in w["layers"]]
    return out


def as_f32(arrays):
    """Exact float32 values of storage-dtype arrays (bf16 bits are upcast)."""
    return [bf16_bits_to_f32(a) if a.dtype == np.uint16 else a for a in arrays]


def make_hidden(d: Dims, seed: int, req: int, start: int, n: int) -> List[np.ndarray]:
    """Verifier hidden states of request `req`, rows start..start+n-1, one array
    [n, Dt] per tapped layer.  Row values depend only on (seed, req, layer, row):
    rows come in blocks of 64, block b of layer l drawn from the stream keyed
    (2000+seed, 77, req, l, b)."""
    R = _HIDDEN_ROWS_PER_BLOCK
    dt = np.uint16 if d.dtype == "bf16" else np.float32
    b0, b1 = start // R, (start + n + R - 1) // R
    out = [np.empty((n, d.Dt), dt) for _ in range(d.L)]
    if n == 0:
        return out

    def work(job):
        l, b = job
        blk = _fill((R, d.Dt), [2000 + seed, 77, req, l, b], 1.0, 0.0, d.dtype)
        lo = max(start, b * R)
        hi = min(start + n, (b + 1) * R)
        out[l][lo - start:hi - start] = blk[lo - b * R:hi - b * R]

    jobs = [(l, b) for l in range(d.L) for b in range(b0, b1)]
    if len(jobs) <= 4:
        for j in jobs:
            work(j)
    else:
        list(_pool().map(work, jobs))
    return out


def make_suffix_hidden(d: Dims, seed: int, req: int, rnd: int, n: int) -> List[np.ndarray]:
    """Verifier features [n, Dt] per tapped layer for the n reusable rejected
    positions of request `req` in round `rnd` (a stream of its own: these are
    states of a branch that is not committed)."""
    out = []
    for l in range(d.L):
        out.append(_fill((n, d.Dt), [2000 + seed, 88, req, rnd, l], 1.0, 0.0, d.dtype) if n
                   else np.zeros((0, d.Dt), dtype=np.float32 if d.dtype == "f32" else np.uint16))
    return out


def draw_accepted(bs: int, rounds: int, B: int, seed: int) -> np.ndarray:
    """Accepted candidate counts n ~ U{0..B-1} per (round, request)."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([3000 + seed, 7])))
    return rng.integers(0, B, size=(rounds, bs))


def make_anchors(d: Dims, seed: int, bs: int) -> np.ndarray:
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([2000 + seed, 5])))
    return rng.integers(0, d.V, size=bs).astype(np.int32)


def draw_first_mismatch(kind: str, bs: int, B: int, seed: int) -> np.ndarray:
    """First mismatch position m per request, m in 0..B-1 (tau = m + 1).

    kind "uniform": m ~ U{0..B-1}; kind "geometric": tau = min(Geom(p), B)
    with p chosen so the clamped mean is 6.5."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([3000 + seed, 1])))
    if kind == "uniform":
        return rng.integers(0, B, size=bs).astype(np.int32)
    if kind == "geometric":
        tau = np.minimum(rng.geometric(GEOM_P_MEAN_6_5, size=bs), B)
        return (tau - 1).astype(np.int32)
    raise KeyError(kind)


def make_targets(cand: np.ndarray, m: np.ndarray, V: int, seed: int) -> np.ndarray:
    """Verifier argmax tokens t [bs, B] built so the first mismatch with the
    candidates c [bs, B-1] sits at m: t_j = c_{j+1} for j < m, t_m differs from
    c_{m+1} (when m < B-1), all other entries uniform."""
    bs, Bm1 = cand.shape
    B = Bm1 + 1
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([3000 + seed, 2])))
    t = rng.integers(0, V, size=(bs, B)).astype(np.int64)
    shift = rng.integers(0, V - 1, size=bs)
    for r in range(bs):
        mr = int(m[r])
        t[r, :mr] = cand[r, :mr]
        if mr < B - 1:
            t[r, mr] = (int(cand[r, mr]) + 1 + int(shift[r])) % V
    return t.astype(np.int32)


def make_sampling_logits(bs: int, B: int, V: int, seed: int, peaks: int = 4):
    """Drafter and verifier logit rows for speculative sampling at T > 0.

    Verifier row j (0..B-1) of request r is peaked: 2 N(0, 1) over the whole
    vocabulary plus U(6, 12) on `peaks` random ids.  Drafter row j (offset j,
    1..B-1) scores the same position as verifier row j-1: that row plus
    sigma_r N(0, 1) on every entry, sigma_r ~ U(0.3, 1.5) per request, and with
    probability 0.2 its peaks moved to other random ids (a wrong draft), so
    acceptance varies across offsets and requests.  Returns float32 arrays
    draft [bs, B-1, V] and target [bs, B, V]."""
    K = B - 1
    draft = np.empty((bs, K, V), dtype=np.float32)
    target = np.empty((bs, B, V), dtype=np.float32)
    for r in range(bs):
        rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([4000 + seed, r])))
        sigma = rng.uniform(0.3, 1.5)
        for j in range(B):
            row = 2.0 * rng.standard_normal(V)
            ids = rng.choice(V, size=min(peaks, V), replace=False)
            row[ids] += rng.uniform(6.0, 12.0, size=ids.size)
            target[r, j] = row
            if j < K:
                d = row + sigma * rng.standard_normal(V)
                if rng.random() < 0.2:
                    moved = rng.choice(V, size=ids.size, replace=False)
                    d[moved] += rng.uniform(6.0, 12.0, size=ids.size)
                    d[ids] -= row[ids] - 2.0 * rng.standard_normal(ids.size)
                draft[r, j] = d
    return draft, target
