"""Model and workload shapes.

Dimensions follow the Qwen3-4B / Qwen3-8B shaped drafters and the tiny fp32
drafter used for CPU-seconds checks.  "Shaped" means dimensions only: no
QK-norm, no biases, no sliding window.  Embedding and LM head are tied in every
synthetic model here (the library also accepts untied heads).
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List

import numpy as np


@dataclass(frozen=True)
class Dims:
    name: str
    dtype: str          # "f32" or "bf16": storage dtype of weights and inputs
    D: int              # drafter hidden size
    L: int              # tapped target layers
    Dt: int             # target hidden size per tapped layer
    N: int              # drafter layers
    Hq: int             # query heads
    Hkv: int            # key/value heads
    hd: int             # head dim
    I: int              # SwiGLU intermediate size
    V: int              # vocabulary size
    B: int              # block size: anchor + (B-1) masks
    rope_base: float = 10000.0
    rms_eps: float = 1e-6
    use_rope: bool = True

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv


@dataclass(frozen=True)
class Workload:
    """One steady-state draft step over `bs` requests.

    Request r already holds `ctx[r] - n_new[r]` fused context tokens; the step
    fuses `n_new[r]` more (the tokens committed by the previous round), drafts
    a block at absolute positions ctx[r]..ctx[r]+B-1 and runs acceptance.
    """
    dims: Dims
    bs: int
    ctx: List[int]
    n_new: List[int]
    seed: int
    note: str = ""
    rounds: int = 1     # draft-verify rounds (the relay workload iterates)


def _tiny(B=8, L=3) -> Dims:
    return Dims("tiny", "f32", D=256, L=L, Dt=256, N=2, Hq=4, Hkv=4, hd=64,
                I=512, V=1024, B=B)


QWEN3_4B = Dims("qwen3_4b", "bf16", D=2560, L=5, Dt=2560, N=5, Hq=32, Hkv=8,
                hd=128, I=9728, V=151936, B=16)
QWEN3_8B = Dims("qwen3_8b", "bf16", D=4096, L=5, Dt=4096, N=5, Hq=32, Hkv=8,
                hd=128, I=12288, V=151936, B=16)

# Geometric acceptance with clamped mean 6.5 on {1..16}: p solves
# sum_{t=1}^{16} t p (1-p)^(t-1) + 16 (1-p)^16 = 6.5.
GEOM_P_MEAN_6_5 = 0.1401


def clamped_geom_mean(p: float, B: int) -> float:
    q = 1.0 - p
    return sum(t * p * q ** (t - 1) for t in range(1, B)) + B * q ** (B - 1)


def _tau_geometric(rng: np.random.Generator, n: int, B: int) -> List[int]:
    return [int(min(rng.geometric(GEOM_P_MEAN_6_5), B)) for _ in range(n)]


def get_config(name: str) -> Workload:
    """Build a workload by name; every random draw is seeded."""
    if name == "tiny":
        # 64 context tokens, prefilled in one fuse call (n_new = ctx).
        return Workload(_tiny(), bs=1, ctx=[64], n_new=[64], seed=1,
                        note="tiny fp32 drafter, prefill fuse of 64 tokens")
    if name == "qwen3_4b_bs1":
        rng = np.random.Generator(np.random.PCG64(2002))
        n_new = int(rng.integers(1, 17))
        return Workload(QWEN3_4B, bs=1, ctx=[2048], n_new=[n_new], seed=2,
                        note="Qwen3-4B-shaped drafter, ctx 2048, tau_prev ~ U{1..16}")
    if name == "qwen3_8b_bs1":
        return Workload(QWEN3_8B, bs=1, ctx=[4096], n_new=[7], seed=4,
                        note="Qwen3-8B-shaped drafter, bs 1, ctx 4096, 7 new tokens")
    if name == "qwen3_8b_bs32":
        rng = np.random.Generator(np.random.PCG64(2003))
        ctx = [int(c) for c in rng.integers(512, 8193, size=32)]
        n_new = _tau_geometric(rng, 32, 16)
        return Workload(QWEN3_8B, bs=32, ctx=ctx, n_new=n_new, seed=3,
                        note="Qwen3-8B-shaped drafter, bs 32 ragged, ctx ~ U{512..8192}, "
                             "tau_prev ~ clamped geometric mean 6.5")
    if name == "dflow_relay":
        # Tiny drafter with 5 tapped target layers and B = 16; 8 requests
        # prefilled with 64 context tokens, then 64 draft-verify rounds with
        # accepted counts drawn from U{0..15}.
        return Workload(_tiny(B=16, L=5), bs=8, ctx=[64] * 8, n_new=[64] * 8, seed=5,
                        note="DFlow relay on the tiny fp32 drafter, L 5, B 16, bs 8, 64 rounds",
                        rounds=64)
    if name == "dflash2_select":
        # Tiny drafter with B = 16, 16 requests prefilled with 64 context tokens;
        # top-16 candidates per position feed the path selector.
        return Workload(_tiny(B=16), bs=16, ctx=[64] * 16, n_new=[64] * 16, seed=6,
                        note="DFlash 2 path selector on the tiny fp32 drafter, B 16, bs 16")
    raise KeyError(name)


CONFIGS = ("tiny", "qwen3_4b_bs1", "qwen3_8b_bs1", "qwen3_8b_bs32", "dflow_relay", "dflash2_select")
