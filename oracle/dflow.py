"""Float64 NumPy oracle of the DFlow relay (test infrastructure only).

Source: "DFlow 完全拆解：让验证器信息流穿过拒绝边界的块扩散投机解码"
(pinghaoyang.com.cn): the opening section (accepted prefix, first rejection,
bonus token; the 16-guessed / 4-accepted example), relay steps 1-3 (shared W_c
projection, one-position shift with the 10/11/12 example, MLP modulation and
the injection equation), and the inference-loop section (relay keyed by
absolute position, cleared each round, bound to the request).

Block indexing used throughout: offset 0 is the anchor at absolute position
P, offsets 1..B-1 hold the drafted candidates c_1..c_{B-1} at P+1..P+B-1.
After verification n candidates are accepted, candidate c_{n+1} is the first
rejection (replaced by the bonus token) and the next block's anchor (the
bonus) sits at P+n+1.
"""
from __future__ import annotations

from typing import Dict, List, Sequence, Tuple

import numpy as np

from .dflash import F, _f64, fuse_context, silu

LN_EPS = 1e-5


def layer_norm(x: np.ndarray, eps: float = LN_EPS) -> np.ndarray:
    """LayerNorm over the last axis, no affine: (x - mean) / sqrt(var + eps).

    The injection equation of relay step 3 normalises the verifier
    representation with LN; the page gives neither eps nor an affine part
    (reading: eps = 1e-5, no affine, population variance)."""
    x = _f64(x)
    mu = np.mean(x, axis=-1, keepdims=True)
    var = np.mean((x - mu) ** 2, axis=-1, keepdims=True)
    return (x - mu) / np.sqrt(var + eps)


def relay_plan(anchor_pos: int, n_accepted: int, B: int) -> List[Tuple[int, int, int]]:
    """Where the verifier states of a round's rejected suffix go.

    Returns (source block offset, absolute target position, next-block offset)
    for every reusable state, in order of position.

    * The reusable suffix starts one past the first rejection (the loop of the
      inference-loop pseudocode starts at accepted length + 1 in drafted-token
      numbering, i.e. block offset n + 2 here): the first rejected position's
      own state was computed on the wrong token.
    * Relay step 2: the verifier is a next-token predictor, so the state at
      absolute position q serves the prediction of position q + 1.
    * The next block starts at the bonus token, P + n + 1, so the state of
      block offset o lands at next-block offset o - n (always 2..B-1-n).
    """
    if not 0 <= n_accepted <= B - 1:
        raise ValueError("accepted count must be in 0..B-1")
    next_anchor = anchor_pos + n_accepted + 1
    plan = []
    for o in range(n_accepted + 2, B):
        q = anchor_pos + o
        target = q + 1
        plan.append((o, target, target - next_anchor))
    return plan


def relay_inputs(w: dict, d, rw: dict, hidden: Sequence[np.ndarray], bonus: int,
                 first_rejected: int) -> np.ndarray:
    """Next-round block inputs at the relay positions.

    hidden: L arrays [k, Dt], the verifier features of the k reusable suffix
    positions (all tapped layers), in position order.

    * Relay step 1: h = RMSNorm(W_c [H^(l1); ...; H^(lL)]), the shared fusion
      projection (same W_c, gain and eps as the context fusion).
    * Relay step 3: [beta; gamma] = MLP([E(bonus); E(first rejection); h]) and
      x = E_mask + beta * LN(h) + gamma.  The MLP is two bias-free layers of
      width D with a SiLU between them: W1 [D, 3D], W2 [2D, D]; the first D
      outputs are beta, the next D gamma (reading: the bracket order of the
      page's equation).
    Returns [k, D]."""
    h = fuse_context(w["w_c"], w["g_c"], hidden, d.rms_eps)
    k = h.shape[0]
    E = w["embed"]
    cond = np.concatenate([np.repeat(_f64(E[bonus])[None], k, 0),
                           np.repeat(_f64(E[first_rejected])[None], k, 0), h], axis=1)
    s = silu(cond @ _f64(rw["w1"]).T)
    bg = s @ _f64(rw["w2"]).T
    beta, gamma = bg[:, :d.D], bg[:, d.D:]
    return _f64(w["e_mask"])[None] + beta * layer_norm(h) + gamma


def block_inputs(w: dict, d, anchor: int, relay: Dict[int, np.ndarray]) -> np.ndarray:
    """Block input rows [B, D]: E[anchor], then the mask embedding, with relay
    rows substituted at their next-block offsets (inference-loop pseudocode:
    a position found in the relay cache gets the relayed input, any other
    position the plain mask embedding)."""
    x = np.stack([_f64(w["embed"][anchor])] + [_f64(w["e_mask"])] * (d.B - 1))
    for off, row in relay.items():
        x[off] = row
    return x


class RelayState:
    """Per-request relay cache keyed by next-block offset.  It lives for one
    round only (the pseudocode clears it after every verification) and is bound
    to the request, not to the batch."""

    def __init__(self):
        self.rows: Dict[int, Dict[int, np.ndarray]] = {}

    def set(self, r: int, n_accepted: int, B: int, x: np.ndarray) -> None:
        plan = relay_plan(0, n_accepted, B)
        if len(plan) != x.shape[0]:
            raise ValueError("relay rows do not match the reusable suffix")
        self.rows[r] = {off: x[i] for i, (_, _, off) in enumerate(plan)}

    def take(self, r: int) -> Dict[int, np.ndarray]:
        return self.rows.pop(r, {})
