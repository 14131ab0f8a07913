"""Float64 NumPy oracle of the DFlash 2 additions (test infrastructure only):
the path selector and the two-tap dynamic depthwise convolution.

Source: "DFlash 2：正确 token 已在候选里，选一条连贯的路就好".

Path selector — the section on the first insight (selection is cheaper than
prediction: keep the top-16 candidates of every position, score every
adjacent candidate pair with a low-rank bilinear term, then walk the
precomputed scores greedily along the best successor), Tables 1-2 (top-16
recall, the selector's cost).  Readings (the page leaves them open):
  * U_t(b) is the drafter's raw logit of candidate b at position t.
  * H(h_t) = sigmoid(W_H h_t), W_H [256, D], h_t the final normed hidden state
    of position t (the LM head's input); the page calls H a gate from the
    context hidden state.
  * The first drafted position scores its candidates against the anchor
    (a = the last verified token).
  * Ties go to the lower candidate rank.

Two-tap convolution — the section on the second insight (suffix decay is a
local problem): Conv_k(x)_t = k_{t,0} * x_t + k_{t,1} * x_{t-1} along the
block, the taps being a base kernel plus a small correction computed from the
current hidden state, one correction per 16 channels, the block's first
position reading the last verified token; inserted before and after the
attention and FFN sub-layers of every layer (16.5M extra parameters at the
5-layer drafter).  Readings:
  * k_{t,j}[c] = kbase_j[c] + (W_j x_t)[c // 16] with W_j [D/16, D], linear,
    no bias; x_t is the convolution's own input row.
  * Block offsets are numbered from the anchor: the first drafted position
    (offset 1) reads the anchor (offset 0), the last verified token; the
    anchor has no left neighbour in the block and its left tap reads zero.
  * Four sites per layer: the normed attention input, the attention output
    (after W_o) before the residual add, the normed FFN input, and the FFN
    output before the residual add.
"""
from __future__ import annotations

from typing import List, Tuple

import numpy as np

from .dflash import F, _f64


def gate(w_h: np.ndarray, h: np.ndarray) -> np.ndarray:
    """H(h) = sigmoid(W_H h) per row: h [T, D] -> [T, R]."""
    z = _f64(h) @ _f64(w_h).T
    return 1.0 / (1.0 + np.exp(-z))


def pair_scores(u_t: np.ndarray, prev_ids: np.ndarray, ids: np.ndarray, A: np.ndarray, Bt: np.ndarray,
                g_t: np.ndarray) -> np.ndarray:
    """S_t(a, b) = U_t(b) + <A(a) * H(h_t), B(b)> for every a in prev_ids and
    b in ids: [len(prev_ids), len(ids)].  A and Bt are the two compact
    embedding tables [V, R]; u_t holds U_t of the candidates in `ids`."""
    left = _f64(A)[np.asarray(prev_ids)] * _f64(g_t)[None]      # [na, R]
    right = _f64(Bt)[np.asarray(ids)]                              # [nb, R]
    return _f64(u_t)[None] + left @ right.T


def walk(first: np.ndarray, tables: List[np.ndarray]) -> List[int]:
    """Greedy best-successor walk over precomputed scores: `first` [k] scores
    the candidates of the first position (against the anchor); tables[t-1]
    [k, k] scores position t+1's candidates (columns) after each candidate of
    position t (rows).  Returns the chosen candidate rank per position; ties to
    the lower rank (first maximum)."""
    path = [int(np.argmax(first))]
    for tab in tables:
        path.append(int(np.argmax(tab[path[-1]])))
    return path


CONV_SITES = ("attn_in", "attn_out", "ffn_in", "ffn_out")


def two_tap_conv(x: np.ndarray, w: np.ndarray, kbase: np.ndarray) -> np.ndarray:
    """Two-tap dynamic depthwise convolution along the block.

    x [B, D] rows in block-offset order; w [2 * D/16, D] holds W_0 (first D/16
    rows) and W_1; kbase [2, D].  Returns y [B, D] with
    y_t = k_{t,0} * x_t + k_{t,1} * x_{t-1}, x_{-1} = 0."""
    x = _f64(x)
    B, D = x.shape
    G = D // 16
    z = x @ _f64(w).T
    k0 = _f64(kbase[0])[None] + np.repeat(z[:, :G], 16, axis=1)
    k1 = _f64(kbase[1])[None] + np.repeat(z[:, G:], 16, axis=1)
    left = np.zeros_like(x)
    left[1:] = x[:-1]
    return k0 * x + k1 * left


def draft_block_conv(w: dict, d, cache, anchor: int, conv, block_inputs=None) -> dict:
    """The DFlash draft forward with the two-tap convolution at the four sites
    of every layer.  conv: per layer a dict site -> {"w", "kbase"}."""
    from .dflash import draft_block

    def hook(site):
        return lambda v: two_tap_conv(v, site["w"], site["kbase"])
    hooks = [tuple(hook(layer[s]) for s in CONV_SITES) for layer in conv]
    return draft_block(w, d, cache, anchor, block_inputs, conv=hooks)


def conv_param_count(D: int, layers: int) -> int:
    """Extra parameters of the convolution: per site two correction matrices
    [D/16, D] and the two base kernels [D]."""
    return layers * len(CONV_SITES) * (2 * (D // 16) * D + 2 * D)


def select_path(anchor: int, cand: np.ndarray, u: np.ndarray, A: np.ndarray, Bt: np.ndarray,
                gates: np.ndarray) -> Tuple[np.ndarray, np.ndarray, List[np.ndarray]]:
    """The selector for one block.

    cand [T, k] candidate ids per drafted position (T = B-1, rank order),
    u [T, k] their logits, gates [T, R] = H(h_t).  All pair tables are computed
    first (they do not depend on the path); then the greedy walk.
    Returns (path ids [T], first-position scores [k], tables [T-1] of [k, k])."""
    T = cand.shape[0]
    first = pair_scores(u[0], np.array([anchor]), cand[0], A, Bt, gates[0])[0]
    tables = [pair_scores(u[t], cand[t - 1], cand[t], A, Bt, gates[t]) for t in range(1, T)]
    ranks = walk(first, tables)
    path = np.array([cand[t][ranks[t]] for t in range(T)], dtype=np.int32)
    return path, first, tables
