"""Float64 NumPy oracle of lossless speculative sampling at temperature T > 0
(test infrastructure only).

Sources: "DFlash 投机解码：块扩散草稿与 KV 注入", section 四 (the inference loop
resamples the rejected position from the target distribution and the last
position yields the bonus token); "DFlash 2：正确 token 已在候选里，选一条连贯的路就好"
(the introduction and the selector section: outputs stay lossless through
rejection sampling, which restores the target distribution; the comparison
section samples at temperature 1.0).

The pages name the step but do not write it out.  Reading taken: the standard
rejection rule of speculative sampling.  With drafter distributions q_j over
the vocabulary for block offsets j = 1..K (K = B-1) and verifier distributions
p_j for the token after offset j (j = 0..K; p_j is the distribution of the
token at offset j+1, the same layout as the greedy targets t_j):
  * the drafted token at offset j is x_j ~ q_j, drawn by the Gumbel-max rule
    argmax_v (logit_v / T + G_v), G_v standard Gumbel;
  * walking j = 1..K, x_j is accepted when r_j * q_j(x_j) < p_{j-1}(x_j),
    r_j ~ U(0, 1), i.e. with probability min(1, p/q);
  * at the first rejection j the emitted token is drawn from the residual
    norm(max(0, p_{j-1} - q_j)) and the block stops; when all K are accepted
    the bonus token is drawn from p_K;
  * tau = accepted + 1 (the replacement or bonus token counts, as in the
    greedy scan).
Distributions are softmax(logits / T) for both models at the same temperature
(no top-p / top-k truncation).

Every categorical draw (the drafted tokens, the replacement, the bonus) is taken
in two stages, an exact composition: the vocabulary is cut into blocks of
BLOCK consecutive ids; a block b is chosen by inverse CDF over the block masses
with one uniform (cum_{b-1} <= u S < cum_b), then an id within b by Gumbel-max
(argmax of log-weight + Gumbel noise, ties to the lower id), so
P(v) = (mass_b / S)(w_v / mass_b) = w_v / S.  The pages fix the distribution,
not the sampling algorithm; this one needs generator output for one block of
ids per draw instead of the whole vocabulary.

Random numbers come from one counter-based generator, Philox4x64-10 (Salmon,
Moraes, Dror, Shaw, "Parallel random numbers: as easy as 1, 2, 3", SC 2011;
the generator behind numpy.random.Philox), with key (seed, stream) and counter
(v // 8, row, request, 0).  The output block holds four 64-bit words; index v
takes word (v % 8) // 2, its high 32-bit half for even v and its low half for
odd v, and keeps the top 24 bits k of that half: u = (k + 0.5) * 2^-24 in
(0, 1).  Streams: 0 drafted tokens, Gumbel noise (row = offset - 1, index =
token id); 1 acceptance draws (row 0, index = offset - 1); 2 the replacement /
bonus draw, Gumbel noise (row 0, index = token id); 3 and 4 the block choice
of the drafted tokens (row = offset - 1) and of the replacement / bonus (row
0), index 0.

A rejection implies p(x) < q(x) for the drafted x, so the residual has
positive mass in exact arithmetic; should rounding leave it empty, the
replacement is drawn from the verifier's row with the same random numbers.
"""
from __future__ import annotations

from typing import Dict

import numpy as np

_M32 = np.uint64(0xFFFFFFFF)
_S32 = np.uint64(32)
PHILOX_M = (np.uint64(0xD2E7470EE14C6C93), np.uint64(0xCA5A826395121157))
PHILOX_W = (np.uint64(0x9E3779B97F4A7C15), np.uint64(0xBB67AE8584CAA73B))

STREAM_DRAFT, STREAM_ACCEPT, STREAM_RESIDUAL, STREAM_DRAFT_BLOCK, STREAM_RESIDUAL_BLOCK = 0, 1, 2, 3, 4
BLOCK = 16384  # vocabulary ids per block of the two-stage draw


def _mulhilo64(a, b):
    """(high, low) 64-bit halves of the 128-bit product of uint64 arrays."""
    al, ah = a & _M32, a >> _S32
    bl, bh = b & _M32, b >> _S32
    ll, lh, hl, hh = al * bl, al * bh, ah * bl, ah * bh
    mid = (ll >> _S32) + (lh & _M32) + (hl & _M32)
    lo = (ll & _M32) | ((mid & _M32) << _S32)
    hi = hh + (lh >> _S32) + (hl >> _S32) + (mid >> _S32)
    return hi, lo


def philox4x64_10(ctr: np.ndarray, key: np.ndarray) -> np.ndarray:
    """Philox4x64 with 10 rounds: ctr [..., 4], key [..., 2] (uint64) -> [..., 4]
    uint64.  Each round forms the 128-bit products of words 0 and 2 with the two
    round multipliers, mixes their high halves with words 1 and 3 and the key,
    and bumps the key by the two Weyl constants."""
    c = [np.asarray(ctr[..., i], dtype=np.uint64) for i in range(4)]
    k0 = np.asarray(key[..., 0], dtype=np.uint64)
    k1 = np.asarray(key[..., 1], dtype=np.uint64)
    with np.errstate(over="ignore"):
        for rnd in range(10):
            hi0, lo0 = _mulhilo64(PHILOX_M[0], c[0])
            hi1, lo1 = _mulhilo64(PHILOX_M[1], c[2])
            c = [hi1 ^ c[1] ^ k0, lo1, hi0 ^ c[3] ^ k1, lo0]
            if rnd < 9:
                k0 = k0 + PHILOX_W[0]
                k1 = k1 + PHILOX_W[1]
    return np.stack(c, axis=-1)


def uniforms(seed: int, stream: int, req: int, row: int, n: int) -> np.ndarray:
    """n uniforms in (0, 1) (float64, 24-bit resolution) for indices 0..n-1 of
    (seed, stream, request, row): eight per generator block, one per 32-bit
    half of its four words (high half first)."""
    blocks = (n + 7) // 8
    ctr = np.zeros((blocks, 4), dtype=np.uint64)
    ctr[:, 0] = np.arange(blocks, dtype=np.uint64)
    ctr[:, 1] = row
    ctr[:, 2] = req
    key = np.broadcast_to(np.array([seed, stream], dtype=np.uint64), (blocks, 2))
    x = philox4x64_10(ctr, key)
    halves = np.stack([x >> _S32, x & _M32], axis=-1).reshape(-1)[:n]
    return ((halves >> np.uint64(8)).astype(np.float64) + 0.5) * 2.0 ** -24


def gumbel(u: np.ndarray) -> np.ndarray:
    """Standard Gumbel draws from uniforms in (0, 1)."""
    return -np.log(-np.log(u))


def softmax(logits: np.ndarray, temp: float) -> np.ndarray:
    z = np.asarray(logits, dtype=np.float64) / float(temp)
    z = z - z.max(axis=-1, keepdims=True)
    e = np.exp(z)
    return e / e.sum(axis=-1, keepdims=True)


def argmax_low(v: np.ndarray) -> int:
    """Index of the maximum, the lowest index among equal maxima."""
    return int(np.flatnonzero(v == v.max())[0])


# The three decisions of the rejection rule (module level, one place each).
def verifier_row(j: int) -> int:
    """Row of the verifier logits that scores the token drafted at offset j
    (1-based): the verifier's distribution after offset j - 1."""
    return j - 1


def accepts(r: float, q_x: float, p_x: float) -> bool:
    """Keep the drafted token x when r * q(x) < p(x) (probability min(1, p/q))."""
    return r * q_x < p_x


def residual(p_row: np.ndarray, q_row: np.ndarray) -> np.ndarray:
    """Unnormalised replacement distribution after a rejection: max(0, p - q)."""
    return np.maximum(p_row - q_row, 0.0)


def block_choice(weights: np.ndarray, u: float) -> int:
    """Inverse CDF over the masses of the BLOCK-id blocks of `weights` (>= 0):
    the block b with cum_{b-1} <= u * S < cum_b."""
    w = np.asarray(weights, dtype=np.float64)
    mass = np.add.reduceat(w, np.arange(0, w.size, BLOCK))
    cum = np.cumsum(mass)
    return min(int(np.searchsorted(cum, u * cum[-1], side="right")), mass.size - 1)


def two_stage_draw(logw: np.ndarray, seed: int, stream_block: int, stream_entry: int, req: int, row: int) -> int:
    """Id v with probability exp(logw_v) / sum_v exp(logw_v) (logw may hold
    -inf): a block by block_choice with uniform 0 of stream_block, then the
    Gumbel-max over that block's ids with the noise of index v from
    stream_entry."""
    logw = np.asarray(logw, dtype=np.float64)
    with np.errstate(under="ignore"):
        w = np.exp(logw - logw.max())
    b = block_choice(w, uniforms(seed, stream_block, req, row, 1)[0])
    lo, hi = b * BLOCK, min(logw.size, (b + 1) * BLOCK)
    g = gumbel(uniforms(seed, stream_entry, req, row, hi)[lo:])
    return lo + argmax_low(logw[lo:hi] + g)


def draft_tokens(draft_logits: np.ndarray, temp: float, seed: int, req: int) -> np.ndarray:
    """x_j ~ softmax(l_j / T), one row per drafted offset j (row j - 1 of the
    generator counters)."""
    K, V = draft_logits.shape
    out = np.zeros(K, dtype=np.int64)
    for j in range(K):
        out[j] = two_stage_draw(np.asarray(draft_logits[j], dtype=np.float64) / temp, seed, STREAM_DRAFT_BLOCK,
                                STREAM_DRAFT, req, j)
    return out


def spec_sample(draft_logits: np.ndarray, target_logits: np.ndarray, cand: np.ndarray, temp: float,
                seed: int, req: int) -> Dict[str, object]:
    """One block of speculative sampling for one request.

    draft_logits [K, V] (offsets 1..K), target_logits [K+1, V] (row j = the
    verifier's logits after offset j), cand [K] the drafted tokens.  Returns the
    emitted tokens (accepted candidates, then the replacement or bonus token),
    tau and the number accepted."""
    q = softmax(draft_logits, temp)
    p = softmax(target_logits, temp)
    K, V = q.shape
    r = uniforms(seed, STREAM_ACCEPT, req, 0, K)
    n = 0
    while n < K:
        x = int(cand[n])
        if accepts(r[n], q[n, x], p[verifier_row(n + 1), x]):
            n += 1
        else:
            break
    row = verifier_row(n + 1) if n < K else K
    w = residual(p[row], q[n]) if n < K else np.zeros(V)
    if np.any(w > 0):
        with np.errstate(divide="ignore"):
            logw = np.where(w > 0, np.log(np.where(w > 0, w, 1.0)), -np.inf)
    else:  # the bonus token, or an empty residual (rounding only)
        logw = np.asarray(target_logits[row], dtype=np.float64) / temp
    last = two_stage_draw(logw, seed, STREAM_RESIDUAL_BLOCK, STREAM_RESIDUAL, req, 0)
    return {"tokens": [int(t) for t in cand[:n]] + [last], "tau": n + 1, "accepted": n}


def first_token_distribution(q: np.ndarray, p: np.ndarray, grid: int = 1 << 14) -> np.ndarray:
    """Distribution of the first emitted token for a block with one drafted
    token (q over the vocabulary for offset 1, p the verifier's row that
    scores it), summed over every draft x ~ q and both outcomes of the
    acceptance draw; the probability of keeping x is the measure of the r in
    (0, 1) that `accepts` keeps, taken on a midpoint grid of `grid` points
    (exact up to 1/grid), and a rejected draft is replaced from
    norm(residual(p, q))."""
    q = np.asarray(q, dtype=np.float64)
    p = np.asarray(p, dtype=np.float64)
    V = q.shape[0]
    r = (np.arange(grid) + 0.5) / grid
    keep = np.array([np.mean(accepts(r, q[x], p[x])) if q[x] > 0 else 0.0 for x in range(V)])
    w = residual(p, q)
    resid = w / w.sum() if w.sum() > 0 else np.zeros_like(w)
    reject = float(np.sum(q * (1.0 - keep)))
    return q * keep + reject * resid


def tau_distribution(q: np.ndarray, p: np.ndarray) -> np.ndarray:
    """Exact distribution of tau when the drafter's and the verifier's
    distributions do not depend on the drafted prefix (q [K, V], p [K+1, V]):
    offset j is accepted with probability beta_j = sum_v min(q_j(v),
    p_{j-1}(v)), independently, so P(tau = n+1) = prod_{i<=n} beta_i *
    (1 - beta_{n+1}) and P(tau = K+1) = prod_i beta_i."""
    q = np.asarray(q, dtype=np.float64)
    p = np.asarray(p, dtype=np.float64)
    K = q.shape[0]
    beta = np.minimum(q, p[:K]).sum(axis=1)
    out = np.zeros(K + 1)
    run = 1.0
    for n in range(K):
        out[n] = run * (1.0 - beta[n])
        run *= beta[n]
    out[K] = run
    return out


# --------------------------------------------------------------------------
# Plain definitions (no two-stage draw, no generator): the distributions the
# sampling step must produce, written out from the rejection rule itself.
# --------------------------------------------------------------------------

def draft_distribution(draft_row: np.ndarray, temp: float) -> np.ndarray:
    """Distribution of a drafted token: softmax(l / T) over the whole
    vocabulary (the drafter's temperature-T distribution)."""
    return softmax(draft_row, temp)


def emitted_first_token_plain(q: np.ndarray, p: np.ndarray) -> np.ndarray:
    """Distribution of the first token the rejection rule emits, from its
    definition: the draft x ~ q is kept with probability min(1, p(x) / q(x));
    otherwise the token is drawn from norm(max(0, p - q)).  So
      P(v) = q(v) min(1, p(v) / q(v)) + P(reject) max(0, p(v) - q(v)) / Z,
      P(reject) = 1 - sum_x q(x) min(1, p(x) / q(x)),  Z = sum max(0, p - q).
    (Its value is p itself, the losslessness of the rule.)"""
    q = np.asarray(q, dtype=np.float64)
    p = np.asarray(p, dtype=np.float64)
    with np.errstate(divide="ignore", invalid="ignore"):
        keep = np.where(q > 0, np.minimum(1.0, p / np.where(q > 0, q, 1.0)), 0.0)
    kept = q * keep
    reject = 1.0 - kept.sum()
    w = np.maximum(p - q, 0.0)
    z = w.sum()
    return kept + (reject * w / z if z > 0 else 0.0)


def tau_distribution_plain(q: np.ndarray, p: np.ndarray) -> np.ndarray:
    """Distribution of tau (kept drafts + 1) from the definition, when every
    offset j drafts from q_j and is checked against p_{j-1} independently of
    the prefix: offset j survives with probability
    a_j = sum_x q_j(x) min(1, p_{j-1}(x) / q_j(x)), and the walk stops at the
    first offset that does not survive (tau = K + 1 when all K survive)."""
    q = np.asarray(q, dtype=np.float64)
    p = np.asarray(p, dtype=np.float64)
    K = q.shape[0]
    a = np.array([float(np.sum(q[j] * np.minimum(1.0, p[j] / np.where(q[j] > 0, q[j], 1.0))))
                  for j in range(K)])
    out = np.zeros(K + 1)
    alive = 1.0
    for j in range(K):
        out[j] = alive * (1.0 - a[j])
        alive *= a[j]
    out[K] = alive
    return out
