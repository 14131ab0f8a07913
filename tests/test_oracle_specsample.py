"""Pins of the speculative-sampling oracle (lossless rejection sampling at
temperature T > 0, oracle/specsample.py) against facts fixed outside it:

* the generator equals numpy's Philox4x64-10 bit generator (a library routine);
* the defining property of the rejection rule: the emitted token has exactly
  the verifier's distribution, whatever the drafter's (closed form, summed
  over every draft and both outcomes), and the sampler reproduces it;
* the Gumbel-max draw reproduces softmax(l / T); the block stage of the
  two-stage draw is an inverse CDF over the block masses (exact on a grid of
  uniforms) and the composed draw reproduces the weights across blocks;
* the accepted length follows the product of per-offset acceptance masses
  sum_v min(q, p) (closed form) when the distributions do not depend on the
  prefix;
* special cases: q = p accepts every draft; T -> 0 reduces to the greedy
  longest-prefix scan of the DFlash inference loop (oracle.accept);
  1 <= tau <= B.
"""
import numpy as np
import pytest

import oracle
from oracle import specsample as ss

SIGMAS = 5.0  # Monte Carlo bounds: |empirical - exact| <= 5 standard errors (+ a small floor)


def _mc_bound(p, n):
    return SIGMAS * np.sqrt(np.maximum(p * (1 - p), 1e-4) / n) + 2e-3


def test_philox_matches_numpy_philox():
    # numpy's generator bumps its 256-bit counter before each block, so a
    # generator started at counter c - 1 produces block c first
    rng = np.random.default_rng(11)
    cases = [([1, 0, 0, 0], [0, 0]), ([5, 7, 11, 13], [123456789, 987654321]),
             ([2 ** 64 - 1, 3, 0, 0], [2 ** 63 + 5, 17])]
    for _ in range(5):
        cases.append(([int(x) for x in rng.integers(1, 2 ** 63, 4)], [int(x) for x in rng.integers(0, 2 ** 63, 2)]))
    for ctr, key in cases:
        prev = list(ctr)
        prev[0] -= 1  # ctr[0] >= 1 in every case: no borrow
        bg = np.random.Philox(counter=np.array(prev, dtype=np.uint64), key=np.array(key, dtype=np.uint64))
        want = [int(x) for x in bg.random_raw(4)]
        got = ss.philox4x64_10(np.array([ctr], dtype=np.uint64), np.array([key], dtype=np.uint64))[0]
        assert [int(x) for x in got] == want


def test_uniform_layout_against_numpy_philox():
    # indices 8..15 of (seed, stream, req, row) come from counter block
    # (1, row, req, 0): numpy started at (0, row, req, 0) produces it first;
    # index 8 + 2w + h takes the top 24 bits of half h (0 = high) of word w
    seed, stream, req, row = 99, 2, 5, 3
    bg = np.random.Philox(counter=np.array([0, row, req, 0], dtype=np.uint64),
                          key=np.array([seed, stream], dtype=np.uint64))
    words = [int(x) for x in bg.random_raw(4)]
    want = []
    for w in words:
        for half in (w >> 32, w & 0xFFFFFFFF):
            want.append(((half >> 8) + 0.5) / 2 ** 24)
    got = ss.uniforms(seed, stream, req, row, 16)[8:]
    assert list(got) == want


def test_uniforms_open_interval_24_bit():
    u = ss.uniforms(7, 1, 3, 2, 10001)
    assert u.shape == (10001,)
    assert np.all(u > 0) and np.all(u < 1)
    k = u * 2 ** 24 - 0.5
    assert np.array_equal(k, np.round(k))
    assert abs(u.mean() - 0.5) < 0.02
    # distinct streams, rows and requests give different sequences
    assert not np.array_equal(u, ss.uniforms(7, 2, 3, 2, 10001))
    assert not np.array_equal(u, ss.uniforms(7, 1, 4, 2, 10001))
    assert not np.array_equal(u, ss.uniforms(7, 1, 3, 3, 10001))


@pytest.mark.parametrize("V,seed", [(2, 0), (5, 1), (9, 2), (40, 3)])
def test_first_token_distribution_equals_target(V, seed):
    rng = np.random.default_rng(seed)
    q = rng.dirichlet(np.ones(V) * 0.7)
    p = rng.dirichlet(np.ones(V) * 0.7)
    # zeros on either side
    q[0] = 0.0
    q /= q.sum()
    p[-1] = 0.0
    p /= p.sum()
    assert np.allclose(ss.first_token_distribution(q, p), p, atol=2e-4)
    # drafter = verifier: nothing is replaced
    assert np.allclose(ss.first_token_distribution(p, p), p, atol=2e-4)


def test_gumbel_draw_matches_softmax():
    rng = np.random.default_rng(4)
    V, n = 6, 2500
    logits = rng.normal(size=(1, V)) * 1.5
    for temp in (1.0, 0.5):
        want = ss.softmax(logits, temp)[0]
        cnt = np.zeros(V)
        for s in range(n):
            cnt[ss.draft_tokens(logits, temp, s, 0)[0]] += 1
        assert np.all(np.abs(cnt / n - want) <= _mc_bound(want, n))


def test_sampler_emits_the_verifier_distribution():
    rng = np.random.default_rng(5)
    V, n, temp = 6, 2500, 1.0
    dl = rng.normal(size=(1, V)) * 1.2
    tl = rng.normal(size=(2, V)) * 1.2
    want = ss.softmax(tl, temp)[0]  # the row that scores offset 1
    cnt = np.zeros(V)
    for s in range(n):
        cand = ss.draft_tokens(dl, temp, s, 3)
        cnt[ss.spec_sample(dl, tl, cand, temp, s, 3)["tokens"][0]] += 1
    assert np.all(np.abs(cnt / n - want) <= _mc_bound(want, n))


def test_tau_follows_acceptance_masses():
    rng = np.random.default_rng(6)
    V, K, n, temp = 5, 3, 2500, 1.0
    row_q = rng.normal(size=V)
    row_p = rng.normal(size=V)
    dl = np.tile(row_q, (K, 1))
    tl = np.tile(row_p, (K + 1, 1))
    want = ss.tau_distribution(ss.softmax(dl, temp), ss.softmax(tl, temp))
    cnt = np.zeros(K + 1)
    for s in range(n):
        cand = ss.draft_tokens(dl, temp, s, 1)
        cnt[ss.spec_sample(dl, tl, cand, temp, s, 1)["tau"] - 1] += 1
    assert np.all(np.abs(cnt / n - want) <= _mc_bound(want, n))


def test_equal_distributions_accept_every_draft():
    rng = np.random.default_rng(7)
    V, K = 11, 7
    logits = rng.normal(size=(K + 1, V))
    for s in range(40):
        cand = ss.draft_tokens(logits[:K], 0.8, s, 0)
        # the drafter's row for offset j equals the verifier's row that scores it
        out = ss.spec_sample(logits[:K], logits[:K + 1], cand, 0.8, s, 0)
        assert out["tau"] == K + 1 and out["tokens"][:K] == [int(c) for c in cand]


def test_low_temperature_is_the_greedy_scan():
    rng = np.random.default_rng(8)
    V, K, temp = 50, 7, 1e-4
    for s in range(20):
        dl = rng.normal(size=(K, V))
        tl = rng.normal(size=(K + 1, V))
        # first mismatch at a drawn offset: copy the drafter's argmax rows into the verifier
        m = int(rng.integers(0, K + 1))
        for j in range(m):
            tl[j] = dl[j]
        cand = ss.draft_tokens(dl, temp, s, 0)
        assert np.array_equal(cand, dl.argmax(axis=1))
        out = ss.spec_sample(dl, tl, cand, temp, s, 0)
        tau, bonus = oracle.accept(cand, tl.argmax(axis=1))
        assert out["tau"] == tau
        assert out["tokens"] == [int(c) for c in cand[:tau - 1]] + [int(bonus)]


def test_replacement_comes_from_the_residual_and_tau_in_range():
    rng = np.random.default_rng(9)
    V, K, temp = 8, 5, 1.0
    seen = 0
    for s in range(200):
        dl = rng.normal(size=(K, V)) * 2
        tl = rng.normal(size=(K + 1, V)) * 2
        cand = ss.draft_tokens(dl, temp, s, 2)
        out = ss.spec_sample(dl, tl, cand, temp, s, 2)
        assert 1 <= out["tau"] <= K + 1
        n = out["accepted"]
        if n < K:
            seen += 1
            q = ss.softmax(dl, temp)[n]
            p = ss.softmax(tl, temp)[n]
            last = out["tokens"][-1]
            assert p[last] > q[last]
    assert seen > 50


def test_block_choice_is_the_inverse_cdf_of_the_block_masses():
    rng = np.random.default_rng(12)
    V = 3 * ss.BLOCK + 100
    w = rng.random(V) ** 8
    w[ss.BLOCK:2 * ss.BLOCK] = 0.0  # an empty block is never chosen
    mass = np.array([w[b * ss.BLOCK:(b + 1) * ss.BLOCK].sum() for b in range(4)])
    grid = 1 << 13
    counts = np.zeros(4)
    for u in (np.arange(grid) + 0.5) / grid:
        counts[ss.block_choice(w, u)] += 1
    assert counts[1] == 0
    assert np.all(np.abs(counts / grid - mass / mass.sum()) <= 1.0 / grid + 1e-12)


def test_two_stage_draw_across_blocks():
    V = 2 * ss.BLOCK + 7
    ids = np.array([5, ss.BLOCK - 1, ss.BLOCK, 2 * ss.BLOCK + 6, 123])
    logw = np.full(V, -np.inf)
    logw[ids] = np.log([0.3, 0.1, 0.25, 0.15, 0.2])
    want = np.exp(logw[ids]) / np.exp(logw[ids]).sum()
    n = 1500
    cnt = np.zeros(ids.size)
    for s_ in range(n):
        v = ss.two_stage_draw(logw, s_, ss.STREAM_DRAFT_BLOCK, ss.STREAM_DRAFT, 0, 0)
        cnt[int(np.flatnonzero(ids == v)[0])] += 1
    assert np.all(np.abs(cnt / n - want) <= _mc_bound(want, n))


# ---- plain definitions (the distributions the GPU's draws are tested against)

@pytest.mark.parametrize("V,seed", [(5, 0), (64, 1), (1024, 2)])
def test_plain_emitted_token_is_the_verifier_distribution(V, seed):
    """The rejection rule's first emitted token follows p exactly (the
    losslessness the pages attribute to rejection sampling), also where q or p
    has zeros, and the grid form of the same sum agrees."""
    rng = np.random.default_rng(seed)
    q = rng.dirichlet(np.full(V, 0.3))
    p = rng.dirichlet(np.full(V, 0.3))
    q[rng.integers(0, V, size=max(1, V // 5))] = 0.0
    q /= q.sum()
    p[rng.integers(0, V, size=max(1, V // 7))] = 0.0
    p /= p.sum()
    got = ss.emitted_first_token_plain(q, p)
    assert np.allclose(got, p, atol=1e-12, rtol=0)
    assert np.allclose(got, ss.first_token_distribution(q, p), atol=2e-4)
    # q = p keeps every draft: the emitted token is the draft itself
    assert np.allclose(ss.emitted_first_token_plain(p, p), p, atol=1e-15)


def test_plain_draft_distribution_is_softmax_at_temperature():
    l = np.array([0.0, 1.0, 2.0, -1.0])
    for T in (0.5, 1.0, 3.0):
        e = np.exp(l / T)
        assert np.allclose(ss.draft_distribution(l, T), e / e.sum(), rtol=1e-14)


@pytest.mark.parametrize("K", [1, 3, 7])
def test_plain_tau_distribution_matches_product_form_and_enumeration(K):
    """tau from the definition equals the product form prod beta (1 - beta)
    with beta_j = sum min(q_j, p_{j-1}), and, for a 3-token vocabulary, the
    brute-force sum over every drafted sequence of its keep probabilities."""
    rng = np.random.default_rng(K)
    V = 3
    q = rng.dirichlet(np.ones(V), size=K)
    p = rng.dirichlet(np.ones(V), size=K + 1)
    plain = ss.tau_distribution_plain(q, p)
    assert np.isclose(plain.sum(), 1.0)
    assert np.allclose(plain, ss.tau_distribution(q, p), atol=1e-14)
    import itertools
    brute = np.zeros(K + 1)
    for xs in itertools.product(range(V), repeat=K):
        # drafted sequence xs: the walk keeps offsets 1..n and stops at n+1
        # (drafts after the stop only carry their own probability)
        for n in range(K + 1):
            prob = 1.0
            for j in range(n):
                prob *= q[j][xs[j]] * min(1.0, p[j][xs[j]] / q[j][xs[j]])
            if n < K:
                prob *= q[n][xs[n]] * (1.0 - min(1.0, p[n][xs[n]] / q[n][xs[n]]))
                for j in range(n + 1, K):
                    prob *= q[j][xs[j]]
            brute[n] += prob
    assert np.allclose(brute, plain, atol=1e-12)
