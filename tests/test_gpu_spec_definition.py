"""Speculative sampling on the GPU against the plain definition of the
distributions it must produce (not the oracle's two-stage algorithm).

Many draws from dflash_spec_draft / dflash_spec_verify are binned and compared
by a chi-square goodness-of-fit test with the exact distributions written out
in oracle/specsample.py from the rejection rule itself:
  * a drafted token follows softmax(l / T) (draft_distribution);
  * the first emitted token (the kept draft at offset 1, or its replacement
    from norm(max(0, p - q))) follows the verifier's distribution p
    (emitted_first_token_plain; the losslessness the DFlash 2 page attributes
    to rejection sampling);
  * tau follows the survival product of the per-offset keep probabilities
    (tau_distribution_plain).
Each case takes >= 10^5 draws (64 requests per call with distinct request
ids, many seeds; every row of a call carries the same logits, so draws are
identically distributed and independent through the counter generator).  Bins
whose expected count is below 5 are pooled.  A case fails when the chi-square
p-value is below 1e-4 (a correct sampler fails one such case with probability
1e-4; the inputs are seeded, so a run is reproducible)."""
import dataclasses

import numpy as np
import pytest

import synth
from oracle import specsample as ss
from synth.configs import _tiny
from tests._gpu import GpuDraft, log

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("needs a GPU", allow_module_level=True)

P_MIN = 1e-4
NREQ = 64
B = 16
K = B - 1


def _chi2(counts, probs):
    """Chi-square p-value of observed counts against probabilities, pooling
    bins with expected count < 5 into one."""
    from scipy.stats import chi2
    counts = np.asarray(counts, dtype=np.float64)
    n = counts.sum()
    exp = np.asarray(probs, dtype=np.float64) * n
    big = exp >= 5.0
    obs = list(counts[big])
    ex = list(exp[big])
    if (~big).any():
        obs.append(counts[~big].sum())
        ex.append(exp[~big].sum())
    obs, ex = np.array(obs), np.array(ex)
    if ex[-1] == 0:  # nothing expected outside the large bins
        assert obs[-1] == 0, "draws where the distribution has no mass"
        obs, ex = obs[:-1], ex[:-1]
    stat = float(np.sum((obs - ex) ** 2 / ex))
    dof = len(ex) - 1
    return stat, dof, float(chi2.sf(stat, dof))


def _rows(V, seed):
    """One drafter row (offset 1) and one verifier row (after the anchor) of
    the seeded sampling inputs, tiled over every request and offset."""
    dl, tl = synth.make_sampling_logits(1, 2, V, seed=seed)
    q_row, p_row = dl[0, 0], tl[0, 0]
    draft = np.broadcast_to(q_row, (NREQ, K, V)).astype(np.float32)
    target = np.broadcast_to(p_row, (NREQ, B, V)).astype(np.float32)
    return q_row, p_row, torch.from_numpy(np.ascontiguousarray(draft)).cuda(), \
        torch.from_numpy(np.ascontiguousarray(target)).cuda()


def _drafter(V):
    d = dataclasses.replace(_tiny(B=B), V=V)
    return GpuDraft(d, synth.make_weights(d, 0), max_ctx=64, max_slots=1, max_batch=NREQ)


CASES = [(64, 0.7), (64, 1.0), (1024, 0.7), (1024, 1.0)]


@pytest.mark.parametrize("V,temp", CASES)
def test_spec_draft_follows_softmax(V, temp):
    n_calls = -(-100_000 // (NREQ * K))
    log(f"[spec-def] draft V {V} T {temp}: {n_calls} calls x {NREQ * K} draws")
    g = _drafter(V)
    try:
        q_row, _, dlg, _ = _rows(V, 21)
        req = torch.arange(NREQ, dtype=torch.int32, device="cuda")
        cand = torch.zeros((NREQ, K), dtype=torch.int32, device="cuda")
        counts = torch.zeros(V, dtype=torch.int64, device="cuda")
        for c in range(n_calls):
            g.dr.spec_draft(NREQ, dlg, temp, 1000 + c, req, cand, None)
            counts += torch.bincount(cand.reshape(-1).long(), minlength=V)[:V]
        torch.cuda.synchronize()
        counts = counts.cpu().numpy()
        assert counts.sum() == n_calls * NREQ * K
        stat, dof, pv = _chi2(counts, ss.draft_distribution(q_row, temp))
        log(f"[spec-def] draft V {V} T {temp}: chi2 {stat:.1f} on {dof} dof, p = {pv:.3g}")
        assert pv >= P_MIN, f"drafted tokens do not follow softmax(l/T): p = {pv:.3g}"
    finally:
        g.close()


@pytest.mark.parametrize("V,temp", CASES)
def test_spec_verify_emits_the_verifier_distribution(V, temp):
    n_calls = -(-100_000 // NREQ)
    log(f"[spec-def] verify V {V} T {temp}: {n_calls} calls x {NREQ} blocks")
    g = _drafter(V)
    try:
        q_row, p_row, dlg, tlg = _rows(V, 22)
        req = torch.arange(NREQ, dtype=torch.int32, device="cuda")
        cand = torch.zeros((NREQ, K), dtype=torch.int32, device="cuda")
        dlse = torch.zeros((NREQ, K), dtype=torch.float32, device="cuda")
        tokens = torch.zeros((NREQ, B), dtype=torch.int32, device="cuda")
        tau = torch.zeros(NREQ, dtype=torch.int32, device="cuda")
        first = torch.zeros(V, dtype=torch.int64, device="cuda")
        taus = torch.zeros(B + 1, dtype=torch.int64, device="cuda")
        for c in range(n_calls):
            g.dr.spec_draft(NREQ, dlg, temp, 5000 + c, req, cand, dlse)
            g.dr.spec_verify(NREQ, dlg, tlg, cand, temp, 5000 + c, req, tokens, tau, dlse)
            first += torch.bincount(tokens[:, 0].long(), minlength=V)[:V]
            taus += torch.bincount(tau.long(), minlength=B + 1)[:B + 1]
        torch.cuda.synchronize()
        first, taus = first.cpu().numpy(), taus.cpu().numpy()
        assert first.sum() == n_calls * NREQ and taus[0] == 0
        q = ss.draft_distribution(q_row, temp)
        p = ss.draft_distribution(p_row, temp)
        stat, dof, pv = _chi2(first, ss.emitted_first_token_plain(q, p))
        log(f"[spec-def] verify V {V} T {temp}: first token chi2 {stat:.1f} on {dof} dof, p = {pv:.3g}")
        assert pv >= P_MIN, f"first emitted token does not follow the verifier's distribution: p = {pv:.3g}"
        tdist = ss.tau_distribution_plain(np.tile(q, (K, 1)), np.tile(p, (B, 1)))
        stat, dof, pv = _chi2(taus[1:], tdist)
        log(f"[spec-def] verify V {V} T {temp}: tau chi2 {stat:.1f} on {dof} dof, p = {pv:.3g}, "
            f"mean tau {np.dot(np.arange(B + 1), taus) / taus.sum():.3f} vs {np.dot(np.arange(1, B + 1), tdist):.3f}")
        assert pv >= P_MIN, f"tau does not follow the keep-probability product: p = {pv:.3g}"
    finally:
        g.close()
