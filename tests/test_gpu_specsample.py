"""GPU parity of speculative sampling at T > 0 (dflash_spec_draft,
dflash_spec_verify) against the float64 oracle (oracle/specsample.py).

Inputs: seeded synthetic logit rows (synth.make_sampling_logits: peaked
verifier rows, drafter rows = the matching verifier row plus per-request noise,
one in five with its peaks moved), the same arrays on both sides; the
candidates passed to the verifier are the oracle's own drafts.

Bars.  Every draw is two-stage (a vocabulary block by inverse CDF over the
block masses, then a Gumbel-max within it).  The block must be the oracle's
unless u S lies within 1e-4 S of the boundary between the two blocks (fp32
masses).  Within the block the choice must be valid: its float64 key lies
within the key's rounding bound of the oracle's maximum (1e-3 absolute, plus
the cancellation bound of log max(0, p - q) on residual draws); where the
oracle's winner leads by more than that bound the token is the oracle's.  Every acceptance decision equals the oracle's where
|u q - p| > 1e-4 max(u q, p); a request whose walk reaches a closer decision is
compared up to it.  Integer outputs (tau, the kept prefix, the -1 tail) are
exact.  At least 97% of all choices must equal the oracle's outright."""
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

KEY_TOL = 1e-3
ACC_TOL = 1e-4


class Sampler:
    """A ctx of the given vocabulary and block size (tiny fp32 drafter weights:
    the sampling calls read only V, B, max_batch and the workspace)."""

    def __init__(self, V, B, bs, seed=0, misalign=False):
        self.d = dataclasses.replace(_tiny(B=B), V=V)
        self.g = GpuDraft(self.d, synth.make_weights(self.d, seed), max_ctx=64, max_slots=1, max_batch=bs)
        self.dr = self.g.dr
        self.misalign = misalign

    def dev(self, a):
        """Device copy; with misalign, the rows start 4 bytes past a 16-byte
        boundary (the kernels then take their element-load path)."""
        a = np.ascontiguousarray(a, dtype=np.float32)
        if not self.misalign:
            return torch.from_numpy(a).cuda()
        buf = torch.zeros(a.size + 1, dtype=torch.float32, device="cuda")
        buf[1:] = torch.from_numpy(a.reshape(-1)).cuda()
        return buf[1:].view(a.shape)

    def draft(self, dl, temp, seed, req, lse=False):
        """Drafted ids [n, K]; with lse=True also the rows' log-sum-exps as a
        device tensor (verify input)."""
        n, K = dl.shape[0], dl.shape[1]
        dlg = self.dev(dl)
        rq = torch.tensor(np.asarray(req, dtype=np.int32), device="cuda")
        cand = torch.full((n, K), -7, dtype=torch.int32, device="cuda")
        dlse = torch.full((n, K), float("nan"), dtype=torch.float32, device="cuda") if lse else None
        self.dr.spec_draft(n, dlg, temp, seed, rq, cand, dlse)
        torch.cuda.synchronize()
        return (cand.cpu().numpy(), dlse) if lse else cand.cpu().numpy()

    def verify(self, dl, tl, cand, temp, seed, req, dlse=None):
        n, K = dl.shape[0], dl.shape[1]
        dlg = self.dev(dl)
        tlg = self.dev(tl)
        cd = torch.tensor(np.ascontiguousarray(cand, dtype=np.int32), device="cuda")
        rq = torch.tensor(np.asarray(req, dtype=np.int32), device="cuda")
        tokens = torch.full((n, K + 1), -7, dtype=torch.int32, device="cuda")
        tau = torch.full((n,), -7, dtype=torch.int32, device="cuda")
        self.dr.spec_verify(n, dlg, tlg, cd, temp, seed, rq, tokens, tau, dlse)
        torch.cuda.synchronize()
        return tokens.cpu().numpy(), tau.cpu().numpy()

    def close(self):
        self.g.close()


class Tally:
    def __init__(self):
        self.exact = 0
        self.total = 0

    def choice(self, got, keys, err=None, what=""):
        """got: the kernel's id; keys: float64 keys of every id (-inf allowed);
        err: per-id rounding bound of the kernel's key beyond KEY_TOL."""
        keys = np.asarray(keys, dtype=np.float64)
        best = ss.argmax_low(keys)
        e = np.zeros_like(keys) if err is None else err
        assert 0 <= got < keys.size, f"{what}: id {got} outside the vocabulary"
        tol = KEY_TOL + e[best] + e[got]
        assert keys[got] >= keys[best] - tol, f"{what}: chose {got} (key {keys[got]}), best {best} ({keys[best]})"
        others = np.delete(keys, best)
        if others.size and keys[best] - others.max() > KEY_TOL + e[best] + np.max(e):
            assert got == best, f"{what}: chose {got}, oracle {best} wins by a clear margin"
        self.exact += int(got == best)
        self.total += 1

    def rate(self):
        return self.exact / max(1, self.total)


BLOCK_TOL = 1e-4


def check_two_stage(t, got, logw, seed, stream_block, stream_entry, req, row, err=None, what=""):
    """One GPU draw against the oracle's two-stage draw over log-weights logw."""
    logw = np.asarray(logw, dtype=np.float64)
    V = logw.size
    assert 0 <= got < V, f"{what}: id {got} outside the vocabulary"
    with np.errstate(under="ignore"):
        w = np.exp(logw - logw.max())
    mass = np.add.reduceat(w, np.arange(0, V, ss.BLOCK))
    cum = np.cumsum(mass)
    u = ss.uniforms(seed, stream_block, req, row, 1)[0]
    b = ss.block_choice(w, u)
    bg = got // ss.BLOCK
    assert mass[bg] > 0, f"{what}: chose an empty block"
    if bg != b:
        # blocks may differ only where u S sits on the boundary between them
        edge = cum[min(b, bg)]
        assert abs(u * cum[-1] - edge) <= BLOCK_TOL * cum[-1], f"{what}: block {bg}, oracle {b}"
        t.total += 1
        log(f"{what}: block differs at a boundary")
        return
    lo, hi = b * ss.BLOCK, min(V, (b + 1) * ss.BLOCK)
    keys = np.full(V, -np.inf)
    keys[lo:hi] = logw[lo:hi] + ss.gumbel(ss.uniforms(seed, stream_entry, req, row, hi)[lo:])
    t.choice(got, keys, err, what)


def check_draft(sp, dl, temp, seed, req, rows=None, tally=None):
    """Drafted ids against the oracle's Gumbel keys; also checks the rows'
    log-sum-exps (base 2, of l log2(e) / T) that the call returns, and hands
    them back for the verifier."""
    cand, dlse = sp.draft(dl, temp, seed, req, lse=True)
    n, K, V = dl.shape
    z = dl.astype(np.float64) / temp
    zm = z.max(axis=-1, keepdims=True)
    want = (zm[..., 0] + np.log(np.exp(z - zm).sum(-1))) / np.log(2.0)
    got = dlse.cpu().numpy()
    assert np.all(np.abs(got - want) <= 1e-5 * np.maximum(1.0, np.abs(want))), np.abs(got - want).max()
    t = tally or Tally()
    for r in range(n):
        for j in range(K):
            if rows is not None and (r, j) not in rows:
                continue
            check_two_stage(t, int(cand[r, j]), dl[r, j].astype(np.float64) / temp, seed, ss.STREAM_DRAFT_BLOCK,
                            ss.STREAM_DRAFT, req[r], j, what=f"draft r{r} j{j + 1}")
    return cand, dlse, t


def check_verify(sp, dl, tl, cand, temp, seed, req, reqs=None, tally=None, dlse=None):
    """Compare one verify call with the oracle request by request; returns the
    GPU outputs and the tally."""
    tokens, tau = sp.verify(dl, tl, cand, temp, seed, req, dlse)
    n, K, V = dl.shape
    t = tally or Tally()
    for r in range(n):
        # properties that hold for every request
        ng = int(tau[r]) - 1
        assert 0 <= ng <= K, f"r{r}: tau {tau[r]}"
        assert list(tokens[r, :ng]) == [int(c) for c in cand[r, :ng]], f"r{r}: kept prefix"
        assert all(x == -1 for x in tokens[r, ng + 1:]), f"r{r}: tail {tokens[r]}"
        assert 0 <= tokens[r, ng] < V, f"r{r}: emitted id {tokens[r, ng]}"
        if reqs is not None and r not in reqs:
            continue
        want = ss.spec_sample(dl[r], tl[r], cand[r], temp, seed, req[r])
        no = want["accepted"]
        if ng != no:
            # the walks may part only at an acceptance decision within ACC_TOL
            q = ss.softmax(dl[r], temp)
            p = ss.softmax(tl[r], temp)
            u = ss.uniforms(seed, ss.STREAM_ACCEPT, req[r], 0, K)
            j = min(ng, no)
            x = int(cand[r, j])
            a, b = u[j] * q[j, x], p[ss.verifier_row(j + 1), x]
            assert abs(a - b) <= ACC_TOL * max(a, b), f"r{r}: accepted {ng}, oracle {no} (u q {a}, p {b})"
            log(f"r{r}: walks part at a close acceptance decision (offset {j + 1})")
            continue
        # the emitted token
        err = None
        logw = tl[r, ss.verifier_row(no + 1) if no < K else K].astype(np.float64) / temp
        if no < K:
            q = ss.softmax(dl[r, no], temp)
            p = ss.softmax(tl[r, ss.verifier_row(no + 1)], temp)
            w = ss.residual(p, q)
            if np.any(w > 0):
                with np.errstate(divide="ignore"):
                    logw = np.where(w > 0, np.log(np.where(w > 0, w, 1.0)), -np.inf)
                # fp32 probabilities carry ~1e-6 relative error; the difference
                # magnifies it by (p + q) / w in the log
                err = np.where(w > 0, 4e-6 * (p + q) / np.where(w > 0, w, 1.0), 0.0)
        check_two_stage(t, int(tokens[r, ng]), logw, seed, ss.STREAM_RESIDUAL_BLOCK, ss.STREAM_RESIDUAL, req[r], 0,
                        err, what=f"emitted r{r} (n={no})")
    return tokens, tau, t


CASES = [
    # name, V, B, bs, temperature, misaligned rows
    ("tiny", 1024, 8, 4, 1.0, False),
    ("two_chunks", 4160, 5, 3, 0.7, False),      # a 64-entry last chunk
    ("sub_chunk", 64, 4, 2, 1.3, False),         # the vocabulary fills a sixty-fourth of a work-group
    ("one_offset", 1024, 2, 5, 1.0, False),      # B = 2: a single drafted token
    ("cold", 2048, 16, 4, 0.05, False),          # near-greedy
    ("misaligned", 4160, 6, 3, 1.0, True),       # element loads
    ("two_blocks", 20480, 6, 3, 1.0, False),     # two sampling blocks, the second a quarter full
    ("max_batch", 20480, 16, 64, 1.0, False),    # the per-call request limit
]


@pytest.mark.parametrize("name,V,B,bs,temp,mis", CASES)
def test_spec_sampling_parity(name, V, B, bs, temp, mis):
    log(f"[spec] {name}: V {V} B {B} bs {bs} T {temp}")
    sp = Sampler(V, B, bs, misalign=mis)
    try:
        dl, tl = synth.make_sampling_logits(bs, B, V, seed=11)
        req = [3 * r + 1 for r in range(bs)]
        _, dlse, t = check_draft(sp, dl, temp, 1234, req)
        cand = np.stack([ss.draft_tokens(dl[r], temp, 1234, req[r]) for r in range(bs)])
        _, tau, t = check_verify(sp, dl, tl, cand, temp, 5678, req, tally=t)
        # the same with the drafter rows' log-sum-exps handed over by the draft call
        _, tau2, t = check_verify(sp, dl, tl, cand, temp, 5678, req, tally=t, dlse=dlse)
        log(f"[spec] {name}: tau {list(tau)} / {list(tau2)}, exact {t.exact}/{t.total}")
        assert t.rate() >= 0.97
    finally:
        sp.close()


def test_spec_sampling_full_vocab_bs32():
    """Qwen3 vocabulary (151,936), B 16, 32 requests: every row drafted and
    verified on the GPU; the oracle checks 24 sampled draft rows and 8 whole
    requests, the properties hold for all 32."""
    V, B, bs, temp = 151936, 16, 32, 1.0
    log(f"[spec] full vocabulary: V {V} B {B} bs {bs}")
    sp = Sampler(V, B, bs)
    try:
        dl, tl = synth.make_sampling_logits(bs, B, V, seed=5)
        req = list(range(bs))
        rng = np.random.default_rng(0)
        rows = {(int(rng.integers(bs)), int(rng.integers(B - 1))) for _ in range(24)}
        _, dlse, t = check_draft(sp, dl, temp, 77, req, rows=rows)
        cand = np.stack([ss.draft_tokens(dl[r], temp, 77, req[r]) for r in range(bs)])
        _, tau, t = check_verify(sp, dl, tl, cand, temp, 78, req, reqs=set(range(0, bs, 4)), tally=t)
        _, tau2, t = check_verify(sp, dl, tl, cand, temp, 78, req, reqs=set(range(2, bs, 4)), tally=t, dlse=dlse)
        log(f"[spec] full vocabulary: mean tau {tau.mean():.2f}, exact {t.exact}/{t.total}")
        assert t.rate() >= 0.97
        assert tau.min() >= 1 and tau.max() <= B
    finally:
        sp.close()


def test_spec_sampling_full_vocab_bs1():
    """One request at the full vocabulary: 4096-id pieces for drafting, 2048-id
    pieces for the replacement draw (the other piece sizes run above)."""
    V, B, bs, temp = 151936, 16, 1, 1.0
    log(f"[spec] full vocabulary, one request: V {V} B {B}")
    sp = Sampler(V, B, bs)
    try:
        dl, tl = synth.make_sampling_logits(bs, B, V, seed=9)
        _, dlse, t = check_draft(sp, dl, temp, 55, [7])
        cand = np.stack([ss.draft_tokens(dl[0], temp, 55, 7)])
        _, _, t = check_verify(sp, dl, tl, cand, temp, 56, [7], tally=t, dlse=dlse)
        _, _, t = check_verify(sp, dl, tl, cand, temp, 57, [7], tally=t)
        assert t.rate() >= 0.9
    finally:
        sp.close()


def test_spec_sampling_full_vocab_misaligned():
    """Element loads at the full vocabulary with enough rows for the
    16384-entry work-groups (16 requests, B 16): sampled rows and requests
    against the oracle."""
    V, B, bs, temp = 151936, 16, 16, 0.8
    log(f"[spec] full vocabulary, misaligned rows: V {V} B {B} bs {bs}")
    sp = Sampler(V, B, bs, misalign=True)
    try:
        dl, tl = synth.make_sampling_logits(bs, B, V, seed=6)
        req = [100 + r for r in range(bs)]
        rng = np.random.default_rng(1)
        rows = {(int(rng.integers(bs)), int(rng.integers(B - 1))) for _ in range(12)}
        _, dlse, t = check_draft(sp, dl, temp, 31, req, rows=rows)
        cand = np.stack([ss.draft_tokens(dl[r], temp, 31, req[r]) for r in range(bs)])
        _, tau, t = check_verify(sp, dl, tl, cand, temp, 32, req, reqs={1, 6, 11}, tally=t, dlse=dlse)
        assert t.rate() >= 0.97
    finally:
        sp.close()


def test_spec_equal_distributions_keep_every_draft():
    """Drafter rows equal to the verifier rows that score them: every draft is
    kept (u q < q for u < 1), tau = B, and the bonus comes from the last row."""
    V, B, bs, temp = 1024, 8, 3, 0.9
    sp = Sampler(V, B, bs)
    try:
        _, tl = synth.make_sampling_logits(bs, B, V, seed=3)
        dl = np.ascontiguousarray(tl[:, :B - 1])
        req = [0, 1, 2]
        cand = np.stack([ss.draft_tokens(dl[r], temp, 9, req[r]) for r in range(bs)])
        tokens, tau, t = check_verify(sp, dl, tl, cand, temp, 10, req)
        assert list(tau) == [B] * bs
        assert t.rate() == 1.0
    finally:
        sp.close()


def test_spec_out_of_vocabulary_candidate_is_rejected():
    V, B, bs, temp = 1024, 6, 2, 1.0
    sp = Sampler(V, B, bs)
    try:
        _, tl = synth.make_sampling_logits(bs, B, V, seed=4)
        dl = np.ascontiguousarray(tl[:, :B - 1])  # every in-vocabulary draft would be kept
        cand = np.stack([ss.draft_tokens(dl[r], temp, 1, r) for r in range(bs)]).astype(np.int32)
        cand[0, 2] = -1
        cand[1, 0] = V
        tokens, tau = sp.verify(dl, tl, cand, temp, 2, [0, 1])
        assert list(tau) == [3, 1]
        assert list(tokens[0, :2]) == list(cand[0, :2]) and list(tokens[0, 3:]) == [-1] * (B - 3)
        assert 0 <= tokens[0, 2] < V and 0 <= tokens[1, 0] < V
    finally:
        sp.close()


def test_spec_repeat_and_streams():
    """Same seed and request ids: identical outputs on a second call (tickets
    and partials reset); other request ids draw differently; an empty call
    is a no-op; arguments outside the documented ranges are refused."""
    import block_diffusion_drafter_fuse_amd as dfa
    V, B, bs, temp = 1024, 8, 4, 1.0
    sp = Sampler(V, B, bs)
    try:
        dl, tl = synth.make_sampling_logits(bs, B, V, seed=8)
        a = sp.draft(dl, temp, 5, [0, 1, 2, 3])
        b = sp.draft(dl, temp, 5, [0, 1, 2, 3])
        c = sp.draft(dl, temp, 5, [4, 5, 6, 7])
        assert np.array_equal(a, b) and not np.array_equal(a, c)
        v1 = sp.verify(dl, tl, a, temp, 6, [0, 1, 2, 3])
        v2 = sp.verify(dl, tl, a, temp, 6, [0, 1, 2, 3])
        assert np.array_equal(v1[0], v2[0]) and np.array_equal(v1[1], v2[1])
        sp.dr.spec_draft(0, None, temp, 1, None, None, None)
        with pytest.raises(dfa.DflashError):
            sp.draft(dl, 0.0, 5, [0, 1, 2, 3])
        big = np.zeros((bs + 1, B - 1, V), dtype=np.float32)
        with pytest.raises(dfa.DflashError):
            sp.draft(big, temp, 5, list(range(bs + 1)))
    finally:
        sp.close()
