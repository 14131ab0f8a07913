"""GPU parity: the HIP path through the C ABI against the float64 oracle.

Tolerances: fp32 storage paths rel <= 1e-4 (max-norm); bf16 logits
max|diff| <= 2e-2 * max|logit| against the plain float64 oracle; token ids
compared wherever the oracle's top-1 minus top-2 logit margin exceeds 0.05
(top-k: both gaps around a rank; for bf16 drafters ranks after the first at
tests._gpu.BF16_RANK_MARGIN); acceptance bit-exact.

bf16 drafters: token-id and tau decisions are compared against the oracle
taken in the kernel's storage precision (oracle.round_bf16 at every activation
a bf16 drafter stores between projections; sums and the residual stream stay
float64).  The plain oracle differs from any bf16 drafter by about 0.02 rms in
the logits at the 8B shape (a float emulation of the storage roundings alone
gives the same figure), which exceeds half the 0.05 margin on some rows.  In
the storage precision about 0.015 rms remains (the softmax weights inside the
attention kernel, accumulation order, and roundings of slightly different
values that land on different bf16 neighbours): enough for a top-1 decision at
the 0.05 margin, but among the ~130 inner ranks of a 16-long list compared per
request an occasional pair whose gap just clears 0.05 trades places, so those
ranks use a margin of about five times the spread of a logit difference."""
import dataclasses

import numpy as np
import pytest

import oracle
import synth
from synth.configs import QWEN3_4B, QWEN3_8B
from tests._gpu import BF16_RANK_MARGIN, GpuDraft, check_top1, check_topk, hidden_rows, log, margin_mask, rel_inf

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("needs a GPU", allow_module_level=True)


def _oracle_for(d, w_np, seed, reqs):
    """reqs: list of (req_index, ctx).  Returns OracleDrafter with caches filled."""
    o = oracle.OracleDrafter(synth.weights_as_f32(w_np), d)
    for r, ctx in reqs:
        if ctx:
            o.fuse(r, synth.as_f32(synth.make_hidden(d, seed, r, 0, ctx)))
    return o


def _store(d):
    """Rounding of the activations a drafter of this dtype stores (None: fp32)."""
    return oracle.round_bf16 if d.dtype == "bf16" else None


def _compare_request(gl, gids, ref_logits, d, tol_logit, label, ref_ids_logits=None):
    """Logits against the plain oracle; top-1 ids against ref_ids_logits (the
    oracle in the drafter's storage precision; default: the plain logits)."""
    if d.dtype == "f32":
        err = rel_inf(gl, ref_logits)
        assert err <= 1e-4, f"{label}: logits rel err {err}"
    else:
        err = np.abs(gl - ref_logits).max() / np.abs(ref_logits).max()
        assert err <= tol_logit, f"{label}: logits err {err}"
    ids_ref = ref_logits if ref_ids_logits is None else ref_ids_logits
    mask, bad = check_top1(gids[:, 0], ids_ref)
    assert len(bad) == 0, f"{label}: top-1 mismatch at rows {bad} (margin-passing rows {mask.sum()})"
    return err, mask


# ------------------------------------------------------------------ tiny fp32

@pytest.fixture(scope="module")
def tiny():
    wl = synth.get_config("tiny")
    d = wl.dims
    w_np = synth.make_weights(d, wl.seed)
    return wl, d, w_np


def test_gpu_tiny_full_step(tiny):
    wl, d, w_np = tiny
    log(f"case tiny full step: D={d.D} ctx={wl.ctx}")
    g = GpuDraft(d, w_np, max_ctx=128, max_slots=2, max_batch=1)
    hid = synth.make_hidden(d, wl.seed, 0, 0, 64)
    g.fuse([1], [64], hid)
    o = _oracle_for(d, w_np, wl.seed, [(0, 64)])
    for l in range(d.N):
        k, v = g.read_cache(1, l, 0, 64)
        assert rel_inf(k, o.cache(0).K[l]) <= 1e-4
        assert rel_inf(v, o.cache(0).V[l]) <= 1e-4
    anchor = synth.make_anchors(d, wl.seed, 1)
    ref = o.draft(0, int(anchor[0]))["logits"]
    ids, vals, lg = g.draft([1], anchor, top_k=1, logits=True)
    _compare_request(lg[0], ids[0], ref, d, 0, "tiny")
    np.testing.assert_allclose(vals[0][:, 0], lg[0].max(axis=1), rtol=0, atol=0)
    ids16, vals16, _ = g.draft([1], anchor, top_k=16)
    cmp, bad = check_topk(ids16[0], ref)
    assert len(bad) == 0, bad
    assert rel_inf(vals16[0], np.take_along_axis(ref, ids16[0].astype(np.int64), 1)) <= 1e-4
    # acceptance on GPU candidates with targets built from the oracle's
    m = synth.draw_first_mismatch("uniform", 1, d.B, wl.seed)
    ref_c, _ = oracle.topk(ref, 1)
    tgt = synth.make_targets(ref_c[:, 0][None], m, d.V, wl.seed)
    tau, bonus = g.accept(ids16, 16, tgt)
    tau_ref, bonus_ref = oracle.accept(ref_c[:, 0], tgt[0])
    mm = margin_mask(ref)
    if mm[:min(tau_ref, d.B - 1)].all():
        assert (tau[0], bonus[0]) == (tau_ref, bonus_ref)
    g.close()


def test_gpu_tiny_ragged_batch_and_rewind(tiny):
    wl, d, w_np = tiny
    log("case tiny ragged batch bs=5")
    ctxs = [0, 1, 17, 64, 100]
    first = [0, 1, 10, 30, 64]
    slots = [4, 0, 3, 1, 2]
    g = GpuDraft(d, w_np, max_ctx=160, max_slots=6, max_batch=5)
    g.fuse(slots, first, hidden_rows(d, wl.seed, [(r, 0, first[r]) for r in range(5)]))
    second = [c - f for c, f in zip(ctxs, first)]
    g.fuse(slots, second, hidden_rows(d, wl.seed, [(r, first[r], second[r]) for r in range(5)]))
    for r in range(5):
        assert g.dr.slot_len(slots[r]) == ctxs[r]
    o = _oracle_for(d, w_np, wl.seed, list(enumerate(ctxs)))
    anchors = synth.make_anchors(d, wl.seed, 5)
    ids, vals, lg = g.draft(slots, anchors, top_k=4, logits=True)
    for r in range(5):
        ref = o.draft(r, int(anchors[r]))["logits"]
        _compare_request(lg[r], ids[r], ref, d, 0, f"tiny r{r}")
        cmp, bad = check_topk(ids[r], ref)
        assert len(bad) == 0
        if ctxs[r]:
            k, v = g.read_cache(slots[r], d.N - 1, 0, ctxs[r])
            assert rel_inf(k, o.cache(r).K[d.N - 1]) <= 1e-4
            assert rel_inf(v, o.cache(r).V[d.N - 1]) <= 1e-4
    # rewind request 4 to 40 tokens and re-append 25 different rows
    g.dr.slot_reset(slots[4], 40)
    alt = hidden_rows(d, wl.seed + 100, [(4, 40, 25)])
    g.fuse([slots[4]], [25], alt)
    o.reset(4, 40)
    o.fuse(4, synth.as_f32(alt))
    ids2, _, lg2 = g.draft([slots[4]], anchors[4:5], top_k=1, logits=True)
    ref2 = o.draft(4, int(anchors[4]))["logits"]
    _compare_request(lg2[0], ids2[0], ref2, d, 0, "tiny rewind")
    g.close()


def test_gpu_tiny_multi_split_ragged(tiny):
    """Contexts from empty to 1000 keys in one batch: 128-key attention splits,
    one to eight per request, last splits shorter and longer than a full one
    (launched longest first, merged in split order), fp32 against the oracle."""
    wl, d, w_np = tiny
    ctxs = [0, 1, 127, 128, 129, 300, 513, 1000]
    n = len(ctxs)
    log(f"case tiny multi-split ragged, ctx {ctxs}")
    slots = list(range(n))
    g = GpuDraft(d, w_np, max_ctx=max(ctxs) + d.B, max_slots=n, max_batch=n)
    g.fuse(slots, ctxs, hidden_rows(d, wl.seed, [(r, 0, ctxs[r]) for r in range(n)]))
    o = _oracle_for(d, w_np, wl.seed, list(enumerate(ctxs)))
    anchors = synth.make_anchors(d, wl.seed, n)
    ids, _, lg = g.draft(slots, anchors, top_k=1, logits=True)
    for r in range(n):
        ref = o.draft(r, int(anchors[r]))["logits"]
        _compare_request(lg[r], ids[r], ref, d, 0, f"tiny multi-split r{r} ctx {ctxs[r]}")
    g.close()


def test_gpu_tiny_deterministic(tiny):
    wl, d, w_np = tiny
    log("case tiny determinism")
    g = GpuDraft(d, w_np, max_ctx=128, max_slots=2, max_batch=2)
    g.fuse([0, 1], [64, 33], hidden_rows(d, wl.seed, [(0, 0, 64), (1, 0, 33)]))
    a = synth.make_anchors(d, wl.seed, 2)
    r1 = g.draft([0, 1], a, top_k=16, logits=True)
    r2 = g.draft([0, 1], a, top_k=16, logits=True)
    for x, y in zip(r1, r2):
        assert np.array_equal(x, y)
    g.close()


def test_gpu_no_rope_identical_mask_outputs(tiny):
    wl, d, w_np = tiny
    log("case tiny use_rope=0")
    d0 = dataclasses.replace(d, use_rope=False)
    g = GpuDraft(d0, w_np, max_ctx=128, max_slots=1, max_batch=1)
    g.fuse([0], [40], synth.make_hidden(d0, wl.seed, 0, 0, 40))
    _, _, lg = g.draft([0], [5], top_k=1, logits=True)
    for j in range(1, d.B - 1):
        np.testing.assert_allclose(lg[0][j], lg[0][0], rtol=1e-6, atol=1e-6)
    o = _oracle_for(d0, w_np, wl.seed, [(0, 40)])
    assert rel_inf(lg[0], o.draft(0, 5)["logits"]) <= 1e-4
    g.close()


def test_gpu_block_size_two_and_empty_context(tiny):
    wl, _, _ = tiny
    d = dataclasses.replace(synth.get_config("tiny").dims, B=2)
    log("case tiny B=2, ctx=0")
    w_np = synth.make_weights(d, 9)
    g = GpuDraft(d, w_np, max_ctx=64, max_slots=1, max_batch=1)
    ids, _, lg = g.draft([0], [17], top_k=2, logits=True)
    o = _oracle_for(d, w_np, 9, [])
    ref = o.draft(0, 17)["logits"]
    _compare_request(lg[0], ids[0], ref, d, 0, "B=2 ctx=0")
    g.close()


def test_gpu_tiny_max_batch_and_full_slots(tiny):
    """The largest call the library takes: 64 requests (the per-call limit) in
    one fusion and one draft, slots permuted against request order, contexts
    ragged from empty to exactly max_ctx."""
    import block_diffusion_drafter_fuse_amd as dfa
    wl, d, w_np = tiny
    n, max_ctx = 64, 96
    log("case tiny max batch 64, ctx 0..96")
    ctxs = [(r * 29) % (max_ctx + 1) for r in range(n)]
    ctxs[0], ctxs[n - 1] = 0, max_ctx
    slots = [n - 1 - r for r in range(n)]
    g = GpuDraft(d, w_np, max_ctx=max_ctx, max_slots=n, max_batch=n)
    g.fuse(slots, ctxs, hidden_rows(d, wl.seed, [(r, 0, ctxs[r]) for r in range(n)]))
    for r in range(n):
        assert g.dr.slot_len(slots[r]) == ctxs[r]
    o = _oracle_for(d, w_np, wl.seed, list(enumerate(ctxs)))
    anchors = synth.make_anchors(d, wl.seed, n)
    ids, _, lg = g.draft(slots, anchors, top_k=4, logits=True)
    for r in range(n):
        ref = o.draft(r, int(anchors[r]))["logits"]
        _compare_request(lg[r], ids[r], ref, d, 0, f"max batch r{r} ctx {ctxs[r]}")
        _, bad = check_topk(ids[r], ref)
        assert len(bad) == 0, f"max batch r{r}: top-k mismatch at rows {bad}"
    # a full slot takes no further row, and the failed call changes nothing
    with pytest.raises(dfa.DflashError) as e:
        g.fuse([slots[n - 1]], [1], hidden_rows(d, wl.seed, [(n - 1, max_ctx, 1)]))
    assert e.value.code == -3 and g.dr.slot_len(slots[n - 1]) == max_ctx
    ids2, _, _ = g.draft(slots, anchors, top_k=4)
    assert np.array_equal(ids2, ids)
    g.close()


def test_gpu_empty_calls_are_no_ops(tiny):
    """Zero requests, and requests with no new rows, launch nothing: slot
    lengths, the caches and the next draft are unchanged, and the caller's
    output buffers are not written."""
    wl, d, w_np = tiny
    log("case empty calls")
    g = GpuDraft(d, w_np, max_ctx=64, max_slots=2, max_batch=2)
    g.fuse([0, 1], [5, 9], hidden_rows(d, wl.seed, [(0, 0, 5), (1, 0, 9)]))
    anchors = synth.make_anchors(d, wl.seed, 2)
    ids, _, lg = g.draft([0, 1], anchors, top_k=2, logits=True)
    k0, v0 = g.read_cache(1, 0, 0, 9)
    # fusion: no requests; requests with zero rows (no hidden-state pointers needed)
    g.dr.fuse_ctx([], [], [])
    g.dr.fuse_ctx([0, 1], [0, 0], [])
    # draft: no requests, with sentinel outputs that must stay untouched
    out = torch.full((1, d.B - 1, 2), 7, dtype=torch.int32, device="cuda")
    g.dr.draft_block([], None, 2, out)
    torch.cuda.synchronize()
    assert int((out != 7).sum()) == 0
    assert g.dr.slot_len(0) == 5 and g.dr.slot_len(1) == 9
    k1, v1 = g.read_cache(1, 0, 0, 9)
    assert np.array_equal(k0, k1) and np.array_equal(v0, v1)
    ids2, _, lg2 = g.draft([0, 1], anchors, top_k=2, logits=True)
    assert np.array_equal(ids2, ids) and np.array_equal(lg2, lg)
    # an empty acceptance scan is a no-op too
    dfa = g.dfa
    dfa.accept(0, d.B, None, d.B - 1, None, None, None)
    g.close()


# Head-dim / dtype pairs the other cases leave out (fp32 runs head dim 64 and
# bf16 head dim 128 elsewhere): each attention instance with its query
# fragments per work-group, over ragged multi-split contexts and more than
# 64 token rows.
CROSS_CASES = [
    # dtype, hd, Hq, Hkv, B
    ("f32", 128, 8, 2, 16),    # four query fragments (G*B = 64)
    ("bf16", 64, 8, 2, 16),    # four query fragments
    ("bf16", 64, 4, 4, 8),     # one query fragment (G*B = 8)
    ("bf16", 128, 8, 4, 16),   # two query fragments (G*B = 32)
]


@pytest.mark.parametrize("dtype,hd,Hq,Hkv,B", CROSS_CASES)
def test_gpu_head_dim_dtype_cross(dtype, hd, Hq, Hkv, B):
    d = dataclasses.replace(synth.get_config("tiny").dims, dtype=dtype, D=512, Dt=256, L=3, Hq=Hq, Hkv=Hkv,
                            hd=hd, I=1024, V=2048, B=B)
    seed = 31
    ctxs = [0, 37, 300, 700, 1000]
    n = len(ctxs)
    log(f"case cross {dtype} hd {hd} Hq {Hq} Hkv {Hkv} B {B}, ctx {ctxs}")
    w_np = synth.make_weights(d, seed)
    g = GpuDraft(d, w_np, max_ctx=1024, max_slots=n, max_batch=n)
    g.fuse(list(range(n)), ctxs, hidden_rows(d, seed, [(r, 0, ctxs[r]) for r in range(n)]))
    anchors = synth.make_anchors(d, seed, n)
    ids, _, lg = g.draft(list(range(n)), anchors, top_k=4, logits=True)
    o = _oracle_for(d, w_np, seed, list(enumerate(ctxs)))
    n_cmp = 0
    for r in range(n):
        ref = o.draft(r, int(anchors[r]))["logits"]
        ref_s = None if dtype == "f32" else o.draft(r, int(anchors[r]), store=_store(d))["logits"]
        _, mask = _compare_request(lg[r], ids[r], ref, d, 2e-2, f"cross {dtype} hd {hd} r{r}", ref_s)
        _, bad = check_topk(ids[r], ref if ref_s is None else ref_s,
                            thr_rest=None if ref_s is None else BF16_RANK_MARGIN)
        assert len(bad) == 0, f"cross {dtype} hd {hd} r{r}: top-4 mismatch at {bad[:5].tolist()}"
        n_cmp += int(mask.sum())
    assert n_cmp > 0, "no row cleared the top-1 margin"
    g.close()


def test_gpu_capacity_errors_leave_state(tiny):
    import block_diffusion_drafter_fuse_amd as dfa
    wl, d, w_np = tiny
    log("case capacity errors")
    g = GpuDraft(d, w_np, max_ctx=64, max_slots=2, max_batch=1)
    g.fuse([0], [60], synth.make_hidden(d, wl.seed, 0, 0, 60))
    with pytest.raises(dfa.DflashError) as e:
        g.fuse([0], [5], synth.make_hidden(d, wl.seed, 0, 60, 5))
    assert e.value.code == -3 and g.dr.slot_len(0) == 60
    with pytest.raises(dfa.DflashError) as e:
        g.draft([0, 1], [1, 2])
    assert e.value.code == -3
    with pytest.raises(dfa.DflashError) as e:
        g.draft([0], [1], top_k=17)
    assert e.value.code == -2
    with pytest.raises(dfa.DflashError):
        g.dr.slot_reset(0, 61)
    g.close()


def test_gpu_accept_bitexact():
    log("case accept")
    rng = np.random.default_rng(0)
    import block_diffusion_drafter_fuse_amd as dfa
    for B, V, n in [(16, 5, 64), (8, 2, 33), (2, 3, 7), (16, 151936, 32)]:
        for k in (1, 3):
            cand_full = rng.integers(0, V, size=(n, B - 1, k)).astype(np.int32)
            m = rng.integers(0, B, size=n)
            tgt = synth.make_targets(cand_full[:, :, 0], m, V, 7)
            c = torch.tensor(cand_full, device="cuda")
            t = torch.tensor(tgt, device="cuda")
            tau = torch.zeros(n, dtype=torch.int32, device="cuda")
            bonus = torch.zeros(n, dtype=torch.int32, device="cuda")
            dfa.accept(n, B, c, k, t, tau, bonus)
            torch.cuda.synchronize()
            for r in range(n):
                assert (int(tau[r]), int(bonus[r])) == oracle.accept(cand_full[r, :, 0], tgt[r])
                assert int(tau[r]) == m[r] + 1


# ------------------------------------------------------------------ full size

def _full_size_case(wl, sample_reqs, label, tau_kind, repeat=False):
    """One steady-state step at full size: prefill, fuse the step's rows, draft
    (top-1 and top-16), then the acceptance scan on targets drawn with the
    workload's tau recipe.  The oracle runs on the sampled requests."""
    d = wl.dims
    log(f"case {label}: generating weights")
    w_np = synth.make_weights(d, wl.seed)
    bs = wl.bs
    max_ctx = max(wl.ctx) + 16
    g = GpuDraft(d, w_np, max_ctx=max_ctx, max_slots=bs, max_batch=bs)
    slots = list(range(bs))
    pre = [c - n for c, n in zip(wl.ctx, wl.n_new)]
    log(f"case {label}: prefill {sum(pre)} rows")
    for r in range(bs):   # per request keeps host memory bounded
        if pre[r]:
            g.fuse([r], [pre[r]], synth.make_hidden(d, wl.seed, r, 0, pre[r]))
    log(f"case {label}: step fuse {sum(wl.n_new)} rows")
    g.fuse(slots, wl.n_new, hidden_rows(d, wl.seed, [(r, pre[r], wl.n_new[r]) for r in range(bs)]))
    anchors = synth.make_anchors(d, wl.seed, bs)
    ids, vals, lg = g.draft(slots, anchors, top_k=1, logits=True)
    if repeat:
        # split-K partial sums and attention splits are combined in a fixed
        # order: a second draft of the same block is bitwise identical
        ids2, vals2, lg2 = g.draft(slots, anchors, top_k=1, logits=True)
        assert np.array_equal(ids, ids2) and np.array_equal(lg, lg2), f"{label}: repeated draft differs"
    ids16, vals16, _ = g.draft(slots, anchors, top_k=16)
    assert np.array_equal(ids16[:, :, 0], ids[:, :, 0]), f"{label}: top-16 rank 0 differs from top-1"
    log(f"case {label}: oracle on requests {sample_reqs}")
    o = oracle.OracleDrafter(synth.weights_as_f32(w_np), d)
    worst = 0.0
    cover = []
    # acceptance targets: built from the oracle's candidates on the sampled
    # requests and from the GPU's elsewhere (there the scan alone is checked)
    cand_for_targets = ids[:, :, 0].copy()
    ref_masks = {}
    plain_agree = []
    worst_s = 0.0
    for r in sample_reqs:
        o.fuse(r, synth.as_f32(synth.make_hidden(d, wl.seed, r, 0, wl.ctx[r])))
        # cache windows: the context's start and, past 4096 rows, the second
        # fusion chunk (both written by the prefill fusion), and its end (the
        # step's own rows)
        n_chk = min(wl.ctx[r], 64)
        starts = {0, wl.ctx[r] - n_chk} | ({4096} if wl.ctx[r] >= 4096 + n_chk else set())
        for l in (0, d.N - 1):
            for pos0 in sorted(starts):
                k, v = g.read_cache(r, l, pos0, n_chk)
                assert rel_inf(k, o.cache(r).K[l][:, pos0:pos0 + n_chk]) <= 2e-2, f"r{r} layer {l} K at {pos0}"
                assert rel_inf(v, o.cache(r).V[l][:, pos0:pos0 + n_chk]) <= 2e-2, f"r{r} layer {l} V at {pos0}"
        ref = o.draft(r, int(anchors[r]))["logits"]
        ref_s = o.draft(r, int(anchors[r]), store=_store(d))["logits"]
        err, mask = _compare_request(lg[r], ids[r], ref, d, 2e-2, f"{label} r{r}", ref_s)
        _, bad = check_topk(ids16[r], ref_s, thr_rest=BF16_RANK_MARGIN)
        assert len(bad) == 0, f"{label} r{r}: top-16 mismatch at (row, rank) {bad[:5].tolist()}"
        plain_mask, plain_bad = check_top1(ids[r][:, 0], ref)
        plain_agree.append((int(plain_mask.sum()) - len(plain_bad), int(plain_mask.sum())))
        worst = max(worst, err)
        worst_s = max(worst_s, float(np.abs(lg[r] - ref_s).max()))
        cover.append(mask.mean())
        cand_for_targets[r] = oracle.topk(ref_s, 1)[0][:, 0]
        ref_masks[r] = mask
        o.caches.pop(r)
    # acceptance rounds: tau drawn with the workload's recipe, sixteen target
    # sets per step (each a fresh draw of the first mismatch)
    n_tau, taus = 0, []
    for k in range(16):
        m = synth.draw_first_mismatch(tau_kind, bs, d.B, wl.seed + 100 * k)
        tgt = synth.make_targets(cand_for_targets, m, d.V, wl.seed + 100 * k)
        tau, bonus = g.accept(ids, 1, tgt)
        for r in range(bs):
            # the scan itself: bit-exact on the GPU's own candidates
            assert (int(tau[r]), int(bonus[r])) == oracle.accept(ids[r, :, 0], tgt[r]), f"{label} r{r}: scan"
            assert 1 <= tau[r] <= d.B
        for r in sample_reqs:
            # tau and the bonus against the oracle's step, wherever every
            # candidate position up to the oracle's tau clears the margin
            tau_ref, bonus_ref = oracle.accept(cand_for_targets[r], tgt[r])
            assert tau_ref == m[r] + 1
            if ref_masks[r][:min(tau_ref, d.B - 1)].all():
                assert (int(tau[r]), int(bonus[r])) == (tau_ref, bonus_ref), f"{label} r{r}: tau/bonus"
                n_tau += 1
                taus.append(tau_ref)
    assert n_tau > 0, f"{label}: no acceptance round had every position up to tau above the margin"
    log(f"case {label}: worst logit err {worst:.3e} (plain oracle), max |diff| {worst_s:.4f} against the "
        f"storage-precision oracle; top-1 ids equal to the plain oracle's on {plain_agree} (equal, compared) rows; "
        f"margin coverage {np.mean(cover):.2f}; tau and bonus equal to the oracle's in {n_tau} of "
        f"{16 * len(sample_reqs)} request rounds (tau drawn {tau_kind}; compared values {sorted(taus)})")
    g.close()


def test_gpu_qwen3_4b_bs1():
    # config tau ~ U{1..16}
    _full_size_case(synth.get_config("qwen3_4b_bs1"), [0], "qwen3_4b_bs1", "uniform")


def test_gpu_qwen3_4b_bs1_decode_loop():
    """Six steady-state steps at the Qwen3-4B bs1 shape: each step drafts on the
    GPU and in the oracle, compares logits and top-1, draws the verifier targets
    from the oracle's candidates (tau ~ U{1..16}), takes tau and the bonus from
    the oracle's scan (the GPU scan is checked on its own candidates), fuses
    the tau committed rows into both and anchors the next block at the bonus
    token; both sides therefore see the same history even where bf16 rounding
    would pick another token on a near tie."""
    wl = synth.get_config("qwen3_4b_bs1")
    d = wl.dims
    steps = 6
    log("case qwen3_4b_bs1 decode loop: generating weights")
    w_np = synth.make_weights(d, wl.seed)
    ctx = wl.ctx[0]
    g = GpuDraft(d, w_np, max_ctx=ctx + 16 * steps + 16, max_slots=1, max_batch=1)
    hid0 = synth.make_hidden(d, wl.seed, 0, 0, ctx)
    g.fuse([0], [ctx], hid0)
    o = oracle.OracleDrafter(synth.weights_as_f32(w_np), d)
    o.fuse(0, synth.as_f32(hid0))
    del hid0
    anchor = int(synth.make_anchors(d, wl.seed, 1)[0])
    taus = []
    for k in range(steps):
        log(f"case qwen3_4b_bs1 decode loop: step {k}, ctx {ctx}")
        ids, _, lg = g.draft([0], [anchor], top_k=1, logits=True)
        ref = o.draft(0, anchor)["logits"]
        ref_s = o.draft(0, anchor, store=_store(d))["logits"]
        _compare_request(lg[0], ids[0], ref, d, 2e-2, f"4B loop step {k}", ref_s)
        cand_o = oracle.topk(ref_s, 1)[0][:, 0]
        m = synth.draw_first_mismatch("uniform", 1, d.B, wl.seed + 7 * k)
        tgt = synth.make_targets(cand_o[None], m, d.V, wl.seed + 7 * k)
        tau, bonus = oracle.accept(cand_o, tgt[0])
        tau_g, bonus_g = g.accept(ids, 1, tgt)
        assert (int(tau_g[0]), int(bonus_g[0])) == oracle.accept(ids[0, :, 0], tgt[0]), f"step {k}: scan"
        # the committed rows: the anchor and the accepted candidates, whose
        # verifier states are the synthetic rows at positions ctx .. ctx + tau - 1
        hid = synth.make_hidden(d, wl.seed, 0, ctx, tau)
        g.fuse([0], [tau], hid)
        o.fuse(0, synth.as_f32(hid))
        ctx += tau
        taus.append(tau)
        assert g.dr.slot_len(0) == ctx
        anchor = int(bonus)
    n = min(32, ctx)
    for l in (0, d.N - 1):
        kc, vc = g.read_cache(0, l, ctx - n, n)
        assert rel_inf(kc, o.cache(0).K[l][:, ctx - n:ctx]) <= 2e-2, f"layer {l} K after the loop"
        assert rel_inf(vc, o.cache(0).V[l][:, ctx - n:ctx]) <= 2e-2, f"layer {l} V after the loop"
    log(f"case qwen3_4b_bs1 decode loop: taus {taus}")
    g.close()


def test_gpu_qwen3_8b_bs1():
    _full_size_case(synth.get_config("qwen3_8b_bs1"), [0], "qwen3_8b_bs1", "geometric")


def test_gpu_qwen3_8b_bs32_sampled():
    # shortest, median and longest context (the longest has the most attention
    # splits); tau drawn clamped-geometric with mean 6.5
    wl = synth.get_config("qwen3_8b_bs32")
    order = np.argsort(wl.ctx)
    _full_size_case(wl, [int(order[0]), int(order[len(order) // 2]), int(order[-1])], "qwen3_8b_bs32",
                    "geometric", repeat=True)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_gpu_topk_width_not_a_multiple_of_the_unroll(dtype):
    """D = 320: the top-k LM head's k-loop (unrolled by 8 k-steps) ends with a
    remainder (fp32: 20 k-steps, bf16: 10); top-4 and top-16 lists against the
    oracle's stable sort."""
    d = dataclasses.replace(synth.get_config("tiny").dims, D=320, dtype=dtype)
    log(f"case top-k at D=320 {dtype}")
    w_np = synth.make_weights(d, 11)
    g = GpuDraft(d, w_np, max_ctx=64, max_slots=2, max_batch=2)
    g.fuse([0, 1], [40, 23], hidden_rows(d, 11, [(0, 0, 40), (1, 0, 23)]))
    o = _oracle_for(d, w_np, 11, [(0, 40), (1, 23)])
    anchors = synth.make_anchors(d, 11, 2)
    ids1, _, lg = g.draft([0, 1], anchors, top_k=1, logits=True)
    for k in (4, 16):
        ids, vals, _ = g.draft([0, 1], anchors, top_k=k)
        for r in range(2):
            ref = o.draft(r, int(anchors[r]))["logits"]
            ref_s = o.draft(r, int(anchors[r]), store=_store(d))["logits"]
            tol = 1e-4 if dtype == "f32" else 2e-2
            _compare_request(lg[r], ids1[r], ref, d, tol, f"D=320 {dtype} r{r}", ref_s)
            _, bad = check_topk(ids[r], ref_s, thr_rest=None if dtype == "f32" else BF16_RANK_MARGIN)
            assert len(bad) == 0, f"D=320 {dtype} r{r} top-{k}: mismatch at {bad[:5].tolist()}"
            # values are the logits of the listed ids
            got = np.take_along_axis(lg[r], ids[r].astype(np.int64), 1)
            assert rel_inf(vals[r], got) <= (1e-5 if dtype == "f32" else 1e-2)
    g.close()


def test_gpu_topk_rejects_rows_beyond_lds():
    """bf16 D = 5120: 16 staged rows exceed a CU's 160 KB of LDS, so top_k > 1
    is refused before any launch; top_k = 1 (the GEMM-engine head) still runs."""
    import block_diffusion_drafter_fuse_amd as dfa
    d = dataclasses.replace(synth.get_config("tiny").dims, D=5120, dtype="bf16")
    log("case top-k LDS limit at D=5120 bf16")
    w_np = synth.make_weights(d, 12)
    g = GpuDraft(d, w_np, max_ctx=32, max_slots=1, max_batch=1)
    g.fuse([0], [8], synth.make_hidden(d, 12, 0, 0, 8))
    with pytest.raises(dfa.DflashError) as e:
        g.draft([0], [3], top_k=16)
    assert e.value.code == -2
    ids, _, lg = g.draft([0], [3], top_k=1, logits=True)
    o = _oracle_for(d, w_np, 12, [(0, 8)])
    _compare_request(lg[0], ids[0], o.draft(0, 3)["logits"], d, 2e-2, "D=5120 bf16",
                     o.draft(0, 3, store=_store(d))["logits"])
    g.close()
