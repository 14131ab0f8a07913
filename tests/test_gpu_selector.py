"""GPU parity of the DFlash 2 path selector (dflash2_select) against the
float64 oracle.

Workload: the selector configuration (tiny fp32 drafter, B 16), 16 requests
with 64 context tokens.  Both sides draft the block; the oracle's top-16
candidates and their logits are the selector's candidate input on both sides;
each side computes the gates from its own final hidden states.  Bars: every
pair score rel <= 1e-4 (fp32, max-norm per request), the chosen path equal to
the oracle's at every position whose walk step wins by more than 1e-3 (the
comparison of a request stops at the first closer step, where the walks may
part), and the top-16 lists equal where the oracle's gaps exceed 0.05 (for a
bf16 drafter the oracle takes its candidates in the drafter's storage
precision, oracle.round_bf16)."""
import dataclasses

import numpy as np
import pytest

import oracle
import synth
from oracle import dflash2 as ds
from synth.configs import QWEN3_4B
from tests._gpu import BF16_RANK_MARGIN, GpuDraft, check_topk, hidden_rows, log, rel_inf

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("needs a GPU", allow_module_level=True)

K = 16


def _run(d, seed, bs, ctx, tables_np, zero_a=False, check_top16=True, conv=False):
    import block_diffusion_drafter_fuse_amd as dfa
    w_np = synth.make_weights(d, seed)
    g = GpuDraft(d, w_np, max_ctx=ctx + d.B, max_slots=bs, max_batch=bs)
    cw32 = None
    if conv:
        cw = synth.make_conv_weights(d, seed)
        g.dr.conv_attach([{st: {k: dfa.to_device(v) for k, v in t.items()} for st, t in layer.items()}
                          for layer in cw])
        cw32 = synth.conv_weights_as_f32(cw)
    slots = list(range(bs))
    g.fuse(slots, [ctx] * bs, hidden_rows(d, seed, [(r, 0, ctx) for r in slots]))
    w32 = synth.weights_as_f32(w_np)
    o = oracle.OracleDrafter(w32, d)
    for r in slots:
        o.fuse(r, synth.as_f32(synth.make_hidden(d, seed, r, 0, ctx)))
    anchors = synth.make_anchors(d, seed, bs)
    ids, vals, _ = g.draft(slots, anchors, top_k=K)
    t32 = {k: synth.as_f32([v])[0] for k, v in tables_np.items()}
    if zero_a:
        t32["a"] = np.zeros_like(t32["a"])
    cand = np.zeros((bs, d.B - 1, K), np.int32)
    u = np.zeros((bs, d.B - 1, K), np.float32)
    ref = []
    # bf16: candidate decisions in the drafter's storage precision
    store = oracle.round_bf16 if d.dtype == "bf16" else None
    for r in slots:
        if conv:
            out = ds.draft_block_conv(w32, d, o.cache(r), int(anchors[r]), cw32)
        else:
            out = o.draft(r, int(anchors[r]), store=store)
        if check_top16:
            _, bad = check_topk(ids[r], out["logits"], thr_rest=BF16_RANK_MARGIN if d.dtype == "bf16" else None)
            assert len(bad) == 0, f"req {r}: top-16 mismatch at {bad[:5]}"
        c, v = oracle.topk(out["logits"], K)
        cand[r], u[r] = c, v
        h = oracle.rms_norm(out["hidden"][1:], w32["g_final"], d.rms_eps)
        gates = ds.gate(t32["w_h"], h)
        ref.append(ds.select_path(int(anchors[r]), c, v.astype(np.float32), t32["a"], t32["b"], gates))
    dev = {k: dfa.to_device(v) for k, v in tables_np.items()}
    if zero_a:
        dev["a"].zero_()
    anc = torch.tensor(anchors, device="cuda")
    ct = torch.tensor(cand, device="cuda")
    ut = torch.tensor(u, device="cuda")
    path = torch.zeros((bs, d.B - 1), dtype=torch.int32, device="cuda")
    scores = torch.zeros((bs, d.B - 1, K, K), dtype=torch.float32, device="cuda")
    g.dr.select(bs, anc, ct, ut, K, dev, path, scores)
    torch.cuda.synchronize()
    g.close()
    return cand, u, path.cpu().numpy(), scores.cpu().numpy(), ref


def _compare(d, bs, path, scores, ref, tol, margin=1e-3):
    compared = 0
    for r in range(bs):
        ref_path, first, tables = ref[r]
        got = [np.repeat(first[None], K, 0)] + list(tables)
        for t in range(d.B - 1):
            err = rel_inf(scores[r, t], got[t])
            assert err <= tol, f"req {r} position {t + 1}: pair scores err {err}"
        prev = 0
        for t in range(d.B - 1):
            row = got[t][prev if t else 0]
            s = np.sort(row)
            if s[-1] - s[-2] <= margin:
                break
            assert path[r, t] == ref_path[t], f"req {r} position {t + 1}: path {path[r, t]} vs {ref_path[t]}"
            compared += 1
            prev = int(np.argmax(row))
    return compared


def test_gpu_selector_matches_oracle():
    wl = synth.get_config("dflash2_select")
    d = wl.dims
    log(f"case dflash2 selector: bs {wl.bs}, B {d.B}")
    tables = synth.make_selector_weights(d, wl.seed)
    cand, u, path, scores, ref = _run(d, wl.seed, wl.bs, wl.ctx[0], tables)
    compared = _compare(d, wl.bs, path, scores, ref, 1e-4)
    log(f"path positions compared: {compared} of {wl.bs * (d.B - 1)}")
    assert compared >= wl.bs * (d.B - 1) // 2
    # the walk is not simply the per-position argmax on this workload
    assert np.any(path != cand[:, :, 0])


def test_gpu_selector_with_conv():
    """The selector over a draft made with the two-tap convolution attached:
    the gates read the convolved drafter's final hidden states."""
    wl = synth.get_config("dflash2_select")
    d = wl.dims
    log(f"case dflash2 selector with the convolution: bs {wl.bs}, B {d.B}")
    tables = synth.make_selector_weights(d, wl.seed)
    cand, u, path, scores, ref = _run(d, wl.seed, wl.bs, wl.ctx[0], tables, conv=True)
    compared = _compare(d, wl.bs, path, scores, ref, 1e-4)
    log(f"path positions compared: {compared} of {wl.bs * (d.B - 1)}")
    assert compared >= wl.bs * (d.B - 1) // 2


def test_gpu_selector_zero_a_is_per_position_argmax():
    wl = synth.get_config("dflash2_select")
    d = wl.dims
    log("case dflash2 selector, A = 0")
    tables = synth.make_selector_weights(d, wl.seed)
    cand, u, path, _, _ = _run(d, wl.seed, 4, 32, tables, zero_a=True)
    assert np.array_equal(path, cand[:, :, 0])


def test_gpu_selector_bf16_qwen3_4b_shape():
    d = QWEN3_4B
    log("case dflash2 selector, Qwen3-4B shape bf16")
    tables = synth.make_selector_weights(d, 8)
    cand, u, path, scores, ref = _run(d, 8, 2, 96, tables)
    _compare(d, 2, path, scores, ref, 2e-2, margin=0.05)
