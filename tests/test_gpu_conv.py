"""GPU parity of the DFlash 2 two-tap dynamic convolution (dflash2_conv_attach
+ dflash_draft_block) against the float64 oracle.

Workload: the selector configuration (tiny fp32 drafter, B 16), 16 requests
with 64 context tokens, 5 requests (a partial last row tile) and 11 requests
with B 6 — the many-row form: corrections GEMM on 64-token tiles with split
K, then the tap-mix kernel — and 1, 3 or 4 requests (the few-row form, the
tap mix in a GEMV epilogue, B 16 and B 6), convolution weights from synth.make_conv_weights at all four sites of
every layer.  Bars: logits rel <= 1e-4 (fp32), top-1 ids where the oracle's
margin exceeds 0.05; bf16 at the Qwen3-4B shape (2 requests: few rows; 5
requests: many rows): logits within 2e-2 of max |logit|.  An identity convolution (W = 0, kbase = (1, 0))
reproduces the plain draft, and detaching restores it bit for bit."""
import dataclasses

import numpy as np
import pytest

import oracle
import synth
from oracle import dflash2 as ds
from synth.configs import QWEN3_4B
from tests._gpu import GpuDraft, check_top1, hidden_rows, log, rel_inf

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("needs a GPU", allow_module_level=True)


def _dev_conv(cw):
    import block_diffusion_drafter_fuse_amd as dfa
    return [{s: {k: dfa.to_device(v) for k, v in t.items()} for s, t in layer.items()} for layer in cw]


def _setup(d, seed, bs, ctx):
    w_np = synth.make_weights(d, seed)
    g = GpuDraft(d, w_np, max_ctx=ctx + d.B, max_slots=bs, max_batch=bs)
    slots = list(range(bs))
    g.fuse(slots, [ctx] * bs, hidden_rows(d, seed, [(r, 0, ctx) for r in slots]))
    w32 = synth.weights_as_f32(w_np)
    o = oracle.OracleDrafter(w32, d)
    for r in slots:
        o.fuse(r, synth.as_f32(synth.make_hidden(d, seed, r, 0, ctx)))
    return g, o, w32, slots


def test_gpu_conv_matches_oracle():
    wl = synth.get_config("dflash2_select")
    d, bs = wl.dims, wl.bs
    log(f"case dflash2 conv: bs {bs}, B {d.B}, D {d.D}, N {d.N}")
    g, o, w32, slots = _setup(d, wl.seed, bs, wl.ctx[0])
    cw = synth.make_conv_weights(d, wl.seed)
    g.dr.conv_attach(_dev_conv(cw))
    cw32 = synth.conv_weights_as_f32(cw)
    anchors = synth.make_anchors(d, wl.seed, bs)
    ids, _, lg = g.draft(slots, anchors, top_k=1, logits=True)
    plain_diff = 0.0
    for r in slots:
        ref = ds.draft_block_conv(w32, d, o.cache(r), int(anchors[r]), cw32)["logits"]
        err = rel_inf(lg[r], ref)
        assert err <= 1e-4, f"req {r}: logits rel err {err}"
        _, bad = check_top1(ids[r][:, 0], ref)
        assert len(bad) == 0, f"req {r}: top-1 mismatch at {bad}"
        plain_diff = max(plain_diff, rel_inf(ref, o.draft(r, int(anchors[r]))["logits"]))
    # the convolution changes the draft (the comparison is not vacuous)
    assert plain_diff > 1e-2
    g.close()


@pytest.mark.parametrize("bs,B", [(1, 16), (4, 16), (3, 6)])
def test_gpu_conv_few_rows_matches_oracle(bs, B):
    """Few token rows take the one-launch form (tap mix in the corrections
    GEMM's epilogue on a GEMV engine); B = 6 puts a block boundary inside a
    16-row fragment, so row m - 1's scale is reduced by the epilogue itself."""
    wl = synth.get_config("dflash2_select")
    d = dataclasses.replace(wl.dims, B=B)
    log(f"case dflash2 conv, few rows: bs {bs}, B {B}")
    g, o, w32, slots = _setup(d, wl.seed, bs, 40)
    cw = synth.make_conv_weights(d, wl.seed)
    g.dr.conv_attach(_dev_conv(cw))
    cw32 = synth.conv_weights_as_f32(cw)
    anchors = synth.make_anchors(d, wl.seed, bs)
    ids, _, lg = g.draft(slots, anchors, top_k=1, logits=True)
    for r in slots:
        ref = ds.draft_block_conv(w32, d, o.cache(r), int(anchors[r]), cw32)["logits"]
        err = rel_inf(lg[r], ref)
        assert err <= 1e-4, f"req {r}: logits rel err {err}"
        _, bad = check_top1(ids[r][:, 0], ref)
        assert len(bad) == 0, f"req {r}: top-1 mismatch at {bad}"
    g.close()


@pytest.mark.parametrize("bs,B", [(5, 16), (11, 6)])
def test_gpu_conv_many_rows_ragged_matches_oracle(bs, B):
    """More than 64 token rows take the many-row form: 80 rows leave the
    last 64-token tile of the corrections GEMM part empty; with B = 6 (66
    rows) blocks straddle its tiles and the tap mix reads left neighbours
    across them."""
    wl = synth.get_config("dflash2_select")
    d = dataclasses.replace(wl.dims, B=B)
    log(f"case dflash2 conv, many rows: bs {bs}, B {B}, rows {bs * B}")
    g, o, w32, slots = _setup(d, wl.seed, bs, 40)
    cw = synth.make_conv_weights(d, wl.seed)
    g.dr.conv_attach(_dev_conv(cw))
    cw32 = synth.conv_weights_as_f32(cw)
    anchors = synth.make_anchors(d, wl.seed, bs)
    ids, _, lg = g.draft(slots, anchors, top_k=1, logits=True)
    for r in slots:
        ref = ds.draft_block_conv(w32, d, o.cache(r), int(anchors[r]), cw32)["logits"]
        err = rel_inf(lg[r], ref)
        assert err <= 1e-4, f"req {r}: logits rel err {err}"
        _, bad = check_top1(ids[r][:, 0], ref)
        assert len(bad) == 0, f"req {r}: top-1 mismatch at {bad}"
    g.close()


def test_gpu_conv_identity_and_detach():
    wl = synth.get_config("dflash2_select")
    d = wl.dims
    log("case dflash2 conv identity / detach")
    g, o, w32, slots = _setup(d, wl.seed, 4, 40)
    anchors = synth.make_anchors(d, wl.seed, 4)
    ids0, _, lg0 = g.draft(slots, anchors, top_k=1, logits=True)
    G = d.D // 16
    ident = {"w": np.zeros((2 * G, d.D), np.float32),
             "kbase": np.stack([np.ones(d.D, np.float32), np.zeros(d.D, np.float32)])}
    g.dr.conv_attach(_dev_conv([{s: ident for s in ds.CONV_SITES} for _ in range(d.N)]))
    _, _, lg1 = g.draft(slots, anchors, top_k=1, logits=True)
    assert rel_inf(lg1, lg0) <= 1e-5
    g.dr.conv_attach(None)
    ids2, _, lg2 = g.draft(slots, anchors, top_k=1, logits=True)
    assert np.array_equal(lg2, lg0) and np.array_equal(ids2, ids0)
    g.close()


def test_gpu_conv_rejects_unsupported_width():
    import block_diffusion_drafter_fuse_amd as dfa
    wl = synth.get_config("dflash2_select")
    d = dataclasses.replace(wl.dims, D=320)
    log("case dflash2 conv, D = 320")
    g = GpuDraft(d, synth.make_weights(d, 3), max_ctx=32, max_slots=1, max_batch=1)
    cw = _dev_conv(synth.make_conv_weights(dataclasses.replace(d, D=256), 3))
    with pytest.raises(dfa.DflashError) as e:
        g.dr.conv_attach(cw)
    assert e.value.code == -2
    g.close()


@pytest.mark.parametrize("bs", [2, 5])
def test_gpu_conv_bf16_qwen3_4b_shape(bs):
    """bf16 at the Qwen3-4B shape: 32 token rows (few-row form) and 80 rows
    (many-row form, a part-empty last token tile; the first, middle and last
    requests are compared)."""
    d = QWEN3_4B
    log(f"case dflash2 conv, Qwen3-4B shape bf16, bs {bs}")
    g, o, w32, slots = _setup(d, 8, bs, 96)
    cw = synth.make_conv_weights(d, 8)
    g.dr.conv_attach(_dev_conv(cw))
    anchors = synth.make_anchors(d, 8, bs)
    ids, _, lg = g.draft(slots, anchors, top_k=1, logits=True)
    cw32 = synth.conv_weights_as_f32(cw)
    for r in sorted({slots[0], slots[len(slots) // 2], slots[-1]}):
        ref = ds.draft_block_conv(w32, d, o.cache(r), int(anchors[r]), cw32)["logits"]
        err = np.abs(lg[r] - ref).max() / np.abs(ref).max()
        assert err <= 2e-2, f"req {r}: logits err {err}"
        _, bad = check_top1(ids[r][:, 0], ref, thr=0.05)
        assert len(bad) == 0, f"req {r}: top-1 mismatch at {bad}"
    g.close()
