"""A whole draft step captured in a HIP graph (torch.cuda.CUDAGraph) replays to
the same bits as the eager step.

The step is fuse_ctx (each request's new verifier rows) + draft_block (top-4
ids, values and all logits) + accept, for a ragged batch of the tiny fp32
drafter, then the same for the Qwen3-8B-shaped bf16 drafter at bs 4 (split-K
tiled GEMMs, split-KV attention).  No call on the step path allocates,
copies to or from the host, or clears memory; kernel arguments (slot lengths,
split plans) are fixed at capture, so the host-side slot lengths are rewound
after capture exactly as after an eager step.  The graph is replayed several
times with eager library work and synchronisations in between, and every
replay is compared with the eager result.  The DFlash 2 convolution is
captured the same way at both of its launch forms."""
import numpy as np
import pytest

import synth
from synth.configs import QWEN3_8B
from tests._gpu import GpuDraft, hidden_rows, log

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("needs a GPU", allow_module_level=True)


def _run(d, w_np, seed, ctxs, news, top_k, replays=4, conv=False):
    bs = len(ctxs)
    slots = list(range(bs))
    g = GpuDraft(d, w_np, max_ctx=max(ctxs) + max(news) + d.B, max_slots=bs, max_batch=bs)
    dr, dfa = g.dr, g.dfa
    if conv:
        cw = synth.make_conv_weights(d, seed)
        dr.conv_attach([{st: {k: dfa.to_device(v) for k, v in t.items()} for st, t in layer.items()}
                        for layer in cw])
    g.fuse(slots, ctxs, hidden_rows(d, seed, [(r, 0, ctxs[r]) for r in slots]))
    hid = [dfa.to_device(h) for h in hidden_rows(d, seed, [(r, ctxs[r], news[r]) for r in slots])]
    anchor = torch.tensor(synth.make_anchors(d, seed, bs), device="cuda")
    ids = torch.zeros((bs, d.B - 1, top_k), dtype=torch.int32, device="cuda")
    vals = torch.zeros((bs, d.B - 1, top_k), dtype=torch.float32, device="cuda")
    logits = torch.zeros((bs, d.B - 1, d.V), dtype=torch.float32, device="cuda")
    rng = np.random.default_rng(seed)
    target = torch.tensor(rng.integers(0, d.V, size=(bs, d.B)).astype(np.int32), device="cuda")
    tau = torch.zeros(bs, dtype=torch.int32, device="cuda")
    bonus = torch.zeros(bs, dtype=torch.int32, device="cuda")

    def step():
        dr.fuse_ctx(slots, news, hid)
        dr.draft_block(slots, anchor, top_k, ids, vals, logits)
        dfa.accept(bs, d.B, ids, top_k, target, tau, bonus)

    def rewind():
        for r in slots:
            dr.slot_reset(r, ctxs[r])

    def snapshot():
        torch.cuda.synchronize()
        return [t.clone() for t in (ids, vals, logits, tau, bonus)]

    # eager reference (twice: the first call also sets kernel attributes)
    step()
    rewind()
    step()
    rewind()
    ref = snapshot()
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            step()
    torch.cuda.current_stream().wait_stream(side)
    rewind()  # capture advanced the host-side lengths; the graph itself does not
    for i in range(replays):
        for t in (ids, vals, logits, tau, bonus):
            t.fill_(-3)
        graph.replay()
        got = snapshot()
        for a, b in zip(got, ref):
            assert torch.equal(a, b), f"replay {i} differs from the eager step"
        # eager work between replays: a different draft on the same slots
        dr.draft_block(slots, torch.flip(anchor, [0]), top_k, ids, vals, logits)
        torch.cuda.synchronize()
        log(f"[graph] replay {i} identical")
    for r in slots:
        assert dr.slot_len(r) == ctxs[r]
    g.close()


def test_gpu_graph_replay_tiny_ragged():
    wl = synth.get_config("tiny")
    d = wl.dims
    log("[graph] tiny fp32, bs 4 ragged")
    _run(d, synth.make_weights(d, wl.seed), wl.seed, ctxs=[0, 17, 64, 100], news=[3, 0, 8, 1], top_k=4)


@pytest.mark.parametrize("bs", [4, 16])
def test_gpu_graph_replay_with_conv(bs):
    """The same with the DFlash 2 convolution attached (4 requests: one launch
    per site; 16: the corrections GEMM with split K, then the tap mix)."""
    wl = synth.get_config("dflash2_select")
    d = wl.dims
    log(f"[graph] dflash2 conv, fp32, bs {bs}")
    ctxs = [(7 * r + 5) % 70 for r in range(bs)]
    news = [(3 * r) % 9 for r in range(bs)]
    _run(d, synth.make_weights(d, wl.seed), wl.seed, ctxs=ctxs, news=news, top_k=1, conv=True)


def test_gpu_graph_replay_qwen3_8b_bs4():
    d = QWEN3_8B
    log("[graph] qwen3-8b shape bf16, bs 4")
    _run(d, synth.make_weights(d, 4), 4, ctxs=[512, 1500, 64, 3000], news=[7, 1, 16, 4], top_k=1, replays=3)
