"""dflash_spec_draft_static (the drafting call that allocates nothing: its
scratch is a fixed per-GPU array) against dflash_spec_draft on a ctx of the
same vocabulary and block size, through the C ABI: drafted ids and the rows'
log-sum-exps bit-identical, on two calls in a row, the second smaller (fewer
requests, a smaller vocabulary and block), so stale scratch contents from the
first call must not leak into the second."""
import dataclasses

import numpy as np
import pytest

import synth
from synth.configs import _tiny
from tests._gpu import GpuDraft, log

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("needs a GPU", allow_module_level=True)


def _ctx_draft(V, B, n, dl, temp, seed, req):
    d = dataclasses.replace(_tiny(B=B), V=V)
    g = GpuDraft(d, synth.make_weights(d, 0), max_ctx=32, max_slots=1, max_batch=n)
    try:
        cand = torch.full((n, B - 1), -7, dtype=torch.int32, device="cuda")
        lse = torch.full((n, B - 1), float("nan"), dtype=torch.float32, device="cuda")
        g.dr.spec_draft(n, dl, temp, seed, req, cand, lse)
        torch.cuda.synchronize()
        return cand.cpu().numpy(), lse.cpu().numpy()
    finally:
        g.close()


def _static_draft(V, B, n, dl, temp, seed, req):
    import block_diffusion_drafter_fuse_amd as dfa
    cand = torch.full((n, B - 1), -7, dtype=torch.int32, device="cuda")
    lse = torch.full((n, B - 1), float("nan"), dtype=torch.float32, device="cuda")
    dfa.spec_draft_static(n, V, B, dl, temp, seed, req, cand, lse)
    torch.cuda.synchronize()
    return cand.cpu().numpy(), lse.cpu().numpy()


@pytest.mark.parametrize("order", ["large_then_small"])
def test_spec_draft_static_matches_ctx_call(order):
    cases = [(151936, 16, 32, 1.0, 77), (1024, 5, 3, 0.7, 78)]
    for V, B, n, temp, seed in cases:
        log(f"[no-alloc] V {V} B {B} n_req {n} T {temp}")
        dl_np, _ = synth.make_sampling_logits(n, B, V, seed=seed)
        dl = torch.from_numpy(np.ascontiguousarray(dl_np)).cuda()
        req = torch.tensor([5 * r + 2 for r in range(n)], dtype=torch.int32, device="cuda")
        c_ref, l_ref = _ctx_draft(V, B, n, dl, temp, seed, req)
        c_got, l_got = _static_draft(V, B, n, dl, temp, seed, req)
        assert np.array_equal(c_got, c_ref), f"V {V} B {B}: drafted ids differ"
        assert np.array_equal(l_got, l_ref), f"V {V} B {B}: log-sum-exps differ"
        assert (c_got >= 0).all() and (c_got < V).all()


def test_spec_draft_static_limits():
    import block_diffusion_drafter_fuse_amd as dfa
    dl = torch.zeros((1, 15, 64), dtype=torch.float32, device="cuda")
    req = torch.zeros(1, dtype=torch.int32, device="cuda")
    cand = torch.zeros((1, 15), dtype=torch.int32, device="cuda")
    for args, code in [((65, 64, 16), -3), ((1, 262145, 16), -3), ((1, 64, 17), -2), ((1, 64, 1), -2)]:
        with pytest.raises(dfa.DflashError) as e:
            dfa.spec_draft_static(*args, dl, 1.0, 1, req, cand)
        assert e.value.code == code, args
