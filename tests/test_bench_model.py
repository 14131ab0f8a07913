"""The benchmark's algorithmic work model (bytes and flops per step, the
roofline denominators) against the figures derived independently for the
measured runs: 8B bs 1 moves 3.510 GB and computes 57 GFLOP; the 4B bs 1 step
moves 1.947 GB; the 8B bs 32 step moves the 3.43 GB of weights plus 20 KB of
context K/V per cached token and computes 1.82 TFLOP."""
import bench
import synth


def _work(name):
    wl = synth.get_config(name)
    return wl, bench.step_work(wl.dims, wl)


def test_bs1_8b_work():
    _, (byts, flops) = _work("qwen3_8b_bs1")
    assert abs(byts / 3.510e9 - 1) < 1e-3
    assert abs(flops / 57e9 - 1) < 0.01


def test_bs1_4b_work():
    _, (byts, _) = _work("qwen3_4b_bs1")
    assert abs(byts / 1.947e9 - 1) < 2e-3


def test_bs32_8b_work():
    wl, (byts, flops) = _work("qwen3_8b_bs32")
    kv_per_token = wl.dims.N * 2 * wl.dims.Hkv * wl.dims.hd * 2  # 20 KB
    assert kv_per_token == 20480
    assert abs((byts - sum(wl.ctx) * kv_per_token) / 3.43e9 - 1) < 0.01
    assert abs(flops / 1.82e12 - 1) < 0.01


def test_kernel_work_sums_to_step_flops():
    for name in ("qwen3_8b_bs1", "qwen3_8b_bs32", "qwen3_4b_bs1"):
        wl, (_, flops) = _work(name)
        kw = bench.kernel_work(wl.dims, wl)
        assert abs(sum(f * c for _, f, c in kw.values()) - flops) <= 1e-6 * flops
