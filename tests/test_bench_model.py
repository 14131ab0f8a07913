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


# ------------------------------------------------------------------ counter parsing

_HDR = ("Correlation_Id,Dispatch_Id,Agent_Id,Queue_Id,Process_Id,Thread_Id,Grid_Size,Kernel_Id,Kernel_Name,"
        "Workgroup_Size,LDS_Block_Size,Scratch_Size,VGPR_Count,Accum_VGPR_Count,SGPR_Count,Counter_Name,"
        "Counter_Value,Start_Timestamp,End_Timestamp\n")


def _csv(path, rows):
    """rows: (dispatch id, kernel name, counter, value); one line each (a
    dispatch's instances are separate lines, as rocprofv3 writes them)."""
    with open(path, "w") as fh:
        fh.write(_HDR)
        for did, name, ctr, val in rows:
            fh.write(f'1,{did},"Agent 1",1,1,1,256,1,"{name}",256,0,0,8,0,16,"{ctr}",{val},0,1\n')
    return str(path)


QKV = "void dfl::gemm_tiled_kernel<unsigned short, 128, 192, 4, 2, 3, false, dfl::EpiQKV<unsigned short> >(x)"
ATTN = "void dfl::attn_kernel<unsigned short, 128, 4, 1, 2, 64, 2>(dfl::AttnArgs<unsigned short>)"
OUT = "void dfl::gemm_tiled_kernel<unsigned short, 128, 128, 2, 4, 3, false, dfl::EpiResidualNorm<unsigned short> >(x)"
SWIGLU = "void dfl::gemm_tiled_kernel<unsigned short, 256, 192, 4, 2, 2, false, dfl::EpiSwiGLU<unsigned short> >(x)"
COPY = "void at::native::vectorized_elementwise_kernel<4, at::native::BitwiseNotFunctor<unsigned char> >(x)"


def test_read_counter_csv_combines_instances():
    import tempfile, os
    with tempfile.TemporaryDirectory() as d:
        p = _csv(os.path.join(d, "c.csv"), [(1, QKV, "FETCH_SIZE", 10.0), (1, QKV, "FETCH_SIZE", 5.0),
                                           (2, ATTN, "FETCH_SIZE", 7.0), (1, QKV, "GRBM_GUI_ACTIVE", 3.0),
                                           (1, QKV, "GRBM_GUI_ACTIVE", 9.0)])
        assert bench.read_counter_csv(p, "FETCH_SIZE") == [(QKV, 15.0), (ATTN, 7.0)]
        assert bench.read_counter_csv(p, "GRBM_GUI_ACTIVE", "max") == [(QKV, 9.0)]


def test_dispatch_kinds_tell_o_from_down():
    # the same residual epilogue is the O projection after attention and the
    # down projection after gate/up
    assert bench.kind_of_dispatch(OUT, "attn_combine") == "o_gemm"
    assert bench.kind_of_dispatch(OUT, "gateup_gemm") == "down_gemm"
    assert bench.kind_of_dispatch(SWIGLU, "o_gemm") == "gateup_gemm"
    assert bench.kind_of_dispatch(COPY, None) is None


def test_counter_summary_per_xcd_cycles_and_mfma_rate():
    import tempfile, os
    gui = 8 * 2.4e9 * 100e-6          # 100 us per XCD at the nominal clock, summed over 8 XCDs
    mops = 2.5e15 * 0.5 * 100e-6 / 512  # half the bf16 peak over those 100 us
    busy = 0.25 * 2.4e9 * 100e-6 * 1024
    with tempfile.TemporaryDirectory() as d:
        p = _csv(os.path.join(d, "m.csv"), [(1, QKV, "GRBM_GUI_ACTIVE", gui),
                                           (1, QKV, "SQ_INSTS_VALU_MFMA_MOPS_BF16", mops / 2),
                                           (1, QKV, "SQ_INSTS_VALU_MFMA_MOPS_BF16", mops / 2),
                                           (1, QKV, "SQ_VALU_MFMA_BUSY_CYCLES", busy)])
        row = bench.counter_summary([p])["qkv_gemm"]
    assert abs(row["busy_us_per_xcd"] - 100.0) < 1e-6
    assert abs(row["mfma_bf16_frac_of_peak"] - 0.5) < 1e-3
    assert abs(row["mfma_busy_frac"] - 0.25) < 1e-3
    assert abs(row["mfma_bf16_flops"] - 512 * mops) < 1.0


def test_traffic_summary_scales_by_the_reference_copy():
    import tempfile, os
    mib = 512
    with tempfile.TemporaryDirectory() as d:
        # the copy reads and writes 512 MiB; the counters report half the reads, all the writes (KiB)
        f = _csv(os.path.join(d, "f.csv"), [(1, QKV, "FETCH_SIZE", 1000.0), (2, COPY, "FETCH_SIZE", mib * 512.0)])
        w = _csv(os.path.join(d, "w.csv"), [(1, QKV, "WRITE_SIZE", 100.0), (2, COPY, "WRITE_SIZE", mib * 1024.0)])
        t = bench.traffic_summary(f, w, mib, "wl")
    assert abs(t["fetch_factor"] - 2.0) < 1e-9 and abs(t["write_factor"] - 1.0) < 1e-9
    k = t["kernels"]["wl:qkv_gemm"]
    assert k["fetch_bytes"] == 2 * 1000 * 1024 and k["write_bytes"] == 100 * 1024
    assert k["bytes_per_launch"] == k["fetch_bytes"] + k["write_bytes"]


def test_more_than_one_gpu_is_refused_with_a_message():
    import subprocess, sys, os
    r = subprocess.run([sys.executable, os.path.join(os.path.dirname(bench.__file__), "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""
