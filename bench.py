#!/usr/bin/env python3
"""Throughput of the DFlash draft step on one MI355X.

One step = dflash_fuse_ctx over the tokens each request committed in the
previous round + dflash_draft_block (top-1 candidates for block offsets
1..B-1) + dflash_accept, for every request of the batch, with all inputs
already resident in HBM.  After each step the slot lengths are rewound on the
host so every step has the same shape.

Headline workload: Qwen3-8B-shaped drafter, bs 32 ragged (context ~ U{512..8192},
previous-round tau ~ clamped geometric with mean 6.5), bf16 weights and inputs,
seeded synthetic data.  The same line carries the bs 1 Qwen3-8B-shaped step
(context 4096, 7 new tokens) under "bs1", the bs 1 Qwen3-4B-shaped step
(context 2048) under "bs1_4b", and context prefill (one fuse call of 2048
tokens at the 4B shape and of 8192 tokens at the 8B shape) under "prefill".
Metric: drafted tokens/s = blocks/s x B; the per-step spread (p10/p50/p90)
comes from an event after every timed step.

`roofline` reports the kernel with the largest time share, timed live with HIP
events recorded by the library on the launch stream over a second pass of the
timed steps (the step time itself comes from an uninstrumented pass);
its achieved rate is the kernel's algorithmic bytes (HBM-bound kernels) or
flops (MFMA-bound) per launch divided by its mean launch time, against the
nominal MI355X peak; `achievable_peaks` adds what standard operations reach
on the same GPU (a plain 1 GiB device copy, a reduction over 1 GiB, an 8192^3
bf16 GEMM of the vendor library) as context for those fractions.
`cpu_baseline` times the float64 CPU oracle on a sample of the same workload's
requests (evenly spaced context quantiles) and scales it to the whole batch
step; it records the host CPU count, the BLAS vendor and threads, and one
single-thread figure.
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0           # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0       # MI355X dense bf16 MFMA
FP32_PEAK_TFLOPS = 157.3        # MI355X fp32 (dense MFMA / vector)
RIDGE = BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)


def elt(d):
    return 2 if d.dtype == "bf16" else 4


def kernel_work(d, wl):
    """Algorithmic (bytes, flops) per launch and launches per step, per kernel
    kind: weights read once, activations read/written once, context K/V read
    once per layer."""
    e = elt(d)
    bs, B = wl.bs, d.B
    M, Mlm = bs * B, bs * (B - 1)
    n = sum(wl.n_new)
    sctx = sum(wl.ctx)
    qkv = (d.Hq + 2 * d.Hkv) * d.hd
    w = {}
    w["fuse_gemm"] = (d.D * d.L * d.Dt * e + n * d.L * d.Dt * e + n * d.D * 4,
                      2.0 * n * d.D * d.L * d.Dt, 1)
    w["fuse_norm"] = (n * d.D * (4 + e), 0.0, 1)
    w["ctx_kv_gemm"] = (d.N * 2 * d.Hkv * d.hd * d.D * e + n * d.D * e + n * d.N * 2 * d.Hkv * d.hd * e,
                        2.0 * n * d.N * 2 * d.Hkv * d.hd * d.D, 1)
    w["embed"] = (M * d.D * (4 + e), 0.0, 1)
    w["norm"] = (M * d.D * (4 + e), 0.0, 2 * d.N + 1)
    w["qkv_gemm"] = (qkv * d.D * e + M * d.D * e + M * qkv * e, 2.0 * M * qkv * d.D, d.N)
    w["attention"] = (sctx * 2 * d.Hkv * d.hd * e + M * (d.Hq + 2 * d.Hkv) * d.hd * e,
                      sum(4.0 * d.Hq * B * (c + B) * d.hd for c in wl.ctx), d.N)
    # the split partials are not algorithmic traffic: only the attention output counts
    w["attn_combine"] = (M * d.Hq * d.hd * e, 0.0, d.N)
    w["o_gemm"] = (d.D * d.Hq * d.hd * e + M * d.Hq * d.hd * e + 2 * M * d.D * 4,
                   2.0 * M * d.D * d.Hq * d.hd, d.N)
    w["gateup_gemm"] = (2 * d.I * d.D * e + M * d.D * e + M * d.I * e, 2.0 * M * 2 * d.I * d.D, d.N)
    w["down_gemm"] = (d.D * d.I * e + M * d.I * e + 2 * M * d.D * 4, 2.0 * M * d.D * d.I, d.N)
    w["lm_head"] = (d.V * d.D * e + Mlm * d.D * e, 2.0 * Mlm * d.V * d.D, 1)
    return w


def step_work(d, wl):
    """Whole-step algorithmic bytes and flops: every weight once, the context
    K/V once per layer, the fused rows in and their K/V out."""
    e = elt(d)
    n = sum(wl.n_new)
    weights = (d.D * d.L * d.Dt + d.N * 2 * d.D * d.Hkv * d.hd
               + d.N * (d.D * d.Hq * d.hd + 2 * d.D * d.Hkv * d.hd + d.Hq * d.hd * d.D + 3 * d.D * d.I)
               + d.V * d.D)
    byts = e * weights + sum(wl.ctx) * d.N * 2 * d.Hkv * d.hd * e + n * (d.L * d.Dt + d.N * 2 * d.Hkv * d.hd) * e
    kw = kernel_work(d, wl)
    flops = sum(f * c for _, f, c in kw.values())
    return byts, flops


def roof_entry(kind, d, wl, ms_per_launch, traffic):
    byts, flops, _ = kernel_work(d, wl)[kind]
    if flops / max(byts, 1) >= RIDGE:
        ach = flops / (ms_per_launch * 1e-3) / 1e12
        peak = BF16_PEAK_TFLOPS if d.dtype == "bf16" else FP32_PEAK_TFLOPS
        return {"bound": "mfma", "achieved": round(ach, 2), "peak": peak, "unit": "TFLOP/s",
                "frac": round(ach / peak, 4), "traffic": traffic, "kernel": kind,
                "launch_ms": round(ms_per_launch, 5), "algorithmic_flops": flops}
    ach = byts / (ms_per_launch * 1e-3) / 1e9
    return {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": traffic, "kernel": kind,
            "launch_ms": round(ms_per_launch, 5), "algorithmic_bytes": byts}


# Kernel kind of a dispatch from its (demangled) name, in draft-step order; the
# output and down projections share an epilogue and alternate within a layer.
KIND_PATTERNS = (("EpiQKV", "qkv_gemm"), ("attn_combine", "attn_combine"), ("attn_kernel", "attention"),
                 ("EpiSwiGLU", "gateup_gemm"), ("EpiTop1", "lm_head"), ("lmhead_lds", "lm_head"),
                 ("topk_merge", "topk_merge"), ("embed_kernel", "embed"))


def kind_of_dispatch(name, prev):
    if "EpiResidualNorm" in name:
        return "down_gemm" if prev == "gateup_gemm" else "o_gemm"
    for pat, kind in KIND_PATTERNS:
        if pat in name:
            return kind
    return None


def read_counter_csv(path, counter, reduce="sum"):
    """[(kernel name, value)] per dispatch, in dispatch order, from a rocprofv3
    counter_collection.csv (rows of one dispatch combined by sum or max)."""
    per = {}
    with open(path) as fh:
        for r in csv.DictReader(fh):
            if r["Counter_Name"] != counter:
                continue
            did = int(r["Dispatch_Id"])
            v = float(r["Counter_Value"])
            if did in per:
                name, old = per[did]
                v = old + v if reduce == "sum" else max(old, v)
            else:
                name = r["Kernel_Name"]
            per[did] = (name, v)
    return [per[k] for k in sorted(per)]


SIMDS = 1024       # MI355X: 256 CUs x 4 SIMDs
XCDS = 8           # GRBM_GUI_ACTIVE of a dispatch comes summed over the 8 XCDs
GPU_CLOCK_HZ = 2.4e9


def counter_summary(paths):
    """Per kernel kind of the draft step: the median over dispatches of every
    counter in the given rocprofv3 counter_collection.csv files (SQ counters
    summed over the instances of a dispatch, GRBM_GUI_ACTIVE its maximum), and
    where the counters are present the derived figures: the dispatch's busy
    cycles per XCD (GRBM_GUI_ACTIVE / 8, which includes the counter window's own
    overhead, so the fractions below are lower bounds), the MFMA utilisation
    SQ_VALU_MFMA_BUSY_CYCLES / (cycles per XCD x SIMDs), the executed bf16 MFMA
    flops 512 x SQ_INSTS_VALU_MFMA_MOPS_BF16 (padding of partial tiles
    included), and their rate over those cycles at the nominal 2.4 GHz clock."""
    table = {}
    for path in paths:
        counters = set()
        with open(path) as fh:
            for r in csv.DictReader(fh):
                counters.add(r["Counter_Name"])
        for c in sorted(counters):
            prev = None
            for name, v in read_counter_csv(path, c, "max" if c.startswith("GRBM") else "sum"):
                kind = kind_of_dispatch(name, prev)
                if kind is None:
                    continue
                prev = kind
                table.setdefault(kind, {}).setdefault(c, []).append(v)
    out = {}
    for kind, cs in table.items():
        row = {c: float(np.median(v)) for c, v in cs.items()}
        row["dispatches"] = max(len(v) for v in cs.values())
        gui = row.get("GRBM_GUI_ACTIVE")
        if gui:
            gui /= XCDS
            row["busy_us_per_xcd"] = round(gui / GPU_CLOCK_HZ * 1e6, 1)
        if gui and "SQ_VALU_MFMA_BUSY_CYCLES" in row:
            row["mfma_busy_frac"] = round(row["SQ_VALU_MFMA_BUSY_CYCLES"] / (gui * SIMDS), 4)
        if gui and "SQ_INSTS_VALU_MFMA_MOPS_BF16" in row:
            row["mfma_bf16_flops"] = 512.0 * row["SQ_INSTS_VALU_MFMA_MOPS_BF16"]
            tf = row["mfma_bf16_flops"] / (gui / GPU_CLOCK_HZ) / 1e12
            row["mfma_bf16_tflops"] = round(tf, 1)
            row["mfma_bf16_frac_of_peak"] = round(tf / BF16_PEAK_TFLOPS, 4)
        out[kind] = row
    return out


def traffic_summary(fetch_csv, write_csv, copy_mib, workload):
    """HBM bytes per launch per kernel kind from one FETCH_SIZE and one
    WRITE_SIZE run (KiB per dispatch), each scaled by what the same counter
    reads for the reference pass over copy_mib MiB (the last elementwise dispatch
    of the run: copy_mib MiB read, copy_mib MiB written)."""
    out = {}
    for path, counter, key in ((fetch_csv, "FETCH_SIZE", "fetch"), (write_csv, "WRITE_SIZE", "write")):
        disp = read_counter_csv(path, counter)
        copies = [v for n, v in disp if "elementwise" in n]
        if not copies or copies[-1] <= 0:
            raise SystemExit(f"{path}: no reference copy dispatch with a {counter} value")
        factor = copy_mib * 1024.0 / copies[-1]
        out[f"{key}_factor"] = round(factor, 4)
        prev = None
        vals = {}
        for name, v in disp:
            kind = kind_of_dispatch(name, prev)
            if kind is None:
                continue
            prev = kind
            vals.setdefault(kind, []).append(v * factor * 1024.0)
        out[key] = {k: (float(np.median(v)), len(v)) for k, v in vals.items()}
    kernels = {}
    for kind in out["fetch"]:
        if kind not in out["write"]:
            continue
        fb, n = out["fetch"][kind]
        wb, _ = out["write"][kind]
        kernels[f"{workload}:{kind}"] = {"bytes_per_launch": int(fb + wb), "fetch_bytes": int(fb),
                                         "write_bytes": int(wb), "dispatches": n}
    return {"fetch_factor": out["fetch_factor"], "write_factor": out["write_factor"], "kernels": kernels}


def source_sha():
    h = hashlib.sha256()
    cdir = os.path.join(ROOT, "block_diffusion_drafter_fuse_amd", "csrc")
    for f in sorted(os.listdir(cdir)):
        h.update(open(os.path.join(cdir, f), "rb").read())
    return h.hexdigest()[:16]


def traffic_for(kind, workload):
    """HBM bytes per launch from committed rocprofv3 counter summaries, if they
    were taken on the current kernel sources; else None."""
    p = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(p):
        return None
    try:
        t = json.load(open(p))
    except ValueError:
        return None
    if t.get("source_sha") != source_sha():
        return None
    k = t.get("kernels", {}).get(f"{workload}:{kind}")
    return None if k is None else k.get("bytes_per_launch")


class Workbench:
    """Drafter + resident inputs for one workload."""

    def __init__(self, wl, w_dev, torch):
        import block_diffusion_drafter_fuse_amd as dfa
        import synth
        self.torch = torch
        self.wl = wl
        d = wl.dims
        self.d = d
        bs = wl.bs
        self.slots = list(range(bs))
        self.dr = dfa.Drafter(d, w_dev, max(wl.ctx) + d.B, bs, bs)
        self.pre = [c - n for c, n in zip(wl.ctx, wl.n_new)]
        for r in range(bs):
            if self.pre[r]:
                hid = [dfa.to_device(h) for h in synth.make_hidden(d, wl.seed, r, 0, self.pre[r])]
                self.dr.fuse_ctx([r], [self.pre[r]], hid)
                del hid
        rows = [synth.make_hidden(d, wl.seed, r, self.pre[r], wl.n_new[r]) for r in range(bs)]
        self.hid = [dfa.to_device(np.ascontiguousarray(np.concatenate([x[l] for x in rows], 0)))
                    for l in range(d.L)]
        self.anchor = torch.tensor(synth.make_anchors(d, wl.seed, bs), device="cuda")
        self.ids = torch.zeros((bs, d.B - 1, 1), dtype=torch.int32, device="cuda")
        m = synth.draw_first_mismatch("geometric", bs, d.B, wl.seed)
        self.m = m
        self.target = None
        self.tau = torch.zeros(bs, dtype=torch.int32, device="cuda")
        self.bonus = torch.zeros(bs, dtype=torch.int32, device="cuda")
        self.dfa = dfa
        torch.cuda.synchronize()

    def step(self):
        wl = self.wl
        self.dr.fuse_ctx(self.slots, wl.n_new, self.hid)
        self.dr.draft_block(self.slots, self.anchor, 1, self.ids)
        self.dfa.accept(wl.bs, self.d.B, self.ids, 1, self.target, self.tau, self.bonus)
        for r in self.slots:
            self.dr.slot_reset(r, self.pre[r])

    def prepare_targets(self):
        """Targets giving the drawn acceptance lengths on this drafter's own
        candidates (timing input only; acceptance parity is tested elsewhere)."""
        import synth
        self.dr.fuse_ctx(self.slots, self.wl.n_new, self.hid)
        self.dr.draft_block(self.slots, self.anchor, 1, self.ids)
        self.torch.cuda.synchronize()
        cand = self.ids[:, :, 0].cpu().numpy()
        for r in self.slots:
            self.dr.slot_reset(r, self.pre[r])
        tgt = synth.make_targets(cand, self.m, self.d.V, self.wl.seed)
        self.target = self.torch.tensor(tgt, device="cuda")

    def breakdown(self, steps=3):
        self.dr.profile_enable(list(self.dfa.KERNEL_KINDS[:-1]), 4096)
        for _ in range(steps):
            self.step()
        res = self.dr.profile_read()
        self.dr.profile_enable([], 0)
        return {k: (ms / steps, cnt // steps) for k, (ms, cnt) in res.items()}

    def timed(self, steps, warmup, kind):
        """Step time over `steps` uninstrumented steps, then (kind given) the
        mean duration of that kernel kind from the library's HIP events around
        each of its launches over a second pass of the same `steps` steps.  The
        passes are separate because an event pair around a launch idles the GPU
        for a few microseconds, which would inflate the step time."""
        torch = self.torch
        for _ in range(warmup):
            self.step()
        # one event after every step (recording an event does not wait), for
        # the per-step spread as well as the mean
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        evs[0].record()
        for i in range(steps):
            self.step()
            evs[i + 1].record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        ms = evs[0].elapsed_time(evs[-1]) / steps
        self.step_ms = [evs[i].elapsed_time(evs[i + 1]) for i in range(steps)]
        kern = None
        if kind:
            kinds = [kind] if isinstance(kind, str) else list(kind)
            self.dr.profile_enable(kinds, 64 * len(kinds) * (steps + 1))
            for _ in range(steps):
                self.step()
            torch.cuda.synchronize()
            res = self.dr.profile_read()
            self.dr.profile_enable([], 0)
            per = {}
            for k in kinds:
                tot, cnt = res.get(k, (0.0, 0))
                per[k] = (tot / max(cnt, 1), cnt)
            kern = per[kind] if isinstance(kind, str) else per
        return ms, wall / steps * 1e3, kern


def measure_conv(wb, steps, warmup, label):
    """The same step with the DFlash 2 two-tap convolution attached at all four
    sites of every layer (seeded synthetic weights); the convolution's own
    kernels (tap-correction GEMMs and tap mixes) are timed with events."""
    import synth
    d = wb.d
    cw = synth.make_conv_weights(d, wb.wl.seed)
    dev = [{s: {k: wb.dfa.to_device(v) for k, v in t.items()} for s, t in layer.items()} for layer in cw]
    wb.dr.conv_attach(dev)
    ms, _, kern = wb.timed(steps, warmup, "conv")
    wb.dr.conv_attach(None)
    e = elt(d)
    byts = 4 * d.N * ((d.D // 8) * d.D + 2 * d.D) * e
    return {"workload": f"{label} step with the two-tap convolution",
            "ms_per_step": round(ms, 4), "conv_ms_per_step": round(kern[0] * kern[1] / steps, 4),
            "conv_launches_per_step": kern[1] // steps, "conv_weight_bytes": byts,
            "note": "4 sites x N layers: tap-correction GEMM (64-token tiles, split K) + tap-mix kernel; with "
                    "at most 64 token rows one launch per site (the mix in the GEMV's epilogue); "
                    "ms_per_step is the whole step with the convolution attached"}


def measure(wl, w_dev, torch, steps, warmup, label, conv=False):
    wb = Workbench(wl, w_dev, torch)
    wb.prepare_targets()
    for _ in range(2):
        wb.step()
    torch.cuda.synchronize()
    bd = wb.breakdown()
    # the three kernel kinds with the most time per step: the first is the
    # dominant kernel of the roofline, the next two (close behind at bs 32, in
    # an order that can change from run to run) are reported beside it
    top = sorted(bd, key=lambda k: -bd[k][0])[:3]
    dom = top[0]
    ms, wall_ms, kerns = wb.timed(steps, warmup, top)
    kern = kerns[dom]
    d = wl.dims
    byts, flops = step_work(d, wl)
    blocks_s = wl.bs / (ms * 1e-3)
    out = {
        "workload": label,
        "ms_per_step": round(ms, 4),
        "wall_ms_per_step": round(wall_ms, 4),
        "blocks_per_s": round(blocks_s, 1),
        "drafted_tokens_per_s": round(blocks_s * d.B, 1),
        "step_algorithmic_bytes": byts,
        "step_algorithmic_flops": flops,
        "step_hbm_roof_frac": round(byts / (ms * 1e-3) / (HBM_PEAK_GBS * 1e9), 4),
        "step_mfma_roof_frac": round(flops / (ms * 1e-3) / (BF16_PEAK_TFLOPS * 1e12), 4),
        "step_ms_p10_p50_p90": [round(float(x), 4) for x in np.percentile(wb.step_ms, [10, 50, 90])],
        "breakdown_ms": {k: round(v[0], 4) for k, v in sorted(bd.items(), key=lambda kv: -kv[1][0])},
        "roofline": roof_entry(dom, d, wl, kern[0], traffic_for(dom, label)),
    }
    out["roofline"]["launches_timed"] = kern[1]
    out["roofline_next"] = []
    for nxt in top[1:]:
        if nxt in kernel_work(d, wl):
            e = roof_entry(nxt, d, wl, kerns[nxt][0], traffic_for(nxt, label))
            e["launches_timed"] = kerns[nxt][1]
            out["roofline_next"].append(e)
    if conv:
        out["conv"] = measure_conv(wb, steps, warmup, label)
        out["conv"]["overhead_frac"] = round(out["conv"]["ms_per_step"] / ms - 1.0, 4)
    wb.dr.close()
    del wb
    torch.cuda.synchronize()
    return out


def measure_lm_shard(workloads, w_dev, torch, steps, warmup, shards=8):
    """The LM head as one GPU of a vocabulary-sharded deployment would run it:
    the same step with the vocabulary cut to its first ceil(V/shards) rows,
    rounded up to whole 64-row groups (the
    embedding stays tied, anchors drawn inside the shard), the LM-head kernel
    timed with events.  Each GPU would then all-gather bs*(B-1)*k (value, id)
    pairs and merge them; that exchange is not part of this single-GPU run."""
    import dataclasses
    out = {}
    for wl in workloads:
        d = dataclasses.replace(wl.dims, V=-(-wl.dims.V // (shards * 64)) * 64)  # rows kept whole 64-row groups
        wls = dataclasses.replace(wl, dims=d)
        w = dict(w_dev)
        w["embed"] = w_dev["embed"][:d.V]
        w["w_lm"] = w_dev["w_lm"][:d.V]
        wb = Workbench(wls, w, torch)
        wb.prepare_targets()
        ms, _, kern = wb.timed(steps, warmup, "lm_head")
        us = kern[0] * 1000
        rows = wl.bs * (d.B - 1)
        byts = d.V * d.D * (2 if d.dtype == "bf16" else 4)
        flops = 2.0 * rows * d.V * d.D
        ent = {"vocab_rows": d.V, "token_rows": rows, "us_per_launch": round(us, 1),
               "hbm_GBs": round(byts / us / 1e3, 1), "hbm_roof_frac": round(byts / us / 1e3 / HBM_PEAK_GBS, 4),
               "mfma_TFLOPs": round(flops / us / 1e6, 1),
               "mfma_roof_frac": round(flops / us / 1e6 / BF16_PEAK_TFLOPS, 4),
               "allgather_bytes_top16": rows * 16 * 8}
        out[f"{wl.dims.name}_bs{wl.bs}"] = ent
        del wb
        torch.cuda.synchronize()
    return out


def measure_prefill(d, w_dev, torch, n_tok, seed, reps=3):
    """Context prefill: one dflash_fuse_ctx call that fuses `n_tok` verifier
    rows of one request (fusion GEMM, RMSNorm and the per-layer context K/V
    projection into the cache), timed with events over `reps` calls (the slot
    is rewound between calls).  Above the ridge: reported against the MFMA
    peak."""
    import block_diffusion_drafter_fuse_amd as dfa
    import synth
    dr = dfa.Drafter(d, w_dev, n_tok + d.B, 1, 1)
    hid = [dfa.to_device(h) for h in synth.make_hidden(d, seed, 0, 0, n_tok)]
    dr.fuse_ctx([0], [n_tok], hid)
    dr.slot_reset(0, 0)
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    ms = 0.0
    for _ in range(reps):
        start.record()
        dr.fuse_ctx([0], [n_tok], hid)
        stop.record()
        torch.cuda.synchronize()
        ms += start.elapsed_time(stop)
        dr.slot_reset(0, 0)
    ms /= reps
    e = elt(d)
    flops = 2.0 * n_tok * (d.D * d.L * d.Dt + d.N * 2 * d.D * d.Hkv * d.hd)
    byts = e * (d.D * d.L * d.Dt + d.N * 2 * d.D * d.Hkv * d.hd) + n_tok * (d.L * d.Dt + d.N * 2 * d.Hkv * d.hd) * e
    dr.close()
    del dr, hid
    torch.cuda.synchronize()
    return {"workload": f"{d.name} prefill fuse of {n_tok} tokens", "ms_per_call": round(ms, 4),
            "tokens_per_s": round(n_tok / (ms * 1e-3), 1), "algorithmic_flops": flops, "algorithmic_bytes": byts,
            "mfma_roof_frac": round(flops / (ms * 1e-3) / (BF16_PEAK_TFLOPS * 1e12), 4)}


def measure_relay(wl, w_dev, torch, steps, warmup):
    """dflow_relay on the workload's shape: every request relays the reusable
    rejected suffix of a round that accepted tau_prev - 1 candidates (rows
    max(0, B-2-n)); inputs resident in HBM.  Timed per call with events, and
    per kernel kind with the library's event timing."""
    import block_diffusion_drafter_fuse_amd as dfa
    import synth
    d, bs, B = wl.dims, wl.bs, wl.dims.B
    n_acc = [int(t) - 1 for t in wl.n_new]
    k = [max(0, B - 2 - n) for n in n_acc]
    rows = sum(k)
    rw = {n: dfa.to_device(v) for n, v in synth.make_relay_weights(d, wl.seed).items()}
    dr = dfa.Drafter(d, w_dev, 64, bs, bs)
    parts = [synth.make_suffix_hidden(d, wl.seed, r, 0, k[r]) for r in range(bs)]
    hid = [dfa.to_device(np.ascontiguousarray(np.concatenate([p[l] for p in parts], 0))) for l in range(d.L)]
    rng = np.random.default_rng(wl.seed)
    cand = torch.tensor(rng.integers(0, d.V, size=(bs, B - 1)).astype(np.int32), device="cuda")
    bonus = torch.tensor(rng.integers(0, d.V, size=bs).astype(np.int32), device="cuda")
    slots = list(range(bs))

    def call():
        dr.relay(slots, n_acc, cand, 1, bonus, hid, rw["w1"], rw["w2"])

    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    dr.profile_enable(["fuse_gemm", "relay"], 16 * (steps + 1))
    for _ in range(steps):
        call()
    prof = dr.profile_read()
    dr.profile_enable([], 0)
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for _ in range(steps):
        call()
    stop.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / steps
    e = elt(d)
    byts = e * (d.D * d.L * d.Dt + 3 * d.D * d.D + 2 * d.D * d.D) + rows * (d.L * d.Dt * e + 2 * d.D * e + d.D * 4)
    flops = 2.0 * rows * (d.D * d.L * d.Dt + 3 * d.D * d.D + 2 * d.D * d.D)
    bd = {kk: round(v[0] / steps, 4) for kk, v in prof.items()}
    dr.close()
    del dr
    torch.cuda.synchronize()
    return {"workload": f"{wl.dims.name} relay, bs {bs}, {rows} suffix rows", "ms_per_call": round(ms, 4),
            "rows": rows, "algorithmic_bytes": byts, "algorithmic_flops": flops,
            "hbm_roof_frac": round(byts / (ms * 1e-3) / (HBM_PEAK_GBS * 1e9), 4),
            "mfma_roof_frac": round(flops / (ms * 1e-3) / (BF16_PEAK_TFLOPS * 1e12), 4),
            "breakdown_ms": bd,
            "note": "fuse_gemm = suffix projection through the shared W_c; relay = assembly + MLP GEMMs"}


def measure_select(wl, w_dev, torch, steps, warmup):
    """dflash2_select on the workload's batch: the gates come from one draft of
    the batch (context-free, so only the block feeds it); the top-16 candidate
    lists and logits are seeded synthetic inputs.  Timed per call with events."""
    import block_diffusion_drafter_fuse_amd as dfa
    import synth
    d, bs, B, K = wl.dims, wl.bs, wl.dims.B, 16
    tabs = {n: dfa.to_device(v) for n, v in synth.make_selector_weights(d, wl.seed).items()}
    dr = dfa.Drafter(d, w_dev, 64, bs, bs)
    slots = list(range(bs))
    anchor = torch.tensor(synth.make_anchors(d, wl.seed, bs), device="cuda")
    ids = torch.zeros((bs, B - 1, 1), dtype=torch.int32, device="cuda")
    dr.draft_block(slots, anchor, 1, ids)
    rng = np.random.default_rng(wl.seed)
    cand = torch.tensor(rng.integers(0, d.V, size=(bs, B - 1, K)).astype(np.int32), device="cuda")
    ul = torch.tensor(np.sort(rng.standard_normal((bs, B - 1, K)).astype(np.float32), -1)[..., ::-1].copy(),
                      device="cuda")
    path = torch.zeros((bs, B - 1), dtype=torch.int32, device="cuda")

    def call():
        dr.select(bs, anchor, cand, ul, K, tabs, path)

    for _ in range(warmup):
        call()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for _ in range(steps):
        call()
    stop.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / steps
    e = elt(d)
    R = 256
    rows = bs * (B - 1)
    byts = e * (R * d.D) + rows * d.D * e + rows * K * 8 + rows * (K + 1) * 2 * R * e
    dr.close()
    del dr
    torch.cuda.synchronize()
    return {"workload": f"{wl.dims.name} selector, bs {bs}, top-{K}, rank {R}", "ms_per_call": round(ms, 4),
            "algorithmic_bytes": byts, "hbm_roof_frac": round(byts / (ms * 1e-3) / (HBM_PEAK_GBS * 1e9), 4),
            "note": "gate GEMM over the draft's final hidden rows + pair tables + greedy walk; "
                    "the draft's top-16 LM head is not included"}


def measure_spec(wl, w_dev, torch, steps, warmup, temperature=1.0):
    """Speculative sampling at T > 0 on the workload's batch and vocabulary:
    dflash_spec_draft over the drafter's B-1 rows and dflash_spec_verify over
    those rows and the verifier's B rows per request.  The logit rows are
    seeded synthetic inputs (synth.make_sampling_logits), resident in HBM.  The
    draft call hands the drafter rows' log-sum-exps to the verify call, which
    then reads only the verifier rows in full.  The calls are timed with events
    over `steps` calls each, and each kernel kind with the library's events on
    a second pass."""
    import block_diffusion_drafter_fuse_amd as dfa
    import synth
    d, bs, B = wl.dims, wl.bs, wl.dims.B
    K, V = B - 1, d.V
    dl, tl = synth.make_sampling_logits(bs, B, V, wl.seed)
    dlg = torch.from_numpy(dl).cuda()
    tlg = torch.from_numpy(tl).cuda()
    del dl, tl
    dr = dfa.Drafter(d, w_dev, 64, bs, bs)
    req = torch.arange(bs, dtype=torch.int32, device="cuda")
    cand = torch.zeros((bs, K), dtype=torch.int32, device="cuda")
    dlse = torch.zeros((bs, K), dtype=torch.float32, device="cuda")
    tokens = torch.zeros((bs, B), dtype=torch.int32, device="cuda")
    tau = torch.zeros(bs, dtype=torch.int32, device="cuda")

    def draft(i):
        dr.spec_draft(bs, dlg, temperature, 1000 + i, req, cand, dlse)

    def verify(i):
        dr.spec_verify(bs, dlg, tlg, cand, temperature, 2000 + i, req, tokens, tau, dlse)

    def clock(fn):
        for i in range(warmup):
            fn(i)
        start = torch.cuda.Event(enable_timing=True)
        stop = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        start.record()
        for i in range(steps):
            fn(i)
        stop.record()
        torch.cuda.synchronize()
        return start.elapsed_time(stop) / steps

    draft(0)
    ms_draft = clock(draft)
    ms_verify = clock(verify)
    dr.profile_enable(["spec_draft", "spec_stats", "spec_resample"], 8 * (steps + 1))
    for i in range(steps):
        draft(i)
        verify(i)
    torch.cuda.synchronize()
    res = dr.profile_read()
    dr.profile_enable([], 0)
    taus = tau.cpu().numpy()
    rej = int((taus <= K).sum())
    row = V * 4
    byts = {"spec_draft": bs * K * row + bs * (K * 8 + 4),
            "spec_stats": bs * (K + 1) * row + bs * K * (4 + 4 + 8),
            "spec_resample": (bs + rej) * row + bs * (B * 4 + 4)}
    kernels = {}
    for k, b in byts.items():
        tot, cnt = res.get(k, (0.0, 0))
        us = tot / max(cnt, 1) * 1e3
        gbs = b / (us * 1e-6) / 1e9 if us > 0 else None
        kernels[k] = {"us_per_launch": round(us, 2), "algorithmic_bytes": b,
                      "achieved_GBs": None if gbs is None else round(gbs, 1),
                      "hbm_roof_frac": None if gbs is None else round(gbs / HBM_PEAK_GBS, 4)}
    dr.close()
    del dr, dlg, tlg
    torch.cuda.synchronize()
    return {"workload": f"{d.name} speculative sampling, bs {bs}, V {V}, B {B}, T {temperature}",
            "draft_ms_per_call": round(ms_draft, 4), "verify_ms_per_call": round(ms_verify, 4),
            "mean_tau": round(float(taus.mean()), 3), "kernels": kernels,
            "note": "fp32 logit rows resident in HBM; spec_draft times both drafting kernels (block masses, "
                    "block draw) and spec_resample both replacement kernels; bytes count each logit row read "
                    "once (draft: the drafter rows; stats: the verifier rows; resample: the verifier row, plus "
                    "the drafter row where a draft was rejected)"}


def _blas_info():
    """(vendor string, thread count) of the BLAS numpy calls."""
    try:
        from threadpoolctl import threadpool_info
        infos = [i for i in threadpool_info() if i.get("user_api") == "blas"] or threadpool_info()
        vendor = ",".join(sorted({f"{i.get('internal_api')} {i.get('version')}" for i in infos})) or "unknown"
        threads = max([i.get("num_threads", 1) for i in infos] or [1])
    except Exception:  # pragma: no cover
        vendor, threads = "unknown", os.cpu_count() or 1
    return vendor, int(threads)


def cpu_baseline(wl, w_np, n_sample=6):
    """The float64 oracle, as it stands, on a sample of the workload's
    requests.  The oracle drafts one request at a time, so a step of the whole
    batch costs the sum of its requests' costs: each sampled request (evenly
    spaced context quantiles) is timed once over fuse(its new rows) + draft +
    accept, and the batch step is estimated as bs / n_sample times their sum.
    One more request (the median context) is timed with BLAS limited to one
    thread.  Returns drafted tokens/s of the batch (blocks/s x B)."""
    import oracle
    import synth
    vendor, threads = _blas_info()
    d = wl.dims
    order = np.argsort(wl.ctx, kind="stable")
    k = min(n_sample, wl.bs)
    pick = sorted({int(order[int(round(i * (wl.bs - 1) / max(k - 1, 1)))]) for i in range(k)})
    w32 = synth.weights_as_f32(w_np)
    anchors = synth.make_anchors(d, wl.seed, wl.bs)

    def one(r):
        pre = wl.ctx[r] - wl.n_new[r]
        o = oracle.OracleDrafter(w32, d)
        if pre:
            o.fuse(r, synth.as_f32(synth.make_hidden(d, wl.seed, r, 0, pre)))
        new = synth.as_f32(synth.make_hidden(d, wl.seed, r, pre, wl.n_new[r]))
        t0 = time.perf_counter()
        o.fuse(r, new)
        res = o.draft(r, int(anchors[r]))
        cand, _ = oracle.topk(res["logits"], 1)
        oracle.accept(cand[:, 0], np.zeros(d.B, np.int64))
        return time.perf_counter() - t0

    per = {r: one(r) for r in pick}
    step_s = sum(per.values()) * wl.bs / len(pick)
    single = None
    try:
        from threadpoolctl import threadpool_limits
        r1 = int(order[len(order) // 2])
        with threadpool_limits(limits=1, user_api="blas"):
            t1 = one(r1)
        single = {"value": round(d.B / t1, 3), "unit": "drafted tokens/s (one request stream)", "threads": 1,
                  "sample": f"request with ctx {wl.ctx[r1]}, {t1:.2f} s"}
    except Exception as e:  # pragma: no cover
        single = {"error": str(e)}
    return {"value": round(wl.bs * d.B / step_s, 3), "unit": "drafted tokens/s", "cores": threads,
            "kind": "oracle", "host_cpus": os.cpu_count(), "blas": vendor, "blas_threads": threads,
            "sample": f"{len(pick)} of the {wl.bs} requests (contexts {[wl.ctx[r] for r in pick]}), each timed "
                      f"once over fuse + draft + accept in float64 ({', '.join(f'{per[r]:.2f}' for r in pick)} s); "
                      f"batch step = {wl.bs}/{len(pick)} x their sum = {step_s:.1f} s",
            "single_thread": single}


def achievable_peaks(torch, reps=10):
    """Measured ceilings beside the nominal peaks: HBM read+write rate of a
    plain device-to-device copy of 1 GiB (torch's copy kernel), HBM read rate of
    a reduction over 1 GiB (torch's sum), and the bf16 rate of one large square
    GEMM (torch.mm, i.e. the vendor library, 8192^3).  Context for the roofline
    fractions, which stay against the nominal peaks."""
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    src.fill_(1)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for _ in range(2):
        dst.copy_(src)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    copy_gbs = 2.0 * n * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del dst
    x = src.view(torch.float32)  # 1 GiB read by a reduction (the read-only ceiling)
    for _ in range(2):
        x.sum()
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        x.sum()
    e1.record()
    torch.cuda.synchronize()
    read_gbs = 1.0 * n * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del src, x
    m = 8192
    a = torch.randn(m, m, device="cuda").to(torch.bfloat16)
    b = torch.randn(m, m, device="cuda").to(torch.bfloat16)
    for _ in range(2):
        torch.mm(a, b)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        torch.mm(a, b)
    e1.record()
    torch.cuda.synchronize()
    tflops = 2.0 * m ** 3 * reps / (e0.elapsed_time(e1) * 1e-3) / 1e12
    del a, b
    torch.cuda.synchronize()
    return {"hbm_copy_GBs": round(copy_gbs, 1), "hbm_copy_frac_of_peak": round(copy_gbs / HBM_PEAK_GBS, 4),
            "hbm_read_GBs": round(read_gbs, 1), "hbm_read_frac_of_peak": round(read_gbs / HBM_PEAK_GBS, 4),
            "bf16_gemm_8192_TFLOPs": round(tflops, 1),
            "bf16_gemm_frac_of_peak": round(tflops / BF16_PEAK_TFLOPS, 4)}


def blas_reference(wl, torch, reps=20):
    """The vendor library's bf16 GEMM (torch.nn.functional.linear, which calls
    hipBLASLt) on the projection shapes of the workload's draft step, with
    weights cycled through enough copies (>= 600 MB) that each call reads its
    weight from HBM as the step does.  Context for the MFMA fraction of the
    library's own GEMM kernels; no part of the draft step."""
    d = wl.dims
    M, Mlm = wl.bs * d.B, wl.bs * (d.B - 1)
    qkv = (d.Hq + 2 * d.Hkv) * d.hd
    shapes = {"qkv_gemm": (M, qkv, d.D), "o_gemm": (M, d.D, d.Hq * d.hd), "gateup_gemm": (M, 2 * d.I, d.D),
              "down_gemm": (M, d.D, d.I), "lm_head": (Mlm, d.V, d.D)}
    out = {}
    for kind, (m, n, k) in shapes.items():
        a = torch.randn(m, k, device="cuda").to(torch.bfloat16)
        w = (torch.randn(n, k, device="cuda") * 0.02).to(torch.bfloat16)
        ws = [w] + [w.clone() for _ in range(max(0, -(-600_000_000 // (n * k * 2)) - 1))]
        for i in range(3):
            torch.nn.functional.linear(a, ws[i % len(ws)])
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(reps):
            torch.nn.functional.linear(a, ws[i % len(ws)])
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) / reps * 1000
        tf = 2.0 * m * n * k / us / 1e6
        out[kind] = {"shape_mnk": [m, n, k], "us_per_call": round(us, 1), "tflops": round(tf, 1),
                     "mfma_roof_frac": round(tf / BF16_PEAK_TFLOPS, 4)}
        del ws, w, a
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="qwen3_8b_bs32")
    ap.add_argument("--companion", default="qwen3_8b_bs1", help="second workload reported under 'bs1' ('' for none)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="the draft-step workloads only (implies --no-4b and --no-relay, skips prefill): "
                         "for kernel traces and counter runs of the step")
    ap.add_argument("--no-4b", action="store_true",
                    help="skip the Qwen3-4B-shaped bs1 step and its 2048-token prefill")
    ap.add_argument("--no-relay", action="store_true",
                    help="skip the DFlow relay, DFlash 2 selector and convolution, and speculative sampling "
                         "measurements")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="after timing, copy one buffer of this many MiB (reference dispatch for byte counters)")
    ap.add_argument("--blas-reference", action="store_true",
                    help="also time torch's bf16 linear (hipBLASLt) on the step's projection shapes, cold weights")
    ap.add_argument("--counter-summary", nargs="+", metavar="CSV",
                    help="print per-kind medians of the counters in rocprofv3 counter_collection.csv files "
                         "(and the derived MFMA utilisation); needs no GPU")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write profiles/traffic.json from two rocprofv3 --pmc counter_collection.csv files "
                         "(FETCH_SIZE, WRITE_SIZE) of a run with --copy-probe-mib; needs no GPU")
    args = ap.parse_args()
    if args.no_extras:
        args.no_4b = args.no_relay = True
    if args.counter_summary:
        print(json.dumps(counter_summary(args.counter_summary), indent=1, sort_keys=True))
        return
    if args.traffic_from:
        if not args.copy_probe_mib:
            ap.error("--traffic-from needs the --copy-probe-mib of the profiled run")
        t = traffic_summary(args.traffic_from[0], args.traffic_from[1], args.copy_probe_mib, args.workload)
        p = os.path.join(ROOT, "profiles", "traffic.json")
        old = {}
        if os.path.exists(p):
            try:
                old = json.load(open(p))
            except ValueError:
                old = {}
        kernels = old.get("kernels", {}) if old.get("source_sha") == source_sha() else {}
        kernels.update(t["kernels"])
        doc = {"source_sha": source_sha(), "copy_probe_mib": args.copy_probe_mib,
               "factors": {**old.get("factors", {}),
                           args.workload: {"fetch": t["fetch_factor"], "write": t["write_factor"]}},
               "kernels": kernels}
        os.makedirs(os.path.dirname(p), exist_ok=True)
        with open(p, "w") as fh:
            json.dump(doc, fh, indent=1, sort_keys=True)
        print(json.dumps(doc["kernels"], indent=1))
        return
    if args.gpus != 1:
        print(f"bench.py: the library runs on one GPU per process; --gpus {args.gpus} is not supported "
              "(the draft step would shard by request across GPUs with no exchange)",
              file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    import block_diffusion_drafter_fuse_amd as dfa
    import synth

    wl = synth.get_config(args.workload)
    print(f"[bench] generating weights for {wl.dims.name}", file=sys.stderr, flush=True)
    w_np = synth.make_weights(wl.dims, wl.seed)
    w_dev = dfa.Drafter.upload_weights(w_np)
    print(f"[bench] measuring {args.workload}", file=sys.stderr, flush=True)
    main_res = measure(wl, w_dev, torch, args.steps, args.warmup, args.workload, conv=not args.no_relay)
    comp = None
    if args.companion:
        wc = synth.get_config(args.companion)
        assert wc.dims == wl.dims, "companion must share the model shape"
        print(f"[bench] measuring {args.companion}", file=sys.stderr, flush=True)
        comp = measure(wc, w_dev, torch, args.steps, args.warmup, args.companion)
    prefill = [] if args.no_extras else [measure_prefill(wl.dims, w_dev, torch, 8192, wl.seed)]
    bs1_4b = None
    if not args.no_4b:
        w4 = synth.get_config("qwen3_4b_bs1")
        print("[bench] measuring qwen3_4b_bs1", file=sys.stderr, flush=True)
        w4_dev = dfa.Drafter.upload_weights(synth.make_weights(w4.dims, w4.seed))
        r4 = measure(w4, w4_dev, torch, args.steps, args.warmup, "qwen3_4b_bs1")
        bs1_4b = {k: r4[k] for k in ("workload", "drafted_tokens_per_s", "blocks_per_s", "ms_per_step",
                                     "step_ms_p10_p50_p90", "step_hbm_roof_frac", "roofline", "breakdown_ms")}
        prefill.insert(0, measure_prefill(w4.dims, w4_dev, torch, 2048, w4.seed))
        del w4_dev
        torch.cuda.synchronize()
    relay = select = spec = shard = None
    if not args.no_extras:
        print(f"[bench] measuring the LM head on one of 8 vocabulary shards", file=sys.stderr, flush=True)
        shard = measure_lm_shard([wl] + ([synth.get_config(args.companion)] if args.companion else []), w_dev,
                                 torch, args.steps, args.warmup)
    if not args.no_relay:
        print(f"[bench] measuring the DFlow relay at {args.workload}", file=sys.stderr, flush=True)
        relay = measure_relay(wl, w_dev, torch, args.steps, args.warmup)
        print(f"[bench] measuring the DFlash 2 selector at {args.workload}", file=sys.stderr, flush=True)
        select = measure_select(wl, w_dev, torch, args.steps, args.warmup)
        print(f"[bench] measuring speculative sampling at {args.workload}", file=sys.stderr, flush=True)
        spec = measure_spec(wl, w_dev, torch, args.steps, args.warmup)
    if args.copy_probe_mib:
        n = args.copy_probe_mib << 20
        src = torch.full((n,), 7, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        torch.bitwise_not(src, out=dst)  # one elementwise kernel: n bytes in, n bytes out
        torch.cuda.synchronize()
        del src, dst
    blas = blas_reference(wl, torch) if args.blas_reference else None
    peaks = None if args.no_extras else achievable_peaks(torch)
    cpu = None
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle", file=sys.stderr, flush=True)
        cpu = cpu_baseline(wl, w_np)
    d = wl.dims
    line = {
        "metric": "drafted tokens/s (blocks/s x B) at Qwen3-8B shape",
        "value": main_res["drafted_tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": main_res["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": d.dtype,
        "data": "synthetic (seeded random-init weights and verifier features)",
        "config": {"workload": args.workload, "batch": wl.bs, "block": d.B, "hidden": d.D,
                   "draft_layers": d.N, "vocab": d.V, "ctx_sum": sum(wl.ctx), "new_rows": sum(wl.n_new),
                   "top_k": 1},
        "blocks_per_s": main_res["blocks_per_s"],
        "roofline": main_res["roofline"],
        "roofline_next": main_res.get("roofline_next"),
        "step_hbm_roof_frac": main_res["step_hbm_roof_frac"],
        "step_mfma_roof_frac": main_res["step_mfma_roof_frac"],
        "step_ms_p10_p50_p90": main_res["step_ms_p10_p50_p90"],
        "breakdown_ms": main_res["breakdown_ms"],
        "cpu_baseline": cpu,
    }
    if comp:
        line["bs1"] = {k: comp[k] for k in ("workload", "drafted_tokens_per_s", "blocks_per_s", "ms_per_step",
                                            "step_ms_p10_p50_p90", "step_hbm_roof_frac", "roofline", "breakdown_ms")}
    if bs1_4b:
        line["bs1_4b"] = bs1_4b
    if prefill:
        line["prefill"] = prefill
    if relay:
        line["relay"] = relay
    if "conv" in main_res:
        line["conv"] = main_res["conv"]
    if select:
        line["select"] = select
    if spec:
        line["spec_sampling"] = spec
    if blas:
        line["blas_reference"] = blas
    if shard:
        line["lm_head_vocab_shard"] = shard
    if peaks:
        line["achievable_peaks"] = peaks
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
