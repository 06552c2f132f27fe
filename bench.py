#!/usr/bin/env python3
"""Throughput of the TokenMixer-Large block-stack forward on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload N] [--no-cpu-baseline]
    python bench.py --workload 2                   # the dense per-token SwiGLU stack
    python bench.py --workload rankmixer_d256      # the RankMixer block stack

The default workload is the large MoE stack (B 8192, T = H = 32, D 768, E 32,
top-4, 8 blocks, ~15.4e9 weights), the largest configuration that fits one
GPU. A step is one tmx_block_stack_forward over one batch of the workload
(all blocks, both sub-layers, inter-residuals) with inputs and weights
already resident in HBM. Prints ONE JSON line.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "block-stack forward samples/s + TFLOP/s (% bf16 MFMA peak), 1×MI355X"
BF16_PEAK_TFLOPS = 2516.6     # 256 CU x 2.4 GHz x 4096 dense bf16 FLOP/clk/CU
FP8_PEAK_TFLOPS = 5033.2      # dense fp8 MFMA: twice the bf16 rate
HBM_PEAK_GBS = 8000.0


# rocprofv3 counter summaries of the dominant kernels; a traffic figure is used
# only while the kernel's sources still hash to the value recorded there
COUNTERS_FILE = os.path.join(ROOT, "profiles", "mlp_dense_workload2_counters.md")
KERNEL_SOURCES = ("token_moe_amd/csrc/tmx_mlp.hip", "token_moe_amd/csrc/tmx_device.h", "token_moe_amd/build.py",
                  "token_moe_amd/csrc/tmx_internal.h")
ROUTED_WIDE_SOURCES = ("token_moe_amd/csrc/tmx_routed.hip", "token_moe_amd/csrc/tmx_device.h", "token_moe_amd/build.py",
                       "token_moe_amd/csrc/tmx_internal.h")
RMX_COUNTERS_FILE = os.path.join(ROOT, "profiles", "rmx_block_{workload}_counters.md")
RMX_KERNEL_SOURCES = ("token_moe_amd/csrc/tmx_rankmixer.hip", "token_moe_amd/csrc/tmx_device.h",
                      "token_moe_amd/build.py", "token_moe_amd/csrc/tmx_internal.h")


def kernel_source_hash(sources=KERNEL_SOURCES):
    import hashlib
    h = hashlib.sha256()
    for rel in sources:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(workload, counters_file=COUNTERS_FILE, sources=KERNEL_SOURCES):
    """HBM bytes per launch of the dominant kernel from the committed counter
    summary (FETCH_SIZE and WRITE_SIZE, each scaled by a plain copy's reading),
    or None when it was taken on other kernel sources or another workload."""
    try:
        with open(counters_file) as f:
            text = f.read()
    except OSError:
        return None
    vals = {}
    for line in text.splitlines():
        line = line.strip().strip("`")
        if ":" in line and line.split(":", 1)[0] in ("kernel_source_sha256", "workload",
                                                      "traffic_bytes_per_launch"):
            k, v = line.split(":", 1)
            vals[k] = v.strip()
    if vals.get("kernel_source_sha256") != kernel_source_hash(sources) or vals.get("workload") != workload:
        return None
    try:
        return int(vals["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def time_launches(fn, reps, stream):
    """Average duration (ms) of `fn()` launches with HIP events on `stream`."""
    import torch
    fn()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for _ in range(reps):
        fn()
    end.record(stream)
    end.synchronize()
    return start.elapsed_time(end) / reps


def cpu_cores():
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def cpu_baseline(wl, banks, x, budget_s):
    """The oracle as it stands, on a bounded sample of the same workload.

    The oracle's cost is affine in the sample count (a fixed per-call part
    for the weight slices plus a per-sample part), so two probe runs fix both
    and the sample is sized to fill about `budget_s` seconds. MoE stacks run
    the first block only (its weight slices alone take seconds to decode per
    block) and the rate is scaled to the L-block stack."""
    import datagen as dg
    import oracle as orc
    ws = dg.WeightSource(wl, banks)

    one_block = wl.moe and not wl.rankmixer
    if wl.rankmixer:
        forward = orc.rankmixer_stack
    elif one_block:
        def forward(xx, w, s):
            return orc.block_forward(xx, w, 1, s, None, w.bf16_values)
    else:
        forward = orc.stack_forward

    def run(n):
        t0 = time.perf_counter()
        forward(x[:n].astype(np.float64), wl, ws)
        return time.perf_counter() - t0

    if not one_block:
        run(2)                                 # first-touch costs out of the probes
    # grow the probe until it takes a quarter of the budget, then extrapolate
    # from the last two probes (per-sample cost rises with n: cache effects;
    # for MoE stacks every run also decodes the block's weight slices, a
    # fixed part that the difference of two probes leaves out)
    n_prev, t_prev = 8, run(8)
    n_cur, t_cur = n_prev, t_prev
    while t_cur < budget_s / 4 and n_cur < wl.B:
        n_prev, t_prev = n_cur, t_cur
        n_cur = min(wl.B, n_cur * 4)
        t_cur = run(n_cur)
    # with a single probe (the first already took a quarter of the budget)
    # its whole time counts as per-sample cost, which can only shrink the sample
    per = (t_cur - t_prev) / (n_cur - n_prev) if n_cur > n_prev else t_cur / n_cur
    per = max(per, t_cur / (4.0 * n_cur), 1e-6)
    n = int(min(wl.B, max(n_cur, n_cur + (budget_s - t_cur) / per)))
    dt = run(n)
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = 1
    if one_block:
        what = (f"first {n} of {wl.B} samples of the same workload through block 1 of {wl.L} in fp64 numpy "
                f"({dt:.1f} s), rate divided by {wl.L} for the stack")
        value = n / (dt * wl.L)
    else:
        what = (f"first {n} of {wl.B} samples of the same workload, full {wl.L}-block stack "
                f"in fp64 numpy ({dt:.1f} s)")
        value = n / dt
    return {"value": value, "unit": "samples/s", "cores": cpu_cores(), "blas_threads": int(threads),
            "kind": "oracle", "sample": what}


def routed_is_wide(wl):
    """Whether the library runs this workload's routed experts in a 128-row
    wide kernel (W 768, h_e 384: bf16 or MXFP8; W 512, h_e 256: bf16)
    rather than the fused MLP kernel."""
    if wl.dtype == "bf16" and wl.width(1) == 512 and wl.expert_hidden == 256:
        return True
    return wl.dtype in ("bf16", "mxfp8") and wl.width(1) == 768 and wl.expert_hidden == 384


def routed_kernel_name(wl):
    if routed_is_wide(wl):
        if wl.dtype == "mxfp8":
            return "routed_mx_kernel<768, 384> (128-row tiles, MXFP8)"
        return f"routed_kernel<{wl.width(1)}, {wl.expert_hidden}> (128-row tiles)"
    return f"mlp_kernel<{wl.width(1)}, ROUTED{', MXFP8' if wl.dtype == 'mxfp8' else ''}>"


def moe_kernel_work(wl):
    """Algorithmic work per launch of each MoE kernel, as (bound, amount):
    FLOPs for the GEMM kernels (2 per multiply-add; the top_k chosen experts
    of every row for the routed launch, the shared expert for the other), HBM
    bytes for the router (rows read, normalised rows written -- bf16, or for
    MXFP8 one code byte per element and one exponent byte per 32 -- routing
    table written, router weights read) and the bucket kernel (routing table
    read, row lists written). P * W = T * D in both sub-layers; P averages H
    and T."""
    TD = wl.T * wl.D
    P = (wl.H + wl.T) / 2.0
    xhat_bytes = TD * (33.0 / 32.0) if wl.dtype == "mxfp8" else TD * 2.0
    return {
        "mlp_routed": ("mfma", 2.0 * wl.B * wl.top_k * TD * 3 * wl.expert_hidden),
        "mlp_shared": ("mfma", 2.0 * wl.B * TD * 3 * wl.shared_hidden),
        "router": ("hbm", wl.B * (TD * 2.0 + xhat_bytes) + wl.B * P * wl.top_k * 8 + TD * wl.E * 2),
        "bucket": ("hbm", wl.B * P * wl.top_k * 8.0),
    }


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="5",
                    help="workload id 1..5 (default 5, the large MoE stack) or a RankMixer workload "
                         "(rankmixer_d256, rankmixer_d512, rankmixer_moe_d256)")
    ap.add_argument("--kernel-reps", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--dtype", choices=("bf16", "mxfp8"), default="bf16",
                    help="mxfp8: the workload with MXFP8 GEMM operands (bf16 activations; dense sub-layers "
                         "of width 256 or 512, MoE sub-layers of width 512 or 768: workloads 2, 3, 4, 5)")
    args = ap.parse_args(argv)

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the block stack runs on a single MI355X "
              "(across GPUs, samples would shard with the weights replicated).",
              file=sys.stderr)
        return 2

    import torch
    import datagen as dg
    from token_moe_amd import runner, tmx
    import oracle as orc

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    tmx.load_library()
    if args.workload in dg.RANKMIXER_WORKLOADS:
        wl = dg.RANKMIXER_WORKLOADS[args.workload]
    elif args.workload.isdigit() and int(args.workload) in dg.WORKLOADS:
        wl = dg.WORKLOADS[int(args.workload)]
    else:
        print(f"unknown workload {args.workload!r}", file=sys.stderr)
        return 2
    if args.dtype == "mxfp8":
        widths = {wl.width(0), wl.width(1)}
        ok = (wl.dtype == "bf16" and not wl.rankmixer and
              (widths <= {256, 512} if not wl.moe else widths <= {512, 768}))
        if not ok:
            print("--dtype mxfp8 applies to the bf16 workloads whose sub-layer widths are 256 or 512 "
                  "(dense) or 512 or 768 (MoE): workloads 2, 3, 4, 5", file=sys.stderr)
            return 2
        wl = wl.with_(dtype="mxfp8")
    log("workload", wl)
    t0 = time.perf_counter()
    banks = dg.weight_banks(wl)
    x = dg.make_x(wl)
    log(f"generated inputs in {time.perf_counter() - t0:.1f} s")
    ctx = runner.make_context(wl, banks)
    xd = runner.host_tensor(wl, x).cuda()
    yd = torch.empty_like(xd)
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream
    log("weights resident; warming up")

    for _ in range(args.warmup):
        ctx.block_stack_forward(xd, yd, wl.B, sp)
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(args.steps):
        ctx.block_stack_forward(xd, yd, wl.B, sp)
    end.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / args.steps
    flops = (orc.rankmixer_flops_per_sample(wl) if wl.rankmixer else orc.flops_per_sample(wl)) * wl.B
    samples_s = wl.B / (ms / 1e3)
    tflops = flops / (ms / 1e3) / 1e12
    log(f"{ms:.3f} ms/step, {samples_s:.0f} samples/s, {tflops:.1f} TFLOP/s")
    if not np.all(np.isfinite(yd[:64].float().cpu().numpy())):
        raise RuntimeError("non-finite output")

    # dominant kernel: the fused per-position SwiGLU MLP. For a dense workload
    # one sub-layer call is exactly one launch of it.
    roofline = None
    kernel = {}
    if wl.rankmixer:
        # the stack is L launches of the fused block kernel and nothing else,
        # so one launch takes the stack's event-timed time / L
        kms = time_launches(lambda: ctx.block_stack_forward(xd, yd, wl.B, sp), args.kernel_reps, stream) / wl.L
        kfl = float(orc.rankmixer_flops_per_sample(wl) // wl.L * wl.B)
        if wl.moe:
            # ReLU-routed experts: only the experts a row activates are the
            # method's work. The share of positive gates is measured on the
            # first block's router (outside the timed region, torch matmuls
            # in fp32 on the library's own S); the kernel itself evaluates
            # every expert that some row of its 64-row tile activates.
            s_dev = torch.empty_like(xd)
            ctx.sublayer_forward(0, 0, xd, None, None, s_dev, wl.B, sp)
            wr = runner.host_tensor(wl, banks[(1, 1, dg.K_ROUTER)]).cuda().float()       # [T, D, E]
            logits = torch.bmm(s_dev.float().transpose(0, 1).contiguous(), wr)          # [T, B, E]
            active = float((logits > 0).float().mean().item())
            per_row_expert = 2.0 * 2 * wl.D * wl.expert_hidden
            executed = kfl
            kfl = wl.B * wl.T * (2.0 * wl.D * wl.E + active * wl.E * per_row_expert)
            kernel["active_expert_frac"] = round(active, 4)
            kernel["executed_flop_per_launch"] = executed
            flops = kfl * wl.L
            tflops = flops / (ms / 1e3) / 1e12
        achieved = kfl / (kms / 1e3) / 1e12
        roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": BF16_PEAK_TFLOPS,
                    "unit": "TFLOP/s", "frac": round(achieved / BF16_PEAK_TFLOPS, 4),
                    "traffic": measured_traffic(wl.name, RMX_COUNTERS_FILE.format(workload=wl.name),
                                                RMX_KERNEL_SOURCES),
                    "kernel": f"rmx_block_kernel<{wl.D}, fused{f', {wl.E} experts' if wl.moe else ''}>",
                    "flop_per_launch": kfl,
                    "launch_ms": round(kms, 5)}
        kernel["rmx_block_ms"] = round(kms, 5)
        log(f"fused RankMixer block kernel: {kms:.4f} ms/launch, {achieved:.1f} TFLOP/s")
    elif wl.moe:
        # An MoE sub-layer runs four kernels. Their own durations come from
        # HIP events the library records around each launch on the launch
        # stream (tmx_set_kernel_timing), over as many steps as the timed
        # region, run right after it.
        ctx.set_kernel_timing(True)
        for _ in range(args.steps):
            ctx.block_stack_forward(xd, yd, wl.B, sp)
        torch.cuda.synchronize()
        times = ctx.kernel_times()
        ctx.set_kernel_timing(False)
        kinfo = moe_kernel_work(wl)
        mfma_peak = FP8_PEAK_TFLOPS if wl.dtype == "mxfp8" else BF16_PEAK_TFLOPS
        kernels = {}
        for name, (tot, n) in times.items():
            kms = tot / n
            rec = {"launches_per_step": n / args.steps, "ms": round(kms, 5)}
            work = kinfo.get(name)
            if work is not None:
                bound, amount = work
                if bound == "mfma":
                    rec.update(bound="mfma", flop_per_launch=amount,
                               achieved_tflops=round(amount / (kms / 1e3) / 1e12, 2),
                               frac=round(amount / (kms / 1e3) / 1e12 / mfma_peak, 4))
                else:
                    rec.update(bound="hbm", bytes_per_launch=amount,
                               achieved_gbs=round(amount / (kms / 1e3) / 1e9, 1),
                               frac=round(amount / (kms / 1e3) / 1e9 / HBM_PEAK_GBS, 4))
            kernels[name] = rec
        step_sum = sum(t for t, _ in times.values()) / args.steps
        log(f"kernel times sum to {step_sum:.3f} ms/step (timed step {ms:.3f} ms)")
        for name, rec in kernels.items():
            log(f"  {name}: {rec}")
        dom = max(times, key=lambda k: times[k][0])
        d = kernels[dom]
        roofline = {"bound": d["bound"], "achieved": d.get("achieved_tflops", d.get("achieved_gbs")),
                    "peak": mfma_peak if d["bound"] == "mfma" else HBM_PEAK_GBS,
                    "unit": "TFLOP/s" if d["bound"] == "mfma" else "GB/s", "frac": d["frac"],
                    "traffic": measured_traffic(wl.name, os.path.join(ROOT, "profiles", f"{dom}_{wl.name}_counters.md"),
                                                ROUTED_WIDE_SOURCES if dom == "mlp_routed" and routed_is_wide(wl)
                                                else KERNEL_SOURCES) if wl.dtype == "bf16" else None,
                    "kernel": {"mlp_routed": routed_kernel_name(wl),
                               "mlp_shared": f"mlp_kernel<{wl.width(1)}, SHARED"
                                             f"{', MXFP8' if wl.dtype == 'mxfp8' else ''}>"}.get(dom, dom),
                    "flop_per_launch": d.get("flop_per_launch"), "launch_ms": d["ms"]}
        kernel["kernels"] = kernels
        kernel["kernel_ms_sum_per_step"] = round(step_sum, 4)
    elif not wl.moe:
        xr = torch.empty_like(xd)
        per = []
        for sub in (0, 1):
            P, W, h = wl.positions(sub), wl.width(sub), wl.hidden(sub)
            if sub == 0:
                fn = lambda: ctx.sublayer_forward(0, 0, xd, None, None, xr, wl.B, sp)
            else:
                fn = lambda: ctx.sublayer_forward(0, 1, xr, xd, None, yd, wl.B, sp)
            kms = time_launches(fn, args.kernel_reps, stream)
            kfl = 2.0 * wl.B * P * 3 * W * h
            per.append((kms, kfl))
            kernel[f"mlp_{'mix' if sub == 0 else 'revert'}_ms"] = round(kms, 5)
        kms = sum(p[0] for p in per) / len(per)
        kfl = sum(p[1] for p in per) / len(per)
        achieved = kfl / (kms / 1e3) / 1e12
        peak = FP8_PEAK_TFLOPS if wl.dtype == "mxfp8" else BF16_PEAK_TFLOPS
        roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak,
                    "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                    "traffic": measured_traffic(wl.name) if wl.dtype == "bf16" else None,
                    "kernel": " / ".join(dict.fromkeys(
                        f"mlp_kernel<{wl.width(sub)}, DENSE{', MXFP8' if wl.dtype == 'mxfp8' else ''}>"
                        for sub in (0, 1))) + " (mean of the Mix and Revert launches)",
                    "flop_per_launch": kfl, "launch_ms": round(kms, 5)}
        log(f"fused MLP kernel: {kms:.4f} ms/launch, {achieved:.1f} TFLOP/s")

    out = {
        "metric": METRIC, "value": round(samples_s, 1), "unit": "samples/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": {"bf16": "bf16", "mxfp8": "mxfp8"}.get(wl.dtype, "f32"), "data": "synthetic",
        "tflops": round(tflops, 2),
        "mfma_frac": round(tflops / (FP8_PEAK_TFLOPS if wl.dtype == "mxfp8" else BF16_PEAK_TFLOPS), 4),
        "config": {"workload": wl.name, "block": wl.block, "B": wl.B, "T": wl.T, "H": wl.H, "D": wl.D, "L": wl.L,
                   "hidden": [wl.hidden_mix, wl.hidden_rev], "E": wl.E, "top_k": wl.top_k,
                   "expert_hidden": wl.expert_hidden, "shared_hidden": wl.shared_hidden,
                   "flop_per_step": flops},
        "roofline": roofline,
    }
    out.update(kernel)
    if not args.no_cpu_baseline:
        log("timing the oracle on the host")
        out["cpu_baseline"] = cpu_baseline(wl, banks, x, args.cpu_seconds)
    # a plain copy of known size outside the timed region, the calibration
    # kernel for rocprofv3 FETCH_SIZE / WRITE_SIZE: 512 MiB read + 512 MiB
    # written, the source first pushed out of L2 by an unrelated 256 MiB fill
    calib_src = torch.full((128 << 20,), 1.0, dtype=torch.float32, device="cuda")
    calib_flush = torch.zeros((64 << 20,), dtype=torch.float32, device="cuda")
    calib_dst = torch.empty_like(calib_src)
    torch.cuda.synchronize()
    calib_dst.copy_(calib_src)
    torch.cuda.synchronize()
    del calib_src, calib_flush, calib_dst
    ctx.close()
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
