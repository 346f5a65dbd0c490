"""Benchmark of the fused exact-attention forward on one MI355X.

One step = one attention forward (one kernel launch) over the whole batch of
the workload, inputs already resident in HBM.  Prints ONE JSON line:
  value   : algorithmic TFLOP/s (4*d FLOP per visible (query, key) pair) over
            exactly --steps launches (default: at least 100, and at least 0.2 s of
            launches), timed between device synchronisations;
  roofline: the kernel's average launch duration from HIP events recorded on
            the stream it is launched on, against MI355X dense MFMA peak
            (bf16/fp16 2.5 PFLOP/s, fp8 5.0 PFLOP/s); `traffic` is the HBM
            bytes per launch from rocprofv3 FETCH_SIZE/WRITE_SIZE counters
            (profiles/*_pmc.txt) scaled by a copy-kernel calibration, reported
            only while the kernel source is unchanged since the counters were
            taken;
  cpu_baseline: the fp64 CPU oracle timed on this host's cores on a bounded
            sample of the same workload (whole heads), in the same unit.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

DEFAULT_WORKLOAD = "bf16_b2_h16_s4096_d128"
# Under back-to-back launches MI355X raises its engine clock over the first 30-50 ms (measured on
# the default workload: 299 us per launch over the first 20 launches, 265 us around launch 50,
# 255 us from launch 120 on).  Before the warmup steps, the same launch runs for CLOCK_SETTLE_S so
# that the timed steps see the clock a sustained workload runs at; the line reports it.
CLOCK_SETTLE_S = 0.25
MIN_STEPS = 100        # timed steps at least, by default
MIN_TIMED_S = 0.2      # and at least this much timed launch time, by default
WARMUP_SECONDS = 0.25
PEAK_TFLOPS = {"bf16": 2500.0, "f16": 2500.0, "fp8": 5000.0, "e5m2": 5000.0}
KERNEL_SRC = os.path.join(ROOT, "exact_attention_32_amd", "csrc", "attn_fwd.hip")
PROFILES = os.path.join(ROOT, "profiles")


def kernel_sha() -> str:
    """Hash of the kernel source's code: line comments, trailing spaces and blank lines removed, so
    that an edit of comments alone does not invalidate counters taken on the same compiled code."""
    code = []
    with open(KERNEL_SRC, encoding="utf-8") as f:
        for line in f:
            line = line.split("//", 1)[0].rstrip()
            if line:
                code.append(line)
    return hashlib.sha256("\n".join(code).encode()).hexdigest()[:16]


def counter_traffic(kernel: str, workload: str):
    """HBM bytes per launch from the committed PMC summary of this kernel and workload, if taken on
    this kernel source."""
    path = os.path.join(PROFILES, f"{kernel}_{workload}_pmc.txt")
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                fields[k.strip()] = v.strip()
    if fields.get("kernel_source_sha256_16") != kernel_sha():
        return None
    try:
        return int(float(fields["traffic_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


def settle_clock(step, seconds: float) -> int:
    """Back-to-back launches of the step for `seconds` (the engine clock's ramp); returns the count."""
    import torch

    n, t0 = 0, time.perf_counter()
    while seconds > 0:
        for _ in range(10):
            step()
        n += 10
        torch.cuda.synchronize()
        if time.perf_counter() - t0 >= seconds:
            break
    return n


def warm_up(step, warmup: int) -> int:
    """Run the untimed warmup steps and return how many ran: exactly `warmup`, or for warmup < 0
    (the default) batches of 10 until WARMUP_SECONDS have passed."""
    import torch

    if warmup >= 0:
        for _ in range(warmup):
            step()
        torch.cuda.synchronize()
        return warmup
    n, t0 = 0, time.perf_counter()
    while True:
        for _ in range(10):
            step()
        n += 10
        torch.cuda.synchronize()
        if time.perf_counter() - t0 >= WARMUP_SECONDS:
            return n


def run_gpu(work, x, steps, warmup: int, settle_s: float):
    """Settle the clock, warm up, then time `steps` launches (None: at least MIN_STEPS and enough for
    MIN_TIMED_S of launches, from the duration of 20 untimed ones), each between HIP events on the
    launch stream."""
    import torch

    import exact_attention_32_amd as ea
    from exact_attention_32_amd import inputs as I

    dev = torch.device("cuda:0")
    q, k, v = x.q.to(dev), x.k.to(dev), x.v.to(dev)
    o = torch.empty((work.B, work.H, work.S_q, work.d), device=dev,
                    dtype=torch.float16 if work.dtype == "f16" else torch.bfloat16)
    lse = torch.empty((work.B, work.H, work.S_q), device=dev, dtype=torch.float32)
    if I.is_fp8(work.dtype):
        qd, kd, vd = x.q_descale.to(dev), x.k_descale.to(dev), x.v_descale.to(dev)
        fmt = "e5m2" if work.dtype == "e5m2" else "e4m3"

        def step():
            ea.fwd_fp8(q, k, v, qd, kd, vd, causal=work.causal, scale=work.scale, out=o, lse=lse, fmt=fmt)
    else:
        def step():
            ea.fwd(q, k, v, causal=work.causal, scale=work.scale, out=o, lse=lse)

    settled = settle_clock(step, settle_s)
    warmed = warm_up(step, warmup)
    if steps is None:
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(20):
            step()
        torch.cuda.synchronize()
        per = (time.perf_counter() - t0) / 20
        steps = max(MIN_STEPS, int(MIN_TIMED_S / per) + 1)
    stream = torch.cuda.current_stream(dev)   # the stream the kernel is launched on
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        starts[i].record(stream)
        step()
        ends[i].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per_launch_ms = [s.elapsed_time(e) for s, e in zip(starts, ends)]
    return wall, per_launch_ms, warmed, settled


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps; default: at least %d, and enough for %.1f s of timed launches "
                         "(the attention benchmark; the other modes default to %d)" % (MIN_STEPS, MIN_TIMED_S, MIN_STEPS))
    ap.add_argument("--warmup", type=int, default=-1,
                    help="untimed warmup steps; default: until %.2f s have passed (the clock ramp)" % WARMUP_SECONDS)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--clock-settle", type=float, default=CLOCK_SETTLE_S, metavar="SECONDS",
                    help="back-to-back launches before the warmup steps, so the timed steps run at the "
                         "sustained engine clock (0: none); default %(default)s")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="CPU work budget of the oracle baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="instead of the benchmark, run a plain device copy of MIB MiB (HBM counter calibration)")
    ap.add_argument("--mfma-ceiling", nargs="?", const="bf16", default=None, choices=["bf16", "fp8", "bf16-regs", "fp8-regs"],
                    help="instead of the attention benchmark, time the matrix-core calibration kernel "
                         "(back-to-back MFMAs on random N(0,1) operands from LDS, two waves per SIMD; bf16: "
                         "32x32x16, fp8: the scaled 32x32x64 with E4M3 operands; bf16-regs, fp8-regs: the same with the A "
                         "operand in registers instead of LDS): the dense rate the chip "
                         "sustains under its power limit")
    ap.add_argument("--quantize", action="store_true",
                    help="instead of the attention benchmark, time the per-block E4M3 quantiser on the fp32 Q, K, V "
                         "of the fp8 workload (HBM-bound; reports GB/s)")
    ap.add_argument("--qknorm", action="store_true",
                    help="instead of the attention benchmark, time the QK-RMSNorm across heads on the Q and K of "
                         "the bf16 workload (HBM-bound; reports GB/s)")
    args = ap.parse_args(argv)

    if args.gpus != 1:
        print(f"bench.py: this library runs on one GPU only (--gpus {args.gpus} requested); every (b, h) head is "
              "independent, so sharding heads over GPUs needs no communication, but no multi-GPU path is built.",
              file=sys.stderr)
        return 2
    if (args.steps is not None and args.steps < 1) or args.warmup < -1:
        print("bench.py: --steps must be >= 1 and --warmup >= 0", file=sys.stderr)
        return 2

    if args.copy_calibration > 0:
        return copy_calibration(args.copy_calibration, max(1, args.steps or MIN_STEPS))
    if args.mfma_ceiling:
        return bench_mfma_ceiling(args.steps or MIN_STEPS, args.warmup, args.clock_settle, args.mfma_ceiling)
    if args.quantize:
        return bench_quantize(args.steps or MIN_STEPS, args.warmup, not args.no_cpu_baseline)
    if args.qknorm:
        return bench_qknorm(args.steps or MIN_STEPS, args.warmup, not args.no_cpu_baseline)

    import numpy as np

    from exact_attention_32_amd import inputs as I

    if args.workload not in I.WORKLOADS:
        print(f"bench.py: unknown workload {args.workload}; choose from {sorted(I.WORKLOADS)}", file=sys.stderr)
        return 2
    work = I.WORKLOADS[args.workload]
    x = I.make_inputs(work)

    wall, per_launch, warmed, settled = run_gpu(work, x, args.steps, args.warmup, args.clock_settle)
    steps = len(per_launch)
    flops = work.flops()
    ms_per_step = wall * 1e3 / steps
    value = flops / (ms_per_step * 1e-3) / 1e12
    avg_launch_ms = float(np.mean(per_launch))
    achieved = flops / (avg_launch_ms * 1e-3) / 1e12
    peak = PEAK_TFLOPS[work.dtype]
    import exact_attention_32_amd as ea

    dt_code = {"bf16": ea.ATTN_BF16, "f16": ea.ATTN_F16, "fp8": ea.ATTN_FP8_E4M3, "e5m2": ea.ATTN_FP8_E5M2}[work.dtype]
    kernel = ea.kernel_name(work.d, work.causal, dt_code)

    result = {
        "metric": "attention fwd TFLOP/s and % of MI355X peak MFMA (bf16, fp8)",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmed,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": work.dtype,
        "clock_settle": {"seconds": args.clock_settle, "launches": settled,
                         "why": "MI355X ramps its engine clock over the first ~50 ms of sustained launches; "
                                "these untimed launches precede the warmup steps"},
        "data": "synthetic (seeded N(0,1) inputs of the workload's shape)",
        "config": {"workload": work.name, "B": work.B, "H": work.H, "S_q": work.S_q, "S_k": work.S_k, "d": work.d,
                   "causal": work.causal, "dtype": work.dtype, "scale": work.scale},
        "roofline": {
            "bound": "mfma",
            "achieved": round(achieved, 2),
            "peak": peak,
            "unit": "TFLOP/s",
            "frac": round(achieved / peak, 4),
            "traffic": counter_traffic(kernel, work.name),
            "kernel": kernel,
            "avg_launch_us": round(avg_launch_ms * 1e3, 2),
            "median_launch_us": round(float(np.median(per_launch)) * 1e3, 2),
            "min_launch_us": round(float(np.min(per_launch)) * 1e3, 2),
            "algorithmic_flop_per_launch": flops,
            "algorithmic_hbm_bytes_per_launch": work.hbm_bytes(),
        },
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = run_cpu_baseline(work, x, args.cpu_seconds)
    print(json.dumps(result), flush=True)
    return 0


def copy_calibration(mib: int, reps: int) -> int:
    """A plain device-to-device copy of known size: what FETCH_SIZE / WRITE_SIZE read per byte moved."""
    import torch

    n = mib * 1024 * 1024 // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read": n * 4, "copy_calibration_bytes_written": n * 4,
                      "launches": reps}), flush=True)
    return 0


def bench_mfma_ceiling(steps: int, warmup: int, settle_s: float, kind: str = "bf16") -> int:
    """One step = one launch of the matrix-core calibration kernel on every CU."""
    import ctypes

    import numpy as np
    import torch

    from exact_attention_32_amd import build as B

    if not os.path.exists(B.RATE_LIB):
        raise RuntimeError(f"calibration library not built: {B.RATE_LIB}")
    L = ctypes.CDLL(B.RATE_LIB)
    fp8 = kind.startswith("fp8")
    regs = kind.endswith("-regs")
    fn = {("bf16", False): L.attn_mfma_rate, ("bf16", True): L.attn_mfma_rate_regs,
          ("fp8", False): L.attn_mfma_rate_fp8, ("fp8", True): L.attn_mfma_rate_fp8_regs}[("fp8" if fp8 else "bf16", regs)]
    fn.restype = ctypes.c_int
    fn.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    dev = torch.device("cuda:0")
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    g = torch.Generator().manual_seed(11)
    if fp8:   # E4M3 codes of N(0,1) values (finite: no NaN code)
        table = torch.randn(65536, generator=g).to(torch.float8_e4m3fn).view(torch.uint8).to(dev)
    else:
        table = torch.randn(32768, generator=g).to(torch.bfloat16).to(dev)
    out = torch.empty(cus * 512, dtype=torch.float32, device=dev)
    iters = 2000
    stream = torch.cuda.current_stream(dev)

    def step():
        rc = fn(table.data_ptr(), cus, iters, out.data_ptr(), ctypes.c_void_p(stream.cuda_stream))
        if rc != 0:
            raise RuntimeError(f"attn_mfma_rate ({kind}): {rc}")

    settled = settle_clock(step, settle_s)
    warmed = warm_up(step, warmup)
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        starts[i].record(stream)
        step()
        ends[i].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = [a.elapsed_time(b) for a, b in zip(starts, ends)]
    kdepth, peak = (64, 5000.0) if fp8 else (16, 2500.0)
    flops = cus * 8 * 16 * iters * 32 * 32 * kdepth * 2
    avg = float(np.mean(per))
    result = {
        "metric": f"dense {'fp8' if fp8 else 'bf16'} MFMA rate on random operands (matrix-core calibration)",
        "value": round(flops / (wall / steps) / 1e12, 1), "unit": "TFLOP/s",
        "n_gpus": 1, "steps": steps, "warmup": warmed, "ms_per_step": round(wall * 1e3 / steps, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "fp8 e4m3" if fp8 else "bf16",
        "data": "synthetic",
        "clock_settle": {"seconds": settle_s, "launches": settled},
        "config": {"workload": ("mfma_scale_32x32x64_e4m3" if fp8 else "mfma_32x32x16_bf16")
                   + ("_random_register_operands" if regs else "_random_lds_operands"),
                   "cus": cus, "waves_per_simd": 2, "mfmas_per_wave": 16 * iters},
        "roofline": {"bound": "mfma", "achieved": round(flops / (avg * 1e-3) / 1e12, 1), "peak": peak,
                     "unit": "TFLOP/s", "frac": round(flops / (avg * 1e-3) / 1e12 / peak, 4), "traffic": None,
                     "kernel": "mfma_rate_kernel", "avg_launch_us": round(avg * 1e3, 2),
                     "algorithmic_flop_per_launch": flops},
    }
    print(json.dumps(result), flush=True)
    return 0


def bench_quantize(steps: int, warmup: int, cpu: bool) -> int:
    """One step = E4M3 block quantisation of the fp32 Q, K and V of the fp8 workload (one launch)."""
    import numpy as np
    import torch

    import exact_attention_32_amd as ea
    from exact_attention_32_amd import inputs as I

    work = I.WORKLOADS["fp8_b2_h16_s4096_d128"]
    x = I.make_inputs(work)
    dev = torch.device("cuda:0")
    srcs = [torch.from_numpy(a).to(dev) for a in (x.q32, x.k32, x.v32)]
    outs = [(torch.empty(t.shape, dtype=torch.uint8, device=dev),
             torch.empty((work.B, work.H, (t.shape[2] + 127) // 128), dtype=torch.float32, device=dev)) for t in srcs]
    L = ea.load_library()
    B, H, S, d = srcs[0].shape
    args = ([t.data_ptr() for t in srcs] + [ea.ATTN_F32, ea.ATTN_FP8_E4M3] + [c.data_ptr() for c, _ in outs]
            + [x.data_ptr() for _, x in outs] + [B, H, S, S, d])

    def step():
        ea._check(L.attn_quantize_qkv(*args, ea._stream(dev)))

    warmup = warm_up(step, warmup)
    stream = torch.cuda.current_stream(dev)
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    t0 = time.perf_counter()
    for i in range(steps):
        starts[i].record(stream)
        step()
        ends[i].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = [a.elapsed_time(b) for a, b in zip(starts, ends)]
    elems = sum(t.numel() for t in srcs)
    nblk = sum(d.numel() for _, d in outs)
    alg_bytes = elems * (4 + 1) + nblk * 4      # fp32 in, code out, descale out, each once
    ms_step = wall * 1e3 / steps
    avg = float(np.mean(per))
    result = {
        "metric": "fp8 block quantisation of Q, K, V (HBM GB/s)",
        "value": round(alg_bytes / (ms_step * 1e-3) / 1e9, 1),
        "unit": "GB/s",
        "n_gpus": 1, "steps": steps, "warmup": warmup, "ms_per_step": round(ms_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32->e4m3",
        "data": "synthetic (the fp32 N(0,1) draws of the fp8 workload)",
        "config": {"workload": "quantize_" + work.name, "tensors": 3, "shape": list(srcs[0].shape)},
        "roofline": {"bound": "hbm", "achieved": round(alg_bytes / (avg * 1e-3) / 1e9, 1), "peak": 8000.0,
                     "unit": "GB/s", "frac": round(alg_bytes / (avg * 1e-3) / 1e9 / 8000.0, 4), "traffic": None,
                     "kernel": "quantize_fp8_kernel (Q, K, V in one launch)", "avg_step_us": round(avg * 1e3, 2),
                     "algorithmic_bytes_per_step": alg_bytes},
    }
    if cpu:
        from oracle import attn_oracle

        orc = attn_oracle.get()
        a = np.ascontiguousarray(x.q32[:1, :2])   # 2 heads of Q
        t1 = time.perf_counter()
        orc.quantize_e4m3_blocks(a)
        dt = time.perf_counter() - t1
        result["cpu_baseline"] = {"value": round(a.size * 5 / dt / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
                                  "sample": f"2 of 32 (b,h) heads of Q ({a.size} elements), single-threaded; {dt:.2f} s"}
    print(json.dumps(result), flush=True)
    return 0


def bench_qknorm(steps: int, warmup: int, cpu: bool) -> int:
    """One step = RMSNorm across heads of the bf16 Q and K of the bench's default workload (one launch)."""
    import numpy as np
    import torch

    import exact_attention_32_amd as ea
    from exact_attention_32_amd import inputs as I

    work = I.WORKLOADS[DEFAULT_WORKLOAD]
    x = I.make_inputs(work)
    dev = torch.device("cuda:0")
    q, k = x.q.to(dev), x.k.to(dev)
    g = torch.Generator().manual_seed(1)
    wq = torch.empty(work.H * work.d).uniform_(0.5, 1.5, generator=g).to(torch.bfloat16).to(dev)
    wk = torch.empty(work.H * work.d).uniform_(0.5, 1.5, generator=g).to(torch.bfloat16).to(dev)
    qo, ko = torch.empty_like(q), torch.empty_like(k)
    ea.qk_rmsnorm(q, k, wq, wk, 1e-6, q_out=qo, k_out=ko)   # the binding's checks, once
    L = ea.load_library()
    args = [t.data_ptr() for t in (q, k, wq, wk, qo, ko)] + [work.B, work.H, work.S_q, work.S_k, work.d]
    args += [1e-6, ea.ATTN_BF16, ea._stream(dev)]

    def step():   # the C entry point directly: a 22 us kernel would otherwise wait on Python
        ea._check(L.attn_qk_rmsnorm(*args))

    warmup = warm_up(step, warmup)
    stream = torch.cuda.current_stream(dev)
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    t0 = time.perf_counter()
    for i in range(steps):
        starts[i].record(stream)
        step()
        ends[i].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = [a.elapsed_time(b) for a, b in zip(starts, ends)]
    alg_bytes = 2 * (q.numel() + k.numel()) * 2 + 2 * wq.numel() * 2   # Q, K read and written once; weights
    ms_step = wall * 1e3 / steps
    avg = float(np.mean(per))
    result = {
        "metric": "QK-RMSNorm across heads of Q and K (HBM GB/s)",
        "value": round(alg_bytes / (ms_step * 1e-3) / 1e9, 1),
        "unit": "GB/s",
        "n_gpus": 1, "steps": steps, "warmup": warmup, "ms_per_step": round(ms_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (the bf16 N(0,1) Q and K of the default workload, uniform weights)",
        "config": {"workload": "qknorm_" + work.name, "shape": list(q.shape)},
        "roofline": {"bound": "hbm", "achieved": round(alg_bytes / (avg * 1e-3) / 1e9, 1), "peak": 8000.0,
                     "unit": "GB/s", "frac": round(alg_bytes / (avg * 1e-3) / 1e9 / 8000.0, 4), "traffic": None,
                     "kernel": "qk_rmsnorm_kernel", "avg_launch_us": round(avg * 1e3, 2),
                     "algorithmic_bytes_per_launch": alg_bytes},
    }
    if cpu:
        from oracle import attn_oracle

        orc = attn_oracle.get()
        a = x.q[:1].double().numpy()            # one batch entry of Q (all heads, all tokens)
        w64 = wq.cpu().double().numpy()
        reps, t1 = 0, time.perf_counter()
        while reps == 0 or time.perf_counter() - t1 < 2.0:
            orc.rmsnorm_across_heads(a, w64, 1e-6)
            reps += 1
        dt = time.perf_counter() - t1
        result["cpu_baseline"] = {"value": round(reps * a.size * 4 / dt / 1e9, 4), "unit": "GB/s", "cores": 1,
                                  "kind": "oracle",
                                  "sample": f"batch entry 0 of Q ({a.size} elements, bf16 bytes in and out), "
                                            f"{reps} repetitions, single-threaded fp64; {dt:.2f} s"}
    print(json.dumps(result), flush=True)
    return 0


def run_cpu_baseline(work, x, target_s: float):
    """The fp64 oracle on whole (b, h) heads of the same workload, sized to about target_s seconds."""
    import numpy as np

    from oracle import attn_oracle

    orc = attn_oracle.get()
    threads, cpus = cpu_share()
    BH = work.B * work.H

    qa, ka, va = _oracle_arrays(work, x, orc)

    def timed(n):
        q = np.ascontiguousarray(qa.reshape(BH, *qa.shape[2:])[:n][None])
        k = np.ascontiguousarray(ka.reshape(BH, *ka.shape[2:])[:n][None])
        v = np.ascontiguousarray(va.reshape(BH, *va.shape[2:])[:n][None])
        t0 = time.perf_counter()
        orc.attention(q, k, v, work.causal, work.scale, nthreads=threads)
        return time.perf_counter() - t0

    t1 = timed(1)
    n = int(min(BH, max(1, round(target_s / max(t1, 1e-6)))))
    t = timed(n) if n > 1 else t1
    flops = work.flops() * n // BH
    used = orc.last_threads
    return {"value": round(flops / t / 1e12, 6), "unit": "TFLOP/s", "cores": used, "kind": "oracle",
            "host_cpus": cpus,
            "sample": f"{n} of {BH} (b,h) heads of {work.name}, all {work.S_q} query rows each, fp64 explicit "
                      f"softmax; {t:.2f} s on {used} threads (host: {cpus['nproc']} CPUs, "
                      f"{cpus['affinity']} in this process's affinity set, CPU share {cpus['share']})"}


def cpu_share():
    """Threads for the oracle baseline: every CPU of this process's affinity set, or the host's CPU
    share for this GPU where the environment states one (OMP_NUM_THREADS), whichever is smaller;
    and the counts behind that choice."""
    affinity = len(os.sched_getaffinity(0))
    nproc = os.cpu_count() or affinity
    try:
        share = int(os.environ.get("OMP_NUM_THREADS", "0"))
    except ValueError:
        share = 0
    threads = min(affinity, share) if share > 0 else affinity
    return max(1, threads), {"nproc": nproc, "affinity": affinity, "share": share if share > 0 else None}


def _oracle_arrays(work, x, orc):
    from exact_attention_32_amd import inputs as I

    if I.is_fp8(work.dtype):
        fmt = "e5m2" if work.dtype == "e5m2" else "e4m3"
        return tuple(orc.decode_fp8_blocks(c.numpy(), ds.numpy(), fmt)
                     for c, ds in ((x.q, x.q_descale), (x.k, x.k_descale), (x.v, x.v_descale)))
    return x.q.double().numpy(), x.k.double().numpy(), x.v.double().numpy()


if __name__ == "__main__":
    sys.exit(main())
