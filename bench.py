"""Benchmark of the fp16 -> fp32-accumulate GEMM on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--layout nn|nt]
                    [--shape M N K] [--dtype f16|bf16] [--no-cpu-baseline]
                    [--epilogue none|bias|relu|gelu|silu]

A step is one C = A*B + C GEMM (the whole hot path: staging, MFMA K loop,
epilogue) on the square workload M = N = K = 8192, fp16 A, B, C uniform
[-1, 1) from seed 0, alpha = beta = 1, fp16 output, with A, B and C resident
in HBM before timing starts.  W untimed warm-up steps, then K timed steps
bracketed by device synchronisation; the kernel's own duration is measured
with HIP events recorded on the stream the kernel is launched on.  Prints one
JSON line (value = TFLOP/s, 2*M*N*K flops per step).  --dtype bf16 runs the
same workload with bfloat16 A, B and C (the bfloat16 entry points);
--epilogue adds the fused epilogue C = act(A*B + C + bias) (a seeded fp32
bias of N values; "bias" alone, or with ReLU / GELU / SiLU).

The CPU baseline is the oracle (a plain fp64 triple loop on the host cores),
timed on a bounded sample of the same workload: a fixed set of rows of C.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_F16_TFLOPS = 2516.6     # 256 CU x 2.4 GHz x 4096 dense fp16 (or bf16) flop/clk/CU
PEAK_HBM_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--layout", choices=["nn", "nt"], default="nn")
    ap.add_argument("--shape", type=int, nargs=3, default=[8192, 8192, 8192])
    ap.add_argument("--dtype", choices=["f16", "bf16"], default="f16",
                    help="element type of A, B and C (default f16)")
    ap.add_argument("--epilogue", choices=["none", "bias", "relu", "gelu", "silu"],
                    default="none", help="fused epilogue (default none)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=2048)
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="calibration only: time a plain device copy of this many "
                         "bytes (for scaling the FETCH_SIZE / WRITE_SIZE counters)")
    return ap.parse_args()


def copy_calibration(nbytes, steps):
    """A plain device-to-device copy of known size; its FETCH_SIZE and
    WRITE_SIZE counter readings give the factor that turns those counters
    into bytes for the GEMM kernel."""
    import torch
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda:0").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    ev0.record()
    for _ in range(steps):
        dst.copy_(src)
    ev1.record()
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / steps
    print(json.dumps({"calibration": "device copy", "bytes_read": nbytes,
                      "bytes_written": nbytes, "ms": round(ms, 5),
                      "GB/s": round(2 * nbytes / ms / 1e6, 1)}), flush=True)


def kernel_source_hash():
    """Hash of the library's code (kernels, planner, ABI header) with comments
    and whitespace removed: a profile taken from other code no longer
    describes the kernel, while a comment edit does not change it."""
    import glob
    import hashlib
    import re
    files = sorted(glob.glob(os.path.join(ROOT, "mixed_precision_gemm_amd", "csrc", "*"))) + \
        sorted(glob.glob(os.path.join(ROOT, "include", "*.h")))
    h = hashlib.sha256()
    for f in files:
        h.update(os.path.basename(f).encode())
        with open(f, "r", encoding="utf-8") as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)   # block comments
        text = re.sub(r"//[^\n]*", " ", text)                 # line comments
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def profiled_traffic(layout, shape, dtype="f16"):
    """HBM-side bytes per launch (FETCH_SIZE + WRITE_SIZE, scaled by the copy
    calibration) from the committed rocprofv3 summary of this workload, or
    None when there is none or the kernels have changed since it was taken."""
    if tuple(shape) != (8192, 8192, 8192):
        return None
    suffix = "" if dtype == "f16" else f"_{dtype}"
    path = os.path.join(ROOT, "profiles", f"gemm_direct_256x256_8192cube_{layout}{suffix}.md")
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as fh:
        for line in fh:
            if ":" in line and not line.startswith(" "):
                k, v = line.split(":", 1)
                fields[k.strip()] = v.strip()
    if fields.get("kernel_source_hash") != kernel_source_hash():
        return None
    try:
        return int(float(fields["traffic_bytes"]))
    except (KeyError, ValueError):
        return None


def cpu_baseline(case, nrows, bias=None, act=0):
    """Times the oracle on `nrows` rows of C (fixed, spread over M)."""
    import numpy as np
    import torch
    import oracle
    u16 = lambda t: t.view(torch.int16).numpy().view(np.uint16)
    rows = np.linspace(0, case.M - 1, num=min(nrows, case.M)).astype(np.int64)
    threads = min(16, os.cpu_count() or 1)
    t0 = time.perf_counter()
    bf = case.meta.get("in_dtype") == "bf16"
    oracle.gemm(case.M, case.N, case.K, u16(case.A), u16(case.B), u16(case.C),
                alpha=case.alpha, beta=case.beta, layout_a=case.layout_a,
                layout_b=case.layout_b, out_type=case.out_type,
                in_type=oracle.IN_BF16 if bf else oracle.IN_F16,
                bias=None if bias is None else bias.cpu().numpy(), activation=act,
                rows=rows, nthreads=threads)
    dt = time.perf_counter() - t0
    flops = 2.0 * rows.size * case.N * case.K
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s",
            "cores": threads, "kind": "oracle",
            "sample": f"{rows.size} of {case.M} rows of C (all {case.N} columns, "
                      f"full K={case.K}), {dt:.1f} s wall including operand decode"}


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this GEMM is built and measured on "
              "a single MI355X (run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    if args.copy_bytes:
        copy_calibration(args.copy_bytes, args.steps)
        return

    import torch
    import gemm_inputs as gi
    import mixed_precision_gemm_amd as mpg

    M, N, K = args.shape
    lb = gi.COL_MAJOR if args.layout == "nt" else gi.ROW_MAJOR
    case = gi.make_case(M, N, K, layout_b=lb, alpha=1.0, beta=1.0, seed=0,
                        in_dtype=args.dtype,
                        out_type=gi.OUT_BF16 if args.dtype == "bf16" else gi.OUT_F16)
    dev = torch.device("cuda:0")
    dA, dB, dC = case.A.to(dev), case.B.to(dev), case.C.to(dev)
    plan = mpg.Plan(M, N, K, case.layout_a, case.layout_b, case.out_type,
                    case.lda, case.ldb, case.ldc, dtype=args.dtype)
    stream = torch.cuda.current_stream(dev)
    bias = None
    act = {"none": 0, "bias": 0, "relu": 1, "gelu": 2, "silu": 3}[args.epilogue]
    if args.epilogue != "none":
        g = torch.Generator("cpu").manual_seed(1)
        bias = (torch.rand(N, generator=g) * 2 - 1).to(dev)
        plan.set_epilogue(bias, act)
    print(f"# kernel {plan.kernel}, {M}x{N}x{K} {args.layout.upper()} {args.dtype}",
          file=sys.stderr, flush=True)

    for _ in range(args.warmup):
        plan.run(dA, dB, dC, 1.0, 1.0, stream=stream)
    torch.cuda.synchronize()

    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        plan.run(dA, dB, dC, 1.0, 1.0, stream=stream)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_events = ev0.elapsed_time(ev1)
    ms_per_step = ms_events / args.steps
    flops = 2.0 * M * N * K
    tflops = flops / (ms_per_step * 1e-3) / 1e12
    plan.close()

    tname = "bf16" if args.dtype == "bf16" else "fp16"
    out = {
        "metric": (f"{tname.upper()} GEMM TFLOP/s (fp32 acc) at M=N=K=8192; "
                   f"% of MFMA {tname.upper()} peak"),
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": args.dtype,
        "data": "synthetic",
        "config": {"workload": f"gemm {M}x{N}x{K} {args.layout.upper()} alpha=1 beta=1, "
                               f"{tname} A/B/C uniform[-1,1) seed 0, fp32 accumulation, "
                               f"{tname} out",
                   "M": M, "N": N, "K": K, "layout": args.layout.upper(),
                   "kernel": plan.kernel, "epilogue": args.epilogue},
        "pct_of_peak": round(100.0 * tflops / PEAK_F16_TFLOPS, 2),
        "wall_s_timed": round(wall, 4),
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2),
                     "peak": PEAK_F16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tflops / PEAK_F16_TFLOPS, 4),
                     "traffic": (profiled_traffic(args.layout, (M, N, K), args.dtype)
                                 if args.epilogue == "none" else None)},
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(case, args.cpu_rows, bias, act)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
