"""Benchmark of the fp16 -> fp32-accumulate GEMM on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--layout nn|nt]
                    [--workload square|small|edge|linear|batched] [--case C]
                    [--shape M N K] [--dtype f16|bf16] [--no-cpu-baseline]
                    [--epilogue none|bias|relu|gelu|silu]

Default workload (the headline): a step is one C = A*B + C GEMM (the whole hot
path: staging, MFMA K loop, epilogue) at M = N = K = 8192, fp16 A, B, C
uniform [-1, 1) from seed 0, alpha = beta = 1, fp16 output, with A, B and C
resident in HBM before timing starts.  W untimed warm-up steps, then K timed
steps bracketed by device synchronisation; the time per step comes from HIP
events recorded on the stream the kernels are launched on.  Prints one JSON
line (value = TFLOP/s, 2*M*N*K flops per step).

Other workloads, one GEMM configuration per run (--case picks it):
  small    256^3 NN, beta = 0;
  edge     (1,4096,4096), (1000,1000,1000), (127,257,33), (4097,63,1025) NN,
           beta = 0 (--case 0..3);
  linear   X (M x 4096) ~ N(0,1) times W^T, W stored N x 4096 ~ N(0, 0.02),
           beta = 0 (--case M,N with M in 16,128,2048,8192 and N in
           4096,11008,12288);
  batched  512 x (64x64 @ 64x64) NN, or 256 x Q(128x64) @ K^T(64x128)
           (--case sq64|qk); values N(0,1)/8, fp32 C, beta = 0.
  layernorm  the linear layer with its residual and LayerNorm: Y =
           LayerNorm(X W^T + bias + R) gamma + beta_ln, X (M x 4096) ~ N(0,1),
           W stored N x 4096 ~ N(0, 0.02), residual R ~ N(0,1) (beta = 1)
           (--case M,N, default 2048,4096); a step is the GEMM and the row pass.
  attention  fused softmax(Q K^T / sqrt(D)) V, fp16 Q, K, V, O ~ N(0,1):
           --case qk (256 heads of 128 x 128, D = 64: the batched Q K^T shape),
           prefill (4 x 16 heads of 4096 x 4096, D = 128) or prefill_causal;
           flops 4 Sq Sk D per head (half of that, plus the diagonal, causal).
  conv     implicit-GEMM convolution, NHWC fp16 ~ N(0,1), KRSC filters:
           --case r50 (32 x 56 x 56 x 64 -> 64, 3x3, pad 1: a ResNet-50 stage-2
           layer, the default) or stem (32 x 224 x 224 x 3 -> 64, 7x7, stride
           2, pad 3); flops 2 N P Q K R S C.
  softmax  row softmax of 8192 rows x --case cols (default 4096), fp16 in
           and out, x ~ N(0, 4); HBM-bound: 4 bytes per element.
Products bound by HBM bytes (intensity below the ridge of 2516.6 TFLOP/s /
8 TB/s = 315 flop/B) report their roofline in GB/s of algorithmic bytes
(each operand once, C read when beta != 0 and written) against 8 TB/s; the
others in TFLOP/s against the dense MFMA peak.  An HBM-bound GEMM whose
inputs and output are smaller than 512 MiB would be served from the 256 MB
Infinity Cache when repeated: such runs rotate through enough independent
input sets (device copies of the seeded set) to exceed 512 MiB, one set per
step.

The GPU clock is read (amdsmi's GPU metrics, when the box exposes them) over
a window of further steps of the same kernel right after the timed ones --
the firmware refreshes its clock readings only every few hundred
milliseconds; `pct_of_measured_clock_peak` prices the throughput against
256 CUs x 4096 flop/clk x that clock.  The CPU baseline is the oracle (a plain
fp64 triple loop on the host cores), timed on a bounded sample of the same
workload: a fixed set of rows of C.
"""
import argparse
import json
import math
import os
import sys
import threading
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_F16_TFLOPS = 2516.6     # 256 CU x 2.4 GHz x 4096 dense fp16 (or bf16) flop/clk/CU
PEAK_HBM_GBS = 8000.0
RIDGE = PEAK_F16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)   # flop per byte
NUM_CUS = 256
FLOP_PER_CLK_CU = 4096
ROTATE_BYTES = 512 << 20
EDGE_SHAPES = [(1, 4096, 4096), (1000, 1000, 1000), (127, 257, 33), (4097, 63, 1025)]
LINEAR_M = (16, 128, 2048, 8192)
LINEAR_N = (4096, 11008, 12288)


def parse(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", choices=["square", "small", "edge", "linear", "batched",
                                           "layernorm", "attention", "softmax", "conv"],
                    default="square")
    ap.add_argument("--case", default=None,
                    help="edge: 0..3; linear: M,N; batched: sq64|qk")
    ap.add_argument("--layout", choices=["nn", "nt"], default="nn",
                    help="square workload: B row-major (nn) or column-major (nt)")
    ap.add_argument("--shape", type=int, nargs=3, default=[8192, 8192, 8192],
                    help="square workload: M N K")
    ap.add_argument("--dtype", choices=["f16", "bf16"], default="f16",
                    help="element type of A, B and a 16-bit C (default f16)")
    ap.add_argument("--epilogue", choices=["none", "bias", "relu", "gelu", "silu"],
                    default="none", help="fused epilogue (default none)")
    ap.add_argument("--clock-window", type=float, default=1.5,
                    help="seconds of further steps, after the timed ones, over which "
                         "the GPU clock is sampled (0: no clock reading)")
    ap.add_argument("--graph", dest="graph", action="store_true", default=None,
                    help="time the steps as one captured HIP graph (no host launch "
                         "cost between kernels; the default for all but the square "
                         "workload)")
    ap.add_argument("--no-graph", dest="graph", action="store_false")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=2048)
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="calibration only: time a plain device copy of this many "
                         "bytes (for scaling the FETCH_SIZE / WRITE_SIZE counters)")
    return ap.parse_args(argv)


# ------------------------------------------------------------ workloads

def make_workload(args):
    """(case, description, cpu_rows) of the selected workload; the case comes
    from the shared seeded generator (gemm_inputs)."""
    import gemm_inputs as gi
    dt = args.dtype
    out16 = gi.OUT_BF16 if dt == "bf16" else gi.OUT_F16
    tname = "bf16" if dt == "bf16" else "fp16"
    w = args.workload
    if w == "square":
        M, N, K = args.shape
        lb = gi.COL_MAJOR if args.layout == "nt" else gi.ROW_MAJOR
        case = gi.make_case(M, N, K, layout_b=lb, alpha=1.0, beta=1.0, seed=0,
                            in_dtype=dt, out_type=out16)
        desc = (f"gemm {M}x{N}x{K} {args.layout.upper()} alpha=1 beta=1, {tname} A/B/C "
                f"uniform[-1,1) seed 0, fp32 accumulation, {tname} out")
        return case, desc, args.cpu_rows
    if w == "small":
        case = gi.make_case(256, 256, 256, seed=0, in_dtype=dt, out_type=out16)
        return case, f"gemm 256x256x256 NN alpha=1 beta=0, {tname} uniform[-1,1) seed 0", 256
    if w == "edge":
        i = int(args.case or 0)
        M, N, K = EDGE_SHAPES[i]
        case = gi.make_case(M, N, K, seed=0, in_dtype=dt, out_type=out16)
        return case, f"edge gemm {M}x{N}x{K} NN alpha=1 beta=0, {tname} uniform[-1,1) seed 0", M
    if w == "linear":
        M, N = (int(v) for v in (args.case or "16,11008").split(","))
        if M not in LINEAR_M or N not in LINEAR_N:
            raise SystemExit(f"linear --case M,N with M in {LINEAR_M} and N in {LINEAR_N}")
        case = gi.linear_case(M, N, in_dtype=dt)
        return case, (f"linear layer X({M}x4096) W^T, W stored {N}x4096 (NT), X~N(0,1), "
                      f"W~N(0,0.02), beta=0, {tname} out"), min(M, 256)
    if w == "layernorm":
        M, N = (int(v) for v in (args.case or "2048,4096").split(","))
        out = gi.OUT_BF16 if dt == "bf16" else gi.OUT_F16
        case = gi.make_case(M, N, 4096, layout_b=gi.COL_MAJOR, dist_a="normal", dist_b="normal",
                            dist_c="normal", sigma_a=1.0, sigma_b=0.02, sigma_c=1.0, beta=1.0,
                            seed=0, in_dtype=dt, out_type=out)
        return case, (f"linear layer + residual + LayerNorm: X({M}x4096) W^T + bias + R, W stored "
                      f"{N}x4096, X~N(0,1), W~N(0,0.02), R~N(0,1), eps 1e-5, {tname} out"), min(M, 256)
    if w == "batched":
        kind = args.case or "sq64"
        case = gi.batched_case(kind)
        if dt == "bf16":
            raise SystemExit("the batched workload is fp16 (fp32 C)")
        desc = ("batched 512 x (64x64 @ 64x64) NN" if kind == "sq64" else
                "batched 256 x Q(128x64) @ K^T(64x128) NT") + ", N(0,1)/8, fp32 C, beta=0"
        return case, desc, case.M
    raise SystemExit(w)


def algorithmic_bytes(case):
    """Each operand moved once: A and B (logical elements), C read when beta
    != 0, C written."""
    in_b = 2
    out_b = 4 if case.out_type == 1 else 2
    per = in_b * (case.M * case.K + case.K * case.N) + out_b * case.M * case.N * (
        2 if case.beta != 0 else 1)
    return per * case.batch


# ------------------------------------------------------------ GPU clock

class ClockSampler:
    """The GPU's graphics clock (MHz, mean over the XCDs) from amdsmi's GPU
    metrics.  The firmware refreshes that table only every few hundred
    milliseconds, so the clock is sampled over a window of sustained load
    (the benchmark keeps launching its step meanwhile) and only readings with
    a new firmware timestamp and the engine at least half busy are kept.  Inert where
    amdsmi or the metrics are unavailable."""

    def __init__(self, enabled=True):
        self.samples = []
        self.power_w = []        # socket power (W) of the same readings
        self.power_cap_w = None
        self._power = None
        self._handle = None
        self._last_ts = None
        self.error = None
        if not enabled:         # --clock-window 0: amdsmi is not touched at all
            return
        try:
            import amdsmi
            amdsmi.amdsmi_init()
            self._amdsmi = amdsmi
            self._handle = amdsmi.amdsmi_get_processor_handles()[0]
            self._last_ts = self._read()[0]
            try:
                cap = amdsmi.amdsmi_get_power_cap_info(self._handle).get("power_cap")
                self.power_cap_w = cap / 1e6 if isinstance(cap, (int, float)) and cap > 0 else None
            except Exception:
                pass
        except Exception as e:   # no amdsmi, no permission, no device
            self.error = f"{type(e).__name__}: {e}"[:120]
            self._handle = None

    def _read(self):
        m = self._amdsmi.amdsmi_get_gpu_metrics_info(self._handle)
        clks = [c for c in (m.get("current_gfxclks") or []) if isinstance(c, (int, float)) and c > 0]
        if not clks and isinstance(m.get("current_gfxclk"), (int, float)):
            clks = [m["current_gfxclk"]]
        busy = m.get("average_gfx_activity")
        power = m.get("current_socket_power")
        self._power = power if isinstance(power, (int, float)) and power > 0 else None
        return m.get("firmware_timestamp"), (sum(clks) / len(clks) if clks else None), busy

    def poll(self):
        """Takes a reading if the firmware has refreshed the table since the
        last one and reports the graphics engine busy."""
        if self._handle is None:
            return
        try:
            ts, mhz, busy = self._read()
        except Exception:
            return
        if ts is not None and ts != self._last_ts:
            self._last_ts = ts
            if mhz is not None and isinstance(busy, (int, float)) and busy >= 50:
                self.samples.append(mhz)
                if self._power is not None:
                    self.power_w.append(self._power)

    @property
    def available(self):
        return self._handle is not None

    def mean_mhz(self):
        return sum(self.samples) / len(self.samples) if self.samples else None

    def mean_power_w(self):
        return sum(self.power_w) / len(self.power_w) if self.power_w else None


# ------------------------------------------------------------ helpers

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


def bench_key(args):
    """The key under which a committed profile describes this run."""
    if args.workload == "square":
        M, N, K = args.shape
        return f"square {args.layout} {M}x{N}x{K} {args.dtype}"
    case = args.case if args.case is not None else {
        "edge": "0", "linear": "16,11008", "batched": "sq64", "layernorm": "2048,4096",
        "attention": "prefill", "conv": "r50", "softmax": "4096"}.get(args.workload, "0")
    return f"{args.workload} {case} {args.dtype}"


def profile_fields(path):
    fields = {}
    with open(path) as fh:
        for line in fh:
            if ":" in line and not line.startswith(" "):
                k, v = line.split(":", 1)
                fields[k.strip()] = v.strip()
    return fields


def profiled_traffic(key):
    """HBM-side bytes per step (FETCH_SIZE + WRITE_SIZE of the library's
    kernels, scaled by the copy calibration) from the committed rocprofv3
    summary whose bench_key is `key`, or None when there is none or the
    kernels have changed since it was taken."""
    import glob
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "*.md"))):
        fields = profile_fields(path)
        if fields.get("bench_key") != key:
            continue
        if fields.get("kernel_source_hash") != kernel_source_hash():
            return None
        try:
            return int(float(fields["traffic_bytes"]))
        except (KeyError, ValueError):
            return None
    return None


def cpu_baseline(case, nrows, bias=None, act=0, ln=None):
    """Times the oracle on `nrows` rows of C (fixed, spread over M; every
    batch item) -- about 5-15 s on 16 host threads for the largest
    workloads."""
    import numpy as np
    import torch
    import oracle
    u16 = lambda t: t.view(torch.int16).numpy().view(np.uint16)
    rows = np.linspace(0, case.M - 1, num=min(nrows, case.M)).astype(np.int64)
    rows = np.unique(rows)
    nproc = os.cpu_count() or 1
    threads = min(16, nproc)
    bf = case.meta.get("in_dtype") == "bf16"
    cdata = u16(case.C) if case.out_type != 1 else case.C.numpy()
    t0 = time.perf_counter()
    if ln is not None:
        gamma, beta_ln, eps = ln
        oracle.gemm_layernorm(case.M, case.N, case.K, u16(case.A), u16(case.B), cdata,
                              gamma=gamma.cpu().numpy(), beta_ln=beta_ln.cpu().numpy(), eps=eps,
                              alpha=case.alpha, beta=case.beta,
                              bias=None if bias is None else bias.cpu().numpy(),
                              layout_a=case.layout_a, layout_b=case.layout_b,
                              out_type=case.out_type, in_type=oracle.IN_BF16 if bf else oracle.IN_F16,
                              lda=case.lda, ldb=case.ldb, ldc=case.ldc, rows=rows, nthreads=threads)
    else:
        oracle.gemm(case.M, case.N, case.K, u16(case.A), u16(case.B), cdata,
                    alpha=case.alpha, beta=case.beta, layout_a=case.layout_a,
                    layout_b=case.layout_b, out_type=case.out_type,
                    in_type=oracle.IN_BF16 if bf else oracle.IN_F16,
                    lda=case.lda, ldb=case.ldb, ldc=case.ldc, batch=case.batch,
                    stride_a=case.stride_a, stride_b=case.stride_b, stride_c=case.stride_c,
                    bias=None if bias is None else bias.cpu().numpy(), activation=act,
                    rows=rows, nthreads=threads)
    dt = time.perf_counter() - t0
    flops = 2.0 * rows.size * case.N * case.K * case.batch
    batch = f" x {case.batch} batch items" if case.batch > 1 else ""
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s",
            "cores": threads, "nproc": nproc, "kind": "oracle",
            "sample": f"{rows.size} of {case.M} rows of C (all {case.N} columns, "
                      f"full K={case.K}){batch}, {dt:.2f} s wall including operand decode"}


ATTN_CASES = {"qk": (2, 128, 128, 128, 64, False), "prefill": (4, 16, 4096, 4096, 128, False),
              "prefill_causal": (4, 16, 4096, 4096, 128, True)}


def run_attention_bench(args):
    """The fused attention or row-softmax workload: one launch per step,
    timed like the GEMM workloads (graph replay by default, rotating input
    sets when HBM-bound)."""
    import torch
    import mixed_precision_gemm_amd as mpg
    dev = torch.device("cuda:0")
    g = torch.Generator("cpu").manual_seed(0)
    stream = torch.cuda.current_stream(dev)
    if args.workload == "attention":
        case = args.case or "prefill"
        B, H, S, _, D, causal = ATTN_CASES[case]
        q, k, v = ((torch.randn((B, H, S, D), generator=g)).half().to(dev) for _ in range(3))
        o = torch.empty_like(q)
        st3 = lambda t: (t.stride(0), t.stride(1), t.stride(2))
        st, h = mpg.attn_f16_plan(B, H, S, S, D, st3(q), st3(k), st3(v), st3(o), int(causal), 0)
        if st != mpg.GEMM_OK:
            raise mpg.GemmError(st, "attn_f16_plan")
        kernel = mpg.attn_f16_plan_kernel(h)
        pairs = S * (S + 1) / 2 if causal else S * S
        flops = 4.0 * pairs * D * B * H
        abytes = 4 * B * H * S * D * 2
        unit_sets = [(q, k, v, o)]
        set_bytes = abytes
        run = lambda t: mpg.library().attn_f16_run(h, t[0].data_ptr(), t[1].data_ptr(),
                                                   t[2].data_ptr(), t[3].data_ptr(),
                                                   1.0 / math.sqrt(D), stream.cuda_stream)
        desc = (f"fused attention {B}x{H} heads, Sq=Sk={S}, D={D}{' causal' if causal else ''}, "
                f"fp16 Q/K/V/O ~ N(0,1), scale 1/sqrt(D)")
        cfg = {"batch": B, "heads": H, "Sq": S, "Sk": S, "D": D, "causal": causal}
    elif args.workload == "conv":
        case = args.case or "r50"
        N, H, W, C, K, R, S, st_, pd = {"r50": (32, 56, 56, 64, 64, 3, 3, 1, 1),
                                        "stem": (32, 224, 224, 3, 64, 7, 7, 2, 3)}[case]
        x = torch.randn((N, H, W, C), generator=g).half().to(dev)
        w = (torch.randn((K, R, S, C), generator=g) / math.sqrt(R * S * C)).half().to(dev)
        st, h = mpg.conv_f16_plan(N, H, W, C, K, R, S, (st_, st_), (pd, pd), (1, 1), 0)
        if st != mpg.GEMM_OK:
            raise mpg.GemmError(st, "conv_f16_plan")
        _, P, Q = mpg.conv_f16_output_size(h)
        y = torch.empty((N, P, Q, K), dtype=torch.float16, device=dev)
        kernel = mpg.conv_f16_plan_kernel(h)
        flops = 2.0 * N * P * Q * K * R * S * C
        abytes = 2 * (x.numel() + w.numel() + y.numel())
        unit_sets = [(x, w, y)]
        set_bytes = abytes
        run = lambda t: mpg.library().conv_f16_run(h, t[0].data_ptr(), t[1].data_ptr(),
                                                   t[2].data_ptr(), 1.0, 0.0, None, 0,
                                                   stream.cuda_stream)
        desc = (f"implicit-GEMM conv {N}x{H}x{W}x{C} -> {K}, {R}x{S} stride {st_} pad {pd}, "
                f"fp16 NHWC/KRSC/NPQK")
        cfg = {"N": N, "H": H, "W": W, "C": C, "K": K, "R": R, "S": S, "stride": st_, "pad": pd}
    else:
        cols = int(args.case or 4096)
        rows = 8192
        x = (torch.randn((rows, cols), generator=g) * 4).half().to(dev)
        y = torch.empty_like(x)
        kernel = ("softmax_rows_online" if cols > 8192 else
                  "softmax_rows_vec" if cols % 8 == 0 else "softmax_rows_reg")
        flops = 0.0
        abytes = rows * cols * 4
        unit_sets = [(x, y)]
        set_bytes = abytes
        run = lambda t: mpg.library().attn_softmax_rows(rows, cols, t[0].data_ptr(), cols, 0,
                                                        t[1].data_ptr(), cols, 0, stream.cuda_stream)
        desc = f"row softmax {rows} x {cols}, fp16 in and out, x ~ N(0, 4)"
        cfg = {"rows": rows, "cols": cols}
    hbm_bound = flops / abytes < RIDGE
    nsets = (math.ceil(ROTATE_BYTES / set_bytes) + 1 if hbm_bound and set_bytes < ROTATE_BYTES else 1)
    sets = unit_sets + [tuple(t.clone() for t in unit_sets[0]) for _ in range(nsets - 1)]
    print(f"# kernel {kernel}, {desc}, {nsets} input set(s)", file=sys.stderr, flush=True)

    def step(i):
        st = run(sets[i % nsets])
        if st != mpg.GEMM_OK:
            raise mpg.GemmError(st, args.workload)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    graph = None
    if args.graph:
        graph = torch.cuda.CUDAGraph()
        gs = torch.cuda.Stream()
        gs.wait_stream(stream)
        outer = stream
        stream = gs
        with torch.cuda.graph(graph, stream=gs):
            for i in range(args.steps):
                step(i)
        stream = outer
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    if graph is not None:
        graph.replay()
    else:
        for i in range(args.steps):
            step(i)
    ev1.record(stream)
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / args.steps
    if args.workload == "attention":
        mpg.attn_f16_destroy(h)
    elif args.workload == "conv":
        mpg.conv_f16_destroy(h)
    tflops = flops / (ms * 1e-3) / 1e12
    gbs = abytes / (ms * 1e-3) / 1e9
    traffic = profiled_traffic(bench_key(args))
    if hbm_bound:
        roof = {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": traffic, "algorithmic_bytes": abytes}
    else:
        roof = {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_F16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(tflops / PEAK_F16_TFLOPS, 4), "traffic": traffic,
                "algorithmic_bytes": abytes}
    what = "(fp32 accumulation)" if args.workload == "conv" else "(fp32 softmax)"
    out = {"metric": f"FP16 {args.workload} {'GB/s' if hbm_bound else 'TFLOP/s'} {what}",
           "value": round(gbs if hbm_bound else tflops, 2),
           "unit": "GB/s" if hbm_bound else "TFLOP/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": "f16", "data": "synthetic",
           "config": dict(workload=desc, kernel=kernel, input_sets=nsets,
                          timing="hip graph replay" if graph is not None else "stream launches", **cfg),
           "tflop_per_s": round(tflops, 2), "gb_per_s": round(gbs, 1), "flop_per_step": flops,
           "roofline": roof}
    print(json.dumps(out), flush=True)


def main():
    args = parse()
    if args.graph is None:
        args.graph = args.workload != "square"
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this GEMM is built and measured on "
              "a single MI355X (run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    if args.copy_bytes:
        copy_calibration(args.copy_bytes, args.steps)
        return

    if args.workload in ("attention", "softmax", "conv"):
        run_attention_bench(args)
        return

    import torch
    import mixed_precision_gemm_amd as mpg

    case, desc, cpu_rows = make_workload(args)
    M, N, K = case.M, case.N, case.K
    dev = torch.device("cuda:0")
    dA, dB, dC = case.A.to(dev), case.B.to(dev), case.C.to(dev)
    plan = mpg.Plan(M, N, K, case.layout_a, case.layout_b, case.out_type,
                    case.lda, case.ldb, case.ldc, case.batch, case.stride_a,
                    case.stride_b, case.stride_c, dtype=args.dtype)
    stream = torch.cuda.current_stream(dev)
    bias = None
    act = {"none": 0, "bias": 0, "relu": 1, "gelu": 2, "silu": 3}[args.epilogue]
    if args.epilogue != "none" or args.workload == "layernorm":
        g = torch.Generator("cpu").manual_seed(1)
        bias = (torch.rand(N, generator=g) * 2 - 1).to(dev)
        plan.set_epilogue(bias, act)
    if args.workload == "layernorm":
        g = torch.Generator("cpu").manual_seed(2)
        ln_gamma = (1 + 0.3 * torch.randn(N, generator=g)).to(dev)
        ln_beta = (0.2 * torch.randn(N, generator=g)).to(dev)
        plan.set_layernorm(ln_gamma, ln_beta, 1e-5)

    # HBM-bound products rotate through independent input sets past the
    # Infinity Cache when one set is small; compute-bound ones (the headline
    # among them) run back to back on one set.
    flops = 2.0 * M * N * K * case.batch
    abytes = algorithmic_bytes(case)
    hbm_bound = flops / abytes < RIDGE
    set_bytes = dA.numel() * 2 + dB.numel() * 2 + dC.numel() * dC.element_size()
    nsets = (math.ceil(ROTATE_BYTES / set_bytes) + 1
             if hbm_bound and set_bytes < ROTATE_BYTES else 1)
    sets = [(dA, dB, dC)] + [(dA.clone(), dB.clone(), dC.clone()) for _ in range(nsets - 1)]
    ws_bytes = plan.workspace_bytes()
    ws = torch.zeros(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    print(f"# kernel {plan.kernel}, {desc}, {nsets} input set(s) of "
          f"{set_bytes / 2**20:.1f} MiB, workspace {ws_bytes} B", file=sys.stderr, flush=True)

    # One C-ABI call per step with its arguments prepared beforehand, so that
    # the host's per-launch cost stays below the shortest kernels' duration.
    run_fn = mpg.gemm_bf16f32_run if args.dtype == "bf16" else mpg.gemm_f16f32_run
    lib_run = getattr(mpg.library(), run_fn.__name__)
    sargs = [(plan.handle, a.data_ptr(), b.data_ptr(), c.data_ptr(), case.alpha, case.beta,
              ws.data_ptr(), ws.numel(), stream.cuda_stream) for a, b, c in sets]

    def step(i):
        st = lib_run(*sargs[i % nsets])
        if st != mpg.GEMM_OK:
            raise mpg.GemmError(st, run_fn.__name__)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    graph, gs = None, None
    if args.graph:
        # The timed steps captured once and replayed: no host work between
        # kernels (for products shorter than a launch's host cost).
        graph = torch.cuda.CUDAGraph()
        gs = torch.cuda.Stream()
        gs.wait_stream(stream)
        with torch.cuda.graph(graph, stream=gs):
            sargs = [a[:-1] + (gs.cuda_stream,) for a in sargs]
            for i in range(args.steps):
                step(i)
        torch.cuda.synchronize()
        graph.replay()          # untimed: the first replay uploads the graph
        torch.cuda.synchronize()

    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    if graph is not None:
        graph.replay()
    else:
        for i in range(args.steps):
            step(i)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    # Clock under sustained load of the same step, after the timed region.
    # Bursts of about 25 ms of steps, two in flight, so the engine never idles.
    clock = ClockSampler(args.clock_window > 0)
    if clock.available and args.clock_window > 0:
        per_step = ev0.elapsed_time(ev1) / args.steps * 1e-3
        burst = max(1, int(25e-3 / max(per_step, 1e-7)))
        t_end = time.perf_counter() + args.clock_window
        i, pending = 0, None
        while time.perf_counter() < t_end:
            if graph is not None:
                for _ in range(max(1, burst // args.steps)):
                    graph.replay()
            else:
                for _ in range(burst):
                    step(i)
                    i += 1
            done = torch.cuda.Event()
            done.record(gs if graph is not None else stream)
            if pending is not None:
                while not pending.query():
                    clock.poll()
                    time.sleep(0.005)
            pending = done
        torch.cuda.synchronize()
    ms_events = ev0.elapsed_time(ev1)
    ms_per_step = ms_events / args.steps
    plan.close()

    tflops = flops / (ms_per_step * 1e-3) / 1e12
    gbs = abytes / (ms_per_step * 1e-3) / 1e9
    mhz = clock.mean_mhz()

    tname = "bf16" if args.dtype == "bf16" else "fp16"
    if args.workload == "square" and (M, N, K) == (8192, 8192, 8192):
        metric = (f"{tname.upper()} GEMM TFLOP/s (fp32 acc) at M=N=K=8192; "
                  f"% of MFMA {tname.upper()} peak")
    else:
        metric = f"{tname.upper()} GEMM TFLOP/s (fp32 acc), {args.workload} workload"
    config = {"workload": desc, "M": M, "N": N, "K": K, "batch": case.batch,
              "layout": ("N" if case.layout_a == 0 else "T") + ("N" if case.layout_b == 0 else "T"),
              "kernel": plan.kernel, "epilogue": args.epilogue, "input_sets": nsets,
              "timing": "hip graph replay" if args.graph else "stream launches"}
    traffic = profiled_traffic(bench_key(args)) if args.epilogue == "none" else None
    if hbm_bound:
        roof = {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": traffic,
                "algorithmic_bytes": abytes}
    else:
        roof = {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_F16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(tflops / PEAK_F16_TFLOPS, 4),
                "traffic": traffic, "algorithmic_bytes": abytes}
    out = {
        "metric": metric,
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
        "config": config,
        "pct_of_peak": round(100.0 * tflops / PEAK_F16_TFLOPS, 2),
        "gb_per_s": round(gbs, 1),
        "clock_mhz_measured": None if mhz is None else round(mhz, 1),
        "clock_samples": len(clock.samples),
        "socket_power_w_measured": (None if clock.mean_power_w() is None
                                    else round(clock.mean_power_w(), 1)),
        "socket_power_cap_w": clock.power_cap_w,
        "pct_of_measured_clock_peak": (None if mhz is None else
                                       round(100.0 * tflops * 1e12 /
                                             (NUM_CUS * FLOP_PER_CLK_CU * mhz * 1e6), 2)),
        "wall_s_timed": round(wall, 4),
        "roofline": roof,
    }
    if mhz is None and clock.error:
        out["clock_note"] = clock.error
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(case, cpu_rows, bias, act,
                                           (ln_gamma, ln_beta, 1e-5) if args.workload == "layernorm" else None)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
