"""Helpers shared by the GPU parity tests: run a case through the C ABI,
compute the oracle on the same inputs, and apply the acceptance bound.

Acceptance bound (per output element, both operands finite):
    |gpu - ref| <= 2e-3 * S + (fp16 C ? ulp16(|ref|) : bf16 C ? ulpbf16(|ref|) : 0)
where ref is the oracle's fp64 value and S = |alpha| sum_k |a_ik b_kj| +
|beta| |c_ij| its error scale.  fp32 accumulation over K <= 8192 terms errs by
at most K * 2^-24 * S <= 4.9e-4 * S in any order, the fp32 epilogue by
2^-24 of its terms, and the final binary16 rounding by half an ulp, so the
bound holds for any correct summation order.  ulp16(x) = 2^(max(floor(log2
x), -14) - 10), ulp16(0) = 2^-24.  A reference whose magnitude reaches 65520
rounds to infinity in binary16: the GPU must then return infinity of the same
sign (or, within the bound, the largest finite value).

bfloat16 inputs: a product of two bfloat16 values (8 significant bits each)
is exact in fp32 just as a binary16 product is, so the same 2e-3 * S covers
the fp32 sum; a bfloat16 C adds half a bfloat16 ulp, ulpbf16(x) =
2^(max(floor(log2 x), -126) - 7), ulpbf16(0) = 2^-133, and overflows only
from (2 - 2^-8) 2^127 on.

Fused epilogue C = act(alpha A B + beta C + bias): S (from the oracle)
includes |bias|, so 2e-3 S bounds the error of the pre-activation value x;
an activation with Lipschitz constant L (ReLU 1, GELU and SiLU below 1.13)
carries it into at most L * 2e-3 * S, and its fp32 evaluation (erfcf, expf
and a division, a few ulp) adds 1e-5 |ref|.
"""
import os

import numpy as np
import torch

import gemm_inputs as gi
import mixed_precision_gemm_amd as mpg
import oracle

REL_TOL = 2e-3
F16_OVERFLOW = 65520.0
BF16_OVERFLOW = (2 - 2.0 ** -8) * 2.0 ** 127


def oracle_threads():
    return min(16, os.cpu_count() or 1)


def ulp16(x):
    x = np.abs(np.asarray(x, dtype=np.float64))
    e = np.floor(np.log2(np.where(x > 0, x, 1.0)))
    e = np.maximum(e, -14)
    u = np.exp2(e - 10)
    return np.where(x > 0, u, 2.0 ** -24)


def ulpbf16(x):
    x = np.abs(np.asarray(x, dtype=np.float64))
    e = np.floor(np.log2(np.where(x > 0, x, 1.0)))
    e = np.maximum(e, -126)
    u = np.exp2(e - 7)
    return np.where(x > 0, u, 2.0 ** -133)


LIPSCHITZ = {0: 1.0, 1: 1.0, 2: 1.13, 3: 1.13}   # oracle.ACT_*


def check_bound(gpu, ref, scale, out_type, what="", act=0):
    """Asserts the acceptance bound element-wise; returns the worst ratio
    |gpu - ref| / bound over finite references.  act: the fused epilogue's
    activation (oracle.ACT_*), 0 for none."""
    gpu = np.asarray(gpu, dtype=np.float64)
    assert gpu.shape == ref.shape, (gpu.shape, ref.shape)
    bound = LIPSCHITZ[act] * REL_TOL * scale
    if act != 0:
        bound = bound + 1e-5 * np.abs(ref)
    if out_type == gi.OUT_F16:
        bound = bound + ulp16(ref)
    elif out_type == gi.OUT_BF16:
        bound = bound + ulpbf16(ref)
    with np.errstate(invalid="ignore"):
        err = np.abs(gpu - ref)
    ok = err <= bound
    inf_gpu = np.isinf(gpu)
    # infinity accepted where the reference (plus the bound) reaches overflow
    if out_type in (gi.OUT_F16, gi.OUT_BF16):
        top = F16_OVERFLOW if out_type == gi.OUT_F16 else BF16_OVERFLOW
        reach = np.abs(ref) + REL_TOL * scale >= top
        ok |= inf_gpu & reach & (np.sign(gpu) == np.sign(ref))
    bad = ~ok
    if bad.any():
        idx = np.argwhere(bad)[:8]
        detail = [(tuple(i), float(gpu[tuple(i)]), float(ref[tuple(i)]),
                   float(bound[tuple(i)])) for i in idx]
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} outside the "
                             f"bound; first (index, gpu, ref, bound): {detail}")
    fin = np.isfinite(gpu) & (bound > 0)
    return float(np.max(err[fin] / bound[fin])) if fin.any() else 0.0


def to_device(case, device="cuda"):
    """Device copies of the case's storage.  An empty operand (K = 0) gets a
    small zero buffer instead: run() requires non-NULL A and B whenever
    M * N > 0, and a zero-size tensor has no address."""
    dev = lambda t: t.to(device) if t.numel() else torch.zeros(8, dtype=t.dtype, device=device)
    return (dev(case.A), dev(case.B), case.C.to(device))


def run_case(case, dA=None, dB=None, dC=None, stream=None, alpha=None, beta=None,
             bias=None, act=0):
    """Runs a gemm_inputs.Case through the C ABI; returns the device C.
    bias (a device float32 tensor) and act set the fused epilogue."""
    if dA is None:
        dA, dB, dC = to_device(case)
    p = mpg.Plan(case.M, case.N, case.K, case.layout_a, case.layout_b,
                 case.out_type, case.lda, case.ldb, case.ldc, case.batch,
                 case.stride_a, case.stride_b, case.stride_c, dtype=in_dtype(case))
    try:
        if bias is not None or act != 0:
            p.set_epilogue(bias, act)
        p.run(dA, dB, dC, case.alpha if alpha is None else alpha,
              case.beta if beta is None else beta, stream=stream)
    finally:
        p.close()
    return dC


def in_dtype(case):
    return case.meta.get("in_dtype", "f16")


def c_logical(case, C_flat, rows=None):
    """(batch, rows, N) float64 view of a flat C storage (CPU tensor)."""
    C = C_flat.reshape(case.batch, case.M, case.ldc)[:, :, :case.N]
    if rows is not None:
        C = C[:, rows, :]
    return C.to(torch.float64).numpy()


def oracle_for(case, rows=None, bias=None, act=0):
    A = case.A.view(torch.int16).numpy().view(np.uint16)
    B = case.B.view(torch.int16).numpy().view(np.uint16)
    if case.out_type in (gi.OUT_F16, gi.OUT_BF16):
        C = case.C.view(torch.int16).numpy().view(np.uint16)
    else:
        C = case.C.numpy()
    return oracle.gemm(case.M, case.N, case.K, A, B, C, alpha=case.alpha,
                       beta=case.beta, layout_a=case.layout_a,
                       layout_b=case.layout_b, out_type=case.out_type,
                       in_type=oracle.IN_BF16 if in_dtype(case) == "bf16" else oracle.IN_F16,
                       lda=case.lda, ldb=case.ldb, ldc=case.ldc,
                       batch=case.batch, stride_a=case.stride_a,
                       stride_b=case.stride_b, stride_c=case.stride_c,
                       bias=None if bias is None else bias.cpu().numpy()[:case.N], activation=act,
                       rows=rows, nthreads=oracle_threads())


def sample_rows(M, n_random=192, seed=0, tiles=(256, 128, 64, 32)):
    """First and last rows, rows on and next to tile boundaries, and seeded
    random rows (sorted, unique)."""
    rows = {0, M - 1}
    for t in tiles:
        for base in range(t, M, t * 7):
            rows.update(r for r in (base - 1, base, base + 1) if 0 <= r < M)
    rng = np.random.default_rng(seed)
    rows.update(rng.integers(0, M, size=min(n_random, M)).tolist())
    return np.array(sorted(rows), dtype=np.int64)


def parity(case, rows=None, what=""):
    """Runs the case on the GPU and checks it against the oracle."""
    dC = run_case(case)
    torch.cuda.synchronize()
    got = c_logical(case, dC.cpu(), rows)
    ref, scale = oracle_for(case, rows)
    return check_bound(got, ref, scale, case.out_type, what)
