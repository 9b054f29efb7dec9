"""Seeded synthetic operands for the GEMM workloads (shared by tests and bench).

This module only draws numbers and lays them out in storage; it holds none of
the GEMM arithmetic, so both the GPU path's tests and the CPU oracle can take
their inputs from it without sharing any computation.

Recipe (the same on every machine): a CPU torch.Generator seeded with `seed`,
operands drawn in the order A, B, then C (C only when it is read), each in its
full storage shape (padding columns of an `ld` larger than the logical extent
are drawn too), in fp32, then rounded to fp16 (RNE) for A, B and fp16 C --
or to bfloat16 (RNE) for bf16 A, B and C (in_dtype "bf16").
  uniform   : rand * 2 - 1            (uniform on [-1, 1) before rounding)
  normal    : randn * sigma           (sigma is the standard deviation)
  integer   : randint(lo, hi + 1)     (exact in fp16 for |v| <= 2048)
"""
from dataclasses import dataclass, field
from typing import Optional

import torch

ROW_MAJOR, COL_MAJOR = 0, 1
OUT_F16, OUT_F32, OUT_BF16 = 0, 1, 2
_IN_DTYPES = {"f16": torch.float16, "bf16": torch.bfloat16}
_OUT_DTYPES = {OUT_F16: torch.float16, OUT_F32: torch.float32, OUT_BF16: torch.bfloat16}


@dataclass
class Case:
    M: int
    N: int
    K: int
    layout_a: int
    layout_b: int
    out_type: int
    lda: int
    ldb: int
    ldc: int
    batch: int
    stride_a: int
    stride_b: int
    stride_c: int
    alpha: float
    beta: float
    A: torch.Tensor          # flat fp16 (or bf16) storage, batch * stride_a elements
    B: torch.Tensor          # flat fp16 (or bf16) storage
    C: torch.Tensor          # flat fp16 / bf16 / fp32 storage (initial contents)
    meta: dict = field(default_factory=dict)


def _draw(g, n, dist, dtype, sigma, lo, hi):
    if dist == "uniform":
        v = torch.rand(n, generator=g, dtype=torch.float32) * 2 - 1
    elif dist == "normal":
        v = torch.randn(n, generator=g, dtype=torch.float32) * sigma
    elif dist == "integer":
        v = torch.randint(lo, hi + 1, (n,), generator=g).to(torch.float32)
    elif dist == "ones":
        v = torch.ones(n, dtype=torch.float32)
    elif dist == "zeros":
        v = torch.zeros(n, dtype=torch.float32)
    else:
        raise ValueError(dist)
    return v.to(dtype)


def make_case(M, N, K, *, layout_a=ROW_MAJOR, layout_b=ROW_MAJOR,
              out_type=OUT_F16, alpha=1.0, beta=0.0, batch=1,
              lda=None, ldb=None, ldc=None, seed=0,
              dist_a="uniform", dist_b="uniform", dist_c="uniform",
              sigma_a=1.0, sigma_b=1.0, sigma_c=1.0,
              int_range=(-3, 3), c_int_range=(-8, 8),
              draw_c: Optional[bool] = None, in_dtype: str = "f16") -> Case:
    """Draws one seeded case; see the module docstring for the recipe.
    in_dtype "f16" or "bf16" (then out_type is OUT_BF16 or OUT_F32)."""
    idt = _IN_DTYPES[in_dtype]
    if in_dtype == "bf16" and out_type == OUT_F16 or in_dtype == "f16" and out_type == OUT_BF16:
        raise ValueError("a 16-bit C has the type of the inputs")
    lda = lda if lda is not None else (K if layout_a == ROW_MAJOR else M)
    ldb = ldb if ldb is not None else (N if layout_b == ROW_MAJOR else K)
    ldc = ldc if ldc is not None else N
    rows_a = M if layout_a == ROW_MAJOR else K
    rows_b = K if layout_b == ROW_MAJOR else N
    sa, sb, sc = rows_a * lda, rows_b * ldb, M * ldc
    g = torch.Generator("cpu").manual_seed(seed)
    A = _draw(g, batch * sa, dist_a, idt, sigma_a, *int_range)
    B = _draw(g, batch * sb, dist_b, idt, sigma_b, *int_range)
    cdt = _OUT_DTYPES[out_type]
    if draw_c is None:
        draw_c = beta != 0.0
    if draw_c:
        C = _draw(g, batch * sc, dist_c, cdt, sigma_c, *c_int_range)
    else:
        C = torch.zeros(batch * sc, dtype=cdt)
    return Case(M, N, K, layout_a, layout_b, out_type, lda, ldb, ldc, batch,
                sa, sb, sc, float(alpha), float(beta), A, B, C,
                meta={"in_dtype": in_dtype})


def headline_case(n: int = 8192, layout_b: int = ROW_MAJOR, seed: int = 0,
                  in_dtype: str = "f16") -> Case:
    """Square compute-bound workload: M = N = K = n, A, B and C uniform
    [-1, 1) fp16 (or bf16), alpha = beta = 1, 16-bit output of the input
    type; NN (B row-major) or NT (B column-major)."""
    return make_case(n, n, n, layout_b=layout_b, alpha=1.0, beta=1.0, seed=seed,
                     in_dtype=in_dtype,
                     out_type=OUT_BF16 if in_dtype == "bf16" else OUT_F16)


def linear_case(M: int, N: int, K: int = 4096, seed: int = 0, in_dtype: str = "f16") -> Case:
    """Transformer linear layer: X (M x K) ~ N(0, 1), W stored N x K
    (column-major B) ~ N(0, 0.02), beta = 0, 16-bit output of the input type."""
    return make_case(M, N, K, layout_b=COL_MAJOR, dist_a="normal",
                     dist_b="normal", sigma_a=1.0, sigma_b=0.02, seed=seed,
                     in_dtype=in_dtype, out_type=OUT_BF16 if in_dtype == "bf16" else OUT_F16)


def batched_case(kind: str, seed: int = 0) -> Case:
    """Batched small products, values N(0,1)/8, fp32 output, beta = 0.
    kind 'sq64': 512 x (64x64 @ 64x64), NN.
    kind 'qk':   256 x (Q 128x64 @ K^T), K stored 128 x 64 (column-major B)."""
    if kind == "sq64":
        return make_case(64, 64, 64, batch=512, out_type=OUT_F32,
                         dist_a="normal", dist_b="normal",
                         sigma_a=0.125, sigma_b=0.125, seed=seed)
    if kind == "qk":
        return make_case(128, 128, 64, batch=256, layout_b=COL_MAJOR,
                         out_type=OUT_F32, dist_a="normal", dist_b="normal",
                         sigma_a=0.125, sigma_b=0.125, seed=seed)
    raise ValueError(kind)
