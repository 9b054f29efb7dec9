"""GPU parity of the bfloat16-input GEMM against the CPU oracle, through the
C ABI (gemm_bf16f32_plan / gemm_bf16f32_run).

The bfloat16 path runs the same kernels as the fp16 one with the _bf16 MFMAs
and a bfloat16 C, so these tests walk the same kernel families -- the 256
tile, the 128 tile on its two- and four-slot rings, split-K, the four
streaming tiles, the staged tiles (128-bit and element-wide loads) and the
repacking copy -- over all four layouts, bf16 and fp32 C, and batches; on
every element for shapes the oracle finishes in seconds, on sampled rows at
full size.  Bound: tests/parity.py (2e-3 of the error scale plus half a
bfloat16 ulp for a bfloat16 C).
"""
import numpy as np
import pytest
import torch

import gemm_inputs as gi
import mixed_precision_gemm_amd as mpg
from gemm_inputs import COL_MAJOR, OUT_BF16, OUT_F32, ROW_MAJOR
from parity import c_logical, check_bound, oracle_for, parity, run_case, sample_rows

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

LAYOUTS = [(ROW_MAJOR, ROW_MAJOR), (ROW_MAJOR, COL_MAJOR),
           (COL_MAJOR, ROW_MAJOR), (COL_MAJOR, COL_MAJOR)]
LNAME = {(0, 0): "NN", (0, 1): "NT", (1, 0): "TN", (1, 1): "TT"}


def bf16_case(M, N, K, **kw):
    kw.setdefault("out_type", OUT_BF16)
    return gi.make_case(M, N, K, in_dtype="bf16", **kw)


def kernel_of(case):
    with mpg.Plan(case.M, case.N, case.K, case.layout_a, case.layout_b, case.out_type,
                  case.lda, case.ldb, case.ldc, case.batch, case.stride_a, case.stride_b,
                  case.stride_c, dtype="bf16") as p:
        return p.kernel


# (shape, expected tile prefix, sampled rows?)
TILE_CASES = [
    ((1000, 1000, 1000), "gemm_bf16_128x128x64m16d4", False),   # four-slot ring, K tail
    ((2304, 2304, 328), "gemm_bf16_128x128x64m16_", False),     # two-slot split ring
    ((4096, 4096, 392), "gemm_bf16_256x256x64m16_", True),      # 256 tile, K tail
]


@pytest.mark.parametrize("la,lb", LAYOUTS)
@pytest.mark.parametrize("shape,prefix,sampled", TILE_CASES)
def test_bf16_direct_tiles_all_layouts(shape, prefix, sampled, la, lb):
    M, N, K = shape
    out = OUT_BF16 if (la + lb) % 2 == 0 else OUT_F32
    case = bf16_case(M, N, K, layout_a=la, layout_b=lb, out_type=out, alpha=-0.5,
                     beta=1.0, seed=11 + la + 2 * lb)
    assert kernel_of(case).startswith(prefix), kernel_of(case)
    rows = sample_rows(M, n_random=64) if sampled else None
    parity(case, rows=rows, what=f"bf16 {shape} {LNAME[(la, lb)]}")


@pytest.mark.parametrize("lb", [ROW_MAJOR, COL_MAJOR])
def test_bf16_headline_sampled(lb):
    """M = N = K = 8192, beta = 1, bf16 C, sampled rows."""
    case = gi.headline_case(8192, layout_b=lb, in_dtype="bf16")
    assert kernel_of(case).startswith("gemm_bf16_256x256")
    parity(case, rows=sample_rows(8192), what=f"bf16 8192^3 {LNAME[(0, lb)]}")


@pytest.mark.parametrize("M,N,tile", [
    (16, 4096, "stream16x16"), (32, 4096, "stream32x16"), (32, 11008, "stream32x48"),
    (64, 4096, "stream32x64"), (128, 4096, "stream32x64"), (64, 11008, "128x128x64m16d4"),
    (128, 11008, "128x128x64m16d4"),
    (2048, 4096, "128x128x64m16_"),
])
def test_bf16_linear_layer_shapes(M, N, tile):
    """Transformer linear shapes (K = 4096, W stored N x K): the streaming
    kernels, split-K and the two-slot 128 tile."""
    case = gi.linear_case(M, N, in_dtype="bf16")
    assert kernel_of(case).startswith("gemm_bf16_" + tile), kernel_of(case)
    rows = None if M <= 128 else sample_rows(M, n_random=96)
    parity(case, rows=rows, what=f"bf16 linear M={M} N={N}")


@pytest.mark.parametrize("shape,kw,suffix", [
    ((127, 257, 33), {}, "narrow"),                                      # staged, element-wide
    ((64, 96, 200), {}, "vec16"),                                        # staged, 128-bit
    ((4097, 63, 1025), {}, "_pkab"),                                     # repack + split-K
    ((7, 4097, 4099), dict(layout_b=COL_MAJOR), "_pkab"),                # streaming on copies
    ((50, 333, 4100), {}, "_sk8_pkab"),
    ((256, 256, 32768), {}, "_sk8"),                                     # deep split-K
    ((16, 4096, 4096), {}, "_sk8"),
])
def test_bf16_small_ragged_and_split(shape, kw, suffix):
    M, N, K = shape
    case = bf16_case(M, N, K, beta=1.0, seed=21, **kw)
    assert suffix in kernel_of(case), kernel_of(case)
    parity(case, what=f"bf16 {shape}")


@pytest.mark.parametrize("kind", ["sq64", "qk"])
def test_bf16_batched_fp32_out(kind):
    """512 x (64 x 64 @ 64 x 64) and 256 x (Q 128 x 64 @ K^T), values
    N(0, 1) / 8, fp32 C."""
    if kind == "sq64":
        case = bf16_case(64, 64, 64, batch=512, out_type=OUT_F32, dist_a="normal",
                         dist_b="normal", sigma_a=0.125, sigma_b=0.125, seed=31)
    else:
        case = bf16_case(128, 128, 64, batch=256, layout_b=COL_MAJOR, out_type=OUT_F32,
                         dist_a="normal", dist_b="normal", sigma_a=0.125, sigma_b=0.125,
                         seed=32)
    parity(case, what=f"bf16 batched {kind}")


@pytest.mark.parametrize("shape", [(512, 512, 512), (40, 4096, 1024)])
def test_bf16_range_beyond_fp16(shape):
    """Magnitudes fp16 cannot hold (|a|, |b| ~ 1e4, products ~ 1e8, sums
    ~ 1e9-1e10; and |a|, |b| ~ 1e-12, below fp16's smallest subnormal, with
    products ~ 1e-24): bfloat16 keeps fp32's exponent range and the result
    stays within the bound."""
    M, N, K = shape
    big = bf16_case(M, N, K, layout_b=COL_MAJOR, dist_a="normal", dist_b="normal",
                    sigma_a=1e4, sigma_b=1e4, seed=41)
    parity(big, what=f"bf16 large values {shape}")
    tiny = bf16_case(M, N, K, layout_b=COL_MAJOR, dist_a="normal", dist_b="normal",
                     sigma_a=1e-12, sigma_b=1e-12, out_type=OUT_F32, seed=42)
    parity(tiny, what=f"bf16 tiny values {shape}")


@pytest.mark.parametrize("shape", [(60, 70, 1000), (512, 384, 1024), (1024, 1024, 768)])
@pytest.mark.parametrize("la,lb", [(ROW_MAJOR, ROW_MAJOR), (COL_MAJOR, COL_MAJOR)])
def test_bf16_integer_inputs_are_exact(shape, la, lb):
    """Small integers are exact in bfloat16 and every partial sum is an
    integer below 2^24: the fp32 C equals the exact product bit for bit."""
    M, N, K = shape
    case = bf16_case(M, N, K, layout_a=la, layout_b=lb, out_type=OUT_F32, beta=1.0,
                     dist_a="integer", dist_b="integer", dist_c="integer", seed=51)
    dC = run_case(case)
    torch.cuda.synchronize()
    got = c_logical(case, dC.cpu())
    ref, _ = oracle_for(case)
    assert np.array_equal(got, ref)


def test_bf16_misaligned_pointers_repack_at_run():
    """A and B one element past a 16-byte boundary on a direct (split-K)
    plan: the run copies them into the plan's buffer first; a misaligned C
    takes the element-wise stores."""
    M, N, K = 640, 512, 1032
    case = bf16_case(M, N, K, beta=1.0, seed=61)
    assert kernel_of(case) == "gemm_bf16_128x128x64m16d4_nn_direct_sk2"
    A = torch.empty(case.A.numel() + 1, dtype=torch.bfloat16, device="cuda")
    B = torch.empty(case.B.numel() + 1, dtype=torch.bfloat16, device="cuda")
    C = torch.empty(case.C.numel() + 1, dtype=torch.bfloat16, device="cuda")
    A[1:].copy_(case.A)
    B[1:].copy_(case.B)
    C[1:].copy_(case.C)
    with mpg.Plan(M, N, K, dtype="bf16") as p:
        for _ in range(2):   # the second run reuses the plan's buffer
            C[1:].copy_(case.C)
            p.run(A[1:], B[1:], C[1:], case.alpha, case.beta)
    torch.cuda.synchronize()
    ref, scale = oracle_for(case)
    check_bound(c_logical(case, C[1:].cpu()), ref, scale, OUT_BF16, "bf16 misaligned")


def test_bf16_torch_wrapper_views():
    """mpg.gemm on bfloat16 tensors: a transposed view of B (column-major)
    and a fresh bf16 C, against the oracle on the same values."""
    M, N, K = 200, 136, 264
    case = bf16_case(M, N, K, layout_b=COL_MAJOR, seed=71)
    A = case.A.reshape(M, K).cuda()
    Bt = case.B.reshape(N, K).cuda()
    C = mpg.gemm(A, Bt.t())
    assert C.dtype == torch.bfloat16 and C.shape == (M, N)
    torch.cuda.synchronize()
    ref, scale = oracle_for(case)
    check_bound(C.cpu().to(torch.float64).numpy()[None], ref, scale, OUT_BF16, "bf16 wrapper")
    with pytest.raises(TypeError):
        mpg.gemm(A, Bt.t().to(torch.float16))


def _bf16_sweep(n, seed):
    from test_gemm_gpu import _sweep_cases
    return _sweep_cases(n, seed)


@pytest.mark.parametrize("case_args", _bf16_sweep(24, 3131))
def test_bf16_random_sweep(case_args):
    """The plain sweep's seeded shapes (every kernel class, random layouts,
    padding, batch, alpha/beta, output type) in bfloat16."""
    M, N, K, la, lb, pad, batch, out_type, alpha, beta = case_args
    lda = (K if la == ROW_MAJOR else M) + pad
    ldb = (N if lb == ROW_MAJOR else K) + pad
    case = bf16_case(M, N, K, layout_a=la, layout_b=lb,
                     out_type=OUT_BF16 if out_type == 0 else OUT_F32, alpha=alpha, beta=beta,
                     batch=batch, lda=lda, ldb=ldb, seed=(M * 7919 + N * 31 + K) % 1000)
    rows = None if M * N * K * batch <= (1 << 27) else sample_rows(M, n_random=16, tiles=(256, 128))
    parity(case, rows=rows, what=f"{kernel_of(case)} {case_args}")


@pytest.mark.parametrize("epilogue", [False, True])
def test_bf16_run_to_run_bitwise_determinism(epilogue):
    """Same plan and inputs: bitwise identical bf16 output on repeated runs
    and on another stream, with and without a fused epilogue (split-K plan)."""
    case = bf16_case(256, 384, 8192, beta=1.0, seed=17)
    assert "_sk" in kernel_of(case)
    dA, dB, dC0 = case.A.cuda(), case.B.cuda(), case.C.cuda()
    bias = torch.linspace(-1, 1, case.N, device="cuda")
    s2 = torch.cuda.Stream()
    outs = []
    with mpg.Plan(case.M, case.N, case.K, dtype="bf16") as p:
        if epilogue:
            p.set_epilogue(bias, mpg.GEMM_ACT_GELU)
        for stream in (None, None, s2):
            dC = dC0.clone()
            torch.cuda.synchronize()
            p.run(dA, dB, dC, 1.0, 1.0, stream=stream)
            torch.cuda.synchronize()
            outs.append(dC.cpu().view(torch.int16))
    assert torch.equal(outs[0], outs[1]) and torch.equal(outs[0], outs[2])
