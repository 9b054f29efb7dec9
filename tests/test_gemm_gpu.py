"""GPU parity of the HIP GEMM against the CPU oracle, through the C ABI.

Each test draws seeded inputs (gemm_inputs), runs the library's kernel on
cuda:0, and compares with the oracle element by element under the acceptance
bound of tests/parity.py -- on every element for shapes the oracle finishes
in seconds, on sampled rows (first, last, tile boundaries, random) at the full
workload sizes.  Cases whose exact result is representable are compared bit
for bit.
"""
import numpy as np
import pytest
import torch

import gemm_inputs as gi
import mixed_precision_gemm_amd as mpg
from gemm_inputs import COL_MAJOR, OUT_BF16, OUT_F16, OUT_F32, ROW_MAJOR
from parity import (c_logical, check_bound, in_dtype, oracle_for, parity, run_case,
                    sample_rows, to_device)

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

LAYOUTS = [(ROW_MAJOR, ROW_MAJOR), (ROW_MAJOR, COL_MAJOR),
           (COL_MAJOR, ROW_MAJOR), (COL_MAJOR, COL_MAJOR)]
LNAME = {(0, 0): "NN", (0, 1): "NT", (1, 0): "TN", (1, 1): "TT"}


# ------------------------------------------------------------ workloads

def test_square_256_nn():
    """M = N = K = 256, uniform [-1, 1), alpha 1, beta 0, fp16 C."""
    case = gi.make_case(256, 256, 256, seed=0)
    parity(case, what="256^3 NN")


@pytest.mark.parametrize("shape", [(1, 4096, 4096), (1000, 1000, 1000),
                                   (127, 257, 33), (4097, 63, 1025)])
def test_edge_shapes(shape):
    M, N, K = shape
    case = gi.make_case(M, N, K, seed=0)
    parity(case, what=f"edge {shape}")


@pytest.mark.parametrize("la,lb", [(ROW_MAJOR, ROW_MAJOR), (ROW_MAJOR, COL_MAJOR)])
@pytest.mark.parametrize("n", [1024, 2048])
def test_square_beta1_full(n, la, lb):
    case = gi.make_case(n, n, n, layout_a=la, layout_b=lb, alpha=1.0, beta=1.0, seed=0)
    parity(case, what=f"{n}^3 {LNAME[(la, lb)]} beta=1")


@pytest.mark.parametrize("lb", [ROW_MAJOR, COL_MAJOR])
@pytest.mark.parametrize("n", [4096, 8192])
def test_square_beta1_sampled(n, lb):
    """Full-size square GEMMs (the headline size at 8192) on sampled rows."""
    case = gi.headline_case(n, layout_b=lb)
    rows = sample_rows(n)
    parity(case, rows=rows, what=f"{n}^3 {LNAME[(0, lb)]} beta=1 sampled")


@pytest.mark.parametrize("N", [4096, 11008, 12288])
@pytest.mark.parametrize("M", [16, 32, 64, 128, 2048, 8192])
def test_linear_layer_shapes(M, N):
    case = gi.linear_case(M, N)
    rows = None if M <= 128 else sample_rows(M, n_random=96)
    parity(case, rows=rows, what=f"linear M={M} N={N}")


@pytest.mark.parametrize("shape", [(24, 10250, 1000), (5, 10260, 77), (31, 16384, 4104),
                                   (77, 3000, 4104), (33, 130, 200)])
def test_streaming_wide_ragged(shape):
    """The 48- and 64-column streaming workgroups with N off their grid, K off the
    32-deep step, and rows of A past M."""
    M, N, K = shape
    case = gi.make_case(M, N, K, layout_b=COL_MAJOR, alpha=1.5, beta=-1.0, seed=70)
    with mpg.Plan(M, N, K, ROW_MAJOR, COL_MAJOR) as p:
        assert "stream" in p.kernel, p.kernel
    parity(case, what=f"streaming {M}x{N}x{K}")


@pytest.mark.parametrize("shape,kw,frag", [
    ((1, 4096, 4096), {}, "rowvec4x64_nn_direct_sk4"),                    # the edge shape, split
    ((4, 1000, 2048), dict(alpha=-0.75, beta=1.0), "rowvec4x64_nn_direct_sk2"),
    ((3, 200, 77), dict(out_type=OUT_F32, beta=0.5), "rowvec4x64_nn_direct_pka"),   # ragged K
    ((2, 33, 1030), {}, "rowvec4x64_nn_direct_pkab"),                     # ragged N and K, repacked
    ((1, 4104, 8192), dict(batch=3, out_type=OUT_F32), "rowvec4x64_nn_direct_sk2"),  # batched, split
])
def test_row_vector_kernel(shape, kw, frag):
    """M <= 4 with row-major A and B: the row-vector kernel (fp32 FMA dot
    products over B streamed once), unsplit, in K slices, repacked, batched."""
    M, N, K = shape
    kw = dict(kw)
    batch = kw.pop("batch", 1)
    case = gi.make_case(M, N, K, batch=batch, seed=M * 7 + N + K, dist_c="normal", **kw)
    kernel = plan_kernel(case)
    assert frag in kernel, kernel
    parity(case, what=f"row vector {M}x{N}x{K}")


@pytest.mark.parametrize("shape,kw,frag", [
    ((16, 8200, 1024), dict(batch=3, beta=1.0), "stream16x48_nt_direct"),              # batched, ragged N
    ((30, 10300, 640), dict(batch=2, out_type=OUT_F32), "stream32x48_nt_direct"),
    ((100, 1000, 2048), dict(batch=2, alpha=0.5, beta=-1.0), "stream32x64_nt_direct_sk2"),  # row tiles, split
    ((16, 9000, 2048), dict(in_dtype="bf16", out_type=OUT_BF16), "gemm_bf16_stream16x48"),
    ((70, 2048, 4096), dict(in_dtype="bf16", out_type=OUT_BF16, beta=1.0), "gemm_bf16_stream32x64"),
])
def test_streaming_wide_and_row_tiles_batched(shape, kw, frag):
    """The 48-column streaming tiles and the 32 x 64 tile in several row tiles
    over batch items (each item's blocks on their own descriptors), and in
    bfloat16."""
    M, N, K = shape
    kw = dict(kw)
    batch = kw.pop("batch", 1)
    case = gi.make_case(M, N, K, layout_b=COL_MAJOR, batch=batch, seed=M + N + K + 5,
                        dist_c="normal", **kw)
    with mpg.Plan(case.M, case.N, case.K, case.layout_a, case.layout_b, case.out_type,
                  case.lda, case.ldb, case.ldc, case.batch, case.stride_a, case.stride_b,
                  case.stride_c, dtype=in_dtype(case)) as p:
        kernel = p.kernel
    assert frag in kernel, kernel
    rows = sample_rows(M, n_random=32) if M > 64 else None
    parity(case, rows=rows, what=f"streaming {M}x{N}x{K} batch {batch}")


@pytest.mark.parametrize("M", [1, 4])
def test_row_vector_bit_exact_and_repeatable(M):
    """Integer inputs: exact in fp32 in any summation order; two runs give the
    same bits (the split-K slices are summed in slice order)."""
    case = gi.make_case(M, 4096, 4096, out_type=OUT_F32, dist_a="integer", dist_b="integer",
                        int_range=(-8, 8), seed=11)
    kernel = plan_kernel(case)
    assert "rowvec" in kernel and "_sk" in kernel, kernel
    d1 = run_case(case)
    d2 = run_case(case)
    ref, _ = oracle_for(case)
    assert np.array_equal(c_logical(case, d1.cpu()), ref), kernel
    assert torch.equal(d1, d2)


@pytest.mark.parametrize("shape,kw", [
    ((64, 64, 64), dict(batch=512, out_type=OUT_F32)),                        # the batched workload
    ((37, 40, 24), dict(batch=5, beta=1.0)),                                  # ragged M, N, K
    ((64, 64, 64), dict(batch=3, alpha=-0.5, beta=0.5)),                      # fp16 C, alpha, beta
    ((5, 8, 8), dict(batch=2, out_type=OUT_F32)),                             # smallest rows
    ((64, 64, 64), dict(batch=4, in_dtype="bf16", out_type=OUT_BF16, beta=1.0)),
    ((64, 48, 64), dict(batch=6, lda=72, ldb=56)),                            # padded rows
])
def test_small_batched_kernel(shape, kw):
    """Batched products of at most 64 x 64 x 64 with row-major A and B: one
    wave per product (A's fragments from global memory, B transposed out of
    LDS, C^T accumulated)."""
    M, N, K = shape
    kw = dict(kw)
    batch = kw.pop("batch")
    case = gi.make_case(M, N, K, batch=batch, seed=M * 3 + N + K + batch, dist_c="normal", **kw)
    with mpg.Plan(case.M, case.N, case.K, case.layout_a, case.layout_b, case.out_type,
                  case.lda, case.ldb, case.ldc, case.batch, case.stride_a, case.stride_b,
                  case.stride_c, dtype=in_dtype(case)) as p:
        assert "small64_nn_direct" in p.kernel, p.kernel
    parity(case, what=f"small batched {M}x{N}x{K} x {batch}")


def test_small_batched_writes_stay_inside_c_and_skip_nan_c():
    """One wave per product with C's rows padded (ldc > N) and a gap between
    batch items: sentinels outside the logical C survive; with beta = 0 a
    NaN-filled C is never read."""
    M, N, K, ldc, batch = 40, 56, 64, 72, 3
    stride_c = (M + 2) * ldc
    case = gi.make_case(M, N, K, batch=batch, out_type=OUT_F32, seed=13)
    sentinel = -1234.0
    C = torch.full((batch * stride_c,), float("nan"), dtype=torch.float32, device="cuda")
    Cv = C.view(batch, M + 2, ldc)
    Cv[:, :, N:] = sentinel
    Cv[:, M:, :] = sentinel
    with mpg.Plan(M, N, K, ROW_MAJOR, ROW_MAJOR, OUT_F32, case.lda, case.ldb, ldc, batch,
                  case.stride_a, case.stride_b, stride_c) as p:
        assert "small64" in p.kernel, p.kernel
        p.run(case.A.cuda(), case.B.cuda(), C, 1.0, 0.0)
    torch.cuda.synchronize()
    Cv = C.cpu().view(batch, M + 2, ldc)
    assert torch.all(Cv[:, :, N:] == sentinel) and torch.all(Cv[:, M:, :] == sentinel)
    got = Cv[:, :M, :N].double().numpy()
    ref, scale = oracle_for(case)
    assert not np.isnan(got).any()
    check_bound(got, ref, scale, OUT_F32, "small batched, padded C")


def test_small_batched_bit_exact_and_misaligned_fallback():
    """Integer inputs give exact fp32 sums (fragment layouts and the
    transposed B read pinned bit for bit); an A at an odd address takes the
    staged tile's element loads instead, with the same result."""
    case = gi.make_case(64, 64, 64, batch=8, out_type=OUT_F32, dist_a="integer",
                        dist_b="integer", int_range=(-8, 8), seed=12)
    assert "small64" in plan_kernel(case)
    ref, _ = oracle_for(case)
    dC = run_case(case)
    assert np.array_equal(c_logical(case, dC.cpu()), ref)
    A = torch.zeros(case.A.numel() + 1, dtype=torch.float16, device="cuda")
    A[1:] = case.A.cuda()
    B, C = case.B.cuda(), case.C.cuda()
    run_case(case, A[1:], B, C)
    assert np.array_equal(c_logical(case, C.cpu()), ref)


@pytest.mark.parametrize("kind", ["sq64", "qk"])
def test_batched_small(kind):
    case = gi.batched_case(kind)
    parity(case, what=f"batched {kind}")


@pytest.mark.parametrize("la,lb", LAYOUTS)
@pytest.mark.parametrize("shape,tile", [((4000, 4104, 1000), "256x256"),
                                        ((1000, 1000, 1000), "128x128")])
def test_large_tiles_ragged_all_layouts(shape, tile, la, lb):
    """The two large direct tiles with M, N and K all off the tile grid (K
    tail of 40 in the last 64-deep stage) in every layout, beta != 0; the
    row lengths stay multiples of 8 so that the direct path is taken."""
    M, N, K = shape
    case = gi.make_case(M, N, K, layout_a=la, layout_b=lb, alpha=-0.5, beta=2.0,
                        seed=21)
    p = mpg.Plan(M, N, K, la, lb, OUT_F16, case.lda, case.ldb, case.ldc)
    kernel = p.kernel
    p.close()
    assert tile in kernel, kernel
    rows = sample_rows(M, n_random=64) if M > 1000 else None
    parity(case, rows=rows, what=f"{kernel} {M}x{N}x{K}")


# ------------------------------------------------------- whole 256 tiles

@pytest.mark.parametrize("out_type", [OUT_F16, OUT_F32])
@pytest.mark.parametrize("la,lb", LAYOUTS)
def test_tile256_odd_stage_count_all_layouts(la, lb, out_type):
    """512 whole 256 x 256 tiles (two per CU) with an odd number of 64-deep
    stages (K = 320: A's three-slot ring wraps mid-sequence, B's last stage
    sits in slot 0), alpha and beta != 0; sampled rows."""
    M, N, K = 4096, 8192, 320
    case = gi.make_case(M, N, K, layout_a=la, layout_b=lb, out_type=out_type,
                        alpha=1.5, beta=-0.5, seed=80)
    kernel = plan_kernel(case)
    assert "256x256" in kernel, kernel
    parity(case, rows=sample_rows(M, n_random=48), what=f"{kernel} {M}x{N}x{K}")


def test_tile256_uneven_grid():
    """544 tiles of 256 (not a multiple of the CU count), K = 384."""
    M, N, K = 8192, 4352, 384
    case = gi.make_case(M, N, K, beta=1.0, seed=81)
    kernel = plan_kernel(case)
    assert "256x256" in kernel, kernel
    parity(case, rows=sample_rows(M, n_random=64), what=f"{kernel} {M}x{N}x{K}")


@pytest.mark.parametrize("lb", [ROW_MAJOR, COL_MAJOR])
def test_tile128_single_stage(lb):
    """Shallow K on the two-slot 128 tile: one 64-deep stage (K = 64) and a
    stage tail (K = 40), 2176 tiles."""
    for K in (64, 40):
        M, N = 8192, 4352
        case = gi.make_case(M, N, K, layout_b=lb, beta=1.0, seed=84)
        kernel = plan_kernel(case)
        assert "128x128x64m16_" in kernel, kernel
        parity(case, rows=sample_rows(M, n_random=48), what=f"{kernel} {M}x{N}x{K}")


def test_tile256_batched():
    """Strided batch of 8 products of 2048^2 x 320 on the 256 tile, fp32 C."""
    M, N, K, batch = 2048, 2048, 320, 8
    case = gi.make_case(M, N, K, batch=batch, out_type=OUT_F32, beta=2.0, seed=82)
    kernel = plan_kernel(case)
    assert "256x256" in kernel, kernel
    rows = sample_rows(M, n_random=24)
    dC = run_case(case)
    torch.cuda.synchronize()
    got = c_logical(case, dC.cpu(), rows)
    ref, scale = oracle_for(case, rows)
    check_bound(got, ref, scale, OUT_F32, f"{kernel} batch {batch}")


def test_tile256_misaligned_c():
    """The 256 tile with a C pointer that only allows element-wide access."""
    M, N, K = 4096, 8192, 384
    case = gi.make_case(M, N, K, beta=1.0, seed=83)
    assert "256x256" in plan_kernel(case)
    C = torch.zeros(case.C.numel() + 1, dtype=torch.float16, device="cuda")
    C[1:] = case.C.cuda()
    A, B = case.A.cuda(), case.B.cuda()
    run_case(case, A, B, C[1:])
    rows = sample_rows(M, n_random=32)
    ref, scale = oracle_for(case, rows)
    check_bound(c_logical(case, C[1:].cpu(), rows), ref, scale, OUT_F16, "misaligned C")


# ----------------------------------------------------- layouts and types

SWEEP = [(1, 1, 1), (2, 3, 5), (8, 8, 8), (31, 33, 17), (32, 64, 64),
         (33, 65, 63), (64, 64, 128), (65, 127, 129), (100, 36, 72),
         (129, 255, 200), (257, 129, 96), (300, 300, 65)]


@pytest.mark.parametrize("out_type", [OUT_F16, OUT_F32])
@pytest.mark.parametrize("la,lb", LAYOUTS)
def test_layout_sweep(la, lb, out_type):
    for i, (M, N, K) in enumerate(SWEEP):
        for alpha, beta in ((1.0, 0.0), (-0.5, 2.0)):
            case = gi.make_case(M, N, K, layout_a=la, layout_b=lb,
                                out_type=out_type, alpha=alpha, beta=beta,
                                seed=100 + i)
            parity(case, what=f"{LNAME[(la, lb)]} out={out_type} {M}x{N}x{K} a={alpha} b={beta}")


@pytest.mark.parametrize("la,lb", LAYOUTS)
def test_padded_leading_dims_and_batch(la, lb):
    for M, N, K in [(40, 48, 56), (37, 41, 43), (256, 64, 96)]:
        lda = (K if la == ROW_MAJOR else M) + 8
        ldb = (N if lb == ROW_MAJOR else K) + 16
        ldc = N + 8
        case = gi.make_case(M, N, K, layout_a=la, layout_b=lb, lda=lda, ldb=ldb,
                            ldc=ldc, batch=3, beta=1.0, seed=7)
        parity(case, what=f"padded {LNAME[(la, lb)]} {M}x{N}x{K}")


# --------------------------------------------------------- exact cases

@pytest.mark.parametrize("la,lb", LAYOUTS)
def test_integer_inputs_bit_exact_f16(la, lb):
    """A, B in {-3..3}, K <= 113, C in {-8..8}, beta = 1: every partial sum is
    an integer below 2^11, so the fp16 result is exact in any order."""
    for M, N, K in [(64, 64, 64), (200, 136, 113), (33, 47, 100)]:
        case = gi.make_case(M, N, K, layout_a=la, layout_b=lb, beta=1.0,
                            dist_a="integer", dist_b="integer", dist_c="integer",
                            seed=3)
        dC = run_case(case)
        got = c_logical(case, dC.cpu())
        ref, _ = oracle_for(case)
        assert np.array_equal(got, ref), (M, N, K)


@pytest.mark.parametrize("la,lb", [(ROW_MAJOR, ROW_MAJOR), (ROW_MAJOR, COL_MAJOR)])
def test_integer_inputs_bit_exact_f32(la, lb):
    """A, B in {-8..8}, K = 4096: |C| <= 262144 < 2^24, exact in fp32."""
    case = gi.make_case(512, 512, 4096, layout_a=la, layout_b=lb, out_type=OUT_F32,
                        dist_a="integer", dist_b="integer", int_range=(-8, 8), seed=4)
    dC = run_case(case)
    got = c_logical(case, dC.cpu())
    ref, _ = oracle_for(case)
    assert np.array_equal(got, ref)


# The headline kernels bit for bit.  Integer A, B in {-8..8} and C in
# {-64..64} with K <= 4104 keep every partial sum an integer below 2^24, so
# an fp32 C is exact in any summation order: a missing, repeated or
# misplaced K term, row or column anywhere in a stage, its tail or the
# epilogue changes the bits.
EXACT_KERNELS = [
    ((4096, 4096, 4104), "gemm_256x256x64m16_", True),    # 256 tile, ragged K (K tests)
    ((4096, 4096, 4096), "gemm_256x256x64m16_", True),    # 256 tile, K-full variant
    ((3072, 3072, 1000), "gemm_128x128x64m16_", True),    # 128 tile, two slots, no split
    ((1000, 1000, 1000), "gemm_128x128x64m16d4_", False),  # 128 tile, four slots
]


@pytest.mark.parametrize("shape,prefix,sampled", EXACT_KERNELS)
@pytest.mark.parametrize("la,lb", LAYOUTS)
def test_integer_inputs_bit_exact_direct_tiles(shape, prefix, sampled, la, lb):
    M, N, K = shape
    case = gi.make_case(M, N, K, layout_a=la, layout_b=lb, out_type=OUT_F32, alpha=1.0,
                        beta=1.0, dist_a="integer", dist_b="integer", dist_c="integer",
                        int_range=(-8, 8), c_int_range=(-64, 64), seed=6)
    kernel = plan_kernel(case)
    assert kernel.startswith(prefix) and "_sk" not in kernel and "_pk" not in kernel, kernel
    dC = run_case(case)
    rows = sample_rows(M, n_random=48) if sampled else None
    got = c_logical(case, dC.cpu(), rows)
    ref, _ = oracle_for(case, rows)
    bad = np.argwhere(got != ref)
    assert bad.size == 0, f"{kernel}: {len(bad)} inexact, first {bad[:4].tolist()}"


@pytest.mark.parametrize("M,N", [(16, 4096), (32, 11008), (64, 4096), (16, 11008), (16, 8192),
                                 (27, 8200), (128, 4096), (100, 2048), (48, 512)])
def test_integer_inputs_bit_exact_streaming(M, N):
    """Every streaming form: 16, 48 and 64 columns, A staged through LDS (M
    <= 16) or loaded into registers, unsplit and in K slices (27 x 8200, 100
    x 2048), several 32-row tiles (128, 100 and 48 rows); integer sums stay
    below 2^24, exact in fp32 in any order."""
    case = gi.make_case(M, N, 4096, layout_b=COL_MAJOR, out_type=OUT_F32,
                        dist_a="integer", dist_b="integer", int_range=(-8, 8), seed=7)
    kernel = plan_kernel(case)
    assert kernel.startswith("gemm_stream"), kernel
    dC = run_case(case)
    ref, _ = oracle_for(case)
    assert np.array_equal(c_logical(case, dC.cpu()), ref), kernel


@pytest.mark.parametrize("la,lb", LAYOUTS)
@pytest.mark.parametrize("side", ["A", "B"])
def test_one_hot_permutation_on_the_256_tile(la, lb, side):
    """A (or B) is a permutation matrix, the other operand holds distinct
    integers: C is the other operand with its rows (columns) permuted, bit
    for bit, on all 16.8 M outputs of the 256 tile's 16 x 16 x 32 fragments
    (every lane, register, fragment and K step of the fragment maps)."""
    n = 4096
    perm = (torch.arange(n) * 1237 + 91) % n                      # a permutation (1237 odd)
    vals = ((torch.arange(n)[:, None] * 31 + torch.arange(n)[None, :] * 17) % 2001 - 1000).half()
    P = torch.zeros(n, n, dtype=torch.float16)
    if side == "A":
        P[torch.arange(n), perm] = 1.0          # C[i, :] = vals[perm[i], :]
        Am, Bm, want = P, vals, vals[perm, :]
    else:
        P[perm, torch.arange(n)] = 1.0          # C[:, j] = vals[:, perm[j]]
        Am, Bm, want = vals, P, vals[:, perm]
    A = Am if la == ROW_MAJOR else Am.t().contiguous()
    B = Bm if lb == ROW_MAJOR else Bm.t().contiguous()
    C = torch.full((n, n), 7.0, dtype=torch.float16, device="cuda")
    with mpg.Plan(n, n, n, la, lb, OUT_F16, n, n, n) as p:
        assert p.kernel.startswith("gemm_256x256x64m16_"), p.kernel
        p.run(A.cuda(), B.cuda(), C)
    torch.cuda.synchronize()
    got = C.cpu()
    bad = (got != want).nonzero()
    assert bad.numel() == 0, f"{LNAME[(la, lb)]} {side}: {bad.shape[0]} wrong, first {bad[:4].tolist()}"


@pytest.mark.parametrize("K", [1, 7, 64, 2048, 4097])
def test_all_ones_gives_K(K):
    case = gi.make_case(96, 80, K, dist_a="ones", dist_b="ones", seed=0)
    dC = run_case(case)
    got = dC.cpu().reshape(96, 80)
    want = torch.full((96, 80), float(K), dtype=torch.float16)   # RNE of K
    assert torch.equal(got, want)


@pytest.mark.parametrize("la,lb", LAYOUTS)
def test_identity_returns_other_operand(la, lb):
    n, N = 160, 72
    g = torch.Generator().manual_seed(5)
    Bm = (torch.rand(n, N, generator=g) * 2 - 1).half()
    eye = torch.eye(n, dtype=torch.float16)
    A = eye if la == ROW_MAJOR else eye.t().contiguous()
    B = Bm if lb == ROW_MAJOR else Bm.t().contiguous()
    lda = n
    ldb = N if lb == ROW_MAJOR else n
    C = torch.zeros(n, N, dtype=torch.float16, device="cuda")
    with mpg.Plan(n, N, n, la, lb, OUT_F16, lda, ldb, N) as p:
        p.run(A.cuda(), B.cuda(), C)
    assert torch.equal(C.cpu(), Bm)


def test_fragment_layout_one_hot():
    """Batch of 32x32x16 products of one-hot matrices: item t has A = e_i e_k^T
    and B = e_k' e_j^T; C must be e_i e_j^T when k == k' and zero otherwise.
    Pins which lane and register of the MFMA fragments hold which (i, j, k)."""
    items = []
    for i in range(32):
        for j in range(32):
            k = (i * 5 + j) % 16
            items.append((i, j, k, k))
            if (i + j) % 8 == 0:
                items.append((i, j, k, (k + 1 + i % 15) % 16))
    T = len(items)
    A = torch.zeros(T, 32, 16, dtype=torch.float16)
    B = torch.zeros(T, 16, 32, dtype=torch.float16)
    for t, (i, j, k, k2) in enumerate(items):
        A[t, i, k] = 1.0
        B[t, k2, j] = 1.0
    C = torch.full((T, 32, 32), 7.0, dtype=torch.float16, device="cuda")
    with mpg.Plan(32, 32, 16, ROW_MAJOR, ROW_MAJOR, OUT_F16, 16, 32, 32, T,
                  32 * 16, 16 * 32, 32 * 32) as p:
        p.run(A.cuda(), B.cuda(), C)
    C = C.cpu()
    for t, (i, j, k, k2) in enumerate(items):
        want = torch.zeros(32, 32, dtype=torch.float16)
        if k == k2:
            want[i, j] = 1.0
        assert torch.equal(C[t], want), (t, i, j, k, k2)


def test_overflow_rounds_to_infinity():
    """|sum| = 2 * 200 * 200 = 80000 >= 65520 -> +-inf in fp16."""
    A = torch.full((64, 2), 200.0, dtype=torch.float16)
    B = torch.full((2, 64), 200.0, dtype=torch.float16)
    B[:, 32:] = -200.0
    C = torch.zeros(64, 64, dtype=torch.float16, device="cuda")
    with mpg.Plan(64, 64, 2, lda=2, ldb=64, ldc=64) as p:
        p.run(A.cuda(), B.cuda(), C)
    C = C.cpu().float()
    assert torch.all(C[:, :32] == float("inf"))
    assert torch.all(C[:, 32:] == float("-inf"))


# ---------------------------------------------- reads and writes respected

@pytest.mark.parametrize("la,lb", LAYOUTS)
def test_nan_in_padding_and_c_not_read_when_beta_zero(la, lb):
    M, N, K = 70, 90, 50
    lda = (K if la == ROW_MAJOR else M) + 6
    ldb = (N if lb == ROW_MAJOR else K) + 6
    case = gi.make_case(M, N, K, layout_a=la, layout_b=lb, lda=lda, ldb=ldb, seed=9)
    # NaN in every padding element of A and B, NaN in all of C (beta = 0)
    A = case.A.reshape(-1, lda).clone()
    A[:, (K if la == ROW_MAJOR else M):] = float("nan")
    B = case.B.reshape(-1, ldb).clone()
    B[:, (N if lb == ROW_MAJOR else K):] = float("nan")
    case.A, case.B = A.reshape(-1), B.reshape(-1)
    case.C = torch.full_like(case.C, float("nan"))
    dC = run_case(case)
    got = c_logical(case, dC.cpu())
    assert np.isfinite(got).all()
    ref, scale = oracle_for(case)
    check_bound(got, ref, scale, OUT_F16, "nan padding")


def test_writes_stay_inside_c():
    """Sentinels in C's ld padding, in the rows after M and in the batch gap
    must survive."""
    M, N, K, ldc, batch = 77, 45, 64, 56, 2
    stride_c = (M + 3) * ldc
    case = gi.make_case(M, N, K, batch=batch, seed=11)
    sentinel = -1234.0
    C = torch.full((batch * stride_c,), sentinel, dtype=torch.float16, device="cuda")
    with mpg.Plan(M, N, K, ldc=ldc, batch=batch, stride_a=case.stride_a,
                  stride_b=case.stride_b, stride_c=stride_c) as p:
        p.run(case.A.cuda(), case.B.cuda(), C)
    C = C.cpu().reshape(batch, M + 3, ldc)
    assert torch.all(C[:, :, N:] == sentinel)
    assert torch.all(C[:, M:, :] == sentinel)
    assert not torch.any(C[:, :M, :N] == sentinel)


def test_misaligned_pointers_take_the_narrow_path():
    M, N, K = 96, 64, 128
    case = gi.make_case(M, N, K, beta=1.0, seed=12)
    A = torch.zeros(case.A.numel() + 1, dtype=torch.float16, device="cuda")
    B = torch.zeros(case.B.numel() + 3, dtype=torch.float16, device="cuda")
    C = torch.zeros(case.C.numel() + 1, dtype=torch.float16, device="cuda")
    A[1:] = case.A.cuda()
    B[3:] = case.B.cuda()
    C[1:] = case.C.cuda()
    run_case(case, A[1:], B[3:], C[1:])
    got = c_logical(case, C[1:].cpu())
    ref, scale = oracle_for(case)
    check_bound(got, ref, scale, OUT_F16, "misaligned")


def test_degenerate_extents():
    # K = 0: C <- beta * C
    case = gi.make_case(50, 40, 0, beta=0.5, lda=1, seed=13)
    dC = run_case(case)
    assert torch.equal(dC.cpu(), (case.C.float() * 0.5).half())
    # M = 0: no-op, even with null pointers
    with mpg.Plan(0, 40, 30) as p:
        assert mpg.gemm_f16f32_run(p.handle, 0, 0, 0, 1.0, 0.0, None) == 0
    # alpha = 0: beta * C
    case = gi.make_case(33, 65, 17, alpha=0.0, beta=2.0, seed=14)
    dC = run_case(case)
    assert torch.equal(dC.cpu(), (case.C.float() * 2.0).half())


def test_k_zero_on_the_direct_tile():
    """K = 0 on a shape the direct 128 tile serves (aligned leading
    dimensions): C <- beta * C, with every load failing its range check --
    the operands hold NaN, and none of it may reach C."""
    M, N = 1024, 1024
    with mpg.Plan(M, N, 0, lda=8) as p:
        assert p.kernel == "gemm_128x128x64m16_nn_direct", p.kernel
        A = torch.full((M * 8,), float("nan"), dtype=torch.float16, device="cuda")
        B = torch.full((N * 8,), float("nan"), dtype=torch.float16, device="cuda")
        g = torch.Generator("cpu").manual_seed(15)
        C0 = (torch.rand(M * N, generator=g) * 2 - 1).half()
        C = C0.cuda()
        p.run(A, B, C, 1.0, -0.5)
        torch.cuda.synchronize()
    assert torch.equal(C.cpu(), (C0.float() * -0.5).half())


def test_split_k_on_two_streams_with_own_workspaces():
    """One split-K plan run concurrently on two streams, each run with its
    own workspace (a plan is immutable host data): both results match the
    oracle, and each workspace's counter words are zero again afterwards."""
    c1 = gi.make_case(64, 4096, 4096, beta=1.0, seed=41)
    c2 = gi.make_case(64, 4096, 4096, beta=1.0, seed=42)
    p = mpg.Plan(c1.M, c1.N, c1.K, c1.layout_a, c1.layout_b, c1.out_type, c1.lda, c1.ldb, c1.ldc)
    assert "_sk" in p.kernel, p.kernel
    need = p.workspace_bytes()
    ws = [torch.zeros(need, dtype=torch.uint8, device="cuda") for _ in range(2)]
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    (A1, B1, C1), (A2, B2, C2) = to_device(c1), to_device(c2)
    torch.cuda.synchronize()
    for _ in range(4):
        C1.copy_(c1.C.cuda())
        C2.copy_(c2.C.cuda())
        torch.cuda.synchronize()
        p.run(A1, B1, C1, c1.alpha, c1.beta, stream=s1, workspace=ws[0])
        p.run(A2, B2, C2, c2.alpha, c2.beta, stream=s2, workspace=ws[1])
        torch.cuda.synchronize()
    p.close()
    for case, C in ((c1, C1), (c2, C2)):
        ref, scale = oracle_for(case)
        check_bound(c_logical(case, C.cpu()), ref, scale, OUT_F16, "split-K, two streams")
    for w in ws:
        assert torch.count_nonzero(w[:4096]).item() == 0


def test_workspace_init_clears_counters():
    """gemm_f16f32_workspace_init zero-fills a dirty buffer's counter words
    (stream-ordered, no allocation), after which a split-K run is correct."""
    case = gi.make_case(16, 4096, 4096, seed=43)
    with mpg.Plan(case.M, case.N, case.K) as p:
        need = p.workspace_bytes()
        ws = torch.full((need,), 7, dtype=torch.uint8, device="cuda")
        stream = torch.cuda.current_stream().cuda_stream
        assert mpg.gemm_f16f32_workspace_init(ws.data_ptr(), need, stream) == 0
        torch.cuda.synchronize()
        assert torch.count_nonzero(ws[:4096]).item() == 0
        assert torch.all(ws[4096:] == 7)
        A, B, C = to_device(case)
        p.run(A, B, C, 1.0, 0.0, workspace=ws)
        torch.cuda.synchronize()
    ref, scale = oracle_for(case)
    check_bound(c_logical(case, C.cpu()), ref, scale, OUT_F16, "after workspace_init")


# ------------------------------------------------------- 64-bit offsets

@pytest.mark.parametrize("shape,tile,lda", [((600, 4096, 256), "128x128", 1 << 22),
                                            ((2048, 8192, 384), "256x256", 1 << 22),
                                            ((600, 4096, 256), "128x128", (1 << 22) + 8)])
def test_huge_leading_dimension(shape, tile, lda):
    """A row-major with lda = 2^22 (8 MiB between rows): A spans 4.7 or 16
    GiB, so tile origins lie beyond 2^32 bytes while each tile's lane
    offsets stay below 2^31.  Above 2^22 the plan repacks both operands
    into the workspace first.  The oracle runs on the compact copy."""
    M, N, K = shape
    case = gi.make_case(M, N, K, beta=1.0, seed=95)
    A = torch.zeros((M - 1) * lda + K, dtype=torch.float16, device="cuda")
    A.as_strided((M, K), (lda, 1)).copy_(case.A.view(M, K).cuda())
    B, C = case.B.cuda(), case.C.cuda()
    with mpg.Plan(M, N, K, ROW_MAJOR, ROW_MAJOR, OUT_F16, lda, case.ldb, case.ldc) as p:
        assert tile in p.kernel, p.kernel
        assert p.kernel.endswith("_pkab") == (lda > (1 << 22)), p.kernel
        p.run(A, B, C, case.alpha, case.beta)
    torch.cuda.synchronize()
    del A
    rows = sample_rows(M, n_random=24)
    ref, scale = oracle_for(case, rows)
    check_bound(c_logical(case, C.cpu(), rows), ref, scale, OUT_F16, f"lda={lda} {shape}")


@pytest.mark.parametrize("N", [512, 1040])
def test_streaming_kernel_large_column_pitch(N):
    """The streaming kernel with column-major B at ldb = 2^22: B spans 4 or
    8 GiB, so columns past the first 256 (512) lie beyond 2^31 (2^32) bytes
    from B's base.  Each workgroup's descriptor starts at its own first
    column, so every lane offset stays small; the oracle runs on a compact
    copy of B."""
    M, K, ldb = 16, 64, 1 << 22
    case = gi.make_case(M, N, K, layout_b=COL_MAJOR, beta=0.5, seed=97)
    B = torch.zeros((N - 1) * ldb + K, dtype=torch.float16, device="cuda")
    B.as_strided((N, K), (ldb, 1)).copy_(case.B.view(N, K).cuda())
    A, C = case.A.cuda(), case.C.cuda()
    with mpg.Plan(M, N, K, ROW_MAJOR, COL_MAJOR, OUT_F16, case.lda, ldb, case.ldc) as p:
        assert p.kernel == "gemm_stream16x16_nt_direct", p.kernel
        p.run(A, B, C, case.alpha, case.beta)
    torch.cuda.synchronize()
    del B
    ref, scale = oracle_for(case)
    check_bound(c_logical(case, C.cpu()), ref, scale, OUT_F16, f"stream ldb=2^22 N={N}")


def test_huge_batch_stride():
    """A strided batch whose A items lie 3 * 2^30 elements (6 GiB) apart, on
    the 128 tile; the oracle runs on the compact copy."""
    M, N, K, batch = 1024, 1024, 256, 2
    sa = 3 << 30
    case = gi.make_case(M, N, K, batch=batch, beta=0.5, seed=96)
    A = torch.zeros(sa + M * K, dtype=torch.float16, device="cuda")
    src = case.A.view(batch, M * K).cuda()
    for b in range(batch):
        A[b * sa:b * sa + M * K].copy_(src[b])
    B, C = case.B.cuda(), case.C.cuda()
    with mpg.Plan(M, N, K, ROW_MAJOR, ROW_MAJOR, OUT_F16, case.lda, case.ldb, case.ldc,
                  batch, sa, case.stride_b, case.stride_c) as p:
        assert "128x128" in p.kernel, p.kernel
        p.run(A, B, C, case.alpha, case.beta)
    torch.cuda.synchronize()
    del A
    rows = sample_rows(M, n_random=16)
    ref, scale = oracle_for(case, rows)
    check_bound(c_logical(case, C.cpu(), rows), ref, scale, OUT_F16, "batch stride 3*2^30")


# ------------------------------------------------------- random sweep

def _sweep_cases(n, seed):
    """Seeded shapes from four classes -- small (staged and streaming
    kernels), skinny and deep (streaming, split-K), medium (128 tile, two- and
    four-slot rings), large (256 tile) -- with random layouts, leading
    dimensions that are multiples of 8 or not (repacking), batch, alpha/beta
    and output type."""
    rng = np.random.default_rng(seed)

    def dim(lo, hi):
        v = int(rng.integers(lo, hi))
        return v - v % 8 if (rng.random() < 0.5 and v >= 8) else v

    out = []
    for i in range(n):
        cls = i % 4
        if cls == 0:
            M, N, K = dim(1, 300), dim(1, 300), dim(1, 300)
        elif cls == 1:
            M, N, K = dim(1, 160), dim(900, 5000), dim(900, 5000)
        elif cls == 2:
            M, N, K = dim(400, 2600), dim(400, 2600), dim(64, 3000)
        else:
            M, N = (int(rng.choice([4096, 4352, 5120])) for _ in range(2))
            K = int(rng.integers(5, 19)) * 64
        la, lb = (int(x) for x in rng.integers(0, 2, size=2))
        pad = int(rng.choice([0, 0, 8, 3])) if cls != 3 else 0
        batch = int(rng.choice([1, 1, 1, 2])) if cls in (0, 2) else 1
        out_type = int(rng.integers(0, 2))
        alpha, beta = float(rng.choice([1.0, -0.5])), float(rng.choice([0.0, 1.0, 2.0]))
        out.append((M, N, K, la, lb, pad, batch, out_type, alpha, beta))
    return out


@pytest.mark.parametrize("case_args", _sweep_cases(40, 2026))
def test_random_sweep(case_args):
    M, N, K, la, lb, pad, batch, out_type, alpha, beta = case_args
    lda = (K if la == ROW_MAJOR else M) + pad
    ldb = (N if lb == ROW_MAJOR else K) + pad
    case = gi.make_case(M, N, K, layout_a=la, layout_b=lb, out_type=out_type, alpha=alpha,
                        beta=beta, batch=batch, lda=lda, ldb=ldb, seed=hash(case_args) % 1000)
    kernel = plan_kernel(case)
    rows = None if M * N * K * batch <= (1 << 27) else sample_rows(M, n_random=16, tiles=(256, 128))
    parity(case, rows=rows, what=f"{kernel} {case_args}")


# ---------------------------------------------------------- determinism

def test_run_to_run_bitwise_determinism():
    """Same plan, same inputs: bitwise identical output, also on another
    stream (a missing barrier shows up as run-to-run differences)."""
    case = gi.make_case(1536, 1280, 1000, beta=1.0, seed=15)
    dA, dB, dC0 = to_device(case)
    outs = []
    s2 = torch.cuda.Stream()
    for stream in (None, None, s2):
        dC = dC0.clone()
        torch.cuda.synchronize()
        run_case(case, dA, dB, dC, stream=stream)
        torch.cuda.synchronize()
        outs.append(dC.cpu())
    assert torch.equal(outs[0], outs[1]) and torch.equal(outs[0], outs[2])


# ------------------------------------------------------------- split-K

@pytest.mark.parametrize("la,lb", LAYOUTS)
def test_split_k_all_layouts(la, lb):
    """Skinny-M shapes whose 128 tiles cannot fill the CUs take split-K."""
    M, N, K = 64, 2048, 4096
    case = gi.make_case(M, N, K, layout_a=la, layout_b=lb, alpha=1.0, beta=1.0, seed=31)
    p = mpg.Plan(M, N, K, la, lb, OUT_F16, case.lda, case.ldb, case.ldc)
    kernel = p.kernel
    p.close()
    if (la, lb) != (ROW_MAJOR, COL_MAJOR):       # NT with M <= 64 streams instead
        assert "_sk" in kernel, kernel
    parity(case, what=f"{kernel} {M}x{N}x{K}")


def test_split_k_fp32_ragged_alpha_beta():
    """Ragged N and a short last K slice (K = 3000 in slices of 384), fp32 C,
    alpha = 2, beta = -0.5."""
    M, N, K = 100, 1000, 3000
    case = gi.make_case(M, N, K, out_type=OUT_F32, alpha=2.0, beta=-0.5, seed=32)
    p = mpg.Plan(M, N, K, ROW_MAJOR, ROW_MAJOR, OUT_F32, case.lda, case.ldb, case.ldc)
    assert "_sk" in p.kernel, p.kernel
    p.close()
    parity(case, what="split-K fp32 ragged")


@pytest.mark.parametrize("la,lb", LAYOUTS)
def test_split_k_two_slot_ring(la, lb):
    """Split-K on the two-slot (split-ring) 128 tile: 144 tiles x 2 slices =
    288 workgroups, two per CU, the arrival flag inside the ring's LDS; K
    with and without a tail inside the last stage; fp32 C, beta != 0;
    sampled rows."""
    for K in (4096, 4000):
        M, N = 1536, 1536
        case = gi.make_case(M, N, K, layout_a=la, layout_b=lb, out_type=OUT_F32,
                            alpha=0.75, beta=-1.5, seed=90)
        kernel = plan_kernel(case)
        assert "128x128x64m16_" in kernel and "_sk2" in kernel, kernel
        parity(case, rows=sample_rows(M, n_random=24), what=f"{kernel} {M}x{N}x{K}")


def test_split_k_repeatable_and_interleaved():
    """The arrival counters return to zero after every launch: a split-K plan
    run twice gives the same bits, also with another split-K plan launched in
    between on the same stream."""
    c1 = gi.linear_case(128, 6144)
    c2 = gi.make_case(16, 4096, 4096, seed=33)
    p1 = mpg.Plan(c1.M, c1.N, c1.K, c1.layout_a, c1.layout_b, c1.out_type, c1.lda, c1.ldb, c1.ldc)
    p2 = mpg.Plan(c2.M, c2.N, c2.K, c2.layout_a, c2.layout_b, c2.out_type, c2.lda, c2.ldb, c2.ldc)
    assert "_sk" in p1.kernel and "_sk" in p2.kernel, (p1.kernel, p2.kernel)
    A1, B1, C1 = to_device(c1)
    A2, B2, C2 = to_device(c2)
    outs = []
    for _ in range(3):
        C1.zero_()
        p1.run(A1, B1, C1, c1.alpha, c1.beta)
        p2.run(A2, B2, C2, c2.alpha, c2.beta)
        torch.cuda.synchronize()
        outs.append(C1.clone())
    p1.close()
    p2.close()
    assert all(torch.equal(outs[0], o) for o in outs[1:])
    ref, scale = oracle_for(c1)
    check_bound(c_logical(c1, outs[0].cpu()), ref, scale, c1.out_type, "split-K repeat")
    ref2, scale2 = oracle_for(c2)
    check_bound(c_logical(c2, C2.cpu()), ref2, scale2, c2.out_type, "split-K interleaved")


@pytest.mark.parametrize("shape,kw,frag", [
    ((20, 8192, 4096), {}, "stream32x64_nt_direct_sk4"),
    ((17, 9000, 4096), dict(out_type=OUT_F32, alpha=0.5, beta=-1.0), "stream32x64_nt_direct_sk4"),
    ((24, 8200, 3000), dict(beta=1.0), "stream32x64_nt_direct_sk2"),        # ragged N, short last slice
    ((32, 8192, 4096), dict(out_type=OUT_F32), "stream32x64_nt_direct_sk4"),  # two row blocks
    ((27, 8256, 2048), dict(beta=1.0), "stream32x64_nt_direct_sk2"),        # rows of A past M
    ((96, 2048, 4096), {}, "stream32x64_nt_direct_sk4"),                    # three row tiles
    ((100, 1000, 3000), dict(beta=1.0, out_type=OUT_F32), "stream32x64_nt_direct_sk2"),  # ragged
])
def test_streaming_split_k(shape, kw, frag):
    """The 64-column streaming tile with K slices summed by the last slice to
    arrive: parity with the oracle, the same bits on a second run, and the
    counter words zero again afterwards."""
    M, N, K = shape
    kw = dict(kw)
    batch = kw.pop("batch", 1)
    case = gi.make_case(M, N, K, layout_b=COL_MAJOR, batch=batch, seed=M + N + K, **kw)
    with mpg.Plan(case.M, case.N, case.K, case.layout_a, case.layout_b, case.out_type, case.lda,
                  case.ldb, case.ldc, case.batch, case.stride_a, case.stride_b, case.stride_c) as p:
        assert frag in p.kernel, p.kernel
        ws = torch.zeros(p.workspace_bytes(), dtype=torch.uint8, device="cuda")
        A, B, C = to_device(case)
        C0 = C.clone()
        outs = []
        for _ in range(2):
            C.copy_(C0)
            p.run(A, B, C, case.alpha, case.beta, workspace=ws)
            torch.cuda.synchronize()
            outs.append(C.clone())
    assert torch.equal(outs[0], outs[1])
    assert torch.count_nonzero(ws[:4096]).item() == 0
    ref, scale = oracle_for(case)
    check_bound(c_logical(case, outs[0].cpu()), ref, scale, case.out_type, f"{frag} {shape}")


def test_split_k_plan_with_misaligned_pointer_repacks():
    """A split-K plan run with a misaligned A: A is copied into the padded
    area of the workspace and the split kernel runs on the copy."""
    M, N, K = 16, 1024, 2048
    case = gi.make_case(M, N, K, beta=1.0, seed=34)
    p = mpg.Plan(M, N, K)
    assert "_sk" in p.kernel, p.kernel
    p.close()
    A = torch.zeros(case.A.numel() + 1, dtype=torch.float16, device="cuda")
    A[1:] = case.A.cuda()
    B, C = case.B.cuda(), case.C.cuda()
    run_case(case, A[1:], B, C)
    ref, scale = oracle_for(case)
    check_bound(c_logical(case, C.cpu()), ref, scale, OUT_F16, "split-K plan, misaligned A")


# ------------------------------------------------------------ repacking

def plan_kernel(case):
    with mpg.Plan(case.M, case.N, case.K, case.layout_a, case.layout_b, case.out_type,
                  case.lda, case.ldb, case.ldc, case.batch, case.stride_a,
                  case.stride_b, case.stride_c) as p:
        return p.kernel


def expected_pack_suffix(case):
    """Operands whose rows do not allow 16-byte loads: _pka, _pkb, _pkab."""
    ca = case.K if case.layout_a == ROW_MAJOR else case.M
    cb = case.N if case.layout_b == ROW_MAJOR else case.K
    sa = case.stride_a if case.batch > 1 else 0
    sb = case.stride_b if case.batch > 1 else 0
    pa = any(v % 8 for v in (ca, case.lda, sa))
    pb = any(v % 8 for v in (cb, case.ldb, sb))
    return "_pk" + ("a" if pa else "") + ("b" if pb else "") if (pa or pb) else ""


def nan_padding(case):
    """NaN in every element of A and B beyond the logical rows' ends (the
    repacking copies only the logical elements and zero-fills the rest)."""
    ca = case.K if case.layout_a == ROW_MAJOR else case.M
    cb = case.N if case.layout_b == ROW_MAJOR else case.K
    A = case.A.reshape(-1, case.lda).clone()
    A[:, ca:] = float("nan")
    B = case.B.reshape(-1, case.ldb).clone()
    B[:, cb:] = float("nan")
    case.A, case.B = A.reshape(-1), B.reshape(-1)


@pytest.mark.parametrize("out_type", [OUT_F16, OUT_F32])
@pytest.mark.parametrize("la,lb", LAYOUTS)
def test_repacked_operands_all_layouts(la, lb, out_type):
    """Shapes for the direct kernels (128 tile, split-K) whose row lengths
    are not multiples of 8: odd M, N and K (so the K tail ends inside an
    8-element chunk of a K-contiguous row), leading dimensions with
    NaN-filled padding, beta on and off."""
    shapes = [(300, 260, 1500, 3), (1000, 1000, 999, 0), (50, 333, 4100, 5),
              (4097, 63, 1025, 1)]
    for i, (M, N, K, extra) in enumerate(shapes):
        lda = (K if la == ROW_MAJOR else M) + extra
        ldb = (N if lb == ROW_MAJOR else K) + extra
        case = gi.make_case(M, N, K, layout_a=la, layout_b=lb, out_type=out_type,
                            lda=lda, ldb=ldb, alpha=-0.5, beta=0.0 if i == 1 else 2.0,
                            seed=40 + i)
        nan_padding(case)
        kernel = plan_kernel(case)
        suffix = expected_pack_suffix(case)
        assert "direct" in kernel and kernel.endswith(suffix), (kernel, suffix)
        rows = sample_rows(M, n_random=32) if M >= 1000 else None
        parity(case, rows=rows, what=f"{kernel} {M}x{N}x{K} lda={lda} ldb={ldb}")


def test_repacked_batched_odd_strides():
    """Strided batch on the 128 tile with odd leading dimensions and hence
    odd batch strides for A and B."""
    M, N, K, batch = 520, 520, 200, 4
    case = gi.make_case(M, N, K, lda=K + 1, ldb=N + 1, batch=batch, beta=1.0, seed=50)
    kernel = plan_kernel(case)
    assert "128x128" in kernel and kernel.endswith("_pkab"), kernel
    parity(case, what=f"{kernel} batch {batch}")


@pytest.mark.parametrize("M", [7, 40])
def test_repacked_streaming(M):
    """Skinny NT (streaming kernel) with K odd: both operands repacked."""
    N, K = 4097, 4099
    case = gi.linear_case(M, N, K, seed=51)
    kernel = plan_kernel(case)
    assert "stream" in kernel and kernel.endswith("_pkab"), kernel
    parity(case, what=f"{kernel} {M}x{N}x{K}")


def test_repacked_full_tile_sampled():
    """The 256 tile on 4095^3 (every operand repacked), sampled rows."""
    n = 4095
    case = gi.make_case(n, n, n, layout_b=COL_MAJOR, beta=1.0, seed=52)
    kernel = plan_kernel(case)
    assert "256x256" in kernel and kernel.endswith("_pkab"), kernel
    parity(case, rows=sample_rows(n, n_random=48), what=kernel)


def test_misaligned_pointers_repack_on_direct_tile_and_reuse_buffer():
    """A direct-tile plan given misaligned A and B pointers copies both; a
    second run of the same plan with other data reuses the copies."""
    M, N, K = 1000, 1000, 1000
    p = mpg.Plan(M, N, K, ROW_MAJOR, COL_MAJOR)
    assert "direct" in p.kernel and "_pk" not in p.kernel, p.kernel
    try:
        for seed, (oa, ob) in ((60, (1, 3)), (61, (5, 2))):
            case = gi.make_case(M, N, K, layout_b=COL_MAJOR, beta=1.0, seed=seed)
            A = torch.zeros(case.A.numel() + oa, dtype=torch.float16, device="cuda")
            B = torch.zeros(case.B.numel() + ob, dtype=torch.float16, device="cuda")
            A[oa:] = case.A.cuda()
            B[ob:] = case.B.cuda()
            C = case.C.cuda()
            p.run(A[oa:], B[ob:], C, case.alpha, case.beta)
            torch.cuda.synchronize()
            rows = sample_rows(M, n_random=32)
            ref, scale = oracle_for(case, rows)
            check_bound(c_logical(case, C.cpu(), rows), ref, scale, OUT_F16,
                        f"misaligned run seed {seed}")
    finally:
        p.close()
