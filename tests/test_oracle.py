"""Pins for the CPU oracle (no GPU).

The oracle (oracle/ref_gemm.c) is the plain definition of
C = alpha*A*B + beta*C in fp64.  These tests pin it to things other than
itself: numpy's binary16 conversions, binary32's bit layout and torch's
rounding for bfloat16, exact rational arithmetic on tiny inputs (brute
force), numpy's int64 matrix product on integer inputs, the binary16 and
bfloat16 landmarks the pages state (tests/golden/), and closed forms.  The
logical matrices are built first and laid out into storage with numpy
transposes, so the oracle's own index formulas are checked, not retyped.
"""
import itertools
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
import torch

from oracle import COL_MAJOR, IN_BF16, IN_F16, OUT_BF16, OUT_F16, OUT_F32, ROW_MAJOR

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
LAYOUTS = [(ROW_MAJOR, ROW_MAJOR), (ROW_MAJOR, COL_MAJOR),
           (COL_MAJOR, ROW_MAJOR), (COL_MAJOR, COL_MAJOR)]


# ---------------------------------------------------------------- helpers

def to_storage(logical: np.ndarray, layout: int, ld: int, fill=0):
    """Lays a logical rows x cols matrix (fp16 values, or bfloat16 bit
    patterns as uint16) out with leading dimension ld.  Row-major: ld >=
    cols, element (r, c) at r*ld + c.  Column-major: the transpose is stored
    row-major, element (r, c) at r + c*ld."""
    mat = logical if layout == ROW_MAJOR else logical.T
    rows, cols = mat.shape
    store = np.full((rows, ld), fill, dtype=logical.dtype)
    store[:, :cols] = mat
    return store.ravel()


def stack_batches(mats, layout, ld, fill=0):
    parts = [to_storage(m, layout, ld, fill) for m in mats]
    return np.concatenate(parts), parts[0].size


def exact_product(A_log, B_log, C_log, alpha, beta):
    """alpha * A @ B + beta * C in exact rationals; also the error scale
    |alpha| sum|a b| + |beta| |c|.  C_log is ignored when beta == 0."""
    M, K = A_log.shape
    N = B_log.shape[1]
    fa = [[Fraction(float(A_log[i, k])) for k in range(K)] for i in range(M)]
    fb = [[Fraction(float(B_log[k, j])) for j in range(N)] for k in range(K)]
    al, be = Fraction(float(np.float32(alpha))), Fraction(float(np.float32(beta)))
    ref = np.empty((M, N), dtype=object)
    sc = np.empty((M, N), dtype=object)
    for i in range(M):
        for j in range(N):
            s = sum((fa[i][k] * fb[k][j] for k in range(K)), Fraction(0))
            t = sum((abs(fa[i][k] * fb[k][j]) for k in range(K)), Fraction(0))
            c = Fraction(float(C_log[i, j])) if beta != 0 else Fraction(0)
            ref[i, j] = al * s + be * c
            sc[i, j] = abs(al) * t + abs(be) * abs(c)
    return ref, sc


def rand_f16(rng, shape):
    return (rng.uniform(-1, 1, size=shape)).astype(np.float16)


BF16_NAN = 0x7FC0


def bf16_bits(values) -> np.ndarray:
    """float32-representable values -> bfloat16 bits, rounded by torch (a
    conversion written independently of the oracle)."""
    t = torch.from_numpy(np.ascontiguousarray(values, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def bf16_values(bits) -> np.ndarray:
    """bfloat16 bits -> float64: the binary32 whose upper half they are."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    with np.errstate(invalid="ignore"):   # signalling NaN patterns
        return b.view(np.float32).astype(np.float64)


def rand_bf16(rng, shape):
    """Uniform [-1, 1) rounded to bfloat16: (bits, values)."""
    bits = bf16_bits(rng.uniform(-1, 1, size=shape).astype(np.float32))
    return bits, bf16_values(bits)


# ------------------------------------------------------- binary16 decoding

def test_dec16_exhaustive_against_numpy():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = oracle.dec16(bits)
    want = bits.view(np.float16).astype(np.float64)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])
    # signed zeros keep their sign
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(want[~nan]))


def test_binary16_landmarks_golden():
    path = os.path.join(GOLDEN, "binary16_landmarks.txt")
    rows = []
    with open(path) as fh:
        for line in fh:
            line = line.split("#")[0].strip()
            if not line:
                continue
            parts = line.split()
            rows.append((int(parts[0], 16), float(parts[1])))
    assert len(rows) >= 10
    for bits, value in rows:
        got = float(oracle.dec16(np.array([bits]))[0])
        assert got == value and np.signbit(got) == np.signbit(value), hex(bits)
        if not np.isinf(value):
            assert int(oracle.enc16(np.array([value]))[0]) == bits, hex(bits)


# ------------------------------------------------------- binary16 encoding

def _encode_probe_values():
    rng = np.random.default_rng(1)
    finite = np.arange(0, 0x7C00, dtype=np.uint16).view(np.float16).astype(np.float64)
    nxt = np.nextafter(finite[:-1], np.inf)
    mids = (finite[:-1] + finite[1:]) / 2          # exact ties in double
    vals = [finite, mids, np.nextafter(mids, np.inf), np.nextafter(mids, -np.inf),
            nxt,
            np.exp2(rng.uniform(-30, 17, 20000)),
            np.array([65504.0, 65519.99999, 65520.0, 65520.00001, 65536.0,
                      1e9, 2.0 ** -25, 2.0 ** -25 * 1.0000001, 2.0 ** -24 * 1.5,
                      2.0 ** -24 * 2.5, 2.0 ** -14 - 2.0 ** -25, 1e-300])]
    v = np.concatenate(vals)
    return np.concatenate([v, -v])


def test_enc16_matches_numpy_round_to_nearest_even():
    v = _encode_probe_values()
    got = oracle.enc16(v)
    with np.errstate(over="ignore"):
        want = v.astype(np.float16).view(np.uint16)   # numpy: RNE from double
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(v[i], hex(got[i]), hex(want[i])) for i in bad[:5]]


def test_enc16_specials():
    got = oracle.enc16(np.array([np.inf, -np.inf, np.nan, -0.0, 0.0]))
    assert got[0] == 0x7C00 and got[1] == 0xFC00
    assert (got[2] & 0x7C00) == 0x7C00 and (got[2] & 0x3FF) != 0
    assert got[3] == 0x8000 and got[4] == 0x0000


# ------------------------------------------------ exact brute force (tiny)

def _draw16(rng, shape, in_bf16):
    """(storage, values, NaN fill) of a uniform [-1, 1) 16-bit matrix."""
    if in_bf16:
        bits, vals = rand_bf16(rng, shape)
        return bits, vals, BF16_NAN
    h = rand_f16(rng, shape)
    return h, h.astype(np.float64), np.nan


def _run_case(lib, M, N, K, la, lb, out_type, alpha, beta, batch, pad, rng,
              in_type=IN_F16):
    bf = in_type == IN_BF16
    Ad = [_draw16(rng, (M, K), bf) for _ in range(batch)]
    Bd = [_draw16(rng, (K, N), bf) for _ in range(batch)]
    if out_type in (OUT_F16, OUT_BF16):
        Cd = [_draw16(rng, (M, N), out_type == OUT_BF16) for _ in range(batch)]
    else:
        Cd = [(c, c.astype(np.float64), np.nan) for c in
              (rng.uniform(-4, 4, (M, N)).astype(np.float32) for _ in range(batch))]
    lda = (K if la == ROW_MAJOR else M) + pad
    ldb = (N if lb == ROW_MAJOR else K) + pad
    ldc = N + pad
    A, sa = stack_batches([d[0] for d in Ad], la, lda, fill=Ad[0][2])
    B, sb = stack_batches([d[0] for d in Bd], lb, ldb, fill=Bd[0][2])
    cst = []
    for c, _, fill in Cd:
        s = np.full((M, ldc), fill, dtype=c.dtype)
        s[:, :N] = c
        cst.append(s.ravel())
    C = np.concatenate(cst)
    ref, sc = oracle.gemm(M, N, K, A, B, C, alpha=alpha, beta=beta,
                          layout_a=la, layout_b=lb, out_type=out_type,
                          in_type=in_type,
                          lda=lda, ldb=ldb, ldc=ldc, batch=batch,
                          stride_a=sa, stride_b=sb, stride_c=M * ldc,
                          nthreads=2, lib=lib)
    for b in range(batch):
        ex, exs = exact_product(Ad[b][1], Bd[b][1], Cd[b][1], alpha, beta)
        for i in range(M):
            for j in range(N):
                tol = float(exs[i, j]) * 2.0 ** -50
                assert abs(Fraction(ref[b, i, j]) - ex[i, j]) <= Fraction(tol), \
                    (M, N, K, la, lb, in_type, out_type, alpha, beta, b, i, j)
                assert abs(Fraction(sc[b, i, j]) - exs[i, j]) <= Fraction(tol)


ALPHA_BETA = [(1.0, 0.0), (-0.5, 2.0), (0.0, 1.0)]


def _brute_force(lib, shapes, full_combos, in_type=IN_F16):
    rng = np.random.default_rng(7)
    outs = (OUT_F16, OUT_F32) if in_type == IN_F16 else (OUT_BF16, OUT_F32)
    n = 0
    for idx, (M, N, K) in enumerate(shapes):
        for li, (la, lb) in enumerate(LAYOUTS):
            if full_combos:
                combos = [(o, ab) for o in outs for ab in ALPHA_BETA]
            else:
                k = idx * 4 + li
                combos = [(outs[k % 2], ALPHA_BETA[k % 3])]
            for out_type, (alpha, beta) in combos:
                batch = 1 + (n % 2)
                pad = n % 3
                _run_case(lib, M, N, K, la, lb, out_type, alpha, beta, batch,
                          pad, rng, in_type)
                n += 1
    return n


def test_brute_force_all_small_shapes():
    shapes = list(itertools.product(range(1, 9), repeat=3))
    assert _brute_force(None, shapes, full_combos=False) == 512 * 4


def test_brute_force_odd_shapes_all_combinations():
    shapes = [(1, 1, 1), (3, 5, 7), (17, 9, 33)]
    _brute_force(None, shapes, full_combos=True)


def test_brute_force_bf16_small_shapes():
    shapes = list(itertools.product(range(1, 7), repeat=3))
    assert _brute_force(None, shapes, full_combos=False, in_type=IN_BF16) == 216 * 4


def test_brute_force_bf16_odd_shapes_all_combinations():
    shapes = [(1, 1, 1), (3, 5, 7), (17, 9, 33)]
    _brute_force(None, shapes, full_combos=True, in_type=IN_BF16)


# ------------------------------------------------------ bfloat16 decoding

def test_decbf16_exhaustive_against_binary32_upper_half():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = oracle.decbf16(bits)
    want = bf16_values(bits)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(want[~nan]))
    # and torch's own bfloat16 -> float64 conversion agrees
    t = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(got[~nan], t[~nan])


def test_bfloat16_landmarks_golden():
    path = os.path.join(GOLDEN, "bfloat16_landmarks.txt")
    rows = []
    with open(path) as fh:
        for line in fh:
            line = line.split("#")[0].strip()
            if not line:
                continue
            parts = line.split()
            rows.append((int(parts[0], 16), float(parts[1])))
    assert len(rows) >= 10
    for bits, value in rows:
        got = float(oracle.decbf16(np.array([bits]))[0])
        assert got == value and np.signbit(got) == np.signbit(value), hex(bits)
        if not np.isinf(value):
            assert int(oracle.encbf16(np.array([value]))[0]) == bits, hex(bits)
    # the page's rounded figures: largest finite about 3.4e38, smallest
    # normal about 1e-38, the exponent range of fp32
    assert abs(oracle.decbf16(np.array([0x7F7F]))[0] / 3.4e38 - 1) < 0.01
    assert 1e-38 < oracle.decbf16(np.array([0x0080]))[0] < 1.2e-38
    assert oracle.decbf16(np.array([0x0080]))[0] == float(np.finfo(np.float32).tiny)


# ------------------------------------------------------ bfloat16 encoding

def _encode_bf16_probe_values():
    """Values exactly representable in float32 (torch rounds float32 to
    bfloat16 once, so its result is the correctly rounded one)."""
    rng = np.random.default_rng(2)
    fin = bf16_values(np.arange(0, 0x7F80, dtype=np.uint32).astype(np.uint16))
    f32 = lambda x: np.asarray(x, dtype=np.float32)
    mids = f32((fin[:-1] + fin[1:]) / 2)               # exact ties (9 bits)
    up = np.nextafter(mids, f32(np.inf))
    dn = np.nextafter(mids, f32(0))
    rnd = f32(np.exp2(rng.uniform(-140, 128, 40000)))
    edge = f32([3.3895313892515355e38, 3.3961775292304e38, 3.4028234663852886e38,
                2.0 ** -133, 2.0 ** -134, 3 * 2.0 ** -134, 2.0 ** -126 - 2.0 ** -134,
                1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, 255.5, 256.5, 257.0])
    v = np.concatenate([f32(fin), mids, up, dn, rnd, edge]).astype(np.float64)
    return np.concatenate([v, -v])


def test_encbf16_matches_torch_round_to_nearest_even():
    v = _encode_bf16_probe_values()
    got = oracle.encbf16(v)
    want = bf16_bits(v.astype(np.float32))
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(v[i], hex(got[i]), hex(want[i])) for i in bad[:5]]


def test_encbf16_double_only_values_and_specials():
    # values no float32 holds, checked against the rounding rule by hand
    cases = {1e300: 0x7F80, -1e300: 0xFF80, 1e-300: 0x0000, -1e-300: 0x8000,
             (2 - 2.0 ** -8) * 2.0 ** 127: 0x7F80,                 # tie at the top -> inf
             (2 - 2.0 ** -8) * 2.0 ** 127 * (1 - 2.0 ** -40): 0x7F7F,
             1.0 + 2.0 ** -8 + 2.0 ** -40: 0x3F81,                 # just above a tie
             2.0 ** -134 * (1 + 2.0 ** -40): 0x0001}
    for x, bits in cases.items():
        assert int(oracle.encbf16(np.array([x]))[0]) == bits, (x, hex(bits))
    got = oracle.encbf16(np.array([np.inf, -np.inf, np.nan, -0.0, 0.0]))
    assert got[0] == 0x7F80 and got[1] == 0xFF80
    assert (got[2] & 0x7F80) == 0x7F80 and (got[2] & 0x7F) != 0
    assert got[3] == 0x8000 and got[4] == 0x0000


# -------------------------------------------------------------- closed forms

@pytest.mark.parametrize("la,lb", LAYOUTS)
@pytest.mark.parametrize("K", [1, 7, 64, 2048, 4097])
def test_all_ones_gives_K(la, lb, K):
    M, N = 5, 3
    A = to_storage(np.ones((M, K), np.float16), la, K if la == ROW_MAJOR else M)
    B = to_storage(np.ones((K, N), np.float16), lb, N if lb == ROW_MAJOR else K)
    ref, sc = oracle.gemm(M, N, K, A, B, layout_a=la, layout_b=lb)
    assert np.all(ref == K) and np.all(sc == K)
    # the fp16 output is the round-to-nearest-even of K (4097 -> 4096)
    enc = oracle.enc16(ref.ravel())
    assert np.all(enc == np.float16(K).view(np.uint16))
    if K == 4097:
        assert np.all(enc == 0x6C00)


@pytest.mark.parametrize("la,lb", LAYOUTS)
def test_identity_returns_other_operand(la, lb):
    rng = np.random.default_rng(3)
    M, N = 37, 23
    Bm = rand_f16(rng, (M, N))
    eye = np.eye(M, dtype=np.float16)
    ref, _ = oracle.gemm(M, N, M, to_storage(eye, la, M), to_storage(Bm, lb, N if lb == ROW_MAJOR else M),
                         layout_a=la, layout_b=lb)
    assert np.array_equal(ref[0], Bm.astype(np.float64))
    Am = rand_f16(rng, (M, N))
    eyeN = np.eye(N, dtype=np.float16)
    ref, _ = oracle.gemm(M, N, N, to_storage(Am, la, N if la == ROW_MAJOR else M), to_storage(eyeN, lb, N),
                         layout_a=la, layout_b=lb)
    assert np.array_equal(ref[0], Am.astype(np.float64))


def test_rank_one_K1_is_a_single_exact_product():
    rng = np.random.default_rng(4)
    M, N = 19, 11
    a = rand_f16(rng, (M, 1))
    b = rand_f16(rng, (1, N))
    alpha = -1.75
    ref, _ = oracle.gemm(M, N, 1, to_storage(a, ROW_MAJOR, 1), to_storage(b, ROW_MAJOR, N), alpha=alpha)
    want = alpha * np.outer(a.astype(np.float64), b.astype(np.float64))
    assert np.array_equal(ref[0], want)


# ------------------------------------------------------------ integer exact

@pytest.mark.parametrize("in_type", [IN_F16, IN_BF16])
@pytest.mark.parametrize("la,lb", LAYOUTS)
def test_integer_inputs_match_int64_matmul(la, lb, in_type):
    rng = np.random.default_rng(5)
    M, N, K, batch = 33, 41, 113, 3
    Ai = rng.integers(-3, 4, (batch, M, K))
    Bi = rng.integers(-3, 4, (batch, K, N))
    Ci = rng.integers(-8, 9, (batch, M, N))
    lda = (K if la == ROW_MAJOR else M) + 5
    ldb = (N if lb == ROW_MAJOR else K) + 2
    if in_type == IN_F16:
        enc, fill, out = (lambda m: m.astype(np.float16)), np.nan, OUT_F16
    else:   # small integers are exact in bfloat16 (8 significant bits)
        enc, fill, out = (lambda m: bf16_bits(m.astype(np.float32))), BF16_NAN, OUT_BF16
    A, sa = stack_batches([enc(m) for m in Ai], la, lda, fill=fill)
    B, sb = stack_batches([enc(m) for m in Bi], lb, ldb, fill=fill)
    C = enc(Ci).ravel()
    ref, sc = oracle.gemm(M, N, K, A, B, C, alpha=1.0, beta=1.0, layout_a=la,
                          layout_b=lb, lda=lda, ldb=ldb, batch=batch,
                          stride_a=sa, stride_b=sb, stride_c=M * N,
                          in_type=in_type, out_type=out)
    want = np.matmul(Ai, Bi) + Ci
    assert np.array_equal(ref, want.astype(np.float64))
    want_s = np.matmul(np.abs(Ai), np.abs(Bi)) + np.abs(Ci)
    assert np.array_equal(sc, want_s.astype(np.float64))


def test_all_ones_bf16_rounds_K_to_bfloat16():
    """K ones: the sum is exactly K; its bfloat16 is the nearest of the
    values 2^e (1 + f/128) -- 4097 and 4100 round to 4096, 4112 to 4096 (a
    tie, to even), 4113 to 4128."""
    M, N = 3, 2
    for K, bits in [(7, 0x40E0), (256, 0x4380), (4097, 0x4580), (4112, 0x4580), (4113, 0x4581)]:
        A = np.full(M * K, 0x3F80, np.uint16)
        B = np.full(K * N, 0x3F80, np.uint16)
        ref, sc = oracle.gemm(M, N, K, A, B, in_type=IN_BF16, out_type=OUT_BF16)
        assert np.all(ref == K) and np.all(sc == K)
        assert np.all(oracle.encbf16(ref.ravel()) == bits), K


def test_fp32_c_is_read_as_fp32():
    rng = np.random.default_rng(6)
    M, N, K = 4, 6, 3
    A = np.zeros(M * K, np.float16)
    B = np.zeros(K * N, np.float16)
    C = rng.uniform(-1, 1, M * N).astype(np.float32)
    ref, _ = oracle.gemm(M, N, K, A, B, C, alpha=1.0, beta=-3.0, out_type=OUT_F32)
    assert np.array_equal(ref.ravel(), -3.0 * C.astype(np.float64))


# -------------------------------------------------------------- invariants

def test_beta_zero_never_reads_c():
    rng = np.random.default_rng(8)
    M, N, K = 9, 7, 5
    A = rand_f16(rng, M * K)
    B = rand_f16(rng, K * N)
    C = np.full(M * N, np.nan, np.float16)
    ref, sc = oracle.gemm(M, N, K, A, B, C, alpha=1.0, beta=0.0)
    assert np.all(np.isfinite(ref)) and np.all(np.isfinite(sc))


def test_alpha_zero_gives_beta_c():
    rng = np.random.default_rng(9)
    M, N, K = 6, 5, 4
    A = rand_f16(rng, M * K)
    B = rand_f16(rng, K * N)
    C = rand_f16(rng, M * N)
    ref, _ = oracle.gemm(M, N, K, A, B, C, alpha=0.0, beta=0.5)
    assert np.array_equal(ref.ravel(), 0.5 * C.astype(np.float64))


def test_row_subset_and_threads_are_consistent():
    rng = np.random.default_rng(10)
    M, N, K = 50, 30, 70
    A = rand_f16(rng, M * K)
    B = rand_f16(rng, K * N)
    full1, s1 = oracle.gemm(M, N, K, A, B, nthreads=1)
    full8, s8 = oracle.gemm(M, N, K, A, B, nthreads=8)
    assert np.array_equal(full1, full8) and np.array_equal(s1, s8)
    rows = [49, 0, 17, 17, 3]
    sub, ssub = oracle.gemm(M, N, K, A, B, rows=rows, nthreads=3)
    assert np.array_equal(sub[0], full1[0][rows])
    assert np.array_equal(ssub[0], s1[0][rows])


def test_layout_only_changes_storage():
    """NN with B vs NT with B materialised transposed: identical references."""
    rng = np.random.default_rng(11)
    M, N, K = 21, 13, 29
    Am = rand_f16(rng, (M, K))
    Bm = rand_f16(rng, (K, N))
    r_nn, _ = oracle.gemm(M, N, K, to_storage(Am, ROW_MAJOR, K), to_storage(Bm, ROW_MAJOR, N))
    r_nt, _ = oracle.gemm(M, N, K, to_storage(Am, ROW_MAJOR, K), to_storage(Bm, COL_MAJOR, K),
                          layout_b=COL_MAJOR)
    r_tt, _ = oracle.gemm(M, N, K, to_storage(Am, COL_MAJOR, M), to_storage(Bm, COL_MAJOR, K),
                          layout_a=COL_MAJOR, layout_b=COL_MAJOR)
    assert np.array_equal(r_nn, r_nt) and np.array_equal(r_nn, r_tt)


def test_degenerate_sizes():
    A = np.zeros(0, np.float16)
    ref, sc = oracle.gemm(0, 5, 3, A, np.zeros(15, np.float16))
    assert ref.shape == (1, 0, 5)
    C = np.arange(6, dtype=np.float16)
    ref, _ = oracle.gemm(2, 3, 0, A, A, C, beta=2.0)       # K = 0: beta * C
    assert np.array_equal(ref.ravel(), 2.0 * C.astype(np.float64))
    with pytest.raises(RuntimeError):
        oracle.gemm(-1, 3, 3, A, A)


def test_fp32_accumulation_beats_fp16_accumulation():
    """The hand-written GEMM kernel page (§6.2) reports that summing a
    4096-long fp16 dot product in fp16 gives tens of times the relative error
    of fp32 accumulation.  Measured here against the oracle's exact-product
    fp64 sum; documents why the accumulators are fp32 (not a gate on the GPU)."""
    rng = np.random.default_rng(12)
    K = 4096
    ratios = []
    for _ in range(8):
        a = rng.uniform(0, 1, K).astype(np.float16)
        b = rng.uniform(0, 1, K).astype(np.float16)
        ref, _ = oracle.gemm(1, 1, K, a, b, layout_b=COL_MAJOR)
        exact = ref[0, 0, 0]
        s16 = np.float16(0)
        s32 = np.float32(0)
        for x, y in zip(a, b):
            p = np.float32(x) * np.float32(y)      # exact in fp32
            s16 = np.float16(s16 + np.float16(p))
            s32 = np.float32(s32 + p)
        ratios.append(abs(float(s16) - exact) / max(abs(float(s32) - exact), 1e-30))
    assert np.median(ratios) > 10.0


# --------------------------------------------------------- fused epilogue

from oracle import ACT_GELU, ACT_NONE, ACT_RELU, ACT_SILU  # noqa: E402


def scipy_activation(act, x):
    """The activations from library routines: ReLU max(x, 0), GELU
    x * Phi(x) (scipy.special.ndtr), SiLU x * sigmoid(x) (scipy.special.expit)."""
    import scipy.special as sp
    x = np.asarray(x, dtype=np.float64)
    if act == ACT_RELU:
        return np.maximum(x, 0.0)
    if act == ACT_GELU:
        return x * sp.ndtr(x)
    if act == ACT_SILU:
        return x * sp.expit(x)
    return x


ACT_PROBE = np.concatenate([np.linspace(-12, 12, 4801), [0.0, 1e-300, -1e-300, 1e-8, -1e-8,
                                                          40.0, -40.0, 700.0, -700.0, 1e4, -1e4]])


@pytest.mark.parametrize("act", [ACT_NONE, ACT_RELU, ACT_GELU, ACT_SILU])
def test_activation_against_scipy(act):
    got = oracle.activate(act, ACT_PROBE)
    want = scipy_activation(act, ACT_PROBE)
    assert np.allclose(got, want, rtol=1e-13, atol=1e-300), act


def test_activation_odd_part_and_landmarks():
    x = np.linspace(-9, 9, 3601)
    for act in (ACT_GELU, ACT_SILU):
        # x Phi(x) + x Phi(-x) = x, and x s(x) + x s(-x) = x
        d = oracle.activate(act, x) - oracle.activate(act, -x)
        assert np.allclose(d, x, rtol=1e-14, atol=1e-14), act
    # Phi(1) from the normal table, 1 / (1 + e^-1)
    assert abs(oracle.activate(ACT_GELU, [1.0])[0] - 0.8413447460685429) < 1e-15
    assert abs(oracle.activate(ACT_SILU, [1.0])[0] - 0.7310585786300049) < 1e-15
    assert oracle.activate(ACT_RELU, [-3.0, 2.5]).tolist() == [0.0, 2.5]
    assert oracle.activate(ACT_GELU, [0.0])[0] == 0.0 and oracle.activate(ACT_SILU, [0.0])[0] == 0.0


def _epilogue_case(lib, M, N, K, la, lb, act, rng, alpha=-0.75, beta=0.5):
    A_log = rand_f16(rng, (M, K))
    B_log = rand_f16(rng, (K, N))
    C_log = rng.uniform(-2, 2, (M, N)).astype(np.float32)
    bias = rng.uniform(-1, 1, N).astype(np.float32)
    lda = K if la == ROW_MAJOR else M
    ldb = N if lb == ROW_MAJOR else K
    A = to_storage(A_log, la, lda)
    B = to_storage(B_log, lb, ldb)
    ref, sc = oracle.gemm(M, N, K, A, B, C_log.ravel(), alpha=alpha, beta=beta,
                          layout_a=la, layout_b=lb, out_type=OUT_F32, bias=bias,
                          activation=act, lib=lib)
    ex, exs = exact_product(A_log, B_log, C_log, alpha, beta)
    for i in range(M):
        for j in range(N):
            x = ex[i, j] + Fraction(float(bias[j]))
            s_x = exs[i, j] + abs(Fraction(float(bias[j])))
            assert abs(Fraction(sc[0, i, j]) - s_x) <= s_x * Fraction(2.0 ** -50), (i, j)
            if act == ACT_NONE:
                assert abs(Fraction(ref[0, i, j]) - x) <= s_x * Fraction(2.0 ** -50), (i, j)
            else:
                want = float(scipy_activation(act, float(x)))
                tol = 1.2 * 2.0 ** -48 * float(s_x) + 1e-13 * abs(want) + 1e-300
                assert abs(ref[0, i, j] - want) <= tol, (M, N, K, la, lb, act, i, j)


def test_epilogue_bias_and_activation_brute_force(lib=None):
    rng = np.random.default_rng(13)
    for (M, N, K) in [(1, 1, 1), (3, 5, 7), (6, 4, 9), (2, 9, 3)]:
        for la, lb in LAYOUTS:
            for act in (ACT_NONE, ACT_RELU, ACT_GELU, ACT_SILU):
                _epilogue_case(lib, M, N, K, la, lb, act, rng)


def test_epilogue_activation_follows_the_residual_add():
    """act(alpha A B + beta C + bias): with A B = 2, beta C = -3 and bias 0
    ReLU gives 0 (ReLU before the add would give -1)."""
    A = np.array([1.0, 1.0], np.float16)          # 1 x 2
    B = np.array([1.0, 1.0], np.float16)          # 2 x 1
    C = np.array([-3.0], np.float32)
    ref, sc = oracle.gemm(1, 1, 2, A, B, C, beta=1.0, out_type=OUT_F32,
                          bias=np.zeros(1, np.float32), activation=ACT_RELU)
    assert ref[0, 0, 0] == 0.0 and sc[0, 0, 0] == 5.0
    ref, _ = oracle.gemm(1, 1, 2, A, B, C, beta=1.0, out_type=OUT_F32,
                         bias=np.array([4.5], np.float32), activation=ACT_RELU)
    assert ref[0, 0, 0] == 3.5
    with pytest.raises(RuntimeError):
        oracle.gemm(1, 1, 2, A, B, C, beta=1.0, out_type=OUT_F32, activation=7)
