"""GPU parity of the fused attention and row softmax kernels against the
CPU oracle (oracle/ref_attention.c), through the C ABI.

Acceptance bound for attention (per output, from the kernel's arithmetic):
    |O - O_ref| <= (2e-3 + 4 D 2^-24 a_i) * E_ic + (fp16 O ? ulp16(|O_ref|) : 0)
with E_ic = sum_j P_ij |V_jc| and a_i = max_j scale sum_d |Q_id K_jd| from the
oracle.  P is rounded to binary16 before the product with V (relative 2^-11 =
4.9e-4 of each term of E); fp32 sums over the keys and the rescaling factors
of the online softmax stay far below 1e-4 of E; a score's fp32 error is at
most D 2^-24 a_i and moves each weight by at most twice that relative
(exp turns an absolute score error into a relative weight error); the final
division and rounding add one rounding of O.

Row softmax bound: |y - y_ref| <= 1e-6 (4 + n/256 + |x| + |x - m|) y_ref +
(fp16 y ? ulp16(y_ref) : 2^-126): x log2 e and x - m are rounded in fp32 (2^-24
relative to |x| and |x - m|, turned into a relative error of y by exp),
v_exp_f32 and the reciprocal add a few ulp, and each thread sums at most n/256
terms before an 8-level merge; an fp32 weight below the smallest normal
fp32 value may be returned as zero.
"""
import math

import numpy as np
import pytest
import torch

import mixed_precision_gemm_amd as mpg
import oracle
from parity import oracle_threads, ulp16

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def draw(shape, seed, scale=1.0):
    g = torch.Generator("cpu").manual_seed(seed)
    return (torch.randn(shape, generator=g) * scale).half()


def attn_bound(ref, err, smax, D, out_f32):
    b = (2e-3 + 4 * D * 2.0 ** -24 * smax[..., None]) * err
    if not out_f32:
        b = b + ulp16(ref)
    return b


def run_attention(B, H, Sq, Sk, D, causal=False, seed=0, layout="bhsd", out_f32=False,
                  scale=None, rows=None, qscale=1.0):
    """Runs the GPU kernel and the oracle on the same seeded Q, K, V; checks
    the bound; returns (gpu O as float64 (B, H, Sq, D), kernel name)."""
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    if layout == "bhsd":
        q = draw((B, H, Sq, D), seed, qscale)
        k = draw((B, H, Sk, D), seed + 1)
        v = draw((B, H, Sk, D), seed + 2)
    else:   # (B, S, H, D) storage, viewed as (B, H, S, D)
        q = draw((B, Sq, H, D), seed, qscale).transpose(1, 2)
        k = draw((B, Sk, H, D), seed + 1).transpose(1, 2)
        v = draw((B, Sk, H, D), seed + 2).transpose(1, 2)
    dq, dk, dv = q.cuda(), k.cuda(), v.cuda()
    out = torch.full((B, H, Sq, D), float("nan"), dtype=torch.float32 if out_f32 else torch.float16,
                     device="cuda")
    st3 = lambda t: (t.stride(0), t.stride(1), t.stride(2))
    st, h = mpg.attn_f16_plan(B, H, Sq, Sk, D, st3(dq), st3(dk), st3(dv), st3(out), int(causal),
                              mpg.GEMM_OUT_F32 if out_f32 else mpg.GEMM_OUT_F16)
    assert st == mpg.GEMM_OK, mpg.gemm_f16f32_status_string(st)
    name = mpg.attn_f16_plan_kernel(h)
    st = mpg.attn_f16_run(h, dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), out.data_ptr(), scale,
                          torch.cuda.current_stream().cuda_stream)
    mpg.attn_f16_destroy(h)
    assert st == mpg.GEMM_OK
    torch.cuda.synchronize()
    got = out.cpu().double().numpy()
    u16 = lambda t: t.contiguous().view(torch.int16).numpy().view(np.uint16).ravel()
    # the oracle reads the same storage with the same strides
    base = lambda t: t.as_strided((t.untyped_storage().nbytes() // 2,), (1,))
    ref, err, smax = oracle.attention(
        B, H, Sq, Sk, D, u16(base(q)), u16(base(k)), u16(base(v)), scale=scale, causal=causal,
        q_strides=st3(q), k_strides=st3(k), v_strides=st3(v), rows=rows,
        nthreads=oracle_threads())
    if rows is not None:
        got = got[:, :, rows]
    bound = attn_bound(ref, err, smax, D, out_f32)
    diff = np.abs(got - ref)
    bad = ~(diff <= bound)
    assert not bad.any(), (f"{name}: {int(bad.sum())} of {bad.size} outside the bound; first "
                           f"{[(tuple(i), got[tuple(i)], ref[tuple(i)], bound[tuple(i)]) for i in np.argwhere(bad)[:4]]}")
    return got, name


# (B, H, Sq, Sk, D) shapes: the batched Q K^T configuration as attention
# (256 heads of 128 x 128, head dimension 64), ragged lengths off the 128-row
# and 64-key tiles, single rows and keys, and both head dimensions.
SHAPES = [(2, 128, 128, 128, 64), (1, 3, 200, 333, 64), (2, 2, 77, 50, 128), (1, 1, 1, 1, 64),
          (1, 2, 1, 300, 128), (1, 1, 300, 1, 64), (3, 1, 129, 65, 128), (1, 4, 256, 256, 128)]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", SHAPES)
def test_attention_parity(shape, causal):
    B, H, Sq, Sk, D = shape
    _, name = run_attention(B, H, Sq, Sk, D, causal=causal, seed=B * 7 + Sq)
    assert name == f"attn_fwd_d{D}_q128_k64{'_causal' if causal else ''}_f16"


@pytest.mark.parametrize("D", [64, 128])
def test_attention_fp32_output_and_heads_interleaved_layout(D):
    """O in fp32, and Q, K, V stored (batch, seq, head, d) as models keep them."""
    run_attention(2, 3, 150, 190, D, causal=True, seed=11, layout="bshd", out_f32=True)
    run_attention(2, 3, 150, 190, D, causal=False, seed=12, layout="bshd")


def test_attention_fully_masked_rows_are_zero():
    """Causal with Sq > Sk: query i sees keys up to i + Sk - Sq, so the first
    Sq - Sk rows see none and are written as zeros; Sk = 0 masks every row."""
    got, _ = run_attention(1, 2, 300, 100, 64, causal=True, seed=13)
    assert np.array_equal(got[:, :, :200], np.zeros((1, 2, 200, 64)))
    out = torch.full((1, 1, 40, 64), float("nan"), dtype=torch.float16, device="cuda")
    q = torch.zeros((1, 1, 40, 64), dtype=torch.float16, device="cuda")
    mpg.attention(q, q[:, :, :0], q[:, :, :0], out=out)
    torch.cuda.synchronize()
    assert torch.equal(out.cpu(), torch.zeros_like(out.cpu()))


def test_attention_large_scores():
    """Scores spanning tens of units (Q scaled by 8): the online maximum moves
    across tiles and exp would overflow without it."""
    run_attention(1, 2, 256, 512, 128, causal=False, seed=14, qscale=8.0)
    run_attention(1, 2, 256, 512, 64, causal=True, seed=15, qscale=8.0)


@pytest.mark.parametrize("causal", [False, True])
def test_attention_long_sequence_sampled(causal):
    """4096 x 4096 with head dimension 128 on sampled query rows."""
    rows = np.unique(np.concatenate([[0, 1, 127, 128, 4095], np.random.default_rng(3).integers(0, 4096, 60)]))
    run_attention(1, 2, 4096, 4096, 128, causal=causal, seed=16, rows=rows)


def test_attention_run_to_run_bitwise():
    q, k, v = (draw((2, 4, 333, 128), s).cuda() for s in (21, 22, 23))
    a = mpg.attention(q, k, v, causal=True)
    b = mpg.attention(q, k, v, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


# ------------------------------------------------------------ row softmax

def softmax_bound(ref, x, m, n, out_f32):
    with np.errstate(invalid="ignore"):
        spread = np.where(np.isfinite(x), np.abs(x) + np.abs(x - m[:, None]), 0.0)
    b = 1e-6 * (4 + n / 256 + spread) * ref
    # fp32 y: weights below the smallest normal fp32 (2^-126) may come out as
    # zero (v_exp_f32 does not produce subnormals); fp16 y: one rounding
    b = b + (2.0 ** -126 if out_f32 else ulp16(ref))
    return b


@pytest.mark.parametrize("cols", [1, 100, 2048, 2049, 4096, 8192, 8193, 20000])
@pytest.mark.parametrize("in32,out32", [(False, False), (True, True), (False, True)])
@pytest.mark.parametrize("aligned", [False, True])
def test_softmax_rows_parity(cols, in32, out32, aligned):
    """Rows of any length; with aligned rows (length, leading dimension and
    bases multiples of 8 elements and 16 bytes) the 16-byte-access kernel
    takes rows of up to 8192."""
    rows = 37
    ld = (cols + 7) // 8 * 8 + 8 if aligned else cols + 5
    g = torch.Generator("cpu").manual_seed(cols)
    x = torch.randn(rows, ld, generator=g) * 6
    x[:, : cols // 3] -= 40.0                                 # maximum late in the row
    x[3, :cols] = float("-inf")                              # a fully masked row
    x[5, ::3] = float("-inf")                                # masked elements
    x[7, :cols] += 300.0                                     # large values
    xt = x.float() if in32 else x.half()
    y = torch.full((rows, ld), float("nan"), dtype=torch.float32 if out32 else torch.float16)
    dx, dy = xt.cuda(), y.cuda()
    st = mpg.attn_softmax_rows(rows, cols, dx.data_ptr(), ld, int(in32), dy.data_ptr(), ld,
                               int(out32), torch.cuda.current_stream().cuda_stream)
    assert st == mpg.GEMM_OK
    torch.cuda.synchronize()
    got = dy.cpu().double().numpy()[:, :cols]
    assert np.all(np.isnan(dy.cpu().double().numpy()[:, cols:]))    # padding untouched
    xs = xt.numpy() if in32 else xt.view(torch.int16).numpy().view(np.uint16)
    ref = oracle.softmax(rows, cols, xs.ravel(), ld=ld)
    xv = xt.double().numpy()[:, :cols]
    m = np.max(xv, axis=1)
    bound = softmax_bound(ref, xv, m, cols, out32)
    assert np.array_equal(got[3], np.zeros(cols))
    bad = ~(np.abs(got - ref) <= bound)
    assert not bad.any(), f"{int(bad.sum())} outside; first {np.argwhere(bad)[:4].tolist()}"


def test_softmax_in_place_and_torch_wrapper():
    x = (torch.randn(64, 3000, generator=torch.Generator().manual_seed(5)) * 4).cuda()
    want = torch.softmax(x.double(), dim=1)
    y = mpg.softmax(x.clone())
    x2 = x.clone()
    mpg.softmax(x2, out=x2)
    torch.cuda.synchronize()
    assert torch.allclose(y.double(), want, rtol=1e-4, atol=1e-12)
    assert torch.equal(x2, y)
