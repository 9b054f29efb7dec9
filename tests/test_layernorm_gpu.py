"""GPU parity of the linear layer fused with its residual and LayerNorm
(gemm_f16f32_set_layernorm) against the oracle (oracle/ref_layernorm.c),
through the C ABI.

Acceptance bound per output (derived from the arithmetic):
    |Y - Y_ref| <= 1.1 T + 1e-5 |gamma_j| (|Z_ij - mu_i| + A_i) / s_i
                   + 1e-6 |beta_j| + (16-bit C ? one rounding of Y_ref : 0)
T (from the oracle) carries the GEMM bound 2e-3 S to first order through the
normalisation: every element of the row of Z is within D_i = 2e-3 max_j S_ij
of exact, which moves the mean and s = sqrt(var + eps) by at most D_i each
(1.1 covers the second-order terms).  The row pass itself runs in fp32: its
sums (at most N/256 terms per thread, then an 8-level tree) err by a few
1e-6 of A_i = mean |Z_i|, relative to s_i; the division, the scale and the
shift add a few ulp.
"""
import numpy as np
import pytest
import torch

import gemm_inputs as gi
import mixed_precision_gemm_amd as mpg
import oracle
from gemm_inputs import COL_MAJOR, OUT_BF16, OUT_F16, OUT_F32, ROW_MAJOR
from parity import c_logical, in_dtype, oracle_threads, sample_rows, to_device, ulp16, ulpbf16

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def params(N, seed):
    g = torch.Generator("cpu").manual_seed(seed)
    bias = torch.randn(N, generator=g)
    gamma = 1 + 0.3 * torch.randn(N, generator=g)
    beta_ln = 0.2 * torch.randn(N, generator=g)
    return bias, gamma, beta_ln


def ln_parity(case, eps=1e-5, with_bias=True, rows=None, seed=1):
    """Runs the case with the LayerNorm epilogue and checks the bound; returns
    the kernel name."""
    bias, gamma, beta_ln = params(case.N, seed)
    dA, dB, dC = to_device(case)
    dbias, dgamma, dbeta = bias.cuda(), gamma.cuda(), beta_ln.cuda()
    p = mpg.Plan(case.M, case.N, case.K, case.layout_a, case.layout_b, case.out_type, case.lda,
                 case.ldb, case.ldc, case.batch, case.stride_a, case.stride_b, case.stride_c,
                 dtype=in_dtype(case))
    try:
        if with_bias:
            p.set_epilogue(dbias, mpg.GEMM_ACT_NONE)
        p.set_layernorm(dgamma, dbeta, eps)
        p.run(dA, dB, dC, case.alpha, case.beta)
        torch.cuda.synchronize()
        kernel = p.kernel
    finally:
        p.close()
    got = c_logical(case, dC.cpu(), rows)
    u16 = lambda t: t.view(torch.int16).numpy().view(np.uint16)
    cin = u16(case.C) if case.out_type in (OUT_F16, OUT_BF16) else case.C.numpy()
    y, t, st = oracle.gemm_layernorm(
        case.M, case.N, case.K, u16(case.A), u16(case.B), cin, gamma=gamma.numpy(),
        beta_ln=beta_ln.numpy(), eps=eps, alpha=case.alpha, beta=case.beta,
        bias=bias.numpy() if with_bias else None, layout_a=case.layout_a,
        layout_b=case.layout_b, out_type=case.out_type,
        in_type=oracle.IN_BF16 if in_dtype(case) == "bf16" else oracle.IN_F16,
        lda=case.lda, ldb=case.ldb, ldc=case.ldc, batch=case.batch, stride_a=case.stride_a,
        stride_b=case.stride_b, stride_c=case.stride_c, rows=rows, nthreads=oracle_threads())
    z = (y - beta_ln.numpy()[None, None, :]) / np.where(gamma.numpy() == 0, 1, gamma.numpy())
    dev = np.abs(z) * st[..., 1:2]                      # |Z - mu| from Y
    g = np.abs(gamma.numpy().astype(np.float64))
    bound = (1.1 * t + 1e-5 * g * (dev + st[..., 2:3]) / st[..., 1:2]
             + 1e-6 * np.abs(beta_ln.numpy().astype(np.float64)))
    if case.out_type == OUT_F16:
        bound = bound + ulp16(y)
    elif case.out_type == OUT_BF16:
        bound = bound + ulpbf16(y)
    bad = ~(np.abs(got - y) <= bound)
    assert not bad.any(), (f"{kernel}: {int(bad.sum())} of {bad.size} outside; first "
                           f"{[(tuple(i), got[tuple(i)], y[tuple(i)], bound[tuple(i)]) for i in np.argwhere(bad)[:4]]}")
    return kernel


def linear_residual(M, N, K=4096, seed=0, in_dtype="f16"):
    """The transformer linear-layer workload with a residual: X ~ N(0,1), W
    stored N x K ~ N(0, 0.02), residual C ~ N(0, 1), beta = 1."""
    out = OUT_BF16 if in_dtype == "bf16" else OUT_F16
    return gi.make_case(M, N, K, layout_b=COL_MAJOR, dist_a="normal", dist_b="normal",
                        dist_c="normal", sigma_a=1.0, sigma_b=0.02, sigma_c=1.0, beta=1.0,
                        seed=seed, in_dtype=in_dtype, out_type=out)


@pytest.mark.parametrize("M,N", [(16, 4096), (128, 4096), (128, 11008), (2048, 4096), (512, 12288)])
def test_layernorm_linear_layer_shapes(M, N):
    case = linear_residual(M, N, seed=M + N)
    rows = sample_rows(M, n_random=64) if M > 256 else None
    ln_parity(case, rows=rows)


@pytest.mark.parametrize("shape,kw,frag", [
    ((300, 260, 1500), dict(layout_a=COL_MAJOR), "128x128"),        # two-slot 128 tile
    ((16, 2048, 4096), {}, "_sk"),                                   # split-K
    ((1000, 1001, 999), {}, "_pk"),                                  # repacked operands
    ((64, 64, 64), dict(batch=8), "small64"),                        # one wave per product
    ((64, 64, 64), dict(batch=8, layout_a=COL_MAJOR), "64x64"),      # batched staged tile
    ((127, 257, 33), {}, "narrow"),                                  # element-wide loads
    ((4096, 4096, 4096), dict(layout_b=COL_MAJOR), "256x256"),       # the 256 tile
])
def test_layernorm_on_every_kernel_family(shape, kw, frag):
    M, N, K = shape
    batch = kw.pop("batch", 1)
    case = gi.make_case(M, N, K, alpha=0.5, beta=-1.0, batch=batch, seed=M + K,
                        dist_c="normal", **kw)
    rows = sample_rows(M, n_random=48) if M >= 1000 else None
    kernel = ln_parity(case, rows=rows)
    assert frag in kernel, kernel


def test_layernorm_fp32_and_bf16_outputs_and_k_zero():
    ln_parity(gi.make_case(200, 300, 250, out_type=OUT_F32, beta=1.0, seed=3))
    ln_parity(linear_residual(64, 2048, seed=4, in_dtype="bf16"))
    ln_parity(gi.make_case(100, 128, 0, lda=8, beta=1.0, dist_c="normal", seed=5))


def test_layernorm_long_rows_and_no_bias():
    """N = 20000 takes the row pass that reads a row three times."""
    ln_parity(gi.make_case(64, 20000, 256, layout_b=COL_MAJOR, beta=0.0, seed=6), with_bias=False)


def test_layernorm_constant_rows_give_the_shift():
    """B with equal columns: every row of Z is constant (the residual too), so
    every output is beta_ln within the bound (the variance is eps alone)."""
    M, N, K = 64, 256, 64
    case = gi.make_case(M, N, K, dist_a="integer", dist_b="integer", seed=7)
    col = case.B.view(K, N)[:, :1].clone()
    case.B.view(K, N)[:] = col
    ln_parity(case, with_bias=False, eps=1e-3)


def test_layernorm_reset_and_determinism():
    """Two runs give the same bits; removing the normalisation restores the
    plain GEMM bit for bit."""
    case = linear_residual(256, 4096, seed=8)
    bias, gamma, beta_ln = (t.cuda() for t in params(case.N, 9))
    dA, dB, dC = to_device(case)
    outs = []
    with mpg.Plan(case.M, case.N, case.K, case.layout_a, case.layout_b, case.out_type,
                  case.lda, case.ldb, case.ldc) as p:
        p.set_layernorm(gamma, beta_ln, 1e-5)
        for _ in range(2):
            c = dC.clone()
            p.run(dA, dB, c, 1.0, 1.0)
            outs.append(c)
        p.set_layernorm(None)
        c1 = dC.clone()
        p.run(dA, dB, c1, 1.0, 1.0)
    with mpg.Plan(case.M, case.N, case.K, case.layout_a, case.layout_b, case.out_type,
                  case.lda, case.ldb, case.ldc) as q:
        c2 = dC.clone()
        q.run(dA, dB, c2, 1.0, 1.0)
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1])
    assert torch.equal(c1, c2)
