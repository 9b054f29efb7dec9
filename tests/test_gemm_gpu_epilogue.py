"""GPU parity of the fused epilogue C = act(alpha A B + beta C + bias[n])
against the oracle, through the C ABI (gemm_f16f32_set_epilogue).

A plan with an epilogue runs the epilogue instantiation of its kernel, so
these tests walk every kernel family -- the 256 tile, the 128 tile on two
and four slots, split-K, the streaming tiles, the staged tiles (128-bit and
element-wide loads), batches -- with each activation, a bias, a residual
(beta = 1), fp16 / bf16 / fp32 C, and ragged edges.  The bias buffer holds
NaN past its N values, so a read beyond column N - 1 would show.  Bound:
tests/parity.py, with the activation's Lipschitz factor.
"""
import numpy as np
import pytest
import torch

import gemm_inputs as gi
import mixed_precision_gemm_amd as mpg
from gemm_inputs import COL_MAJOR, OUT_BF16, OUT_F16, OUT_F32, ROW_MAJOR
from parity import c_logical, check_bound, oracle_for, run_case, sample_rows

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

NONE, RELU, GELU, SILU = (mpg.GEMM_ACT_NONE, mpg.GEMM_ACT_RELU, mpg.GEMM_ACT_GELU,
                          mpg.GEMM_ACT_SILU)
ACTS = [NONE, RELU, GELU, SILU]
ANAME = {NONE: "bias", RELU: "relu", GELU: "gelu", SILU: "silu"}


def make_bias(N, seed, scale=1.0):
    """N uniform values on the device, followed by NaN (never to be read)."""
    g = torch.Generator("cpu").manual_seed(seed)
    full = torch.full((N + 64,), float("nan"), dtype=torch.float32)
    full[:N] = (torch.rand(N, generator=g) * 2 - 1) * scale
    return full.cuda()


def epilogue_parity(case, act, rows=None, bias_scale=1.0, with_bias=True, what=""):
    bias = make_bias(case.N, seed=case.N + act, scale=bias_scale) if with_bias else None
    dC = run_case(case, bias=bias, act=act)
    torch.cuda.synchronize()
    got = c_logical(case, dC.cpu(), rows)
    ref, scale = oracle_for(case, rows, bias=bias, act=act)
    assert not np.isnan(got).any(), f"{what}: NaN in C (bias read past N?)"
    return check_bound(got, ref, scale, case.out_type, what, act=act)


def kernel_of(case):
    with mpg.Plan(case.M, case.N, case.K, case.layout_a, case.layout_b, case.out_type,
                  case.lda, case.ldb, case.ldc, case.batch, case.stride_a, case.stride_b,
                  case.stride_c, dtype=case.meta.get("in_dtype", "f16")) as p:
        return p.kernel


# (shape, kwargs, kernel-name fragment, sampled rows?)
FAMILIES = [
    ((4096, 4096, 392), dict(layout_b=COL_MAJOR), "256x256", True),
    ((2304, 2304, 328), {}, "128x128x64m16_", False),
    ((1000, 1000, 1000), dict(layout_a=COL_MAJOR), "m16d4_tn", False),
    ((256, 256, 32768), {}, "_sk8", False),
    ((16, 4096, 4096), dict(layout_b=COL_MAJOR), "stream16x16", False),
    ((40, 4096, 1024), dict(layout_b=COL_MAJOR), "stream32x64", False),
    ((40, 512, 8448), dict(layout_b=COL_MAJOR), "stream64x16", False),
    ((127, 257, 33), {}, "narrow", False),
    ((64, 96, 200), dict(layout_a=COL_MAJOR, layout_b=COL_MAJOR), "vec16", False),
    ((4097, 63, 1025), {}, "_sk2_pkab", False),                   # repacked, split-K
    ((7, 4097, 4099), dict(layout_b=COL_MAJOR), "stream16x16_nt_direct_pkab", False),
]


@pytest.mark.parametrize("act", ACTS)
@pytest.mark.parametrize("shape,kw,frag,sampled", FAMILIES)
def test_epilogue_every_kernel_family(shape, kw, frag, sampled, act):
    """Residual (beta = 1) plus bias plus activation; fp16 C for the odd
    activations, fp32 C for the others."""
    M, N, K = shape
    out = OUT_F16 if act in (RELU, SILU) else OUT_F32
    case = gi.make_case(M, N, K, out_type=out, alpha=0.75, beta=1.0, seed=90 + act, **kw)
    assert frag in kernel_of(case), kernel_of(case)
    rows = sample_rows(M, n_random=48) if sampled else None
    epilogue_parity(case, act, rows=rows, what=f"{shape} {ANAME[act]}")


@pytest.mark.parametrize("act", [RELU, GELU, SILU])
def test_epilogue_activation_without_bias_and_beta0(act):
    case = gi.make_case(600, 520, 264, layout_b=COL_MAJOR, seed=97)
    epilogue_parity(case, act, with_bias=False, what=f"no bias {ANAME[act]}")


@pytest.mark.parametrize("act", ACTS)
def test_epilogue_bf16(act):
    """bfloat16 inputs and C with the epilogue (the 128 tile and a streaming
    tile)."""
    for shape, kw in [((1000, 1000, 1000), {}), ((32, 11008, 4096), dict(layout_b=COL_MAJOR))]:
        case = gi.make_case(*shape, in_dtype="bf16", out_type=OUT_BF16, beta=1.0, seed=77, **kw)
        epilogue_parity(case, act, what=f"bf16 {shape} {ANAME[act]}")


def test_epilogue_batched_and_wide_range():
    """A batch shares the bias; pre-activations spread over +-40 reach the
    activations' tails (GELU's erfc and SiLU's overflowing exponential)."""
    case = gi.make_case(64, 64, 64, batch=512, out_type=OUT_F32, dist_a="normal",
                        dist_b="normal", sigma_a=0.125, sigma_b=0.125, seed=98)
    for act in ACTS:
        epilogue_parity(case, act, what=f"batched {ANAME[act]}")
    wide = gi.make_case(512, 384, 256, out_type=OUT_F32, dist_a="normal", dist_b="normal",
                        sigma_a=1.0, sigma_b=1.0, seed=99)
    for act in (GELU, SILU):
        epilogue_parity(wide, act, bias_scale=30.0, what=f"wide {ANAME[act]}")


@pytest.mark.parametrize("shape", [(8192, 8192, 8192)])
def test_epilogue_headline_size_sampled(shape):
    """The 8192^3 NN product with residual, bias and GELU, sampled rows."""
    case = gi.headline_case(shape[0])
    epilogue_parity(case, GELU, rows=sample_rows(shape[0], n_random=64), what="8192^3 gelu")


def test_epilogue_reset_restores_the_plain_product():
    """Clearing the epilogue (NULL bias, GEMM_ACT_NONE) runs the plain
    kernel again: its result equals a plan that never had one, bit for bit."""
    case = gi.make_case(1024, 768, 512, beta=1.0, seed=100)
    dA, dB, _ = case.A.cuda(), case.B.cuda(), None
    bias = make_bias(case.N, 5)
    outs = []
    for reset in (False, True):
        dC = case.C.cuda()
        with mpg.Plan(case.M, case.N, case.K) as p:
            if reset:
                p.set_epilogue(bias, GELU)
                p.set_epilogue(None, NONE)
            p.run(dA, dB, dC, case.alpha, case.beta)
        torch.cuda.synchronize()
        outs.append(dC.cpu())
    assert torch.equal(outs[0].view(torch.int16), outs[1].view(torch.int16))


def test_epilogue_torch_wrapper():
    M, N, K = 300, 200, 136
    case = gi.make_case(M, N, K, seed=101)
    A = case.A.reshape(M, K).cuda()
    B = case.B.reshape(K, N).cuda()
    bias = make_bias(N, 7)
    C = mpg.gemm(A, B, bias=bias[:N], activation=SILU)
    torch.cuda.synchronize()
    ref, scale = oracle_for(case, bias=bias, act=SILU)
    check_bound(C.cpu().to(torch.float64).numpy()[None], ref, scale, OUT_F16, "wrapper silu",
                act=SILU)


@pytest.mark.parametrize("act", ACTS)
def test_epilogue_degenerate_sizes(act):
    """K = 0: C = act(beta C + bias); M = 0: no-op even with an epilogue."""
    case = gi.make_case(300, 136, 0, lda=1, beta=1.5, seed=102)
    epilogue_parity(case, act, what=f"K=0 {ANAME[act]}")
    with mpg.Plan(0, 64, 64) as p:
        p.set_epilogue(None, act)
        p.run(0, 0, 0, 1.0, 0.0)


def _sweep_with_epilogue(n, seed):
    """The plain GEMM sweep's seeded shapes (every kernel class, random
    layouts, padding, batch, alpha/beta), each with a random activation and
    input type and a bias on two cases of three."""
    from test_gemm_gpu import _sweep_cases
    rng = np.random.default_rng(seed)
    return [(args, int(rng.integers(0, 4)), bool(rng.random() < 0.67),
             "bf16" if rng.random() < 0.4 else "f16") for args in _sweep_cases(n, seed)]


@pytest.mark.parametrize("sweep", _sweep_with_epilogue(24, 4242))
def test_epilogue_random_sweep(sweep):
    (M, N, K, la, lb, pad, batch, out_type, alpha, beta), act, with_bias, dt = sweep
    lda = (K if la == ROW_MAJOR else M) + pad
    ldb = (N if lb == ROW_MAJOR else K) + pad
    if dt == "bf16" and out_type == OUT_F16:
        out_type = OUT_BF16
    case = gi.make_case(M, N, K, layout_a=la, layout_b=lb, out_type=out_type, alpha=alpha,
                        beta=beta, batch=batch, lda=lda, ldb=ldb, in_dtype=dt,
                        seed=(M * 7919 + N * 31 + K) % 1000)
    rows = None if M * N * K * batch <= (1 << 27) else sample_rows(M, n_random=16, tiles=(256, 128))
    epilogue_parity(case, act, rows=rows, with_bias=with_bias,
                    what=f"{kernel_of(case)} {sweep}")
