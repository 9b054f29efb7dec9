"""GPU parity of the implicit-GEMM convolution against the oracle
(oracle/ref_conv.c), through the C ABI.

The convolution is a GEMM of the same fp16 products summed in fp32 over
R S C terms, so the GEMM's acceptance bound applies unchanged:
    |y - y_ref| <= 2e-3 S + (fp16 y ? ulp16(|y_ref|) : 0)
with S = |alpha| sum |x w| + |beta| |y_old| + |bias| from the oracle (ReLU
is 1-Lipschitz; the fused activations carry the GEMM epilogue's 1e-5 |y|).
"""
import numpy as np
import pytest
import torch

import mixed_precision_gemm_amd as mpg
import oracle
from parity import LIPSCHITZ, oracle_threads, ulp16

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def run_conv(N, H, W, C, K, R, S, stride=(1, 1), pad=(0, 0), dil=(1, 1), seed=0, alpha=1.0,
             beta=0.0, bias=False, act=0, out_f32=False, rows=None, offset=0):
    g = torch.Generator("cpu").manual_seed(seed)
    x = (torch.randn(N * H * W * C, generator=g)).half()
    w = (torch.randn(K * R * S * C, generator=g) * (1.0 / np.sqrt(R * S * C))).half()
    st, h = mpg.conv_f16_plan(N, H, W, C, K, R, S, stride, pad, dil, int(out_f32))
    assert st == mpg.GEMM_OK, mpg.gemm_f16f32_status_string(st)
    _, P, Q = mpg.conv_f16_output_size(h)
    M = N * P * Q
    ydt = torch.float32 if out_f32 else torch.float16
    y0 = torch.randn(M * K, generator=g).to(ydt) if beta != 0 else torch.full((M * K,), float("nan"), dtype=ydt)
    b = torch.randn(K, generator=g) if bias else None
    # offset > 0 places x and w off 16-byte alignment (the element-wise path)
    dx = torch.zeros(x.numel() + offset, dtype=torch.float16, device="cuda")
    dw = torch.zeros(w.numel() + offset, dtype=torch.float16, device="cuda")
    dx[offset:] = x.cuda()
    dw[offset:] = w.cuda()
    dy = y0.cuda()
    db = b.cuda() if b is not None else None
    kernel = mpg.conv_f16_plan_kernel(h)
    st = mpg.conv_f16_run(h, dx[offset:].data_ptr(), dw[offset:].data_ptr(), dy.data_ptr(), alpha,
                          beta, None if db is None else db.data_ptr(), act,
                          torch.cuda.current_stream().cuda_stream)
    mpg.conv_f16_destroy(h)
    assert st == mpg.GEMM_OK
    torch.cuda.synchronize()
    got = dy.cpu().double().numpy().reshape(M, K)
    u16 = lambda t: t.view(torch.int16).numpy().view(np.uint16)
    yold = (y0.numpy() if out_f32 else u16(y0)) if beta != 0 else None
    ref, scale = oracle.conv2d(N, H, W, C, K, R, S, u16(x), u16(w), yold, stride=stride, pad=pad,
                               dil=dil, alpha=alpha, beta=beta,
                               bias=None if b is None else b.numpy(), activation=act,
                               out_type=oracle.OUT_F32 if out_f32 else oracle.OUT_F16, rows=rows,
                               nthreads=oracle_threads())
    if rows is not None:
        got = got[rows]
    bound = LIPSCHITZ[act] * 2e-3 * scale + (1e-5 * np.abs(ref) if act else 0.0)
    if not out_f32:
        bound = bound + ulp16(ref)
    bad = ~(np.abs(got - ref) <= bound)
    assert not bad.any(), (f"{kernel}: {int(bad.sum())} of {bad.size} outside; first "
                           f"{[(tuple(i), got[tuple(i)], ref[tuple(i)], bound[tuple(i)]) for i in np.argwhere(bad)[:4]]}")
    return kernel


# (N, H, W, C, K, R, S, stride, pad, dil, kernel fragment)
SHAPES = [
    (2, 16, 16, 64, 64, 3, 3, (1, 1), (1, 1), (1, 1), "64x64x64_vec16"),        # a 3x3 layer
    (16, 33, 33, 32, 136, 3, 3, (1, 1), (1, 1), (1, 1), "128x128x64_vec16"),    # the 128 tile
    (32, 32, 32, 16, 40, 3, 3, (1, 1), (1, 1), (1, 1), "256x64x64_vec16"),      # 256 x 64, K < 64
    (16, 32, 32, 5, 24, 3, 3, (1, 1), (1, 1), (1, 1), "128x64x64_narrow"),      # 128 x 64, C = 5
    (4, 14, 14, 256, 96, 1, 1, (1, 1), (0, 0), (1, 1), "vec16"),                # 1x1 (a GEMM)
    (2, 17, 19, 16, 40, 3, 5, (2, 3), (1, 2), (1, 1), "vec16"),                 # strides, odd sizes
    (1, 20, 20, 24, 16, 3, 3, (1, 1), (2, 2), (2, 2), "vec16"),                 # dilation
    (2, 30, 30, 3, 32, 7, 7, (2, 2), (3, 3), (1, 1), "narrow"),                 # C = 3 stem
    (1, 9, 11, 5, 7, 2, 3, (1, 2), (0, 1), (2, 1), "narrow"),                   # C = 5, ragged all
    (1, 6, 6, 200, 300, 3, 3, (1, 1), (1, 1), (1, 1), "vec16"),                 # C, K past one tile
]


@pytest.mark.parametrize("shape", SHAPES)
def test_conv_parity(shape):
    *dims, frag = shape
    N, H, W, C, K, R, S, stride, pad, dil = dims
    kernel = run_conv(N, H, W, C, K, R, S, stride, pad, dil, seed=C + K)
    assert frag in kernel, kernel


@pytest.mark.parametrize("act", [0, 1, 2, 3])
def test_conv_epilogue_residual_bias_activation(act):
    run_conv(2, 12, 12, 32, 48, 3, 3, pad=(1, 1), seed=act, alpha=0.5, beta=1.0, bias=True, act=act)
    run_conv(2, 12, 12, 32, 48, 3, 3, pad=(1, 1), seed=act + 10, beta=-0.5, bias=True, act=act,
             out_f32=True)


def test_conv_misaligned_pointers_take_element_loads():
    kernel = run_conv(2, 10, 10, 16, 24, 3, 3, pad=(1, 1), seed=5, offset=3)
    assert kernel.endswith("vec16")     # the plan's choice; the run reads element-wise


def test_conv_resnet_layer_sampled():
    """A ResNet-50 stage-2 3x3 layer at batch 32 (M = 100352) on sampled pixels,
    the first and last ones included; also with the fused epilogue."""
    rng = np.random.default_rng(7)
    rows = np.unique(np.r_[0, 32 * 56 * 56 - 1, rng.integers(0, 32 * 56 * 56, 300)])
    kernel = run_conv(32, 56, 56, 64, 64, 3, 3, pad=(1, 1), seed=6, rows=rows)
    assert "256x64x64_vec16" in kernel, kernel
    run_conv(32, 56, 56, 64, 64, 3, 3, pad=(1, 1), seed=16, rows=rows, beta=1.0, bias=True, act=1)


def test_conv_stem_layer_sampled():
    """The ResNet stem (C = 3, 7x7, stride 2) at batch 32: the 128 x 64 tile
    with element-wise loads."""
    rows = np.unique(np.random.default_rng(9).integers(0, 32 * 112 * 112, 200))
    kernel = run_conv(32, 224, 224, 3, 64, 7, 7, stride=(2, 2), pad=(3, 3), seed=9, rows=rows)
    assert "128x64x64_narrow" in kernel, kernel


def test_conv_torch_wrapper_and_determinism():
    g = torch.Generator("cpu").manual_seed(8)
    x = torch.randn(4, 20, 20, 32, generator=g).half().cuda()
    w = (torch.randn(48, 3, 3, 32, generator=g) / 17).half().cuda()
    a = mpg.conv2d(x, w, padding=(1, 1))
    b = mpg.conv2d(x, w, padding=(1, 1))
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    want = torch.nn.functional.conv2d(x.permute(0, 3, 1, 2).float(), w.permute(0, 3, 1, 2).float(),
                                      padding=1).permute(0, 2, 3, 1)
    assert torch.allclose(a.float(), want, rtol=1e-2, atol=1e-2)
