"""Pins of the 2-D convolution oracle (oracle/ref_conv.c), no GPU.

  - torch.nn.functional.conv2d in float64 on the CPU (a library routine) over
    strides, paddings, dilations and rectangular filters (NCHW there, NHWC and
    KRSC here: the permutation is the only translation);
  - a 1 x 1 filter with stride 1 and no padding is the matrix product of the
    N H W x C activations with the C x K filters: the pinned GEMM oracle;
  - closed forms: the identity filter (a 3 x 3 filter whose centre is the
    identity over channels, padding 1) returns x; all-ones x and w give, at
    every output, C times the number of filter taps inside the image;
  - the output-size formula on known cases, and windows that do not fit;
  - alpha, beta, bias and ReLU composed as the GEMM epilogue is;
  - a pure-Python brute force on tiny shapes;
  - the error scale: with x, w >= 0 it equals the value.
"""
import numpy as np
import pytest
import torch

import oracle

RNG = np.random.default_rng(4242)


def f16(x):
    h = np.asarray(x, dtype=np.float64).astype(np.float16)
    return h.view(np.uint16), h.astype(np.float64)


def torch_conv(xv, wv, stride, pad, dil):
    """x (N, H, W, C), w (K, R, S, C) float64 -> (N, P, Q, K)."""
    x = torch.from_numpy(np.ascontiguousarray(xv.transpose(0, 3, 1, 2)))
    w = torch.from_numpy(np.ascontiguousarray(wv.transpose(0, 3, 1, 2)))
    y = torch.nn.functional.conv2d(x, w, stride=stride, padding=pad, dilation=dil)
    return y.numpy().transpose(0, 2, 3, 1)


@pytest.mark.parametrize("N,H,W,C,K,R,S,stride,pad,dil", [
    (1, 5, 5, 3, 2, 3, 3, (1, 1), (0, 0), (1, 1)),
    (2, 9, 7, 8, 5, 3, 3, (2, 1), (1, 1), (1, 1)),
    (1, 12, 10, 16, 4, 3, 2, (1, 2), (2, 0), (2, 3)),
    (3, 6, 6, 5, 7, 1, 1, (1, 1), (0, 0), (1, 1)),
    (1, 14, 14, 4, 3, 5, 5, (3, 3), (2, 2), (1, 1)),
])
def test_conv_matches_torch(N, H, W, C, K, R, S, stride, pad, dil):
    xb, xv = f16(RNG.standard_normal((N, H, W, C)))
    wb, wv = f16(RNG.standard_normal((K, R, S, C)))
    ref, _ = oracle.conv2d(N, H, W, C, K, R, S, xb, wb, stride=stride, pad=pad, dil=dil)
    want = torch_conv(xv, wv, stride, pad, dil)
    assert ref.shape == (want.shape[0] * want.shape[1] * want.shape[2], K)
    assert np.allclose(ref, want.reshape(-1, K), rtol=1e-12, atol=1e-12)


def test_one_by_one_filter_is_the_gemm():
    N, H, W, C, K = 2, 4, 6, 24, 10
    xb, _ = f16(RNG.standard_normal((N, H, W, C)))
    wb, _ = f16(RNG.standard_normal((K, 1, 1, C)))
    ref, _ = oracle.conv2d(N, H, W, C, K, 1, 1, xb, wb)
    # A = x as (N H W) x C row-major, B = w as C x K column-major (ldb = C)
    g, _ = oracle.gemm(N * H * W, K, C, xb, wb, layout_b=oracle.COL_MAJOR, out_type=oracle.OUT_F32)
    assert np.array_equal(ref, g[0])


def test_identity_filter_returns_the_input():
    N, H, W, C = 1, 7, 5, 6
    xb, xv = f16(RNG.standard_normal((N, H, W, C)))
    w = np.zeros((C, 3, 3, C))
    for c in range(C):
        w[c, 1, 1, c] = 1.0
    wb, _ = f16(w)
    ref, _ = oracle.conv2d(N, H, W, C, C, 3, 3, xb, wb, pad=(1, 1))
    assert np.array_equal(ref, xv.reshape(-1, C))


def test_all_ones_count_the_taps_inside_the_image():
    N, H, W, C, K, R, S = 1, 6, 5, 3, 2, 3, 3
    xb, _ = f16(np.ones((N, H, W, C)))
    wb, _ = f16(np.ones((K, R, S, C)))
    ref, _ = oracle.conv2d(N, H, W, C, K, R, S, xb, wb, pad=(1, 1))
    P, Q = H, W
    for p in range(P):
        for q in range(Q):
            rows_in = sum(0 <= p - 1 + r < H for r in range(R))
            cols_in = sum(0 <= q - 1 + s < W for s in range(S))
            assert np.all(ref[p * Q + q] == C * rows_in * cols_in)


def test_output_size():
    assert oracle.conv_out_dim(56, 3, 1, 1, 1) == 56
    assert oracle.conv_out_dim(56, 3, 2, 1, 1) == 28
    assert oracle.conv_out_dim(224, 7, 2, 3, 1) == 112
    assert oracle.conv_out_dim(10, 3, 1, 0, 4) == 2          # span 9
    assert oracle.conv_out_dim(4, 5, 1, 0, 1) == -1          # does not fit
    with pytest.raises(ValueError):
        oracle.conv2d(1, 4, 4, 1, 1, 5, 5, np.zeros(16, np.uint16), np.zeros(25, np.uint16))


def test_epilogue_composition():
    N, H, W, C, K, R, S = 1, 5, 5, 4, 3, 3, 3
    xb, xv = f16(RNG.standard_normal((N, H, W, C)))
    wb, wv = f16(RNG.standard_normal((K, R, S, C)))
    P = Q = 3
    yb, yv = f16(RNG.standard_normal((N * P * Q, K)))
    bias = RNG.standard_normal(K).astype(np.float32)
    ref, scale = oracle.conv2d(N, H, W, C, K, R, S, xb, wb, yb, alpha=0.5, beta=-2.0, bias=bias,
                               activation=oracle.ACT_RELU)
    conv = torch_conv(xv, wv, (1, 1), (0, 0), (1, 1)).reshape(-1, K)
    want = np.maximum(0.5 * conv - 2.0 * yv + bias.astype(np.float64), 0.0)
    assert np.allclose(ref, want, rtol=1e-12, atol=1e-12)
    absconv = torch_conv(np.abs(xv), np.abs(wv), (1, 1), (0, 0), (1, 1)).reshape(-1, K)
    assert np.allclose(scale, 0.5 * absconv + 2.0 * np.abs(yv) + np.abs(bias.astype(np.float64)),
                       rtol=1e-12)


def _brute(xv, wv, stride, pad, dil):
    N, H, W, C = xv.shape
    K, R, S, _ = wv.shape
    P = (H + 2 * pad[0] - dil[0] * (R - 1) - 1) // stride[0] + 1
    Q = (W + 2 * pad[1] - dil[1] * (S - 1) - 1) // stride[1] + 1
    out = np.zeros((N, P, Q, K))
    for n in range(N):
        for p in range(P):
            for q in range(Q):
                for k in range(K):
                    acc = []
                    for r in range(R):
                        for s in range(S):
                            ih = p * stride[0] - pad[0] + r * dil[0]
                            iw = q * stride[1] - pad[1] + s * dil[1]
                            if 0 <= ih < H and 0 <= iw < W:
                                acc += [xv[n, ih, iw, c] * wv[k, r, s, c] for c in range(C)]
                    out[n, p, q, k] = sum(acc)
    return out.reshape(-1, K)


@pytest.mark.parametrize("shape", [(1, 3, 3, 1, 1, 2, 2, (1, 1), (0, 0), (1, 1)),
                                   (1, 5, 4, 2, 2, 3, 2, (2, 1), (1, 1), (1, 2))])
def test_conv_pure_python_brute_force(shape):
    N, H, W, C, K, R, S, stride, pad, dil = shape
    xb, xv = f16(RNG.integers(-4, 5, size=(N, H, W, C)))
    wb, wv = f16(RNG.integers(-4, 5, size=(K, R, S, C)))
    ref, _ = oracle.conv2d(N, H, W, C, K, R, S, xb, wb, stride=stride, pad=pad, dil=dil)
    assert np.array_equal(ref, _brute(xv, wv, stride, pad, dil))


def test_scale_equals_value_for_nonnegative_inputs():
    xb, _ = f16(np.abs(RNG.standard_normal((1, 6, 6, 4))))
    wb, _ = f16(np.abs(RNG.standard_normal((3, 3, 3, 4))))
    ref, scale = oracle.conv2d(1, 6, 6, 4, 3, 3, 3, xb, wb, pad=(1, 1))
    assert np.allclose(ref, scale, rtol=1e-15)
