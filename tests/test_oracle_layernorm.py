"""Pins of the residual + LayerNorm linear-layer oracle (oracle/ref_layernorm.c),
no GPU.

The oracle's GEMM part is oracle_gemm (pinned in test_oracle.py); these pins
tie the normalisation and its composition to other sources:
  - torch.nn.functional.layer_norm in float64 (a library routine) applied to
    the GEMM oracle's Z;
  - closed forms: a row whose entries are all equal normalises to beta_ln; a
    row with half its entries a and half b normalises to
    +-(a - b)/2 / sqrt((a - b)^2/4 + eps) * gamma + beta_ln;
  - invariances: a constant added to every entry of a row (through the
    residual) changes nothing; with eps = 0 a positive alpha changes nothing;
  - a pure-Python brute force of the whole layer on tiny shapes;
  - the bound term T's definition on a known row.
"""
import math

import numpy as np
import pytest
import torch

import oracle

RNG = np.random.default_rng(777)


def f16(x):
    h = np.asarray(x, dtype=np.float64).astype(np.float16)
    return h.view(np.uint16), h.astype(np.float64)


def case(M, N, K, seed=0, beta=0.0):
    rng = np.random.default_rng(seed)
    ab, av = f16(rng.standard_normal((M, K)))
    bb, bv = f16(rng.standard_normal((K, N)) * 0.05)
    cb, cv = f16(rng.standard_normal((M, N)))
    bias = rng.standard_normal(N).astype(np.float32)
    gamma = (1 + 0.3 * rng.standard_normal(N)).astype(np.float32)
    beta_ln = (0.2 * rng.standard_normal(N)).astype(np.float32)
    return ab, av, bb, bv, cb, cv, bias, gamma, beta_ln


@pytest.mark.parametrize("M,N,K,beta", [(5, 64, 32, 0.0), (17, 333, 70, 1.0), (3, 1, 9, 0.5)])
def test_layernorm_matches_torch_on_the_gemm_oracle(M, N, K, beta):
    ab, _, bb, _, cb, _, bias, gamma, beta_ln = case(M, N, K, seed=M, beta=beta)
    eps = 1e-5
    z, _ = oracle.gemm(M, N, K, ab, bb, cb, alpha=0.75, beta=beta, bias=bias)
    want = torch.nn.functional.layer_norm(torch.from_numpy(z[0]), (N,),
                                          torch.from_numpy(gamma.astype(np.float64)),
                                          torch.from_numpy(beta_ln.astype(np.float64)),
                                          eps=float(np.float32(eps))).numpy()
    y, _, st = oracle.gemm_layernorm(M, N, K, ab, bb, cb, gamma=gamma, beta_ln=beta_ln, eps=eps,
                                     alpha=0.75, beta=beta, bias=bias)
    assert np.allclose(y[0], want, rtol=1e-12, atol=1e-12)
    assert np.allclose(st[0, :, 0], z[0].mean(axis=1), rtol=1e-13, atol=1e-15)


def test_constant_row_gives_beta_ln():
    """B with equal columns makes every entry of a row of A B equal: zero
    deviation from the mean, so Y = beta_ln whatever gamma is."""
    M, N, K = 4, 40, 16
    ab, _ = f16(RNG.integers(-4, 5, size=(M, K)))
    col, _ = f16(RNG.integers(-4, 5, size=(K, 1)))
    bb = np.repeat(col.reshape(K, 1), N, axis=1).ravel()
    gamma = RNG.standard_normal(N).astype(np.float32)
    beta_ln = RNG.standard_normal(N).astype(np.float32)
    y, _, st = oracle.gemm_layernorm(M, N, K, ab, bb, gamma=gamma, beta_ln=beta_ln, eps=1e-3)
    assert np.array_equal(y[0], np.broadcast_to(beta_ln.astype(np.float64), (M, N)))
    assert np.allclose(st[0, :, 1], math.sqrt(float(np.float32(1e-3))), rtol=1e-15)


def test_two_point_row_closed_form():
    """K = 1, A = 1: row i of Z is B's row, half a and half b."""
    N, a, b, eps = 10, 3.0, -1.0, 0.25
    bb, _ = f16(np.array([a] * 5 + [b] * 5))
    ab, _ = f16(np.array([1.0]))
    gamma = np.full(N, 2.0, dtype=np.float32)
    beta_ln = np.full(N, 0.5, dtype=np.float32)
    y, _, _ = oracle.gemm_layernorm(1, N, 1, ab, bb, gamma=gamma, beta_ln=beta_ln, eps=eps)
    d = (a - b) / 2 / math.sqrt((a - b) ** 2 / 4 + eps)
    want = np.array([d] * 5 + [-d] * 5) * 2.0 + 0.5
    assert np.allclose(y[0, 0], want, rtol=1e-15, atol=1e-15)


def test_row_constant_residual_and_positive_alpha_change_nothing():
    M, N, K = 6, 50, 24
    ab, _, bb, _, _, _, bias, gamma, beta_ln = case(M, N, K, seed=3)
    y0, _, _ = oracle.gemm_layernorm(M, N, K, ab, bb, gamma=gamma, beta_ln=beta_ln, eps=1e-5,
                                     bias=bias)
    shifts = RNG.integers(-20, 21, size=M).astype(np.float64)
    cb, _ = f16(np.repeat(shifts[:, None], N, axis=1))            # exact small integers
    y1, _, _ = oracle.gemm_layernorm(M, N, K, ab, bb, cb, gamma=gamma, beta_ln=beta_ln,
                                     eps=1e-5, beta=1.0, bias=bias)
    assert np.allclose(y0, y1, rtol=1e-11, atol=1e-11)
    ya, _, _ = oracle.gemm_layernorm(M, N, K, ab, bb, gamma=gamma, beta_ln=beta_ln, eps=0.0,
                                     alpha=1.0)
    yb, _, _ = oracle.gemm_layernorm(M, N, K, ab, bb, gamma=gamma, beta_ln=beta_ln, eps=0.0,
                                     alpha=4.0)
    assert np.allclose(ya, yb, rtol=1e-12, atol=1e-12)


def _brute(av, bv, cv, bias, gamma, beta_ln, eps, alpha, beta):
    M, K = av.shape
    N = bv.shape[1]
    out = np.zeros((M, N))
    for i in range(M):
        z = [alpha * math.fsum(av[i, k] * bv[k, n] for k in range(K)) + beta * cv[i, n]
             + float(bias[n]) for n in range(N)]
        mu = math.fsum(z) / N
        var = math.fsum((x - mu) ** 2 for x in z) / N
        for n in range(N):
            out[i, n] = (z[n] - mu) / math.sqrt(var + eps) * float(gamma[n]) + float(beta_ln[n])
    return out


@pytest.mark.parametrize("M,N,K", [(1, 2, 1), (3, 7, 5), (4, 16, 9)])
def test_layer_pure_python_brute_force(M, N, K):
    ab, av, bb, bv, cb, cv, bias, gamma, beta_ln = case(M, N, K, seed=N)
    eps = float(np.float32(1e-5))
    y, _, _ = oracle.gemm_layernorm(M, N, K, ab, bb, cb, gamma=gamma, beta_ln=beta_ln, eps=1e-5,
                                    alpha=1.5, beta=-0.5, bias=bias)
    want = _brute(av.reshape(M, K), bv.reshape(K, N), cv.reshape(M, N), bias, gamma, beta_ln,
                  eps, 1.5, -0.5)
    assert np.allclose(y[0], want, rtol=1e-12, atol=1e-12)


def test_bound_term_definition():
    """T = |gamma| (2 D + |Z - mu| D / s) / s with D = 2e-3 max_n S: for
    A = 1 (K = 1, S = |B|) the row is B's row."""
    vals = np.array([1.0, -2.0, 4.0, 0.5])
    bb, _ = f16(vals)
    ab, _ = f16(np.array([1.0]))
    gamma = np.array([1.0, -2.0, 0.5, 3.0], dtype=np.float32)
    beta_ln = np.zeros(4, dtype=np.float32)
    _, t, st = oracle.gemm_layernorm(1, 4, 1, ab, bb, gamma=gamma, beta_ln=beta_ln, eps=0.0)
    mu = vals.mean()
    s = math.sqrt(((vals - mu) ** 2).mean())
    D = 2e-3 * 4.0
    want = np.abs(gamma.astype(np.float64)) * (2 * D + np.abs(vals - mu) * D / s) / s
    assert np.allclose(t[0, 0], want, rtol=1e-14)
    assert np.allclose(st[0, 0], [mu, s, np.abs(vals).mean()], rtol=1e-15)
