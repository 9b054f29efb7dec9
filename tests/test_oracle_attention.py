"""Pins of the softmax and attention oracle (oracle/ref_attention.c), no GPU.

Each pin ties the oracle to something other than itself:
  - scipy.special.softmax (a library routine) for the row softmax, masked
    elements included;
  - the online recurrence of the operator-practice page (§2.2) against the
    two-pass definition (§2.1): two independent formulations of one value;
  - torch's scaled_dot_product_attention in float64 on the CPU (a library
    routine) for attention, with and without the causal mask;
  - closed forms: scores that are all equal give the mean of the visible V
    rows; one dominant score gives the textbook weighted average
    (e^c v_j + sum_{k != j} v_k) / (e^c + n - 1);
  - invariances: a component common to every key shifts each row's scores
    by a constant and leaves O unchanged; permuting keys and values together
    leaves O unchanged; strides describing the same tensors give the same O;
  - a pure-Python brute force (math.exp, math.fsum) on tiny shapes;
  - the error scales: with V >= 0 the scale sum_j P_ij |V_jc| equals O, with
    V <= 0 it equals -O; with Q, K >= 0 and scale > 0 the score bound equals
    the largest score.
Fully masked rows (every key hidden by the causal mask, or no keys) give
zeros: the reading of the page's masked-row case (§2.5) taken here.
"""
import math

import numpy as np
import pytest
import torch

import oracle

RNG = np.random.default_rng(20260)


def f16(x):
    """float64 values rounded to binary16, returned as (bits, exact float64 values)."""
    h = np.asarray(x, dtype=np.float64).astype(np.float16)
    return h.view(np.uint16), h.astype(np.float64)


def rand16(*shape, scale=1.0):
    return f16(RNG.standard_normal(shape) * scale)


# ------------------------------------------------------------ row softmax

@pytest.mark.parametrize("n", [1, 2, 7, 64, 333, 4097])
def test_softmax_row_matches_scipy(n):
    from scipy.special import softmax
    for offset in (0.0, 700.0, -700.0):
        x = RNG.standard_normal(n) * 5 + offset
        got = oracle.softmax_row(x)
        want = softmax(x)
        assert np.allclose(got, want, rtol=1e-13, atol=0.0)
        assert abs(got.sum() - 1.0) < 1e-13 * n


def test_softmax_row_masked_elements_and_rows():
    from scipy.special import softmax
    x = RNG.standard_normal(50) * 3
    mask = RNG.random(50) < 0.4
    x[mask] = -np.inf
    got = oracle.softmax_row(x)
    assert np.all(got[mask] == 0.0)
    assert np.allclose(got[~mask], softmax(x[~mask]), rtol=1e-13, atol=0.0)
    # every element masked: the constant (zero) output, not NaN
    assert np.array_equal(oracle.softmax_row(np.full(9, -np.inf)), np.zeros(9))
    assert oracle.softmax_row(np.zeros(0)).size == 0
    # one visible element takes all the weight
    y = np.full(5, -np.inf)
    y[3] = -123.0
    assert np.array_equal(oracle.softmax_row(y), np.eye(5)[3])


@pytest.mark.parametrize("block", [1, 3, 64, 1000])
def test_online_recurrence_equals_two_pass(block):
    for n, offset in [(1, 0.0), (257, 0.0), (1000, 300.0)]:
        x = RNG.standard_normal(n) * 8 + offset
        x[: n // 3] -= 50.0          # the running maximum moves late in the row
        if n > 10:
            x[:5] = -np.inf          # and the first block may be fully masked
        a = oracle.softmax_row(x)
        b = oracle.softmax_row_online(x, block)
        assert np.allclose(a, b, rtol=1e-12, atol=0.0)


def test_softmax_matrix_on_binary16_and_fp32_storage():
    from scipy.special import softmax
    rows, cols, ld = 6, 37, 40
    bits, vals = rand16(rows * ld, scale=4.0)
    got = oracle.softmax(rows, cols, bits, ld=ld)
    want = softmax(vals.reshape(rows, ld)[:, :cols], axis=1)
    assert np.allclose(got, want, rtol=1e-13, atol=0.0)
    x32 = (RNG.standard_normal(rows * ld) * 4).astype(np.float32)
    got = oracle.softmax(rows, cols, x32, ld=ld)
    want = softmax(x32.astype(np.float64).reshape(rows, ld)[:, :cols], axis=1)
    assert np.allclose(got, want, rtol=1e-13, atol=0.0)


# ------------------------------------------------------------ attention

def sdpa(qv, kv, vv, scale, causal):
    """torch's float64 CPU attention on (B, H, S, D) arrays."""
    q, k, v = (torch.from_numpy(np.ascontiguousarray(a)) for a in (qv, kv, vv))
    return torch.nn.functional.scaled_dot_product_attention(
        q, k, v, is_causal=causal, scale=scale).numpy()


@pytest.mark.parametrize("B,H,Sq,Sk,D,Dv", [(1, 1, 5, 9, 8, 8), (2, 3, 33, 47, 64, 64),
                                           (1, 2, 128, 128, 128, 128), (2, 1, 17, 65, 16, 24)])
def test_attention_matches_torch_sdpa(B, H, Sq, Sk, D, Dv):
    qb, qv = rand16(B, H, Sq, D)
    kb, kv = rand16(B, H, Sk, D)
    vb, vv = rand16(B, H, Sk, Dv)
    scale = float(np.float32(1.0 / math.sqrt(D)))
    out, _, _ = oracle.attention(B, H, Sq, Sk, D, qb, kb, vb, Dv=Dv, scale=scale)
    assert np.allclose(out, sdpa(qv, kv, vv, scale, False), rtol=1e-11, atol=1e-13)
    if Sq == Sk:
        out, _, _ = oracle.attention(B, H, Sq, Sk, D, qb, kb, vb, Dv=Dv, scale=scale, causal=True)
        assert np.allclose(out, sdpa(qv, kv, vv, scale, True), rtol=1e-11, atol=1e-13)


def test_causal_mask_aligns_the_last_query_with_the_last_key():
    """Sq < Sk: query i sees keys 0 .. i + Sk - Sq, i.e. it is row
    i + Sk - Sq of the square causal problem."""
    B, H, Sq, Sk, D = 1, 2, 12, 40, 16
    qb, qv = rand16(B, H, Sq, D)
    kb, kv = rand16(B, H, Sk, D)
    vb, vv = rand16(B, H, Sk, D)
    scale = 0.25
    out, _, _ = oracle.attention(B, H, Sq, Sk, D, qb, kb, vb, scale=scale, causal=True)
    qfull = np.zeros((B, H, Sk, D))
    qfull[:, :, Sk - Sq:] = qv
    want = sdpa(qfull, kv, vv, scale, True)[:, :, Sk - Sq:]
    assert np.allclose(out, want, rtol=1e-11, atol=1e-13)


def test_fully_masked_rows_and_no_keys_give_zeros():
    B, H, Sq, Sk, D = 1, 1, 10, 4, 8
    qb, _ = rand16(B, H, Sq, D)
    kb, kv = rand16(B, H, Sk, D)
    vb, vv = rand16(B, H, Sk, D)
    out, err, _ = oracle.attention(B, H, Sq, Sk, D, qb, kb, vb, causal=True)
    assert np.array_equal(out[0, 0, :Sq - Sk], np.zeros((Sq - Sk, D)))    # no visible key
    assert np.array_equal(err[0, 0, :Sq - Sk], np.zeros((Sq - Sk, D)))
    assert np.all(np.isfinite(out))
    # the first row with a visible key sees exactly key 0
    assert np.array_equal(out[0, 0, Sq - Sk], vv[0, 0, 0])
    out, _, _ = oracle.attention(1, 1, 3, 0, D, qb, kb[:0], vb[:0])
    assert np.array_equal(out, np.zeros((1, 1, 3, D)))


def test_uniform_scores_give_the_mean_of_the_visible_values():
    B, H, Sq, Sk, D = 1, 2, 6, 11, 8
    qb = np.zeros(B * H * Sq * D, dtype=np.uint16)           # Q = 0: all scores 0
    kb, _ = rand16(B, H, Sk, D)
    vb, vv = rand16(B, H, Sk, D)
    out, _, _ = oracle.attention(B, H, Sq, Sk, D, qb, kb, vb)
    assert np.allclose(out, np.broadcast_to(vv.mean(axis=2, keepdims=True), out.shape),
                       rtol=1e-14, atol=1e-15)
    out, _, _ = oracle.attention(B, H, Sq, Sk, D, qb, kb, vb, causal=True)
    for i in range(Sq):
        nvis = i + Sk - Sq + 1
        assert np.allclose(out[:, :, i], vv[:, :, :nvis].mean(axis=2), rtol=1e-14, atol=1e-15)


def test_one_dominant_score_closed_form():
    """Q_i = c e_0 / scale and K rows orthogonal to e_0 except key j(i) = e_0:
    s_i = c at j(i), 0 elsewhere."""
    Sq, Sk, D, c = 4, 9, 8, 6.0
    scale = 0.5
    q = np.zeros((1, 1, Sq, D))
    q[0, 0, :, 0] = c / scale
    k = np.zeros((1, 1, Sk, D))
    k[0, 0, :, 1] = 1.0
    js = [2, 5, 0, 8]
    vb, vv = rand16(1, 1, Sk, D)
    outs = []
    for i, j in enumerate(js):
        kk = k.copy()
        kk[0, 0, j] = 0.0
        kk[0, 0, j, 0] = 1.0
        qb_, _ = f16(q)
        kb_, _ = f16(kk)
        o, _, _ = oracle.attention(1, 1, Sq, Sk, D, qb_, kb_, vb, scale=scale, rows=[i])
        outs.append(o[0, 0, 0])
        others = [r for r in range(Sk) if r != j]
        want = (math.exp(c) * vv[0, 0, j] + vv[0, 0, others].sum(axis=0)) / (math.exp(c) + Sk - 1)
        assert np.allclose(o[0, 0, 0], want, rtol=1e-14, atol=1e-15)


def test_common_key_component_and_key_permutation_leave_o_unchanged():
    B, H, Sq, Sk, D = 1, 1, 7, 13, 16
    qi = RNG.integers(-3, 4, size=(B, H, Sq, D)).astype(np.float64)
    ki = RNG.integers(-3, 4, size=(B, H, Sk, D)).astype(np.float64)
    u = RNG.integers(-3, 4, size=D).astype(np.float64)
    vb, vv = rand16(B, H, Sk, D)
    qb, _ = f16(qi)
    kb, _ = f16(ki)
    kub, _ = f16(ki + u)          # exact in binary16: small integers
    o1, _, _ = oracle.attention(B, H, Sq, Sk, D, qb, kb, vb, scale=0.125)
    o2, _, _ = oracle.attention(B, H, Sq, Sk, D, qb, kub, vb, scale=0.125)
    assert np.allclose(o1, o2, rtol=1e-12, atol=1e-14)
    perm = RNG.permutation(Sk)
    kpb, _ = f16(ki[:, :, perm])
    vpb = vb.reshape(B, H, Sk, D)[:, :, perm].copy()
    o3, _, _ = oracle.attention(B, H, Sq, Sk, D, qb, kpb, vpb, scale=0.125)
    assert np.allclose(o1, o3, rtol=1e-12, atol=1e-14)


def test_strides_describe_the_tensors():
    """The same Q, K, V stored [batch][seq][head][d] (heads interleaved in a
    row) and [batch][head][seq][d] give the same O."""
    B, H, Sq, Sk, D = 2, 3, 9, 14, 8
    qb, _ = rand16(B, H, Sq, D)
    kb, _ = rand16(B, H, Sk, D)
    vb, _ = rand16(B, H, Sk, D)
    dense, _, _ = oracle.attention(B, H, Sq, Sk, D, qb, kb, vb, causal=True)
    bshd = lambda x, S: np.ascontiguousarray(x.reshape(B, H, S, D).transpose(0, 2, 1, 3)).ravel()
    out, _, _ = oracle.attention(B, H, Sq, Sk, D, bshd(qb, Sq), bshd(kb, Sk), bshd(vb, Sk),
                                 causal=True, q_strides=(Sq * H * D, D, H * D),
                                 k_strides=(Sk * H * D, D, H * D), v_strides=(Sk * H * D, D, H * D))
    assert np.array_equal(out, dense)


def _brute(qv, kv, vv, scale, causal):
    Sq, D = qv.shape
    Sk, Dv = vv.shape
    out = np.zeros((Sq, Dv))
    for i in range(Sq):
        vis = range(Sk) if not causal else range(max(0, min(Sk, i + Sk - Sq + 1)))
        s = {j: scale * math.fsum(qv[i, d] * kv[j, d] for d in range(D)) for j in vis}
        if not s:
            continue
        m = max(s.values())
        w = {j: math.exp(s[j] - m) for j in s}
        tot = math.fsum(w.values())
        for c in range(Dv):
            out[i, c] = math.fsum(w[j] / tot * vv[j, c] for j in s)
    return out


@pytest.mark.parametrize("Sq,Sk,D,Dv,causal", [(1, 1, 1, 1, False), (3, 5, 4, 2, False),
                                               (5, 3, 4, 3, True), (4, 4, 8, 8, True)])
def test_attention_pure_python_brute_force(Sq, Sk, D, Dv, causal):
    qb, qv = rand16(Sq, D, scale=2.0)
    kb, kv = rand16(Sk, D, scale=2.0)
    vb, vv = rand16(Sk, Dv)
    out, _, _ = oracle.attention(1, 1, Sq, Sk, D, qb, kb, vb, Dv=Dv, scale=0.75, causal=causal)
    assert np.allclose(out[0, 0], _brute(qv, kv, vv, float(np.float32(0.75)), causal),
                       rtol=1e-13, atol=1e-15)


def test_error_scales():
    B, H, Sq, Sk, D = 1, 2, 6, 10, 8
    qb, qv = f16(np.abs(RNG.standard_normal((B, H, Sq, D))))
    kb, kv = f16(np.abs(RNG.standard_normal((B, H, Sk, D))))
    vpb, _ = f16(np.abs(RNG.standard_normal((B, H, Sk, D))))
    vnb, _ = f16(-np.abs(RNG.standard_normal((B, H, Sk, D))))
    o, e, smax = oracle.attention(B, H, Sq, Sk, D, qb, kb, vpb, scale=0.5)
    assert np.allclose(e, o, rtol=1e-15, atol=0.0)
    o, e, _ = oracle.attention(B, H, Sq, Sk, D, qb, kb, vnb, scale=0.5)
    assert np.allclose(e, -o, rtol=1e-15, atol=0.0)
    scores = 0.5 * np.einsum("bhid,bhjd->bhij", qv, kv)
    assert np.allclose(smax, scores.max(axis=3), rtol=1e-14, atol=0.0)
