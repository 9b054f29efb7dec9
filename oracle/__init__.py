"""CPU oracle for C = alpha*A*B + beta*C with binary16 or bfloat16 A, B, and
for row softmax and attention (test infrastructure).

TEST INFRASTRUCTURE ONLY.  Only tests/, the smoke check in __graft_entry__ and
the CPU-baseline leg of bench.py may import this package.  It shares no code
with the GPU path (mixed_precision_gemm_amd) and never imports it.

The arithmetic is in ref_gemm.c (plain fp64 triple loop, own binary16 and
bfloat16 decoders and encoders), ref_attention.c (softmax by its
definition and by the online recurrence, attention in fp64) and
ref_layernorm.c (the linear layer fused with its residual and LayerNorm)
and ref_conv.c (2-D convolution by its definition); this module only
marshals numpy arrays through ctypes.  See the headers of the C files for what
each function follows on the pages.
"""
import ctypes
import os
import numpy as np

from . import build as _build

ROW_MAJOR, COL_MAJOR = 0, 1
OUT_F16, OUT_F32, OUT_BF16 = 0, 1, 2
IN_F16, IN_BF16 = 0, 1
ACT_NONE, ACT_RELU, ACT_GELU, ACT_SILU = 0, 1, 2, 3

_lib = None


def load_library(path):
    """Opens an oracle shared library at `path` and declares its functions."""
    lib = ctypes.CDLL(path)
    i64, dbl, vp = ctypes.c_int64, ctypes.c_double, ctypes.c_void_p
    lib.oracle_dec16.argtypes = [ctypes.c_uint16]
    lib.oracle_dec16.restype = dbl
    lib.oracle_enc16.argtypes = [dbl]
    lib.oracle_enc16.restype = ctypes.c_uint16
    lib.oracle_decbf16.argtypes = [ctypes.c_uint16]
    lib.oracle_decbf16.restype = dbl
    lib.oracle_encbf16.argtypes = [dbl]
    lib.oracle_encbf16.restype = ctypes.c_uint16
    lib.oracle_activate.argtypes = [ctypes.c_int, dbl]
    lib.oracle_activate.restype = dbl
    lib.oracle_gemm.argtypes = [i64, i64, i64, i64,
                                ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                i64, i64, i64, i64, i64, i64,
                                vp, vp, vp, dbl, dbl, vp, ctypes.c_int, vp, i64, vp, vp,
                                ctypes.c_int]
    lib.oracle_gemm.restype = ctypes.c_int
    if hasattr(lib, "oracle_attention"):
        dp = ctypes.POINTER(ctypes.c_double)
        lib.oracle_softmax_row.argtypes = [vp, i64, vp]
        lib.oracle_softmax_row.restype = None
        lib.oracle_softmax_row_online.argtypes = [vp, i64, i64, vp]
        lib.oracle_softmax_row_online.restype = None
        lib.oracle_softmax.argtypes = [i64, i64, vp, ctypes.c_int, i64, vp]
        lib.oracle_softmax.restype = ctypes.c_int
        lib.oracle_attention.argtypes = [i64, i64, i64, i64, i64, i64,
                                         vp, i64, i64, i64, vp, i64, i64, i64,
                                         vp, i64, i64, i64, dbl, ctypes.c_int, vp, i64,
                                         vp, vp, vp, ctypes.c_int]
        lib.oracle_attention.restype = ctypes.c_int
        del dp
    if hasattr(lib, "oracle_gemm_layernorm"):
        lib.oracle_layernorm_row.argtypes = [vp, i64, vp, vp, dbl, vp, vp]
        lib.oracle_layernorm_row.restype = None
        lib.oracle_gemm_layernorm.argtypes = [i64, i64, i64, i64,
                                              ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                              i64, i64, i64, i64, i64, i64,
                                              vp, vp, vp, dbl, dbl, vp, vp, vp, dbl, vp, i64,
                                              vp, vp, vp, ctypes.c_int]
        lib.oracle_gemm_layernorm.restype = ctypes.c_int
    if hasattr(lib, "oracle_conv2d"):
        lib.oracle_conv_out_dim.argtypes = [i64, i64, i64, i64, i64]
        lib.oracle_conv_out_dim.restype = i64
        lib.oracle_conv2d.argtypes = [i64] * 13 + [vp, vp, vp, ctypes.c_int, dbl, dbl, vp,
                                                  ctypes.c_int, vp, i64, vp, vp, ctypes.c_int]
        lib.oracle_conv2d.restype = ctypes.c_int
    return lib


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        _lib = load_library(_build.LIB)
    return _lib


def dec16(bits, lib=None) -> np.ndarray:
    """binary16 bit patterns (any int array) -> float64, element by element."""
    lib = lib or _load()
    flat = np.asarray(bits, dtype=np.uint16).ravel()
    out = np.array([lib.oracle_dec16(int(h)) for h in flat], dtype=np.float64)
    return out.reshape(np.shape(bits))


def enc16(values, lib=None) -> np.ndarray:
    """float64 values -> binary16 bit patterns (round to nearest, ties even)."""
    lib = lib or _load()
    flat = np.asarray(values, dtype=np.float64).ravel()
    out = np.array([lib.oracle_enc16(float(v)) for v in flat], dtype=np.uint16)
    return out.reshape(np.shape(values))


def decbf16(bits, lib=None) -> np.ndarray:
    """bfloat16 bit patterns (any int array) -> float64, element by element."""
    lib = lib or _load()
    flat = np.asarray(bits, dtype=np.uint16).ravel()
    out = np.array([lib.oracle_decbf16(int(h)) for h in flat], dtype=np.float64)
    return out.reshape(np.shape(bits))


def encbf16(values, lib=None) -> np.ndarray:
    """float64 values -> bfloat16 bit patterns (round to nearest, ties even)."""
    lib = lib or _load()
    flat = np.asarray(values, dtype=np.float64).ravel()
    out = np.array([lib.oracle_encbf16(float(v)) for v in flat], dtype=np.uint16)
    return out.reshape(np.shape(values))


def activate(act, values, lib=None) -> np.ndarray:
    """The epilogue activation ACT_* applied to float64 values."""
    lib = lib or _load()
    flat = np.asarray(values, dtype=np.float64).ravel()
    out = np.array([lib.oracle_activate(int(act), float(v)) for v in flat], dtype=np.float64)
    return out.reshape(np.shape(values))


def _as_u16(x) -> np.ndarray:
    a = np.ascontiguousarray(x)
    if a.dtype == np.float16:
        a = a.view(np.uint16)
    if a.dtype != np.uint16:
        raise TypeError(f"expected 16-bit storage, got {a.dtype}")
    return a


def gemm(M, N, K, A, B, C=None, *, alpha=1.0, beta=0.0,
         layout_a=ROW_MAJOR, layout_b=ROW_MAJOR, out_type=OUT_F16,
         in_type=IN_F16, bias=None, activation=ACT_NONE, lda=None, ldb=None, ldc=None, batch=1,
         stride_a=0, stride_b=0, stride_c=0, rows=None, nthreads=None,
         lib=None):
    """Reference result and error scale, each shaped (batch, nrows, N).

    A, B: flat 16-bit storage (uint16 or float16 numpy arrays) in the
    layouts given, binary16 (in_type IN_F16) or bfloat16 bits (IN_BF16); C:
    binary16 (out_type OUT_F16), bfloat16 bits (OUT_BF16) or float32
    storage, read only when beta != 0.  bias: None or N float32 values added
    to every row; activation: ACT_* applied last (the returned scale is that
    of the pre-activation value).  alpha, beta are rounded to fp32 first, as the
    library receives them.  rows: optional row indices (sampled rows).
    lib: an alternative library handle from load_library (tests only).
    """
    lib = lib or _load()
    lda = lda if lda is not None else (K if layout_a == ROW_MAJOR else M)
    ldb = ldb if ldb is not None else (N if layout_b == ROW_MAJOR else K)
    ldc = ldc if ldc is not None else N
    a = _as_u16(A)
    b = _as_u16(B)
    c = None
    if beta != 0.0:
        if C is None:
            raise ValueError("beta != 0 needs C")
        c = np.ascontiguousarray(C)
        if out_type in (OUT_F16, OUT_BF16):
            c = _as_u16(c)
        elif c.dtype != np.float32:
            raise TypeError("fp32 C expected")
    bias_arr = None
    if bias is not None:
        bias_arr = np.ascontiguousarray(np.asarray(bias, dtype=np.float32))
        if bias_arr.size < N:
            raise ValueError("bias needs N values")
    rows_arr = None
    nrows = M
    if rows is not None:
        rows_arr = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        nrows = rows_arr.size
    shape = (max(batch, 0), max(nrows, 0), max(N, 0))   # C rejects negatives
    ref = np.zeros(shape, dtype=np.float64)
    scale = np.zeros(shape, dtype=np.float64)
    if nthreads is None:
        nthreads = os.cpu_count() or 1
    alpha32 = float(np.float32(alpha))
    beta32 = float(np.float32(beta))
    ptr = lambda x: None if x is None else x.ctypes.data
    rc = lib.oracle_gemm(batch, M, N, K, layout_a, layout_b, in_type, out_type,
                         lda, ldb, ldc, stride_a, stride_b, stride_c,
                         ptr(a), ptr(b), ptr(c), alpha32, beta32,
                         ptr(bias_arr), int(activation), ptr(rows_arr), nrows, ptr(ref), ptr(scale), int(nthreads))
    if rc != 0:
        raise RuntimeError(f"oracle_gemm failed with {rc}")
    return ref, scale


# ------------------------------------------------------------ softmax, attention

def softmax_row(x, lib=None) -> np.ndarray:
    """Softmax of one float64 row by the definition (two passes)."""
    lib = lib or _load()
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float64))
    y = np.zeros_like(x)
    lib.oracle_softmax_row(x.ctypes.data, x.size, y.ctypes.data)
    return y


def softmax_row_online(x, block, lib=None) -> np.ndarray:
    """The same softmax by the online recurrence, `block` elements at a time."""
    lib = lib or _load()
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float64))
    y = np.zeros_like(x)
    lib.oracle_softmax_row_online(x.ctypes.data, x.size, int(block), y.ctypes.data)
    return y


def softmax(rows, cols, X, ld=None, lib=None) -> np.ndarray:
    """Row softmax of a rows x cols matrix stored with leading dimension ld:
    binary16 storage (uint16/float16 arrays) or float32.  Returns float64
    (rows, cols)."""
    lib = lib or _load()
    ld = cols if ld is None else ld
    x = np.ascontiguousarray(X)
    in_f32 = x.dtype == np.float32
    if not in_f32:
        x = _as_u16(x)
    y = np.zeros((max(rows, 0), max(cols, 0)), dtype=np.float64)
    rc = lib.oracle_softmax(rows, cols, x.ctypes.data, int(in_f32), ld, y.ctypes.data)
    if rc != 0:
        raise RuntimeError(f"oracle_softmax failed with {rc}")
    return y


def attention(batch, heads, Sq, Sk, D, Q, K, V, *, Dv=None, scale=None, causal=False,
              q_strides=None, k_strides=None, v_strides=None, rows=None, nthreads=None,
              lib=None):
    """Reference O = softmax(scale Q K^T [causal mask]) V in float64.

    Q, K, V: flat binary16 storage (uint16 or float16 arrays); strides are
    (batch, head, row) in elements, defaulting to dense [batch][heads][S][D]
    (Dv for V).  scale defaults to 1/sqrt(D) and is rounded to fp32 first, as
    the GPU library receives it.  rows: optional query rows.  Returns (O,
    err, smax): O and err shaped (batch, heads, nrows, Dv), smax shaped
    (batch, heads, nrows) -- see ref_attention.c."""
    lib = lib or _load()
    Dv = D if Dv is None else Dv
    scale = (1.0 / np.sqrt(D)) if scale is None else scale
    scale32 = float(np.float32(scale))
    qs = q_strides or (heads * Sq * D, Sq * D, D)
    ks = k_strides or (heads * Sk * D, Sk * D, D)
    vs = v_strides or (heads * Sk * Dv, Sk * Dv, Dv)
    q, k, v = _as_u16(Q), _as_u16(K), _as_u16(V)
    rows_arr, nrows = None, Sq
    if rows is not None:
        rows_arr = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        nrows = rows_arr.size
    out = np.zeros((batch, heads, nrows, Dv), dtype=np.float64)
    err = np.zeros_like(out)
    smax = np.zeros((batch, heads, nrows), dtype=np.float64)
    if nthreads is None:
        nthreads = os.cpu_count() or 1
    ptr = lambda x: None if x is None else x.ctypes.data
    rc = lib.oracle_attention(batch, heads, Sq, Sk, D, Dv, ptr(q), *qs, ptr(k), *ks,
                              ptr(v), *vs, scale32, int(bool(causal)), ptr(rows_arr), nrows,
                              ptr(out), ptr(err), ptr(smax), int(nthreads))
    if rc != 0:
        raise RuntimeError(f"oracle_attention failed with {rc}")
    return out, err, smax


# ------------------------------------------------------------ residual + LayerNorm linear

def layernorm_row(z, gamma, beta_ln, eps, lib=None):
    """LayerNorm of one float64 row; returns (y, (mu, s, mean|z|))."""
    lib = lib or _load()
    z = np.ascontiguousarray(np.asarray(z, dtype=np.float64))
    g = np.ascontiguousarray(np.asarray(gamma, dtype=np.float32))
    b = np.ascontiguousarray(np.asarray(beta_ln, dtype=np.float32))
    y = np.zeros_like(z)
    st = np.zeros(3)
    lib.oracle_layernorm_row(z.ctypes.data, z.size, g.ctypes.data, b.ctypes.data, float(eps),
                             y.ctypes.data, st.ctypes.data)
    return y, tuple(st)


def gemm_layernorm(M, N, K, A, B, C=None, *, gamma, beta_ln, eps, alpha=1.0, beta=0.0,
                   bias=None, layout_a=ROW_MAJOR, layout_b=ROW_MAJOR, out_type=OUT_F16,
                   in_type=IN_F16, lda=None, ldb=None, ldc=None, batch=1, stride_a=0,
                   stride_b=0, stride_c=0, rows=None, nthreads=None, lib=None):
    """Reference Y = LayerNorm(alpha A B + beta C + bias) * gamma + beta_ln per
    row, with the arguments of gemm().  Returns (Y, T, stats): Y and the bound
    term T shaped (batch, nrows, N), stats (batch, nrows, 3) = mu, s =
    sqrt(var + eps), mean |Z| (see ref_layernorm.c).  eps is rounded to fp32
    first, as the library receives it."""
    lib = lib or _load()
    lda = lda if lda is not None else (K if layout_a == ROW_MAJOR else M)
    ldb = ldb if ldb is not None else (N if layout_b == ROW_MAJOR else K)
    ldc = ldc if ldc is not None else N
    a, b = _as_u16(A), _as_u16(B)
    c = None
    if beta != 0.0:
        c = np.ascontiguousarray(C)
        c = _as_u16(c) if out_type in (OUT_F16, OUT_BF16) else c
    g = np.ascontiguousarray(np.asarray(gamma, dtype=np.float32))
    bl = np.ascontiguousarray(np.asarray(beta_ln, dtype=np.float32))
    bias_arr = None if bias is None else np.ascontiguousarray(np.asarray(bias, dtype=np.float32))
    rows_arr, nrows = None, M
    if rows is not None:
        rows_arr = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        nrows = rows_arr.size
    y = np.zeros((batch, nrows, N))
    t = np.zeros_like(y)
    stats = np.zeros((batch, nrows, 3))
    if nthreads is None:
        nthreads = os.cpu_count() or 1
    ptr = lambda x: None if x is None else x.ctypes.data
    rc = lib.oracle_gemm_layernorm(batch, M, N, K, layout_a, layout_b, in_type, out_type,
                                   lda, ldb, ldc, stride_a, stride_b, stride_c,
                                   ptr(a), ptr(b), ptr(c), float(np.float32(alpha)),
                                   float(np.float32(beta)), ptr(bias_arr), ptr(g), ptr(bl),
                                   float(np.float32(eps)), ptr(rows_arr), nrows, ptr(y), ptr(t),
                                   ptr(stats), int(nthreads))
    if rc != 0:
        raise RuntimeError(f"oracle_gemm_layernorm failed with {rc}")
    return y, t, stats


# ------------------------------------------------------------ convolution

def conv_out_dim(size, k, stride, pad, dil, lib=None):
    return (lib or _load()).oracle_conv_out_dim(size, k, stride, pad, dil)


def conv2d(N, H, W, C, K, R, S, x, w, y_old=None, *, stride=(1, 1), pad=(0, 0), dil=(1, 1),
           alpha=1.0, beta=0.0, bias=None, activation=ACT_NONE, out_type=OUT_F16, rows=None,
           nthreads=None, lib=None):
    """Reference 2-D convolution: x NHWC, w KRSC (flat binary16 storage), y_old
    NPQK (binary16 or fp32, read when beta != 0).  Returns (ref, scale), each
    shaped (nrows, K) with nrows = N*P*Q unless rows (output pixels) is given."""
    lib = lib or _load()
    P = conv_out_dim(H, R, stride[0], pad[0], dil[0], lib)
    Q = conv_out_dim(W, S, stride[1], pad[1], dil[1], lib)
    if P < 0 or Q < 0:
        raise ValueError("the filter window does not fit the padded input")
    xa, wa = _as_u16(x), _as_u16(w)
    yo = None
    if beta != 0.0:
        yo = np.ascontiguousarray(y_old)
        yo = yo if out_type == OUT_F32 else _as_u16(yo)
    bias_arr = None if bias is None else np.ascontiguousarray(np.asarray(bias, dtype=np.float32))
    rows_arr, nrows = None, N * P * Q
    if rows is not None:
        rows_arr = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        nrows = rows_arr.size
    ref = np.zeros((nrows, K))
    scale = np.zeros((nrows, K))
    if nthreads is None:
        nthreads = os.cpu_count() or 1
    ptr = lambda a: None if a is None else a.ctypes.data
    rc = lib.oracle_conv2d(N, H, W, C, K, R, S, stride[0], stride[1], pad[0], pad[1], dil[0],
                           dil[1], ptr(xa), ptr(wa), ptr(yo), int(out_type == OUT_F32),
                           float(np.float32(alpha)), float(np.float32(beta)), ptr(bias_arr),
                           int(activation), ptr(rows_arr), nrows, ptr(ref), ptr(scale),
                           int(nthreads))
    if rc != 0:
        raise RuntimeError(f"oracle_conv2d failed with {rc}")
    return ref, scale
