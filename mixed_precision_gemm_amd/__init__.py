"""Python binding of the MI355X fp16 / bf16 -> fp32-accumulate GEMM library.

Thin ctypes marshalling over the C ABI declared in include/gemm_f16f32.h and
include/gemm_bf16f32.h: the functions below carry the same names and
arguments as the C entry points, and
every step of the computation runs in the HIP kernels of libmpgemm.so.  There
is no fallback: if the library is missing, loading raises.  torch is used only
for device buffers (operands and the caller-owned workspace) and streams, in
the convenience layer (`Plan`, `gemm`).
"""
import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmpgemm.so")

GEMM_ROW_MAJOR, GEMM_COL_MAJOR = 0, 1
GEMM_OUT_F16, GEMM_OUT_F32, GEMM_OUT_BF16 = 0, 1, 2
GEMM_ACT_NONE, GEMM_ACT_RELU, GEMM_ACT_GELU, GEMM_ACT_SILU = 0, 1, 2, 3
GEMM_OK = 0
GEMM_ERR_INVALID_ARG = -1
GEMM_ERR_UNSUPPORTED = -2
GEMM_ERR_HIP = -3
GEMM_ERR_NOMEM = -4
GEMM_ERR_SCRATCH = -5
GEMM_WS_ANY_ALIGNMENT = 1

EXPORTED = ("gemm_f16f32_plan", "gemm_f16f32_run", "gemm_f16f32_destroy",
            "gemm_f16f32_status_string", "gemm_f16f32_plan_kernel",
            "gemm_bf16f32_plan", "gemm_bf16f32_run", "gemm_f16f32_set_epilogue",
            "gemm_f16f32_workspace_size", "gemm_f16f32_workspace_init",
            "gemm_f16f32_run_noalloc", "gemm_f16f32_set_layernorm",
            "attn_f16_plan", "attn_f16_run", "attn_f16_destroy", "attn_f16_plan_kernel",
            "attn_softmax_rows",
            "conv_f16_plan", "conv_f16_output_size", "conv_f16_run", "conv_f16_destroy",
            "conv_f16_plan_kernel")

_lib = None


class GemmError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {gemm_f16f32_status_string(status)} ({status})")
        self.status = status


def library() -> ctypes.CDLL:
    """Loads libmpgemm.so (built by mixed_precision_gemm_amd.build)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is missing: build it with "
                "`python -m mixed_precision_gemm_amd.build` (no fallback exists)")
        lib = ctypes.CDLL(LIB_PATH)
        i64, vp = ctypes.c_int64, ctypes.c_void_p
        for fam in ("f16f32", "bf16f32"):
            plan_fn = getattr(lib, f"gemm_{fam}_plan")
            plan_fn.argtypes = [ctypes.POINTER(vp), i64, i64, i64,
                                ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                i64, i64, i64, i64, i64, i64, i64]
            plan_fn.restype = ctypes.c_int
            run_fn = getattr(lib, f"gemm_{fam}_run")
            run_fn.argtypes = [vp, vp, vp, vp, ctypes.c_float, ctypes.c_float, vp, i64, vp]
            run_fn.restype = ctypes.c_int
        lib.gemm_f16f32_workspace_size.argtypes = [vp, ctypes.c_int, ctypes.POINTER(i64)]
        lib.gemm_f16f32_workspace_size.restype = ctypes.c_int
        lib.gemm_f16f32_workspace_init.argtypes = [vp, i64, vp]
        lib.gemm_f16f32_workspace_init.restype = ctypes.c_int
        lib.gemm_f16f32_run_noalloc.argtypes = [vp, vp, vp, vp, ctypes.c_float, ctypes.c_float, vp]
        lib.gemm_f16f32_run_noalloc.restype = ctypes.c_int
        st3 = ctypes.c_int64 * 3
        lib.attn_f16_plan.argtypes = [ctypes.POINTER(vp), i64, i64, i64, i64, i64,
                                      st3, st3, st3, st3, ctypes.c_int, ctypes.c_int]
        lib.attn_f16_plan.restype = ctypes.c_int
        lib.attn_f16_run.argtypes = [vp, vp, vp, vp, vp, ctypes.c_float, vp]
        lib.attn_f16_run.restype = ctypes.c_int
        lib.attn_f16_destroy.argtypes = [vp]
        lib.attn_f16_destroy.restype = ctypes.c_int
        lib.attn_f16_plan_kernel.argtypes = [vp]
        lib.attn_f16_plan_kernel.restype = ctypes.c_char_p
        lib.attn_softmax_rows.argtypes = [i64, i64, vp, i64, ctypes.c_int, vp, i64, ctypes.c_int, vp]
        lib.attn_softmax_rows.restype = ctypes.c_int
        lib.conv_f16_plan.argtypes = [ctypes.POINTER(vp)] + [i64] * 13 + [ctypes.c_int]
        lib.conv_f16_plan.restype = ctypes.c_int
        lib.conv_f16_output_size.argtypes = [vp, ctypes.POINTER(i64), ctypes.POINTER(i64)]
        lib.conv_f16_output_size.restype = ctypes.c_int
        lib.conv_f16_run.argtypes = [vp, vp, vp, vp, ctypes.c_float, ctypes.c_float, vp,
                                     ctypes.c_int, vp]
        lib.conv_f16_run.restype = ctypes.c_int
        lib.conv_f16_destroy.argtypes = [vp]
        lib.conv_f16_destroy.restype = ctypes.c_int
        lib.conv_f16_plan_kernel.argtypes = [vp]
        lib.conv_f16_plan_kernel.restype = ctypes.c_char_p
        lib.gemm_f16f32_set_epilogue.argtypes = [vp, vp, ctypes.c_int]
        lib.gemm_f16f32_set_epilogue.restype = ctypes.c_int
        lib.gemm_f16f32_set_layernorm.argtypes = [vp, vp, vp, ctypes.c_float]
        lib.gemm_f16f32_set_layernorm.restype = ctypes.c_int
        lib.gemm_f16f32_destroy.argtypes = [vp]
        lib.gemm_f16f32_destroy.restype = ctypes.c_int
        lib.gemm_f16f32_status_string.argtypes = [ctypes.c_int]
        lib.gemm_f16f32_status_string.restype = ctypes.c_char_p
        lib.gemm_f16f32_plan_kernel.argtypes = [vp]
        lib.gemm_f16f32_plan_kernel.restype = ctypes.c_char_p
        _lib = lib
    return _lib


# ----------------------------------------------------------- C entry points

def gemm_f16f32_plan(M, N, K, layout_a, layout_b, out_type, lda, ldb, ldc,
                     batch=1, stride_a=0, stride_b=0, stride_c=0):
    """Returns (status, plan_handle); the handle is None unless status == 0."""
    h = ctypes.c_void_p()
    st = library().gemm_f16f32_plan(ctypes.byref(h), M, N, K, layout_a, layout_b,
                                    out_type, lda, ldb, ldc, batch, stride_a,
                                    stride_b, stride_c)
    return st, (h.value if st == GEMM_OK else None)


def gemm_f16f32_run(plan, A, B, C, alpha, beta, workspace=None, workspace_bytes=0,
                    stream=None):
    """A, B, C, workspace: device addresses (ints; workspace None when the
    plan needs none); stream: hipStream_t as int or None."""
    return library().gemm_f16f32_run(plan, A, B, C, alpha, beta, workspace,
                                     workspace_bytes, stream)


def gemm_f16f32_run_noalloc(plan, A, B, C, alpha, beta, stream=None):
    """Runs a plan of either input type with the library's static device
    scratch as workspace (no allocation; calls on one device must not
    overlap in time)."""
    return library().gemm_f16f32_run_noalloc(plan, A, B, C, alpha, beta, stream)


def gemm_f16f32_workspace_size(plan, flags=0):
    """Returns (status, bytes)."""
    n = ctypes.c_int64(-1)
    st = library().gemm_f16f32_workspace_size(plan, flags, ctypes.byref(n))
    return st, n.value


def gemm_f16f32_workspace_init(workspace, nbytes, stream=None):
    """Zero-fills the workspace's counter words on the stream (no allocation)."""
    return library().gemm_f16f32_workspace_init(workspace, nbytes, stream)


def gemm_bf16f32_plan(M, N, K, layout_a, layout_b, out_type, lda, ldb, ldc,
                      batch=1, stride_a=0, stride_b=0, stride_c=0):
    """bfloat16 A and B; out_type GEMM_OUT_BF16 or GEMM_OUT_F32.  Returns
    (status, plan_handle); the handle is None unless status == 0."""
    h = ctypes.c_void_p()
    st = library().gemm_bf16f32_plan(ctypes.byref(h), M, N, K, layout_a, layout_b,
                                     out_type, lda, ldb, ldc, batch, stride_a,
                                     stride_b, stride_c)
    return st, (h.value if st == GEMM_OK else None)


def gemm_bf16f32_run(plan, A, B, C, alpha, beta, workspace=None, workspace_bytes=0,
                     stream=None):
    """Runs a plan made by gemm_bf16f32_plan (device addresses as ints)."""
    return library().gemm_bf16f32_run(plan, A, B, C, alpha, beta, workspace,
                                      workspace_bytes, stream)


def gemm_f16f32_set_epilogue(plan, bias, activation):
    """bias: device address of N fp32 values (int) or None; activation GEMM_ACT_*."""
    return library().gemm_f16f32_set_epilogue(plan, bias, activation)


def gemm_f16f32_set_layernorm(plan, gamma, beta_ln, eps):
    """gamma, beta_ln: device addresses of N fp32 values (ints), gamma None to
    remove the normalisation; eps: fp32."""
    return library().gemm_f16f32_set_layernorm(plan, gamma, beta_ln, eps)


def gemm_f16f32_destroy(plan):
    return library().gemm_f16f32_destroy(plan)


def gemm_f16f32_status_string(status):
    return library().gemm_f16f32_status_string(status).decode()


def gemm_f16f32_plan_kernel(plan):
    return library().gemm_f16f32_plan_kernel(plan).decode()


# ------------------------------------------------------- convenience layer

class Plan:
    """Owns a plan handle; `run` launches on a stream (torch's current one by
    default).  dtype: "f16" (binary16 A and B, C binary16 or fp32) or
    "bf16" (bfloat16 A and B; out_type defaults to GEMM_OUT_BF16).

    The workspace a run needs is the caller's: pass one (a zero-filled CUDA
    tensor of at least `workspace_bytes()` bytes, or a raw address with its
    size) to `run`, or let the Plan keep its own -- a zero-filled torch
    tensor, made on first need and enlarged when misaligned operands call
    for room to repack them -- used by the runs that pass none.  Runs that
    may execute at the same time need distinct workspaces."""

    def __init__(self, M, N, K, layout_a=GEMM_ROW_MAJOR, layout_b=GEMM_ROW_MAJOR,
                 out_type=None, lda=None, ldb=None, ldc=None, batch=1,
                 stride_a=0, stride_b=0, stride_c=0, dtype="f16"):
        if dtype not in ("f16", "bf16"):
            raise ValueError(f"dtype must be 'f16' or 'bf16', not {dtype!r}")
        lda = lda if lda is not None else (K if layout_a == GEMM_ROW_MAJOR else M)
        ldb = ldb if ldb is not None else (N if layout_b == GEMM_ROW_MAJOR else K)
        ldc = ldc if ldc is not None else N
        if out_type is None:
            out_type = GEMM_OUT_BF16 if dtype == "bf16" else GEMM_OUT_F16
        plan_fn = gemm_bf16f32_plan if dtype == "bf16" else gemm_f16f32_plan
        st, h = plan_fn(M, N, K, layout_a, layout_b, out_type, lda, ldb,
                        ldc, batch, stride_a, stride_b, stride_c)
        if st != GEMM_OK:
            raise GemmError(st, plan_fn.__name__)
        self.dtype = dtype
        self._run = gemm_bf16f32_run if dtype == "bf16" else gemm_f16f32_run
        self.handle = h
        self.shape = (M, N, K)
        self.kernel = gemm_f16f32_plan_kernel(h)
        self._ws = None

    def workspace_bytes(self, flags=0):
        st, n = gemm_f16f32_workspace_size(self.handle, flags)
        if st != GEMM_OK:
            raise GemmError(st, "gemm_f16f32_workspace_size")
        return n

    def _own_workspace(self, A, B, device):
        """The Plan's own workspace, large enough for these operands."""
        import torch
        ptr = lambda t: t if isinstance(t, int) else t.data_ptr()
        misaligned = ptr(A) % 16 != 0 or ptr(B) % 16 != 0
        need = self.workspace_bytes(GEMM_WS_ANY_ALIGNMENT if misaligned else 0)
        if need == 0:
            return None, 0
        if self._ws is None or self._ws.numel() < need:
            # zero-filled on torch's current stream: the counter words start at 0
            self._ws = torch.zeros(need, dtype=torch.uint8, device=device)
        return self._ws.data_ptr(), self._ws.numel()

    def run(self, A, B, C, alpha=1.0, beta=0.0, stream=None, workspace=None,
            workspace_bytes=None):
        """A, B, C: torch tensors (device) or raw device addresses.  workspace:
        a CUDA tensor, a raw address (with workspace_bytes), or None for the
        Plan's own."""
        ptr = lambda t: t if isinstance(t, int) or t is None else t.data_ptr()
        import torch
        if stream is None:
            stream = torch.cuda.current_stream().cuda_stream
        elif not isinstance(stream, int):
            stream = stream.cuda_stream
        if workspace is None:
            dev = C.device if hasattr(C, "device") else torch.device("cuda", torch.cuda.current_device())
            ws, nbytes = self._own_workspace(A, B, dev)
        elif isinstance(workspace, int):
            ws, nbytes = workspace, int(workspace_bytes or 0)
        else:
            ws, nbytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
        st = self._run(self.handle, ptr(A), ptr(B), ptr(C), alpha, beta, ws, nbytes, stream)
        if st != GEMM_OK:
            raise GemmError(st, self._run.__name__)

    def set_epilogue(self, bias=None, activation=GEMM_ACT_NONE):
        """Fused epilogue of later runs: C = act(alpha A B + beta C + bias).
        bias: None, a device address, or a CUDA float32 tensor of N values
        (the caller keeps it alive while runs use it)."""
        addr = bias if bias is None or isinstance(bias, int) else bias.data_ptr()
        if bias is not None and not isinstance(bias, int):
            import torch
            if bias.dtype != torch.float32 or bias.numel() < self.shape[1] or not bias.is_contiguous():
                raise TypeError("bias must be a contiguous float32 tensor of N values")
        st = gemm_f16f32_set_epilogue(self.handle, addr, activation)
        if st != GEMM_OK:
            raise GemmError(st, "gemm_f16f32_set_epilogue")
        self._bias = bias

    def set_layernorm(self, gamma=None, beta_ln=None, eps=1e-5):
        """Later runs: C = LayerNorm(alpha A B + beta C + bias) * gamma + beta_ln
        per row.  gamma, beta_ln: contiguous CUDA float32 tensors of N values
        (kept alive here), or None to remove the normalisation."""
        addr = lambda t: None if t is None else (t if isinstance(t, int) else t.data_ptr())
        for t in (gamma, beta_ln):
            if t is not None and not isinstance(t, int):
                import torch
                if t.dtype != torch.float32 or t.numel() < self.shape[1] or not t.is_contiguous():
                    raise TypeError("gamma and beta_ln must be contiguous float32 tensors of N values")
        st = gemm_f16f32_set_layernorm(self.handle, addr(gamma), addr(beta_ln), eps)
        if st != GEMM_OK:
            raise GemmError(st, "gemm_f16f32_set_layernorm")
        self._ln = (gamma, beta_ln)
        self._ws = None if self._ws is not None and self._ws.numel() < self.workspace_bytes() else self._ws

    def close(self):
        if self.handle is not None:
            gemm_f16f32_destroy(self.handle)
            self.handle = None
        self._ws = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()


def _layout_of(t, rows, cols):
    """(layout, ld) of a 2-D (or batched 3-D) torch view, or None."""
    s_r, s_c = t.stride(-2), t.stride(-1)
    if s_c == 1 and (s_r >= max(cols, 1) or rows <= 1):
        return GEMM_ROW_MAJOR, max(s_r, cols, 1)
    if s_r == 1 and (s_c >= max(rows, 1) or cols <= 1):
        return GEMM_COL_MAJOR, max(s_c, rows, 1)
    return None


def gemm(A, B, C=None, alpha=1.0, beta=0.0, out_dtype=None, bias=None,
         activation=GEMM_ACT_NONE):
    """C = alpha * A @ B + beta * C for float16 (or bfloat16) CUDA tensors A
    (.., M, K) and B (.., K, N); layouts and leading dimensions come from the
    strides.  Returns C (allocated when None; the input type unless
    out_dtype is torch.float32).  bias (float32, N values) and activation
    (GEMM_ACT_*) select the fused epilogue C = act(alpha A B + beta C + bias)."""
    import torch
    if A.dtype != B.dtype or A.dtype not in (torch.float16, torch.bfloat16):
        raise TypeError("A and B must both be float16 or both bfloat16")
    dtype = "bf16" if A.dtype == torch.bfloat16 else "f16"
    batched = A.dim() == 3
    M, K = A.shape[-2:]
    K2, N = B.shape[-2:]
    if K != K2:
        raise ValueError("inner dimensions differ")
    batch = A.shape[0] if batched else 1
    la = _layout_of(A, M, K)
    lb = _layout_of(B, K, N)
    if la is None:
        A = A.contiguous(); la = _layout_of(A, M, K)
    if lb is None:
        B = B.contiguous(); lb = _layout_of(B, K, N)
    if C is None:
        dt = out_dtype or A.dtype
        C = torch.empty((batch, M, N) if batched else (M, N), dtype=dt, device=A.device)
        beta = 0.0
    if C.dtype not in (torch.float32, A.dtype):
        raise TypeError("C must be float32 or the input type")
    out_type = (GEMM_OUT_F32 if C.dtype == torch.float32 else
                GEMM_OUT_BF16 if dtype == "bf16" else GEMM_OUT_F16)
    if C.stride(-1) != 1:
        raise ValueError("C must be row-major")
    ldc = max(C.stride(-2), N, 1)
    sa = A.stride(0) if batched else 0
    sb = B.stride(0) if batched else 0
    sc = C.stride(0) if batched else 0
    key = (M, N, K, la, lb, out_type, ldc, batch, sa, sb, sc, dtype, C.device)
    p = _plan_cache.get(key)
    if p is None:
        if len(_plan_cache) >= _PLAN_CACHE_SIZE:
            _plan_cache.pop(next(iter(_plan_cache))).close()
        p = Plan(M, N, K, la[0], lb[0], out_type, la[1], lb[1], ldc, batch,
                 sa, sb, sc, dtype=dtype)
        _plan_cache[key] = p
    # The epilogue is part of the plan: set for this call (host only).
    p.set_epilogue(bias, activation)
    p.run(A, B, C, alpha, beta)
    return C


# Plans (with their workspaces) of recent `gemm` calls, by problem description.
# Runs of one cached plan on the same stream share its workspace in order; a
# caller that runs the same shape on several streams at once should make its
# own Plan per stream.
_PLAN_CACHE_SIZE = 64
_plan_cache = {}


# ------------------------------------------------------------ attention, softmax

def attn_f16_plan(batch, heads, Sq, Sk, D, q_strides, k_strides, v_strides, o_strides,
                  causal=0, out_type=GEMM_OUT_F16):
    """Returns (status, plan_handle); strides are (batch, head, row) in elements."""
    st3 = ctypes.c_int64 * 3
    h = ctypes.c_void_p()
    st = library().attn_f16_plan(ctypes.byref(h), batch, heads, Sq, Sk, D, st3(*q_strides),
                                 st3(*k_strides), st3(*v_strides), st3(*o_strides),
                                 int(causal), out_type)
    return st, (h.value if st == GEMM_OK else None)


def attn_f16_run(plan, Q, K, V, O, scale, stream=None):
    """Q, K, V, O: device addresses (ints); stream: hipStream_t as int or None."""
    return library().attn_f16_run(plan, Q, K, V, O, scale, stream)


def attn_f16_destroy(plan):
    return library().attn_f16_destroy(plan)


def attn_f16_plan_kernel(plan):
    return library().attn_f16_plan_kernel(plan).decode()


def attn_softmax_rows(rows, cols, x, ldx, in_type, y, ldy, out_type, stream=None):
    """Row softmax of device storage x into y (addresses as ints)."""
    return library().attn_softmax_rows(rows, cols, x, ldx, in_type, y, ldy, out_type, stream)


def _strides3(t):
    """(batch, head, row) element strides of a (B, H, S, D) tensor view."""
    if t.stride(-1) != 1:
        raise ValueError("the last dimension must be contiguous")
    return (t.stride(0), t.stride(1), t.stride(2))


def attention(q, k, v, scale=None, causal=False, out=None, out_dtype=None):
    """O = softmax(scale Q K^T [causal]) V for float16 CUDA tensors of shape
    (batch, heads, S, D) (any strides with the last dimension contiguous;
    D = 64 or 128).  Returns O (allocated when None: float16 unless out_dtype
    is torch.float32)."""
    import math
    import torch
    if q.dtype != torch.float16 or k.dtype != torch.float16 or v.dtype != torch.float16:
        raise TypeError("Q, K and V must be float16")
    B, H, Sq, D = q.shape
    Sk = k.shape[2]
    if out is None:
        out = torch.empty((B, H, Sq, D), dtype=out_dtype or torch.float16, device=q.device)
    out_type = GEMM_OUT_F32 if out.dtype == torch.float32 else GEMM_OUT_F16
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    st, h = attn_f16_plan(B, H, Sq, Sk, D, _strides3(q), _strides3(k), _strides3(v),
                          _strides3(out), int(causal), out_type)
    if st != GEMM_OK:
        raise GemmError(st, "attn_f16_plan")
    try:
        st = attn_f16_run(h, q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), scale,
                          torch.cuda.current_stream().cuda_stream)
        if st != GEMM_OK:
            raise GemmError(st, "attn_f16_run")
    finally:
        attn_f16_destroy(h)
    return out


def softmax(x, out=None):
    """Row softmax of a 2-D float16 or float32 CUDA tensor (rows contiguous).
    out: a tensor of the same shape (float16 or float32), or None for one of
    x's type; may be x itself."""
    import torch
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be 2-D with contiguous rows")
    if out is None:
        out = torch.empty_like(x)
    types = {torch.float16: GEMM_OUT_F16, torch.float32: GEMM_OUT_F32}
    st = attn_softmax_rows(x.shape[0], x.shape[1], x.data_ptr(), max(x.stride(0), x.shape[1]),
                           types[x.dtype], out.data_ptr(), max(out.stride(0), out.shape[1]),
                           types[out.dtype], torch.cuda.current_stream().cuda_stream)
    if st != GEMM_OK:
        raise GemmError(st, "attn_softmax_rows")
    return out


# ------------------------------------------------------------ convolution

def conv_f16_plan(N, H, W, C, K, R, S, stride=(1, 1), pad=(0, 0), dil=(1, 1),
                  out_type=GEMM_OUT_F16):
    """Returns (status, plan_handle)."""
    h = ctypes.c_void_p()
    st = library().conv_f16_plan(ctypes.byref(h), N, H, W, C, K, R, S, stride[0], stride[1],
                                 pad[0], pad[1], dil[0], dil[1], out_type)
    return st, (h.value if st == GEMM_OK else None)


def conv_f16_output_size(plan):
    """Returns (status, P, Q)."""
    P, Q = ctypes.c_int64(), ctypes.c_int64()
    st = library().conv_f16_output_size(plan, ctypes.byref(P), ctypes.byref(Q))
    return st, P.value, Q.value


def conv_f16_run(plan, x, w, y, alpha=1.0, beta=0.0, bias=None, activation=GEMM_ACT_NONE,
                 stream=None):
    """x, w, y, bias: device addresses (ints; bias may be None)."""
    return library().conv_f16_run(plan, x, w, y, alpha, beta, bias, activation, stream)


def conv_f16_destroy(plan):
    return library().conv_f16_destroy(plan)


def conv_f16_plan_kernel(plan):
    return library().conv_f16_plan_kernel(plan).decode()


def conv2d(x, w, stride=(1, 1), padding=(0, 0), dilation=(1, 1), bias=None,
           activation=GEMM_ACT_NONE, out=None, alpha=1.0, beta=0.0, out_dtype=None):
    """Convolution of a float16 NHWC CUDA tensor x (N, H, W, C) with float16
    filters w (K, R, S, C), both contiguous.  Returns y (N, P, Q, K), float16
    unless out_dtype is torch.float32 (or out is given)."""
    import torch
    if x.dtype != torch.float16 or w.dtype != torch.float16:
        raise TypeError("x and w must be float16")
    if not x.is_contiguous() or not w.is_contiguous():
        raise ValueError("x (NHWC) and w (KRSC) must be contiguous")
    N, H, W_, C = x.shape
    K, R, S, C2 = w.shape
    if C != C2:
        raise ValueError("channel counts differ")
    out_type = GEMM_OUT_F32 if (out is not None and out.dtype == torch.float32) or \
        out_dtype == torch.float32 else GEMM_OUT_F16
    st, h = conv_f16_plan(N, H, W_, C, K, R, S, stride, padding, dilation, out_type)
    if st != GEMM_OK:
        raise GemmError(st, "conv_f16_plan")
    try:
        _, P, Q = conv_f16_output_size(h)
        if out is None:
            out = torch.empty((N, P, Q, K), dtype=torch.float32 if out_type == GEMM_OUT_F32
                              else torch.float16, device=x.device)
        st = conv_f16_run(h, x.data_ptr(), w.data_ptr(), out.data_ptr(), alpha, beta,
                          None if bias is None else bias.data_ptr(), activation,
                          torch.cuda.current_stream().cuda_stream)
        if st != GEMM_OK:
            raise GemmError(st, "conv_f16_run")
    finally:
        conv_f16_destroy(h)
    return out
