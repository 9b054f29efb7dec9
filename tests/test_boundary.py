"""C-ABI boundary tests that need no GPU.

The library must load and export every function include/*.h declares; the
planner (which makes no HIP call) must enforce every documented rule; run must
reject bad arguments before it reaches the HIP runtime.
"""
import glob
import os
import re

import pytest

import mixed_precision_gemm_amd as mpg
from mixed_precision_gemm_amd import (GEMM_COL_MAJOR, GEMM_ERR_INVALID_ARG,
                                      GEMM_ERR_UNSUPPORTED, GEMM_OK,
                                      GEMM_OUT_F16, GEMM_OUT_F32,
                                      GEMM_ROW_MAJOR)

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        for m in re.finditer(r"\b((?:gemm|attn|conv)_\w+)\s*\(", text):
            names.add(m.group(1))
    return names


def test_library_exports_every_declared_symbol():
    names = declared_functions()
    assert names, "no declarations found"
    lib = mpg.library()
    for n in sorted(names):
        assert hasattr(lib, n), n
    assert names == set(mpg.EXPORTED)


def plan(M=64, N=64, K=64, la=GEMM_ROW_MAJOR, lb=GEMM_ROW_MAJOR, out=GEMM_OUT_F16,
         lda=None, ldb=None, ldc=None, batch=1, sa=0, sb=0, sc=0):
    lda = lda if lda is not None else (K if la == GEMM_ROW_MAJOR else M)
    ldb = ldb if ldb is not None else (N if lb == GEMM_ROW_MAJOR else K)
    ldc = ldc if ldc is not None else N
    st, h = mpg.gemm_f16f32_plan(M, N, K, la, lb, out, lda, ldb, ldc, batch, sa, sb, sc)
    if h is not None:
        mpg.gemm_f16f32_destroy(h)
    return st


def test_valid_plans():
    assert plan() == GEMM_OK
    for la in (0, 1):
        for lb in (0, 1):
            for out in (0, 1):
                assert plan(127, 257, 33, la, lb, out) == GEMM_OK
    assert plan(1, 4096, 4096) == GEMM_OK
    assert plan(64, 64, 64, batch=512, sa=4096, sb=4096, sc=4096) == GEMM_OK
    # degenerate extents are valid
    assert plan(0, 5, 5, ldc=5) == GEMM_OK
    assert plan(5, 0, 5, ldb=1, ldc=1) == GEMM_OK
    assert plan(5, 5, 0, lda=1) == GEMM_OK


@pytest.mark.parametrize("kw", [
    dict(M=-1), dict(N=-1), dict(K=-1),
    dict(la=2), dict(lb=-1), dict(out=7),
    dict(lda=63), dict(ldb=63), dict(ldc=63),
    dict(la=GEMM_COL_MAJOR, M=100, lda=99),
    dict(lb=GEMM_COL_MAJOR, K=100, ldb=99),
    dict(batch=0), dict(batch=2, sa=-1, sb=0, sc=64 * 64),
    dict(batch=2, sa=0, sb=0, sc=64 * 64 - 1),     # C batch items overlap
])
def test_invalid_plans(kw):
    assert plan(**kw) == GEMM_ERR_INVALID_ARG


def test_large_leading_dimensions_repack_both_operands():
    """Tile offsets are 32-bit: A or B with a leading dimension above 2^22
    elements is read from packed copies (both operands), C's is unlimited;
    only a row or column longer than 2^22 elements is unsupported."""
    def kern(*a, **k):
        with mpg.Plan(*a, **k) as p:
            return p.kernel, p.workspace_bytes()
    big = (1 << 22) + 8
    for shape, kw in [((64, 64, 64), dict(lda=big)),
                      ((2048, 2048, 2048), dict(ldb=big)),
                      ((16, 4096, 4096), dict(layout_b=GEMM_COL_MAJOR, ldb=big)),
                      ((8192, 8192, 1024), dict(lda=big))]:
        name, ws = kern(*shape, **kw)
        assert name.endswith("_pkab"), (shape, kw, name)
        M, N, K = shape
        assert ws >= 4096 + 2 * (M * K + K * N)
    name, ws = kern(64, 64, 64, ldc=big)
    assert "_pk" not in name and ws == 0
    assert plan(lda=1 << 22) == GEMM_OK
    # K = 0 reads no operand: no copies whatever the leading dimension
    assert kern(64, 64, 0, lda=big)[1] == 0
    assert plan(M=8, N=8, K=(1 << 22) + 1, lda=big) == GEMM_ERR_UNSUPPORTED
    assert plan(M=(1 << 22) + 1, N=8, K=8, la=GEMM_COL_MAJOR, lda=big) == GEMM_ERR_UNSUPPORTED


def test_streaming_plan_with_large_column_pitch():
    """A streaming plan whose B spans far more than 2^31 bytes (ldb = 2^22,
    N = 512) is accepted and reads B in place: its lane offsets are taken
    from each workgroup's first column."""
    with mpg.Plan(16, 512, 64, layout_b=GEMM_COL_MAJOR, ldb=1 << 22) as p:
        assert p.kernel == "gemm_stream16x16_nt_direct"
        assert p.workspace_bytes() == 0
    with mpg.Plan(16, 152064, 8192, layout_b=GEMM_COL_MAJOR) as p:
        # wide N: 48 columns per workgroup, unsplit
        assert p.kernel == "gemm_stream16x48_nt_direct"


def test_null_out_pointer():
    lib = mpg.library()
    assert lib.gemm_f16f32_plan(None, 1, 1, 1, 0, 0, 0, 1, 1, 1, 1, 0, 0, 0) == GEMM_ERR_INVALID_ARG


def test_destroy_null_and_status_strings():
    assert mpg.gemm_f16f32_destroy(None) == GEMM_OK
    for st in (0, -1, -2, -3, -4, -5):
        s = mpg.gemm_f16f32_status_string(st)
        assert s.startswith("GEMM_")
    assert mpg.gemm_f16f32_status_string(12345) == "unknown status"
    assert mpg.gemm_f16f32_plan_kernel(None) == "invalid"


def test_kernel_choice_by_regime():
    def kern(*a, **k):
        p = mpg.Plan(*a, **k)
        name = p.kernel
        p.close()
        return name
    assert kern(8192, 8192, 8192).startswith("gemm_256x256")
    assert kern(8192, 8192, 8192, layout_b=GEMM_COL_MAJOR).endswith("nt_direct")
    # skinny, K-contiguous A and B: streaming kernel; other layouts: small tiles
    assert kern(16, 4096, 4096, layout_b=GEMM_COL_MAJOR).startswith("gemm_stream16x16")
    # at most 4 rows with row-major A and B: the row-vector kernel, K slices of
    # at least 1024 for about 256 workgroups; other layouts keep the tiles
    assert kern(1, 4096, 4096) == "gemm_rowvec4x64_nn_direct_sk4"
    assert kern(4, 11008, 4096) == "gemm_rowvec4x64_nn_direct_sk2"
    assert kern(3, 4096, 512) == "gemm_rowvec4x64_nn_direct"
    assert kern(5, 4096, 4096).startswith("gemm_128x128")
    assert kern(1, 4096, 4096, layout_a=GEMM_COL_MAJOR).startswith("gemm_128x128")
    # M <= 16 with N >= 8192: 48 columns per workgroup (171 or more), not split
    assert kern(16, 11008, 4096, layout_b=GEMM_COL_MAJOR) == "gemm_stream16x48_nt_direct"
    assert kern(16, 8192, 4096, layout_b=GEMM_COL_MAJOR) == "gemm_stream16x48_nt_direct"
    assert kern(16, 8192, 3000, layout_b=GEMM_COL_MAJOR) == "gemm_stream16x48_nt_direct"
    assert kern(16, 8192, 4096, layout_b=GEMM_COL_MAJOR, batch=2, stride_a=16 * 4096,
                stride_b=8192 * 4096, stride_c=16 * 8192) == "gemm_stream16x48_nt_direct"
    # 16 < M <= 32: 64 columns for N = 8192 .. 10239, fewer than 160
    # workgroups in K slices of >= 1024; 48 columns from N = 10240
    assert kern(32, 10176, 4096, layout_b=GEMM_COL_MAJOR) == "gemm_stream32x64_nt_direct_sk4"
    assert kern(20, 8192, 3000, layout_b=GEMM_COL_MAJOR) == "gemm_stream32x64_nt_direct_sk2"
    assert kern(20, 8192, 1024, layout_b=GEMM_COL_MAJOR) == "gemm_stream32x64_nt_direct"
    assert kern(20, 10239, 4096, layout_b=GEMM_COL_MAJOR) == "gemm_stream32x64_nt_direct"
    assert kern(32, 10240, 4096, layout_b=GEMM_COL_MAJOR) == "gemm_stream32x48_nt_direct"
    # up to 128 rows: the 32 x 64 streaming tile while ceil(M/32) x ceil(N/64)
    # workgroups fit one per CU and K <= 8192 (split as above below 160)
    assert kern(40, 4096, 4096, layout_b=GEMM_COL_MAJOR) == "gemm_stream32x64_nt_direct_sk4"
    assert kern(128, 4096, 4096, layout_b=GEMM_COL_MAJOR) == "gemm_stream32x64_nt_direct"
    assert kern(64, 8192, 4096, layout_b=GEMM_COL_MAJOR) == "gemm_stream32x64_nt_direct"
    assert kern(96, 2048, 4096, layout_b=GEMM_COL_MAJOR) == "gemm_stream32x64_nt_direct_sk4"
    assert kern(128, 4096, 8192, layout_b=GEMM_COL_MAJOR) == "gemm_stream32x64_nt_direct"
    assert kern(128, 6144, 4096, layout_b=GEMM_COL_MAJOR).startswith("gemm_128x128")
    assert kern(128, 2048, 16384, layout_b=GEMM_COL_MAJOR).startswith("gemm_128x128")
    assert not kern(128, 4096, 512, layout_b=GEMM_COL_MAJOR).startswith("gemm_stream")
    assert kern(64, 4096, 4096, layout_b=GEMM_COL_MAJOR, batch=3, stride_a=64 * 4096,
                stride_b=4096 * 4096, stride_c=64 * 4096).startswith("gemm_stream64x16")
    assert kern(40, 4096, 16384, layout_b=GEMM_COL_MAJOR).startswith("gemm_stream64x16")
    # wide N: 48 or 64 columns per streaming workgroup (M <= 32); past one pass
    # of 32 x 64 tiles, more rows go to the 128 tile
    assert kern(32, 11008, 4096, layout_b=GEMM_COL_MAJOR) == "gemm_stream32x48_nt_direct"
    assert kern(32, 8192, 4096, layout_b=GEMM_COL_MAJOR) == "gemm_stream32x64_nt_direct_sk4"
    assert kern(32, 4096, 4096, layout_b=GEMM_COL_MAJOR).startswith("gemm_stream32x16")
    assert kern(64, 11008, 4096, layout_b=GEMM_COL_MAJOR).endswith("d4_nt_direct_sk2")
    # skinny with row-major B: too few tiles for the CUs, so the 128 tile with
    # its K cut into slices (split-K, suffix _sk<slices>)
    assert kern(16, 4096, 4096) == "gemm_128x128x64m16d4_nn_direct_sk8"
    assert kern(128, 11008, 4096, layout_b=GEMM_COL_MAJOR).endswith("d4_nt_direct_sk2")
    # 2048^2 already fills the CUs with 128 tiles; short K is not cut
    assert not kern(2048, 2048, 2048).endswith(tuple(f"_sk{k}" for k in range(2, 9)))
    assert "_sk" not in kern(16, 4096, 512)
    # batched small products are not put on tiles far larger than themselves:
    # at most 64 x 64 x 64 with row-major A and B, one wave per product
    assert mpg.Plan(64, 64, 64, batch=512, stride_a=4096, stride_b=4096,
                    stride_c=4096).kernel == "gemm_small64_nn_direct"
    assert mpg.Plan(50, 40, 32, batch=3, stride_a=50 * 32, stride_b=32 * 40,
                    stride_c=2000).kernel == "gemm_small64_nn_direct"
    assert mpg.Plan(50, 40, 33, batch=3, stride_a=50 * 33, stride_b=33 * 40,
                    stride_c=2000).kernel == "gemm_64x64x64_nn_narrow"    # no copies
    assert mpg.Plan(64, 64, 64).kernel.startswith("gemm_64x64")              # one product
    assert mpg.Plan(65, 64, 64, batch=4, stride_a=65 * 64, stride_b=4096,
                    stride_c=65 * 64).kernel.startswith("gemm_64x64")        # 65 rows
    assert not mpg.Plan(64, 64, 64, layout_b=GEMM_COL_MAJOR, batch=4, stride_a=4096,
                        stride_b=4096, stride_c=4096).kernel.startswith("gemm_small")   # NT
    assert kern(1024, 1024, 1024).startswith("gemm_128x128")
    # the 128 tile on a four-slot ring when its grid is one wave at one
    # workgroup per CU, with four or more stages
    assert kern(2048, 2048, 2048).startswith("gemm_128x128x64m16d4")
    assert kern(2048, 4096, 4096, layout_b=GEMM_COL_MAJOR).startswith("gemm_128x128x64m16_")
    assert kern(3072, 3072, 3072).startswith("gemm_128x128x64m16_")
    # shallow K goes to the 128 tile (epilogue-bound), and so do half-empty
    # 128 tiles of streaming-bound batched products
    assert kern(8192, 8192, 256).startswith("gemm_128x128x64m16_")
    assert kern(8192, 8192, 512).startswith("gemm_256x256")
    assert mpg.Plan(1024, 64, 1024, batch=128, stride_a=1024 * 1024, stride_b=1024 * 64,
                    stride_c=1024 * 64).kernel.startswith("gemm_128x128")
    assert kern(1024, 1024, 128).startswith("gemm_128x128x64m16_")
    assert "narrow" in kern(127, 257, 33)
    assert kern(0, 8, 8) == "none"


def test_repacking_choice():
    """Rows that are not multiples of 8 elements: shapes for the direct or
    streaming kernels repack the offending operands (suffix _pka/_pkb/_pkab);
    small products use the staged kernel's element-wide loads instead."""
    def kern(*a, **k):
        with mpg.Plan(*a, **k) as p:
            return p.kernel
    assert kern(4095, 4095, 4095) == "gemm_256x256x64m16_nn_direct_pkab"
    # K odd: only K-contiguous operands are affected
    assert kern(1000, 1000, 999).endswith("nn_direct_pka")
    assert kern(1000, 1000, 999, layout_b=GEMM_COL_MAJOR).endswith("nt_direct_pkab")
    assert kern(1000, 1000, 999, layout_a=GEMM_COL_MAJOR).endswith("tn_direct")
    # odd leading dimension with aligned extents
    assert kern(1024, 1024, 1024, lda=1025).endswith("nn_direct_pka")
    assert kern(1024, 1024, 1024, ldb=1028).endswith("nn_direct_pkb")
    # deep K with few tiles: repacked and split
    assert kern(50, 333, 4100) == "gemm_128x128x64m16d4_nn_direct_sk8_pkab"
    # skinny NT: streaming kernel on repacked operands
    assert kern(7, 4097, 4099, layout_b=GEMM_COL_MAJOR) == "gemm_stream16x16_nt_direct_pkab"
    # small or batched-small: no copies
    assert kern(127, 257, 33) == "gemm_64x64x64_nn_narrow"
    assert kern(33, 33, 33, batch=1000, stride_a=33 * 33, stride_b=33 * 33,
                stride_c=33 * 33).endswith("narrow")
    # K = 0 reads no operand
    assert "_pk" not in kern(1000, 1000, 0, lda=1)


def test_workspace_size_rules():
    """Workspace: none for plain plans; 4096 counter bytes plus 64 KiB per
    (slice, tile) for split-K; the shape-driven copies; and, on request,
    room to repack misaligned pointers (direct and streaming kernels only)."""
    from mixed_precision_gemm_amd import GEMM_WS_ANY_ALIGNMENT as ANY
    with mpg.Plan(8192, 8192, 8192) as p:
        assert p.workspace_bytes() == 0
        assert p.workspace_bytes(ANY) == 4096 + 2 * 2 * 8192 * 8192
    with mpg.Plan(16, 4096, 4096) as p:          # 32 tiles x 8 slices
        assert p.kernel.endswith("_sk8")
        assert p.workspace_bytes() == 4096 + 8 * 32 * 128 * 128 * 4
        assert p.workspace_bytes(ANY) == 4096 + 8 * 32 * 65536 + 2 * (16 * 4096 + 4096 * 4096)
    with mpg.Plan(1000, 1000, 999) as p:         # A repacked: 1000 rows of 1000
        assert p.kernel.endswith("_pka")
        assert p.workspace_bytes() == 4096 + (1000 * 1000 * 2 + 255) // 256 * 256
    with mpg.Plan(127, 257, 33) as p:            # staged tile: reads in place
        assert p.workspace_bytes() == 0 and p.workspace_bytes(ANY) == 0
    with mpg.Plan(0, 64, 64) as p:
        assert p.workspace_bytes(ANY) == 0
    with mpg.Plan(64, 64, 64) as p:
        assert mpg.gemm_f16f32_workspace_size(p.handle, 2)[0] == GEMM_ERR_INVALID_ARG
        lib = mpg.library()
        assert lib.gemm_f16f32_workspace_size(p.handle, 0, None) == GEMM_ERR_INVALID_ARG
    assert mpg.gemm_f16f32_workspace_size(None, 0)[0] == GEMM_ERR_INVALID_ARG


def test_run_and_init_reject_bad_workspaces_before_launch():
    base = 1 << 30
    A, B, C = base, base + (1 << 26), base + (2 << 26)
    with mpg.Plan(16, 4096, 4096) as p:          # split-K: needs a workspace
        need = p.workspace_bytes()
        ws = base + (3 << 26)
        run = lambda w, n: mpg.gemm_f16f32_run(p.handle, A, B, C, 1.0, 0.0, w, n, None)
        assert run(None, 0) == GEMM_ERR_INVALID_ARG
        assert run(ws, need - 1) == GEMM_ERR_INVALID_ARG
        assert run(ws + 16, need) == GEMM_ERR_INVALID_ARG      # not 256-byte aligned
        assert run(None, need) == GEMM_ERR_INVALID_ARG
        assert run(ws, -1) == GEMM_ERR_INVALID_ARG
        assert run(C - 256, need) == GEMM_ERR_INVALID_ARG      # overlaps C
    assert mpg.gemm_f16f32_workspace_init(None, 4096) == GEMM_ERR_INVALID_ARG
    assert mpg.gemm_f16f32_workspace_init(base + 8, 4096) == GEMM_ERR_INVALID_ARG
    assert mpg.gemm_f16f32_workspace_init(base, -1) == GEMM_ERR_INVALID_ARG
    assert mpg.gemm_f16f32_workspace_init(None, 0) == GEMM_OK   # nothing to clear


def test_noalloc_refuses_plans_beyond_its_scratch_before_any_hip_call():
    """gemm_f16f32_run_noalloc holds 64 MiB of static scratch per device: a
    plan needing more is refused with GEMM_ERR_SCRATCH, checked on the host
    before the device is touched (so this runs without a GPU)."""
    from mixed_precision_gemm_amd import GEMM_ERR_SCRATCH
    base = 1 << 30
    with mpg.Plan(4201, 4201, 4201) as p:            # both operands repacked: 2 x 35 MB
        assert p.kernel.endswith("_pkab")
        assert p.workspace_bytes() > 64 << 20
        assert mpg.gemm_f16f32_run_noalloc(p.handle, base, base + (1 << 26),
                                           base + (2 << 26), 1.0, 0.0) == GEMM_ERR_SCRATCH
    assert mpg.gemm_f16f32_run_noalloc(None, base, base, base, 1.0, 0.0) == GEMM_ERR_INVALID_ARG
    with mpg.Plan(0, 64, 64) as p:
        assert mpg.gemm_f16f32_run_noalloc(p.handle, 0, 0, 0, 1.0, 0.0) == GEMM_OK


def test_run_rejects_null_operands_even_when_k_is_zero():
    """A and B must be non-NULL whenever M * N > 0 (K = 0 reads neither)."""
    base = 1 << 30
    with mpg.Plan(1024, 1024, 0, lda=1) as p:
        assert mpg.gemm_f16f32_run(p.handle, 0, base, base + (1 << 26), 1.0, 1.0) == GEMM_ERR_INVALID_ARG
        assert mpg.gemm_f16f32_run(p.handle, base, 0, base + (1 << 26), 1.0, 1.0) == GEMM_ERR_INVALID_ARG


def test_run_rejects_bad_arguments_before_launch():
    with mpg.Plan(64, 64, 64) as p:
        h = p.handle
        assert mpg.gemm_f16f32_run(None, 16, 16, 16, 1.0, 0.0, None) == GEMM_ERR_INVALID_ARG
        assert mpg.gemm_f16f32_run(h, 0, 1 << 20, 1 << 24, 1.0, 0.0, None) == GEMM_ERR_INVALID_ARG
        assert mpg.gemm_f16f32_run(h, 1 << 20, 0, 1 << 24, 1.0, 0.0, None) == GEMM_ERR_INVALID_ARG
        assert mpg.gemm_f16f32_run(h, 1 << 20, 1 << 21, 0, 1.0, 0.0, None) == GEMM_ERR_INVALID_ARG
        # C overlapping A or B (addresses only; nothing is launched)
        base = 1 << 30
        assert mpg.gemm_f16f32_run(h, base, base + (1 << 20), base + 100, 1.0, 0.0, None) == GEMM_ERR_INVALID_ARG
        assert mpg.gemm_f16f32_run(h, base + (1 << 20), base, base + 100, 1.0, 0.0, None) == GEMM_ERR_INVALID_ARG
    # an empty product is a no-op even with NULL pointers
    with mpg.Plan(0, 64, 64) as p:
        assert mpg.gemm_f16f32_run(p.handle, 0, 0, 0, 1.0, 0.0, None) == GEMM_OK


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(mpg, "_lib", None)
    monkeypatch.setattr(mpg, "LIB_PATH", str(tmp_path / "absent.so"))
    with pytest.raises(ImportError):
        mpg.library()


# ------------------------------------------------------------- bfloat16

def test_bf16_plan_out_types():
    from mixed_precision_gemm_amd import GEMM_OUT_BF16

    def st(fn, out):
        s, h = fn(64, 64, 64, GEMM_ROW_MAJOR, GEMM_ROW_MAJOR, out, 64, 64, 64)
        if h is not None:
            mpg.gemm_f16f32_destroy(h)
        return s
    assert st(mpg.gemm_bf16f32_plan, GEMM_OUT_BF16) == GEMM_OK
    assert st(mpg.gemm_bf16f32_plan, GEMM_OUT_F32) == GEMM_OK
    assert st(mpg.gemm_bf16f32_plan, GEMM_OUT_F16) == GEMM_ERR_INVALID_ARG
    assert st(mpg.gemm_f16f32_plan, GEMM_OUT_BF16) == GEMM_ERR_INVALID_ARG
    assert st(mpg.gemm_bf16f32_plan, 3) == GEMM_ERR_INVALID_ARG
    # the other rules are the fp16 family's
    s, h = mpg.gemm_bf16f32_plan(64, 64, 64, 0, 0, GEMM_OUT_BF16, 63, 64, 64)
    assert s == GEMM_ERR_INVALID_ARG and h is None


def test_run_rejects_plan_of_the_other_input_type():
    """Checked before any HIP call: no launch happens."""
    base = 1 << 30
    with mpg.Plan(64, 64, 64) as p16, mpg.Plan(64, 64, 64, dtype="bf16") as pbf:
        assert mpg.gemm_bf16f32_run(p16.handle, base, base + (1 << 20), base + (2 << 20),
                                    1.0, 0.0, None) == GEMM_ERR_INVALID_ARG
        assert mpg.gemm_f16f32_run(pbf.handle, base, base + (1 << 20), base + (2 << 20),
                                   1.0, 0.0, None) == GEMM_ERR_INVALID_ARG
    assert mpg.gemm_bf16f32_run(None, 0, 0, 0, 1.0, 0.0, None) == GEMM_ERR_INVALID_ARG


@pytest.mark.parametrize("shape,kw", [
    ((8192, 8192, 8192), {}), ((8192, 8192, 8192), dict(layout_b=GEMM_COL_MAJOR)),
    ((16, 4096, 4096), dict(layout_b=GEMM_COL_MAJOR)), ((32, 11008, 4096), dict(layout_b=GEMM_COL_MAJOR)),
    ((64, 11008, 4096), dict(layout_b=GEMM_COL_MAJOR)), ((16, 4096, 4096), {}),
    ((2048, 2048, 2048), {}), ((3072, 3072, 3072), {}), ((4095, 4095, 4095), {}),
    ((127, 257, 33), {}), ((50, 333, 4100), {}), ((0, 8, 8), {}),
    ((64, 64, 64), dict(batch=512, stride_a=4096, stride_b=4096, stride_c=4096)),
])
def test_bf16_kernel_choice_matches_fp16(shape, kw):
    with mpg.Plan(*shape, **kw) as a, mpg.Plan(*shape, dtype="bf16", **kw) as b:
        if a.kernel == "none":
            assert b.kernel == "none"
        else:
            assert b.kernel == a.kernel.replace("gemm_", "gemm_bf16_", 1)
    assert mpg.Plan(128, 128, 128, dtype="bf16").kernel.startswith("gemm_bf16_")
    with pytest.raises(ValueError):
        mpg.Plan(8, 8, 8, dtype="fp8")


# ------------------------------------------------------------ fused epilogue

def test_set_epilogue_validation():
    from mixed_precision_gemm_amd import GEMM_ACT_GELU, GEMM_ACT_NONE, GEMM_ACT_SILU
    assert mpg.gemm_f16f32_set_epilogue(None, None, GEMM_ACT_NONE) == GEMM_ERR_INVALID_ARG
    with mpg.Plan(64, 64, 64) as p, mpg.Plan(64, 64, 64, dtype="bf16") as q:
        for plan in (p, q):
            assert mpg.gemm_f16f32_set_epilogue(plan.handle, None, GEMM_ACT_SILU) == GEMM_OK
            assert mpg.gemm_f16f32_set_epilogue(plan.handle, 1 << 30, GEMM_ACT_GELU) == GEMM_OK
            assert mpg.gemm_f16f32_set_epilogue(plan.handle, (1 << 30) + 2, 0) == GEMM_ERR_INVALID_ARG
            assert mpg.gemm_f16f32_set_epilogue(plan.handle, None, 4) == GEMM_ERR_INVALID_ARG
            assert mpg.gemm_f16f32_set_epilogue(plan.handle, None, -1) == GEMM_ERR_INVALID_ARG
            assert mpg.gemm_f16f32_set_epilogue(plan.handle, None, GEMM_ACT_NONE) == GEMM_OK
        with pytest.raises(mpg.GemmError):
            p.set_epilogue(None, 9)


def test_run_rejects_bias_overlapping_c_before_launch():
    """The bias range [bias, bias + 4N) may not overlap C; checked before
    any HIP call."""
    base = 1 << 30
    with mpg.Plan(64, 64, 64) as p:
        C = base + (1 << 24)
        assert mpg.gemm_f16f32_set_epilogue(p.handle, C + 64, 1) == GEMM_OK
        assert mpg.gemm_f16f32_run(p.handle, base, base + (1 << 20), C, 1.0, 0.0,
                                   None) == GEMM_ERR_INVALID_ARG


# ------------------------------------------------------------ attention

def attn_plan(B=2, H=3, Sq=100, Sk=130, D=64, qs=None, ks=None, vs=None, os_=None,
              causal=0, out=GEMM_OUT_F16):
    dense = lambda S: (H * S * D, S * D, D)
    st, h = mpg.attn_f16_plan(B, H, Sq, Sk, D, qs or dense(Sq), ks or dense(Sk),
                              vs or dense(Sk), os_ or dense(Sq), causal, out)
    name = mpg.attn_f16_plan_kernel(h) if h else None
    if h:
        mpg.attn_f16_destroy(h)
    return st, name


def test_attention_plan_rules():
    assert attn_plan() == (GEMM_OK, "attn_fwd_d64_q128_k64_f16")
    assert attn_plan(D=128, causal=1, out=GEMM_OUT_F32) == (GEMM_OK, "attn_fwd_d128_q128_k64_causal_f32")
    assert attn_plan(Sq=0) == (GEMM_OK, "none")
    assert attn_plan(Sk=0)[0] == GEMM_OK                 # every row fully masked: zeros
    for kw in [dict(B=0), dict(H=0), dict(Sq=-1), dict(Sk=-1), dict(causal=2), dict(out=2),
               dict(qs=(0, 0, 63)), dict(ks=(-8, 0, 64))]:
        assert attn_plan(**kw)[0] == GEMM_ERR_INVALID_ARG, kw
    for kw in [dict(D=96), dict(D=32), dict(qs=(100 * 64 * 3, 100 * 64, 68)),
               dict(os_=(1, 1, 64)), dict(Sk=1 << 25, ks=(0, 0, 64), vs=(0, 0, 64))]:
        assert attn_plan(**kw)[0] == GEMM_ERR_UNSUPPORTED, kw
    assert mpg.attn_f16_plan_kernel(None) == "invalid"
    assert mpg.attn_f16_destroy(None) == GEMM_OK


def test_attention_run_and_softmax_reject_bad_arguments_before_launch():
    base = 1 << 30
    st, h = mpg.attn_f16_plan(1, 1, 64, 64, 64, (0, 0, 64), (0, 0, 64), (0, 0, 64), (0, 0, 64), 0, 0)
    assert st == GEMM_OK
    try:
        Q, K, V, O = base, base + (1 << 20), base + (2 << 20), base + (3 << 20)
        assert mpg.attn_f16_run(None, Q, K, V, O, 0.125) == GEMM_ERR_INVALID_ARG
        assert mpg.attn_f16_run(h, 0, K, V, O, 0.125) == GEMM_ERR_INVALID_ARG
        assert mpg.attn_f16_run(h, Q + 8, K, V, O, 0.125) == GEMM_ERR_INVALID_ARG   # misaligned
        assert mpg.attn_f16_run(h, Q, K, V, Q + 64, 0.125) == GEMM_ERR_INVALID_ARG  # O overlaps Q
    finally:
        mpg.attn_f16_destroy(h)
    sm = mpg.attn_softmax_rows
    assert sm(-1, 8, base, 8, 0, base + 4096, 8, 0) == GEMM_ERR_INVALID_ARG
    assert sm(4, 8, base, 7, 0, base + 4096, 8, 0) == GEMM_ERR_INVALID_ARG       # ldx < cols
    assert sm(4, 8, base, 8, 3, base + 4096, 8, 0) == GEMM_ERR_INVALID_ARG       # type
    assert sm(4, 8, base, 8, 0, base + 8, 8, 0) == GEMM_ERR_INVALID_ARG          # partial overlap
    assert sm(0, 8, 0, 8, 0, 0, 8, 0) == GEMM_OK                                 # empty: no-op


# ------------------------------------------------------------ residual + LayerNorm

def test_set_layernorm_validation_and_workspace():
    from mixed_precision_gemm_amd import GEMM_ACT_GELU, GEMM_ACT_NONE
    base = 1 << 30
    assert mpg.gemm_f16f32_set_layernorm(None, base, base + 4096, 1e-5) == GEMM_ERR_INVALID_ARG
    with mpg.Plan(2048, 4096, 4096, layout_b=GEMM_COL_MAJOR) as p:
        h = p.handle
        plain = p.workspace_bytes()
        assert plain == 0
        assert mpg.gemm_f16f32_set_layernorm(h, base + 2, base + 4096, 1e-5) == GEMM_ERR_INVALID_ARG
        assert mpg.gemm_f16f32_set_layernorm(h, base, None, 1e-5) == GEMM_ERR_INVALID_ARG
        assert mpg.gemm_f16f32_set_layernorm(h, base, base + 4096, -1.0) == GEMM_ERR_INVALID_ARG
        assert mpg.gemm_f16f32_set_layernorm(h, base, base + 4096, float("nan")) == GEMM_ERR_INVALID_ARG
        assert mpg.gemm_f16f32_set_epilogue(h, None, GEMM_ACT_GELU) == GEMM_OK
        assert mpg.gemm_f16f32_set_layernorm(h, base, base + 4096, 1e-5) == GEMM_ERR_INVALID_ARG
        assert mpg.gemm_f16f32_set_epilogue(h, base + 8192, GEMM_ACT_NONE) == GEMM_OK
        assert mpg.gemm_f16f32_set_layernorm(h, base, base + 4096, 1e-5) == GEMM_OK
        assert mpg.gemm_f16f32_set_epilogue(h, base + 8192, GEMM_ACT_GELU) == GEMM_ERR_INVALID_ARG
        # Z in fp32 after the reserved counter area
        assert p.workspace_bytes() == 4096 + 2048 * 4096 * 4
        assert mpg.gemm_f16f32_set_layernorm(h, None, None, 0.0) == GEMM_OK
        assert p.workspace_bytes() == plain
    with mpg.Plan(16, 4095, 4096) as p:          # split-K and a repacked B, plus Z
        assert mpg.gemm_f16f32_set_layernorm(p.handle, base, base + 4096 * 4, 0.0) == GEMM_OK
        gemm_part = 4096 + 8 * 32 * 65536 + (4096 * 4096 * 2)
        z = (16 * 4096 * 4 + 255) // 256 * 256
        assert "_sk8" in p.kernel and p.kernel.endswith("_pkb")
        assert p.workspace_bytes() == (gemm_part + 255) // 256 * 256 + z


# ------------------------------------------------------------ convolution

def test_conv_plan_rules():
    def plan(N=2, H=16, W=16, C=64, K=32, R=3, S=3, stride=(1, 1), pad=(1, 1), dil=(1, 1), out=0):
        st, h = mpg.conv_f16_plan(N, H, W, C, K, R, S, stride, pad, dil, out)
        res = (st, mpg.conv_f16_plan_kernel(h) if h else None,
               mpg.conv_f16_output_size(h)[1:] if h else None)
        if h:
            mpg.conv_f16_destroy(h)
        return res
    assert plan() == (GEMM_OK, "conv_implicit_64x64x64_vec16", (16, 16))
    # the tile's width follows the output channels; the 64 tile below 128 workgroups
    assert plan(N=32, H=56, W=56, C=64, K=64) == (GEMM_OK, "conv_implicit_256x64x64_vec16", (56, 56))
    assert plan(N=32, H=56, W=56, C=64, K=65)[1] == "conv_implicit_128x128x64_vec16"
    assert plan(N=32, H=224, W=224, C=3, K=64, R=7, S=7, stride=(2, 2),
                pad=(3, 3))[1] == "conv_implicit_128x64x64_narrow"
    assert plan(N=16, H=32, W=32, C=16, K=64)[1] == "conv_implicit_64x64x64_vec16"    # 64 tiles
    assert plan(N=32, H=32, W=32, C=16, K=64)[1] == "conv_implicit_256x64x64_vec16"   # 128 tiles
    assert plan(C=3, stride=(2, 2)) == (GEMM_OK, "conv_implicit_64x64x64_narrow", (8, 8))
    assert plan(H=224, W=224, C=3, K=64, R=7, S=7, stride=(2, 2), pad=(3, 3))[2] == (112, 112)
    assert plan(R=5, S=5, pad=(0, 0), dil=(4, 4))[0] == GEMM_ERR_INVALID_ARG     # window too large
    assert plan(N=0)[1] == "none" and plan(K=0)[1] == "none"
    for kw in [dict(H=0), dict(C=0), dict(R=0), dict(stride=(0, 1)), dict(pad=(-1, 0)),
               dict(dil=(1, 0)), dict(out=2), dict(N=-1)]:
        assert plan(**kw)[0] == GEMM_ERR_INVALID_ARG, kw
    assert plan(N=1 << 14, H=256, W=256, C=64)[0] == GEMM_ERR_UNSUPPORTED   # input past 2^31 bytes
    assert mpg.conv_f16_plan_kernel(None) == "invalid"
    assert mpg.conv_f16_destroy(None) == GEMM_OK
    st, h = mpg.conv_f16_plan(1, 8, 8, 8, 8, 3, 3, (1, 1), (1, 1), (1, 1), 0)
    try:
        base = 1 << 30
        run = lambda *a: mpg.conv_f16_run(h, *a)
        assert run(0, base + 4096, base + 8192) == GEMM_ERR_INVALID_ARG
        assert run(base, base + 4096, base + 100) == GEMM_ERR_INVALID_ARG   # y overlaps x
        assert run(base, base + 4096, base + 8192, 1.0, 0.0, base + 2) == GEMM_ERR_INVALID_ARG
        assert run(base, base + 4096, base + 8192, 1.0, 0.0, None, 7) == GEMM_ERR_INVALID_ARG
        assert mpg.conv_f16_run(None, base, base, base) == GEMM_ERR_INVALID_ARG
    finally:
        mpg.conv_f16_destroy(h)
