"""The no-allocation entry point, gemm_f16f32_run_noalloc, against the
ordinary run with a caller workspace.

Both launch the same kernels with the same summation order, so their outputs
must agree bit for bit; each is also checked against the oracle under the
acceptance bound.  The calls come in a row on one stream, the later ones
smaller than the first, so the library's static scratch is reused with the
previous call's contents still in it (split-K counters must be zero again,
stale partial tiles and copies must not leak into the next result).
"""
import numpy as np
import pytest
import torch

import gemm_inputs as gi
import mixed_precision_gemm_amd as mpg
from gemm_inputs import COL_MAJOR, OUT_F16, OUT_F32, ROW_MAJOR
from parity import c_logical, check_bound, in_dtype, oracle_for, to_device

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def _plan(case):
    return mpg.Plan(case.M, case.N, case.K, case.layout_a, case.layout_b, case.out_type,
                    case.lda, case.ldb, case.ldc, case.batch, case.stride_a, case.stride_b,
                    case.stride_c, dtype=in_dtype(case))


def _both(case, offsets=(0, 0)):
    """(C from run with a zeroed torch workspace, C from run_noalloc), with A
    and B placed `offsets` elements past 16-byte-aligned addresses."""
    dA, dB, dC = to_device(case)
    oa, ob = offsets
    if oa or ob:
        A = torch.zeros(dA.numel() + oa, dtype=dA.dtype, device="cuda")
        B = torch.zeros(dB.numel() + ob, dtype=dB.dtype, device="cuda")
        A[oa:] = dA
        B[ob:] = dB
        dA, dB = A[oa:], B[ob:]
    c_ref, c_new = dC.clone(), dC.clone()
    stream = torch.cuda.current_stream().cuda_stream
    with _plan(case) as p:
        p.run(dA, dB, c_ref, case.alpha, case.beta)
        st = mpg.gemm_f16f32_run_noalloc(p.handle, dA.data_ptr(), dB.data_ptr(), c_new.data_ptr(),
                                         case.alpha, case.beta, stream)
        assert st == mpg.GEMM_OK, mpg.gemm_f16f32_status_string(st)
        kernel = p.kernel
    torch.cuda.synchronize()
    return c_ref, c_new, kernel


def _check(case, what, offsets=(0, 0)):
    c_ref, c_new, kernel = _both(case, offsets)
    assert torch.equal(c_ref, c_new), f"{what} ({kernel}): run_noalloc differs from run"
    ref, scale = oracle_for(case)
    check_bound(c_logical(case, c_new.cpu()), ref, scale, case.out_type, f"{what} {kernel}")
    return kernel


def test_noalloc_matches_run_on_calls_in_a_row():
    """Split-K plans (counters and 16, then 4 MiB of partial tiles in the
    scratch), a repacked one, a bfloat16 one and a plain one, in a row,
    each smaller than the first."""
    k1 = _check(gi.make_case(128, 4096, 4096, beta=1.0, seed=201), "split-K 8")
    assert "_sk8" in k1, k1
    k2 = _check(gi.make_case(64, 2048, 2048, beta=0.5, alpha=-1.25, seed=202), "split-K 4")
    assert "_sk4" in k2, k2
    k3 = _check(gi.make_case(1000, 1000, 999, seed=203), "repacked A")
    assert k3.endswith("_pka"), k3
    k4 = _check(gi.make_case(96, 1024, 2048, out_type=OUT_F32, in_dtype="bf16", seed=204),
                "bf16 split-K")
    assert "_sk" in k4, k4
    _check(gi.make_case(256, 256, 256, seed=205), "plain 256^3")


def test_noalloc_misaligned_operands_repack_into_scratch():
    """A and B at odd addresses: the direct kernel's plan repacks both into
    the scratch, as run does into a workspace sized for any alignment."""
    case = gi.make_case(512, 384, 640, layout_a=COL_MAJOR, beta=1.0, seed=206)
    _check(case, "misaligned A and B", offsets=(3, 5))


def test_noalloc_rejects_plans_beyond_the_scratch():
    """A plan whose workspace would exceed the 64 MiB scratch is refused with
    GEMM_ERR_SCRATCH before anything is launched; the next call still works."""
    with mpg.Plan(4201, 4201, 4201) as p:
        assert p.workspace_bytes() > 64 << 20
        base = 1 << 30
        st = mpg.gemm_f16f32_run_noalloc(p.handle, base, base + (1 << 26), base + (2 << 26),
                                         1.0, 0.0, None)
        assert st == mpg.GEMM_ERR_SCRATCH
    _check(gi.make_case(16, 4096, 4096, seed=207), "after a refused call")
