// Host-side planner of the fp16 (or bf16) -> fp32-accumulate GEMM: argument validation,
// tile, K-split and repacking choice, grid shape and workspace size.  Nothing
// here makes a HIP call, so it runs (and is tested) on machines without a
// GPU; a plan is host memory only.
//
// Pages cited (titles as printed):
//   [GEMM]    "手写GEMM内核：矩阵乘法性能优化的完整工程实践" (hand-written GEMM kernel)
//   [OPS]     CUDA operator practice page (Softmax and GEMM)
//   [CATLASS] CATLASS template library page
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <math.h>

#include <algorithm>
#include <new>

#include "gemm_bf16f32.h"
#include "gemm_f16f32.h"
#include "gemm_internal.h"

using namespace mpgemm;

namespace {

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Elements spanned by one operand over the whole batch (0 when empty).
int64_t operand_extent(int64_t rows, int64_t cols, int64_t ld, int64_t batch,
                       int64_t stride) {
    if (rows == 0 || cols == 0) return 0;
    return (batch - 1) * stride + (rows - 1) * ld + cols;
}

// Tile choice.  [GEMM] §1.3 rules out autotuning and run-time selection among
// many kernels; the choice here is a fixed rule on the shape.  [OPS] §4.3
// asks that the grid fill the device.  A tile is taken only if the padding it
// adds wastes little work (fill = useful outputs / computed outputs) and it
// yields enough workgroups: the 256 x 256 tile needs a full wave of 256 CUs,
// the 128 x 128 tile (two workgroups per CU) a quarter of one; otherwise the
// small staged tiles, the 32-row one for skinny M (token counts of a linear
// layer).
int choose_tile(int64_t M, int64_t N, int64_t K, int64_t batch, bool kc_both, bool nn,
                bool vec_ok) {
    // At most 4 rows with row-major A and B (a matrix-vector product in the
    // NN layout): B streamed into registers, fp32 dot products.
    if (nn && M <= 4 && K > 0) return TILE_ROWVEC;
    // Batches of products of at most 64 x 64 x 64 with row-major A and B:
    // one wave per product, its loads all in flight at once (512 x 64^3:
    // see the kernel).
    if (nn && vec_ok && batch > 1 && M <= 64 && N <= 64 && K <= 64 && K > 0) return TILE_SMALL64;
    // Skinny M with K-contiguous A and B streams B through LDS.  Every
    // workgroup re-reads its rows of A, so wide N takes more columns per
    // workgroup: 48 for M <= 16 from N = 8192 and for M <= 32 from N = 10240
    // (171 or more workgroups, about one per CU, none split), 64 for
    // 16 < M <= 32 at N = 8192 .. 10239 (128 to 159 workgroups, split-K
    // below).  48 columns against 64: 16 x 11008 19.3 against 20.7 us,
    // 16 x 12288 20.8 against 21.8, 32 x 11008 23.4 against 27.0; at
    // N = 8192, 16 rows 16.7 (unsplit) against 16.9 (four slices), 32 rows
    // 21.6 against 20.6.  (Measured on the K = 4096 linear shapes.)
    if (kc_both && M <= 16) return N >= 8192 ? TILE_STREAM16W : TILE_STREAM16;
    if (kc_both && M <= 32)
        return N >= 10240 ? TILE_STREAM32N : N >= 8192 ? TILE_STREAM32W : TILE_STREAM32;
    // Up to 128 rows, the 32 x 64 streaming tile while its grid fits one
    // workgroup per CU and K is 1024 to 8192: more workgroups stream B than
    // the 128 tile's split-K grid, without its partial tiles.  (Measured at
    // K = 4096: 64 x 4096 18.2 against 22.0 us, 128 x 4096 21.8 against
    // 29.0, 96 x 2048 17.2 against 21.0; beyond one pass, 128 x 6144 36.2
    // against 27.2; at K = 16384, 128 x 2048 41.6 against 38.5.)
    if (kc_both && M <= 128 && K >= 1024 && K <= 8192 &&
        ceil_div(M, 32) * ceil_div(N, 64) * batch <= kNumCUs)
        return TILE_STREAM32W;
    if (kc_both && M <= 64 && ceil_div(N, 128) < 64) return TILE_STREAM64;
    auto count = [&](int t) {
        return ceil_div(M, kTiles[t].bm) * ceil_div(N, kTiles[t].bn) * batch;
    };
    auto fill = [&](int t) {
        const double pm = (double)ceil_div(M, kTiles[t].bm) * kTiles[t].bm;
        const double pn = (double)ceil_div(N, kTiles[t].bn) * kTiles[t].bn;
        return (double)M * (double)N / (pm * pn);
    };
    // Shallow K (at most four stages) is bound by the epilogue's C traffic:
    // the 128 tile, two workgroups per CU, overlaps one's epilogue with the
    // other's loads, where the 256 tile (one per CU) cannot.  The 128 tile
    // also takes half-empty tiles (N or M = 64): such products are bound by
    // streaming the other operand, not by MFMA.  (Measured: 8192^2 x 128
    // fp32 C 87 -> 70 us, 128 x (1024 x 64 x 1024) 144 -> 66 us.)
    if (K > 256 && count(TILE_256x256) >= kNumCUs && fill(TILE_256x256) >= 0.8) return TILE_256x256;
    if (count(TILE_128x128) >= kNumCUs / 4 && fill(TILE_128x128) >= 0.5) return TILE_128x128;
    // Too few tiles to fill the CUs but enough K to cut: the 128 tile with
    // split-K (choose_ksplit) puts up to one workgroup on every CU.
    if (vec_ok && batch == 1 && K >= 1024 && count(TILE_128x128) < kNumCUs) return TILE_128x128;
    if (M <= 32) return TILE_32x64;
    return TILE_64x64;
}

// K slices for the direct 128 tile: as many as keep the grid within one
// workgroup per CU (at least two), each slice at least 512 deep and a
// multiple of the 64-deep stage, at most 8 slices.  Tiles that already fill
// a quarter of the CUs are cut only when K is deep: the partial tiles and
// their reduction cost more than they gain at K ~ 1024 (measured at 1024^3).
//
// K slices for the 48- and 64-column streaming tiles.  With 160 or more
// workgroups a tile is not split: its waves keep their batches streaming
// back to back, and a split only adds the partial sums' round trips at the
// end (16 x 11008 x 4096 on 64 columns: 20.9 us unsplit, 22.0 in four
// slices, 24.7 in two; 16 x 16384: 28.2 against 34.9).  Fewer workgroups
// (the 64-column tiles from N = 8192, and the many-row tiles of up to 128
// rows) are cut into up to four slices of at least 1024 (16 x 8192 x 4096
// on 64 columns: 16.7 us against 19.9 unsplit, 18.9 in two, 21.5 in eight;
// 32 x 8192: 20.6 against 25.3 on the 16-column tile).  The last slice of a
// block to finish sums the partial blocks in slice order.
void choose_ksplit_stream(gemm_f16f32_plan_s *p, int64_t tiles) {
    if (p->tile == TILE_ROWVEC) {
        // Row vectors: enough K slices of at least 1024 for about 256
        // workgroups, at most 8.
        int64_t ks = std::min<int64_t>(8, std::min<int64_t>(ceil_div(kNumCUs, tiles), p->K / 1024));
        if (ks < 2 || tiles > kMaxCounters) return;
        const int64_t chunk = ceil_div(ceil_div(p->K, ks), 64) * 64;
        const int64_t n = ceil_div(p->K, chunk);
        if (n < 2) return;
        p->kchunk = chunk;
        p->ksplit = (int)n;
        p->split_bytes = n * tiles * kTiles[p->tile].bm * kTiles[p->tile].bn * 4;
        return;
    }
    if (p->tile != TILE_STREAM16W && p->tile != TILE_STREAM32W && p->tile != TILE_STREAM32N) return;
    if (tiles >= kNumCUs * 5 / 8 || tiles > kMaxCounters) return;
    int64_t ks = std::min<int64_t>(4, p->K / 1024);
    if (ks < 2) return;
    const int64_t chunk = ceil_div(ceil_div(p->K, ks), 64) * 64;
    const int64_t n = ceil_div(p->K, chunk);
    if (n < 2) return;
    p->kchunk = chunk;
    p->ksplit = (int)n;
    p->split_bytes = n * tiles * kTiles[p->tile].bm * kTiles[p->tile].bn * 4;
}

void choose_ksplit(gemm_f16f32_plan_s *p, int64_t tiles) {
    p->ksplit = 1;
    p->kchunk = p->K;
    if (kTiles[p->tile].kind == KIND_STREAM && p->vec_ok) {
        choose_ksplit_stream(p, tiles);
        return;
    }
    if (p->tile != TILE_128x128 || !p->vec_ok || p->batch != 1 || tiles >= kNumCUs) return;
    if (tiles >= kNumCUs / 4 && p->K < 2048) return;
    int64_t ks = std::max<int64_t>(2, kNumCUs / tiles);
    ks = std::min<int64_t>(ks, p->K / 512);
    ks = std::min<int64_t>(ks, 8);
    if (ks < 2 || tiles > kMaxCounters) return;
    const int64_t chunk = ceil_div(ceil_div(p->K, ks), 64) * 64;
    p->kchunk = chunk;
    p->ksplit = (int)ceil_div(p->K, chunk);
    if (p->ksplit < 2) { p->ksplit = 1; p->kchunk = p->K; return; }
    p->split_bytes = (int64_t)p->ksplit * tiles * 128 * 128 * 4;
}

// A plan for A and B of input type in_type (IN_F16 or IN_BF16).  The tile,
// split and repacking rules do not depend on the type: both run the same
// kernels, only the MFMA and the 16-bit C conversion differ.
int make_plan(int in_type, gemm_f16f32_plan_t *out, int64_t M, int64_t N, int64_t K,
              int layout_a, int layout_b, int out_type, int64_t lda, int64_t ldb,
              int64_t ldc, int64_t batch, int64_t stride_a, int64_t stride_b,
              int64_t stride_c) {
    if (!out) return GEMM_ERR_INVALID_ARG;
    *out = nullptr;
    if (M < 0 || N < 0 || K < 0) return GEMM_ERR_INVALID_ARG;
    if (layout_a != GEMM_ROW_MAJOR && layout_a != GEMM_COL_MAJOR)
        return GEMM_ERR_INVALID_ARG;
    if (layout_b != GEMM_ROW_MAJOR && layout_b != GEMM_COL_MAJOR)
        return GEMM_ERR_INVALID_ARG;
    // C is fp32 or the 16-bit type of the inputs.
    const int out16 = in_type == IN_BF16 ? GEMM_OUT_BF16 : GEMM_OUT_F16;
    if (out_type != out16 && out_type != GEMM_OUT_F32)
        return GEMM_ERR_INVALID_ARG;
    if (batch < 1) return GEMM_ERR_INVALID_ARG;
    const int64_t min_lda = layout_a == GEMM_ROW_MAJOR ? K : M;
    const int64_t min_ldb = layout_b == GEMM_ROW_MAJOR ? N : K;
    if (lda < 1 || lda < min_lda) return GEMM_ERR_INVALID_ARG;
    if (ldb < 1 || ldb < min_ldb) return GEMM_ERR_INVALID_ARG;
    if (ldc < 1 || ldc < N) return GEMM_ERR_INVALID_ARG;
    if (batch > 1) {
        if (stride_a < 0 || stride_b < 0 || stride_c < 0)
            return GEMM_ERR_INVALID_ARG;
        if (M > 0 && N > 0 && stride_c < M * ldc) return GEMM_ERR_INVALID_ARG;
    } else {
        stride_a = stride_b = stride_c = 0;
    }
    if (batch > (int64_t(1) << 24)) return GEMM_ERR_UNSUPPORTED;

    gemm_f16f32_plan_s *p = new (std::nothrow) gemm_f16f32_plan_s();
    if (!p) return GEMM_ERR_NOMEM;
    p->M = M; p->N = N; p->K = K;
    p->layout_a = layout_a; p->layout_b = layout_b; p->out_type = out_type;
    p->in_type = in_type;
    p->lda = lda; p->ldb = ldb; p->ldc = ldc;
    p->batch = batch;
    p->stride_a = stride_a; p->stride_b = stride_b; p->stride_c = stride_c;
    p->extent_a = operand_extent(layout_a == GEMM_ROW_MAJOR ? M : K,
                                 layout_a == GEMM_ROW_MAJOR ? K : M, lda, batch,
                                 stride_a);
    p->extent_b = operand_extent(layout_b == GEMM_ROW_MAJOR ? K : N,
                                 layout_b == GEMM_ROW_MAJOR ? N : K, ldb, batch,
                                 stride_b);
    p->extent_c = operand_extent(M, N, ldc, batch, stride_c);
    if (M == 0 || N == 0) {
        p->tile = -1;
        snprintf(p->kernel_name, sizeof p->kernel_name, "none");
        *out = p;
        return GEMM_OK;
    }
    // 128-bit loads need every 8-element vector along an operand's contiguous
    // dimension to be either wholly inside the matrix or zero, and every row
    // (and batch item) to start on a 16-byte boundary.
    const int64_t contig_a = layout_a == GEMM_ROW_MAJOR ? K : M;
    const int64_t contig_b = layout_b == GEMM_ROW_MAJOR ? N : K;
    const int64_t outer_a = layout_a == GEMM_ROW_MAJOR ? M : K;
    const int64_t outer_b = layout_b == GEMM_ROW_MAJOR ? K : N;
    const bool a_ok = (contig_a % 8 == 0) && (lda % 8 == 0) && (stride_a % 8 == 0);
    const bool b_ok = (contig_b % 8 == 0) && (ldb % 8 == 0) && (stride_b % 8 == 0);
    const bool kc_both = layout_a == GEMM_ROW_MAJOR && layout_b == GEMM_COL_MAJOR;
    const bool nn = layout_a == GEMM_ROW_MAJOR && layout_b == GEMM_ROW_MAJOR;
    // Copies padded to 8-element rows; sized here, made only by a run that
    // packs (an operand of this shape, or a misaligned pointer).
    p->ld8_a = ceil_div(contig_a, 8) * 8;
    p->ld8_b = ceil_div(contig_b, 8) * 8;
    p->pack_a_bytes = ceil_div(batch * outer_a * p->ld8_a * 2, 256) * 256;
    p->pack_b_bytes = ceil_div(batch * outer_b * p->ld8_b * 2, 256) * 256;
    // Lane offsets within an operand tile are 32-bit byte offsets: a tile
    // spans at most 256 rows (or 64 K steps) of an operand, so leading
    // dimensions up to 2^22 elements keep them below 2^31.  Larger ones are
    // read from packed copies (whose leading dimension is the row length
    // rounded up to 8); both operands are then copied, so that no kernel
    // ever reads the large-pitch operand in place.
    const int64_t kMaxLd = int64_t(1) << 22;
    const bool chunks_ok =
        batch * (outer_a * (p->ld8_a / 8) + outer_b * (p->ld8_b / 8)) < (int64_t(1) << 31);
    const bool huge_ld = K > 0 && (lda > kMaxLd || ldb > kMaxLd);
    if (huge_ld && (p->ld8_a > kMaxLd || p->ld8_b > kMaxLd || !chunks_ok)) {
        delete p;
        return GEMM_ERR_UNSUPPORTED;
    }
    // The row-vector kernel's B offsets span K rows of ldb elements in 32 bits.
    const bool rv_ok = (K + 1) * std::max(ldb, p->ld8_b) * 2 < (int64_t(1) << 31) &&
                       M * std::max(lda, p->ld8_a) * 2 < (int64_t(1) << 30);
    p->tile = choose_tile(M, N, K, batch, kc_both, nn && rv_ok, true);
    if (huge_ld) {
        p->vec_ok = 1;
        p->pack = 3;
    } else if (a_ok && b_ok) {
        p->vec_ok = 1;
    } else if (kTiles[p->tile].kind != KIND_STAGED && kTiles[p->tile].kind != KIND_SMALL && K > 0 &&
               chunks_ok) {
        // Shapes for the direct or streaming kernels repack the unaligned
        // operands: one extra pass over them instead of element-wide loads
        // for the whole K loop (copies of A and B below 2^31 16-byte chunks).
        p->vec_ok = 1;
        p->pack = (a_ok ? 0 : 1) | (b_ok ? 0 : 2);
    } else {
        // Small and batched-small products keep the operands in place: the
        // staged kernel with element-wide loads, whose largest tile is 128.
        p->vec_ok = 0;
        p->tile = choose_tile(M, N, K, batch, kc_both, nn && rv_ok, false);
    }
    // Operands given at misaligned addresses are repacked at run time only
    // for the direct and streaming kernels (and only when the workspace
    // holds the copies); the staged tiles read them with element-wide loads,
    // and so do batched small products (their staged tile).
    p->fast = p->vec_ok && kTiles[p->tile].kind != KIND_STAGED && kTiles[p->tile].kind != KIND_SMALL &&
              K > 0 && chunks_ok;
    for (int cand : {p->tile, narrow_tile(p->tile)}) {
        const TileShape &c = kTiles[cand];
        if (ceil_div(M, c.bm) * ceil_div(N, c.bn) * batch > 0x7fffffff) {
            delete p;
            return GEMM_ERR_UNSUPPORTED;
        }
    }
    p->ln_ldz = ceil_div(N, 4) * 4;
    p->ln_z_bytes = align256(batch * M * p->ln_ldz * 4);
    p->group_m = 4;
    const int64_t tiles = ceil_div(M, kTiles[p->tile].bm) * ceil_div(N, kTiles[p->tile].bn) * batch;
    choose_ksplit(p, tiles);
    // The 128 tile on a four-slot ring (three stages in flight, one
    // workgroup per CU) when its grid is one wave at that occupancy, with K
    // slices of at least four stages.  (Measured against the two-slot split
    // ring at two workgroups per CU: 1.2-1.5x on 1000^3-2048^3 and on deep-K
    // split-K shapes; 10-37% slower on grids beyond one wave, 576-2304
    // workgroups.)
    if (p->tile == TILE_128x128 && p->vec_ok) {
        const int64_t wgs = tiles * p->ksplit;
        if (wgs <= kNumCUs && p->kchunk >= 4 * kTiles[p->tile].bk) p->tile = TILE_128x128_D4;
    }
    const int t = p->vec_ok ? p->tile : narrow_tile(p->tile);
    char split[16] = "";
    if (p->ksplit > 1) snprintf(split, sizeof split, "_sk%d", p->ksplit);
    static const char *const kPackSuffix[4] = {"", "_pka", "_pkb", "_pkab"};
    snprintf(p->kernel_name, sizeof p->kernel_name, "gemm_%s%s_%c%c_%s%s%s",
             in_type == IN_BF16 ? "bf16_" : "", kTiles[t].name, layout_a == GEMM_ROW_MAJOR ? 'n' : 't',
             layout_b == GEMM_ROW_MAJOR ? 'n' : 't',
             p->vec_ok ? (kTiles[t].kind == KIND_STAGED ? "vec16" : "direct")
                       : "narrow", split, kPackSuffix[p->pack]);
    *out = p;
    return GEMM_OK;
}

}  // namespace

extern "C" int gemm_f16f32_plan(gemm_f16f32_plan_t *out, int64_t M, int64_t N,
                                int64_t K, int layout_a, int layout_b,
                                int out_type, int64_t lda, int64_t ldb,
                                int64_t ldc, int64_t batch, int64_t stride_a,
                                int64_t stride_b, int64_t stride_c) {
    return make_plan(IN_F16, out, M, N, K, layout_a, layout_b, out_type, lda, ldb, ldc,
                     batch, stride_a, stride_b, stride_c);
}

extern "C" int gemm_bf16f32_plan(gemm_f16f32_plan_t *out, int64_t M, int64_t N,
                                 int64_t K, int layout_a, int layout_b,
                                 int out_type, int64_t lda, int64_t ldb,
                                 int64_t ldc, int64_t batch, int64_t stride_a,
                                 int64_t stride_b, int64_t stride_c) {
    return make_plan(IN_BF16, out, M, N, K, layout_a, layout_b, out_type, lda, ldb, ldc,
                     batch, stride_a, stride_b, stride_c);
}

extern "C" int gemm_f16f32_set_layernorm(gemm_f16f32_plan_t plan, const void *gamma,
                                         const void *beta_ln, float eps) {
    if (!plan) return GEMM_ERR_INVALID_ARG;
    if (!gamma) {                      // back to the plain (or activation) epilogue
        plan->ln = 0;
        plan->ln_gamma = plan->ln_beta = nullptr;
        return GEMM_OK;
    }
    if (!beta_ln || (uintptr_t)gamma % 4 != 0 || (uintptr_t)beta_ln % 4 != 0) return GEMM_ERR_INVALID_ARG;
    if (!(eps >= 0.0f) || eps == INFINITY) return GEMM_ERR_INVALID_ARG;
    if (plan->act != ACT_NONE) return GEMM_ERR_INVALID_ARG;   // the normalisation replaces it
    plan->ln = 1;
    plan->ln_gamma = (const float *)gamma;
    plan->ln_beta = (const float *)beta_ln;
    plan->ln_eps = eps;
    return GEMM_OK;
}

extern "C" int gemm_f16f32_set_epilogue(gemm_f16f32_plan_t plan, const void *bias,
                                        int activation) {
    if (!plan) return GEMM_ERR_INVALID_ARG;
    if (activation < ACT_NONE || activation > ACT_SILU) return GEMM_ERR_INVALID_ARG;
    if (plan->ln && activation != ACT_NONE) return GEMM_ERR_INVALID_ARG;
    if ((uintptr_t)bias % 4 != 0) return GEMM_ERR_INVALID_ARG;
    plan->bias = (const float *)bias;
    plan->act = activation;
    return GEMM_OK;
}

extern "C" int gemm_f16f32_workspace_size(gemm_f16f32_plan_t plan, int flags, int64_t *bytes) {
    if (!plan || !bytes || (flags & ~GEMM_WS_ANY_ALIGNMENT) != 0) return GEMM_ERR_INVALID_ARG;
    int mask = plan->pack;
    if ((flags & GEMM_WS_ANY_ALIGNMENT) && plan->fast) mask = 3;
    *bytes = plan_workspace(*plan, mask);
    return GEMM_OK;
}

extern "C" int gemm_f16f32_destroy(gemm_f16f32_plan_t plan) {
    delete plan;   // host memory only: runs never depend on the plan after launch
    return GEMM_OK;
}

extern "C" const char *gemm_f16f32_status_string(int status) {
    switch (status) {
    case GEMM_OK: return "GEMM_OK";
    case GEMM_ERR_INVALID_ARG: return "GEMM_ERR_INVALID_ARG: an argument violates the documented rules";
    case GEMM_ERR_UNSUPPORTED: return "GEMM_ERR_UNSUPPORTED: valid, but outside what the kernels cover";
    case GEMM_ERR_HIP: return "GEMM_ERR_HIP: the HIP runtime refused the launch";
    case GEMM_ERR_NOMEM: return "GEMM_ERR_NOMEM: host allocation of a plan failed";
    case GEMM_ERR_SCRATCH:
        return "GEMM_ERR_SCRATCH: the plan needs more device scratch than the no-allocation "
               "entry point holds (64 MiB per device)";
    default: return "unknown status";
    }
}

extern "C" const char *gemm_f16f32_plan_kernel(gemm_f16f32_plan_t plan) {
    if (!plan) return "invalid";
    return plan->kernel_name;
}
