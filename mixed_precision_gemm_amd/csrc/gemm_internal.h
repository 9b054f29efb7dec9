// Internal plan structure and tile table shared by the planner (host C++)
// and the launcher (HIP).  Not part of the C ABI.
#pragma once

#include <stdint.h>

namespace mpgemm {

// Workgroup tile shapes.  BM x BN is the output tile of one workgroup, BK the
// K depth of one LDS stage, WGM x WGN the grid of 64-lane waves that split the
// output tile.  Each wave owns (BM/WGM) x (BN/WGN) outputs as MFMA accumulator
// blocks (16 x 16 in the direct kernels, 32 x 32 in the staged one).
enum TileId : int {
    TILE_256x256 = 0,        // compute-bound square-ish problems
    TILE_128x128 = 1,        // medium problems: more workgroups to fill 256 CUs
    TILE_64x64 = 2,          // small and batched-small products
    TILE_32x64 = 3,          // skinny M (tokens) problems
    TILE_128x128_STAGED = 4, // narrow-load fallback of the two direct tiles
    TILE_STREAM16 = 5,       // skinny M <= 16, K-contiguous A and B
    TILE_STREAM32 = 6,       // skinny M <= 32
    TILE_STREAM64 = 7,       // skinny M <= 64
    TILE_STREAM32W = 8,      // skinny M <= 32, wide N: 64 columns per workgroup; M <= 128 as row tiles
    TILE_128x128_D4 = 9,     // the 128 tile on a four-slot ring (one workgroup per CU)
    TILE_STREAM16W = 10,     // skinny M <= 16, wide N: 48 columns per workgroup
    TILE_ROWVEC = 11,        // M <= 4, row-major A and B: B streamed into registers, fp32 FMAs
    TILE_STREAM32N = 12,     // skinny M <= 32, N >= 10240: 48 columns per workgroup
    TILE_SMALL64 = 13,       // batched products of at most 64 x 64 x 64, NN: one wave each
    NUM_TILES = 14
};

// Three kernel families share the tile table:
//   KIND_DIRECT16: a two- or four-slot LDS ring filled by direct-to-LDS buffer loads
//                (no register staging) and computed with 16 x 16 x 32 MFMAs,
//                for 16-byte-aligned operands; split-K capable;
//   KIND_STAGED: a two-slot ring filled through registers (global -> VGPR ->
//                LDS), used for the small tiles and for the narrow-load path;
//   KIND_STREAM:  skinny M with K-contiguous A and B: K split over 8 waves,
//                each streaming its B rows through its own LDS region
//                (direct-to-LDS loads) and its A fragments into registers;
//   KIND_SMALL:   a batch of products of at most 64 x 64 x 64, one wave each.
enum KernelKind : int { KIND_STAGED = 1, KIND_STREAM = 2, KIND_DIRECT16 = 3, KIND_SMALL = 4 };

struct TileShape {
    int bm, bn, bk, wgm, wgn, stages, kind;
    const char *name;
};

constexpr TileShape kTiles[NUM_TILES] = {
    {256, 256, 64, 2, 2, 2, KIND_DIRECT16, "256x256x64m16"},
    {128, 128, 64, 2, 2, 2, KIND_DIRECT16, "128x128x64m16"},
    {64, 64, 64, 2, 2, 2, KIND_STAGED, "64x64x64"},
    {32, 64, 64, 1, 2, 2, KIND_STAGED, "32x64x64"},
    {128, 128, 64, 2, 2, 2, KIND_STAGED, "128x128x64"},
    {16, 16, 32, 1, 1, 1, KIND_STREAM, "stream16x16"},
    {32, 16, 32, 1, 1, 1, KIND_STREAM, "stream32x16"},
    {64, 16, 32, 1, 1, 1, KIND_STREAM, "stream64x16"},
    {32, 64, 32, 1, 1, 1, KIND_STREAM, "stream32x64"},
    {128, 128, 64, 2, 2, 4, KIND_DIRECT16, "128x128x64m16d4"},
    {16, 48, 32, 1, 1, 1, KIND_STREAM, "stream16x48"},
    {4, 64, 32, 1, 1, 1, KIND_STREAM, "rowvec4x64"},
    {32, 48, 32, 1, 1, 1, KIND_STREAM, "stream32x48"},
    {64, 64, 64, 1, 1, 1, KIND_SMALL, "small64"},
};

// Tile of the staged kernel that serves operands the direct kernel cannot
// take (unaligned rows or pointers).
constexpr int narrow_tile(int t) {
    return kTiles[t].kind == KIND_STREAM ? (kTiles[t].bm <= 32 ? TILE_32x64 : TILE_64x64)
           : kTiles[t].kind == KIND_SMALL ? TILE_64x64
           : kTiles[t].kind != KIND_STAGED ? TILE_128x128_STAGED : t;
}

constexpr int kNumCUs = 256;

// Element type of A and B (and of a 16-bit C): IEEE binary16, or bfloat16.
enum InputType : int { IN_F16 = 0, IN_BF16 = 1 };

// Activation of the fused epilogue (the values of GEMM_ACT_*).
enum Activation : int { ACT_NONE = 0, ACT_RELU = 1, ACT_GELU = 2, ACT_SILU = 3 };

// Workspace layout (caller-owned device memory, 256-byte aligned):
//   [0, 4096)                        split-K arrival counters, one int per tile
//                                    (zero between runs);
//   [4096, 4096 + split_bytes)       split-K fp32 partial tiles;
//   then, 256-byte aligned           the packed copy of A, then that of B
//                                    (only those the run makes).
// A plan that needs neither needs no workspace.  The counter area is reserved
// whenever a workspace is used, so copies never land on another plan's
// counters when runs of several plans share one buffer.
constexpr int64_t kCounterBytes = 4096;
constexpr int kMaxCounters = (int)(kCounterBytes / 4);

// Workspace bytes of a run that splits K (split_bytes) and repacks the
// operands in pack_mask (bit 0 A, bit 1 B); 0 if it does neither.
inline int64_t workspace_bytes(int64_t split_bytes, int pack_mask, int64_t pack_a_bytes,
                               int64_t pack_b_bytes) {
    const int64_t packs = ((pack_mask & 1) ? pack_a_bytes : 0) + ((pack_mask & 2) ? pack_b_bytes : 0);
    if (split_bytes == 0 && packs == 0) return 0;
    return kCounterBytes + split_bytes + packs;
}

// Residual + LayerNorm plans (gemm_f16f32_set_layernorm) also keep the fp32
// product Z = alpha A B in the workspace: its last ln_z_bytes, 256-byte
// aligned, after the counters and whatever the GEMM itself needs (so at or
// past kCounterBytes even when the GEMM needs nothing).
inline int64_t align256(int64_t x) { return (x + 255) / 256 * 256; }

// The fp32 row pass of a LayerNorm plan (gemm_layernorm.cpp's launcher, in the
// host part of gemm_kernels.hip): Y = LayerNorm(Z + beta C + bias) gamma +
// beta_ln over each of rows = batch * M rows of N, written into C.
struct LayerNormArgs {
    const float *Z;
    void *C;                  // 16-bit (out_type) or fp32 storage
    const float *bias, *gamma, *beta_ln;
    int64_t N, M, ldz, sz, ldc, sc, rows;
    float beta, eps;
    int out_type;             // GEMM_OUT_*
};

}  // namespace mpgemm

struct gemm_f16f32_plan_s {
    int64_t M, N, K;
    int layout_a, layout_b, out_type;
    int in_type;           // mpgemm::InputType of A and B (and of a 16-bit C)
    int64_t lda, ldb, ldc;
    int64_t batch, stride_a, stride_b, stride_c;
    int tile;              // mpgemm::TileId for 16-byte-aligned operands
    int vec_ok;            // shapes allow 128-bit loads (pointers checked at run)
    int group_m;           // tile rows per rasterisation group
    int64_t extent_a, extent_b, extent_c;  // elements spanned by each operand
    int ksplit;            // K slices per output tile (split-K when > 1)
    int64_t kchunk;        // K indices per slice, a multiple of 64
    int64_t split_bytes;   // fp32 partial tiles of split-K (ksplit * tiles * 64 KiB), else 0
    // Repacking: an operand whose rows do not allow 128-bit loads (leading
    // dimension, contiguous extent or batch stride not a multiple of 8), or
    // whose leading dimension is too large for 32-bit tile offsets, is copied,
    // before the product, into the workspace as a dense array with rows padded
    // to a multiple of 8 elements (zeros in the padding).
    int pack;              // operands repacked because of their shape: bit 0 A, bit 1 B
    int fast;              // a direct or streaming kernel: misaligned pointers are repacked too
    int64_t ld8_a, ld8_b;  // leading dimensions of the packed copies
    int64_t pack_a_bytes, pack_b_bytes;  // bytes of each copy (256-byte multiples)
    // Fused epilogue (gemm_f16f32_set_epilogue): C = act(alpha A B + beta C + bias).
    const float *bias;     // device pointer to N fp32 values, or NULL
    int act;               // mpgemm::Activation
    // Residual + LayerNorm (gemm_f16f32_set_layernorm): C = LayerNorm(alpha A B +
    // beta C + bias) * gamma + beta_ln over each row of C.
    int ln;                // 0 or 1
    const float *ln_gamma, *ln_beta;
    float ln_eps;
    int64_t ln_ldz;        // row stride of the fp32 Z (N rounded up to 4)
    int64_t ln_z_bytes;    // bytes of Z (batch * M * ln_ldz * 4, 256-byte multiple)
    char kernel_name[64];
};

namespace mpgemm {

// Workspace bytes of a run of plan p that repacks the operands in pack_mask:
// the GEMM's own part, then, for a LayerNorm plan, room for Z after it.
inline int64_t plan_workspace(const gemm_f16f32_plan_s &p, int pack_mask) {
    if (p.tile < 0) return 0;
    const int64_t n = workspace_bytes(p.split_bytes, pack_mask, p.pack_a_bytes, p.pack_b_bytes);
    if (!p.ln) return n;
    return align256(n > kCounterBytes ? n : kCounterBytes) + p.ln_z_bytes;
}

}  // namespace mpgemm

