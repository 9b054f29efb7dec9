// fp16 x fp16 (or bf16 x bf16) -> fp32-accumulate GEMM kernels for gfx950
// (MI355X), and the C-ABI entry points that launch them.
//
// Pages cited (titles as printed):
//   [GEMM]    "手写GEMM内核：矩阵乘法性能优化的完整工程实践" (hand-written GEMM kernel)
//   [OPS]     CUDA operator practice page (Softmax and GEMM)
//   [CATLASS] CATLASS template library page
//
// Structure of one workgroup (the pages' three-level data flow, [CATLASS] §2.2
// and [GEMM] §3, rebuilt for CDNA4):
//   * it owns one BM x BN tile of C ([GEMM] §3.1, [CATLASS] §2.1) -- or, with
//     split-K, one K slice of it -- and walks K in steps of BK, keeping the
//     fp32 accumulators in registers for the whole K loop ([GEMM] §3.2, §6.2);
//   * each K step stages an A tile (BM x BK) and a B tile (BK x BN) from global
//     memory into one slot of a multi-slot LDS ring ([OPS] §3.5, [GEMM] §4.1):
//     the direct kernels (gemm_direct16) use buffer loads that write LDS
//     without passing through registers, the staged kernel (gemm_staged)
//     128-bit loads through registers; the loads for a later step are issued
//     among the MFMAs of the current one ([GEMM] §5.1, §5.4: issue the
//     future, wait for the past);
//   * out-of-range elements (rows >= M or N, the K remainder) are loaded as
//     zeros through the buffer descriptor's range check, so the main loop has
//     no data-dependent branch ([GEMM] §3.4: zero padding, not predication);
//   * LDS rows are XOR-swizzled by the row index so that the fragment reads
//     are free of bank conflicts ([OPS] §3.3 and [GEMM] §4.3 pad rows
//     instead; the swizzle costs no LDS).  The direct kernels keep each
//     operand in its global orientation and read MN-contiguous fragments with
//     transposing LDS reads; the staged kernel transposes in registers;
//   * 64-lane waves accumulate with v_mfma_f32_16x16x32_f16 (direct and
//     streaming kernels) or v_mfma_f32_32x32x16_f16 (staged kernel): fp16
//     products, fp32 sums ([GEMM] §2.3, §6.2);
//   * the epilogue forms alpha*acc + beta*C in fp32, rounds once to fp16 (RNE)
//     or stores fp32, and masks the tile edges ([CATLASS] §2.1, [OPS] §3.2).
// Every kernel is a template on the input type TI: _Float16, or __bf16 for
// bfloat16 A and B ([CATLASS] §3.2, [GEMM] §6: the wide-range 16-bit format).
// Loads, LDS layouts and fragment reads move 16-bit elements and do not
// depend on TI; only the MFMA (the _bf16 forms of the same shapes) and the
// 16-bit C of the epilogue (bfloat16 C, rounded to nearest even) change.
// An optional fused epilogue ([CATLASS] §5.2: keep the main loop, replace the
// epilogue) turns the final value into act(alpha*acc + beta*C + bias[n]),
// applied once per output just before its rounding and store.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>

#include <algorithm>
#include <mutex>
#include <new>
#include <type_traits>
#include <utility>

#include "conv_f16.h"
#include "gemm_bf16f32.h"
#include "gemm_f16f32.h"
#include "gemm_internal.h"

// The library is built either as one translation unit (MPGEMM_PART unset)
// or in parts compiled in parallel from this same file: part 0 holds the
// host code, the kernel table and the copy kernel; parts 1-4 instantiate the
// GEMM kernels of one input type and epilogue flag each (fp16 plain, fp16
// epilogue, bf16 plain, bf16 epilogue) and fill their entries of the table.
#ifndef MPGEMM_PART
#define MPGEMM_PART -1
#endif
#define MPGEMM_HOST_PART (MPGEMM_PART <= 0)

namespace mpgemm {

struct GemmArgs {
    const uint16_t *A;            // 16-bit elements of the kernel's input type
    const uint16_t *B;
    void *C;
    int64_t M, N, K;
    int64_t lda, ldb, ldc;
    int64_t sa, sb, sc;
    int64_t extent_a, extent_b;   // elements per batch item reachable from its base
    float alpha, beta;
    int tiles_m, tiles_n;
    int group_m;
    int total_tiles;
    int out_f32;
    int c_vec;                    // C rows allow 4-element vector access
    // Fused epilogue: epi != 0 when a bias (N fp32 values) or an activation
    // (mpgemm::Activation) is set.
    int epi;
    int act;
    const float *bias;
    // Split-K (direct 128 x 128 tile only): K is cut into ksplit slices of
    // kchunk indices; grid = total_tiles * ksplit, block id = slice *
    // total_tiles + tile.  ws holds one fp32 partial tile per (slice, tile),
    // ws_count one arrival counter per tile (zero between launches).
    int ksplit;
    int64_t kchunk;
    float *ws;
    int *ws_count;
    // Implicit-GEMM convolution (conv_f16_run): A is the unrolled input,
    // read through ConvLoader with this geometry; unused by the GEMM.
    struct {
        int H, W, C, P, Q, R, S, sh, sw, ph, pw, dh, dw;
    } cv;
};

typedef void (*KernelFn)(GemmArgs);
typedef KernelFn TileKernels[NUM_TILES][2][2][2];   // [tile][A K-contig][B K-contig][vec]
typedef KernelFn FullKernels[NUM_TILES][2][2];      // K a multiple of BK: [tile][A][B]

// Table entries of one input type and epilogue flag (one part each).
void fill_kernels_f16_plain(TileKernels &k, FullKernels &kfull);
void fill_kernels_f16_epi(TileKernels &k, FullKernels &kfull);
void fill_kernels_bf16_plain(TileKernels &k, FullKernels &kfull);
void fill_kernels_bf16_epi(TileKernels &k, FullKernels &kfull);

}  // namespace mpgemm

using namespace mpgemm;

namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Byte offset that fails the buffer range check: the load returns zeros.
constexpr uint32_t kOutOfRange = 0x80000000u;
// Word 3 of a gfx9 buffer descriptor: 32-bit data format, raw addressing.
constexpr int kRsrcWord3 = 0x00020000;


// Restricts the arguments to K slice `slice` (split-K): operands advance by
// the slice's first K index, K shrinks to the slice.
__device__ inline void apply_k_slice(GemmArgs &p, int slice, bool a_kc, bool b_kc) {
    const int64_t k0 = (int64_t)slice * p.kchunk;
    const int64_t kc = p.K - k0 < p.kchunk ? p.K - k0 : p.kchunk;
    const int64_t da = a_kc ? k0 : k0 * p.lda, db = b_kc ? k0 : k0 * p.ldb;
    p.A += da; p.extent_a -= da;
    p.B += db; p.extent_b -= db;
    p.K = kc;
}

__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void *base, int64_t bytes) {
    const int32_t n = bytes <= 0 ? 0 : (bytes >= 0x7fffffff ? 0x7fffffff : (int32_t)bytes);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, n, kRsrcWord3);
}

// The MFMAs of input type TI on fragments of 8 16-bit values per lane (held
// in half8 registers whatever TI is), fp32 accumulation.
template <typename TI>
__device__ inline floatx4 mfma16(half8 a, half8 b, floatx4 c) {
    if constexpr (std::is_same<TI, __bf16>::value)
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
template <typename TI>
__device__ inline floatx16 mfma32(half8 a, half8 b, floatx16 c) {
    if constexpr (std::is_same<TI, __bf16>::value)
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// Four consecutive C elements of type T (fp32, fp16 or bf16) as one vector.
template <typename T> struct C4 { using type = half4; };
template <> struct C4<float> { using type = floatx4; };
template <> struct C4<__bf16> { using type = bf16x4; };
template <typename T>
using c4_t = typename C4<T>::type;

// XOR swizzle of the 16-byte vector index within an LDS row of VPR vectors,
// chosen so that the ds_read_b128 fragment reads (32 consecutive rows at one
// vector column per half-wave) and the row-major stores are free of bank
// conflicts.  Both forms were checked with the SQ_LDS_BANK_CONFLICT counter on
// gfx950 against the exact read pattern of the kernels: zero conflict cycles,
// where an unswizzled layout costs 12 (VPR 4) or 28 (VPR 8) extra cycles per
// read and other XOR choices for VPR 4 still cost 4.
template <int VPR>
__device__ __host__ constexpr int swz(int row) {
    static_assert(VPR == 4 || VPR == 8, "rows of 64 or 128 bytes");
    if constexpr (VPR == 8) {
        return (row ^ (row >> 3)) & 7;
    } else {
        return (row >> 2) & 3;
    }
}

// Chunk XOR for 128-byte K rows read as 16 x 16 x 32 fragments (16 rows at
// four K chunks per instruction).  ds_read_b128 serves 16 lanes a pass,
// lanes i..i+7 together with i+32..i+39: eight rows at two chunks two apart.
// Row bits (1, 3, 2) become chunk bits (0, 1, 2): within every 8-row group
// the even (and the odd) rows take one XOR from each class {c, c^2}, and
// across 16 rows all eight values, so each pass touches 64 distinct banks.
// A 64-bank model fitted to the counter (zero for the 32-row reads above,
// two-way for this read pattern under swz<8>) gives zero conflicts for this
// form.  It depends on row % 16 only.
__device__ __host__ constexpr int swz16(int row) {
    return ((row >> 1) & 1) | (((row >> 3) & 1) << 1) | (((row >> 2) & 1) << 2);
}

// Transposes an 8 x 8 block of fp16: in[c] holds row c (8 elements along the
// contiguous dimension), out[e] receives column e (8 elements, one per row).
__device__ inline void transpose8x8(const u32x4 in[8], u32x4 out[8]) {
#pragma unroll
    for (int d = 0; d < 4; ++d) {       // dword d of an input row: elements 2d, 2d+1
#pragma unroll
        for (int e = 0; e < 4; ++e) {   // dword e of an output row: rows 2e, 2e+1
            const uint32_t lo = in[2 * e][d];
            const uint32_t hi = in[2 * e + 1][d];
            out[2 * d][e] = __builtin_amdgcn_perm(hi, lo, 0x05040100u);
            out[2 * d + 1][e] = __builtin_amdgcn_perm(hi, lo, 0x07060302u);
        }
    }
}

// Loader of one operand tile (R rows of the MN dimension x BK) into LDS rows
// that are K-contiguous.  KC: the operand's storage is K-contiguous (row-major
// A, column-major B).  VEC: 128-bit loads (every 8-vector wholly in or out).
template <int R, int BK, int NT, bool KC, bool VEC>
struct TileLoader {
    static constexpr int VPR = BK / 8;                         // vectors per LDS row
    static constexpr int UNITS = KC || !VEC ? R * VPR : (R / 8) * VPR;  // per stage
    static constexpr int PER_THREAD = (UNITS + NT - 1) / NT;
    static constexpr int REGS = KC || !VEC ? PER_THREAD : PER_THREAD * 8;

    u32x4 stage[REGS];
    uint32_t off[PER_THREAD];   // byte offset of the unit, relative to the K-step base
    int kin[PER_THREAD];        // K index (relative to the step) of the unit
    bool live[PER_THREAD];      // unit exists and its MN rows are in range

    // Per-tile set-up.  r0: first MN row of the tile; rtot: M or N; ld: leading
    // dimension in elements.
    __device__ void init(int tid, int64_t r0, int64_t rtot, int64_t ld) {
#pragma unroll
        for (int q = 0; q < PER_THREAD; ++q) {
            const int idx = q * NT + tid;
            live[q] = idx < UNITS;
            if constexpr (KC) {
                const int r = idx / VPR, kv = idx % VPR;
                off[q] = (uint32_t)((r * ld + kv * 8) * 2);
                kin[q] = kv * 8;
                live[q] = live[q] && (r0 + r < rtot);
            } else if constexpr (VEC) {
                const int rb = idx % (R / 8), kb = idx / (R / 8);
                off[q] = (uint32_t)((kb * 8 * ld + rb * 8) * 2);
                kin[q] = kb * 8;
                live[q] = live[q] && (r0 + rb * 8 < rtot);
            } else {
                const int r = idx % R, kv = idx / R;
                off[q] = (uint32_t)((r + kv * 8 * ld) * 2);
                kin[q] = kv * 8;
                live[q] = live[q] && (r0 + r < rtot);
            }
        }
    }

    // Issues the global loads of the K step whose first K index is k0.
    // base points at element (r0, k0) of the operand.
    __device__ void load(const uint16_t *base, int64_t bytes_left, int64_t k0,
                         int64_t K, int64_t ld) {
        const __amdgpu_buffer_rsrc_t rs = make_rsrc(base, bytes_left);
#pragma unroll
        for (int q = 0; q < PER_THREAD; ++q) {
            if constexpr (VEC && KC) {
                const uint32_t o = (live[q] && k0 + kin[q] < K) ? off[q] : kOutOfRange;
                stage[q] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, o, 0, 0));
            } else if constexpr (VEC) {
#pragma unroll
                for (int c = 0; c < 8; ++c) {
                    const uint32_t o = (live[q] && k0 + kin[q] + c < K)
                                           ? off[q] + (uint32_t)(c * ld * 2) : kOutOfRange;
                    stage[q * 8 + c] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, o, 0, 0));
                }
            } else {
                // Narrow path: eight 16-bit loads, each range-checked on its own.
                uint32_t h[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const bool ok = live[q] && (k0 + kin[q] + e < K);
                    const uint32_t step = KC ? (uint32_t)(e * 2) : (uint32_t)(e * ld * 2);
                    const uint32_t o = ok ? off[q] + step : kOutOfRange;
                    h[e] = __builtin_amdgcn_raw_buffer_load_b16(rs, o, 0, 0);
                }
                u32x4 v;
                v[0] = h[0] | (h[1] << 16);
                v[1] = h[2] | (h[3] << 16);
                v[2] = h[4] | (h[5] << 16);
                v[3] = h[6] | (h[7] << 16);
                stage[q] = v;
            }
        }
    }

    // Writes the staged registers into an LDS slot holding R rows of VPR vectors.
    __device__ void store(u32x4 *lds, int tid) {
#pragma unroll
        for (int q = 0; q < PER_THREAD; ++q) {
            const int idx = q * NT + tid;
            if (UNITS % NT != 0 && idx >= UNITS) continue;
            if constexpr (KC) {
                const int r = idx / VPR, kv = idx % VPR;
                lds[r * VPR + (kv ^ swz<VPR>(r))] = stage[q];
            } else if constexpr (VEC) {
                const int rb = idx % (R / 8), kb = idx / (R / 8);
                u32x4 t[8];
                transpose8x8(&stage[q * 8], t);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int r = rb * 8 + e;
                    lds[r * VPR + (kb ^ swz<VPR>(r))] = t[e];
                }
            } else {
                const int r = idx % R, kv = idx / R;
                lds[r * VPR + (kv ^ swz<VPR>(r))] = stage[q];
            }
        }
    }
};

// Loader of the unrolled input of an implicit-GEMM convolution ([CATLASS]
// §5.1: the tile iterator maps row m to an input position and column k to a
// filter position, so the unrolled matrix never exists in memory).  Row m of
// A is output pixel (n, p, q); column k = (r S + s) C + c is filter tap
// (r, s) and channel c; A(m, k) = x[n, p sh - ph + r dh, q sw - pw + s dw, c]
// of the NHWC input, zero outside the image.  The tile is stored like a
// K-contiguous operand's (rows of BK, 16-byte chunks of 8 consecutive k).
// Every chunk of a thread sits at the same k within a stage, so each thread
// keeps one (r, s, c) position and advances it by BK per stage (no division
// in the K loop); per unit it keeps the window's origin and the image base.
// VEC: C is a multiple of 8, so a chunk is 8 consecutive channels of one
// tap, one 16-byte load; otherwise each element is loaded on its own.
template <int R, int BK, int NT, bool VEC>
struct ConvLoader {
    static constexpr int VPR = BK / 8;
    static constexpr int UNITS = R * VPR;
    static constexpr int PER_THREAD = (UNITS + NT - 1) / NT;
    static_assert(NT % VPR == 0, "one K chunk position per thread");

    u32x4 stage[PER_THREAD];
    int ih0[PER_THREAD], iw0[PER_THREAD], pix[PER_THREAD];   // window origin, n H W
    bool live[PER_THREAD];
    int cr, cs, cc;      // (r, s, c) of this thread's K index in the next stage
    int64_t kk;          // that K index

    template <typename G>
    __device__ __forceinline__ void init(int tid, int64_t m0, int64_t M, const G &g) {
        const int kin = (tid % VPR) * 8;
#pragma unroll
        for (int q = 0; q < PER_THREAD; ++q) {
            const int idx = q * NT + tid;
            const int64_t m = m0 + idx / VPR;
            live[q] = idx < UNITS && m < M;
            const int64_t pq = (int64_t)g.P * g.Q;
            const int64_t n = m / pq, rem = m - n * pq;
            const int p = (int)(rem / g.Q), qq = (int)(rem - (int64_t)p * g.Q);
            ih0[q] = p * g.sh - g.ph;
            iw0[q] = qq * g.sw - g.pw;
            pix[q] = (int)(n * g.H * g.W);
        }
        cc = kin;
        cs = 0;
        cr = 0;
        while (cc >= g.C) {
            cc -= g.C;
            if (++cs == g.S) { cs = 0; ++cr; }
        }
        kk = kin;
    }

    // One element (or chunk) at tap (r, s), channel c of unit q: its byte
    // offset in x, or kOutOfRange outside the image, past K or past M.
    template <typename G>
    __device__ __forceinline__ uint32_t offset(int q, int r, int s, int c, int64_t k, int64_t K, const G &g) const {
        const int ih = ih0[q] + r * g.dh, iw = iw0[q] + s * g.dw;
        const bool ok = live[q] && k < K && (unsigned)ih < (unsigned)g.H && (unsigned)iw < (unsigned)g.W;
        return ok ? (uint32_t)(((int64_t)(pix[q] + ih * g.W + iw) * g.C + c) * 2) : kOutOfRange;
    }

    // Loads the stage at the current position, then moves it on by BK.
    template <typename G>
    __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t rs, int64_t K, const G &g) {
#pragma unroll
        for (int q = 0; q < PER_THREAD; ++q) {
            if constexpr (VEC) {
                stage[q] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                       rs, offset(q, cr, cs, cc, kk, K, g), 0, 0));
            } else {
                int r = cr, s = cs, c = cc;
                uint32_t h[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    h[e] = __builtin_amdgcn_raw_buffer_load_b16(rs, offset(q, r, s, c, kk + e, K, g), 0, 0);
                    if (++c == g.C) {
                        c = 0;
                        if (++s == g.S) { s = 0; ++r; }
                    }
                }
                u32x4 v;
                v[0] = h[0] | (h[1] << 16);
                v[1] = h[2] | (h[3] << 16);
                v[2] = h[4] | (h[5] << 16);
                v[3] = h[6] | (h[7] << 16);
                stage[q] = v;
            }
        }
        cc += BK;
        while (cc >= g.C) {
            cc -= g.C;
            if (++cs == g.S) { cs = 0; ++cr; }
        }
        kk += BK;
    }

    __device__ __forceinline__ void store(u32x4 *lds, int tid) {
#pragma unroll
        for (int q = 0; q < PER_THREAD; ++q) {
            const int idx = q * NT + tid;
            if (UNITS % NT != 0 && idx >= UNITS) continue;
            const int r = idx / VPR, kv = idx % VPR;
            lds[r * VPR + (kv ^ swz<VPR>(r))] = stage[q];
        }
    }
};

// Maps a workgroup id to (batch item, tile row, tile column).  Workgroups are
// dispatched round-robin over the 8 XCDs, each with its own L2; the id is first
// remapped so that each XCD receives a contiguous run of logical tile ids, and
// logical ids walk C in groups of group_m tile rows so that the tiles resident
// on one XCD at a time share A rows and B columns in that XCD's L2.
__device__ inline void tile_coords(const GemmArgs &p, int wg, int &b, int &tm, int &tn) {
    constexpr int kXcds = 8;
    const int total = p.total_tiles;
    const int q = total / kXcds, rem = total % kXcds;
    const int xcd = wg % kXcds, local = wg / kXcds;
    const int logical = xcd * q + (xcd < rem ? xcd : rem) + local;
    const int per = p.tiles_m * p.tiles_n;
    b = logical / per;
    const int t = logical - b * per;
    const int width = p.group_m * p.tiles_n;
    const int group = t / width;
    const int first_m = group * p.group_m;
    const int gsz = min(p.tiles_m - first_m, p.group_m);
    const int tw = t - group * width;
    tm = first_m + tw % gsz;
    tn = tw / gsz;
}

// erfc(z) by formula 7.1.26 of Abramowitz and Stegun's Handbook of
// Mathematical Functions: erfc(|z|) = (a1 t + ... + a5 t^5) e^(-z^2) with
// t = 1 / (1 + p |z|), |error| <= 1.5e-7, and erfc(z) = 2 - erfc(-z) for
// z < 0.  About a third of the instructions of the library's erfcf; in the
// GELU below the error stays under 3e-7 |x| (checked in fp32 over |x| <= 40).
// Divisions in the activations use the hardware reciprocal (v_rcp_f32,
// about 1 ulp) rather than the correctly rounded division sequence, and
// exponentials the hardware 2^x (v_exp_f32) of x log2(e): rounding the
// product costs a relative error below 1e-5 where e^(-z^2) still matters,
// far inside the epilogue's tolerance (checked in fp32: GELU and SiLU
// within 3e-7 |x| over |x| <= 40).
constexpr float kLog2e = 1.44269504088896341f;
__device__ __forceinline__ float exp_hw(float x) { return __builtin_amdgcn_exp2f(x * kLog2e); }

__device__ __forceinline__ float erfc_as7126(float z) {
    const float a = fabsf(z);
    const float t = __builtin_amdgcn_rcpf(1.0f + 0.3275911f * a);
    const float poly =
        t * (0.254829592f + t * (-0.284496736f + t * (1.421413741f + t * (-1.453152027f + t * 1.061405429f))));
    const float r = poly * exp_hw(-a * a);
    return z >= 0.0f ? r : 2.0f - r;
}

// Fused-epilogue activations in fp32: ReLU max(x, 0); GELU x Phi(x) =
// x/2 erfc(-x / sqrt 2) (the erfc form keeps the left tail); SiLU
// x / (1 + e^-x), which tends to -0 as e^-x overflows (rcp(inf) = 0).
__device__ __forceinline__ float activate(int act, float x) {
    switch (act) {
    case ACT_RELU: return fmaxf(x, 0.0f);
    case ACT_GELU: return 0.5f * x * erfc_as7126(-x * 0.70710678118654752f);
    case ACT_SILU: return x * __builtin_amdgcn_rcpf(1.0f + exp_hw(-x));
    default: return x;
    }
}

// Bias of columns n..n+3 (zeros past N, or without a bias).
__device__ __forceinline__ floatx4 load_bias4(const GemmArgs &p, int64_t n) {
    floatx4 b = {0.0f, 0.0f, 0.0f, 0.0f};
    if (p.bias) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
            if (n + e < p.N) b[e] = p.bias[n + e];
    }
    return b;
}

// The epilogue of four columns on their pre-activation values.  Only the
// kernels instantiated with EPI = true contain it (the others clear p.epi at
// compile time, so the code is dead there): compiled into every kernel, the
// activations raised the register pressure of the whole kernel until the
// 256 tile's accumulators spilled inside its K loop (measured 17x slower with
// no epilogue set), and a call instead of inlining made every kernel need
// scratch (+3 us per launch on the short split-K grids).  Forced inline: with
// up to 48 call sites in one kernel the compiler otherwise emits calls and
// keeps the accumulators in a scratch frame.
__device__ __forceinline__ floatx4 epilogue4(const GemmArgs &p, floatx4 v, floatx4 bias4) {
    v += bias4;
    if (p.act != ACT_NONE) {
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = activate(p.act, v[e]);
    }
    return v;
}

// The same activations with the choice made at compile time (the direct
// kernels' epilogue dispatches once per tile on the plan's activation, so no
// branch sits between the batched loads and stores of C).
template <int ACT>
__device__ __forceinline__ floatx4 activate4(floatx4 v) {
    if constexpr (ACT != ACT_NONE) {
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = activate(ACT, v[e]);
    }
    return v;
}

// Epilogue shared by both kernels: C = alpha * acc + beta * C on the wave's
// FM x FN blocks of 32 x 32, rounded once to fp16 (RNE) or stored as fp32,
// masked at the M and N edges.  Accumulator register r of lane l in block
// (i, j) holds C(m, n) with m = l % 32 and n = 8*(r/4) + 4*(l/32) + r%4
// (block-local), so each lane owns runs of 4 consecutive n of one row.
// Four consecutive C elements from column n of one row as fp32: one vector
// access when full, else element by element up to N (zeros beyond).
template <typename T>
__device__ __forceinline__ floatx4 read_c4(const T *C, bool full, int64_t left) {
    floatx4 c = {0.0f, 0.0f, 0.0f, 0.0f};
    if constexpr (sizeof(T) == 4) {
        if (full) return *(const floatx4 *)C;
    } else if (full) {
        const c4_t<T> h = *(const c4_t<T> *)C;
#pragma unroll
        for (int e = 0; e < 4; ++e) c[e] = (float)h[e];
        return c;
    }
    for (int e = 0; e < 4 && e < left; ++e) c[e] = (float)C[e];
    return c;
}

template <typename T>
__device__ __forceinline__ void write_c4(T *C, bool full, int64_t left, floatx4 v) {
    if constexpr (sizeof(T) == 4) {
        if (full) {
            *(floatx4 *)C = v;
            return;
        }
    } else if (full) {
        *(c4_t<T> *)C = c4_t<T>{(T)v[0], (T)v[1], (T)v[2], (T)v[3]};
        return;
    }
    for (int e = 0; e < 4 && e < left; ++e) C[e] = (T)v[e];
}

// Epilogue of the staged kernel: C = alpha * acc + beta * C on the wave's
// FM x FN blocks of 32 x 32, rounded once to fp16 (RNE) or stored as fp32,
// masked at the M and N edges.  Accumulator register r of lane l in block
// (i, j) holds C(m, n) with m = l % 32 and n = 8*(r/4) + 4*(l/32) + r%4
// (block-local), so each lane owns runs of 4 consecutive n of one row.  Each
// run is read, combined and written by one straight sequence (one copy of the
// fused activation per run): with one copy per store form the unrolled body
// outgrew the compiler's unroll limit and the accumulators went to scratch.
template <typename T16, bool EPI, int FM, int FN, int WTM, int WTN>
__device__ inline void store_tile(const GemmArgs &p, const floatx16 (&acc)[FM][FN],
                                  int b, int64_t m0, int64_t n0, int wm, int wn,
                                  int lane) {
    const float alpha = p.alpha, beta = p.beta;
    const bool epi = EPI && p.epi;   // no epilogue code unless EPI
#pragma unroll
    for (int i = 0; i < FM; ++i) {
        const int64_t m = m0 + wm * WTM + i * 32 + (lane & 31);
        if (m >= p.M) continue;
#pragma unroll
        for (int j = 0; j < FN; ++j) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int64_t n = n0 + wn * WTN + j * 32 + 8 * g + 4 * (lane >> 5);
                if (n >= p.N) continue;
                const int64_t off = b * p.sc + m * p.ldc + n;
                const int64_t left = p.N - n;
                const bool full = p.c_vec && left >= 4;
                floatx4 v;
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] = alpha * acc[i][j][4 * g + e];
                if (beta != 0.0f) {
                    const floatx4 c = p.out_f32 ? read_c4((const float *)p.C + off, full, left)
                                                : read_c4((const T16 *)p.C + off, full, left);
#pragma unroll
                    for (int e = 0; e < 4; ++e) v[e] += beta * c[e];
                }
                if (epi) v = epilogue4(p, v, load_bias4(p, n));
                if (p.out_f32) write_c4((float *)p.C + off, full, left, v);
                else write_c4((T16 *)p.C + off, full, left, v);
            }
        }
    }
}

template <typename TI, int BM, int BN, int BK, int WGM, int WGN, bool AK, bool BKC, bool VEC,
          bool EPI, bool CONV = false>
__global__ __launch_bounds__(64 * WGM * WGN) void gemm_staged(GemmArgs p) {
    constexpr int NT = 64 * WGM * WGN;
    constexpr int VPR = BK / 8;
    constexpr int WTM = BM / WGM, WTN = BN / WGN;
    constexpr int FM = WTM / 32, FN = WTN / 32;
    constexpr int SLOT = (BM + BN) * VPR;          // 16-byte vectors per ring slot
    static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tile must be 32-aligned");
    static_assert(BK % 16 == 0, "BK must be a multiple of the MFMA K (16)");

    __shared__ u32x4 lds[2 * SLOT];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave / WGN, wn = wave % WGN;

    int b, tm, tn;
    tile_coords(p, blockIdx.x, b, tm, tn);
    const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;

    const uint16_t *Ab = p.A + b * p.sa;
    const uint16_t *Bb = p.B + b * p.sb;
    // Per-tile bases and K-step strides (elements) of each operand.
    const int64_t a_tile = AK ? m0 * p.lda : m0;
    const int64_t a_kstep = AK ? BK : BK * p.lda;
    const int64_t b_tile = BKC ? n0 * p.ldb : n0;
    const int64_t b_kstep = BKC ? BK : BK * p.ldb;

    static_assert(!CONV || AK, "the unrolled input is K-contiguous");
    using ALoader = typename std::conditional<CONV, ConvLoader<BM, BK, NT, VEC>,
                                              TileLoader<BM, BK, NT, AK, VEC>>::type;
    ALoader la;
    TileLoader<BN, BK, NT, BKC, VEC> lb;
    if constexpr (CONV) la.init(tid, m0, p.M, p.cv);
    else la.init(tid, m0, p.M, p.lda);
    lb.init(tid, n0, p.N, p.ldb);
    // The convolution's input as one range-checked buffer (NHWC, < 2^31 bytes).
    [[maybe_unused]] const __amdgpu_buffer_rsrc_t rx = make_rsrc(p.A, CONV ? p.extent_a * 2 : 0);

    floatx16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    const int64_t nk = (p.K + BK - 1) / BK;

    auto issue = [&](int64_t kt) {
        const int64_t k0 = kt * BK;
        const int64_t ao = a_tile + kt * a_kstep, bo = b_tile + kt * b_kstep;
        if constexpr (CONV) la.load(rx, p.K, p.cv);   // stages in order: 0, 1, 2, ...
        else la.load(Ab + ao, (p.extent_a - ao) * 2, k0, p.K, p.lda);
        lb.load(Bb + bo, (p.extent_b - bo) * 2, k0, p.K, p.ldb);
    };

    if (nk > 0) {
        issue(0);
        la.store(lds, tid);
        lb.store(lds + BM * VPR, tid);
    }
    __syncthreads();

    for (int64_t kt = 0; kt < nk; ++kt) {
        const int cur = (int)(kt & 1);
        const bool more = kt + 1 < nk;
        if (more) issue(kt + 1);

        const u32x4 *sa = lds + cur * SLOT;
        const u32x4 *sb = sa + BM * VPR;
#pragma unroll
        for (int s = 0; s < BK / 16; ++s) {
            const int kv = 2 * s + (lane >> 5);
            half8 af[FM], bf[FN];
#pragma unroll
            for (int i = 0; i < FM; ++i) {
                const int r = wm * WTM + i * 32 + (lane & 31);
                af[i] = __builtin_bit_cast(half8, sa[r * VPR + (kv ^ swz<VPR>(r))]);
            }
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                const int r = wn * WTN + j * 32 + (lane & 31);
                bf[j] = __builtin_bit_cast(half8, sb[r * VPR + (kv ^ swz<VPR>(r))]);
            }
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    // src0 = B fragment (rows n), src1 = A fragment (columns m):
                    // the block accumulates C^T, so each lane ends up holding
                    // runs of 4 consecutive n of one row m of C.
                    acc[i][j] = mfma32<TI>(bf[j], af[i], acc[i][j]);
        }

        if (more) {
            u32x4 *dst = lds + (cur ^ 1) * SLOT;
            la.store(dst, tid);
            lb.store(dst + BM * VPR, tid);
        }
        __syncthreads();
    }

    store_tile<TI, EPI, FM, FN, WTM, WTN>(p, acc, b, m0, n0, wm, wn, lane);
}

// ---------------------------------------------------------------------------
// Direct kernel: S-slot LDS ring filled by direct-to-LDS buffer loads.
//
// Every wave instruction `buffer_load_dwordx4 ... lds` writes the 16 bytes of
// lane t at LDS address M0 + 16 t, i.e. one contiguous 1 KiB run per
// instruction; the swizzled LDS layout is produced by choosing which global
// 16-byte chunk each lane fetches.  Lanes whose chunk lies outside the matrix
// are given an offset that fails the buffer range check, which writes zeros.
//   K-contiguous operand:  LDS rows [r][k], BK/8 chunks per row, chunk
//                          c stored at c ^ swz16(r); fragments by ds_read_b128.
//   MN-contiguous operand: LDS rows [k][r], R/8 chunks per row, chunk c stored
//                          at c ^ mn_swz(k); fragments by two ds_read_b64_tr_b16,
//                          which transpose 16-bit elements across each group of
//                          16 lanes (lane j addresses row k0 + j/4 at column
//                          n0 + 4 (j%4); lane i receives column n0 + i of rows
//                          k0..k0+3).
// ---------------------------------------------------------------------------

typedef short v4i16 __attribute__((ext_vector_type(4)));

// Chunk XOR of row k of an MN-contiguous tile (rows are multiples of 256
// bytes long, so only the chunk index picks the bank).  A transpose read
// touches four consecutive rows (k%4 = 0..3) per 16 lanes.  For a 32 x 32
// fragment a 32-lane pass covers those four rows over a 64-byte column span;
// for a 16 x 16 fragment it covers rows k..k+3 and k+8..k+11 over a 32-byte
// span.  XOR values {0, 10, 4, 14} by k%4, with chunk bit 1 flipped by bit 3
// of k, give every 8-byte piece of either pass its own bank (checked against
// a 64-bank, 4-byte model for 16- and 32-lane passes).
template <int R>
__device__ __host__ constexpr int mn_swz(int k) {
    static_assert(R / 8 >= 16, "MN-contiguous rows need at least 16 chunks");
    // k%4 -> 0, 10, 4, 14, and bit 3 of k flips chunk bit 1: rows k and k+8
    // are read by the two halves of one 32-lane pass of the 16 x 16 fragment
    // read, rows k..k+3 by one 16-lane group of either fragment read.
    return ((0xE4A0 >> (4 * (k & 3))) & 15) ^ (((k >> 3) & 1) << 1);
}

// Byte offset of a __shared__ object within the workgroup's LDS allocation.
__device__ inline uint32_t lds_offset(const void *p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)p;
}

// Buffer descriptor as four scalar words, for inline assembly.
typedef int32_t sgpr4 __attribute__((ext_vector_type(4)));

__device__ inline sgpr4 make_rsrc_words(const void *base, int64_t bytes) {
    const uint64_t a = (uint64_t)base;
    const int32_t n = bytes <= 0 ? 0 : (bytes >= 0x7fffffff ? 0x7fffffff : (int32_t)bytes);
    sgpr4 r;
    r[0] = __builtin_amdgcn_readfirstlane((int32_t)(uint32_t)a);
    r[1] = __builtin_amdgcn_readfirstlane((int32_t)(uint32_t)(a >> 32) & 0xffff);  // stride 0
    r[2] = __builtin_amdgcn_readfirstlane(n);
    r[3] = kRsrcWord3;
    return r;
}

// One 16-byte-per-lane direct-to-LDS load: lane t's data lands at LDS byte
// address lds_addr + 16 t.  Issued as assembly so that the compiler's
// wait-count insertion does not treat later LDS reads of other ring slots as
// dependent on it; the kernel orders it explicitly (vmcnt waits + barriers).
// lds_addr is the same for every lane (it is read from the first lane so the
// compiler can keep it in a scalar register).
__device__ inline void lds_dma16(sgpr4 rs, uint32_t lds_addr, uint32_t voff) {
    const uint32_t m0v = (uint32_t)__builtin_amdgcn_readfirstlane((int)lds_addr);
    asm volatile("s_mov_b32 m0, %1\n\tbuffer_load_dwordx4 %0, %2, 0 offen lds"
                 :
                 : "v"(voff), "s"(m0v), "s"(rs)
                 : "m0");
}

// Waits until at most N vector-memory operations of this wave are pending.
template <int N>
__device__ inline void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}

// Workgroup barrier that is also a compiler memory barrier, without the
// wait for all outstanding memory operations that a fenced barrier implies.
__device__ inline void barrier() { asm volatile("s_barrier" : : : "memory"); }

// Four consecutive elements of one C row of type T, kept in T: a vector
// access where the row and alignment allow it (vec), element by element (up
// to N, zeros beyond) otherwise.
template <typename T>
__device__ inline c4_t<T> load_c4(const GemmArgs &p, int64_t off, int64_t n, bool vec) {
    const T *C = (const T *)p.C + off;
    if (vec) return *(const c4_t<T> *)C;
    c4_t<T> c = {};
    for (int e = 0; e < 4 && n + e < p.N; ++e) c[e] = C[e];
    return c;
}

// C is written once and not read again by this launch: the vector stores
// carry the non-temporal hint, so the output streams out instead of
// displacing the operand panels the other workgroups are reading from the
// L2 (measured: 1.1-1.4x on products bound by their C traffic, e.g. 2048^2
// x 128 batched 236 -> 187 us; no change at 8192^3).
template <typename T>
__device__ inline void store_c4(const GemmArgs &p, int64_t off, int64_t n, bool vec, floatx4 v) {
    T *C = (T *)p.C + off;
    if (vec) {
        if constexpr (sizeof(T) == 4)
            __builtin_nontemporal_store(v, (floatx4 *)C);
        else
            __builtin_nontemporal_store(c4_t<T>{(T)v[0], (T)v[1], (T)v[2], (T)v[3]}, (c4_t<T> *)C);
        return;
    }
    for (int e = 0; e < 4 && n + e < p.N; ++e) C[e] = (T)v[e];
}

// Epilogue of the direct kernels, C = alpha * acc + beta * C ([GEMM] §4.4:
// scale, add the old C, round once to the output type), staged through the
// LDS ring once the main loop has drained it.  In each pass the waves that own
// a band of PR rows write alpha * acc there in fp32; then every wave reads
// whole rows back, so that each global load and store instruction covers
// complete, contiguous row segments of C (the accumulator layout alone would
// touch 32 rows 16 bytes at a time).  C is loaded in batches of 8 row
// groups, double-buffered, the first batch of a pass issued before its LDS
// staging so that its latency overlaps it.  Tiles wholly inside C with
// vector-aligned rows (FULL) test nothing; edge tiles test every row and
// column (batching them too took 1000^3 with beta = 1 from 20.0 to 18.2 us:
// in a one-wave grid the slowest tile, an edge tile, sets the time).
// Staged rows are BN fp32 values; 16-byte granule g of row r sits at granule
// g ^ (r & 15), so neither the column-wise writes nor the row-wise reads
// conflict on banks.
template <typename T, bool FULL, int BM, int BN, int WGM, int WGN, int LDS_BYTES, int MB,
          bool EPI, typename AccT, int FM, int FN>
__device__ __forceinline__ void store_tile_lds(const GemmArgs &p, const AccT (&acc)[FM][FN],
                                      u32x4 *lds, int b, int64_t m0, int64_t n0,
                                      int wave, int lane) {
    constexpr int WTM = BM / WGM, WTN = BN / WGN;
    constexpr int NW = WGM * WGN;
    constexpr int GPR = BN / 4;                      // granules per staged row
    constexpr int PR0 = LDS_BYTES / (BN * 4);
    constexpr int PR = PR0 < BM ? PR0 : BM;          // rows per pass
    constexpr int NPASS = BM / PR;
    constexpr int RPI = 64 / GPR;                    // rows per wave instruction
    constexpr int IT = PR / (RPI * NW);              // row groups per thread and pass
    constexpr int CB = IT < 8 ? IT : 8;              // C row groups per load batch
    constexpr int SW = GPR >= 16 ? 15 : GPR - 1;
    static_assert(FM * MB == WTM && FN * MB == WTN, "accumulator shape");
    static_assert(sizeof(AccT) == MB * MB / 64 * 4, "MFMA block");
    static_assert(GPR <= 64 && 64 % GPR == 0 && GPR >= 8, "row width");
    static_assert(PR % WTM == 0 && BM % PR == 0 && PR % (RPI * NW) == 0, "pass shape");
    static_assert(IT % CB == 0, "load batches");
    const int wm = wave / WGN, wn = wave % WGN;
    char *base = (char *)lds;
    const float alpha = p.alpha, beta = p.beta;
    const int r_in = lane / GPR, g = lane % GPR;
    const int64_t n = n0 + 4 * g;
    const bool n_ok = FULL || n < p.N;
    const bool vec = FULL || (p.c_vec && n + 4 <= p.N);
    const int64_t cbase = b * p.sc + n;
    const floatx4 bias4 = (p.epi && n_ok) ? load_bias4(p, n) : floatx4{0.0f, 0.0f, 0.0f, 0.0f};
    // Two register batches of C: batch k + 1 is in flight while batch k is
    // combined and stored.
    c4_t<T> cv[2][CB];
    auto load_batch = [&](int pass, int it0, int buf) __attribute__((always_inline)) {
        if (beta == 0.0f) return;
#pragma unroll
        for (int t = 0; t < CB; ++t) {
            const int r = ((it0 + t) * NW + wave) * RPI + r_in;
            const int64_t m = m0 + pass * PR + r;
            cv[buf][t] = (FULL || (m < p.M && n_ok)) ? load_c4<T>(p, cbase + m * p.ldc, n, vec)
                                                     : c4_t<T>{};
        }
    };
#pragma unroll
    for (int pass = 0; pass < NPASS; ++pass) {
        load_batch(pass, 0, 0);
        if ((wm * WTM) / PR == pass) {
            const int rb = wm * WTM - pass * PR;
            // MFMA block layout (operands swapped so that C is not
            // transposed): in a 32 x 32 block lane l holds row l%32, columns
            // 8q + 4(l/32) + 0..3 in registers 4q..4q+3; in a 16 x 16 block
            // lane l holds row l%16, columns 4(l/16) + 0..3.
#pragma unroll
            for (int i = 0; i < FM; ++i) {
                const int rl = rb + i * MB + (lane % MB);
#pragma unroll
                for (int j = 0; j < FN; ++j)
#pragma unroll
                    for (int q = 0; q < MB * MB / 256; ++q) {
                        const int gr = (wn * WTN + j * MB) / 4 + (MB == 32 ? 2 * q + (lane >> 5) : (lane >> 4));
                        const floatx4 v = {alpha * acc[i][j][4 * q], alpha * acc[i][j][4 * q + 1],
                                           alpha * acc[i][j][4 * q + 2], alpha * acc[i][j][4 * q + 3]};
                        *(floatx4 *)(base + rl * BN * 4 + ((gr ^ (rl & SW)) << 4)) = v;
                    }
            }
        }
        asm volatile("s_waitcnt lgkmcnt(0)" : : : "memory");
        barrier();
        // The staged rows in one fully unrolled loop: C loaded in batches
        // (the next batch in flight while one is combined), beta * C and the
        // bias added, then either stored (no activation: one rounding per
        // output) or, with an activation, written back to the lane's own
        // staging slot (one reader per slot).  The activation then runs in a
        // second, rolled loop chosen once per tile, so that no branch sits
        // between the batched loads and stores, and the fully unrolled loop
        // is not repeated per activation.
        const bool act = EPI && p.act != ACT_NONE;
#pragma unroll
        for (int it0 = 0; it0 < IT; it0 += CB) {
            const int buf = (it0 / CB) & 1;
            if (it0 + CB < IT) load_batch(pass, it0 + CB, buf ^ 1);
#pragma unroll
            for (int t = 0; t < CB; ++t) {
                const int r = ((it0 + t) * NW + wave) * RPI + r_in;
                const int64_t m = m0 + pass * PR + r;
                floatx4 *slot = (floatx4 *)(base + r * BN * 4 + ((g ^ (r & SW)) << 4));
                floatx4 v = *slot;
                if (beta != 0.0f) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) v[e] += beta * (float)cv[buf][t][e];
                }
                if constexpr (EPI) v += bias4;
                if (act)
                    *slot = v;
                else if (FULL || (m < p.M && n_ok))
                    store_c4<T>(p, cbase + m * p.ldc, n, vec, v);
            }
        }
        if constexpr (EPI) {
            auto act_rows = [&](auto actc) __attribute__((always_inline)) {
                constexpr int ACT = decltype(actc)::value;
#pragma unroll 4
                for (int it = 0; it < IT; ++it) {
                    const int r = (it * NW + wave) * RPI + r_in;
                    const int64_t m = m0 + pass * PR + r;
                    const floatx4 v = activate4<ACT>(*(const floatx4 *)(base + r * BN * 4 + ((g ^ (r & SW)) << 4)));
                    if (FULL || (m < p.M && n_ok)) store_c4<T>(p, cbase + m * p.ldc, n, vec, v);
                }
            };
            switch (p.act) {
            case ACT_RELU: act_rows(std::integral_constant<int, ACT_RELU>{}); break;
            case ACT_GELU: act_rows(std::integral_constant<int, ACT_GELU>{}); break;
            case ACT_SILU: act_rows(std::integral_constant<int, ACT_SILU>{}); break;
            default: break;
            }
        }
        if (pass + 1 < NPASS) {
            asm volatile("s_waitcnt lgkmcnt(0)" : : : "memory");
            barrier();
        }
    }
}

// Split-K epilogue ([GEMM] §4.4's epilogue, applied once per output after
// the K slices are summed).  Every workgroup stages its raw fp32 accumulators
// through the drained LDS ring and writes them, row by row, as the partial
// tile (slice, tile) of the workspace; then it fences and counts itself on
// the tile's counter.  The last to arrive sums the slices in slice order
// 0..ksplit-1 -- a fixed order, so results do not depend on which slice
// finished last -- applies alpha * sum + beta * C, rounds once, stores C, and
// resets the counter for the next launch.
template <typename T, int BM, int BN, int WGM, int WGN, int LDS_BYTES, int MB,
          typename AccT, int FM, int FN>
__device__ __forceinline__ void store_tile_splitk(const GemmArgs &p, const AccT (&acc)[FM][FN],
                                         u32x4 *lds, int tile, int slice, int b,
                                         int64_t m0, int64_t n0, int wave, int lane) {
    constexpr int WTM = BM / WGM, WTN = BN / WGN;
    constexpr int NW = WGM * WGN;
    constexpr int GPR = BN / 4;
    constexpr int RPI = 64 / GPR;
    constexpr int IT = BM / (RPI * NW);
    constexpr int SW = GPR >= 16 ? 15 : GPR - 1;
    static_assert(BM * BN * 4 <= LDS_BYTES, "one staging pass");
    static_assert(FM * MB == WTM && FN * MB == WTN, "accumulator shape");
    static_assert(GPR <= 64 && 64 % GPR == 0 && BM % (RPI * NW) == 0, "row mapping");
    const int wm = wave / WGN, wn = wave % WGN;
    char *base = (char *)lds;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
        const int rl = wm * WTM + i * MB + (lane % MB);
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int q = 0; q < MB * MB / 256; ++q) {
                const int gr = (wn * WTN + j * MB) / 4 + (MB == 32 ? 2 * q + (lane >> 5) : (lane >> 4));
                const floatx4 v = {acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
                *(floatx4 *)(base + rl * BN * 4 + ((gr ^ (rl & SW)) << 4)) = v;
            }
    }
    asm volatile("s_waitcnt lgkmcnt(0)" : : : "memory");
    barrier();
    const int r_in = lane / GPR, g = lane % GPR;
    const int64_t tile_elems = (int64_t)BM * BN;
    // Partials bypass the per-XCD L2 (cache policy sc0 sc1, system scope:
    // stores are written through to memory, loads miss in the L2 and read
    // memory), so the slices of a tile may run on different XCDs without an
    // L2-wide write-back or invalidate.  Ordering then needs no fence: the
    // device-scope atomic below is coherent across XCDs by itself (an
    // acquire-release version differs only by a whole-L2 write-back before
    // and invalidate after it, which protect cached data, and no L2 ever
    // holds a partial); each lane waits for its stores' acknowledgement
    // (vmcnt(0)) and the barrier puts all of them before lane 0's atomic;
    // the reducer's loads are issued only after the atomic's result has
    // passed a second barrier.
    constexpr int kCoherent = 1 | 16;
    const __amdgpu_buffer_rsrc_t rws = make_rsrc(p.ws, (int64_t)p.ksplit * p.total_tiles * tile_elems * 4);
    const uint32_t mine = (uint32_t)(((int64_t)slice * p.total_tiles + tile) * tile_elems * 4);
#pragma unroll
    for (int it = 0; it < IT; ++it) {
        const int r = (it * NW + wave) * RPI + r_in;
        const u32x4 v = *(const u32x4 *)(base + r * BN * 4 + ((g ^ (r & SW)) << 4));
        __builtin_amdgcn_raw_buffer_store_b128(v, rws, mine + (uint32_t)((r * BN + 4 * g) * 4), 0, kCoherent);
    }
    asm volatile("s_waitcnt vmcnt(0)" : : : "memory");   // this lane's partial is in memory
    __syncthreads();
    // The arrival flag lives in the LDS word right after the staging area
    // (the caller's buffer extends past LDS_BYTES).
    volatile int *last_flag = (volatile int *)(base + LDS_BYTES);
    if (threadIdx.x == 0)
        *last_flag = __hip_atomic_fetch_add(&p.ws_count[tile], 1, __ATOMIC_RELAXED,
                                            __HIP_MEMORY_SCOPE_AGENT) == p.ksplit - 1;
    __syncthreads();
    if (!*last_flag) return;
    const float alpha = p.alpha, beta = p.beta;
    const int64_t n = n0 + 4 * g;
    const bool n_ok = n < p.N;
    const bool vec = p.c_vec && n + 4 <= p.N;
    const floatx4 bias4 = (p.epi && n_ok) ? load_bias4(p, n) : floatx4{0.0f, 0.0f, 0.0f, 0.0f};
    const uint32_t tile0 = (uint32_t)((int64_t)tile * tile_elems * 4);
    const uint32_t slice_stride = (uint32_t)((int64_t)p.total_tiles * tile_elems * 4);
    // All slices of RB row groups (and their C) are requested before any is
    // summed: the partials come from memory, so the reduction is latency
    // bound unless many loads are in flight (half the 128 tile's rows at a
    // time: against a quarter, 3-9 % faster on the split-K shapes, e.g.
    // 128 x 4096 x 4096 in eight slices 25.9 -> 23.5 us).  Slices are summed
    // in order.
    constexpr int KSMAX = 8, RB = IT >= 8 ? 8 : IT;
    static_assert(IT % RB == 0, "row batches");
#pragma unroll 1
    for (int it0 = 0; it0 < IT; it0 += RB) {
        floatx4 part[RB][KSMAX];
        c4_t<T> cv[RB];
#pragma unroll
        for (int u = 0; u < RB; ++u) {
            const int r = ((it0 + u) * NW + wave) * RPI + r_in;
            const int64_t m = m0 + r;
#pragma unroll
            for (int sl = 0; sl < KSMAX; ++sl)
                part[u][sl] = sl < p.ksplit
                    ? __builtin_bit_cast(floatx4, __builtin_amdgcn_raw_buffer_load_b128(
                          rws, tile0 + (uint32_t)sl * slice_stride + (uint32_t)((r * BN + 4 * g) * 4), 0, kCoherent))
                    : floatx4{0.0f, 0.0f, 0.0f, 0.0f};
            cv[u] = (beta != 0.0f && m < p.M && n_ok) ? load_c4<T>(p, b * p.sc + m * p.ldc + n, n, vec) : c4_t<T>{};
        }
#pragma unroll
        for (int u = 0; u < RB; ++u) {
            const int r = ((it0 + u) * NW + wave) * RPI + r_in;
            const int64_t m = m0 + r;
            floatx4 sum = part[u][0];
#pragma unroll
            for (int sl = 1; sl < KSMAX; ++sl)
                if (sl < p.ksplit) sum += part[u][sl];
            if (m < p.M && n_ok) {
                floatx4 v = alpha * sum;
                if (beta != 0.0f) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) v[e] += beta * (float)cv[u][e];
                }
                if (p.epi) v = epilogue4(p, v, bias4);
                store_c4<T>(p, b * p.sc + m * p.ldc + n, n, vec, v);
            }
        }
    }
    if (threadIdx.x == 0)
        __hip_atomic_store(&p.ws_count[tile], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int R, int BK, int NW, bool KC>
struct DirectOperand {
    static constexpr int VPR = BK / 8;                 // chunks per [r][k] row
    static constexpr int CPR = R / 8;                  // chunks per [k][r] row
    static constexpr int CHUNKS = R * BK / 8;          // 16-byte chunks per stage
    static constexpr int INSTR = CHUNKS / 64;          // 1 KiB instructions per stage
    static constexpr int PER_WAVE = INSTR / NW;
    static_assert(CHUNKS % 64 == 0 && INSTR % NW == 0, "stage must split evenly over waves");

    uint32_t off[PER_WAVE];   // byte offset of this lane's chunk, kOutOfRange if past the rows
    uint32_t kin4[(PER_WAVE + 3) / 4];  // K index (< BK) of each chunk, four per word

    __device__ void init(int wave, int lane, int64_t r0, int64_t rtot, int64_t ld) {
#pragma unroll
        for (int i = 0; i < (PER_WAVE + 3) / 4; ++i) kin4[i] = 0;
#pragma unroll
        for (int i = 0; i < PER_WAVE; ++i) {
            const int p = (i * NW + wave) * 64 + lane;
            bool ok;
            int kin;
            if constexpr (KC) {
                const int r = p / VPR, c = (p % VPR) ^ swz16(r);
                off[i] = (uint32_t)((r * ld + c * 8) * 2);
                kin = c * 8;
                ok = r0 + r < rtot;
            } else {
                const int k = p / CPR, c = (p % CPR) ^ mn_swz<R>(k);
                off[i] = (uint32_t)((k * ld + c * 8) * 2);
                kin = k;
                ok = r0 + c * 8 < rtot;
            }
            if (!ok) off[i] = kOutOfRange;
            kin4[i / 4] |= (uint32_t)kin << (8 * (i % 4));
        }
    }

    // Number of K indices left in the stage that starts at k0, clamped to
    // [0, BK] (uniform over the wave).
    __device__ static int stage_left(int64_t k0, int64_t K) {
        const int64_t left64 = K - k0;
        return __builtin_amdgcn_readfirstlane(left64 <= 0 ? 0 : (left64 >= BK ? BK : (int)left64));
    }
    __device__ sgpr4 stage_rsrc(const uint16_t *base, int64_t bytes_left) const {
        return make_rsrc_words(base, bytes_left);
    }
    // For K-contiguous 128-byte rows the K index of load i depends on i only
    // through (i NW + wave) % 2 (load i covers rows 8 (i NW + wave) .. + 7,
    // and of their row bits swz16 takes bit 3 from that index): with an even
    // number of loading waves, one K class per wave, and the K test of a
    // stage is a single compare (kmask) and one select per load
    // (issue_one_masked).
    static constexpr int KCL = NW % 2 == 0 ? 1 : 2;
    __device__ bool kmask(int left) const {
        static_assert(KC && VPR == 8 && KCL == 1, "one K class");
        return (int)(kin4[0] & 0xffu) < left;
    }
    __device__ void issue_one_masked(int i, sgpr4 rs, uint32_t lds_addr, int wave, bool ok) const {
        lds_dma16(rs, lds_addr + (uint32_t)((i * NW + wave) * 64 * 16), ok ? off[i] : kOutOfRange);
    }

    // Load i of a stage that lies wholly inside K: no K test.
    __device__ void issue_one_full(int i, sgpr4 rs, uint32_t lds_addr, int wave) const {
        lds_dma16(rs, lds_addr + (uint32_t)((i * NW + wave) * 64 * 16), off[i]);
    }
    // Load i of this wave's share of a stage; chunks at K indices >= left
    // fail the range check and write zeros.
    __device__ void issue_one(int i, sgpr4 rs, uint32_t lds_addr, int wave, int left) const {
        const int kin = (int)((kin4[i / 4] >> (8 * (i % 4))) & 0xffu);
        const uint32_t o = kin < left ? off[i] : kOutOfRange;
        lds_dma16(rs, lds_addr + (uint32_t)((i * NW + wave) * 64 * 16), o);
    }

    // Issues this wave's share of one stage.  base: element (r0, k0) of the
    // operand; lds: the operand's region of the ring slot.  Stages at or
    // beyond the end of K fail every range check and write zeros.
    __device__ void issue(const uint16_t *base, int64_t bytes_left, uint32_t lds_addr,
                          int wave, int64_t k0, int64_t K) {
        const sgpr4 rs = make_rsrc_words(base, bytes_left);
        const int left = stage_left(k0, K);
#pragma unroll
        for (int i = 0; i < PER_WAVE; ++i) issue_one(i, rs, lds_addr, wave, left);
    }

};

// Per-lane LDS byte offsets of one operand's 16 x 16 x 32 fragments for one
// wave (rows or columns wb .. wb + 16 NBLK - 1 of a BK = 64 ring slot), so
// that every fragment read is a base register plus an immediate offset.  Two
// sets: `cur` addresses the slot of the stage being computed (read by its
// head K step), `nxt` the slot of the next one (read by its tail K step).
// Slot s starts s slot sizes (a power of two) above slot 0, which starts at
// 0, and every slot-0 address is below the slot size, so moving a base on by
// a stage is one add-and-wrap (one XOR for a two-slot ring; step()) and no
// other address arithmetic is left in the K loop.  The kernel moves the
// bases one register at a time between MFMAs: each cur base during a stage's
// tail (after the head's last read of it), each nxt base during a stage's
// head (before the tail reads it).  Both start at stage 0; the first head
// moves nxt to stage 1.
//   K-contiguous: row r = wb + 16 i + l%16 keeps its K chunk kv = 4 s + l/16
//     at kv ^ swz16(r) = (l/16 ^ swz16(l%16)) ^ 4 s (swz16 depends on r % 16
//     only): two bases, by s, and 16 rows per block as immediates.
//   MN-contiguous: column n = wb + 16 i + 4 (l%4) of row
//     k = 32 s + 4 t + 8 (l/16) + (l%16)/4 sits in chunk (n >> 3) ^ mn_swz(k),
//     and mn_swz(k) depends only on k%4 and bit 3 of k, both fixed by the
//     lane: one base per block i, rows 32 s + 4 t as immediates.
template <int R, int BK, bool KC, int NBLK, int SLOT_BYTES, int NSLOT, int BASE>
struct Frag16 {
    static_assert(BK == 64, "128-byte K rows");
    static_assert((SLOT_BYTES & (SLOT_BYTES - 1)) == 0 && SLOT_BYTES <= 65536,
                  "slot size a power of two");
    static_assert(NSLOT >= 2 && NSLOT <= 4 && BASE + NSLOT * SLOT_BYTES <= 160 * 1024,
                  "two to four slots inside the LDS");
    static_assert(NSLOT != 4 || BASE < SLOT_BYTES, "four slots: operand region inside an interleaved slot");
    static constexpr int NCLS = KC ? 2 : NBLK;
    uint32_t cur[NCLS], nxt[NCLS];

    // Bases for stage 0 (slot 0) in cur and in nxt.
    __device__ void setup(int lane, int wb) {
        constexpr uint32_t region = (uint32_t)BASE;
        const int lr = lane & 15, lg = lane >> 4;
        if constexpr (KC) {
            const int X = lg ^ swz16(lr);
#pragma unroll
            for (int c = 0; c < 2; ++c)
                cur[c] = region + (uint32_t)((wb + lr) * BK * 2 + 16 * (X ^ (4 * c)));
        } else {
            const int W = ((lr & 3) >> 1) ^ mn_swz<R>(8 * lg + (lr >> 2));
#pragma unroll
            for (int i = 0; i < NBLK; ++i)
                cur[i] = region + (uint32_t)((8 * lg + (lr >> 2)) * R * 2 +
                                             16 * ((wb / 8 + 2 * i) ^ W) + 8 * (lr & 1));
        }
#pragma unroll
        for (int c = 0; c < NCLS; ++c) nxt[c] = cur[c];
    }

    // Next stage: a base moves one slot on, wrapping around the ring.  Two
    // slots at BASE and BASE + SLOT_BYTES: one XOR.  Three (at 0): the
    // smaller of x + SLOT and x - 2 SLOT as unsigned values (the second
    // wraps below zero unless x + SLOT has passed the ring's end).  Four
    // (interleaved, BASE inside the first slot): add and mask.  Written as
    // volatile assembly so that each update stays between the MFMAs the
    // kernel places it after (plain arithmetic was gathered into one burst).
    __device__ static void step(uint32_t &x) {
        if constexpr (NSLOT == 2) {
            // One XOR moves base + offset to base + SLOT + offset only if
            // base + offset == base | offset: a slot-aligned base.
            static_assert(BASE % SLOT_BYTES == 0, "two slots: slot-aligned base");
            constexpr uint32_t flip = (uint32_t)BASE ^ (uint32_t)(BASE + SLOT_BYTES);
            asm volatile("v_xor_b32 %0, %1, %0" : "+v"(x) : "i"(flip));
        } else if constexpr (NSLOT == 3) {
            static_assert(BASE == 0 && 3 * SLOT_BYTES < (1 << 30), "three slots from LDS address 0");
            uint32_t t;
            asm volatile("v_add_u32 %0, %2, %1\n\tv_add_u32 %1, %3, %1\n\tv_min_u32 %1, %0, %1"
                         : "=&v"(t), "+v"(x)
                         : "i"(SLOT_BYTES), "i"(-2 * SLOT_BYTES));
        } else {
            asm volatile("v_add_u32 %0, %1, %0\n\tv_and_b32 %0, %2, %0"
                         : "+v"(x)
                         : "i"(SLOT_BYTES), "i"(NSLOT * SLOT_BYTES - 1));
        }
    }
    __device__ void advance_cur(int c) { step(cur[c]); }
    __device__ void advance_nxt(int c) { step(nxt[c]); }

    // Fragment of block i, K step s (32 deep) of the current (NEXT = false)
    // or next stage: lane l receives row (or column) wb + 16 i + l%16,
    // k = 32 s + 8 (l/16) + 0..7.
    template <bool NEXT>
    __device__ half8 read(const u32x4 *lds, int i, int s) const {
        const char *bytes = (const char *)lds;
        const uint32_t *b = NEXT ? nxt : cur;
        if constexpr (KC) {
            return __builtin_bit_cast(half8, *(const u32x4 *)(bytes + b[s] + 16 * BK * 2 * i));
        } else {
            v4i16 h[2];
#pragma unroll
            for (int t = 0; t < 2; ++t)
                h[t] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (__attribute__((address_space(3))) v4i16 *)(bytes + b[i] + (32 * s + 4 * t) * R * 2));
            const v4i16 lo = h[0], hi = h[1];
            return __builtin_bit_cast(half8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        }
    }
};

// A buffer descriptor moved on by a fixed byte step per stage (the K-full
// direct kernels' loads): 64-bit base, bytes left from it (negative past the
// operand's end, where the descriptor holds zero records).  The words are
// kept current, so a stage's loads use them as they are; advance() is four
// scalar instructions.  Callers guarantee that bytes left and the step stay
// within +-2^31 and that the base stays below 2^48 (word 1's stride bits are
// never touched).
struct RunRsrc {
    int32_t w0, w1, w2;   // base low, base high, records
    int32_t left, step;
    __device__ void init(const void *base, int64_t bytes_left, int64_t step_bytes) {
        const uint64_t a = (uint64_t)base;
        w0 = __builtin_amdgcn_readfirstlane((int32_t)(uint32_t)a);
        w1 = __builtin_amdgcn_readfirstlane((int32_t)((uint32_t)(a >> 32) & 0xffffu));
        left = __builtin_amdgcn_readfirstlane((int32_t)bytes_left);
        step = __builtin_amdgcn_readfirstlane((int32_t)step_bytes);
        w2 = left > 0 ? left : 0;
    }
    __device__ sgpr4 words() const {
        sgpr4 r;
        r[0] = w0;
        r[1] = w1;
        r[2] = w2;
        r[3] = kRsrcWord3;
        return r;
    }
    __device__ void advance() {
        // Plain scalar arithmetic; readfirstlane keeps every word provably
        // uniform (free when it already is), whatever register the compiler
        // picked for an intermediate, so the loads' descriptor stays scalar.
        const uint64_t a = (((uint64_t)(uint32_t)w1 << 32) | (uint32_t)w0) + (uint64_t)(int64_t)step;
        w0 = __builtin_amdgcn_readfirstlane((int32_t)(uint32_t)a);
        w1 = __builtin_amdgcn_readfirstlane((int32_t)(uint32_t)(a >> 32));
        left = __builtin_amdgcn_readfirstlane(left - step);
        w2 = __builtin_amdgcn_readfirstlane(left > 0 ? left : 0);
    }
};

// Position (the MFMA it follows) of bookkeeping item t of NB in a K step of
// NQ MFMAs: spread evenly, moved on past any position that follows a fragment
// read (R - 1 mod R) or a load (OFF mod T, when the step loads).
__host__ __device__ constexpr int book_pos(int t, int nb, int nq, int r, int tl, int off, int nl) {
    const int base = (t * nq) / nb;
    for (int d = 0; d < 4; ++d) {
        const int q = (base + d) % nq;
        const bool read = r >= 1 && q % r == r - 1;
        const bool load = nl > 0 && tl >= 1 && q >= off && (q - off) % tl == 0 && (q - off) / tl < nl;
        if (!read && !load) return q;
    }
    return base;
}

// For each MFMA position of a K step, the set of bookkeeping items (a bit
// mask) placed after it, evaluated at compile time.
template <int NB, int NQ, int R, int TL, int OFF, int NL>
struct BookTable {
    static_assert(NB <= 32, "item mask in one word");
    struct Masks {
        uint32_t at[NQ];
    };
    static constexpr Masks make() {
        Masks m{};
        for (int t = 0; t < NB; ++t) m.at[book_pos(t, NB, NQ, R, TL, OFF, NL)] |= 1u << t;
        return m;
    }
    static constexpr Masks masks = make();
};

// Calls f(std::integral_constant<int, I>) for I = 0 .. N-1 in order: a loop
// unrolled by construction, whose index is a compile-time constant.
template <typename F, int... I>
__device__ __forceinline__ void unroll_seq(std::integer_sequence<int, I...>, F &&f) {
    (f(std::integral_constant<int, I>{}), ...);
}

// ---------------------------------------------------------------------------
// Direct kernel on 16 x 16 x 32 MFMAs (256 x 256 and 128 x 128 tiles): the
// ring, loads and swizzles above; each wave owns (BM/WGM) x (BN/WGN) outputs as 16 x 16
// accumulator blocks.  With a 128 x 128 wave tile a 32-deep K step is 64
// MFMAs of 16 cycles fed by 16 one-KiB fragment reads -- the same LDS traffic
// per flop as 32 x 32 blocks -- and back-to-back 16 x 16 x 32 MFMAs on
// independent accumulators keep the matrix core busier than 32 x 32 x 16
// ones do on gfx950 (measured: 97 % against 75 % of peak for the same 128 x
// 128 register tile with no memory traffic at all).
//
// Stage kt (BK = 64: two K steps) lives in ring slot kt % S of B's ring (S =
// 2 or 4 slots) and of A's (S, or 3 for a split two-slot ring).  The K loop
// is rotated so that its back edge follows the stage barrier:
//   head(kt): K step 0 of stage kt, reading the fragments of K step 1 (split
//             ring: and loading stage kt+2's A tile into the A slot of
//             stage kt-1); wait for this lane's loads of stage kt+1 and for
//             all LDS reads; barrier -- stage kt+1 is readable and stage
//             kt's slots are free;
//   tail(kt): K step 1 of stage kt, reading the fragments of stage kt+1 K
//             step 0 and issuing the loads of stage kt+S (split ring: its B
//             tile) into stage kt's slots.
// A four-slot ring keeps three stages in flight, for grids too small to hide
// HBM latency with more workgroups.  Each stage issues exactly L loads per
// lane (stages past the end of K fail the range check and write zeros), so
// the wait counts are exact.
// ---------------------------------------------------------------------------
template <typename TI, int BM, int BN, int BK, int WGM, int WGN, int S, bool AK, bool BKC, bool KFULL,
          bool EPI>
__global__ __launch_bounds__(64 * WGM * WGN)
__attribute__((amdgpu_waves_per_eu(BM * BN >= 65536 ? 1 : 2, BM * BN >= 65536 ? 1 : 2)))
void gemm_direct16(GemmArgs pin) {
    GemmArgs p = pin;
    if constexpr (!EPI) p.epi = 0;   // no epilogue code in this instantiation
    constexpr int NW = WGM * WGN;
    constexpr int WTM = BM / WGM, WTN = BN / WGN;
    constexpr int FM = WTM / 16, FN = WTN / 16;
    constexpr int NKS = BK / 32;
    constexpr int A_CH = BM * BK / 8, B_CH = BN * BK / 8;
    constexpr int SLOT = A_CH + B_CH;                 // 16-byte chunks per slot
    using OpA = DirectOperand<BM, BK, NW, AK>;
    using OpB = DirectOperand<BN, BK, NW, BKC>;
    constexpr int L = OpA::PER_WAVE + OpB::PER_WAVE;  // loads per lane per stage
    static_assert(S == 2 || S == 4, "a two- or four-slot ring");
    static_assert((S - 1) * L < 64, "vmcnt range");
    static_assert(NKS == 2, "head and tail are one K step each");
    static_assert(L < 64, "vmcnt range");

    // Ring layout.  Interleaved (four slots): S slots of [A tile][B tile].
    // Split (two-slot rings): A on three slots and B on two -- 5 x 32 KiB,
    // all of the LDS, for the 256 tile; 5 x 16 KiB, two workgroups per CU,
    // for the 128 tile.  Stage kt + 2's A tile then goes into the slot of stage kt - 1,
    // free since the barrier ending head(kt - 1), so its loads are issued in
    // head(kt) and only B's in tail(kt): each K step carries half of a
    // stage's loads instead of the tail carrying all of them, which kept the
    // load unit's address and command queues full.
    constexpr bool SPLIT = S == 2;
    constexpr int SA = SPLIT ? 3 : S;
    constexpr int A_SLOT = SPLIT ? A_CH * 16 : SLOT * 16;   // bytes between A slots
    constexpr int B_SLOT = SPLIT ? B_CH * 16 : SLOT * 16;
    constexpr int A_BASE = 0, B_BASE = SPLIT ? SA * A_CH * 16 : A_CH * 16;
    constexpr int PA = OpA::PER_WAVE, PB = OpB::PER_WAVE;
    // Split-K's epilogue stages S * SLOT chunks and keeps one flag word after
    // them: inside the split ring, one extra chunk for the interleaved one.
    constexpr int RING = SPLIT ? SA * A_CH + S * B_CH : S * SLOT;
    __shared__ u32x4 lds[RING > S * SLOT ? RING : S * SLOT + 1];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WGN, wn = wave % WGN;

    const int slice = (int)(blockIdx.x / (unsigned)p.total_tiles);
    const int tile = (int)(blockIdx.x - (unsigned)slice * (unsigned)p.total_tiles);
    if (p.ksplit > 1) apply_k_slice(p, slice, AK, BKC);
    int b, tm, tn;
    tile_coords(p, tile, b, tm, tn);
    const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
    const uint16_t *Ab = p.A + b * p.sa;
    const uint16_t *Bb = p.B + b * p.sb;
    const int64_t a_tile = AK ? m0 * p.lda : m0;
    const int64_t a_kstep = AK ? BK : BK * p.lda;
    const int64_t b_tile = BKC ? n0 * p.ldb : n0;
    const int64_t b_kstep = BKC ? BK : BK * p.ldb;

    OpA opa;
    OpB opb;
    opa.init(wave, lane, m0, p.M, p.lda);
    opb.init(wave, lane, n0, p.N, p.ldb);

    floatx4 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};

    const int64_t nk = (p.K + BK - 1) / BK;
    const uint32_t lds_base = lds_offset(lds);

    auto issue = [&](int64_t st) __attribute__((always_inline)) {
        const uint32_t sa = lds_base + (uint32_t)(A_BASE + (st % SA) * A_SLOT);
        const uint32_t sb = lds_base + (uint32_t)(B_BASE + (st % S) * B_SLOT);
        const int64_t ao = a_tile + st * a_kstep, bo = b_tile + st * b_kstep;
        opa.issue(Ab + ao, (p.extent_a - ao) * 2, sa, wave, st * BK, p.K);
        opb.issue(Bb + bo, (p.extent_b - bo) * 2, sb, wave, st * BK, p.K);
    };

    // K-full kernels (launched only when both operands, and S + 2 stages past
    // their ends, lie within 2^30 bytes of their tile bases) keep each
    // operand's buffer descriptor for the next stage it loads and move it on
    // by one stage after use: a 64-bit base add and a 32-bit bytes-left
    // subtract, clamped at zero, instead of forming the stage offset and a
    // 64-bit clamp at every stage.  Loads of each operand go out stage by
    // stage in order (stages S, S+1, ... after the prologue's 0 .. S-1).
    RunRsrc ra, rb;
    if constexpr (KFULL) {
        ra.init(Ab + a_tile + S * a_kstep, (p.extent_a - a_tile - S * a_kstep) * 2, a_kstep * 2);
        rb.init(Bb + b_tile + S * b_kstep, (p.extent_b - b_tile - S * b_kstep) * 2, b_kstep * 2);
    }

    static_assert(WTM % 16 == 0 && WTN % 16 == 0, "16-row fragment blocks");
    using FragA = Frag16<BM, BK, AK, FM, A_SLOT, SA, A_BASE>;
    using FragB = Frag16<BN, BK, BKC, FN, B_SLOT, S, B_BASE>;
    FragA fra;
    FragB frb;
    fra.setup(lane, wm * WTM);
    frb.setup(lane, wn * WTN);

    half8 fa[2][FM], fb[2][FN];
    using Z = std::integral_constant<int, 0>;
    using O = std::integral_constant<int, 1>;

    // One K step: the FM*FN MFMAs on fragment buffer CUR, with the reads of
    // the next K step's fragments (ring slot RSL, step RKS, into buffer
    // CUR ^ 1) and, if LOADS, this wave's L direct-to-LDS loads of stage dst
    // (into slot DSL) spread evenly between them in a fixed order.  B
    // fragments are read first: the next step's first FN MFMAs need all of
    // them.  Only K-contiguous operands test K: rows k >= K of an
    // MN-contiguous operand start past its extent and fail the range check.
    // KFULL (K a multiple of BK) tests nothing: every stage inside K is full,
    // and the loads of the S stages past the end (issued by the last tails)
    // are range-checked reads that land in slots no MFMA reads again.
    // BOOK: the head's (0) or the tail's (1) bookkeeping -- the fragment
    // bases and the running descriptors moved on one register or one
    // descriptor at a time, each after the MFMA of its own position, so that
    // no MFMA waits behind a burst of address arithmetic (an MFMA leaves
    // room for three other instructions).
    constexpr int NQ = FM * FN;
    constexpr int NF = FM + FN;
    // LOADS: 0 none, 1 the A loads, 2 the B loads, 3 both, of stage dst;
    // sa and sb are the LDS byte addresses of its A and B slots.
    uint32_t a_ld = (uint32_t)(A_BASE + (2 % SA) * A_SLOT);   // split ring: A slot of stage kt+2
    auto kstep = [&](auto curc, auto nextc, auto rksc, auto loadsc, auto bookc, int64_t dst, uint32_t sa,
                     uint32_t sb) __attribute__((always_inline)) {
        constexpr int CUR = decltype(curc)::value, RKS = decltype(rksc)::value;
        constexpr bool NEXT = decltype(nextc)::value;
        constexpr int LOADS = decltype(loadsc)::value;
        constexpr int BOOK = decltype(bookc)::value;
        constexpr bool LA = LOADS & 1, LB = LOADS & 2;
        constexpr int na = LA ? PA : 0;
        constexpr int nl = na + (LB ? PB : 0);
        sgpr4 rsa = {}, rsb = {};
        bool ma = true, mb = true;
        if constexpr (LOADS != 0) {
            const int left = (!KFULL && (AK || BKC)) ? OpA::stage_left(dst * BK, p.K) : BK;
            if constexpr (LA) {
                if constexpr (KFULL) {
                    rsa = ra.words();
                } else {
                    const int64_t ao = a_tile + dst * a_kstep;
                    rsa = opa.stage_rsrc(Ab + ao, (p.extent_a - ao) * 2);
                    if constexpr (AK) ma = opa.kmask(left);
                }
            }
            if constexpr (LB) {
                if constexpr (KFULL) {
                    rsb = rb.words();
                } else {
                    const int64_t bo = b_tile + dst * b_kstep;
                    rsb = opb.stage_rsrc(Bb + bo, (p.extent_b - bo) * 2);
                    if constexpr (BKC) mb = opb.kmask(left);
                }
            }
        }
        // Load l follows MFMA l T + OFF (T MFMAs apart).  Fragment reads
        // follow MFMAs R - 1, 2 R - 1, ... (R = NQ / NF); when T is a
        // multiple of R, OFF = R/2 - 1 puts each load between two reads,
        // so no MFMA is followed by both a load and a read.
        constexpr int T = nl > 0 ? NQ / nl : 1;
        constexpr int R = NQ / NF;
        constexpr int OFF = nl > 0 && T >= 1 && R >= 2 && T % R == 0 ? R / 2 - 1 : T - 1;
        // Bookkeeping items: the fragment bases of A then B (FragA::NCLS +
        // FragB::NCLS), then (BOOK = head) the A descriptor and the split
        // ring's A slot, or (BOOK = tail) the B descriptor and, with an
        // interleaved ring, the A descriptor; item t follows MFMA book_pos(t).
        constexpr int NBK = FragA::NCLS + FragB::NCLS + 2;
        using Book = BookTable<NBK, NQ, R, T, OFF, nl>;
        unroll_seq(std::make_integer_sequence<int, NQ>{}, [&](auto qc) __attribute__((always_inline)) {
            constexpr int q = decltype(qc)::value;
            constexpr int i = q / FN, j = q % FN;
            acc[i][j] = mfma16<TI>(fb[CUR][j], fa[CUR][i], acc[i][j]);
            unroll_seq(std::make_integer_sequence<int, NBK>{}, [&](auto tc) __attribute__((always_inline)) {
                constexpr int t = decltype(tc)::value;
                if constexpr ((Book::masks.at[q] >> t) & 1u) {
                    if constexpr (t < FragA::NCLS) {
                        if constexpr (BOOK == 0) fra.advance_nxt(t);
                        else fra.advance_cur(t);
                    } else if constexpr (t < FragA::NCLS + FragB::NCLS) {
                        if constexpr (BOOK == 0) frb.advance_nxt(t - FragA::NCLS);
                        else frb.advance_cur(t - FragA::NCLS);
                    } else if constexpr (t == NBK - 2) {
                        if constexpr (KFULL && BOOK == 0 && SPLIT) ra.advance();
                        if constexpr (KFULL && BOOK == 1) rb.advance();
                    } else {
                        if constexpr (BOOK == 0 && SPLIT)
                            a_ld = a_ld + (uint32_t)A_SLOT == (uint32_t)(A_BASE + SA * A_SLOT)
                                       ? (uint32_t)A_BASE
                                       : a_ld + (uint32_t)A_SLOT;
                        if constexpr (KFULL && BOOK == 1 && !SPLIT) ra.advance();
                    }
                }
            });
            if constexpr (nl > 0 && q >= OFF && (q - OFF) % T == 0 && (q - OFF) / T < nl) {
                constexpr int l = (q - OFF) / T;
                if constexpr (l < na) {
                    if constexpr (AK && !KFULL) opa.issue_one_masked(l, rsa, sa, wave, ma);
                    else opa.issue_one_full(l, rsa, sa, wave);
                } else {
                    if constexpr (BKC && !KFULL) opb.issue_one_masked(l - na, rsb, sb, wave, mb);
                    else opb.issue_one_full(l - na, rsb, sb, wave);
                }
            }
#pragma unroll
            for (int f = q * NF / NQ; f < (q + 1) * NF / NQ; ++f) {
                if (f < FN) fb[CUR ^ 1][f] = frb.template read<NEXT>(lds, f, RKS);
                else fa[CUR ^ 1][f - FN] = fra.template read<NEXT>(lds, f - FN, RKS);
            }
            __builtin_amdgcn_sched_barrier(0);
        });
    };
    using NoLd = std::integral_constant<int, 0>;
    using LdA = std::integral_constant<int, 1>;
    using LdB = std::integral_constant<int, 2>;
    using LdAB = std::integral_constant<int, 3>;

    // head(kt): K step 0 of stage kt, reading its K step 1 (split ring: and
    // loading stage kt+2's A tile); then the stage barrier.  tail(kt): K
    // step 1 of stage kt, reading K step 0 of stage kt+1 and loading stage
    // kt+S (split ring: its B tile) into the slots stage kt used.  At the
    // head's wait only the loads issued after stage kt+1's may be pending:
    // the (S-2) L of the later stages, or (split ring) the A loads of stage
    // kt+2 just issued.
    auto head = [&](int64_t kt) __attribute__((always_inline)) {
        if constexpr (SPLIT) {
            kstep(Z{}, std::false_type{}, O{}, LdA{}, Z{}, kt + 2, lds_base + a_ld, 0u);
            wait_vmcnt<PA>();           // this lane's loads of stage kt+1
        } else {
            kstep(Z{}, std::false_type{}, O{}, NoLd{}, Z{}, 0, 0u, 0u);
            wait_vmcnt<(S - 2) * L>();  // this lane's loads of stage kt+1
        }
        asm volatile("s_waitcnt lgkmcnt(0)" : : : "memory");   // reads of stage kt done
        barrier();
    };
    auto tail = [&](int64_t kt) __attribute__((always_inline)) {
        const uint32_t sb = lds_base + (uint32_t)(B_BASE + ((kt + S) & (S - 1)) * B_SLOT);
        if constexpr (SPLIT) {
            kstep(O{}, std::true_type{}, Z{}, LdB{}, O{}, kt + S, 0u, sb);
        } else {
            const uint32_t sa = lds_base + (uint32_t)(A_BASE + ((kt + S) & (S - 1)) * A_SLOT);
            kstep(O{}, std::true_type{}, Z{}, LdAB{}, O{}, kt + S, sa, sb);
        }
    };

    // Prologue: stages 0 .. S-1 whole.
#pragma unroll
    for (int st = 0; st < S; ++st) issue(st);
    wait_vmcnt<(S - 1) * L>();          // stage 0 resident for this lane
    barrier();                          // ... and for every lane
#pragma unroll
    for (int j = 0; j < FN; ++j) fb[0][j] = frb.template read<false>(lds, j, 0);
#pragma unroll
    for (int i = 0; i < FM; ++i) fa[0][i] = fra.template read<false>(lds, i, 0);

    head(0);
    for (int64_t kt = 0; kt + 1 < nk; ++kt) {
        tail(kt);
        head(kt + 1);
    }
    tail(nk - 1);

    // Drain the ring before the epilogue reuses the LDS.
    wait_vmcnt<0>();
    asm volatile("s_waitcnt lgkmcnt(0)" : : : "memory");
    barrier();

    // Split-K stages a whole fp32 tile in the ring, so only tiles that fit
    // take it (the planner splits no other).
    if constexpr (BM * BN * 4 <= S * SLOT * 16) {
        if (p.ksplit > 1) {
            if (p.out_f32)
                store_tile_splitk<float, BM, BN, WGM, WGN, S * SLOT * 16, 16>(p, acc, lds, tile, slice, b, m0, n0, wave, lane);
            else
                store_tile_splitk<TI, BM, BN, WGM, WGN, S * SLOT * 16, 16>(p, acc, lds, tile, slice, b, m0, n0, wave, lane);
            return;
        }
    }
    const bool full = p.c_vec && m0 + BM <= p.M && n0 + BN <= p.N;
    if (p.out_f32) {
        if (full)
            store_tile_lds<float, true, BM, BN, WGM, WGN, S * SLOT * 16, 16, EPI>(p, acc, lds, b, m0, n0, wave, lane);
        else
            store_tile_lds<float, false, BM, BN, WGM, WGN, S * SLOT * 16, 16, EPI>(p, acc, lds, b, m0, n0, wave, lane);
    } else {
        if (full)
            store_tile_lds<TI, true, BM, BN, WGM, WGN, S * SLOT * 16, 16, EPI>(p, acc, lds, b, m0, n0, wave, lane);
        else
            store_tile_lds<TI, false, BM, BN, WGM, WGN, S * SLOT * 16, 16, EPI>(p, acc, lds, b, m0, n0, wave, lane);
    }
}

// ---------------------------------------------------------------------------
// Streaming kernel for skinny problems (M <= 128) whose A and B are both
// K-contiguous (row-major A, column-major B: the linear-layer layout, with W
// stored N x K).  Such a GEMM is bound by reading B once from HBM
// ([OPS] §1.2 and [GEMM] §2.4: classify by arithmetic intensity first), so
// the kernel is built to keep many bytes in flight rather than to reuse tiles:
//   * a workgroup owns NB x 16 columns of C and MB blocks of 16 rows (all M
//     rows up to 64; from 33 rows on the 32 x 64 form also runs as several
//     row tiles) and splits K over its 8 waves, so even N = 4096 yields 256
//     workgroups;
//   * each wave streams its K range in batches of U steps of 32 (U = 2 for
//     48- and 64-column workgroups, else 4): the batch's B rows go straight to the
//     wave's own LDS region by direct-to-LDS loads, each load covering whole
//     128-byte lines of 16/U rows (a load shaped as one MFMA fragment, 16
//     rows x 64 bytes, touches twice the lines for the same bytes and
//     streamed HBM 8-20 % slower), and come back as fragments by
//     ds_read_b128; the next batch's loads are issued as soon as the
//     fragments are in registers, before this batch's MFMAs;
//   * with one 16-row block of A (M <= 16) its batch is staged the same way,
//     after B's in the wave's region (16 x 4096 x 4096: 9.6 us against 10.2
//     with A fragments loaded into registers); with more row blocks the A
//     fragments of v_mfma_f32_16x16x32_f16 (lane l: 8 consecutive k of row
//     l % 16, 16 contiguous bytes) are loaded from global memory into
//     registers.  A is small and stays in L2; each A fragment feeds NB
//     MFMAs.  The range check zero-fills rows >= M, columns >= N and
//     k >= K on both operands;
//   * the 8 partial tiles are summed through LDS and the alpha/beta epilogue
//     is applied once per output.
// ---------------------------------------------------------------------------
typedef float floatx4v __attribute__((ext_vector_type(4)));

template <typename TI, int MB, int NB, bool EPI>
__global__ __launch_bounds__(512) void gemm_stream(GemmArgs pin) {
    GemmArgs p = pin;
    if constexpr (!EPI) p.epi = 0;   // no epilogue code in this instantiation
    constexpr int NW = 8;
    // K steps (32 deep) per batch: a batch of B is NB*16 rows x U*64 bytes,
    // NB*U loads of 1 KiB, each covering 16/U whole rows of U*64 bytes.
    constexpr int U = NB >= 3 ? 2 : 4;
    constexpr int ROWB = U * 64;                 // bytes of one B row in a batch
    constexpr int CPR = ROWB / 16;               // 16-byte chunks per row
    constexpr int NLD = NB * U;                  // B loads per batch
    // With one row block, A's batch (16 rows) is staged the same way, after
    // B's in the wave's region; with more, A fragments go to registers.
    constexpr bool A_LDS = MB == 1;
    constexpr int NLA = A_LDS ? U : 0;           // A loads per batch
    constexpr int WAVE_BYTES = (NLD + NLA) * 1024;  // LDS of one wave's batch
    constexpr int RED_BYTES = NW * MB * 16 * NB * 16 * 4;
    // The split-K arrival flag sits after the reduction buffer.
    constexpr int LDS_BYTES = NW * WAVE_BYTES > RED_BYTES + 16 ? NW * WAVE_BYTES : RED_BYTES + 16;
    static_assert(LDS_BYTES <= 80 * 1024, "two workgroups per CU");
    __shared__ u32x4 lds_raw[LDS_BYTES / 16];
    auto red = reinterpret_cast<float (*)[MB * 16][NB * 16]>(lds_raw);
    int &s_last = *reinterpret_cast<int *>(reinterpret_cast<char *>(lds_raw) + RED_BYTES);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

    // With split-K, block id = slice * total_tiles + tile, and the slice's
    // K range is a multiple of 64 (A and B are K-contiguous here).
    const int slice = (int)(blockIdx.x / (unsigned)p.total_tiles);
    const int tile = (int)(blockIdx.x - (unsigned)slice * (unsigned)p.total_tiles);
    if (p.ksplit > 1) apply_k_slice(p, slice, true, true);
    int b, tm, tn;
    tile_coords(p, tile, b, tm, tn);
    const int64_t m0 = (int64_t)tm * (MB * 16), n0 = (int64_t)tn * (NB * 16);
    const uint16_t *Ab = p.A + b * p.sa;
    const uint16_t *Bb = p.B + b * p.sb;

    // K range of this wave, in steps of 32.
    const int64_t steps = (p.K + 31) / 32;
    const int64_t s_lo = steps * wave / NW, s_hi = steps * (wave + 1) / NW;

    const int r16 = lane & 15;            // row of A this lane loads
    const int kq = 8 * (lane >> 4);       // first of its 8 consecutive k
    // Descriptors based at the workgroup's first row of A and first column
    // of B, so that lane offsets span only MB*16 rows (NB*16 columns) of at
    // most 2^22 elements plus K: below 2^31 bytes however large N * ldb is.
    const int64_t a_base = m0 * p.lda, b_base = n0 * p.ldb;
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(Ab + a_base, (p.extent_a - a_base) * 2);
    [[maybe_unused]] const sgpr4 raw = make_rsrc_words(Ab + a_base, (p.extent_a - a_base) * 2);
    const sgpr4 rb = make_rsrc_words(Bb + b_base, (p.extent_b - b_base) * 2);
    bool a_ok[MB];
    uint32_t a_off[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
        const int64_t ml = mb * 16 + r16;   // row within the workgroup's rows
        a_ok[mb] = m0 + ml < p.M;
        a_off[mb] = (uint32_t)((ml * p.lda + kq) * 2);
    }
    // B rows (columns of the product) are staged in LDS: load j of a batch
    // brings rows j*16/U .. (j+1)*16/U - 1, lane t row j*16/U + t/CPR, its
    // 16-byte slot t%CPR holding chunk (slot ^ bswz(row)) of the row's batch
    // bytes, so that one load reads whole 128-byte lines of whole rows.  The
    // XOR makes the fragment reads (16 rows at one chunk per 16 lanes)
    // free of bank conflicts.
    auto bswz = [](int r) {
        if constexpr (U == 2) return swz16(r);                  // 8 chunks a row
        else return (r & 1) | ((r & 6) << 1);                   // 16 chunks a row
    };
    bool b_ok[NLD];
    uint32_t b_off[NLD];
    int b_k[NLD];                          // first k of the lane's chunk in the batch
#pragma unroll
    for (int j = 0; j < NLD; ++j) {
        const int r = j * (16 / U) + lane / CPR;
        const int c = (lane % CPR) ^ bswz(r & 15);
        b_ok[j] = n0 + r < p.N;
        b_k[j] = 8 * c;
        b_off[j] = (uint32_t)(((int64_t)r * p.ldb + 8 * c) * 2);
    }
    [[maybe_unused]] bool al_ok[NLA > 0 ? NLA : 1];
    [[maybe_unused]] uint32_t al_off[NLA > 0 ? NLA : 1];
    [[maybe_unused]] int al_k[NLA > 0 ? NLA : 1];
#pragma unroll
    for (int j = 0; j < NLA; ++j) {
        const int r = j * (16 / U) + lane / CPR;
        const int c = (lane % CPR) ^ bswz(r & 15);
        al_ok[j] = m0 + r < p.M;
        al_k[j] = 8 * c;
        al_off[j] = (uint32_t)(((int64_t)r * p.lda + 8 * c) * 2);
    }
    const uint32_t wave_lds = lds_offset(lds_raw) + (uint32_t)(wave * WAVE_BYTES);
    // Fragment (u, nb): row nb*16 + l%16, chunk 4u + l/16 of the batch.
    uint32_t frag_addr[U];
#pragma unroll
    for (int u = 0; u < U; ++u)
        frag_addr[u] = (uint32_t)(wave * WAVE_BYTES + r16 * ROWB + 16 * ((4 * u + (lane >> 4)) ^ bswz(r16)));

    floatx4v acc[MB][NB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) acc[mb][nb] = floatx4v{0.f, 0.f, 0.f, 0.f};

    // A fragments of the batch in flight.  With one row block (MB = 1)
    // they are double-buffered and issued with the batch's B loads; with
    // more, the next batch's A loads wait for this batch's MFMAs, so that
    // one set of fragment registers suffices (A comes from L2, whose latency
    // the B stream's hides).
    constexpr bool A_EARLY = MB == 1;
    [[maybe_unused]] half8 fa[U][MB];
    // A chunk of the batch starting at step s is loaded when its step is
    // below s_hi and its first k below K (both limits taken relative to s,
    // so that the per-lane tests are 32-bit).
    auto steps_left = [&](int64_t s) { return (int)(s_hi - s < U ? s_hi - s : U); };
    auto k_left = [&](int64_t s) { return (int)(p.K - s * 32 < 32 * U ? p.K - s * 32 : 32 * U); };
    auto issue_b = [&](int64_t s) __attribute__((always_inline)) {
        const uint32_t kb = (uint32_t)(s * 64);
        const int sl = steps_left(s), kl = k_left(s);
#pragma unroll
        for (int j = 0; j < NLD; ++j) {
            const bool in = b_k[j] < 32 * sl && b_k[j] < kl;
            lds_dma16(rb, wave_lds + (uint32_t)(j * 1024), (b_ok[j] && in) ? b_off[j] + kb : kOutOfRange);
        }
    };
    auto issue_a = [&](int64_t s) __attribute__((always_inline)) {
        const uint32_t kb = (uint32_t)(s * 64);
        const int sl = steps_left(s), kl = k_left(s);
        if constexpr (A_LDS) {
#pragma unroll
            for (int j = 0; j < NLA; ++j) {
                const bool in = al_k[j] < 32 * sl && al_k[j] < kl;
                lds_dma16(raw, wave_lds + (uint32_t)((NLD + j) * 1024),
                          (al_ok[j] && in) ? al_off[j] + kb : kOutOfRange);
            }
            return;
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const bool kin = u < sl && 32 * u + kq < kl;
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
                fa[u][mb] = __builtin_bit_cast(half8, __builtin_amdgcn_raw_buffer_load_b128(
                    ra, (a_ok[mb] && kin) ? a_off[mb] + kb + (uint32_t)(u * 64) : kOutOfRange, 0, 0));
        }
    };

    if (s_lo < s_hi) {
        issue_b(s_lo);
        issue_a(s_lo);
    }
    for (int64_t s0 = s_lo; s0 < s_hi; s0 += U) {
        // The batch's loads (the only ones outstanding) have landed.  The
        // empty statement naming its A fragments is their first use: the
        // compiler's own wait for them goes here, not after the next batch's
        // B loads.  With early A loads the fragments move to fc, freeing fa.
        asm volatile("s_waitcnt vmcnt(0)" : : : "memory");
        half8 fb[U][NB], fc[U][MB];
        const char *base = (const char *)lds_raw;
        if constexpr (A_LDS) {
#pragma unroll
            for (int u = 0; u < U; ++u) fc[u][0] = *(const half8 *)(base + frag_addr[u] + NLD * 1024);
        } else {
#pragma unroll
            for (int u = 0; u < U; ++u)
#pragma unroll
                for (int mb = 0; mb < MB; ++mb) {
                    asm volatile("" : "+v"(fa[u][mb]));
                    fc[u][mb] = fa[u][mb];
                }
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
                fb[u][nb] = *(const half8 *)(base + frag_addr[u] + nb * 16 * ROWB);
        // The region is free once its fragments are in registers: the next
        // batch's B loads go out before this batch's MFMAs.
        asm volatile("s_waitcnt lgkmcnt(0)" : : : "memory");
        const bool more = s0 + U < s_hi;
        if (more) {
            issue_b(s0 + U);
            if constexpr (A_EARLY) issue_a(s0 + U);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                for (int nb = 0; nb < NB; ++nb)
                    acc[mb][nb] = mfma16<TI>(A_EARLY ? fc[u][mb] : fa[u][mb], fb[u][nb], acc[mb][nb]);
        if constexpr (!A_EARLY) {
            __builtin_amdgcn_sched_barrier(0);
            if (more) issue_a(s0 + U);
        }
    }
    // Every wave is done with its LDS region before the reduction reuses it.
    __syncthreads();

    // Accumulator register r of lane l holds row 4*(l/16) + r, column l % 16
    // of each 16 x 16 block.
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                red[wave][mb * 16 + 4 * (lane >> 4) + r][nb * 16 + r16] = acc[mb][nb][r];
    __syncthreads();

    const float alpha = p.alpha, beta = p.beta;
    constexpr int TE = MB * 16 * NB * 16;   // outputs of the block
    if (p.ksplit > 1) {
        // Split-K: the block's fp32 partial (its waves summed in order) goes
        // to the workspace, slice-major, by the ordering rules of the direct
        // kernels' split-K (stores written through to memory and loads that
        // miss the L2, so slices may run on different XCDs; the device-scope
        // counter orders them); the last slice to arrive sums the partials
        // in slice order and applies the epilogue.
        constexpr int kCoherent = 1 | 16;
        const __amdgpu_buffer_rsrc_t rws = make_rsrc(p.ws, (int64_t)p.ksplit * p.total_tiles * TE * 4);
        const uint32_t mine = (uint32_t)(((int64_t)slice * p.total_tiles + tile) * TE * 4);
        for (int o = tid; o < TE; o += NW * 64) {
            const int i = o / (NB * 16), j = o % (NB * 16);
            float v = 0.f;
#pragma unroll
            for (int w = 0; w < NW; ++w) v += red[w][i][j];
            __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), rws,
                                                  mine + (uint32_t)(o * 4), 0, kCoherent);
        }
        asm volatile("s_waitcnt vmcnt(0)" : : : "memory");   // this lane's partial is in memory
        __syncthreads();
        if (tid == 0)
            s_last = __hip_atomic_fetch_add(&p.ws_count[tile], 1, __ATOMIC_RELAXED,
                                            __HIP_MEMORY_SCOPE_AGENT) == p.ksplit - 1;
        __syncthreads();
        if (!s_last) return;
        constexpr int KSMAX = 8;
        const uint32_t tile0 = (uint32_t)((int64_t)tile * TE * 4);
        const uint32_t slice_stride = (uint32_t)((int64_t)p.total_tiles * TE * 4);
        for (int o = tid; o < TE; o += NW * 64) {
            const int i = o / (NB * 16), j = o % (NB * 16);
            float part[KSMAX];
#pragma unroll
            for (int sl = 0; sl < KSMAX; ++sl)
                part[sl] = sl < p.ksplit
                    ? __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                          rws, tile0 + (uint32_t)sl * slice_stride + (uint32_t)(o * 4), 0, kCoherent))
                    : 0.0f;
            float v = part[0];
#pragma unroll
            for (int sl = 1; sl < KSMAX; ++sl)
                if (sl < p.ksplit) v += part[sl];
            const int64_t m = m0 + i, nn = n0 + j;
            if (m >= p.M || nn >= p.N) continue;
            v *= alpha;
            const int64_t off = b * p.sc + m * p.ldc + nn;
            if (p.out_f32) {
                float *C = (float *)p.C + off;
                if (beta != 0.0f) v += beta * *C;
                if (p.epi) v = activate(p.act, p.bias ? v + p.bias[nn] : v);
                *C = v;
            } else {
                TI *C = (TI *)p.C + off;
                if (beta != 0.0f) v += beta * (float)*C;
                if (p.epi) v = activate(p.act, p.bias ? v + p.bias[nn] : v);
                *C = (TI)v;
            }
        }
        if (tid == 0)
            __hip_atomic_store(&p.ws_count[tile], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return;
    }
    for (int o = tid; o < MB * 16 * NB * 16; o += NW * 64) {
        const int i = o / (NB * 16), j = o % (NB * 16);
        const int64_t m = m0 + i, nn = n0 + j;
        if (m >= p.M || nn >= p.N) continue;
        float v = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) v += red[w][i][j];
        v *= alpha;
        const int64_t off = b * p.sc + m * p.ldc + nn;
        if (p.out_f32) {
            float *C = (float *)p.C + off;
            if (beta != 0.0f) v += beta * *C;
            if (p.epi) v = activate(p.act, p.bias ? v + p.bias[nn] : v);
            *C = v;
        } else {
            TI *C = (TI *)p.C + off;
            if (beta != 0.0f) v += beta * (float)*C;
            if (p.epi) v = activate(p.act, p.bias ? v + p.bias[nn] : v);
            *C = (TI)v;
        }
    }
}

// ---------------------------------------------------------------------------
// Row-vector kernel: M <= 4 with row-major A and B (B N-contiguous, the NN
// layout of a matrix-vector product).  Such a product is bound by reading B
// once ([OPS] §1.2, [GEMM] §2.4), and with at most 4 rows of A an MFMA tile
// would be almost all padding, so B is streamed into registers and the dot
// products are fp32 FMAs:
//   * a workgroup owns 64 columns of C (all M rows) and K (or its K slice);
//     each of its 8 waves takes 128 rows of B per round of 1024;
//   * lane t reads 16 consecutive rows (16 (t / 8) + j) at columns
//     8 (t % 8) .. + 7: every load instruction covers 8 rows x 128 bytes,
//     whole lines, and the lane's 16 values of each A row are two 16-byte
//     loads (A is tiny and stays in L1/L2);
//   * the 8 lanes that share columns are summed by lane exchanges, the 8
//     waves through LDS in wave order; split-K partials as in the streaming
//     kernel (the last slice to arrive sums them in slice order).
// ---------------------------------------------------------------------------
// ---------------------------------------------------------------------------
// Batched small products (M, N, K <= 64; A and B row-major): one wave per
// product.  Such products are bound by moving their operands ([GEMM] §2.4,
// [CATLASS] §3.1); with the staged tile's four waves per product, a batch of
// 512 spent about a fifth of its time having its waves dispatched, and the
// waves of one product wait for each other at every barrier.  Here:
//   * A's fragments of v_mfma_f32_16x16x32 (lane l: row l % 16 of a 16-row
//     block, 8 consecutive k from 8 (l / 16)) are 16 contiguous bytes of a
//     row of A, loaded straight into registers, 8 per lane;
//   * B (rows of k, N-contiguous) goes to LDS by 16-byte loads, 8 per lane,
//     issued with A's, and comes back transposed by ds_read_b64_tr_b16, two
//     reads per fragment (lane j of a 16-lane group addresses row k0 + j / 4
//     at column n0 + 4 (j % 4); lane i receives column n0 + i of rows
//     k0 .. k0 + 3);
//   * the wave accumulates C^T (B's fragment as the first operand), so each
//     lane ends with runs of 4 consecutive n of one row of C, stored as one
//     vector each.
// Rows past M, chunks past K and chunks past N read zeros (range check on
// each 8-element chunk; K and N are multiples of 8, or the operands are
// padded copies whose padding is zero).
template <typename TI, bool EPI>
__global__ __launch_bounds__(64) void gemm_small64(GemmArgs pin) {
    GemmArgs p = pin;
    if constexpr (!EPI) p.epi = 0;   // no epilogue code in this instantiation
    __shared__ u32x4 bl[64 * 8];     // B: 64 rows of k, 8 chunks of 8 n
    const int lane = threadIdx.x;
    const int64_t b = blockIdx.x;    // one tile per product: the batch item
    const uint16_t *Ab = p.A + b * p.sa;
    const uint16_t *Bb = p.B + b * p.sb;
    // extent_a / extent_b: elements of one batch item reachable from its base.
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(Ab, p.extent_a * 2);
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(Bb, p.extent_b * 2);
    const int li = lane & 15, g = lane >> 4;

    // B chunk q of this lane: row 8 q + lane / 8, columns 8 (lane % 8) .. + 7.
    u32x4 bv[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        const int row = 8 * q + (lane >> 3), c = lane & 7;
        const bool ok = row < p.K && 8 * c < p.N;
        bv[q] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                    rb, ok ? (uint32_t)(((int64_t)row * p.ldb + 8 * c) * 2) : kOutOfRange, 0, 0));
    }
    // A fragment (mb, ks): row 16 mb + l % 16, k = 32 ks + 8 (l / 16) .. + 7.
    half8 af[4][2];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const int row = 16 * mb + li, k = 32 * ks + 8 * g;
            const bool ok = row < p.M && k < p.K;
            af[mb][ks] = __builtin_bit_cast(half8, __builtin_amdgcn_raw_buffer_load_b128(
                             ra, ok ? (uint32_t)(((int64_t)row * p.lda + k) * 2) : kOutOfRange, 0, 0));
        }
#pragma unroll
    for (int q = 0; q < 8; ++q) bl[(8 * q + (lane >> 3)) * 8 + (lane & 7)] = bv[q];
    __syncthreads();

    floatx4 acc[4][4];   // [nb][mb]
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) acc[nb][mb] = floatx4{0.f, 0.f, 0.f, 0.f};
    const char *lb = (const char *)bl;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
            // Columns 16 nb + l % 16 of rows 32 ks + 8 g .. + 7.
            v4i16 hv[2];
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const int row = 32 * ks + 8 * g + 4 * t + (li >> 2);
                hv[t] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (__attribute__((address_space(3))) v4i16 *)(const void *)(lb + row * 128 + 32 * nb +
                                                                               8 * (li & 3)));
            }
            const half8 bf = __builtin_bit_cast(half8, __builtin_shufflevector(hv[0], hv[1], 0, 1, 2, 3,
                                                                               4, 5, 6, 7));
#pragma unroll
            for (int mb = 0; mb < 4; ++mb) acc[nb][mb] = mfma16<TI>(bf, af[mb][ks], acc[nb][mb]);
        }

    // acc[nb][mb][r] = C(16 mb + l % 16, 16 nb + 4 (l / 16) + r).
    const float alpha = p.alpha, beta = p.beta;
    const bool epi = EPI && p.epi;
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
        const int64_t m = 16 * mb + li;
        if (m >= p.M) continue;
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
            const int64_t n = 16 * nb + 4 * g;
            if (n >= p.N) continue;
            const int64_t off = b * p.sc + m * p.ldc + n;
            const int64_t left = p.N - n;
            const bool full = p.c_vec && left >= 4;
            floatx4 v = acc[nb][mb] * alpha;
            if (beta != 0.0f) {
                const floatx4 c = p.out_f32 ? read_c4((const float *)p.C + off, full, left)
                                            : read_c4((const TI *)p.C + off, full, left);
                v += beta * c;
            }
            if (epi) v = epilogue4(p, v, load_bias4(p, n));
            if (p.out_f32) write_c4((float *)p.C + off, full, left, v);
            else write_c4((TI *)p.C + off, full, left, v);
        }
    }
}

template <typename TI>
__device__ inline float elem_f32(uint32_t w, int hi) {
    const uint32_t h = hi ? (w >> 16) : (w & 0xffffu);
    if constexpr (std::is_same<TI, __bf16>::value) return __builtin_bit_cast(float, h << 16);
    else return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}

template <typename TI, int MB, int NB, bool EPI>
__global__ __launch_bounds__(512) void gemm_rowvec(GemmArgs pin) {
    GemmArgs p = pin;
    if constexpr (!EPI) p.epi = 0;
    constexpr int MR = 4, NW = 8, COLS = 64;
    static_assert(MB == 1 && NB == 4, "4 rows x 64 columns");
    __shared__ float red[NW][MR][COLS];
    __shared__ int s_last;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

    const int slice = (int)(blockIdx.x / (unsigned)p.total_tiles);
    const int tile = (int)(blockIdx.x - (unsigned)slice * (unsigned)p.total_tiles);
    if (p.ksplit > 1) apply_k_slice(p, slice, true, false);
    int b, tm, tn;
    tile_coords(p, tile, b, tm, tn);
    const int64_t n0 = (int64_t)tn * COLS;
    const uint16_t *Ab = p.A + b * p.sa;
    const uint16_t *Bb = p.B + b * p.sb;
    // B's descriptor starts at the workgroup's first column (offsets span
    // K rows of ldb elements: below 2^31 bytes for the ld limit and K).
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(Bb + n0, (p.extent_b - n0) * 2);
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(Ab, p.extent_a * 2);

    const int cg = lane & 7, rg = lane >> 3;            // column group, row group
    const bool col_ok = n0 + 8 * cg < p.N;
    float acc[MR][8];
#pragma unroll
    for (int m = 0; m < MR; ++m)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[m][e] = 0.f;

    for (int64_t k0 = (int64_t)wave * 128; k0 < p.K; k0 += NW * 128) {
        const int64_t kr = k0 + 16 * rg;                // this lane's first row
        u32x4 bv[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const bool ok = col_ok && kr + j < p.K;
            bv[j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                rb, ok ? (uint32_t)(((kr + j) * p.ldb + 8 * cg) * 2) : kOutOfRange, 0, 0));
        }
        u32x4 av[MR][2];
#pragma unroll
        for (int m = 0; m < MR; ++m)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                // Rows of A are 16-byte aligned and K a multiple of 8 here,
                // so an 8-element chunk is wholly inside or outside K.
                const bool ok = m < p.M && kr + 8 * h < p.K;
                av[m][h] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                    ra, ok ? (uint32_t)((m * p.lda + kr + 8 * h) * 2) : kOutOfRange, 0, 0));
            }
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            float bf[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) bf[e] = elem_f32<TI>(bv[j][e >> 1], e & 1);
#pragma unroll
            for (int m = 0; m < MR; ++m) {
                const float a = elem_f32<TI>(av[m][j >> 3][(j & 7) >> 1], j & 1);
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[m][e] = __builtin_fmaf(a, bf[e], acc[m][e]);
            }
        }
    }

    // Lanes t, t ^ 8, t ^ 16, ... share columns: fixed-order pairwise sums.
#pragma unroll
    for (int m = 0; m < MR; ++m)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float v = acc[m][e];
            v += __shfl_xor(v, 8);
            v += __shfl_xor(v, 16);
            v += __shfl_xor(v, 32);
            acc[m][e] = v;
        }
    if (rg == 0) {
#pragma unroll
        for (int m = 0; m < MR; ++m)
#pragma unroll
            for (int e = 0; e < 8; ++e) red[wave][m][8 * cg + e] = acc[m][e];
    }
    __syncthreads();

    // Thread o < 256 owns output (o / 64, o % 64): its sum over the waves.
    const int o = tid, om = o >> 6, oc = o & 63;
    float v = 0.f;
    if (o < MR * COLS) {
#pragma unroll
        for (int w = 0; w < NW; ++w) v += red[w][om][oc];
    }
    const int64_t nn = n0 + oc;
    const float alpha = p.alpha, beta = p.beta;
    constexpr int TE = MR * COLS;
    if (p.ksplit > 1) {
        constexpr int kCoherent = 1 | 16;
        const __amdgpu_buffer_rsrc_t rws = make_rsrc(p.ws, (int64_t)p.ksplit * p.total_tiles * TE * 4);
        if (o < TE)
            __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), rws,
                                                  (uint32_t)((((int64_t)slice * p.total_tiles + tile) * TE + o) * 4),
                                                  0, kCoherent);
        asm volatile("s_waitcnt vmcnt(0)" : : : "memory");   // this lane's partial is in memory
        __syncthreads();
        if (tid == 0)
            s_last = __hip_atomic_fetch_add(&p.ws_count[tile], 1, __ATOMIC_RELAXED,
                                            __HIP_MEMORY_SCOPE_AGENT) == p.ksplit - 1;
        __syncthreads();
        if (!s_last) return;
        constexpr int KSMAX = 8;
        float part[KSMAX];
#pragma unroll
        for (int sl = 0; sl < KSMAX; ++sl)
            part[sl] = (sl < p.ksplit && o < TE)
                ? __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                      rws, (uint32_t)((((int64_t)sl * p.total_tiles + tile) * TE + o) * 4), 0, kCoherent))
                : 0.0f;
        v = part[0];
#pragma unroll
        for (int sl = 1; sl < KSMAX; ++sl)
            if (sl < p.ksplit) v += part[sl];
        if (tid == 0)
            __hip_atomic_store(&p.ws_count[tile], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    if (o >= TE || om >= p.M || nn >= p.N) return;
    v *= alpha;
    const int64_t off = b * p.sc + om * p.ldc + nn;
    if (p.out_f32) {
        float *C = (float *)p.C + off;
        if (beta != 0.0f) v += beta * *C;
        if (p.epi) v = activate(p.act, p.bias ? v + p.bias[nn] : v);
        *C = v;
    } else {
        TI *C = (TI *)p.C + off;
        if (beta != 0.0f) v += beta * (float)*C;
        if (p.epi) v = activate(p.act, p.bias ? v + p.bias[nn] : v);
        *C = (TI)v;
    }
}

#if MPGEMM_HOST_PART
// ---------------------------------------------------------------------------
// Repacking of an operand whose rows are not 16-byte aligned ([GEMM] §3.4:
// edges are handled by zero padding).  Copies `outer` rows of `cols`
// elements (leading dimension ld, batch stride `stride`, any 2-byte
// alignment) into a dense buffer of rows ld8 = cols rounded up to 8, zeros in
// columns cols..ld8-1, so that the direct and streaming kernels can read
// every row as whole 16-byte chunks.  One thread writes one 16-byte chunk: it
// reads the one or two 16-byte-aligned source blocks that hold the chunk's
// valid elements (never a block without one, so every read stays inside the
// pages of the operand) and shifts them into place.  HBM bound: the operand
// is read once and written once.
// ---------------------------------------------------------------------------
struct PackOperand {
    const uint16_t *src;
    uint16_t *dst;
    int64_t ld, stride, outer, cols, ld8;
    uint32_t chunks;   // batch * outer * ld8 / 8
};
struct PackArgs {
    PackOperand op[2];   // op[1].chunks == 0 when only one operand is copied
};

// Copies chunk c of one operand (see above).
__device__ inline void pack_chunk(const PackOperand &a, uint32_t c) {
    const uint32_t cpr = (uint32_t)(a.ld8 / 8);     // chunks per packed row
    const uint32_t outer = (uint32_t)a.outer;
    const uint32_t j = c % cpr, row = c / cpr;      // row over all batch items
    const uint32_t b = row / outer, r = row - b * outer;
    const int64_t left = a.cols - 8 * (int64_t)j;
    const int nvalid = left >= 8 ? 8 : (int)left;   // >= 1: j < ceil(cols / 8)
    const uintptr_t first = (uintptr_t)(a.src + (int64_t)b * a.stride + (int64_t)r * a.ld + 8 * (int64_t)j);
    const uintptr_t blk = first & ~(uintptr_t)15;
    const int sh = (int)(first & 15);                // even: fp16 elements
    const u32x4 w0 = *(const u32x4 *)blk;
    // The second block holds a valid element only if the chunk's valid bytes
    // run past the first.
    const u32x4 w1 = sh + 2 * nvalid > 16 ? *(const u32x4 *)(blk + 16) : u32x4{0, 0, 0, 0};
    const int s4 = sh >> 2, sb = sh & 3;
    uint32_t e[5];
    // e[i] = dword s4 + i of the 8-dword window w0:w1.
#pragma unroll
    for (int i = 0; i < 5; ++i) {
        const int k = s4 + i;
        e[i] = k == 0 ? w0[0] : k == 1 ? w0[1] : k == 2 ? w0[2] : k == 3 ? w0[3]
             : k == 4 ? w1[0] : k == 5 ? w1[1] : k == 6 ? w1[2] : w1[3];
    }
    u32x4 out;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        uint32_t v = __builtin_amdgcn_alignbyte(e[i + 1], e[i], (uint32_t)sb);
        if (2 * i >= nvalid) v = 0;
        else if (2 * i + 1 >= nvalid) v &= 0xffffu;
        out[i] = v;
    }
    *(u32x4 *)(a.dst + (int64_t)row * a.ld8 + 8 * (int64_t)j) = out;
}

// One launch copies one or both operands: chunks [0, op[0].chunks) of A (or
// B), then op[1]'s.  Chunk counts sum below 2^31 (checked by the planner and
// the launcher): 32-bit index math, and c + grid stride stays below 2^32.
__global__ __launch_bounds__(256) void gemm_pack16(PackArgs a) {
    const uint32_t n0 = a.op[0].chunks, total = n0 + a.op[1].chunks;
    for (uint32_t c = blockIdx.x * 256u + threadIdx.x; c < total; c += gridDim.x * 256u) {
        if (c < n0) pack_chunk(a.op[0], c);
        else pack_chunk(a.op[1], c - n0);
    }
}

#endif  // MPGEMM_HOST_PART

template <typename TI, bool EPI, int T, bool AK, bool BKC, bool VEC>
constexpr KernelFn pick_staged() {
    return gemm_staged<TI, kTiles[T].bm, kTiles[T].bn, kTiles[T].bk, kTiles[T].wgm,
                       kTiles[T].wgn, AK, BKC, VEC, EPI>;
}

template <typename TI, bool EPI, int T, bool AK, bool BKC, bool KFULL = false>
constexpr KernelFn pick_direct16() {
    return gemm_direct16<TI, kTiles[T].bm, kTiles[T].bn, kTiles[T].bk, kTiles[T].wgm,
                         kTiles[T].wgn, kTiles[T].stages, AK, BKC, KFULL, EPI>;
}

// Kernel table indexed [input type][fused epilogue][tile][A K-contiguous]
// [B K-contiguous][vec].  Direct tiles have only the vec entry; staged tiles
// have both.
template <typename TI, bool EPI, int T>
void fill_tile(KernelFn (&t)[2][2][2]) {
    if constexpr (kTiles[T].kind == KIND_DIRECT16) {
        t[0][0][1] = pick_direct16<TI, EPI, T, false, false>();
        t[0][1][1] = pick_direct16<TI, EPI, T, false, true>();
        t[1][0][1] = pick_direct16<TI, EPI, T, true, false>();
        t[1][1][1] = pick_direct16<TI, EPI, T, true, true>();
        t[0][0][0] = t[0][1][0] = t[1][0][0] = t[1][1][0] = nullptr;
    } else {
        t[0][0][0] = pick_staged<TI, EPI, T, false, false, false>();
        t[0][0][1] = pick_staged<TI, EPI, T, false, false, true>();
        t[0][1][0] = pick_staged<TI, EPI, T, false, true, false>();
        t[0][1][1] = pick_staged<TI, EPI, T, false, true, true>();
        t[1][0][0] = pick_staged<TI, EPI, T, true, false, false>();
        t[1][0][1] = pick_staged<TI, EPI, T, true, false, true>();
        t[1][1][0] = pick_staged<TI, EPI, T, true, true, false>();
        t[1][1][1] = pick_staged<TI, EPI, T, true, true, true>();
    }
}

template <typename TI, bool EPI, int T>
void fill_kfull(KernelFn (&t)[2][2]) {
    static_assert(kTiles[T].kind == KIND_DIRECT16, "K-full variants are direct16");
    t[0][0] = pick_direct16<TI, EPI, T, false, false, true>();
    t[0][1] = pick_direct16<TI, EPI, T, false, true, true>();
    t[1][0] = pick_direct16<TI, EPI, T, true, false, true>();
    t[1][1] = pick_direct16<TI, EPI, T, true, true, true>();
}

template <typename TI, bool EPI, int T>
void fill_stream(KernelFn (&t)[2][2][2]) {
    // Only the K-contiguous A and B (row-major A, column-major B) 128-bit form.
    t[0][0][0] = t[0][0][1] = t[0][1][0] = t[0][1][1] = nullptr;
    t[1][0][0] = t[1][0][1] = t[1][1][0] = nullptr;
    t[1][1][1] = gemm_stream<TI, kTiles[T].bm / 16, kTiles[T].bn / 16, EPI>;
}

template <typename TI, bool EPI, int T>
void fill_rowvec(KernelFn (&t)[2][2][2]) {
    // Only row-major A and B (A K-contiguous, B N-contiguous), 128-bit form.
    t[0][0][0] = t[0][0][1] = t[0][1][0] = t[0][1][1] = nullptr;
    t[1][0][0] = t[1][1][0] = t[1][1][1] = nullptr;
    t[1][0][1] = gemm_rowvec<TI, kTiles[T].bm / 4, kTiles[T].bn / 16, EPI>;
}

template <typename TI, bool EPI>
void fill_small(KernelFn (&t)[2][2][2]) {
    // Only row-major A and B, 128-bit form.
    t[0][0][0] = t[0][0][1] = t[0][1][0] = t[0][1][1] = nullptr;
    t[1][0][0] = t[1][1][0] = t[1][1][1] = nullptr;
    t[1][0][1] = gemm_small64<TI, EPI>;
}

template <typename TI, bool EPI>
void fill_type(TileKernels &k, FullKernels &kfull) {
    for (auto &t : kfull)
        t[0][0] = t[0][1] = t[1][0] = t[1][1] = nullptr;
    fill_kfull<TI, EPI, TILE_256x256>(kfull[TILE_256x256]);
    fill_kfull<TI, EPI, TILE_128x128>(kfull[TILE_128x128]);
    fill_kfull<TI, EPI, TILE_128x128_D4>(kfull[TILE_128x128_D4]);
    fill_tile<TI, EPI, TILE_256x256>(k[TILE_256x256]);
    fill_tile<TI, EPI, TILE_128x128>(k[TILE_128x128]);
    fill_tile<TI, EPI, TILE_128x128_D4>(k[TILE_128x128_D4]);
    fill_tile<TI, EPI, TILE_64x64>(k[TILE_64x64]);
    fill_tile<TI, EPI, TILE_32x64>(k[TILE_32x64]);
    fill_tile<TI, EPI, TILE_128x128_STAGED>(k[TILE_128x128_STAGED]);
    fill_stream<TI, EPI, TILE_STREAM16>(k[TILE_STREAM16]);
    fill_stream<TI, EPI, TILE_STREAM32>(k[TILE_STREAM32]);
    fill_stream<TI, EPI, TILE_STREAM64>(k[TILE_STREAM64]);
    fill_stream<TI, EPI, TILE_STREAM32W>(k[TILE_STREAM32W]);
    fill_stream<TI, EPI, TILE_STREAM16W>(k[TILE_STREAM16W]);
    fill_stream<TI, EPI, TILE_STREAM32N>(k[TILE_STREAM32N]);
    fill_small<TI, EPI>(k[TILE_SMALL64]);
    fill_rowvec<TI, EPI, TILE_ROWVEC>(k[TILE_ROWVEC]);
}

}  // namespace

#if MPGEMM_PART < 0 || MPGEMM_PART == 1
void mpgemm::fill_kernels_f16_plain(TileKernels &k, FullKernels &kfull) { fill_type<_Float16, false>(k, kfull); }
#endif
#if MPGEMM_PART < 0 || MPGEMM_PART == 2
void mpgemm::fill_kernels_f16_epi(TileKernels &k, FullKernels &kfull) { fill_type<_Float16, true>(k, kfull); }
#endif
#if MPGEMM_PART < 0 || MPGEMM_PART == 3
void mpgemm::fill_kernels_bf16_plain(TileKernels &k, FullKernels &kfull) { fill_type<__bf16, false>(k, kfull); }
#endif
#if MPGEMM_PART < 0 || MPGEMM_PART == 4
void mpgemm::fill_kernels_bf16_epi(TileKernels &k, FullKernels &kfull) { fill_type<__bf16, true>(k, kfull); }
#endif

#if MPGEMM_HOST_PART
namespace {

struct KernelTable {
    KernelFn k[2][2][NUM_TILES][2][2][2];    // [input type][epilogue][tile][A][B][vec]
    KernelFn kfull[2][2][NUM_TILES][2][2];   // direct tiles with K a multiple of BK (else null)
    KernelTable() {
        fill_kernels_f16_plain(k[IN_F16][0], kfull[IN_F16][0]);
        fill_kernels_f16_epi(k[IN_F16][1], kfull[IN_F16][1]);
        fill_kernels_bf16_plain(k[IN_BF16][0], kfull[IN_BF16][0]);
        fill_kernels_bf16_epi(k[IN_BF16][1], kfull[IN_BF16][1]);
    }
};

const KernelTable &kernels() {
    static const KernelTable t;
    return t;
}

bool ranges_overlap(uintptr_t a, int64_t a_bytes, uintptr_t b, int64_t b_bytes) {
    if (a_bytes <= 0 || b_bytes <= 0) return false;
    return a < b + (uintptr_t)b_bytes && b < a + (uintptr_t)a_bytes;
}

// ---------------------------------------------------------------------------
// The row pass of the linear layer fused with its residual and LayerNorm
// ([CATLASS] opening paragraph: the case the page's author was tuning; §3:
// the matrix product in fp16 with fp32 accumulation, the normalisation's
// reductions in fp32).  The GEMM kernels write Z = alpha A B in fp32 into the
// workspace (no rounding in between); one workgroup per row then forms
// x = Z + beta C + bias, its mean and (biased) variance over the N columns by
// two passes over the values it holds in registers, and writes
// (x - mean) / sqrt(var + eps) * gamma + beta_ln into C.  Rows longer than
// 16384 are read three times instead (the second and third reads hit the L2).
// ---------------------------------------------------------------------------
template <typename T>
__device__ inline float load_c_elem(const void *C, int64_t i) { return (float)((const T *)C)[i]; }
template <typename T>
__device__ inline void store_c_elem(void *C, int64_t i, float v) { ((T *)C)[i] = (T)v; }

// Sum over the 256 threads of a workgroup (red: 4 floats of LDS).
__device__ inline float block_sum256(float v, float *red) {
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
    __syncthreads();
    const float t = red[0] + red[1] + red[2] + red[3];
    __syncthreads();
    return t;
}

// VEC: N, ldc and C's batch stride multiples of 4, and C, gamma, beta_ln and
// the bias 16-byte aligned (C 8-byte for 16-bit types): each thread then owns
// runs of four consecutive columns, read and written as one vector each
// (element-wide accesses held the row pass to about 2 TB/s).
template <int VPT, typename T, bool VEC>
__global__ __launch_bounds__(256) void gemm_layernorm_rows(LayerNormArgs a) {
    __shared__ float red[4];
    const int64_t r = blockIdx.x;
    const int64_t b = r / a.M, i = r - b * a.M;
    const float *z = a.Z + b * a.sz + i * a.ldz;
    const int64_t cbase = b * a.sc + i * a.ldc;
    const int t = threadIdx.x;
    const float invn = 1.0f / (float)a.N;
    if constexpr (VEC) {
        static_assert(VPT % 4 == 0 && VPT > 0, "runs of four");
        constexpr int G = VPT / 4;
        floatx4 x[G];
        float s = 0.f;
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const int64_t j = ((int64_t)g * 256 + t) * 4;
            x[g] = floatx4{0.f, 0.f, 0.f, 0.f};
            if (j < a.N) {
                x[g] = *(const floatx4 *)(z + j);
                if (a.beta != 0.0f) {
                    const c4_t<T> c = *(const c4_t<T> *)((const T *)a.C + cbase + j);
#pragma unroll
                    for (int e = 0; e < 4; ++e) x[g][e] += a.beta * (float)c[e];
                }
                if (a.bias) x[g] += *(const floatx4 *)(a.bias + j);
            }
            s += (x[g][0] + x[g][1]) + (x[g][2] + x[g][3]);
        }
        const float mean = block_sum256(s, red) * invn;
        float q = 0.f;
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const int64_t j = ((int64_t)g * 256 + t) * 4;
            if (j < a.N) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float d = x[g][e] - mean;
                    q += d * d;
                }
            }
        }
        const float rs = 1.0f / sqrtf(block_sum256(q, red) * invn + a.eps);
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const int64_t j = ((int64_t)g * 256 + t) * 4;
            if (j < a.N) {
                const floatx4 gm = *(const floatx4 *)(a.gamma + j), bt = *(const floatx4 *)(a.beta_ln + j);
                c4_t<T> y;
#pragma unroll
                for (int e = 0; e < 4; ++e) y[e] = (T)((x[g][e] - mean) * rs * gm[e] + bt[e]);
                *(c4_t<T> *)((T *)a.C + cbase + j) = y;
            }
        }
        return;
    }
    auto input = [&](int64_t j) __attribute__((always_inline)) {
        float x = z[j];
        if (a.beta != 0.0f) x += a.beta * load_c_elem<T>(a.C, cbase + j);
        if (a.bias) x += a.bias[j];
        return x;
    };
    if constexpr (VPT > 0 && !VEC) {
        float x[VPT];
        float s = 0.f;
#pragma unroll
        for (int v = 0; v < VPT; ++v) {
            const int64_t j = (int64_t)v * 256 + t;
            x[v] = j < a.N ? input(j) : 0.f;
            s += x[v];
        }
        const float mean = block_sum256(s, red) * invn;
        float q = 0.f;
#pragma unroll
        for (int v = 0; v < VPT; ++v) {
            const int64_t j = (int64_t)v * 256 + t;
            const float d = x[v] - mean;
            if (j < a.N) q += d * d;
        }
        const float rs = 1.0f / sqrtf(block_sum256(q, red) * invn + a.eps);
#pragma unroll
        for (int v = 0; v < VPT; ++v) {
            const int64_t j = (int64_t)v * 256 + t;
            if (j < a.N) store_c_elem<T>(a.C, cbase + j, (x[v] - mean) * rs * a.gamma[j] + a.beta_ln[j]);
        }
    } else if constexpr (!VEC) {
        float s = 0.f;
        for (int64_t j = t; j < a.N; j += 256) s += input(j);
        const float mean = block_sum256(s, red) * invn;
        float q = 0.f;
        for (int64_t j = t; j < a.N; j += 256) {
            const float d = input(j) - mean;
            q += d * d;
        }
        const float rs = 1.0f / sqrtf(block_sum256(q, red) * invn + a.eps);
        for (int64_t j = t; j < a.N; j += 256)
            store_c_elem<T>(a.C, cbase + j, (input(j) - mean) * rs * a.gamma[j] + a.beta_ln[j]);
    }
}

template <typename T>
int launch_layernorm_t(const LayerNormArgs &a, hipStream_t stream) {
    typedef void (*Fn)(LayerNormArgs);
    auto al = [](const void *q, uintptr_t n) { return (uintptr_t)q % n == 0; };
    const bool vec = a.N % 4 == 0 && a.ldc % 4 == 0 && a.sc % 4 == 0 && a.ldz % 4 == 0 &&
                     a.sz % 4 == 0 && al(a.Z, 16) && al(a.C, sizeof(T) == 4 ? 16 : 8) &&
                     al(a.gamma, 16) && al(a.beta_ln, 16) && (!a.bias || al(a.bias, 16)) &&
                     a.N <= 16384;
    const Fn fn = vec ? (a.N <= 2048 ? gemm_layernorm_rows<8, T, true> : a.N <= 4096 ? gemm_layernorm_rows<16, T, true>
                         : a.N <= 8192 ? gemm_layernorm_rows<32, T, true> : gemm_layernorm_rows<64, T, true>)
                : a.N <= 2048 ? gemm_layernorm_rows<8, T, false> : a.N <= 4096 ? gemm_layernorm_rows<16, T, false>
                : a.N <= 8192 ? gemm_layernorm_rows<32, T, false> : a.N <= 16384 ? gemm_layernorm_rows<64, T, false>
                : gemm_layernorm_rows<0, T, false>;
    LayerNormArgs arg = a;
    void *args[] = {&arg};
    return hipLaunchKernel((const void *)fn, dim3((unsigned)a.rows), dim3(256), args, 0, stream) == hipSuccess
               ? GEMM_OK : GEMM_ERR_HIP;
}

int launch_layernorm(const LayerNormArgs &a, hipStream_t stream) {
    if (a.out_type == GEMM_OUT_F32) return launch_layernorm_t<float>(a, stream);
    if (a.out_type == GEMM_OUT_BF16) return launch_layernorm_t<__bf16>(a, stream);
    return launch_layernorm_t<_Float16>(a, stream);
}

// Zero-fills the first `words` 32-bit words of a workspace (its split-K
// counters).  A kernel rather than hipMemsetAsync, so that the call is an
// ordinary stream-ordered launch wherever it is made.
__global__ __launch_bounds__(256) void gemm_zero_words(uint32_t *p, int words) {
    for (int i = blockIdx.x * 256 + threadIdx.x; i < words; i += gridDim.x * 256) p[i] = 0u;
}

bool aligned16(const void *ptr) { return (uintptr_t)ptr % 16 == 0; }

// One run of a plan of either input type (the entry points below check the
// type against the one they serve) with the caller's workspace.
int run_plan(gemm_f16f32_plan_t plan, const void *A, const void *B, void *C, float alpha,
             float beta, void *ws, int64_t ws_bytes, void *stream) {
    const gemm_f16f32_plan_s &p = *plan;
    if (p.M == 0 || p.N == 0) return GEMM_OK;
    if (!C || !A || !B) return GEMM_ERR_INVALID_ARG;
    if (ws_bytes < 0 || (ws_bytes > 0 && !ws) || (uintptr_t)ws % 256 != 0) return GEMM_ERR_INVALID_ARG;
    if (ws_bytes < plan_workspace(p, p.K > 0 ? p.pack : 0)) return GEMM_ERR_INVALID_ARG;
    const int64_t cbytes = p.extent_c * (p.out_type == GEMM_OUT_F32 ? 4 : 2);
    if (p.K > 0 && (ranges_overlap((uintptr_t)C, cbytes, (uintptr_t)A, p.extent_a * 2) ||
                    ranges_overlap((uintptr_t)C, cbytes, (uintptr_t)B, p.extent_b * 2)))
        return GEMM_ERR_INVALID_ARG;
    if (ranges_overlap((uintptr_t)C, cbytes, (uintptr_t)ws, ws_bytes)) return GEMM_ERR_INVALID_ARG;
    if (p.bias && ranges_overlap((uintptr_t)C, cbytes, (uintptr_t)p.bias, p.N * 4))
        return GEMM_ERR_INVALID_ARG;

    if (p.ln) {
        // Z = alpha A B in fp32 into the last bytes of the workspace (the
        // plan's kernels with an fp32 C, no epilogue), then the row pass.
        const int64_t z_off = (ws_bytes - p.ln_z_bytes) / 256 * 256;
        float *Z = (float *)((char *)ws + z_off);
        gemm_f16f32_plan_s q = p;
        q.out_type = GEMM_OUT_F32;
        q.ldc = p.ln_ldz;
        q.stride_c = p.M * p.ln_ldz;
        q.extent_c = (p.batch - 1) * q.stride_c + (p.M - 1) * q.ldc + p.N;
        q.bias = nullptr;
        q.act = ACT_NONE;
        q.ln = 0;
        const int st = run_plan(&q, A, B, Z, alpha, 0.0f, ws, z_off, stream);
        if (st != GEMM_OK) return st;
        LayerNormArgs la;
        la.Z = Z;
        la.C = C;
        la.bias = p.bias;
        la.gamma = p.ln_gamma;
        la.beta_ln = p.ln_beta;
        la.N = p.N;
        la.M = p.M;
        la.ldz = p.ln_ldz;
        la.sz = q.stride_c;
        la.ldc = p.ldc;
        la.sc = p.stride_c;
        la.rows = p.batch * p.M;
        la.beta = beta;
        la.eps = p.ln_eps;
        la.out_type = p.out_type;
        if (la.rows > 0x7fffffff) return GEMM_ERR_UNSUPPORTED;
        return launch_layernorm(la, (hipStream_t)stream);
    }

    // Operands copied into the workspace first: those whose shape needs it,
    // and, for the direct and streaming kernels, any whose pointer is not
    // 16-byte aligned -- if the workspace holds those copies too.  Otherwise
    // (and always for the staged tiles) a misaligned operand is read in
    // place with element-wide loads by the staged kernel.
    int mask = p.K > 0 ? p.pack : 0;
    if (p.fast) {
        const int want = mask | (aligned16(A) ? 0 : 1) | (aligned16(B) ? 0 : 2);
        if (want != mask && ws_bytes >= workspace_bytes(p.split_bytes, want, p.pack_a_bytes, p.pack_b_bytes))
            mask = want;
    }
    const bool pack_a = mask & 1, pack_b = mask & 2;
    const bool vec = p.vec_ok && (pack_a || aligned16(A)) && (pack_b || aligned16(B));
    const int64_t celem = p.out_type == GEMM_OUT_F32 ? 4 : 2;
    const bool c_vec = (p.ldc % 4 == 0) && (p.stride_c % 4 == 0) &&
                       ((uintptr_t)C % (4 * celem) == 0);
    const int tile = vec ? p.tile : narrow_tile(p.tile);
    const TileShape &ts = kTiles[tile];
    const int64_t tiles_m = (p.M + ts.bm - 1) / ts.bm;
    const int64_t tiles_n = (p.N + ts.bn - 1) / ts.bn;

    GemmArgs a;
    a.A = (const uint16_t *)A;
    a.B = (const uint16_t *)B;
    a.C = C;
    a.M = p.M; a.N = p.N; a.K = p.K;
    a.lda = p.lda; a.ldb = p.ldb; a.ldc = p.ldc;
    a.sa = p.stride_a; a.sb = p.stride_b; a.sc = p.stride_c;
    // Elements reachable from each batch item's base (the range check of the
    // buffer descriptor never lets a load leave the operand).  With K = 0 no
    // element of A or B is read at all.
    a.extent_a = p.K == 0 ? 0 : p.layout_a == GEMM_ROW_MAJOR ? (p.M - 1) * p.lda + p.K
                                                             : (p.K - 1) * p.lda + p.M;
    a.extent_b = p.K == 0 ? 0 : p.layout_b == GEMM_ROW_MAJOR ? (p.K - 1) * p.ldb + p.N
                                                             : (p.N - 1) * p.ldb + p.K;
    a.alpha = alpha;
    a.beta = beta;
    a.tiles_m = (int)tiles_m;
    a.tiles_n = (int)tiles_n;
    a.group_m = p.group_m;
    a.total_tiles = (int)(tiles_m * tiles_n * p.batch);
    a.out_f32 = p.out_type == GEMM_OUT_F32;
    a.c_vec = c_vec;
    a.bias = p.bias;
    a.act = p.act;
    a.epi = p.bias != nullptr || p.act != ACT_NONE;
    a.ksplit = 1;
    a.kchunk = p.K;
    a.ws = nullptr;
    a.ws_count = nullptr;
    if (tile == p.tile && p.ksplit > 1) {
        // Counters at the workspace's start (zero between runs: the workgroup
        // that reduces a tile resets its counter), partial tiles after them.
        a.ksplit = p.ksplit;
        a.kchunk = p.kchunk;
        a.ws_count = (int *)ws;
        a.ws = (float *)((char *)ws + kCounterBytes);
    }

    if (pack_a || pack_b) {
        auto operand = [&](const void *src, int layout, int64_t rows_rm, int64_t cols_rm,
                           int64_t ld, int64_t stride, int64_t ld8, uint16_t *dst) {
            PackOperand o;
            o.src = (const uint16_t *)src;
            o.dst = dst;
            o.ld = ld;
            o.stride = stride;
            o.outer = layout == GEMM_ROW_MAJOR ? rows_rm : cols_rm;
            o.cols = layout == GEMM_ROW_MAJOR ? cols_rm : rows_rm;
            o.ld8 = ld8;
            o.chunks = (uint32_t)(p.batch * o.outer * (ld8 / 8));
            return o;
        };
        PackArgs pa = {};
        int nops = 0;
        char *next = (char *)ws + kCounterBytes + p.split_bytes;
        if (pack_a) {
            uint16_t *dst = (uint16_t *)next;
            next += p.pack_a_bytes;
            pa.op[nops++] = operand(A, p.layout_a, p.M, p.K, p.lda, p.stride_a, p.ld8_a, dst);
            const int64_t outer = p.layout_a == GEMM_ROW_MAJOR ? p.M : p.K;
            a.A = dst;
            a.lda = p.ld8_a;
            a.sa = outer * p.ld8_a;
            a.extent_a = outer * p.ld8_a;
        }
        if (pack_b) {
            uint16_t *dst = (uint16_t *)next;
            pa.op[nops++] = operand(B, p.layout_b, p.K, p.N, p.ldb, p.stride_b, p.ld8_b, dst);
            const int64_t outer = p.layout_b == GEMM_ROW_MAJOR ? p.K : p.N;
            a.B = dst;
            a.ldb = p.ld8_b;
            a.sb = outer * p.ld8_b;
            a.extent_b = outer * p.ld8_b;
        }
        const int64_t chunks = (int64_t)pa.op[0].chunks + pa.op[1].chunks;
        const int64_t blocks = std::min<int64_t>((chunks + 255) / 256, 8192);
        void *pargs[] = {&pa};
        if (hipLaunchKernel((const void *)gemm_pack16, dim3((unsigned)blocks), dim3(256), pargs, 0,
                            (hipStream_t)stream) != hipSuccess)
            return GEMM_ERR_HIP;
    }

    const int ak = p.layout_a == GEMM_ROW_MAJOR;   // A K-contiguous
    const int bkc = p.layout_b == GEMM_COL_MAJOR;  // B K-contiguous
    const int ti = p.in_type == IN_BF16 ? IN_BF16 : IN_F16;
    const int ep = a.epi ? 1 : 0;
    KernelFn fn = kernels().k[ti][ep][tile][ak][bkc][vec ? 1 : 0];
    // K-full variants: every stage inside K (for split-K, every slice: kchunk
    // is a multiple of BK, so K must be too).  K = 0 takes the variant with K
    // tests, whose loads then all fail the range check.  They keep 32-bit
    // byte counts from each tile's base down to S stages past the end of K,
    // so both operands must lie well within 2^31 bytes of that.
    auto within = [&](int64_t extent, bool kc, int64_t ld) {
        const int64_t step = kc ? ts.bk : ts.bk * ld;
        return (extent + (p.K / ts.bk + ts.stages + 1) * step) * 2 < (int64_t(1) << 31);
    };
    if (ts.kind == KIND_DIRECT16 && p.K > 0 && p.K % ts.bk == 0 && within(a.extent_a, ak, a.lda) &&
        within(a.extent_b, bkc, a.ldb))
        fn = kernels().kfull[ti][ep][tile][ak][bkc];
    if (!fn) return GEMM_ERR_UNSUPPORTED;
    void *args[] = {&a};
    const unsigned threads = ts.kind == KIND_STREAM ? 512u : (unsigned)(64 * ts.wgm * ts.wgn);
    hipError_t e = hipLaunchKernel((const void *)fn, dim3((unsigned)a.total_tiles * (unsigned)a.ksplit),
                                   dim3(threads), args, 0,
                                   (hipStream_t)stream);
    return e == hipSuccess ? GEMM_OK : GEMM_ERR_HIP;
}

}  // namespace

extern "C" int gemm_f16f32_run(gemm_f16f32_plan_t plan, const void *A,
                               const void *B, void *C, float alpha, float beta,
                               void *workspace, int64_t workspace_bytes, void *stream) {
    if (!plan || plan->in_type != IN_F16) return GEMM_ERR_INVALID_ARG;
    return run_plan(plan, A, B, C, alpha, beta, workspace, workspace_bytes, stream);
}

extern "C" int gemm_bf16f32_run(gemm_f16f32_plan_t plan, const void *A,
                                const void *B, void *C, float alpha, float beta,
                                void *workspace, int64_t workspace_bytes, void *stream) {
    if (!plan || plan->in_type != IN_BF16) return GEMM_ERR_INVALID_ARG;
    return run_plan(plan, A, B, C, alpha, beta, workspace, workspace_bytes, stream);
}

extern "C" int gemm_f16f32_workspace_init(void *workspace, int64_t bytes, void *stream) {
    if (bytes < 0 || (bytes > 0 && !workspace) || (uintptr_t)workspace % 256 != 0)
        return GEMM_ERR_INVALID_ARG;
    const int words = (int)(std::min<int64_t>(bytes, kCounterBytes) / 4);
    if (words == 0) return GEMM_OK;
    uint32_t *w = (uint32_t *)workspace;
    int n = words;
    void *args[] = {&w, &n};
    return hipLaunchKernel((const void *)gemm_zero_words, dim3(1), dim3(256), args, 0,
                           (hipStream_t)stream) == hipSuccess ? GEMM_OK : GEMM_ERR_HIP;
}

// ---------------------------------------------------------------------------
// No-allocation entry point, for callers that cannot allocate device memory
// (code under stream capture, tight serving loops, harnesses that forbid
// hipMalloc): the workspace is this library's own static device array.  Each
// device that runs the library holds its copy of the array, at its own
// address, for the life of the process.  That address is taken once per
// device with hipGetSymbolAddress (the array's name in host code is only a
// host-side stand-in, never a device address) and is what the kernels get.
// ---------------------------------------------------------------------------
namespace {

constexpr int64_t kScratchBytes = int64_t(64) << 20;
static __device__ __align__(256) __attribute__((used)) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void *g_scratch_ptr[kMaxDevices];   // device address of scratch per device, once set up

// The current device's scratch: its address, looked up on the first call on
// the device (with the device current), and its counter words zero-filled
// once by a kernel on `stream` (split-K runs leave them zero after that).
int device_scratch(void **out, hipStream_t stream) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return GEMM_ERR_HIP;
    if (dev < 0 || dev >= kMaxDevices) return GEMM_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        void *ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return GEMM_ERR_HIP;
        uint32_t *w = (uint32_t *)ptr;
        int words = kMaxCounters;
        void *args[] = {&w, &words};
        if (hipLaunchKernel((const void *)gemm_zero_words, dim3(1), dim3(256), args, 0, stream) != hipSuccess)
            return GEMM_ERR_HIP;
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return GEMM_OK;
}

}  // namespace

extern "C" int gemm_f16f32_run_noalloc(gemm_f16f32_plan_t plan, const void *A, const void *B,
                                       void *C, float alpha, float beta, void *stream) {
    if (!plan) return GEMM_ERR_INVALID_ARG;
    if (plan->M == 0 || plan->N == 0) return GEMM_OK;
    if (plan_workspace(*plan, plan->pack) > kScratchBytes) return GEMM_ERR_SCRATCH;
    if (!A || !B || !C) return GEMM_ERR_INVALID_ARG;
    void *ws = nullptr;
    int64_t ws_bytes = 0;
    // Plans that need scratch, and those that repack misaligned operands into
    // it when it holds the copies, use the device's array.
    if (plan->split_bytes > 0 || plan->pack != 0 || plan->fast || plan->ln) {
        const int st = device_scratch(&ws, (hipStream_t)stream);
        if (st != GEMM_OK) return st;
        ws_bytes = kScratchBytes;
    }
    return run_plan(plan, A, B, C, alpha, beta, ws, ws_bytes, stream);
}

// ---------------------------------------------------------------------------
// Implicit-GEMM convolution: the staged kernel with its A tile read through
// ConvLoader (the unrolled NHWC input), B the KRSC filters as a K-contiguous
// operand (row k of the filters is column k of B, ldb = R S C) and C the NPQK
// output (row-major, ldc = K).
// ---------------------------------------------------------------------------
struct conv_f16_plan_s {
    int64_t N, H, W, C, K, R, S, sh, sw, ph, pw, dh, dw, P, Q;
    int out_type;
    int tile;            // index into kConvTiles
    char kernel_name[64];
};

namespace {

int64_t conv_out_dim(int64_t in, int64_t k, int64_t stride, int64_t pad, int64_t dil) {
    const int64_t span = dil * (k - 1) + 1;
    if (in + 2 * pad < span) return -1;
    return (in + 2 * pad - span) / stride + 1;
}

// Tiles of the convolution (the staged kernel's shapes, BK = 64): the 64
// tile for small problems (fewer than 128 workgroups otherwise), and for the
// rest a 128- or 256-row tile whose width follows the output channels (64
// columns when K <= 64, so that no half-empty tile is computed).
struct ConvTile {
    int bm, bn, wgm, wgn;
    const char *name;
};
constexpr ConvTile kConvTiles[] = {
    {64, 64, 2, 2, "64x64x64"},
    {128, 128, 2, 2, "128x128x64"},
    {128, 64, 2, 2, "128x64x64"},
    {256, 64, 4, 1, "256x64x64"},
};
constexpr int kNumConvTiles = (int)(sizeof kConvTiles / sizeof kConvTiles[0]);

template <int T, bool VEC, bool EPI>
constexpr KernelFn pick_conv() {
    return gemm_staged<_Float16, kConvTiles[T].bm, kConvTiles[T].bn, 64, kConvTiles[T].wgm,
                       kConvTiles[T].wgn, true, true, VEC, EPI, true>;
}

template <int T>
constexpr void fill_conv(KernelFn (&k)[2][2]) {
    k[0][0] = pick_conv<T, false, false>();
    k[0][1] = pick_conv<T, false, true>();
    k[1][0] = pick_conv<T, true, false>();
    k[1][1] = pick_conv<T, true, true>();
}

KernelFn conv_kernel(int tile, bool vec, bool epi) {
    static const auto table = [] {
        struct { KernelFn k[kNumConvTiles][2][2]; } t{};
        fill_conv<0>(t.k[0]);
        fill_conv<1>(t.k[1]);
        fill_conv<2>(t.k[2]);
        fill_conv<3>(t.k[3]);
        return t;
    }();
    return table.k[tile][vec][epi];
}

// Measured on the 3x3 64 -> 64 layer at 32 x 56 x 56 (25 us on 256 x 64 against
// 27 on 64 x 64 and 35 on 128 x 128) and the 7x7 stride-2 stem with C = 3
// (102 us on 128 x 64; its element-wise loads leave the 256-row tile no faster).
int choose_conv_tile(int64_t M, int64_t K, int64_t C) {
    const int t = K > 64 ? 1 : C % 8 == 0 ? 3 : 2;
    const int64_t tiles = ((M + kConvTiles[t].bm - 1) / kConvTiles[t].bm) *
                          ((K + kConvTiles[t].bn - 1) / kConvTiles[t].bn);
    return tiles >= kNumCUs / 2 ? t : 0;
}

}  // namespace

extern "C" int conv_f16_plan(conv_f16_plan_t *out, int64_t N, int64_t H, int64_t W, int64_t C,
                             int64_t K, int64_t R, int64_t S, int64_t stride_h, int64_t stride_w,
                             int64_t pad_h, int64_t pad_w, int64_t dil_h, int64_t dil_w,
                             int out_type) {
    if (!out) return GEMM_ERR_INVALID_ARG;
    *out = nullptr;
    if (N < 0 || K < 0 || H < 1 || W < 1 || C < 1 || R < 1 || S < 1) return GEMM_ERR_INVALID_ARG;
    if (stride_h < 1 || stride_w < 1 || dil_h < 1 || dil_w < 1 || pad_h < 0 || pad_w < 0)
        return GEMM_ERR_INVALID_ARG;
    if (out_type != GEMM_OUT_F16 && out_type != GEMM_OUT_F32) return GEMM_ERR_INVALID_ARG;
    const int64_t lim = int64_t(1) << 31;
    if (H >= lim || W >= lim || R >= lim || S >= lim || pad_h >= lim || pad_w >= lim || stride_h >= lim ||
        stride_w >= lim || dil_h >= lim || dil_w >= lim)
        return GEMM_ERR_UNSUPPORTED;
    const int64_t P = conv_out_dim(H, R, stride_h, pad_h, dil_h), Q = conv_out_dim(W, S, stride_w, pad_w, dil_w);
    if (P < 1 || Q < 1) return GEMM_ERR_INVALID_ARG;
    const int64_t M = N * P * Q, RSC = R * S * C;
    if (N * H * W * C * 2 >= lim || M >= lim || RSC >= lim || K >= lim || 128 * RSC * 2 >= lim)
        return GEMM_ERR_UNSUPPORTED;
    conv_f16_plan_s *p = new (std::nothrow) conv_f16_plan_s();
    if (!p) return GEMM_ERR_NOMEM;
    p->N = N; p->H = H; p->W = W; p->C = C; p->K = K; p->R = R; p->S = S;
    p->sh = stride_h; p->sw = stride_w; p->ph = pad_h; p->pw = pad_w; p->dh = dil_h; p->dw = dil_w;
    p->P = P; p->Q = Q;
    p->out_type = out_type;
    p->tile = choose_conv_tile(M, K, C);
    if (M == 0 || K == 0)
        snprintf(p->kernel_name, sizeof p->kernel_name, "none");
    else
        snprintf(p->kernel_name, sizeof p->kernel_name, "conv_implicit_%s_%s",
                 kConvTiles[p->tile].name, C % 8 == 0 ? "vec16" : "narrow");
    *out = p;
    return GEMM_OK;
}

extern "C" int conv_f16_output_size(conv_f16_plan_t plan, int64_t *P, int64_t *Q) {
    if (!plan || !P || !Q) return GEMM_ERR_INVALID_ARG;
    *P = plan->P;
    *Q = plan->Q;
    return GEMM_OK;
}

extern "C" int conv_f16_run(conv_f16_plan_t plan, const void *x, const void *w, void *y, float alpha,
                            float beta, const float *bias, int activation, void *stream) {
    if (!plan) return GEMM_ERR_INVALID_ARG;
    const conv_f16_plan_s &p = *plan;
    if (activation < ACT_NONE || activation > ACT_SILU || (uintptr_t)bias % 4 != 0)
        return GEMM_ERR_INVALID_ARG;
    const int64_t M = p.N * p.P * p.Q, RSC = p.R * p.S * p.C;
    if (M == 0 || p.K == 0) return GEMM_OK;
    if (!x || !w || !y) return GEMM_ERR_INVALID_ARG;
    const int64_t xb = p.N * p.H * p.W * p.C * 2, wb = p.K * RSC * 2;
    const int64_t yb = M * p.K * (p.out_type == GEMM_OUT_F32 ? 4 : 2);
    if (ranges_overlap((uintptr_t)y, yb, (uintptr_t)x, xb) || ranges_overlap((uintptr_t)y, yb, (uintptr_t)w, wb) ||
        (bias && ranges_overlap((uintptr_t)y, yb, (uintptr_t)bias, p.K * 4)))
        return GEMM_ERR_INVALID_ARG;
    const bool vec = p.C % 8 == 0 && (uintptr_t)x % 16 == 0 && (uintptr_t)w % 16 == 0;
    const ConvTile &ts = kConvTiles[p.tile];
    GemmArgs a = {};
    a.A = (const uint16_t *)x;
    a.B = (const uint16_t *)w;
    a.C = y;
    a.M = M; a.N = p.K; a.K = RSC;
    a.lda = RSC; a.ldb = RSC; a.ldc = p.K;
    a.sa = a.sb = a.sc = 0;
    a.extent_a = p.N * p.H * p.W * p.C;
    a.extent_b = p.K * RSC;
    a.alpha = alpha;
    a.beta = beta;
    a.tiles_m = (int)((M + ts.bm - 1) / ts.bm);
    a.tiles_n = (int)((p.K + ts.bn - 1) / ts.bn);
    a.group_m = 4;
    a.total_tiles = a.tiles_m * a.tiles_n;
    a.out_f32 = p.out_type == GEMM_OUT_F32;
    a.c_vec = p.K % 4 == 0 && (uintptr_t)y % (a.out_f32 ? 16 : 8) == 0;
    a.bias = bias;
    a.act = activation;
    a.epi = bias != nullptr || activation != ACT_NONE;
    a.ksplit = 1;
    a.kchunk = RSC;
    a.cv.H = (int)p.H; a.cv.W = (int)p.W; a.cv.C = (int)p.C; a.cv.P = (int)p.P; a.cv.Q = (int)p.Q;
    a.cv.R = (int)p.R; a.cv.S = (int)p.S; a.cv.sh = (int)p.sh; a.cv.sw = (int)p.sw;
    a.cv.ph = (int)p.ph; a.cv.pw = (int)p.pw; a.cv.dh = (int)p.dh; a.cv.dw = (int)p.dw;
    const KernelFn fn = conv_kernel(p.tile, vec, a.epi != 0);
    void *args[] = {&a};
    return hipLaunchKernel((const void *)fn, dim3((unsigned)a.total_tiles), dim3(64 * ts.wgm * ts.wgn),
                           args, 0, (hipStream_t)stream) == hipSuccess ? GEMM_OK : GEMM_ERR_HIP;
}

extern "C" int conv_f16_destroy(conv_f16_plan_t plan) {
    delete plan;
    return GEMM_OK;
}

extern "C" const char *conv_f16_plan_kernel(conv_f16_plan_t plan) {
    return plan ? plan->kernel_name : "invalid";
}

#endif  // MPGEMM_HOST_PART
