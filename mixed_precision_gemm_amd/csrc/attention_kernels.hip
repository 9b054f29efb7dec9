// Fused attention and row softmax for gfx950 (MI355X), and their C-ABI entry
// points.
//
// Pages cited (titles as printed):
//   [OPS]     CUDA operator practice page (Softmax and GEMM)
//   [GEMM]    "手写GEMM内核：矩阵乘法性能优化的完整工程实践" (hand-written GEMM kernel)
//   [CATLASS] CATLASS template library page
//
// Attention ([GEMM] §1.1: Q K^T, a softmax, a product with V; [CATLASS] §5.2:
// the two products and the softmax in one kernel, the score tile kept on
// chip).  One workgroup of four 64-lane waves owns 128 query rows of one
// (batch, head); each wave owns 32 of them as two blocks of 16.  The keys are
// walked in tiles of 64:
//   * K and V tiles go straight to LDS by direct-to-LDS loads, double
//     buffered: tile t+1 is loaded into the other buffer while tile t is
//     consumed; one wait and one barrier per tile.  Each load instruction
//     fills 1 KiB of whole LDS rows, lane l the 16-byte slot l of them, and
//     fetches the global chunk that the row's swizzle puts in that slot;
//   * S^T = K Q^T on v_mfma_f32_16x16x32_f16 (K fragments from LDS with
//     ds_read_b128, Q fragments held in registers for the whole walk), fp32
//     accumulation.  Computing the transpose puts, in each lane, four keys of
//     one query: the row maximum is lane-local but for two exchanges across
//     the wave's four 16-lane groups, and the row sum stays lane-local until
//     the end;
//   * the online softmax of [OPS] §2.2 in fp32 and in base 2 (scores are
//     multiplied by scale * log2 e once, then v_exp_f32 is 2^x): a new tile
//     with maximum m_new moves the row's reference to m' = max(m, m_new), and
//     the running sum and the output accumulators are rescaled by 2^(m - m');
//   * O^T += V^T P^T on the same MFMA, with P taken straight from the score
//     accumulators (rounded to binary16) as the second operand -- the score
//     tile never leaves registers.  The MFMA sums over its 32 k slots in any
//     order the two operands agree on: lane group g supplies keys
//     4g..4g+3 and 16+4g..16+4g+3 of each 32-key chunk (exactly the keys its
//     score accumulators hold), and the V^T operand is read for the same
//     keys by two transposing LDS reads (ds_read_b64_tr_b16);
//   * masked keys (past Sk, or past the causal diagonal) get a score of -inf;
//     a row with no visible key keeps m = -inf and l = 0 and is written as
//     zeros ([OPS] §2.5: the constant output for a fully masked row);
//   * the end divides by the row sum and rounds once to the output type.
// Row softmax ([OPS] §2.1-§2.4): one workgroup per row; rows of up to 8192
// elements are held in registers and read once; longer rows are read twice,
// the first pass keeping a running maximum and sum per thread by the online
// recurrence and merging them across the workgroup the same way.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <new>

#include "attention_f16.h"

namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef short v4i16 __attribute__((ext_vector_type(4)));

// Byte offset that fails the buffer range check: the load returns zeros.
constexpr uint32_t kOutOfRange = 0x80000000u;
// Word 3 of a gfx9 buffer descriptor: 32-bit data format, raw addressing.
constexpr int kRsrcWord3 = 0x00020000;
constexpr float kLog2e = 1.44269504088896341f;

__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void *base, int64_t bytes) {
    const int32_t n = bytes <= 0 ? 0 : (bytes >= 0x7fffffff ? 0x7fffffff : (int32_t)bytes);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, n, kRsrcWord3);
}

__device__ inline floatx4 mfma16(half8 a, half8 b, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
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
// address lds_addr + 16 t (lds_addr taken from the first lane).  Assembly,
// so the compiler's wait-count insertion does not tie the fragment reads of
// the other buffer to it; the kernel waits for it explicitly before its
// barrier.
__device__ inline void lds_dma16(sgpr4 rs, uint32_t lds_addr, uint32_t voff) {
    const uint32_t m0v = (uint32_t)__builtin_amdgcn_readfirstlane((int)lds_addr);
    asm volatile("s_mov_b32 m0, %1\n\tbuffer_load_dwordx4 %0, %2, 0 offen lds"
                 :
                 : "v"(voff), "s"(m0v), "s"(rs)
                 : "m0");
}

struct AttnArgs {
    const uint16_t *Q, *K, *V;
    void *O;
    int64_t q_sb, q_sh, q_ld, k_sb, k_sh, k_ld, v_sb, v_sh, v_ld, o_sb, o_sh, o_ld;
    int heads, Sq, Sk;
    int nqb;       // query blocks of 128 rows per (batch, head)
    int total;     // workgroups
    float c;       // scale * log2(e)
};

// LDS row swizzles, chosen for the two fragment reads (checked against a
// 64-bank, 4-byte bank model: ds_read_b128 served 16 lanes a pass, lanes
// i..i+7 with i+32..i+39; ds_read_b64_tr_b16 served 32 lanes a pass).
//   K rows (D halves, D/8 16-byte chunks): a pass reads rows r..r+7 (r a
//   multiple of 8) at chunks c and c+2; the XOR moves row bits 0..2 to chunk
//   bits 0, 2, 3 (256-byte rows: 16 distinct chunks), or row bits 1, 2 to
//   chunk bits 0, 2 (128-byte rows, where row bit 0 already picks the bank
//   half).
//   V rows: a pass reads rows k..k+7 at the two chunks of 16 columns (chunk
//   bit 0 differs); the XOR puts row bits 0..2 (256-byte rows) or 1..2
//   (128-byte rows) on chunk bits 1..3.
template <int D>
__device__ __host__ constexpr int kswz(int row) {
    return D == 128 ? ((row & 1) | (((row >> 1) & 1) << 2) | (((row >> 2) & 1) << 3))
                    : ((((row >> 1) & 1)) | (((row >> 2) & 1) << 2));
}
template <int D>
__device__ __host__ constexpr int vswz(int row) {
    return D == 128 ? ((row & 7) << 1) : (((row >> 1) & 3) << 1);
}

template <int D, bool CAUSAL, bool OUT32>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_fwd(AttnArgs p) {
    constexpr int BQ = 128, BN = 64;
    constexpr int NDC = D / 32;          // 32-deep d steps of S^T
    constexpr int NCB = D / 16;          // 16-wide column blocks of O
    constexpr int CPR = D / 8;           // 16-byte chunks per LDS row
    constexpr int TILE = BN * D;         // halves per K (or V) tile
    constexpr int RPI = 1024 / (2 * D);  // rows of a tile per 1 KiB load
    constexpr int NLW = BN / RPI / 4;    // loads per wave per tile, each of K and V
    static_assert(D == 64 || D == 128, "head dimension");
    __shared__ __attribute__((aligned(16))) _Float16 lds[2][2][TILE];   // [buffer][K, V]

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4, li = lane & 15;

    // Workgroups are dispatched round-robin over the 8 XCDs: remap so that
    // consecutive logical ids -- the query blocks of one (batch, head), which
    // read the same K and V -- run on one XCD and share its L2.
    const int total = p.total;
    const int per = total / 8, rem = total % 8;
    const int xcd = (int)blockIdx.x % 8, local = (int)blockIdx.x / 8;
    const int logical = xcd * per + (xcd < rem ? xcd : rem) + local;
    const int bh = logical / p.nqb;
    int qblk = logical - bh * p.nqb;
    if (CAUSAL) qblk = p.nqb - 1 - qblk;    // longest rows first
    const int b = bh / p.heads, h = bh - b * p.heads;

    const int64_t Sq = p.Sq, Sk = p.Sk;
    const int64_t off = Sk - Sq;             // causal: key j visible to query i iff j <= i + off
    const int64_t q0 = (int64_t)qblk * BQ;
    const int64_t wq0 = q0 + 32 * wave;      // this wave's first query row
    const int64_t q_last = std::min<int64_t>(q0 + BQ, Sq) - 1;
    const int64_t wq_last = std::min<int64_t>(wq0 + 31, Sq - 1);
    int64_t kv_end = Sk;
    if (CAUSAL) kv_end = std::min<int64_t>(Sk, q_last + off + 1);
    const int nkv = kv_end > 0 ? (int)((kv_end + BN - 1) / BN) : 0;

    const uint16_t *Qb = p.Q + b * p.q_sb + h * p.q_sh;
    const uint16_t *Kb = p.K + b * p.k_sb + h * p.k_sh;
    const uint16_t *Vb = p.V + b * p.v_sb + h * p.v_sh;
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(Qb, Sq > 0 ? ((Sq - 1) * p.q_ld + D) * 2 : 0);
    const sgpr4 rk = make_rsrc_words(Kb, Sk > 0 ? ((Sk - 1) * p.k_ld + D) * 2 : 0);
    const sgpr4 rv = make_rsrc_words(Vb, Sk > 0 ? ((Sk - 1) * p.v_ld + D) * 2 : 0);

    // Q fragments (second MFMA operand of S^T): lane l holds query row
    // 16 qb + l%16 of the wave's rows, d = 32 dc + 8 (l/16) .. + 7.
    half8 qf[2][NDC];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
        const int64_t row = wq0 + 16 * qb + li;
#pragma unroll
        for (int dc = 0; dc < NDC; ++dc) {
            const uint32_t o = row < Sq ? (uint32_t)((row * p.q_ld + 32 * dc + 8 * g) * 2) : kOutOfRange;
            qf[qb][dc] = __builtin_bit_cast(half8, __builtin_amdgcn_raw_buffer_load_b128(rq, o, 0, 0));
        }
    }

    // Loads of one K and one V tile into buffer buf: wave w's load j fills
    // rows r0 = (NLW w + j) RPI .. + RPI - 1; lane l lands in row r0 + l /
    // CPR, slot l % CPR, which holds the row's chunk slot ^ swizzle (the XOR
    // is its own inverse).  Keys past Sk read zeros (range check).
    const uint32_t lds0 = lds_offset(lds);
    auto issue = [&](int kt, int buf) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < NLW; ++j) {
            const int r0 = (NLW * wave + j) * RPI;
            const int row = r0 + lane / CPR, slot = lane % CPR;
            const int64_t key = (int64_t)kt * BN + row;
            const bool ok = key < Sk;
            const int ck = slot ^ kswz<D>(row), cv = slot ^ vswz<D>(row);
            const uint32_t dst = lds0 + (uint32_t)((buf * 2 * TILE + r0 * D) * 2);
            lds_dma16(rk, dst, ok ? (uint32_t)((key * p.k_ld + 8 * ck) * 2) : kOutOfRange);
            lds_dma16(rv, dst + (uint32_t)(TILE * 2), ok ? (uint32_t)((key * p.v_ld + 8 * cv) * 2) : kOutOfRange);
        }
    };

    // Per-lane LDS element offsets of the fragment reads.
    //  K (first operand of S^T): row 16 kb + l%16, chunk 4 dc + l/16.
    const int kx = kswz<D>(li);              // row % 8 == li % 8
    //  V^T (first operand of O^T), read t of chunk kc: rows 32 kc + 16 t +
    //  4 g + l%16/4, columns 16 cb + 4 (l%4) (lane receives column 16 cb +
    //  l%16 of rows 32 kc + 16 t + 4 g .. + 3).
    const int vrow = 4 * g + (li >> 2);      // row within a 16-row half-chunk
    const int vy = vswz<D>(vrow & 7);
    const int vcol_hi = (li & 3) >> 1, vcol_lo = 4 * (li & 1);

    floatx4 o[NCB][2];
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) o[cb][qb] = floatx4{0.f, 0.f, 0.f, 0.f};
    float m[2] = {-INFINITY, -INFINITY}, l[2] = {0.f, 0.f};

    if (nkv > 0) issue(0, 0);
    asm volatile("s_waitcnt vmcnt(0)" : : : "memory");   // Q fragments and tile 0
    __syncthreads();

    for (int kt = 0; kt < nkv; ++kt) {
        const int buf = kt & 1;
        // The other buffer was last read in tile kt - 1, before the barrier
        // that ended it.
        if (kt + 1 < nkv) issue(kt + 1, buf ^ 1);
        const int64_t k0 = (int64_t)kt * BN;
        // Tiles wholly past this wave's causal limit (or waves past Sq) skip
        // the arithmetic but keep loading and meeting the barrier.
        const bool active = wq0 < Sq && (!CAUSAL || k0 <= wq_last + off);
        if (active) {
            const _Float16 *kt_lds = lds[buf][0];
            const _Float16 *vt_lds = lds[buf][1];
            // The first d step starts from a zero accumulator operand
            // (no register clearing per tile).
            floatx4 s[4][2];
#pragma unroll
            for (int dc = 0; dc < NDC; ++dc)
#pragma unroll
                for (int kb = 0; kb < 4; ++kb) {
                    const half8 kf = *(const half8 *)&kt_lds[(16 * kb + li) * D + 8 * ((4 * dc + g) ^ kx)];
#pragma unroll
                    for (int qb = 0; qb < 2; ++qb)
                        s[kb][qb] = mfma16(kf, qf[qb][dc], dc == 0 ? floatx4{0.f, 0.f, 0.f, 0.f} : s[kb][qb]);
                }
            // Online softmax per query block: lane l's query is row 16 qb +
            // l%16; its keys are k0 + 16 kb + 4 g + r.
            const bool need_mask = (k0 + BN > Sk) || (CAUSAL && k0 + BN - 1 > wq0 + off);
            half8 pf[2][2];   // [32-key chunk][query block]
#pragma unroll
            for (int qb = 0; qb < 2; ++qb) {
                const int64_t qrow = wq0 + 16 * qb + li;
                float sv[4][4];
                float bm = -INFINITY;
#pragma unroll
                for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        float x = s[kb][qb][r] * p.c;
                        if (need_mask) {
                            const int64_t key = k0 + 16 * kb + 4 * g + r;
                            if (key >= Sk || (CAUSAL && key > qrow + off)) x = -INFINITY;
                        }
                        sv[kb][r] = x;
                        bm = fmaxf(bm, x);
                    }
                bm = fmaxf(bm, __shfl_xor(bm, 16));
                bm = fmaxf(bm, __shfl_xor(bm, 32));
                const float mnew = fmaxf(m[qb], bm);
                const bool none = mnew == -INFINITY;        // nothing visible yet
                const float alpha = none ? 1.f : __builtin_amdgcn_exp2f(m[qb] - mnew);
                const float ms = none ? 0.f : mnew;
                float rs = 0.f;
                _Float16 ph[4][4];
#pragma unroll
                for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const float e = __builtin_amdgcn_exp2f(sv[kb][r] - ms);
                        rs += e;
                        ph[kb][r] = (_Float16)e;
                    }
                l[qb] = l[qb] * alpha + rs;
                m[qb] = mnew;
                // Rescaling by 1 changes nothing: skipped when no row of the
                // block has a new maximum (most tiles once the maxima settle).
                if (__builtin_amdgcn_ballot_w64(alpha != 1.f)) {
#pragma unroll
                    for (int cb = 0; cb < NCB; ++cb) o[cb][qb] *= alpha;
                }
#pragma unroll
                for (int kc = 0; kc < 2; ++kc)
                    pf[kc][qb] = half8{ph[2 * kc][0], ph[2 * kc][1], ph[2 * kc][2], ph[2 * kc][3],
                                       ph[2 * kc + 1][0], ph[2 * kc + 1][1], ph[2 * kc + 1][2],
                                       ph[2 * kc + 1][3]};
            }
            // O^T += V^T P^T.
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
                for (int kc = 0; kc < 2; ++kc) {
                    v4i16 hv[2];
#pragma unroll
                    for (int t = 0; t < 2; ++t) {
                        const int row = 32 * kc + 16 * t + vrow;
                        const _Float16 *ptr = &vt_lds[row * D + 8 * ((2 * cb + vcol_hi) ^ vy) + vcol_lo];
                        hv[t] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                            (__attribute__((address_space(3))) v4i16 *)(const void *)ptr);
                    }
                    const half8 vf = __builtin_bit_cast(
                        half8, __builtin_shufflevector(hv[0], hv[1], 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
                    for (int qb = 0; qb < 2; ++qb) o[cb][qb] = mfma16(vf, pf[kc][qb], o[cb][qb]);
                }
        }
        // This wave's loads of tile kt + 1 have landed; after the barrier,
        // every wave's have, and no wave still reads buffer buf.
        asm volatile("s_waitcnt vmcnt(0)" : : : "memory");
        __syncthreads();
    }

    // O(i, c) = O^T(c, i) / l_i: lane l holds columns 16 cb + 4 g + 0..3 of
    // query row 16 qb + l%16.
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
        float lt = l[qb];
        lt += __shfl_xor(lt, 16);
        lt += __shfl_xor(lt, 32);
        const float inv = lt > 0.f ? __builtin_amdgcn_rcpf(lt) : 0.f;
        const int64_t qrow = wq0 + 16 * qb + li;
        if (qrow >= Sq) continue;
        const int64_t obase = b * p.o_sb + h * p.o_sh + qrow * p.o_ld + 4 * g;
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
            const floatx4 v = o[cb][qb] * inv;
            if constexpr (OUT32) {
                *(floatx4 *)((float *)p.O + obase + 16 * cb) = v;
            } else {
                *(half4 *)((_Float16 *)p.O + obase + 16 * cb) =
                    half4{(_Float16)v[0], (_Float16)v[1], (_Float16)v[2], (_Float16)v[3]};
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Row softmax.
// ---------------------------------------------------------------------------
struct SmArgs {
    const void *x;
    void *y;
    int64_t cols, ldx, ldy;
};

template <bool F32>
__device__ inline float load_elem(const void *base, int64_t i) {
    if constexpr (F32) return ((const float *)base)[i];
    else return (float)((const _Float16 *)base)[i];
}
template <bool F32>
__device__ inline void store_elem(void *base, int64_t i, float v) {
    if constexpr (F32) ((float *)base)[i] = v;
    else ((_Float16 *)base)[i] = (_Float16)v;
}

// Maximum and sum merged across the workgroup by the online rule: (m1, s1)
// and (m2, s2) combine to (m, s1 2^(m1 - m) + s2 2^(m2 - m)), m = max(m1,
// m2), in base-2 units (values already multiplied by log2 e).
__device__ inline void merge_ms(float &m, float &s, float m2, float s2) {
    const float mn = fmaxf(m, m2);
    if (mn == -INFINITY) return;
    s = (m == -INFINITY ? 0.f : s * __builtin_amdgcn_exp2f(m - mn)) +
        (m2 == -INFINITY ? 0.f : s2 * __builtin_amdgcn_exp2f(m2 - mn));
    m = mn;
}

__device__ inline void block_merge(float &m, float &s, float *red) {
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) merge_ms(m, s, __shfl_xor(m, d), __shfl_xor(s, d));
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    if (lane == 0) { red[2 * wave] = m; red[2 * wave + 1] = s; }
    __syncthreads();
    m = red[0];
    s = red[1];
    for (int w = 1; w < 4; ++w) merge_ms(m, s, red[2 * w], red[2 * w + 1]);
    __syncthreads();   // red may be reused by the caller
}

// Rows held in registers: VPT values per thread, element j = 256 v + t.
template <int VPT, bool IN32, bool OUT32>
__global__ __launch_bounds__(256) void softmax_rows_reg(SmArgs a) {
    __shared__ float red[8];
    const int64_t row = blockIdx.x;
    const int t = threadIdx.x;
    const void *xr = IN32 ? (const void *)((const float *)a.x + row * a.ldx)
                          : (const void *)((const _Float16 *)a.x + row * a.ldx);
    float v[VPT];
    float m = -INFINITY;
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
        const int64_t j = (int64_t)i * 256 + t;
        v[i] = j < a.cols ? load_elem<IN32>(xr, j) * kLog2e : -INFINITY;
        m = fmaxf(m, v[i]);
    }
    float s = 0.f;
    const float ms = m == -INFINITY ? 0.f : m;
#pragma unroll
    for (int i = 0; i < VPT; ++i) s += __builtin_amdgcn_exp2f(v[i] - ms);
    block_merge(m, s, red);
    const float mm = m == -INFINITY ? 0.f : m;
    const float inv = s > 0.f ? __builtin_amdgcn_rcpf(s) : 0.f;
    void *yr = OUT32 ? (void *)((float *)a.y + row * a.ldy) : (void *)((_Float16 *)a.y + row * a.ldy);
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
        const int64_t j = (int64_t)i * 256 + t;
        if (j < a.cols) store_elem<OUT32>(yr, j, __builtin_amdgcn_exp2f(v[i] - mm) * inv);
    }
}

// Rows held in registers, read and written 16 bytes (fp16) or 32 bytes
// (fp32) at a time: NCH chunks of 8 elements per thread, chunk c of thread t
// covering elements 8 (256 c + t) .. + 7.  For rows whose length, leading
// dimensions and base addresses are multiples of 8 elements and 16 bytes:
// every chunk is then wholly inside or wholly outside the row.  Element-wide
// accesses (the kernel above) move 128 bytes per wave instruction and ran
// at 0.30 of HBM bandwidth on 8192 rows of 4096.
template <int NCH, bool IN32, bool OUT32>
__global__ __launch_bounds__(256) void softmax_rows_vec(SmArgs a) {
    __shared__ float red[8];
    const int64_t row = blockIdx.x;
    const int t = threadIdx.x;
    float v[NCH][8];
    float m = -INFINITY;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        const int64_t j0 = ((int64_t)c * 256 + t) * 8;
        if (j0 < a.cols) {
            if constexpr (IN32) {
                const floatx4 *src = (const floatx4 *)((const float *)a.x + row * a.ldx + j0);
                const floatx4 lo = src[0], hi = src[1];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    v[c][e] = lo[e] * kLog2e;
                    v[c][4 + e] = hi[e] * kLog2e;
                }
            } else {
                const half8 h = *(const half8 *)((const _Float16 *)a.x + row * a.ldx + j0);
#pragma unroll
                for (int e = 0; e < 8; ++e) v[c][e] = (float)h[e] * kLog2e;
            }
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) v[c][e] = -INFINITY;
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) m = fmaxf(m, v[c][e]);
    }
    float s = 0.f;
    const float ms = m == -INFINITY ? 0.f : m;
#pragma unroll
    for (int c = 0; c < NCH; ++c)
#pragma unroll
        for (int e = 0; e < 8; ++e) s += __builtin_amdgcn_exp2f(v[c][e] - ms);
    block_merge(m, s, red);
    const float mm = m == -INFINITY ? 0.f : m;
    const float inv = s > 0.f ? __builtin_amdgcn_rcpf(s) : 0.f;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        const int64_t j0 = ((int64_t)c * 256 + t) * 8;
        if (j0 >= a.cols) continue;
        float y[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) y[e] = __builtin_amdgcn_exp2f(v[c][e] - mm) * inv;
        if constexpr (OUT32) {
            floatx4 *dst = (floatx4 *)((float *)a.y + row * a.ldy + j0);
            dst[0] = floatx4{y[0], y[1], y[2], y[3]};
            dst[1] = floatx4{y[4], y[5], y[6], y[7]};
        } else {
            half8 h;
#pragma unroll
            for (int e = 0; e < 8; ++e) h[e] = (_Float16)y[e];
            *(half8 *)((_Float16 *)a.y + row * a.ldy + j0) = h;
        }
    }
}

// Long rows: pass 1 keeps (m, s) per thread with the online rule, element by
// element; the workgroup merges them; pass 2 re-reads and writes.
template <bool IN32, bool OUT32>
__global__ __launch_bounds__(256) void softmax_rows_online(SmArgs a) {
    __shared__ float red[8];
    const int64_t row = blockIdx.x;
    const int t = threadIdx.x;
    const void *xr = IN32 ? (const void *)((const float *)a.x + row * a.ldx)
                          : (const void *)((const _Float16 *)a.x + row * a.ldx);
    float m = -INFINITY, s = 0.f;
    for (int64_t j = t; j < a.cols; j += 256) {
        const float x = load_elem<IN32>(xr, j) * kLog2e;
        merge_ms(m, s, x, 1.f);
    }
    block_merge(m, s, red);
    const float mm = m == -INFINITY ? 0.f : m;
    const float inv = s > 0.f ? __builtin_amdgcn_rcpf(s) : 0.f;
    void *yr = OUT32 ? (void *)((float *)a.y + row * a.ldy) : (void *)((_Float16 *)a.y + row * a.ldy);
    for (int64_t j = t; j < a.cols; j += 256)
        store_elem<OUT32>(yr, j, __builtin_amdgcn_exp2f(load_elem<IN32>(xr, j) * kLog2e - mm) * inv);
}

bool ranges_overlap(uintptr_t a, int64_t a_bytes, uintptr_t b, int64_t b_bytes) {
    if (a_bytes <= 0 || b_bytes <= 0) return false;
    return a < b + (uintptr_t)b_bytes && b < a + (uintptr_t)a_bytes;
}

}  // namespace

struct attn_f16_plan_s {
    int64_t batch, heads, Sq, Sk, D;
    int64_t qs[3], ks[3], vs[3], os[3];
    int causal, out_type;
    int64_t extent_q, extent_k, extent_v, extent_o;   // elements spanned
    char kernel_name[48];
};

namespace {

int64_t span(int64_t batch, int64_t heads, int64_t rows, int64_t cols, const int64_t st[3]) {
    if (batch == 0 || heads == 0 || rows == 0 || cols == 0) return 0;
    return (batch - 1) * st[0] + (heads - 1) * st[1] + (rows - 1) * st[2] + cols;
}

typedef void (*AttnKernel)(AttnArgs);

AttnKernel pick(int D, bool causal, bool out32) {
    if (D == 64) {
        if (causal) return out32 ? attn_fwd<64, true, true> : attn_fwd<64, true, false>;
        return out32 ? attn_fwd<64, false, true> : attn_fwd<64, false, false>;
    }
    if (causal) return out32 ? attn_fwd<128, true, true> : attn_fwd<128, true, false>;
    return out32 ? attn_fwd<128, false, true> : attn_fwd<128, false, false>;
}

}  // namespace

extern "C" int attn_f16_plan(attn_f16_plan_t *out, int64_t batch, int64_t heads, int64_t Sq,
                             int64_t Sk, int64_t D, const int64_t q_strides[3],
                             const int64_t k_strides[3], const int64_t v_strides[3],
                             const int64_t o_strides[3], int causal, int out_type) {
    if (!out) return GEMM_ERR_INVALID_ARG;
    *out = nullptr;
    if (!q_strides || !k_strides || !v_strides || !o_strides) return GEMM_ERR_INVALID_ARG;
    if (batch < 1 || heads < 1 || Sq < 0 || Sk < 0 || D < 1) return GEMM_ERR_INVALID_ARG;
    if (causal != 0 && causal != 1) return GEMM_ERR_INVALID_ARG;
    if (out_type != GEMM_OUT_F16 && out_type != GEMM_OUT_F32) return GEMM_ERR_INVALID_ARG;
    const int64_t *all[4] = {q_strides, k_strides, v_strides, o_strides};
    for (const int64_t *st : all) {
        if (st[0] < 0 || st[1] < 0 || st[2] < D) return GEMM_ERR_INVALID_ARG;
    }
    if (D != 64 && D != 128) return GEMM_ERR_UNSUPPORTED;
    for (int i = 0; i < 3; ++i)
        for (const int64_t *st : {q_strides, k_strides, v_strides})
            if (st[i] % 8 != 0) return GEMM_ERR_UNSUPPORTED;
    for (int i = 0; i < 3; ++i)
        if (o_strides[i] % 4 != 0) return GEMM_ERR_UNSUPPORTED;
    // 32-bit byte offsets within one (batch, head) slice of Q, K and V.
    const int64_t kMaxSlice = int64_t(1) << 30;
    if ((Sq > 0 && (Sq - 1) * q_strides[2] + D >= kMaxSlice) ||
        (Sk > 0 && (Sk - 1) * k_strides[2] + D >= kMaxSlice) ||
        (Sk > 0 && (Sk - 1) * v_strides[2] + D >= kMaxSlice))
        return GEMM_ERR_UNSUPPORTED;
    const int64_t nqb = (Sq + 127) / 128;
    if (batch * heads * nqb > 0x7fffffff) return GEMM_ERR_UNSUPPORTED;
    attn_f16_plan_s *p = new (std::nothrow) attn_f16_plan_s();
    if (!p) return GEMM_ERR_NOMEM;
    p->batch = batch; p->heads = heads; p->Sq = Sq; p->Sk = Sk; p->D = D;
    for (int i = 0; i < 3; ++i) {
        p->qs[i] = q_strides[i]; p->ks[i] = k_strides[i];
        p->vs[i] = v_strides[i]; p->os[i] = o_strides[i];
    }
    p->causal = causal;
    p->out_type = out_type;
    p->extent_q = span(batch, heads, Sq, D, q_strides);
    p->extent_k = span(batch, heads, Sk, D, k_strides);
    p->extent_v = span(batch, heads, Sk, D, v_strides);
    p->extent_o = span(batch, heads, Sq, D, o_strides);
    if (Sq == 0)
        snprintf(p->kernel_name, sizeof p->kernel_name, "none");
    else
        snprintf(p->kernel_name, sizeof p->kernel_name, "attn_fwd_d%d_q128_k64%s_%s", (int)D,
                 causal ? "_causal" : "", out_type == GEMM_OUT_F32 ? "f32" : "f16");
    *out = p;
    return GEMM_OK;
}

extern "C" int attn_f16_run(attn_f16_plan_t plan, const void *Q, const void *K, const void *V,
                            void *O, float scale, void *stream) {
    if (!plan) return GEMM_ERR_INVALID_ARG;
    const attn_f16_plan_s &p = *plan;
    if (p.Sq == 0) return GEMM_OK;
    if (!Q || !O || (p.Sk > 0 && (!K || !V))) return GEMM_ERR_INVALID_ARG;
    if ((uintptr_t)Q % 16 || (uintptr_t)K % 16 || (uintptr_t)V % 16 || (uintptr_t)O % 16)
        return GEMM_ERR_INVALID_ARG;
    const int64_t obytes = p.extent_o * (p.out_type == GEMM_OUT_F32 ? 4 : 2);
    if (ranges_overlap((uintptr_t)O, obytes, (uintptr_t)Q, p.extent_q * 2) ||
        ranges_overlap((uintptr_t)O, obytes, (uintptr_t)K, p.extent_k * 2) ||
        ranges_overlap((uintptr_t)O, obytes, (uintptr_t)V, p.extent_v * 2))
        return GEMM_ERR_INVALID_ARG;
    AttnArgs a;
    a.Q = (const uint16_t *)Q;
    a.K = (const uint16_t *)K;
    a.V = (const uint16_t *)V;
    a.O = O;
    a.q_sb = p.qs[0]; a.q_sh = p.qs[1]; a.q_ld = p.qs[2];
    a.k_sb = p.ks[0]; a.k_sh = p.ks[1]; a.k_ld = p.ks[2];
    a.v_sb = p.vs[0]; a.v_sh = p.vs[1]; a.v_ld = p.vs[2];
    a.o_sb = p.os[0]; a.o_sh = p.os[1]; a.o_ld = p.os[2];
    a.heads = (int)p.heads;
    a.Sq = (int)p.Sq;
    a.Sk = (int)p.Sk;
    a.nqb = (int)((p.Sq + 127) / 128);
    a.total = (int)(p.batch * p.heads * a.nqb);
    a.c = scale * kLog2e;
    AttnKernel fn = pick((int)p.D, p.causal != 0, p.out_type == GEMM_OUT_F32);
    void *args[] = {&a};
    return hipLaunchKernel((const void *)fn, dim3((unsigned)a.total), dim3(256), args, 0,
                           (hipStream_t)stream) == hipSuccess ? GEMM_OK : GEMM_ERR_HIP;
}

extern "C" int attn_f16_destroy(attn_f16_plan_t plan) {
    delete plan;
    return GEMM_OK;
}

extern "C" const char *attn_f16_plan_kernel(attn_f16_plan_t plan) {
    return plan ? plan->kernel_name : "invalid";
}

extern "C" int attn_softmax_rows(int64_t rows, int64_t cols, const void *x, int64_t ldx,
                                 int in_type, void *y, int64_t ldy, int out_type, void *stream) {
    if (rows < 0 || cols < 0) return GEMM_ERR_INVALID_ARG;
    if ((in_type != GEMM_OUT_F16 && in_type != GEMM_OUT_F32) ||
        (out_type != GEMM_OUT_F16 && out_type != GEMM_OUT_F32))
        return GEMM_ERR_INVALID_ARG;
    if (rows == 0 || cols == 0) return GEMM_OK;
    if (!x || !y || ldx < cols || ldy < cols) return GEMM_ERR_INVALID_ARG;
    if (rows > 0x7fffffff) return GEMM_ERR_UNSUPPORTED;
    const int64_t ib = in_type == GEMM_OUT_F32 ? 4 : 2, ob = out_type == GEMM_OUT_F32 ? 4 : 2;
    const int64_t xbytes = ((rows - 1) * ldx + cols) * ib, ybytes = ((rows - 1) * ldy + cols) * ob;
    const bool in_place = x == y && ib == ob && ldx == ldy;
    if (!in_place && ranges_overlap((uintptr_t)x, xbytes, (uintptr_t)y, ybytes))
        return GEMM_ERR_INVALID_ARG;
    SmArgs a;
    a.x = x;
    a.y = y;
    a.cols = cols;
    a.ldx = ldx;
    a.ldy = ldy;
    const bool i32 = in_type == GEMM_OUT_F32, o32 = out_type == GEMM_OUT_F32;
    typedef void (*SmKernel)(SmArgs);
    // [in fp32][out fp32] per register-resident width, then the two-pass kernel.
    static const SmKernel k2048[2][2] = {{softmax_rows_reg<8, false, false>, softmax_rows_reg<8, false, true>},
                                         {softmax_rows_reg<8, true, false>, softmax_rows_reg<8, true, true>}};
    static const SmKernel k4096[2][2] = {{softmax_rows_reg<16, false, false>, softmax_rows_reg<16, false, true>},
                                         {softmax_rows_reg<16, true, false>, softmax_rows_reg<16, true, true>}};
    static const SmKernel k8192[2][2] = {{softmax_rows_reg<32, false, false>, softmax_rows_reg<32, false, true>},
                                         {softmax_rows_reg<32, true, false>, softmax_rows_reg<32, true, true>}};
    static const SmKernel klong[2][2] = {{softmax_rows_online<false, false>, softmax_rows_online<false, true>},
                                         {softmax_rows_online<true, false>, softmax_rows_online<true, true>}};
    static const SmKernel v2048[2][2] = {{softmax_rows_vec<1, false, false>, softmax_rows_vec<1, false, true>},
                                         {softmax_rows_vec<1, true, false>, softmax_rows_vec<1, true, true>}};
    static const SmKernel v4096[2][2] = {{softmax_rows_vec<2, false, false>, softmax_rows_vec<2, false, true>},
                                         {softmax_rows_vec<2, true, false>, softmax_rows_vec<2, true, true>}};
    static const SmKernel v8192[2][2] = {{softmax_rows_vec<4, false, false>, softmax_rows_vec<4, false, true>},
                                         {softmax_rows_vec<4, true, false>, softmax_rows_vec<4, true, true>}};
    // Whole 16-byte chunks: row length, leading dimensions and bases multiples
    // of 8 elements and 16 bytes.
    const bool vec = cols % 8 == 0 && ldx % 8 == 0 && ldy % 8 == 0 && (uintptr_t)x % 16 == 0 &&
                     (uintptr_t)y % 16 == 0;
    const SmKernel fn = vec && cols <= 8192
        ? (cols <= 2048 ? v2048 : cols <= 4096 ? v4096 : v8192)[i32][o32]
        : (cols <= 2048 ? k2048 : cols <= 4096 ? k4096 : cols <= 8192 ? k8192 : klong)[i32][o32];
    void *args[] = {&a};
    return hipLaunchKernel((const void *)fn, dim3((unsigned)rows), dim3(256), args, 0,
                           (hipStream_t)stream) == hipSuccess ? GEMM_OK : GEMM_ERR_HIP;
}
