// kernels.hip -- gfx950 (MI355X) kernels of the half-precision GEMM library.
//
//  * k_classic_m16 -- classic GEMM, C = A * B (fp32 accumulate, one RNE
//                    cast), 256 x 256 tiles, 8 waves of 128 x 64 on 16x16x32
//                    MFMAs, direct-to-LDS loads (128 x 128 tiles of 8 waves
//                    for long K).  Its partial mode runs one piece of K per
//                    workgroup and writes fp32 partial tiles: for few tiles
//                    (full M x N planes, added by k_split_reduce) or for the
//                    last, partial round of a multi-round grid (compact
//                    tiles, added by k_tail_reduce).
//  * k_classic_q4 -- the same for 128 x 128 tiles: 4 waves (one per SIMD) of
//                    64 x 64 on 32x32x16 MFMAs.
//  * k_skinny     -- M <= 32 products, built to stream B from HBM (private
//                    direct-to-LDS rings per wave, no barrier in the K loop).
//  * k_skinny_shared -- M <= 64 products: one ring shared by the waves of a
//                    workgroup (33..64 rows; up to 32 rows when B has many
//                    column strips).
//  * k_skinny_split, k_split_reduce -- M <= 64 products with K long
//                    against the column strips: the K loop of
//                    k_skinny_shared over one part of K per workgroup, fp32
//                    partials in the workspace, then a second launch adds
//                    them in a fixed order and rounds into C.
//  * k_classic    -- register-staged tiles for the other shapes and for
//                    operands that are not 16-byte aligned.
//  * k_prepass    -- combine-A/B pass: every combined operand of an LCMA scheme,
//                    summed in fp32 and rounded once to the operand type.
//  * k_fused1_m16 -- persistent one-level group kernel on the 16x16x32 engine:
//                    the 7 products of one output coordinate accumulate into
//                    the 4 output tiles in registers (fp32), no product is
//                    written to memory; tail groups may be split over two
//                    workgroups with a last-arriver fp32 fix-up.  Its OUTER
//                    variant runs one outer product of the two-level scheme
//                    (7 inner products on M/4 x N/4 blocks, fused the same
//                    way) and folds the 4 inner outputs into fp32 output
//                    blocks in memory, rounding into C at the last touch.
//  * k_fused_cal_m16 -- the one-level group kernel without a pre-pass: it
//                    loads both input blocks of every combined operand and
//                    adds them in LDS while staging each k-tile.
//  * k_gen_prepass, k_gen_group_m16, k_gen_product -- the unfused
//                    path for any valid description: a runtime-coefficient
//                    combination pass, then the products, each folding W * H
//                    into fp32 output blocks and rounding into C at the last
//                    product feeding a block.  With a round of 256 x 256
//                    positions, one persistent launch runs every product per
//                    position (k_gen_group_m16, reading tile-packed A operands
//                    on whole tiles); otherwise one GEMM launch per product
//                    (128 x 128 tiles on the four-wave engine).
//  * k_fused<2>   -- all 49 products of one output coordinate on one
//                    workgroup (16 outputs on chip, 64 x 64 tiles) on the
//                    register-staged path.
//  * k_ref_mfma, k_ref_copy, k_ref_read -- measured machine references (an
//                    MFMA loop, a device copy, a read-only stream).
//
// Sources: "FalconGEMM: Surpassing Hardware Peaks with Lower-Complexity
// Matrix Multiplication", sections "从 LCMA 到 FalconGEMM" (combine A/B,
// spatial groups accumulated on chip, split over two compute units, L2-aware
// ordering, persistent kernel) and "从缓存重排到 Cost Model" (fp32 on-chip
// combination, one final cast); "CUDA-L2 ..." section "核心贡献与发现的技术"
// (multi-stage staging, wide epilogue stores, block swizzling).
//
// MFMA: v_mfma_f32_16x16x32_{f16,bf16} on the 16x16x32 engine (classic
// 256 x 256 tiles, the fused one-level kernel, the unfused 256 x 256
// products, the on-chip two-level kernel) and v_mfma_f32_32x32x16 on the
// four-wave engine (128 x 128 tiles), the streaming kernel and the
// register-staged fallback.  Operands are fed swapped (the B fragment as the
// A operand), so each lane's accumulators hold 4 consecutive output columns
// of one output row, stored as one 8-byte write (or staged through LDS for
// 16-byte row segments).  The register-staged path stores B transposed in LDS
// (rows padded to 144 bytes); the direct-to-LDS engines keep B row-major as
// in memory, XOR-swizzled, and read it with ds_read_b64_tr_b16.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <mutex>
#include <utility>

#include "kernels.hpp"
#include "schedule.hpp"
#include "strassen.hpp"

namespace lcma {
namespace {

using u16 = uint16_t;
using u32 = uint32_t;
typedef u32 u32x4 __attribute__((ext_vector_type(4)));
typedef u32 u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef __bf16 b8 __attribute__((ext_vector_type(8)));

// MFMA shapes: 32x32x16 (16 fp32 accumulators per lane) and 16x16x32 (4).
template <int MT>
struct Mma;
template <>
struct Mma<32> {
    using acc_t = f32x16;
    static constexpr int NACC = 16;
    static constexpr int KSTEP = 16;
};
template <>
struct Mma<16> {
    using acc_t = f32x4;
    static constexpr int NACC = 4;
    static constexpr int KSTEP = 32;
};

template <bool BF>
__device__ __forceinline__ f32x16 mfma(u32x4 a, u32x4 b, f32x16 c)
{
    if constexpr (BF)
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(b8, a),
                                                       __builtin_bit_cast(b8, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(h8, a),
                                                      __builtin_bit_cast(h8, b), c, 0, 0, 0);
}

template <bool BF>
__device__ __forceinline__ f32x4 mfma(u32x4 a, u32x4 b, f32x4 c)
{
    if constexpr (BF)
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(b8, a),
                                                       __builtin_bit_cast(b8, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8, a),
                                                      __builtin_bit_cast(h8, b), c, 0, 0, 0);
}

// fp32 -> half bits, round to nearest even.
template <bool BF>
__device__ __forceinline__ u16 f2h(float x)
{
    if constexpr (BF)
        return __builtin_bit_cast(u16, (__bf16)x);
    else
        return __builtin_bit_cast(u16, (_Float16)x);
}

template <bool BF>
__device__ __forceinline__ float h2f(u16 x)
{
    if constexpr (BF)
        return __builtin_bit_cast(float, (u32)x << 16);
    else
        return (float)__builtin_bit_cast(_Float16, x);
}

template <bool BF>
__device__ __forceinline__ u32 pack2(float lo, float hi)
{
    return (u32)f2h<BF>(lo) | ((u32)f2h<BF>(hi) << 16);
}

// LDS rows hold 64 halves (128 bytes) padded to 144 bytes: 8 consecutive
// rows at the same 16-byte chunk then start 9 slots apart modulo the 256-byte
// bank width, so the 8 lanes of a 16-byte access phase never share banks,
// and every offset is affine in (row, chunk) (immediate-offset LDS reads).
constexpr u32 kRow = 144;

__device__ __forceinline__ u32 lds_off(u32 row, u32 ch) { return row * kRow + ch * 16u; }

template <int BM_, int BN_, int WM_, int WN_, int MT_ = 32, int BKB_ = 8>
struct Cfg {
    static constexpr int BM = BM_, BN = BN_, BK = 64, WM = WM_, WN = WN_, MT = MT_;
    static constexpr int BKB = BKB_;                      // k rows per staged B block (2, 4 or 8)
    static constexpr int NT = WM * WN * 64;
    static constexpr int WTM = BM / WM, WTN = BN / WN;
    static constexpr int FM = WTM / MT, FN = WTN / MT;
    using acc_t = typename Mma<MT>::acc_t;
    static constexpr int NACC = Mma<MT>::NACC;
    static constexpr int A_CH = BM * 8 / NT;              // 16-byte A chunks per thread
    static constexpr int B_BLK = (BK / BKB) * (BN / 8);   // BKB x 8 B blocks per tile
    static constexpr int B_PER = (B_BLK + NT - 1) / NT;   // B blocks per thread
    static constexpr int A_BYTES = BM * kRow, B_BYTES = BN * kRow;
    static constexpr int STAGE = A_BYTES + B_BYTES;
    static constexpr int LDS = 2 * STAGE;
    static_assert(BM * 8 % NT == 0 && A_CH >= 1, "A tile must split evenly over the threads");
    static_assert(FM >= 1 && FN >= 1, "wave tile must hold one MFMA tile");
    static_assert(LDS <= 160 * 1024, "LDS budget");
    static_assert(BKB == 2 || BKB == 4 || BKB == 8, "B block height");
};

using Cfg256 = Cfg<256, 256, 2, 2, 32, 8>;   // classic: 4 waves of 128 x 128
using Cfg128 = Cfg<128, 128, 2, 2, 32, 4>;   // classic: 4 waves of 64 x 64
using Cfg32 = Cfg<32, 64, 1, 2, 32, 4>;      // classic skinny: 2 waves of 32 x 32
using CfgF2 = Cfg<64, 64, 4, 2, 16, 2>;      // fused two-level: 8 waves of 16 x 32 (16x16x32 MFMA)

// Buffer resources: global loads and stores go through a buffer descriptor
// based at the tile origin with 32-bit byte offsets.  An offset of
// kOob (beyond num_records) reads as zero and drops stores, which handles
// every edge without branches or 64-bit address arithmetic.
constexpr u32 kOob = 0x80000000u;
using rsrc_t = __amdgpu_buffer_rsrc_t;

__device__ __forceinline__ rsrc_t make_rsrc(const void* base)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, 0x7fffffff, 0x00020000);
}

// Where one tile sequence reads from: `a` is the first row of the A tile
// (column 0), `b` is column 0 of the B tile (row 0); rows/cols beyond
// a_rows / b_cols and k beyond K read as zero.  Buffer descriptors are
// re-based at every k-tile so 32-bit offsets stay small for any K (leading
// dimensions are limited to 2^21 elements by the host).
struct Src {
    const u16* a; int lda; int a_rows;
    const u16* b; int ldb; int b_cols;
    int K;
};

__device__ __forceinline__ Src make_src(const u16* a, int64_t lda, int a_rows, const u16* b, int64_t ldb,
                                        int b_cols, int K)
{
    return Src{a, (int)lda, a_rows, b, (int)ldb, b_cols, K};
}

template <class C>
struct Regs {
    u32x4 a[C::A_CH];
    u32x4 b[C::B_PER][C::BKB];
};

__device__ __forceinline__ u32x4 load16(const rsrc_t& r, u32 off)
{
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

// 8 halves starting at element (row, col) of a row-major matrix with leading
// dimension ld; elements with row >= rows or col + x >= cols read as zero.
template <bool VEC>
__device__ __forceinline__ u32x4 load_row8(const rsrc_t& r, int ld, int row, int col, int rows, int cols)
{
    if constexpr (VEC) {
        const u32 off = (row < rows && col < cols) ? (u32)(row * ld + col) * 2u : kOob;
        return load16(r, off);
    } else {
        u32 e[8];
#pragma unroll
        for (int x = 0; x < 8; ++x) {
            const u32 off = (row < rows && col + x < cols) ? (u32)(row * ld + col + x) * 2u : kOob;
            e[x] = __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0);
        }
        return u32x4{e[0] | (e[1] << 16), e[2] | (e[3] << 16), e[4] | (e[5] << 16), e[6] | (e[7] << 16)};
    }
}

// The A chunks of one k-tile: `a` is the tile's first row (column 0).
template <class C, bool VEC>
__device__ __forceinline__ void load_a(u32x4 (&ra8)[C::A_CH], const u16* a, int lda, int a_rows, int k0, int K,
                                       int tid)
{
    const rsrc_t ra = make_rsrc(a + k0);
    const int kleft = K - k0;
#pragma unroll
    for (int i = 0; i < C::A_CH; ++i) {
        const int c = tid + i * C::NT;
        ra8[i] = load_row8<VEC>(ra, lda, c >> 3, (c & 7) * 8, a_rows, kleft);
    }
}

// The B blocks of one k-tile: `b` is the tile's first column (row 0).
template <class C, bool VEC>
__device__ __forceinline__ void load_b(u32x4 (&rb8)[C::B_PER][C::BKB], const u16* b, int ldb, int b_cols, int k0,
                                       int K, int tid)
{
    const rsrc_t rb = make_rsrc(b + (int64_t)k0 * ldb);
    const int kleft = K - k0;
#pragma unroll
    for (int i = 0; i < C::B_PER; ++i) {
        const int blk = tid + i * C::NT;
        if (C::B_BLK % C::NT == 0 || blk < C::B_BLK) {
            const int kb = blk % (C::BK / C::BKB), n = (blk / (C::BK / C::BKB)) * 8;
#pragma unroll
            for (int r = 0; r < C::BKB; ++r)
                rb8[i][r] = load_row8<VEC>(rb, ldb, kb * C::BKB + r, n, kleft, b_cols);
        }
    }
}

template <class C, bool VEC>
__device__ __forceinline__ void load_tile(Regs<C>& R, const Src& s, int k0, int tid)
{
    load_a<C, VEC>(R.a, s.a, s.lda, s.a_rows, k0, s.K, tid);
    load_b<C, VEC>(R.b, s.b, s.ldb, s.b_cols, k0, s.K, tid);
}

// Registers -> LDS stage.  A chunks go straight to their swizzled slot.  Each
// BKB (k) x 8 (n) B block is transposed in registers: output dword (n, k
// pair) takes half n of rows k and k+1 with one byte permute, and column n's
// BKB values are written with one BKB*2-byte LDS store.
template <class C>
__device__ __forceinline__ void store_tile(char* stage, const Regs<C>& R, int tid)
{
    char* sA = stage;
    char* sB = stage + C::A_BYTES;
#pragma unroll
    for (int i = 0; i < C::A_CH; ++i) {
        const int c = tid + i * C::NT;
        *reinterpret_cast<u32x4*>(sA + lds_off(c >> 3, c & 7)) = R.a[i];
    }
#pragma unroll
    for (int i = 0; i < C::B_PER; ++i) {
        const int blk = tid + i * C::NT;
        if (C::B_BLK % C::NT == 0 || blk < C::B_BLK) {
            // consecutive lanes take consecutive k blocks of one 8-column
            // block, so a 16-byte store phase covers 8 distinct rows' slots
            const int kb = blk % (C::BK / C::BKB), nb = blk / (C::BK / C::BKB);
            const int k = kb * C::BKB;               // first k of the block within the tile
#pragma unroll
            for (int n = 0; n < 8; ++n) {
                const int d = n >> 1;
                const u32 sel = (n & 1) ? 0x07060302u : 0x05040100u;
                u32 v[C::BKB / 2];
#pragma unroll
                for (int pr = 0; pr < C::BKB / 2; ++pr)
                    v[pr] = __builtin_amdgcn_perm(R.b[i][2 * pr + 1][d], R.b[i][2 * pr][d], sel);
                char* dst = sB + lds_off(nb * 8 + n, k >> 3) + (k & 7) * 2;
                if constexpr (C::BKB == 8)
                    *reinterpret_cast<u32x4*>(dst) = u32x4{v[0], v[1], v[2], v[3]};
                else if constexpr (C::BKB == 4)
                    *reinterpret_cast<u32x2*>(dst) = u32x2{v[0], v[1]};
                else
                    *reinterpret_cast<u32*>(dst) = v[0];
            }
        }
    }
}

// MFMA fragments of k step `s` of a stage: lane l feeds row (l % MT) of each
// operand tile with 8 consecutive k, k chunk (l / MT) of the step.
template <class C>
__device__ __forceinline__ void read_frags(const char* stage, int s, u32x4 (&af)[C::FM], u32x4 (&bf)[C::FN],
                                           int wm, int wn, int lane)
{
    constexpr int CPS = Mma<C::MT>::KSTEP / 8;   // 16-byte chunks per k step
    const char* sA = stage;
    const char* sB = stage + C::A_BYTES;
    const int r = lane % C::MT, hi = lane / C::MT;
#pragma unroll
    for (int i = 0; i < C::FM; ++i)
        af[i] = *reinterpret_cast<const u32x4*>(sA + lds_off(wm * C::WTM + i * C::MT + r, CPS * s + hi));
#pragma unroll
    for (int j = 0; j < C::FN; ++j)
        bf[j] = *reinterpret_cast<const u32x4*>(sB + lds_off(wn * C::WTN + j * C::MT + r, CPS * s + hi));
}

template <class C, bool BF>
__device__ __forceinline__ void mma_step(const u32x4 (&af)[C::FM], const u32x4 (&bf)[C::FN],
                                         typename C::acc_t (&acc)[C::FM][C::FN])
{
#pragma unroll
    for (int i = 0; i < C::FM; ++i)
#pragma unroll
        for (int j = 0; j < C::FN; ++j)
            acc[i][j] = mfma<BF>(bf[j], af[i], acc[i][j]);
}

// One k-tile from LDS stage `cur`.  Fragments are double-buffered so the
// reads of step s+1 are in flight while step s's MFMAs run.  With MORE, the
// next tile (already loaded into R) is written to stage `nxt` during the last
// MFMA step; `nxt` was last read one tile earlier, before the barrier that
// ended it, so no wave still reads it.
template <class C, bool BF, bool MORE>
__device__ __forceinline__ void ktile(const char* cur, char* nxt, const Regs<C>& R,
                                      typename C::acc_t (&acc)[C::FM][C::FN], int wm, int wn, int lane, int tid)
{
    constexpr int KSTEPS = C::BK / Mma<C::MT>::KSTEP;
    u32x4 af[2][C::FM], bf[2][C::FN];
    read_frags<C>(cur, 0, af[0], bf[0], wm, wn, lane);
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) {
        if (s + 1 < KSTEPS)
            read_frags<C>(cur, s + 1, af[(s + 1) & 1], bf[(s + 1) & 1], wm, wn, lane);
        if (MORE && s == KSTEPS - 1)
            store_tile<C>(nxt, R, tid);
        mma_step<C, BF>(af[s & 1], bf[s & 1], acc);
    }
}

// Stores one accumulator tile: `Cp` is the tile origin, rows/cols the valid
// extent from there.  With operands swapped, lane l holds output row
// (l % MT) and, per group of 4 accumulators, 4 consecutive columns:
// 32x32: column 8*g + 4*(l/32) + e of group g; 16x16: column 4*(l/16) + e.
template <class C, bool BF, bool VEC4>
__device__ __forceinline__ void store_c(const typename C::acc_t (&acc)[C::FM][C::FN], u16* Cp, int64_t ldc,
                                        int rows, int cols, int wm, int wn, int lane)
{
    const rsrc_t rc = make_rsrc(Cp);
    const int ld = (int)ldc;
    const int r = lane % C::MT, hi = lane / C::MT;
#pragma unroll
    for (int i = 0; i < C::FM; ++i) {
        const int m = wm * C::WTM + i * C::MT + r;
#pragma unroll
        for (int j = 0; j < C::FN; ++j)
#pragma unroll
            for (int g = 0; g < C::NACC / 4; ++g) {
                const int n = wn * C::WTN + j * C::MT + (C::MT == 32 ? 8 * g + 4 * hi : 4 * hi);
                const float x0 = acc[i][j][4 * g], x1 = acc[i][j][4 * g + 1];
                const float x2 = acc[i][j][4 * g + 2], x3 = acc[i][j][4 * g + 3];
                if constexpr (VEC4) {
                    // cols is a multiple of 4 here, so the 4 columns are all valid or all not.
                    const u32 off = (m < rows && n < cols) ? (u32)(m * ld + n) * 2u : kOob;
                    __builtin_amdgcn_raw_buffer_store_b64(
                        __builtin_bit_cast(__attribute__((ext_vector_type(2))) unsigned int,
                                           u32x2{pack2<BF>(x0, x1), pack2<BF>(x2, x3)}),
                        rc, off, 0, 0);
                } else {
                    const float xs[4] = {x0, x1, x2, x3};
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const u32 off = (m < rows && n + e < cols) ? (u32)(m * ld + n + e) * 2u : kOob;
                        __builtin_amdgcn_raw_buffer_store_b16(f2h<BF>(xs[e]), rc, off, 0, 0);
                    }
                }
            }
    }
}

template <class C>
__device__ __forceinline__ void zero_acc(typename C::acc_t (&acc)[C::FM][C::FN])
{
#pragma unroll
    for (int i = 0; i < C::FM; ++i)
#pragma unroll
        for (int j = 0; j < C::FN; ++j)
#pragma unroll
            for (int e = 0; e < C::NACC; ++e)
                acc[i][j][e] = 0.0f;
}

// ------------------------------------------------------------------ classic

template <class C, bool BF, bool VEC>
__global__ void __launch_bounds__(C::NT)
k_classic(const u16* __restrict__ A, int64_t lda, const u16* __restrict__ B, int64_t ldb,
          u16* __restrict__ Cm, int64_t ldc, int M, int N, int K, int gy, int gx, int P, int vec4)
{
    __shared__ __attribute__((aligned(16))) char smem[C::LDS];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / C::WN, wn = wave % C::WN;
    int p, q;
    tile_coords((int32_t)blockIdx.x, gy, gx, P, 8, &p, &q);
    const int m0 = p * C::BM, n0 = q * C::BN;
    const Src s = make_src(A + (int64_t)m0 * lda, lda, M - m0, B + n0, ldb, N - n0, K);

    typename C::acc_t acc[C::FM][C::FN];
    zero_acc<C>(acc);
    const int nk = (K + C::BK - 1) / C::BK;
    Regs<C> R;
    load_tile<C, VEC>(R, s, 0, tid);
    store_tile<C>(smem, R, tid);
    __syncthreads();
    // Tile t is computed from stage t % 2 while tile t+1 is fetched into
    // registers and then written to the other stage; one barrier per tile.
    int t = 0;
    for (; t + 1 < nk; ++t) {
        load_tile<C, VEC>(R, s, (t + 1) * C::BK, tid);
        ktile<C, BF, true>(smem + (t & 1) * C::STAGE, smem + ((t + 1) & 1) * C::STAGE, R, acc, wm, wn, lane, tid);
        __syncthreads();
    }
    if (t < nk)
        ktile<C, BF, false>(smem + (t & 1) * C::STAGE, nullptr, R, acc, wm, wn, lane, tid);
    if (vec4)
        store_c<C, BF, true>(acc, Cm + (int64_t)m0 * ldc + n0, ldc, M - m0, N - n0, wm, wn, lane);
    else
        store_c<C, BF, false>(acc, Cm + (int64_t)m0 * ldc + n0, ldc, M - m0, N - n0, wm, wn, lane);
}

template <class C, bool BF, bool VEC>
hipError_t launch_classic_t(const ClassicLaunch& L, hipStream_t st)
{
    const int gy = (L.M + C::BM - 1) / C::BM, gx = (L.N + C::BN - 1) / C::BN;
    const long tiles = (long)gy * gx;
    if (tiles == 0)
        return hipSuccess;
    hipLaunchKernelGGL((k_classic<C, BF, VEC>), dim3((unsigned)tiles), dim3(C::NT), 0, st,
                       (const u16*)L.A, L.lda, (const u16*)L.B, L.ldb, (u16*)L.C, L.ldc, L.M, L.N, L.K,
                       gy, gx, L.P, L.vec4);
    return hipGetLastError();
}

template <class C>
hipError_t launch_classic_c(const ClassicLaunch& L, hipStream_t st)
{
    if (L.bf16)
        return L.vec ? launch_classic_t<C, true, true>(L, st) : launch_classic_t<C, true, false>(L, st);
    return L.vec ? launch_classic_t<C, false, true>(L, st) : launch_classic_t<C, false, false>(L, st);
}

// ------------------------------------------------------------------ pre-pass

template <int LEVELS, bool ALL>
constexpr bool written_a(int r)
{
    int nnz = 0;
    for (int i = 0; i < Scheme<LEVELS>::S; ++i)
        for (int k = 0; k < Scheme<LEVELS>::S; ++k)
            nnz += Scheme<LEVELS>::u(r, i, k) != 0;
    return ALL || nnz > 1;
}

template <int LEVELS, bool ALL>
constexpr bool written_b(int r)
{
    int nnz = 0;
    for (int k = 0; k < Scheme<LEVELS>::S; ++k)
        for (int j = 0; j < Scheme<LEVELS>::S; ++j)
            nnz += Scheme<LEVELS>::v(r, k, j) != 0;
    return ALL || nnz > 1;
}

template <int LEVELS, bool ALL, bool SIDE_B>
constexpr int slot_of(int r)
{
    int s = 0;
    for (int x = 0; x < r; ++x)
        s += SIDE_B ? written_b<LEVELS, ALL>(x) : written_a<LEVELS, ALL>(x);
    return s;
}

struct PrepassParams {
    const u16* A; int64_t lda;
    const u16* B; int64_t ldb;
    int Mb, Kb, Nb;
    u16* outA; u16* outB;
    int64_t strideA, strideB;
    int blocksA;
    int* counters; int n_counters;
};

// One product's combination for one 8-element chunk: fp32 sum of the
// coefficient-weighted blocks in block order, then one RNE rounding.
template <int LEVELS, bool SIDE_B, bool OBF, int R>
__device__ __forceinline__ void combine_one(const float (&x)[Scheme<LEVELS>::S * Scheme<LEVELS>::S][8],
                                            u16* dst)
{
    constexpr int S = Scheme<LEVELS>::S;
    float acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e)
        acc[e] = 0.0f;
    [&]<int... B>(std::integer_sequence<int, B...>) {
        ([&] {
            constexpr int c = SIDE_B ? Scheme<LEVELS>::v(R, B / S, B % S) : Scheme<LEVELS>::u(R, B / S, B % S);
            if constexpr (c != 0) {
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    acc[e] += (float)c * x[B][e];
            }
        }(), ...);
    }(std::make_integer_sequence<int, S * S>{});
    *reinterpret_cast<u32x4*>(dst) = u32x4{pack2<OBF>(acc[0], acc[1]), pack2<OBF>(acc[2], acc[3]),
                                           pack2<OBF>(acc[4], acc[5]), pack2<OBF>(acc[6], acc[7])};
}

template <int LEVELS, bool IBF, bool OBF, bool ALL>
__global__ void __launch_bounds__(256) k_prepass(const PrepassParams pp)
{
    constexpr int S = Scheme<LEVELS>::S, R = Scheme<LEVELS>::R;
    if (blockIdx.x == 0)
        for (int i = threadIdx.x; i < pp.n_counters; i += blockDim.x)
            pp.counters[i] = 0;
    const bool side_b = (int)blockIdx.x >= pp.blocksA;
    const int64_t idx = (int64_t)(side_b ? blockIdx.x - pp.blocksA : blockIdx.x) * blockDim.x + threadIdx.x;
    // A side: positions (i, j8) over Mb x Kb/8 of each block; B side: (k, j8) over Kb x Nb/8.
    const int cols8 = side_b ? pp.Nb / 8 : pp.Kb / 8;
    const int rows = side_b ? pp.Kb : pp.Mb;
    if (idx >= (int64_t)rows * cols8)
        return;
    const int i = (int)(idx / cols8), j = (int)(idx % cols8) * 8;
    const u16* src = side_b ? pp.B : pp.A;
    const int64_t ld = side_b ? pp.ldb : pp.lda;
    const int br = side_b ? pp.Kb : pp.Mb;   // block rows
    const int bc = side_b ? pp.Nb : pp.Kb;   // block cols
    float x[S * S][8];
#pragma unroll
    for (int b = 0; b < S * S; ++b) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(src + (int64_t)((b / S) * br + i) * ld + (b % S) * bc + j);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            x[b][2 * e] = h2f<IBF>((u16)(v[e] & 0xffffu));
            x[b][2 * e + 1] = h2f<IBF>((u16)(v[e] >> 16));
        }
    }
    const int64_t off = (int64_t)i * bc + j;
    if (!side_b) {
        [&]<int... Rs>(std::integer_sequence<int, Rs...>) {
            ([&] {
                if constexpr (written_a<LEVELS, ALL>(Rs))
                    combine_one<LEVELS, false, OBF, Rs>(x, pp.outA + slot_of<LEVELS, ALL, false>(Rs) * pp.strideA + off);
            }(), ...);
        }(std::make_integer_sequence<int, R>{});
    } else {
        [&]<int... Rs>(std::integer_sequence<int, Rs...>) {
            ([&] {
                if constexpr (written_b<LEVELS, ALL>(Rs))
                    combine_one<LEVELS, true, OBF, Rs>(x, pp.outB + slot_of<LEVELS, ALL, true>(Rs) * pp.strideB + off);
            }(), ...);
        }(std::make_integer_sequence<int, R>{});
    }
}

template <int LEVELS, bool IBF, bool OBF, bool ALL>
hipError_t launch_prepass_t(const PrepassLaunch& L, hipStream_t st)
{
    PrepassParams pp;
    pp.A = (const u16*)L.A; pp.lda = L.lda;
    pp.B = (const u16*)L.B; pp.ldb = L.ldb;
    pp.Mb = L.Mb; pp.Kb = L.Kb; pp.Nb = L.Nb;
    pp.outA = (u16*)L.outA; pp.outB = (u16*)L.outB;
    pp.strideA = L.strideA; pp.strideB = L.strideB;
    pp.counters = L.counters; pp.n_counters = L.n_counters;
    const int64_t na = (int64_t)L.Mb * (L.Kb / 8), nb = (int64_t)L.Kb * (L.Nb / 8);
    pp.blocksA = (int)((na + 255) / 256);
    const int blocks = pp.blocksA + (int)((nb + 255) / 256);
    if (blocks == 0)
        return hipSuccess;
    hipLaunchKernelGGL((k_prepass<LEVELS, IBF, OBF, ALL>), dim3(blocks), dim3(256), 0, st, pp);
    return hipGetLastError();
}

// ------------------------------------------------------------------ ping-pong engine
//
// The fast path for 16-byte aligned operands.  A workgroup of 8 waves owns a
// BM x BN output tile; waves w and w+4 share a SIMD.  Tiles of 32 k are
// copied global -> LDS by direct (LDS-DMA) buffer loads into a ring of 4
// stages, two tiles ahead of use, so no VGPR staging and no VALU transposes
// are needed:
//   * A stage: BM rows of 32 k (64 bytes, four 16-byte chunks); logical chunk
//     c of row m sits at chunk c ^ ((m >> 2) & 3).  16 consecutive rows then
//     cover all 16 bank slots, so the 16-byte MFMA operand reads are
//     conflict free.
//   * B stage: 32 k rows of BN columns (row-major, as in memory); logical
//     16-byte chunk c of row k sits at chunk c ^ (4 * (k & 3)).  The MFMA
//     operand (8 consecutive k of one column per lane) is read with two
//     ds_read_b64_tr_b16: within each 16-lane group, source lane s points at
//     B[k0 + s/4][n0 + 4 (s % 4)] and lane i receives B[k0..k0+3][n0 + i].
// The two waves of a SIMD alternate phases: while one issues the k-tile's
// MFMAs from registers, the other reads the next k-tile's fragments from LDS
// (and, for waves 0-3, issues the DMA of the tile two ahead).  A raw
// s_barrier separates phases; explicit waitcnts order the DMA and the reads.
namespace tiles {

typedef short s16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xC07F); }       // lgkmcnt(0)
__device__ __forceinline__ void wait_vm0() { __builtin_amdgcn_s_waitcnt(0x0F70); }         // vmcnt(0)
__device__ __forceinline__ void bar() { asm volatile("s_barrier" ::: "memory"); }

__device__ __forceinline__ u32 a_swz(u32 m) { return (m >> 2) & 3u; }
__device__ __forceinline__ u32 b_swz(u32 k) { return 4u * (k & 3u); }

// Where k-tile data comes from: A rows from `a` (a_rows valid), B columns
// from `b` (b_cols valid), k0 of K.
struct TileSrc {
    const u16* a; int lda; int a_rows;
    const u16* b; int ldb; int b_cols;
    int k0, K;
};

}  // namespace tiles



// ------------------------------------------------------------------ four-wave engine
//
// One wave per SIMD on v_mfma_f32_32x32x16, a 2 x 2 grid of wave tiles
// (here 128 x 128 workgroup tiles: 64 x 64 per wave, 4 MFMA tiles, 64
// accumulator registers).  k-tiles of 32 stream through a 4-stage LDS ring
// by direct-to-LDS loads issued 3 tiles ahead; fragments are double-buffered
// in registers by k-step, so the LDS reads of one k-step run under the MFMAs
// of the other.  One barrier per k-tile.  Used for classic products whose
// 256 x 256 tiles would not fill the compute units, and for the unfused
// path's products of that size.

namespace q4 {

template <int BM_, int BN_>
struct QCfg {
    static constexpr int BM = BM_, BN = BN_, BK = 32, WM = 2, WN = 2, MT = 32;
    static constexpr int NSTAGE = 4, KSTEPS = 2, AHEAD = 3;
    static constexpr int NW = WM * WN;
    static constexpr int NT = NW * 64;
    static constexpr int WTM = BM / WM, WTN = BN / WN;
    static constexpr int FM = WTM / 32, FN = WTN / 32;
    using acc_t = f32x16;
    static constexpr int NACC = 16;
    static constexpr int AROW = BK * 2;
    static constexpr int BROW = BN * 2;
    static constexpr int A_BYTES = BM * AROW;
    static constexpr int B_BYTES = BK * BROW;
    static constexpr int STAGE = A_BYTES + B_BYTES;
    static constexpr int LDS = NSTAGE * STAGE;
    static constexpr int LOADERS = NW;
    static constexpr int A_PER = A_BYTES / 1024 / LOADERS;
    static constexpr int B_PER = B_BYTES / 1024 / LOADERS;
    static constexpr int PER = A_PER + B_PER;                // DMA instructions per wave per k-tile
    static constexpr int SROW = WTN * 2 + 8;                 // staged output row (padded: conflict-free)
    static constexpr int EPI = NW * WTM * SROW;              // output staging, all waves
    static constexpr int LDS_ALLOC = LDS > EPI ? LDS : EPI;
    static_assert(A_BYTES % (1024 * LOADERS) == 0 && B_BYTES % (1024 * LOADERS) == 0, "DMA split");
    static_assert(BROW % 256 == 0 && FM >= 1 && FN >= 1, "tile shape");
    static_assert(LDS <= 160 * 1024 && EPI <= 160 * 1024, "LDS budget");
    static_assert(PER * (AHEAD - 1) < 64, "outstanding DMA count fits the 6-bit vmcnt");
    static_assert(WTN % 8 == 0 && 64 % (WTN / 8) == 0 || WTN % 512 == 0, "staged output rows of 8-column chunks");
    // LDS swizzles (XOR on the 16-byte chunk index of a row): the 32x32x16
    // fragment reads below hit distinct banks with these.
    __device__ static u32 a_swz(u32 m) { return tiles::a_swz(m); }
    __device__ static u32 b_swz(u32 k) { return tiles::b_swz(k); }
};

// Fragments of one k-step (16 k) of a wave tile.
template <class C>
struct Step {
    u32x4 a[C::FM];
    u32x4 b[C::FN];
};

template <class C, bool BF>
__device__ __forceinline__ void mma_step(const Step<C>& F, f32x16 (&acc)[C::FM][C::FN])
{
#pragma unroll
    for (int i = 0; i < C::FM; ++i)
#pragma unroll
        for (int j = 0; j < C::FN; ++j)
            acc[i][j] = mfma<BF>(F.b[j], F.a[i], acc[i][j]);
}

// Buffer descriptor words (base, no stride, 2^31 - 1 bytes, raw dwords),
// matching make_rsrc.
__device__ __forceinline__ u32x4 rsrc_words(const void* base)
{
    const uint64_t a = (uint64_t)(uintptr_t)base;
    return u32x4{(u32)a, (u32)(a >> 32) & 0xffffu, 0x7fffffffu, 0x00020000u};
}

__device__ __forceinline__ u32 lds_addr(const void* p)
{
    return (u32)(uintptr_t)(__attribute__((address_space(3))) const char*)p;
}

// One direct-to-LDS load of 16 bytes per lane: buffer bytes at `off` go to
// LDS address lds + 16 * lane.  Written as inline assembly so the compiler
// does not treat it as a possible writer of every later LDS read (it would
// otherwise drain vmcnt before each transposed read); the kernels order these
// loads against LDS reads themselves with vmcnt waits and barriers.  The
// LDS address goes in M0, which must be written one instruction ahead of
// the load.
__device__ __forceinline__ void dma16(u32x4 rs, u32 off, u32 lds)
{
    asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
                 :
                 : "v"(off), "s"(rs), "{m0}"(lds)
                 : "memory");
}

// Instruction i (0 .. PER-1) of wave xw's share of a k-tile DMA: the first
// A_PER move A rows, the rest B rows.
template <class C, bool EDGE>
__device__ __forceinline__ void dma_one(char* stage, const tiles::TileSrc& s, int xw, int lane, int i)
{
    const int kleft = s.K - s.k0;
    const u32 base = lds_addr(stage);
    if (i < C::A_PER) {
        const int ins = xw * C::A_PER + i;
        const int r = ins * 16 + (lane >> 2);
        const int k = ((lane & 3) ^ (int)C::a_swz(r)) * 8;
        const u32 off0 = (u32)(r * s.lda + k) * 2u;
        const u32 off = !EDGE || ((r < s.a_rows) & (k < kleft)) ? off0 : kOob;
        dma16(rsrc_words(s.a + s.k0), off, base + ins * 1024);
    } else {
        const int ins = xw * C::B_PER + (i - C::A_PER);
        const int byte = ins * 1024 + lane * 16;
        const int r = byte / C::BROW;
        const int n = (((byte % C::BROW) >> 4) ^ (int)C::b_swz(r)) * 8;
        const u32 off0 = (u32)(r * s.ldb + n) * 2u;
        const u32 off = !EDGE || ((r < kleft) & (n < s.b_cols)) ? off0 : kOob;
        dma16(rsrc_words(s.b + (int64_t)s.k0 * s.ldb), off, base + C::A_BYTES + ins * 1024);
    }
}

// DMA of wave xw's share of one k-tile into `stage`.
template <class C, bool EDGE>
__device__ __forceinline__ void dma_tile(char* stage, const tiles::TileSrc& s, int xw, int lane)
{
#pragma unroll
    for (int i = 0; i < C::PER; ++i)
        dma_one<C, EDGE>(stage, s, xw, lane, i);
}

// Interior tiles: one wave's A loads (or B loads) of a k-tile share one M0.  The load's immediate offset moves both the buffer address
// and the LDS address, so load i uses offset 1024 i with its buffer offset
// lowered by the same amount.  With K a multiple of 32 (so lda, ldb >= 32)
// every lowered offset stays non-negative.  The offsets do not depend on the
// k-tile: the descriptor base moves instead.
template <class C>
struct Group {
    u32 a[C::A_PER];
    u32 b[C::B_PER];
};

// PK: A is tile-packed (see dma_group), so a wave's A loads read its
// A_PER kilobytes of the k-tile's block in order, lane l at 16 l.
template <class C, bool PK = false>
__device__ __forceinline__ Group<C> group_offsets(const tiles::TileSrc& s, int xw, int lane)
{
    static_assert(C::A_PER == C::B_PER && (C::A_PER == 1 || C::A_PER == 2 || C::A_PER == 4), "loads per group");
    Group<C> g;
#pragma unroll
    for (int i = 0; i < C::A_PER; ++i) {
        if constexpr (PK) {
            g.a[i] = (u32)(xw * C::A_PER * 1024 + lane * 16);
        } else {
            const int ins = xw * C::A_PER + i;
            const int r = ins * 16 + (lane >> 2);
            const int k = ((lane & 3) ^ (int)C::a_swz(r)) * 8;
            g.a[i] = (u32)(r * s.lda + k) * 2u - 1024u * i;
        }
    }
#pragma unroll
    for (int i = 0; i < C::B_PER; ++i) {
        const int ins = xw * C::B_PER + i;
        const int byte = ins * 1024 + lane * 16;
        const int r = byte / C::BROW;
        const int n = (((byte % C::BROW) >> 4) ^ (int)C::b_swz(r)) * 8;
        g.b[i] = (u32)(r * s.ldb + n) * 2u - 1024u * i;
    }
    return g;
}

template <int N>
__device__ __forceinline__ void dma16xN(u32x4 rs, const u32 (&off)[N], u32 lds)
{
    static_assert(N == 1 || N == 2 || N == 4, "group size");
    if constexpr (N == 1)
        asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds" : : "v"(off[0]), "s"(rs), "{m0}"(lds) : "memory");
    else if constexpr (N == 4)
        asm volatile("s_nop 0\n\t"
                     "buffer_load_dwordx4 %0, %4, 0 offen lds\n\t"
                     "buffer_load_dwordx4 %1, %4, 0 offen offset:1024 lds\n\t"
                     "buffer_load_dwordx4 %2, %4, 0 offen offset:2048 lds\n\t"
                     "buffer_load_dwordx4 %3, %4, 0 offen offset:3072 lds"
                     :
                     : "v"(off[0]), "v"(off[1]), "v"(off[2]), "v"(off[3]), "s"(rs), "{m0}"(lds)
                     : "memory");
    else
        asm volatile("s_nop 0\n\t"
                     "buffer_load_dwordx4 %0, %2, 0 offen lds\n\t"
                     "buffer_load_dwordx4 %1, %2, 0 offen offset:1024 lds"
                     :
                     : "v"(off[0]), "v"(off[1]), "s"(rs), "{m0}"(lds)
                     : "memory");
}

// Wave xw's A loads (side 0) or B loads (side 1) of k-tile source s into `stage`.
// PK: A is tile-packed: s.a is the first row of a BM-row tile row, whose
// k-tile t is one contiguous block of BM x BK elements at s.a + t BK BM, laid
// out byte for byte as the stage's A part (rows of BK elements, 16-byte
// chunks XOR-swizzled by row), so every load reads whole cache lines.
template <class C, bool PK = false>
__device__ __forceinline__ void dma_group(char* stage, const tiles::TileSrc& s, const Group<C>& g, int xw, int side)
{
    const u32 base = lds_addr(stage);
    if (side == 0)
        dma16xN<C::A_PER>(rsrc_words(PK ? s.a + (int64_t)s.k0 * C::BM : s.a + s.k0), g.a, base + xw * C::A_PER * 1024);
    else
        dma16xN<C::B_PER>(rsrc_words(s.b + (int64_t)s.k0 * s.ldb), g.b, base + C::A_BYTES + xw * C::B_PER * 1024);
}

// s_waitcnt vmcnt(N): vmcnt is split over bits 3:0 and 15:14; expcnt and
// lgkmcnt at their maxima (no wait).
template <int N>
__device__ __forceinline__ void wait_vm()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// Wait until at most n k-tiles of this wave's loads are in flight
// (n is capped at AHEAD - 1; n <= 0 waits for all).
template <class C, int K = C::AHEAD - 1>
__device__ __forceinline__ void wait_tiles(int n)
{
    if constexpr (K <= 0) {
        tiles::wait_vm0();
    } else {
        if (n >= K)
            wait_vm<K * C::PER>();
        else
            wait_tiles<C, K - 1>(n);
    }
}


// Single LDS reads of a k-step's fragments, so they can be slotted between
// MFMAs: A fragment i (one 16-byte read) and half h of B fragment j (one
// transposed 8-byte read; h = 0 covers k 0..7 of the step, h = 1 k 8..15).
template <class C>
struct Addr {
    u32 a0;     // A byte offset of fragment 0 at k-step 0
    u32 b[C::FN];
};

template <class C>
__device__ __forceinline__ Addr<C> frag_addr(int wm, int wn, int lane)
{
    Addr<C> ad;
    const u32 m = wm * C::WTM + (lane & 31);
    const u32 f = C::a_swz(m);
    ad.a0 = m * (u32)C::AROW + ((((lane >> 5) ^ f) & 1u) << 4) + ((f & 2u) << 4);
    const int g = lane >> 4, s = lane & 15;
    const u32 kr = 8 * (g >> 1) + (s >> 2);
    const u32 xb = C::b_swz(kr);
#pragma unroll
    for (int j = 0; j < C::FN; ++j) {
        const u32 n = wn * C::WTN + j * 32 + 16 * (g & 1) + 4 * (s & 3);
        ad.b[j] = C::A_BYTES + kr * C::BROW + (((n >> 3) ^ xb) << 4) + (n & 7) * 2;
    }
    return ad;
}

// Read number x (0 .. FM + 2 FN - 1) of k-step st from `stage`.
template <class C>
__device__ __forceinline__ void read_one(const char* stage, const Addr<C>& ad, int st, int x, Step<C>& F,
                                         u32x2 (&bh)[C::FN][2])
{
    if (x < C::FM) {
        F.a[x] = *reinterpret_cast<const u32x4*>(stage + (ad.a0 ^ ((u32)st << 5)) + x * 32 * C::AROW);
    } else {
        const int y = x - C::FM, j = y >> 1, h = y & 1;
        const tiles::s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) tiles::s16x4*)(stage + ad.b[j] + (16 * st + 4 * h) * C::BROW));
        bh[j][h] = __builtin_bit_cast(u32x2, v);
    }
}

template <class C>
__device__ __forceinline__ void join_b(Step<C>& F, const u32x2 (&bh)[C::FN][2])
{
#pragma unroll
    for (int j = 0; j < C::FN; ++j)
        F.b[j] = u32x4{bh[j][0].x, bh[j][0].y, bh[j][1].x, bh[j][1].y};
}

}  // namespace q4

namespace q4 {

// K loop of one output tile through the four-wave engine; k-tile t's
// operands come from src(t), and after(t) runs once k-tile t's MFMAs are
// issued (a fused group folds a finished product into its outputs there).
// Both are called exactly once per k-tile, in increasing t; with GROUPED,
// src(0) is called once more first.
// Direct-to-LDS loads for tile t+3 are slotted between MFMAs, half in each
// k-step, into the stage tile t-1 used (free once this tile's barrier has
// passed).  EDGE applies the row / column / k bounds to the loads; tiles
// wholly inside the operands skip them.  GROUPED issues each half as one
// group under one M0 (offsets computed once: every k-tile must share the
// leading dimensions of src(0)).
template <class C, bool BF, bool EDGE, bool GROUPED, class SrcFn, class AfterFn>
__device__ __forceinline__ void run_tile(char* smem, int nk, SrcFn src, AfterFn after, int wave, int lane,
                                         const Addr<C>& ad, f32x16 (&acc)[C::FM][C::FN])
{
    constexpr int NMF = C::FM * C::FN;
    constexpr int NRD = C::FM + 2 * C::FN;          // LDS reads per k-step
    constexpr int RPS = 3;                          // reads slotted after one MFMA
    constexpr int HALF = C::PER / 2;                // loads per k-step
    constexpr int LSLOT = NRD / RPS;                // first load slot
    constexpr int STEP = NMF - LSLOT >= 2 * HALF ? 2 : 1;
    static_assert(NRD % RPS == 0 && C::PER % 2 == 0 && LSLOT + STEP * (HALF - 1) < NMF, "interleave slots");
    static_assert(C::AHEAD == 3 && C::NSTAGE == 4, "stage reuse below assumes a 4-stage ring, 3 ahead");
    static_assert(C::A_PER == HALF && C::B_PER == HALF, "first half loads A, second half B");
    static_assert(!(GROUPED && EDGE), "grouped loads carry no bounds");
    Step<C> F0, F1;
    u32x2 bh[C::FN][2];
    Group<C> go;
    if constexpr (GROUPED)
        go = group_offsets<C>(src(0), wave, lane);
#pragma unroll
    for (int t = 0; t < C::AHEAD; ++t) {
        if (t < nk) {
            if constexpr (GROUPED) {
                dma_group<C>(smem + t * C::STAGE, src(t), go, wave, 0);
                dma_group<C>(smem + t * C::STAGE, src(t), go, wave, 1);
            } else {
                dma_tile<C, EDGE>(smem + t * C::STAGE, src(t), wave, lane);
            }
        }
    }
    wait_tiles<C>(min(nk, C::AHEAD) - 1);
    tiles::bar();
    if (nk > 0) {
#pragma unroll
        for (int x = 0; x < NRD; ++x)
            read_one<C>(smem, ad, 0, x, F0, bh);
        join_b<C>(F0, bh);
    }
    int t = 0;
    // Steady state: every k-tile has a successor and a tile to prefetch.
    for (; t + C::AHEAD < nk; ++t) {
        const char* cur = smem + (t % C::NSTAGE) * C::STAGE;
        const char* nxt = smem + ((t + 1) % C::NSTAGE) * C::STAGE;
        char* pre = smem + ((t + C::AHEAD) % C::NSTAGE) * C::STAGE;
        const tiles::TileSrc ps = src(t + C::AHEAD);
        // k-step 0 MFMAs; k-step 1 reads and the first half of the prefetch
#pragma unroll
        for (int x = 0; x < NMF; ++x) {
            acc[x / C::FN][x % C::FN] = mfma<BF>(F0.b[x % C::FN], F0.a[x / C::FN], acc[x / C::FN][x % C::FN]);
            __builtin_amdgcn_sched_barrier(0);
            if (x < NRD / RPS) {
#pragma unroll
                for (int r = 0; r < RPS; ++r)
                    read_one<C>(cur, ad, 1, x * RPS + r, F1, bh);
            } else if constexpr (GROUPED) {
                if (x == LSLOT)
                    dma_group<C>(pre, ps, go, wave, 0);
            } else {
                if (x >= LSLOT && (x - LSLOT) % STEP == 0 && (x - LSLOT) / STEP < HALF)
                    dma_one<C, EDGE>(pre, ps, wave, lane, (x - LSLOT) / STEP);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        join_b<C>(F1, bh);
        wait_vm<C::PER>();      // tile t+1 landed (at most one tile's loads in flight)
        tiles::wait_lgkm0();       // k-step 1 fragments are in registers
        tiles::bar();
        __builtin_amdgcn_sched_barrier(0);
        // k-step 1 MFMAs; next tile's k-step 0 reads and the second half of the prefetch
#pragma unroll
        for (int x = 0; x < NMF; ++x) {
            acc[x / C::FN][x % C::FN] = mfma<BF>(F1.b[x % C::FN], F1.a[x / C::FN], acc[x / C::FN][x % C::FN]);
            __builtin_amdgcn_sched_barrier(0);
            if (x < NRD / RPS) {
#pragma unroll
                for (int r = 0; r < RPS; ++r)
                    read_one<C>(nxt, ad, 0, x * RPS + r, F0, bh);
            } else if constexpr (GROUPED) {
                if (x == LSLOT)
                    dma_group<C>(pre, ps, go, wave, 1);
            } else {
                if (x >= LSLOT && (x - LSLOT) % STEP == 0 && (x - LSLOT) / STEP < HALF)
                    dma_one<C, EDGE>(pre, ps, wave, lane, HALF + (x - LSLOT) / STEP);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        join_b<C>(F0, bh);
        after(t);
        __builtin_amdgcn_sched_barrier(0);
    }
    // Last AHEAD k-tiles: nothing left to prefetch.
    for (; t < nk; ++t) {
        const char* cur = smem + (t % C::NSTAGE) * C::STAGE;
#pragma unroll
        for (int x = 0; x < NRD; ++x)
            read_one<C>(cur, ad, 1, x, F1, bh);
        join_b<C>(F1, bh);
        mma_step<C, BF>(F0, acc);
        if (t + 1 < nk) {
            wait_tiles<C>(nk - 2 - t);
            tiles::wait_lgkm0();
            tiles::bar();
#pragma unroll
            for (int x = 0; x < NRD; ++x)
                read_one<C>(smem + ((t + 1) % C::NSTAGE) * C::STAGE, ad, 0, x, F0, bh);
            join_b<C>(F0, bh);
        }
        mma_step<C, BF>(F1, acc);
        after(t);
    }
}

// Output tile store through LDS.  Straight from the accumulators each store
// instruction covers 32 rows with 8 bytes per lane; here each wave first
// writes its bf16/f16 sub-tile into a private LDS region (rows padded by 8
// bytes, so the 32 rows of a write land in distinct banks), then reads it
// back a row segment at a time and stores 16 bytes per lane, WTN*2 bytes per
// row contiguous.  The caller passes a barrier first: the regions overlap the
// LDS ring other waves may still read.  rows / cols: valid extent from the
// tile origin Cp (cols a multiple of 8 and Cp 16-byte aligned, ldc a
// multiple of 8).
template <class C, bool BF>
__device__ __forceinline__ void store_c_staged(const f32x16 (&acc)[C::FM][C::FN], char* smem, u16* Cp, int64_t ldc,
                                               int rows, int cols, int wave, int wm, int wn, int lane)
{
    char* reg = smem + wave * C::WTM * C::SROW;
    const int r = lane & 31, hi = lane >> 5;
#pragma unroll
    for (int i = 0; i < C::FM; ++i)
#pragma unroll
        for (int j = 0; j < C::FN; ++j)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int row = i * 32 + r, col = j * 32 + 8 * g + 4 * hi;
                const u32x2 v{pack2<BF>(acc[i][j][4 * g], acc[i][j][4 * g + 1]),
                              pack2<BF>(acc[i][j][4 * g + 2], acc[i][j][4 * g + 3])};
                *reinterpret_cast<u32x2*>(reg + row * C::SROW + col * 2) = v;
            }
    tiles::wait_lgkm0();
    const rsrc_t rc = make_rsrc(Cp);
    const int ld = (int)ldc;
    constexpr int CHUNKS = C::WTN / 8;            // 16-byte chunks per staged row
    constexpr int RPI = 64 / CHUNKS;              // rows per store instruction
#pragma unroll
    for (int r0 = 0; r0 < C::WTM; r0 += RPI) {
        const int row = r0 + lane / CHUNKS, ch = lane % CHUNKS;
        const u32x4 v = *reinterpret_cast<const u32x4*>(reg + row * C::SROW + ch * 16);
        const int m = wm * C::WTM + row, n = wn * C::WTN + ch * 8;
        const u32 off = (m < rows && n < cols) ? (u32)(m * ld + n) * 2u : kOob;
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(__attribute__((ext_vector_type(4))) unsigned int, v),
                                               rc, off, 0, 0);
    }
}

}  // namespace q4

// ------------------------------------------------------------------ 16x16 engine
//
// The direct-to-LDS engine on v_mfma_f32_16x16x32: on random bf16 data
// 16x16x32 MFMAs sustain about 15% more flops than 32x32x16 (the chip holds
// a higher clock).  Eight waves, two per SIMD, each own 128 x 64 of a
// 256 x 256 tile: 32 accumulator tiles (128 registers) per wave, which the
// compiler keeps in place (64 tiles per wave it does not).  A k-tile of 32
// is one MFMA k-step, so fragments are double-buffered across k-tiles: the
// reads of tile t+1 are slotted among tile t's MFMAs, and the other wave of
// the SIMD covers their latency.

namespace m16 {

template <int BM_, int BN_, int WM_, int WN_, int AHEAD_ = 3>
struct Cfg {
    static constexpr int BM = BM_, BN = BN_, BK = 32, WM = WM_, WN = WN_, MT = 16;
    static constexpr int AHEAD = AHEAD_, NSTAGE = AHEAD_ + 1;   // k-tiles loaded ahead; LDS ring stages
    static constexpr int NW = WM * WN;
    static constexpr int NT = NW * 64;
    static constexpr int WTM = BM / WM, WTN = BN / WN;
    static constexpr int FM = WTM / 16, FN = WTN / 16;
    using acc_t = f32x4;
    static constexpr int NACC = 4;
    static constexpr int AROW = BK * 2;
    static constexpr int BROW = BN * 2;
    static constexpr int A_BYTES = BM * AROW;
    static constexpr int B_BYTES = BK * BROW;
    static constexpr int STAGE = A_BYTES + B_BYTES;
    static constexpr int LDS = NSTAGE * STAGE;
    static constexpr int LOADERS = NW;
    static constexpr int A_PER = A_BYTES / 1024 / LOADERS;
    static constexpr int B_PER = B_BYTES / 1024 / LOADERS;
    static constexpr int PER = A_PER + B_PER;
    static constexpr int SROW = WTN * 2 + 8;
    static constexpr int EPI = NW * WTM * SROW;
    static constexpr int LDS_ALLOC = LDS > EPI ? LDS : EPI;
    static_assert(A_BYTES % (1024 * LOADERS) == 0 && B_BYTES % (1024 * LOADERS) == 0, "DMA split");
    static_assert(BROW % 256 == 0 && FM >= 1 && FN >= 1, "tile shape");
    static_assert(LDS <= 160 * 1024 && EPI <= 160 * 1024, "LDS budget");
    static_assert(PER * (AHEAD - 1) < 64, "vmcnt range");
    static_assert(WTN % 8 == 0 && 64 % (WTN / 8) == 0 || WTN % 512 == 0, "staged output rows of 8-column chunks");
    // LDS swizzles (XOR on the 16-byte chunk index of a row), both measured
    // conflict-free on gfx950 for the fragment reads below.  A: the 16-byte
    // read of rows 0..15 x chunks 0..3 runs at the full 256 B/clk with chunk
    // (lane/16) ^ ((m >> 1) & 3); the (m >> 2) & 3 that suits the 32x32
    // reads reaches only 58% of it.  B: a transposed read pairs k rows r and
    // r + 8 in one access, so bit 3 of the row joins the swizzle (without it
    // the read runs at 3/4 rate).
    __device__ static u32 a_swz(u32 m) { return (m >> 1) & 3u; }
    __device__ static u32 b_swz(u32 k) { return (4u * (k & 3u)) ^ (2u * ((k >> 3) & 1u)); }
};

// Per-lane LDS offsets of a wave's fragments within a stage.  A fragment i:
// row wm*WTM + 16 i + (lane % 16), 8 k from chunk lane / 16 (chunks XOR-
// swizzled by row).  B fragment j, half h: a transposed read whose source
// lane s (of each 16-lane group g) points at k row 8g + 4h + s/4, column
// wn*WTN + 16 j + 4 (s % 4); lane l then holds B[8g+4h .. +3][16 j + l % 16].
template <class C>
struct Addr {
    u32 a0;
    u32 b[C::FN];
};

template <class C>
__device__ __forceinline__ Addr<C> frag_addr(int wm, int wn, int lane)
{
    Addr<C> ad;
    const u32 m = wm * C::WTM + (lane & 15);
    ad.a0 = m * (u32)C::AROW + ((((u32)lane >> 4) ^ C::a_swz(m)) << 4);
    const int g = lane >> 4, s = lane & 15;
    const u32 kr = 8 * g + (s >> 2);
    const u32 xb = C::b_swz(kr);
#pragma unroll
    for (int j = 0; j < C::FN; ++j) {
        const u32 n = wn * C::WTN + j * 16 + 4 * (s & 3);
        ad.b[j] = C::A_BYTES + kr * C::BROW + (((n >> 3) ^ xb) << 4) + (n & 7) * 2;
    }
    return ad;
}

template <class C>
__device__ __forceinline__ void read_a(const char* stage, const Addr<C>& ad, int i, u32x4& a)
{
    a = *reinterpret_cast<const u32x4*>(stage + ad.a0 + i * 16 * C::AROW);
}

// Both halves of B fragment j, straight into its register quad.
template <class C>
__device__ __forceinline__ void read_b(const char* stage, const Addr<C>& ad, int j, u32x4& b)
{
    const u32x2 lo = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) tiles::s16x4*)(stage + ad.b[j])));
    const u32x2 hi = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) tiles::s16x4*)(stage + ad.b[j] + 4 * C::BROW)));
    b = u32x4{lo.x, lo.y, hi.x, hi.y};
}

// One k-tile: MFMA (i, j) = A fragment i x B fragment j, i outer.  A is
// single-buffered: the next tile's A fragment i is read right after the
// last MFMA that uses the current one.  B is double-buffered (Bc -> Bn), its
// reads slotted after the first FN MFMAs.  With PRE the loads of tile t+3
// follow in later slots.
template <class C, bool BF, bool NEXT, bool PRE, bool EDGE, bool GROUPED, bool PK = false>
__device__ __forceinline__ void ktile(u32x4 (&Af)[C::FM], const u32x4 (&Bc)[C::FN], u32x4 (&Bn)[C::FN],
                                      const char* nxt, char* pre, const tiles::TileSrc& ps, const q4::Group<C>& go,
                                      const Addr<C>& ad, int wave, int lane, f32x4 (&acc)[C::FM][C::FN])
{
    constexpr int NMF = C::FM * C::FN;
    constexpr int L0 = C::FN + 1;                   // first load slot
    static_assert(L0 + 2 * (C::PER - 1) < NMF, "load slots");
#pragma unroll
    for (int x = 0; x < NMF; ++x) {
        const int i = x / C::FN, j = x % C::FN;
        acc[i][j] = mfma<BF>(Bc[j], Af[i], acc[i][j]);
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (NEXT) {
            if (x < C::FN)
                read_b<C>(nxt, ad, x, Bn[x]);
            if (j == C::FN - 1)
                read_a<C>(nxt, ad, i, Af[i]);
        }
        if constexpr (PRE) {
            const int y = x - L0;
            if (y >= 0 && (y & 1) == 0 && y / 2 < C::PER) {
                const int k = y / 2;
                if constexpr (GROUPED) {
                    if (k == 0)
                        q4::dma_group<C, PK>(pre, ps, go, wave, 0);
                    else if (k == C::PER / 2)
                        q4::dma_group<C, PK>(pre, ps, go, wave, 1);
                } else {
                    q4::dma_one<C, EDGE>(pre, ps, wave, lane, k);
                }
            }
        }
        __builtin_amdgcn_sched_barrier(0);
    }
}

// K loop of one output tile (same contract as q4::run_tile).  RESTRIDE: the
// sources may change their leading dimensions between k-tiles (the products
// of a fused group: combined blocks and singleton operands differ), so the
// grouped-load offsets are recomputed whenever a source's strides differ from
// the last ones (a uniform branch, taken once per product switch at most),
// and src(0) is not called ahead of the k-tiles (cursor sources may be used).
// PK: A is tile-packed (q4::dma_group); grouped loads only.
template <class C, bool BF, bool EDGE, bool GROUPED, bool RESTRIDE = false, bool PK = false, class SrcFn,
          class AfterFn>
__device__ __forceinline__ void run_tile(char* smem, int nk, SrcFn src, AfterFn after, int wave, int lane,
                                         const Addr<C>& ad, f32x4 (&acc)[C::FM][C::FN])
{
    static_assert(C::AHEAD >= 3 && C::NSTAGE == C::AHEAD + 1, "stage reuse below: tile t + AHEAD goes where tile t - 1 was");
    static_assert(!(GROUPED && EDGE), "grouped loads carry no bounds");
    static_assert(!RESTRIDE || GROUPED, "restriding applies to grouped loads");
    static_assert(!PK || (GROUPED && !RESTRIDE), "packed A takes the grouped loads of one stride");
    u32x4 Af[C::FM], B0[C::FN], B1[C::FN];
    q4::Group<C> go;
    int go_lda = -1, go_ldb = -1;
    auto regroup = [&](const tiles::TileSrc& ps) {
        if constexpr (RESTRIDE) {
            if (ps.lda != go_lda || ps.ldb != go_ldb) {
                go = q4::group_offsets<C, PK>(ps, wave, lane);
                go_lda = ps.lda;
                go_ldb = ps.ldb;
            }
        }
    };
    if constexpr (GROUPED && !RESTRIDE)
        go = q4::group_offsets<C, PK>(src(0), wave, lane);
#pragma unroll
    for (int t = 0; t < C::AHEAD; ++t) {
        if (t < nk) {
            if constexpr (GROUPED) {
                const tiles::TileSrc ps = src(t);
                regroup(ps);
                q4::dma_group<C, PK>(smem + t * C::STAGE, ps, go, wave, 0);
                q4::dma_group<C, PK>(smem + t * C::STAGE, ps, go, wave, 1);
            } else {
                q4::dma_tile<C, EDGE>(smem + t * C::STAGE, src(t), wave, lane);
            }
        }
    }
    q4::wait_tiles<C>(min(nk, C::AHEAD) - 1);
    tiles::bar();
    if (nk > 0) {
#pragma unroll
        for (int i = 0; i < C::FM; ++i)
            read_a<C>(smem, ad, i, Af[i]);
#pragma unroll
        for (int j = 0; j < C::FN; ++j)
            read_b<C>(smem, ad, j, B0[j]);
    }
    // Top of k-tile t: tile t+1 has landed and every wave has finished with
    // tile t-1's stage, which then takes tile t+3.  No LDS-read wait here:
    // reads still in flight target stage t+1 (the fragments of tile t+1),
    // which nothing overwrites before the next barrier, and the reads of
    // stage t-1 were consumed by tile t-1's MFMAs (the compiler waits for
    // each fragment before its first use).
    auto steady = [&](int t, const u32x4 (&Bc)[C::FN], u32x4 (&Bn)[C::FN]) {
        q4::wait_vm<(C::AHEAD - 2) * C::PER>();   // tiles t+2 .. t+AHEAD-1 may be in flight
        tiles::bar();
        __builtin_amdgcn_sched_barrier(0);
        const tiles::TileSrc ps = src(t + C::AHEAD);
        regroup(ps);
        ktile<C, BF, true, true, EDGE, GROUPED, PK>(Af, Bc, Bn, smem + ((t + 1) % C::NSTAGE) * C::STAGE,
                                                smem + ((t + C::AHEAD) % C::NSTAGE) * C::STAGE, ps, go, ad, wave,
                                                lane, acc);
        __builtin_amdgcn_sched_barrier(0);
        after(t);
    };
    int t = 0;
    // Steady state, two k-tiles per trip so the B buffers alternate without
    // copies; both tiles have a successor and a tile to prefetch.
    for (; t + 1 + C::AHEAD < nk; t += 2) {
        steady(t, B0, B1);
        steady(t + 1, B1, B0);
    }
    // At most AHEAD + 1 k-tiles remain; Af and B0 hold tile t's fragments.
    // Plain order: the MFMAs, then the next tile's reads (not overlapped).
    for (; t < nk; ++t) {
#pragma unroll
        for (int i = 0; i < C::FM; ++i)
#pragma unroll
            for (int j = 0; j < C::FN; ++j)
                acc[i][j] = mfma<BF>(B0[j], Af[i], acc[i][j]);
        after(t);
        if (t + 1 < nk) {
            // issued so far: tiles up to min(t+AHEAD-1, nk-1); tile t+1 must have landed
            q4::wait_tiles<C>(min(nk - 2 - t, C::AHEAD - 2));
            tiles::wait_lgkm0();
            tiles::bar();
            if (t + C::AHEAD < nk) {
                const tiles::TileSrc ps = src(t + C::AHEAD);
                char* pre = smem + ((t + C::AHEAD) % C::NSTAGE) * C::STAGE;
                if constexpr (GROUPED) {
                    regroup(ps);
                    q4::dma_group<C, PK>(pre, ps, go, wave, 0);
                    q4::dma_group<C, PK>(pre, ps, go, wave, 1);
                } else {
                    q4::dma_tile<C, EDGE>(pre, ps, wave, lane);
                }
            }
            const char* nxt = smem + ((t + 1) % C::NSTAGE) * C::STAGE;
#pragma unroll
            for (int i = 0; i < C::FM; ++i)
                read_a<C>(nxt, ad, i, Af[i]);
#pragma unroll
            for (int j = 0; j < C::FN; ++j)
                read_b<C>(nxt, ad, j, B0[j]);
        }
    }
}

// K loop of one output tile whose operands are sums of two input tiles
// (combine at load).  A ring stage holds both terms of a k-tile: the first
// term's A and B at the usual offsets, the second's one stage size further.
// Every k-tile moves both terms by direct-to-LDS loads (a term that is
// absent reads as zero: its bounds are empty), so the wait counts are fixed.
// Iteration t, after one barrier: the fragment reads of k-tile t (folded in
// iteration t - 1), comb(t + 1, stage) folding the second terms of k-tile
// t + 1 into its first terms in place (its loads have landed), the loads of
// k-tile t + AHEAD into the stage of k-tile t - 1, and the MFMAs of k-tile
// t.  (Issuing the MFMAs before the fold measured 3-8% slower.)
// GROUPED (interior tiles, K a multiple of 32): grouped loads with the
// per-lane offsets `go` of the inputs' strides, shared by both terms; an
// absent second term then loads the first term again (not folded).
template <class C, bool BF, bool GROUPED, class SrcFn, class CombFn, class AfterFn>
__device__ __forceinline__ void run_tile_cal(char* smem, int nk, SrcFn src, CombFn comb, AfterFn after, int wave,
                                             int lane, const Addr<C>& ad, const q4::Group<C>& go,
                                             f32x4 (&acc)[C::FM][C::FN])
{
    constexpr int ST = 2 * C::STAGE;
    constexpr int P2 = 2 * C::PER;
    static_assert(C::AHEAD >= 2 && C::AHEAD <= 4 && C::NSTAGE == C::AHEAD + 1,
                  "stage reuse (k-tile t + AHEAD goes where k-tile t - 1 was) and wait counts below");
    static_assert(C::NSTAGE * ST <= 160 * 1024, "LDS budget");
    static_assert(P2 * (C::AHEAD - 1) < 64, "vmcnt range");
    auto issue = [&](int t) {
        tiles::TileSrc s1, s2;
        src(t, &s1, &s2);
        char* stage = smem + (t % C::NSTAGE) * ST;
        if constexpr (GROUPED) {
            if (s2.a_rows == 0)
                s2.a = s1.a;
            if (s2.b_cols == 0)
                s2.b = s1.b;
            q4::dma_group<C>(stage, s1, go, wave, 0);
            q4::dma_group<C>(stage, s1, go, wave, 1);
            q4::dma_group<C>(stage + C::STAGE, s2, go, wave, 0);
            q4::dma_group<C>(stage + C::STAGE, s2, go, wave, 1);
        } else {
            q4::dma_tile<C, true>(stage, s1, wave, lane);
            q4::dma_tile<C, true>(stage + C::STAGE, s2, wave, lane);
        }
    };
    if (nk <= 0)
        return;
#pragma unroll
    for (int t = 0; t < C::AHEAD; ++t)
        if (t < nk)
            issue(t);
    // k-tile 0 landed (up to AHEAD - 1 later k-tiles in flight), then folded
    const int later0 = min(nk - 1, C::AHEAD - 1);
    if (later0 >= 3)
        q4::wait_vm<3 * P2>();
    else if (later0 == 2)
        q4::wait_vm<2 * P2>();
    else if (later0 == 1)
        q4::wait_vm<P2>();
    else
        tiles::wait_vm0();
    tiles::bar();
    comb(0, smem);
    tiles::wait_lgkm0();
    for (int t = 0; t < nk; ++t) {
        // k-tile t + 1 must have landed: loads issued after it cover
        // min(nk - 2 - t, AHEAD - 2) k-tiles
        if (t + 1 < nk) {
            const int later = min(nk - 2 - t, C::AHEAD - 2);
            if (later >= 2)
                q4::wait_vm<2 * P2>();
            else if (later == 1)
                q4::wait_vm<P2>();
            else
                tiles::wait_vm0();
        }
        tiles::bar();
        char* stage = smem + (t % C::NSTAGE) * ST;
        u32x4 Af[C::FM], Bf[C::FN];
#pragma unroll
        for (int i = 0; i < C::FM; ++i)
            read_a<C>(stage, ad, i, Af[i]);
#pragma unroll
        for (int j = 0; j < C::FN; ++j)
            read_b<C>(stage, ad, j, Bf[j]);
        if (t + 1 < nk)
            comb(t + 1, smem + ((t + 1) % C::NSTAGE) * ST);
        if (t + C::AHEAD < nk)
            issue(t + C::AHEAD);
#pragma unroll
        for (int i = 0; i < C::FM; ++i)
#pragma unroll
            for (int j = 0; j < C::FN; ++j)
                acc[i][j] = mfma<BF>(Bf[j], Af[i], acc[i][j]);
        after(t);
        tiles::wait_lgkm0();
    }
}

// Output tile store through LDS (16x16 accumulator layout: lane l of tile
// (i, j) holds row 16 i + l % 16, columns 16 j + 4 (l / 16) .. + 3).
template <class C, bool BF>
__device__ __forceinline__ void store_c_staged(const f32x4 (&acc)[C::FM][C::FN], char* smem, u16* Cp, int64_t ldc,
                                               int rows, int cols, int wave, int wm, int wn, int lane)
{
    char* reg = smem + wave * C::WTM * C::SROW;
#pragma unroll
    for (int i = 0; i < C::FM; ++i)
#pragma unroll
        for (int j = 0; j < C::FN; ++j) {
            const int row = i * 16 + (lane & 15), col = j * 16 + 4 * (lane >> 4);
            const u32x2 v{pack2<BF>(acc[i][j][0], acc[i][j][1]), pack2<BF>(acc[i][j][2], acc[i][j][3])};
            *reinterpret_cast<u32x2*>(reg + row * C::SROW + col * 2) = v;
        }
    tiles::wait_lgkm0();
    const rsrc_t rc = make_rsrc(Cp);
    const int ld = (int)ldc;
    constexpr int CHUNKS = C::WTN / 8;
    constexpr int RPI = 64 / CHUNKS;
#pragma unroll
    for (int r0 = 0; r0 < C::WTM; r0 += RPI) {
        const int row = r0 + lane / CHUNKS, ch = lane % CHUNKS;
        const u32x4 v = *reinterpret_cast<const u32x4*>(reg + row * C::SROW + ch * 16);
        const int m = wm * C::WTM + row, n = wn * C::WTN + ch * 8;
        const u32 off = (m < rows && n < cols) ? (u32)(m * ld + n) * 2u : kOob;
        // non-temporal (aux bit 1): C is not read back by the kernel; measured
        // 1-1.5% faster at 4096^3 and 4-30% faster than plain stores on
        // output-bound short-K shapes (16384^2 x 64: 129.6 against 169.0 us)
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(__attribute__((ext_vector_type(4))) unsigned int, v),
                                               rc, off, 0, 2);
    }
}

}  // namespace m16

using MC256 = m16::Cfg<256, 256, 2, 4>;   // 8 waves (2 per SIMD) of 128 x 64, 16x16x32 MFMAs

template <class C, bool BF, bool PART = false>
__global__ void __launch_bounds__(C::NT, 1)
k_classic_m16(const u16* __restrict__ A, int64_t lda, const u16* __restrict__ B, int64_t ldb, u16* __restrict__ Cm,
              int64_t ldc, int M, int N, int K, int gy, int gx, int P, int vec4, int vec8, int tile0, int kh,
              int tcount, int compact, float* __restrict__ part)
{
    __shared__ __attribute__((aligned(1024))) char smem[C::LDS_ALLOC];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / C::WN, wn = wave % C::WN;
    // Block b works tile tile0 + b.  PART: block b is piece b / tcount (k in
    // [piece kh, piece kh + kh)) of tile tile0 + b % tcount and writes an fp32
    // partial tile: into plane `piece` of M x N (row stride N), or, compact,
    // into slot piece * tcount + b % tcount of BM x BN tiles (row stride BN).
    const int idx = PART ? (int)blockIdx.x % tcount : (int)blockIdx.x;
    const int piece = PART ? (int)blockIdx.x / tcount : 0;
    int p, q;
    tile_coords((int32_t)(tile0 + idx), gy, gx, P, 8, &p, &q);
    const int m0 = p * C::BM, n0 = q * C::BN;
    const int kb = piece * kh, klen = PART ? max(0, min(K - kb, kh)) : K;
    const u16* Ab = A + (int64_t)m0 * lda + kb;
    const u16* Bb = B + (int64_t)kb * ldb + n0;
    const int nk = (klen + C::BK - 1) / C::BK;
    f32x4 acc[C::FM][C::FN];
    zero_acc<C>(acc);
    auto src = [&](int t) {
        return tiles::TileSrc{Ab, (int)lda, M - m0, Bb, (int)ldb, N - n0, t * C::BK, klen};
    };
    const m16::Addr<C> ad = m16::frag_addr<C>(wm, wn, lane);
    const bool inside = (m0 + C::BM <= M) & (n0 + C::BN <= N) & (klen % C::BK == 0);
    auto none = [](int) {};
    if (!PART || nk > 0) {
        if (inside)
            m16::run_tile<C, BF, false, true>(smem, nk, src, none, wave, lane, ad, acc);
        else
            m16::run_tile<C, BF, true, false>(smem, nk, src, none, wave, lane, ad, acc);
    }
    if constexpr (PART) {
        // lane l of accumulator tile (i, j): row 16 i + l % 16, columns
        // 16 j + 4 (l / 16) .. + 3 of the wave's tile; N is a multiple of 8
        // on this path, so each 4-column group is wholly inside or out
        const int pld = compact ? C::BN : N;
        const rsrc_t rp = make_rsrc(compact ? part + ((int64_t)piece * tcount + idx) * (C::BM * C::BN)
                                            : part + (int64_t)piece * M * N + (int64_t)m0 * N + n0);
#pragma unroll
        for (int i = 0; i < C::FM; ++i)
#pragma unroll
            for (int j = 0; j < C::FN; ++j) {
                const int m = wm * C::WTM + i * 16 + (lane & 15), n = wn * C::WTN + j * 16 + 4 * (lane >> 4);
                const u32 off = (m < M - m0 && n < N - n0) ? (u32)(m * pld + n) * 4u : kOob;
                __builtin_amdgcn_raw_buffer_store_b128(
                    __builtin_bit_cast(__attribute__((ext_vector_type(4))) unsigned int, acc[i][j]), rp, off, 0, 0);
            }
        return;
    }
    if (vec8) {
        __syncthreads();
        m16::store_c_staged<C, BF>(acc, smem, Cm + (int64_t)m0 * ldc + n0, ldc, M - m0, N - n0, wave, wm, wn, lane);
    } else if (vec4)
        store_c<C, BF, true>(acc, Cm + (int64_t)m0 * ldc + n0, ldc, M - m0, N - n0, wm, wn, lane);
    else
        store_c<C, BF, false>(acc, Cm + (int64_t)m0 * ldc + n0, ldc, M - m0, N - n0, wm, wn, lane);
}

template <class C, bool BF>
hipError_t launch_classic_m16_t(const ClassicLaunch& L, hipStream_t st)
{
    const int gy = (L.M + C::BM - 1) / C::BM, gx = (L.N + C::BN - 1) / C::BN;
    const long tiles = (long)gy * gx;
    if (tiles == 0)
        return hipSuccess;
    const int vec8 = L.vec4 && ((uintptr_t)L.C % 16 == 0) && (L.ldc % 8 == 0) && (L.N % 8 == 0);
    hipLaunchKernelGGL((k_classic_m16<C, BF>), dim3((unsigned)tiles), dim3(C::NT), 0, st,
                       (const u16*)L.A, L.lda, (const u16*)L.B, L.ldb, (u16*)L.C, L.ldc, L.M, L.N, L.K,
                       gy, gx, L.P, L.vec4, vec8, 0, L.K, 1, 0, nullptr);
    return hipGetLastError();
}

using QC128 = q4::QCfg<128, 128>;   // 4 waves of 64 x 64
// 8 waves (2 per SIMD) of 64 x 32, 16x16x32 MFMAs, 7 k-tiles in flight: for
// long K on 128 x 128 tiles (measured 10-24% faster than the four-wave
// kernel from K = 2048, 11-15% slower at K <= 1024, where its deeper
// prologue and epilogue weigh more than the K loop).
using MC128 = m16::Cfg<128, 128, 2, 4, 7>;
constexpr int kLongK128 = 2048;

template <class C, bool BF>
__global__ void __launch_bounds__(C::NT, 1)
k_classic_q4(const u16* __restrict__ A, int64_t lda, const u16* __restrict__ B, int64_t ldb, u16* __restrict__ Cm,
             int64_t ldc, int M, int N, int K, int gy, int gx, int P, int vec4, int vec8)
{
    __shared__ __attribute__((aligned(1024))) char smem[C::LDS_ALLOC];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / C::WN, wn = wave % C::WN;
    int p, q;
    tile_coords((int32_t)blockIdx.x, gy, gx, P, 8, &p, &q);
    const int m0 = p * C::BM, n0 = q * C::BN;
    const u16* Ab = A + (int64_t)m0 * lda;
    const u16* Bb = B + n0;
    const int nk = (K + C::BK - 1) / C::BK;
    f32x16 acc[C::FM][C::FN];
    zero_acc<C>(acc);
    auto src = [&](int t) {
        return tiles::TileSrc{Ab, (int)lda, M - m0, Bb, (int)ldb, N - n0, t * C::BK, K};
    };
    const q4::Addr<C> ad = q4::frag_addr<C>(wm, wn, lane);
    const bool inside = (m0 + C::BM <= M) & (n0 + C::BN <= N) & (K % C::BK == 0);
    auto none = [](int) {};
    if (inside)
        q4::run_tile<C, BF, false, true>(smem, nk, src, none, wave, lane, ad, acc);
    else
        q4::run_tile<C, BF, true, false>(smem, nk, src, none, wave, lane, ad, acc);
    if (vec8) {
        __syncthreads();
        q4::store_c_staged<C, BF>(acc, smem, Cm + (int64_t)m0 * ldc + n0, ldc, M - m0, N - n0, wave, wm, wn, lane);
    } else if (vec4)
        store_c<C, BF, true>(acc, Cm + (int64_t)m0 * ldc + n0, ldc, M - m0, N - n0, wm, wn, lane);
    else
        store_c<C, BF, false>(acc, Cm + (int64_t)m0 * ldc + n0, ldc, M - m0, N - n0, wm, wn, lane);
}

// One product of the unfused path, with an epilogue that folds w[t] * H into
// output targets instead of storing H (modes as in the two-level outer
// level: store, add, add and round into C, round into C).  Products run one
// after another on the stream, so no two launches touch a target at the same
// time.
struct GenTargets {
    float* tgt[kGenMaxBlocks];
    u16* cdst[kGenMaxBlocks];
    float w[kGenMaxBlocks];
    int8_t mode[kGenMaxBlocks];
    int ntgt;
    int64_t ldt, ldc;
};

// One target of a fold: rt is the target's fp32 block and rc its C block,
// both at the tile origin (ld, ldc elements per row).  get(e, m, n, h) gives
// the e-th (0 <= e < NE) 4-column group h of the wave's accumulators at
// (m, n) relative to the tile origin; N is a multiple of 8 on this path, so a
// group is wholly inside the columns or wholly out.  The mode is uniform, so
// it is tested once; the read-modify-write modes issue CH loads before the
// first use, so a fold waits for NE / CH round trips instead of NE.
template <bool CBF, int NE, int CH, class Get>
__device__ __forceinline__ void fold_target(rsrc_t rt, rsrc_t rc, int ld, int ldc, int mode, float wt, int rows,
                                            int cols, Get get)
{
    static_assert(NE % CH == 0, "fold chunks");
    if (mode == kOuterNone)
        return;
    auto off_t = [&](int m, int n) { return (m < rows && n < cols) ? (u32)(m * ld + n) * 4u : kOob; };
    // C gets v + 0: a zero sum written as -0 (a product folded with
    // coefficient -1, say) becomes +0, as the classic product writes it
    auto put_c = [&](int m, int n, const f32x4& v0) {
        const f32x4 v = v0 + 0.0f;
        const u32 oc = (m < rows && n < cols) ? (u32)(m * ldc + n) * 2u : kOob;
        __builtin_amdgcn_raw_buffer_store_b64(
            __builtin_bit_cast(__attribute__((ext_vector_type(2))) unsigned int,
                               u32x2{pack2<CBF>(v.x, v.y), pack2<CBF>(v.z, v.w)}),
            rc, oc, 0, 0);
    };
    auto put_t = [&](int m, int n, const f32x4& v) {
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(__attribute__((ext_vector_type(4))) unsigned int, v),
                                               rt, off_t(m, n), 0, 0);
    };
    if (mode == kOuterStore || mode == kOuterOnly) {
#pragma unroll
        for (int e = 0; e < NE; ++e) {
            int m, n;
            f32x4 h;
            get(e, m, n, h);
            if (mode == kOuterStore)
                put_t(m, n, h * wt);
            else
                put_c(m, n, h * wt);
        }
        return;
    }
#pragma unroll
    for (int e0 = 0; e0 < NE; e0 += CH) {
        f32x4 old[CH];
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            int m, n;
            f32x4 h;
            get(e0 + c, m, n, h);
            old[c] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rt, off_t(m, n), 0, 0));
        }
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            int m, n;
            f32x4 h;
            get(e0 + c, m, n, h);
            const f32x4 v = h * wt + old[c];
            if (mode == kOuterAdd)
                put_t(m, n, v);
            else
                put_c(m, n, v);
        }
    }
}

template <bool CBF, int NE, int CH, class Get>
__device__ __forceinline__ void gen_fold(const GenTargets& tg, int m0, int n0, int rows, int cols, Get get)
{
    for (int t = 0; t < tg.ntgt; ++t)
        fold_target<CBF, NE, CH>(make_rsrc(tg.tgt[t] + (int64_t)m0 * tg.ldt + n0),
                                 make_rsrc(tg.cdst[t] + (int64_t)m0 * tg.ldc + n0), (int)tg.ldt, (int)tg.ldc,
                                 tg.mode[t], tg.w[t], rows, cols, get);
}

// On the four-wave 32x32 engine (128 x 128 tiles; shapes with few tiles).
template <class C, bool BF, bool CBF>
__global__ void __launch_bounds__(C::NT, 1)
k_gen_product(const u16* __restrict__ A, int64_t lda, const u16* __restrict__ B, int64_t ldb, int M, int N, int K,
              int gy, int gx, int P, const GenTargets tg)
{
    __shared__ __attribute__((aligned(1024))) char smem[C::LDS];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / C::WN, wn = wave % C::WN;
    int p, q;
    tile_coords((int32_t)blockIdx.x, gy, gx, P, 8, &p, &q);
    const int m0 = p * C::BM, n0 = q * C::BN;
    const u16* Ab = A + (int64_t)m0 * lda;
    const u16* Bb = B + n0;
    const int nk = (K + C::BK - 1) / C::BK;
    f32x16 acc[C::FM][C::FN];
    zero_acc<C>(acc);
    auto src = [&](int t) {
        return tiles::TileSrc{Ab, (int)lda, M - m0, Bb, (int)ldb, N - n0, t * C::BK, K};
    };
    const q4::Addr<C> ad = q4::frag_addr<C>(wm, wn, lane);
    auto none = [](int) {};
    const bool inside = (m0 + C::BM <= M) & (n0 + C::BN <= N) & (K % C::BK == 0);
    if (inside)
        q4::run_tile<C, BF, false, true>(smem, nk, src, none, wave, lane, ad, acc);
    else
        q4::run_tile<C, BF, true, false>(smem, nk, src, none, wave, lane, ad, acc);
    // lane l of MFMA tile (i, j) holds row (l % 32) and, per group g of 4
    // accumulators, columns 8 g + 4 (l / 32) .. + 3
    const int r = lane & 31, hi = lane >> 5;
    constexpr int NE = C::FM * C::FN * 4;
    gen_fold<CBF, NE, 16>(tg, m0, n0, M - m0, N - n0, [&](int e, int& m, int& n, f32x4& h) {
        const int i = e / (C::FN * 4), j = (e / 4) % C::FN, g = e % 4;
        m = wm * C::WTM + i * 32 + r;
        n = wn * C::WTN + j * 32 + 8 * g + 4 * hi;
        h = f32x4{acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]};
    });
}

// All products of the unfused path in one persistent launch: each workgroup
// owns 256 x 256 output positions (round-robin) and, for each, runs every
// product's K loop in turn and folds it into that position's blocks, so the
// read-modify-write of a block is never shared between workgroups and the
// folds of different workgroups fall at different times.
struct GenGroupParams {
    const u16* A0; int64_t strideA;    // combined A operand r at A0 + r * strideA (M x K, ld K)
    const u16* B0; int64_t strideB;    // combined B operand r at B0 + r * strideB (K x N, ld ldb)
    int ldb;
    int M, N, K, R, P, nout, ncols;
    float* acc;                        // fp32 block o at acc + o * M * N (ld N)
    u16* C; int64_t ldc;               // block o of C at row (o / ncols) * M, column (o % ncols) * N
    int8_t w[kGenMaxRank * kGenMaxBlocks];      // fold coefficient per (run, block)
    int8_t mode[kGenMaxRank * kGenMaxBlocks];   // OuterMode per (run, block)
    int8_t prod[kGenMaxRank];                    // product of run j
    int8_t carry[kGenMaxRank];                   // 0: zero accumulators, 1: keep, 2: negate
};
static_assert(sizeof(GenGroupParams) <= 4096, "kernel argument segment");

// EDGE: some position is a partial tile or K is not a multiple of 32 (then
// every position takes the bounds-checked loads: one K-loop form per kernel
// keeps the persistent loops within the register budget).  PK: the combined
// A operands are tile-packed by the pre-pass (q4::dma_group); interior only.
template <class C, bool BF, bool CBF, bool EDGE, bool PK>
__global__ void __launch_bounds__(C::NT, 1) k_gen_group_m16(const GenGroupParams gp)
{
    static_assert(!(PK && EDGE), "packed operands cover whole tiles");
    __shared__ __attribute__((aligned(1024))) char smem[C::LDS_ALLOC];
    const int tid = threadIdx.x, lane0 = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / C::WN, wn = wave % C::WN;
    const int gy = (gp.M + C::BM - 1) / C::BM, gx = (gp.N + C::BN - 1) / C::BN;
    const int nk = (gp.K + C::BK - 1) / C::BK;
    auto none = [](int) {};
    for (int item = blockIdx.x; item < gy * gx; item += gridDim.x) {
        int p, q;
        tile_coords(item, gy, gx, gp.P, 8, &p, &q);
        const int m0 = p * C::BM, n0 = q * C::BN, rows = gp.M - m0, cols = gp.N - n0;
        f32x4 acc[C::FM][C::FN];
        for (int run = 0; run < gp.R; ++run) {
            const int r = gp.prod[run], cy = gp.carry[run];
            // Opaque per product: keeps lane-derived addresses (fold offsets,
            // fragment offsets) from being hoisted out of the loops and held
            // in registers through every K loop.
            int lane = lane0;
            asm volatile("" : "+v"(lane));
            const m16::Addr<C> ad = m16::frag_addr<C>(wm, wn, lane);
            const u16* Ab = gp.A0 + r * gp.strideA + (int64_t)m0 * gp.K;
            const u16* Bb = gp.B0 + r * gp.strideB + n0;
            auto src = [&](int t) {
                return tiles::TileSrc{Ab, gp.K, rows, Bb, gp.ldb, cols, t * C::BK, gp.K};
            };
            if (cy == 0) {
                zero_acc<C>(acc);
            } else if (cy == 2) {
#pragma unroll
                for (int i = 0; i < C::FM; ++i)
#pragma unroll
                    for (int j = 0; j < C::FN; ++j)
                        acc[i][j] = -acc[i][j];
            }
            __syncthreads();   // every wave is done reading the ring of the previous product
            m16::run_tile<C, BF, EDGE, !EDGE, false, PK>(smem, nk, src, none, wave, lane, ad, acc);
            for (int o = 0; o < gp.nout; ++o) {
                const int mode = gp.mode[run * kGenMaxBlocks + o];
                if (mode == kOuterNone)
                    continue;
                const int bi = o / gp.ncols, bj = o % gp.ncols;
                fold_target<CBF, C::FM * C::FN, 8>(
                    make_rsrc(gp.acc + (int64_t)o * gp.M * gp.N + (int64_t)m0 * gp.N + n0),
                    make_rsrc(gp.C + (int64_t)(bi * gp.M + m0) * gp.ldc + bj * gp.N + n0), gp.N, (int)gp.ldc, mode,
                    (float)gp.w[run * kGenMaxBlocks + o], rows, cols, [&](int e, int& m, int& n, f32x4& h) {
                        const int i = e / C::FN, j = e % C::FN;
                        m = wm * C::WTM + i * 16 + (lane & 15);
                        n = wn * C::WTN + j * 16 + 4 * (lane >> 4);
                        h = acc[i][j];
                    });
            }
        }
    }
}

template <bool BF, bool CBF>
hipError_t launch_gen_group_t(const GenGroupLaunch& L, hipStream_t st)
{
    using C = MC256;
    const int items = ((L.M + C::BM - 1) / C::BM) * ((L.N + C::BN - 1) / C::BN);
    if (items == 0 || L.R == 0)
        return hipSuccess;
    GenGroupParams gp;
    gp.A0 = (const u16*)L.A0; gp.strideA = L.strideA;
    gp.B0 = (const u16*)L.B0; gp.strideB = L.strideB;
    if (L.ldb < L.N || L.ldb >= ((int64_t)1 << 21))
        return hipErrorInvalidValue;
    gp.ldb = (int)L.ldb;
    gp.M = L.M; gp.N = L.N; gp.K = L.K; gp.R = L.R; gp.P = L.P; gp.nout = L.nout; gp.ncols = L.ncols;
    gp.acc = L.acc;
    gp.C = (u16*)L.C; gp.ldc = L.ldc;
    for (int i = 0; i < kGenMaxRank * kGenMaxBlocks; ++i) {
        gp.w[i] = L.w[i];
        gp.mode[i] = L.mode[i];
    }
    for (int i = 0; i < kGenMaxRank; ++i) {
        gp.prod[i] = L.prod[i];
        gp.carry[i] = L.carry[i];
    }
    const bool edge = L.M % C::BM != 0 || L.N % C::BN != 0 || L.K % C::BK != 0;
    if (L.packed_a && (edge || C::BM != kPackRows || C::BK != kPackCols))
        return hipErrorInvalidValue;    // the packed layout needs whole tiles of this shape
    const dim3 grid((unsigned)std::min(items, L.P));
    if (edge)
        hipLaunchKernelGGL((k_gen_group_m16<C, BF, CBF, true, false>), grid, dim3(C::NT), 0, st, gp);
    else if (L.packed_a)
        hipLaunchKernelGGL((k_gen_group_m16<C, BF, CBF, false, true>), grid, dim3(C::NT), 0, st, gp);
    else
        hipLaunchKernelGGL((k_gen_group_m16<C, BF, CBF, false, false>), grid, dim3(C::NT), 0, st, gp);
    return hipGetLastError();
}

template <class C, bool BF, bool CBF>
hipError_t launch_gen_product_t(const GenProductLaunch& L, hipStream_t st)
{
    const int gy = (L.M + C::BM - 1) / C::BM, gx = (L.N + C::BN - 1) / C::BN;
    const long tiles = (long)gy * gx;
    if (tiles == 0)
        return hipSuccess;
    GenTargets tg{};
    for (int t = 0; t < L.ntgt; ++t) {
        tg.tgt[t] = L.tgt[t];
        tg.cdst[t] = (u16*)L.cdst[t];
        tg.w[t] = L.w[t];
        tg.mode[t] = L.mode[t];
    }
    tg.ntgt = L.ntgt;
    tg.ldt = L.ldt;
    tg.ldc = L.ldc;
    hipLaunchKernelGGL((k_gen_product<C, BF, CBF>), dim3((unsigned)tiles), dim3(C::NT), 0, st,
                       (const u16*)L.A, L.lda, (const u16*)L.B, L.ldb, L.M, L.N, L.K, gy, gx, L.P, tg);
    return hipGetLastError();
}

template <class C, bool BF>
hipError_t launch_classic_q4_t(const ClassicLaunch& L, hipStream_t st)
{
    const int gy = (L.M + C::BM - 1) / C::BM, gx = (L.N + C::BN - 1) / C::BN;
    const long tiles = (long)gy * gx;
    if (tiles == 0)
        return hipSuccess;
    const int vec8 = L.vec4 && ((uintptr_t)L.C % 16 == 0) && (L.ldc % 8 == 0) && (L.N % 8 == 0);
    hipLaunchKernelGGL((k_classic_q4<C, BF>), dim3((unsigned)tiles), dim3(C::NT), 0, st,
                       (const u16*)L.A, L.lda, (const u16*)L.B, L.ldb, (u16*)L.C, L.ldc, L.M, L.N, L.K,
                       gy, gx, L.P, L.vec4, vec8);
    return hipGetLastError();
}

// ------------------------------------------------------------------ skinny products
//
// M <= 64 (decode-shaped products): the run time is streaming B once from
// HBM, so the kernel is built for bytes in flight rather than MFMA rate.
// One workgroup per 64-column strip of B; each of its 4 waves takes every
// 4th k-tile of 32 through a private 5-stage direct-to-LDS ring (no
// workgroup barrier inside the K loop: a wave only reads what it loaded),
// which keeps 4 k-tiles per wave, 128 KB per compute unit, in flight.  The
// rows of A (padded to 32 or 64 with zeros) ride along in each k-tile.  The
// four partial tiles are summed through LDS in a fixed order at the end.

namespace sk {

// BK: k-depth of one stage (32: 64-byte A rows; 64: 128-byte A rows, one
// whole cache line per row and request); NW: waves, each streaming every
// NW-th stage through a private ring of NST stages, NST - 1 ahead.
template <int BM_, int BK_ = 32, int NW_ = 4, int NST_ = 5>
struct SCfg {
    static constexpr int BM = BM_, BN = 64, BK = BK_, MT = 32, NW = NW_, NT = NW_ * 64;
    static constexpr int WM = 1, WN = 1, WTM = BM, WTN = BN;    // each wave covers the whole tile
    static constexpr int FM = BM / 32, FN = BN / 32;
    static constexpr int KSTEPS = BK / 16;                       // 32x32x16 k-steps per stage
    using acc_t = f32x16;
    static constexpr int NACC = 16;
    static constexpr int NSTAGE = NST_, AHEAD = NST_ - 1;
    static constexpr int AROW = BK * 2, BROW = BN * 2;
    static constexpr int LPR = AROW / 16;                        // lanes (16-byte chunks) per A row
    static constexpr int A_BYTES = BM * AROW, B_BYTES = BK * BROW;
    static constexpr int STAGE = A_BYTES + B_BYTES;
    static constexpr int RING = NSTAGE * STAGE;                  // per wave
    static constexpr int LDS = NW * RING;
    static constexpr int A_PER = A_BYTES / 1024, B_PER = B_BYTES / 1024, PER = A_PER + B_PER;
    static_assert(BK == 32 || BK == 64, "A row swizzles below");
    static_assert(A_BYTES % 1024 == 0 && B_BYTES % 1024 == 0, "DMA granularity");
    static_assert(LDS <= 160 * 1024, "LDS budget");
    static_assert(PER * AHEAD < 64, "every load in flight stays within the 6-bit vmcnt");
    static_assert(AHEAD >= 1 && AHEAD <= 4, "wait_tiles cases");
    static_assert(NW * FM * FN * NACC * 64 * 4 <= LDS, "partials fit in the ring");
    // XOR swizzle of the 16-byte chunks of A row m: the fragment reads (16
    // consecutive rows, one chunk each) then fall in distinct bank groups.
    __device__ static u32 a_swz(u32 m) { return BK == 32 ? tiles::a_swz(m) : (m >> 1) & 7u; }
};

// One wave's loads of k-tile k0 into `stage` (rows / columns / k beyond the
// operands read as zero).
template <class C>
__device__ __forceinline__ void dma_ktile(char* stage, const tiles::TileSrc& s, int lane)
{
    const u32x4 ra = q4::rsrc_words(s.a + s.k0);
    const u32x4 rb = q4::rsrc_words(s.b + (int64_t)s.k0 * s.ldb);
    const int kleft = s.K - s.k0;
    const u32 base = q4::lds_addr(stage);
#pragma unroll
    for (int i = 0; i < C::A_PER; ++i) {
        const int r = i * (64 / C::LPR) + lane / C::LPR;
        const int k = ((lane % C::LPR) ^ (int)C::a_swz(r)) * 8;
        const u32 off = ((r < s.a_rows) & (k < kleft)) ? (u32)(r * s.lda + k) * 2u : kOob;
        q4::dma16(ra, off, base + i * 1024);
    }
#pragma unroll
    for (int i = 0; i < C::B_PER; ++i) {
        const int byte = i * 1024 + lane * 16;
        const int r = byte / C::BROW;
        const int n = ((byte % C::BROW) >> 4) * 8;
        const u32 off = ((r < kleft) & (n < s.b_cols)) ? (u32)(r * s.ldb + n) * 2u : kOob;
        q4::dma16(rb, off, base + C::A_BYTES + i * 1024);
    }
}

template <class C>
__device__ __forceinline__ void wait_tiles(int n)
{
    static_assert(C::AHEAD <= 4, "cases below");
    if (n >= 3)
        q4::wait_vm<3 * C::PER>();
    else if (n == 2)
        q4::wait_vm<2 * C::PER>();
    else if (n == 1)
        q4::wait_vm<C::PER>();
    else
        tiles::wait_vm0();
}

// All fragments of one stage (KSTEPS k-steps) and their MFMAs, for the wave
// tile whose origin is (row0, col0) in the stage (row0 a multiple of 32).
template <class C, bool BF>
__device__ __forceinline__ void ktile(const char* stage, int lane, f32x16 (&acc)[C::FM][C::FN], u32 row0 = 0,
                                      u32 col0 = 0)
{
    const char* sA = stage + row0 * (u32)C::AROW;
    const char* sB = stage + C::A_BYTES + col0 * 2u;
    const u32 m = lane & 31;
    const int g = lane >> 4, s = lane & 15;
    const u32 kr = 8 * (g >> 1) + (s >> 2);
    u32x4 a[C::KSTEPS][C::FM], b[C::KSTEPS][C::FN];
#pragma unroll
    for (int st = 0; st < C::KSTEPS; ++st) {
        // k-step st, lane half h = lane / 32: logical chunk 2 st + h of row m
        // (rows 32 i + m share the swizzle of m: 32 is a multiple of its period)
        const u32 chunk = (2u * st + ((u32)lane >> 5)) ^ C::a_swz(m);
#pragma unroll
        for (int i = 0; i < C::FM; ++i)
            a[st][i] = *reinterpret_cast<const u32x4*>(sA + m * (u32)C::AROW + chunk * 16u + i * 32 * C::AROW);
#pragma unroll
        for (int j = 0; j < C::FN; ++j) {
            const u32 n = j * 32 + 16 * (g & 1) + 4 * (s & 3);
            const u32 boff = (kr + 16 * st) * C::BROW + n * 2;
            const tiles::s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) tiles::s16x4*)(sB + boff));
            const tiles::s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) tiles::s16x4*)(sB + boff + 4 * C::BROW));
            const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
            b[st][j] = u32x4{l2.x, l2.y, h2.x, h2.y};
        }
    }
#pragma unroll
    for (int st = 0; st < C::KSTEPS; ++st)
#pragma unroll
        for (int i = 0; i < C::FM; ++i)
#pragma unroll
            for (int j = 0; j < C::FN; ++j)
                acc[i][j] = mfma<BF>(b[st][j], a[st][i], acc[i][j]);
}

// Shared-ring variant: the waves (four for 64 rows, two for 32) load each
// 64-k stage together (an equal share of its A rows and of its B rows each)
// into one ring of NST stages, NST - 1 ahead, and after one barrier per stage
// each wave multiplies its 32 x BN/2 part of the BM x BN output tile.  The
// MFMAs spread over the SIMDs, and a stage holds one copy of A's rows for all
// the waves.
template <int NST_ = 5, int BN_ = 64, int BM_ = 64>
struct CCfg {
    static constexpr int BM = BM_, BN = BN_, BK = 64, MT = 32, WM = BM / 32, NW = 2 * WM, NT = NW * 64;
    static constexpr int WN = 2, WTM = 32, WTN = BN / 2;   // wave w: rows 32 (w % WM), columns BN/2 (w / WM)
    static constexpr int FM = 1, FN = WTN / 32;
    static_assert(BM == 32 || BM == 64, "one or two 32-row wave tiles");
    static constexpr int KSTEPS = BK / 16;
    using acc_t = f32x16;
    static constexpr int NACC = 16;
    static constexpr int NSTAGE = NST_, AHEAD = NST_ - 1;
    static constexpr int AROW = BK * 2, BROW = BN * 2;
    static constexpr int LPR = AROW / 16;
    static constexpr int A_BYTES = BM * AROW, B_BYTES = BK * BROW;
    static constexpr int STAGE = A_BYTES + B_BYTES;
    static constexpr int LDS = NSTAGE * STAGE;
    static constexpr int A_PER = A_BYTES / 1024 / NW, B_PER = B_BYTES / 1024 / NW;   // per wave
    static constexpr int PER = A_PER + B_PER;
    static_assert(A_BYTES % (1024 * NW) == 0 && B_BYTES % (1024 * NW) == 0, "DMA granularity");
    static_assert(LDS <= 160 * 1024, "LDS budget");
    static_assert(PER * AHEAD < 64, "every load in flight stays within the 6-bit vmcnt");
    static_assert(AHEAD >= 1, "prefetch depth");
    __device__ static u32 a_swz(u32 m) { return (m >> 1) & 7u; }
};

// Wave `wave`'s share of the loads of k-tile s.k0 into `stage`: A rows
// 16 wave .. 16 wave + 15 and B k-rows 16 wave .. 16 wave + 15 (rows, columns
// and k beyond the operands read as zero).
template <class C>
__device__ __forceinline__ void dma_ktile_shared(char* stage, const tiles::TileSrc& s, int wave, int lane)
{
    const u32x4 ra = q4::rsrc_words(s.a + s.k0);
    const u32x4 rb = q4::rsrc_words(s.b + (int64_t)s.k0 * s.ldb);
    const int kleft = s.K - s.k0;
    const u32 base = q4::lds_addr(stage);
#pragma unroll
    for (int i = 0; i < C::A_PER; ++i) {
        const int ins = wave * C::A_PER + i;
        const int r = ins * (64 / C::LPR) + lane / C::LPR;
        const int k = ((lane % C::LPR) ^ (int)C::a_swz(r)) * 8;
        const u32 off = ((r < s.a_rows) & (k < kleft)) ? (u32)(r * s.lda + k) * 2u : kOob;
        q4::dma16(ra, off, base + ins * 1024);
    }
#pragma unroll
    for (int i = 0; i < C::B_PER; ++i) {
        const int ins = wave * C::B_PER + i;
        const int byte = ins * 1024 + lane * 16;
        const int r = byte / C::BROW;
        const int n = ((byte % C::BROW) >> 4) * 8;
        const u32 off = ((r < kleft) & (n < s.b_cols)) ? (u32)(r * s.ldb + n) * 2u : kOob;
        q4::dma16(rb, off, base + C::A_BYTES + ins * 1024);
    }
}

}  // namespace sk

template <class C, bool BF>
__global__ void __launch_bounds__(C::NT, 1)
k_skinny_shared(const u16* __restrict__ A, int64_t lda, const u16* __restrict__ B, int64_t ldb, u16* __restrict__ Cm,
                int64_t ldc, int M, int N, int K, int vec4)
{
    __shared__ __attribute__((aligned(1024))) char smem[C::LDS];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave % C::WM, wn = wave / C::WM;
    const int n0 = blockIdx.x * C::BN;
    const u16* Bb = B + n0;
    const int nk = (K + C::BK - 1) / C::BK;
    auto src = [&](int t) { return tiles::TileSrc{A, (int)lda, M, Bb, (int)ldb, N - n0, t * C::BK, K}; };
    f32x16 acc[C::FM][C::FN];
    zero_acc<C>(acc);
#pragma unroll
    for (int u = 0; u < C::AHEAD; ++u)
        if (u < nk)
            sk::dma_ktile_shared<C>(smem + u * C::STAGE, src(u), wave, lane);
    // stage offsets of tile t (read) and of tile t + AHEAD (written), advanced
    // by one stage per k-tile with wrap-around
    int rd = 0, wr = C::AHEAD * C::STAGE;
    for (int t = 0; t < nk; ++t) {
        // this wave's loads of tile t landed (tiles up to min(t + AHEAD - 1,
        // nk - 1) were issued); its fragment reads of tile t - 1 completed
        q4::wait_tiles<C>(min(nk - 1 - t, C::AHEAD - 1));
        tiles::wait_lgkm0();
        // every wave's loads of tile t landed, and every wave is done with
        // tile t - 1's stage, which takes tile t + AHEAD
        tiles::bar();
        if (t + C::AHEAD < nk)
            sk::dma_ktile_shared<C>(smem + wr, src(t + C::AHEAD), wave, lane);
        sk::ktile<C, BF>(smem + rd, lane, acc, (u32)(wm * C::WTM), (u32)(wn * C::WTN));
        rd = rd + C::STAGE == C::LDS ? 0 : rd + C::STAGE;
        wr = wr + C::STAGE == C::LDS ? 0 : wr + C::STAGE;
    }
    if (vec4)
        store_c<C, BF, true>(acc, Cm + n0, ldc, M, N - n0, wm, wn, lane);
    else
        store_c<C, BF, false>(acc, Cm + n0, ldc, M, N - n0, wm, wn, lane);
}

template <class C, bool BF>
hipError_t launch_skinny_shared_t(const ClassicLaunch& L, hipStream_t st)
{
    const int gx = (L.N + C::BN - 1) / C::BN;
    if (gx == 0 || L.M == 0)
        return hipSuccess;
    hipLaunchKernelGGL((k_skinny_shared<C, BF>), dim3((unsigned)gx), dim3(C::NT), 0, st, (const u16*)L.A, L.lda,
                       (const u16*)L.B, L.ldb, (u16*)L.C, L.ldc, L.M, L.N, L.K, L.vec4);
    return hipGetLastError();
}

// K split for up to 64 rows (tiles of 32 rows on two waves or 64 rows on
// four): the S workgroups of a 128-column strip (S = 2, 4 or 8; blocks
// 8 S (s / 8) + 8 q + s % 8 for piece q, all on one XCD) each take one S-th
// of K, so each reads S times fewer bytes of A per byte of B than an unsplit
// 64-column kernel, whose time grows with the A bytes every workgroup
// re-reads, and few strips still fill the chip.  The K loop is
// k_skinny_shared's.  Each piece writes the rows below M of its fp32 partial
// tile to the workspace, row-major through LDS (one row of a one-row product
// is 512 contiguous bytes); k_split_reduce, the next launch on the stream,
// adds the S partials in piece order and rounds into C.  The stream orders
// the two kernels, so the workspace needs no clearing and no counters, and
// any call or graph replay finds it ready.  An in-kernel exchange (the last
// of the S pieces to count its arrival in an agent-scope atomic adds the
// partials) measured 1.06-1.5x slower: every piece's release writes its
// XCD's L2 back, and the count, the acquire and the partial loads are
// round trips in series at the end of the kernel.
template <class C, bool BF>
__global__ void __launch_bounds__(C::NT, 1)
k_skinny_split(const u16* __restrict__ A, int64_t lda, const u16* __restrict__ B, int64_t ldb, int M, int N, int K,
               int S, int kh, float* __restrict__ part)
{
    static_assert(C::BN == kSplitCols && C::MT == 32 && C::FM == 1, "strip and tile shape of the workspace layout");
    __shared__ __attribute__((aligned(1024))) char smem[C::LDS];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave % C::WM, wn = wave / C::WM;
    const int b = blockIdx.x, r = b % (8 * S);
    const int strip = (b / (8 * S)) * 8 + r % 8, piece = r / 8;
    const int n0 = strip * C::BN;
    if (n0 >= N)
        return;                     // the grid covers whole groups of 8 strips
    const int kb = piece * kh, klen = max(0, min(K - kb, kh));
    const u16* Ah = A + kb;
    const u16* Bh = B + (int64_t)kb * ldb + n0;
    const int nk = (klen + C::BK - 1) / C::BK;
    auto src = [&](int t) { return tiles::TileSrc{Ah, (int)lda, M, Bh, (int)ldb, N - n0, t * C::BK, klen}; };
    f32x16 acc[C::FM][C::FN];
    zero_acc<C>(acc);
#pragma unroll
    for (int u = 0; u < C::AHEAD; ++u)
        if (u < nk)
            sk::dma_ktile_shared<C>(smem + u * C::STAGE, src(u), wave, lane);
    int rd = 0, wr = C::AHEAD * C::STAGE;
    for (int t = 0; t < nk; ++t) {
        q4::wait_tiles<C>(min(nk - 1 - t, C::AHEAD - 1));
        tiles::wait_lgkm0();
        tiles::bar();
        if (t + C::AHEAD < nk)
            sk::dma_ktile_shared<C>(smem + wr, src(t + C::AHEAD), wave, lane);
        sk::ktile<C, BF>(smem + rd, lane, acc, (u32)(wm * C::WTM), (u32)(wn * C::WTN));
        rd = rd + C::STAGE == C::LDS ? 0 : rd + C::STAGE;
        wr = wr + C::STAGE == C::LDS ? 0 : wr + C::STAGE;
    }
    // The partial tile goes through LDS (the ring is free now) so that its
    // rows below M leave as contiguous 16-byte chunks: chunk c of the tile is
    // row c / 32, columns 4 (c % 32) .. + 3, and thread t writes chunks
    // t + k NT.  Staging rows are padded by 16 bytes against bank conflicts.
    constexpr int SROW = C::BN * 4 + 16, CPR = C::BN / 4, CPT = C::BM * CPR / C::NT;
    static_assert(C::BM * SROW <= C::LDS && C::BM * CPR % C::NT == 0, "staging");
    tiles::bar();                                      // every wave is done reading the ring
    {
        const int m = wm * C::WTM + (lane & 31), hi = lane >> 5;
#pragma unroll
        for (int j = 0; j < C::FN; ++j)
#pragma unroll
            for (int g = 0; g < C::NACC / 4; ++g)
                *reinterpret_cast<f32x4*>(smem + m * SROW + (wn * C::WTN + j * 32 + 8 * g + 4 * hi) * 4) =
                    f32x4{acc[0][j][4 * g], acc[0][j][4 * g + 1], acc[0][j][4 * g + 2], acc[0][j][4 * g + 3]};
    }
    tiles::wait_lgkm0();
    tiles::bar();
    f32x4* tile = reinterpret_cast<f32x4*>(part) + ((int64_t)strip * S + piece) * C::BM * CPR;
#pragma unroll
    for (int k = 0; k < CPT; ++k) {
        const int c = tid + k * C::NT;
        if (c / CPR < M)
            tile[c] = *reinterpret_cast<const f32x4*>(smem + (c / CPR) * SROW + (c % CPR) * 16);
    }
}

// C = the sum of the S partials of each output element, in piece order,
// rounded once.  The partials are tiles of `rows` x W fp32 per strip of W
// columns, the S pieces of a strip one after another (W = 128, rows = the
// streaming kernel's tile rows; or W = N, rows = M: S full planes).  One
// thread per 4 consecutive columns of one row, so consecutive threads read
// consecutive 16-byte chunks of a partial row.
template <bool BF>
__global__ void __launch_bounds__(256) k_split_reduce(const f32x4* __restrict__ part, int S, int rows, int W,
                                                      u16* __restrict__ Cm, int64_t ldc, int M, int N, int vec4)
{
    const int64_t cpr = (N + 3) / 4;
    const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (c >= (int64_t)M * cpr)
        return;
    const int row = (int)(c / cpr), col = (int)(c % cpr) * 4;
    const int64_t cpw = W / 4, tile = (int64_t)rows * cpw;
    const f32x4* p = part + (int64_t)(col / W) * S * tile + (int64_t)row * cpw + (col % W) / 4;
    f32x4 sum = __builtin_nontemporal_load(p);
    for (int q = 1; q < S; ++q)
        sum += __builtin_nontemporal_load(p + q * tile);
    u16* out = Cm + (int64_t)row * ldc + col;
    if (vec4) {
        // C 8-byte aligned, ldc and N multiples of 4: the 4 columns are all valid
        *reinterpret_cast<u32x2*>(out) = u32x2{pack2<BF>(sum.x, sum.y), pack2<BF>(sum.z, sum.w)};
    } else {
        const float xs[4] = {sum.x, sum.y, sum.z, sum.w};
#pragma unroll
        for (int e = 0; e < 4; ++e)
            if (col + e < N)
                out[e] = f2h<BF>(xs[e]);
    }
}

// The reduction launch after a K-split kernel.
template <bool BF>
hipError_t launch_split_reduce(const ClassicLaunch& L, int rows, int W, hipStream_t st)
{
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    const int64_t chunks = (int64_t)L.M * ((L.N + 3) / 4);
    hipLaunchKernelGGL((k_split_reduce<BF>), dim3((unsigned)((chunks + 255) / 256)), dim3(256), 0, st,
                       (const f32x4*)L.split_ws, L.split_s, rows, W, (u16*)L.C, L.ldc, L.M, L.N, L.vec4);
    return hipGetLastError();
}

template <class C, bool BF>
hipError_t launch_skinny_split_t(const ClassicLaunch& L, hipStream_t st)
{
    const int strips = (L.N + C::BN - 1) / C::BN, S = L.split_s;
    if (strips == 0 || L.M == 0)
        return hipSuccess;
    if ((S != 2 && S != 4 && S != 8) || L.M > C::BM || ((uintptr_t)L.split_ws % 256) != 0)
        return hipErrorInvalidValue;
    const int kh = ((L.K + S - 1) / S + C::BK - 1) / C::BK * C::BK;
    hipLaunchKernelGGL((k_skinny_split<C, BF>), dim3((unsigned)((strips + 7) / 8 * 8 * S)), dim3(C::NT), 0, st,
                       (const u16*)L.A, L.lda, (const u16*)L.B, L.ldb, L.M, L.N, L.K, S, kh, (float*)L.split_ws);
    return launch_split_reduce<BF>(L, C::BM, kSplitCols, st);
}

// K split of the 256-row-and-up classic kernel (128 x 128 tiles, long K):
// S pieces of K per tile write S fp32 planes of M x N, then the reduction.
template <class C, bool BF>
hipError_t launch_classic_m16_split_t(const ClassicLaunch& L, hipStream_t st)
{
    const int gy = (L.M + C::BM - 1) / C::BM, gx = (L.N + C::BN - 1) / C::BN, S = L.split_s;
    const long tiles = (long)gy * gx;
    if (tiles == 0)
        return hipSuccess;
    if ((S != 2 && S != 4 && S != 8) || L.N % 4 != 0 || ((uintptr_t)L.split_ws % 256) != 0)
        return hipErrorInvalidValue;
    const int kh = ((L.K + S - 1) / S + C::BK - 1) / C::BK * C::BK;
    hipLaunchKernelGGL((k_classic_m16<C, BF, true>), dim3((unsigned)(tiles * S)), dim3(C::NT), 0, st,
                       (const u16*)L.A, L.lda, (const u16*)L.B, L.ldb, (u16*)L.C, L.ldc, L.M, L.N, L.K,
                       gy, gx, L.P, 0, 0, 0, kh, (int)tiles, 0, (float*)L.split_ws);
    return launch_split_reduce<BF>(L, L.M, L.N, st);
}

// C over the tail tiles tile0 .. tile0 + T - 1 (tile_coords order) = the sum
// of their S compact partial tiles (slot piece * T + i, BM x BN fp32 each),
// in piece order, rounded once.  One thread per 4 consecutive columns of a
// tile row.
template <int BM, int BN, bool BF>
__global__ void __launch_bounds__(256) k_tail_reduce(const f32x4* __restrict__ part, int S, int T, int tile0, int gy,
                                                     int gx, int P, u16* __restrict__ Cm, int64_t ldc, int M, int N,
                                                     int vec4)
{
    constexpr int CPR = BN / 4, CPT = BM * CPR;
    const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (c >= (int64_t)T * CPT)
        return;
    const int i = (int)(c / CPT), r = (int)(c % CPT) / CPR, c4 = (int)(c % CPR);
    int p, q;
    tile_coords((int32_t)(tile0 + i), gy, gx, P, 8, &p, &q);
    const int m = p * BM + r, n = q * BN + c4 * 4;
    if (m >= M || n >= N)
        return;
    const f32x4* src = part + (int64_t)i * CPT + r * CPR + c4;
    f32x4 sum = __builtin_nontemporal_load(src);
    for (int k = 1; k < S; ++k)
        sum += __builtin_nontemporal_load(src + (int64_t)k * T * CPT);
    u16* out = Cm + (int64_t)m * ldc + n;
    if (vec4) {
        // C 8-byte aligned, ldc and N multiples of 4: the 4 columns are all valid
        *reinterpret_cast<u32x2*>(out) = u32x2{pack2<BF>(sum.x, sum.y), pack2<BF>(sum.z, sum.w)};
    } else {
        const float xs[4] = {sum.x, sum.y, sum.z, sum.w};
#pragma unroll
        for (int e = 0; e < 4; ++e)
            if (n + e < N)
                out[e] = f2h<BF>(xs[e]);
    }
}

// The last, partial round of a multi-round classic grid split along K: the
// full rounds run as usual, then the T tail tiles run as S pieces of K each
// (T S workgroups, at most one round) writing compact fp32 partial tiles,
// then k_tail_reduce adds them into C.
template <class C, bool BF>
hipError_t launch_classic_m16_tail_t(const ClassicLaunch& L, hipStream_t st)
{
    const int gy = (L.M + C::BM - 1) / C::BM, gx = (L.N + C::BN - 1) / C::BN, S = L.split_s;
    const long tiles = (long)gy * gx;
    const long full = tiles / L.P * L.P, T = tiles - full;
    if (tiles == 0)
        return hipSuccess;
    if ((S != 2 && S != 4 && S != 8) || full == 0 || T == 0 || T * S > L.P || ((uintptr_t)L.split_ws % 256) != 0)
        return hipErrorInvalidValue;
    const int vec8 = L.vec4 && ((uintptr_t)L.C % 16 == 0) && (L.ldc % 8 == 0) && (L.N % 8 == 0);
    hipLaunchKernelGGL((k_classic_m16<C, BF>), dim3((unsigned)full), dim3(C::NT), 0, st,
                       (const u16*)L.A, L.lda, (const u16*)L.B, L.ldb, (u16*)L.C, L.ldc, L.M, L.N, L.K,
                       gy, gx, L.P, L.vec4, vec8, 0, L.K, 1, 0, nullptr);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    const int kh = ((L.K + S - 1) / S + C::BK - 1) / C::BK * C::BK;
    hipLaunchKernelGGL((k_classic_m16<C, BF, true>), dim3((unsigned)(T * S)), dim3(C::NT), 0, st,
                       (const u16*)L.A, L.lda, (const u16*)L.B, L.ldb, (u16*)L.C, L.ldc, L.M, L.N, L.K,
                       gy, gx, L.P, 0, 0, (int)full, kh, (int)T, 1, (float*)L.split_ws);
    e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    const int64_t chunks = T * (C::BM * C::BN / 4);
    hipLaunchKernelGGL((k_tail_reduce<C::BM, C::BN, BF>), dim3((unsigned)((chunks + 255) / 256)), dim3(256), 0, st,
                       (const f32x4*)L.split_ws, S, (int)T, (int)full, gy, gx, L.P, (u16*)L.C, L.ldc, L.M, L.N,
                       L.vec4);
    return hipGetLastError();
}

template <class C, bool BF>
__global__ void __launch_bounds__(C::NT, 1)
k_skinny(const u16* __restrict__ A, int64_t lda, const u16* __restrict__ B, int64_t ldb, u16* __restrict__ Cm,
         int64_t ldc, int M, int N, int K, int vec4)
{
    __shared__ __attribute__((aligned(1024))) char smem[C::LDS];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n0 = blockIdx.x * C::BN;
    const u16* Bb = B + n0;
    char* ring = smem + wave * C::RING;
    const int nk = (K + C::BK - 1) / C::BK;
    const int nu = nk > wave ? (nk - wave + C::NW - 1) / C::NW : 0;    // k-tiles of this wave
    auto src = [&](int u) {
        return tiles::TileSrc{A, (int)lda, M, Bb, (int)ldb, N - n0, (wave + u * C::NW) * C::BK, K};
    };
    f32x16 acc[C::FM][C::FN];
    zero_acc<C>(acc);
#pragma unroll
    for (int u = 0; u < C::AHEAD; ++u)
        if (u < nu)
            sk::dma_ktile<C>(ring + u * C::STAGE, src(u), lane);
    for (int u = 0; u < nu; ++u) {
        sk::wait_tiles<C>(min(nu - 1 - u, C::AHEAD - 1));   // tile u landed
        sk::ktile<C, BF>(ring + (u % C::NSTAGE) * C::STAGE, lane, acc);
        // tile u-1's stage is free: its fragments were consumed by the MFMAs above
        if (u + C::AHEAD < nu) {
            tiles::wait_lgkm0();
            sk::dma_ktile<C>(ring + ((u + C::AHEAD) % C::NSTAGE) * C::STAGE, src(u + C::AHEAD), lane);
        }
    }
    // Sum the four waves' partial tiles in a fixed order through LDS.
    tiles::wait_vm0();
    __syncthreads();
    float* part = reinterpret_cast<float*>(smem);
    if (wave > 0) {
#pragma unroll
        for (int i = 0; i < C::FM; ++i)
#pragma unroll
            for (int j = 0; j < C::FN; ++j)
#pragma unroll
                for (int e = 0; e < C::NACC; ++e)
                    part[((((wave - 1) * C::FM + i) * C::FN + j) * C::NACC + e) * 64 + lane] = acc[i][j][e];
    }
    __syncthreads();
    if (wave == 0) {
#pragma unroll
        for (int w = 0; w < C::NW - 1; ++w)
#pragma unroll
            for (int i = 0; i < C::FM; ++i)
#pragma unroll
                for (int j = 0; j < C::FN; ++j)
#pragma unroll
                    for (int e = 0; e < C::NACC; ++e)
                        acc[i][j][e] += part[(((w * C::FM + i) * C::FN + j) * C::NACC + e) * 64 + lane];
        if (vec4)
            store_c<C, BF, true>(acc, Cm + n0, ldc, M, N - n0, 0, 0, lane);
        else
            store_c<C, BF, false>(acc, Cm + n0, ldc, M, N - n0, 0, 0, lane);
    }
}

template <class C, bool BF>
hipError_t launch_skinny_t(const ClassicLaunch& L, hipStream_t st)
{
    const int gx = (L.N + C::BN - 1) / C::BN;
    if (gx == 0 || L.M == 0)
        return hipSuccess;
    hipLaunchKernelGGL((k_skinny<C, BF>), dim3((unsigned)gx), dim3(C::NT), 0, st, (const u16*)L.A, L.lda,
                       (const u16*)L.B, L.ldb, (u16*)L.C, L.ldc, L.M, L.N, L.K, L.vec4);
    return hipGetLastError();
}

// ------------------------------------------------------------------ unfused path helpers

// Runtime-coefficient pre-pass: one thread per 8-element chunk position of
// one product's combined operand; it sums the chunk of every block with a
// non-zero coefficient in fp32 (the coefficients are uniform) and rounds once.
struct GenPrepassParams {
    const u16* X;
    int64_t ldx;
    int rows, cols, bcols, nblocks, rank;
    int8_t coef[kGenMaxRank * kGenMaxBlocks];
    u16* out;
    int64_t ldo, stride;
};

// One thread per 8-element chunk position of a block: it reads that chunk of
// every block once (at most kGenMaxBlocks, held in registers), then writes
// the chunk of every combined operand, each summed in fp32 and rounded once.
// PK: the operands are written tile-packed (GenPrepassLaunch::packed).
template <bool IBF, bool OBF, bool PK>
__global__ void __launch_bounds__(256) k_gen_prepass(const GenPrepassParams gp)
{
    const int cpr = gp.cols / 8;                       // chunks per row
    const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (c >= (int64_t)gp.rows * cpr)
        return;
    int row, col;
    u16* out;
    if constexpr (PK) {
        // Threads walk the packed layout (tile row tr, k-tile kt, row rr of
        // the tile, position pos holding chunk pos ^ ((rr >> 1) & 3) of that
        // row).  With an even number of k-tiles, 8 consecutive threads take
        // the 8 chunks of one row over a pair of k-tiles: a wave reads 8 whole
        // 128-byte lines of 8 rows and writes two runs of 512 bytes.  Else 4
        // threads take one k-tile's row (64 bytes read per row).
        const int kts = gp.cols / kPackCols;
        int pos, rr, kt, tr;
        if ((kts & 1) == 0) {
            const int j = (int)(c % 8);
            rr = (int)((c / 8) % kPackRows);
            const int64_t pr = c / (8 * kPackRows);
            tr = (int)(pr / (kts / 2));
            kt = (int)(pr % (kts / 2)) * 2 + j / 4;
            pos = j % 4;
        } else {
            pos = (int)(c % 4);
            rr = (int)((c / 4) % kPackRows);
            const int64_t blk = c / (4 * kPackRows);
            tr = (int)(blk / kts);
            kt = (int)(blk % kts);
        }
        row = tr * kPackRows + rr;
        col = kt * kPackCols + (pos ^ ((rr >> 1) & 3)) * 8;
        out = gp.out + (((int64_t)tr * kts + kt) * kPackRows + rr) * kPackCols + pos * 8;
    } else {
        row = (int)(c / cpr);
        col = (int)(c % cpr) * 8;
        out = gp.out + (int64_t)row * gp.ldo + col;
    }
    u32x4 v[kGenMaxBlocks];
#pragma unroll
    for (int b = 0; b < kGenMaxBlocks; ++b) {
        if (b < gp.nblocks) {
            const int br = b / gp.bcols, bc = b % gp.bcols;
            v[b] = *reinterpret_cast<const u32x4*>(gp.X + (int64_t)(br * gp.rows + row) * gp.ldx +
                                                   (int64_t)bc * gp.cols + col);
        }
    }
    for (int r = 0; r < gp.rank; ++r) {
        float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
        for (int b = 0; b < kGenMaxBlocks; ++b) {
            if (b < gp.nblocks) {
                const int w = gp.coef[r * kGenMaxBlocks + b];
                if (w != 0) {
                    const float fw = (float)w;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        acc[2 * e] += fw * h2f<IBF>((u16)(v[b][e] & 0xffffu));
                        acc[2 * e + 1] += fw * h2f<IBF>((u16)(v[b][e] >> 16));
                    }
                }
            }
        }
        *reinterpret_cast<u32x4*>(out + (int64_t)r * gp.stride) =
            u32x4{pack2<OBF>(acc[0], acc[1]), pack2<OBF>(acc[2], acc[3]), pack2<OBF>(acc[4], acc[5]),
                  pack2<OBF>(acc[6], acc[7])};
    }
}

template <bool IBF, bool OBF>
hipError_t launch_gen_prepass_t(const GenPrepassLaunch& L, hipStream_t st)
{
    const int64_t chunks = (int64_t)L.rows * (L.cols / 8);
    if (chunks == 0 || L.rank == 0)
        return hipSuccess;
    GenPrepassParams gp;
    gp.X = (const u16*)L.X;
    gp.ldx = L.ldx;
    gp.rows = L.rows;
    gp.cols = L.cols;
    gp.bcols = L.bcols;
    gp.nblocks = L.nblocks;
    gp.rank = L.rank;
    for (int i = 0; i < kGenMaxRank * kGenMaxBlocks; ++i)
        gp.coef[i] = L.coef[i];
    gp.out = (u16*)L.out;
    gp.ldo = L.ldo;
    gp.stride = L.stride;
    const dim3 grid((unsigned)((chunks + 255) / 256));
    if (L.packed) {
        if (L.rows % kPackRows != 0 || L.cols % kPackCols != 0)
            return hipErrorInvalidValue;
        hipLaunchKernelGGL((k_gen_prepass<IBF, OBF, true>), grid, dim3(256), 0, st, gp);
    } else {
        hipLaunchKernelGGL((k_gen_prepass<IBF, OBF, false>), grid, dim3(256), 0, st, gp);
    }
    return hipGetLastError();
}

// ------------------------------------------------------------------ fused group kernel

template <int LEVELS>
struct FusedCfg;
template <>
struct FusedCfg<2> { using C = CfgF2; };   // the on-chip two-level kernel

// C_o += W[r][o] * H for every output block o.  The coefficients are
// uniform kernel arguments; zero ones are skipped by a scalar branch.
template <int NOUT, class C>
__device__ __forceinline__ void combine_h(const int8_t* w, const typename C::acc_t (&H)[C::FM][C::FN],
                                          typename C::acc_t (&Cacc)[NOUT][C::FM][C::FN])
{
#pragma unroll
    for (int o = 0; o < NOUT; ++o) {
        const int c = w[o];
        if (c != 0) {
            const float fc = (float)c;
#pragma unroll
            for (int i = 0; i < C::FM; ++i)
#pragma unroll
                for (int j = 0; j < C::FN; ++j)
                    Cacc[o][i][j] += fc * H[i][j];
        }
    }
}

// Outer level of the two-level path: the finished inner outputs of this
// group tile go, scaled by W1[r1][i1, j1], into the fp32 blocks of every
// outer output (i1, j1) that outer product r1 feeds (mode per output: store,
// add, add and round into C, or round into C).  Rows past the block edge get
// an out-of-range offset (loads read zero, stores are dropped); columns come
// in fours and Nb is a multiple of 8.
template <class C, bool CBF>
__device__ __forceinline__ void outer_update(const FusedParams& fp, int m0, int n0,
                                             const f32x4 (&Cacc)[4][C::FM][C::FN], int wm, int wn, int lane)
{
    const int rows = fp.Mb - m0, cols = fp.Nb - n0, ld = fp.Nb;
#pragma unroll
    for (int o1 = 0; o1 < 4; ++o1) {
        const int mode = fp.omode[o1];
        if (mode == kOuterNone)
            continue;
        const float w = fp.ow[o1];
        const int i1 = o1 >> 1, j1 = o1 & 1;
#pragma unroll
        for (int o2 = 0; o2 < 4; ++o2) {
            const int bi = 2 * i1 + (o2 >> 1), bj = 2 * j1 + (o2 & 1);
            const rsrc_t ra = make_rsrc(fp.acc + (int64_t)(bi * 4 + bj) * fp.Mb * fp.Nb + (int64_t)m0 * ld + n0);
            // The mode is uniform: the read-modify-write modes issue all of
            // the block's loads before the first use (one round trip).
            auto off_of = [&](int i, int j) {
                const int m = wm * C::WTM + i * 16 + (lane & 15);
                const int n = wn * C::WTN + j * 16 + 4 * (lane >> 4);
                return (m < rows && n < cols) ? (u32)(m * ld + n) * 4u : kOob;
            };
            f32x4 t[C::FM][C::FN];
            if (mode == kOuterAdd || mode == kOuterFinish) {
#pragma unroll
                for (int i = 0; i < C::FM; ++i)
#pragma unroll
                    for (int j = 0; j < C::FN; ++j)
                        t[i][j] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(ra, off_of(i, j), 0, 0));
#pragma unroll
                for (int i = 0; i < C::FM; ++i)
#pragma unroll
                    for (int j = 0; j < C::FN; ++j)
                        t[i][j] = Cacc[o2][i][j] * w + t[i][j];
            } else {
#pragma unroll
                for (int i = 0; i < C::FM; ++i)
#pragma unroll
                    for (int j = 0; j < C::FN; ++j)
                        t[i][j] = Cacc[o2][i][j] * w;
            }
            if (mode == kOuterStore || mode == kOuterAdd) {
#pragma unroll
                for (int i = 0; i < C::FM; ++i)
#pragma unroll
                    for (int j = 0; j < C::FN; ++j)
                        __builtin_amdgcn_raw_buffer_store_b128(
                            __builtin_bit_cast(__attribute__((ext_vector_type(4))) unsigned int, t[i][j]), ra,
                            off_of(i, j), 0, 0);
            }
            if (mode == kOuterFinish || mode == kOuterOnly) {
                // + 0: a zero sum written as -0 becomes +0 (as in the classic product)
#pragma unroll
                for (int i = 0; i < C::FM; ++i)
#pragma unroll
                    for (int j = 0; j < C::FN; ++j)
                        t[i][j] = t[i][j] + 0.0f;
                store_c<C, CBF, true>(t, fp.C + (int64_t)(bi * fp.Mb + m0) * fp.ldc + bj * fp.Nb + n0, fp.ldc, rows,
                                      cols, wm, wn, lane);
            }
        }
    }
}

// Writes a group's output blocks.  A split piece first publishes its fp32
// partial; the second piece to arrive (one agent-scope acquire/release atomic
// per workgroup on a per-slot counter) adds the other partial, writes C and
// resets the counter.
// fp32 addition commutes, so the result does not depend on arrival order.
// OUTER: the outputs go through outer_update instead of straight into C.
template <int NOUT, class C, bool CBF, bool OUTER = false>
__device__ __forceinline__ void fused_epilogue(const FusedParams& fp, const Item& item, int m0, int n0,
                                               typename C::acc_t (&Cacc)[NOUT][C::FM][C::FN], int tid, int wm,
                                               int wn, int lane, int* sh_old)
{
    constexpr int S = NOUT == 4 ? 2 : 4;
    constexpr int G4 = C::NACC / 4;                     // float4 groups per accumulator tile
    constexpr int PART_F4 = NOUT * C::FM * C::FN * G4;  // float4 per thread in a partial
    bool store = true;
    if (item.slot >= 0) {
        const int which = item.pos0 == 0 ? 0 : 1;
        f32x4* mine = reinterpret_cast<f32x4*>(fp.partial) + ((int64_t)item.slot * 2 + which) * PART_F4 * C::NT;
        const f32x4* other = reinterpret_cast<const f32x4*>(fp.partial) + ((int64_t)item.slot * 2 + (1 - which)) * PART_F4 * C::NT;
#pragma unroll
        for (int o = 0; o < NOUT; ++o)
#pragma unroll
            for (int i = 0; i < C::FM; ++i)
#pragma unroll
                for (int j = 0; j < C::FN; ++j)
#pragma unroll
                    for (int g = 0; g < G4; ++g) {
                        const int e = ((o * C::FM + i) * C::FN + j) * G4 + g;
                        mine[(int64_t)e * C::NT + tid] =
                            f32x4{Cacc[o][i][j][4 * g], Cacc[o][i][j][4 * g + 1],
                                  Cacc[o][i][j][4 * g + 2], Cacc[o][i][j][4 * g + 3]};
                    }
        // Each wave waits until its own partial stores have reached the L2 of
        // its XCD.  Thread 0's agent-scope acquire-release atomic then writes
        // that L2 back to memory once for the whole workgroup (and, on the
        // second arrival, invalidates it before the other piece's partial is
        // read).  A per-thread agent-scope fence here made every wave write
        // back and invalidate the whole L2 of its XCD, which cost more than
        // the split saved.
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (tid == 0)
            *sh_old = __hip_atomic_fetch_add(fp.counters + item.slot, 1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
        __syncthreads();
        store = *sh_old == 1;
        if (store) {
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
#pragma unroll
            for (int o = 0; o < NOUT; ++o) {
                // One output block at a time keeps the partial loads from all
                // being hoisted ahead of the adds.
                asm volatile("" ::: "memory");
#pragma unroll
                for (int i = 0; i < C::FM; ++i)
#pragma unroll
                    for (int j = 0; j < C::FN; ++j)
#pragma unroll
                        for (int g = 0; g < G4; ++g) {
                            const int e = ((o * C::FM + i) * C::FN + j) * G4 + g;
                            const f32x4 v = __builtin_nontemporal_load(other + (int64_t)e * C::NT + tid);
                            Cacc[o][i][j][4 * g] += v.x;
                            Cacc[o][i][j][4 * g + 1] += v.y;
                            Cacc[o][i][j][4 * g + 2] += v.z;
                            Cacc[o][i][j][4 * g + 3] += v.w;
                        }
            }
            if (tid == 0)
                __hip_atomic_store(fp.counters + item.slot, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
    if (store) {
        if constexpr (OUTER) {
            static_assert(NOUT == 4, "the outer level runs the one-level kernel");
            outer_update<C, CBF>(fp, m0, n0, Cacc, wm, wn, lane);
        } else {
#pragma unroll
            for (int o = 0; o < NOUT; ++o) {
                const int bi = o / S, bj = o % S;
                store_c<C, CBF, true>(Cacc[o], fp.C + (int64_t)(bi * fp.Mb + m0) * fp.ldc + bj * fp.Nb + n0, fp.ldc,
                                      fp.Mb - m0, fp.Nb - n0, wm, wn, lane);
            }
        }
    }
}

template <int LEVELS, bool OBF, bool CBF>
__global__ void __launch_bounds__(FusedCfg<LEVELS>::C::NT) k_fused(const FusedParams fp)
{
    using C = typename FusedCfg<LEVELS>::C;
    constexpr int S = Scheme<LEVELS>::S, NOUT = S * S;
    __shared__ __attribute__((aligned(16))) char smem[C::LDS];
    __shared__ int sh_old;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / C::WN, wn = wave % C::WN;
    const int w = blockIdx.x;
    const int n_items = sched_count(fp.sp, w);
    const int nk = (fp.Kb + C::BK - 1) / C::BK;

    for (int it = 0; it < n_items; ++it) {
        const Item item = sched_item(fp.sp, w, it);
        int p, q;
        tile_coords(item.g, fp.sp.gy, fp.sp.gx, fp.sp.P, fp.sp.raster, &p, &q);
        const int m0 = p * C::BM, n0 = q * C::BN;

        typename C::acc_t Cacc[NOUT][C::FM][C::FN];
#pragma unroll
        for (int o = 0; o < NOUT; ++o)
            zero_acc<C>(Cacc[o]);
        typename C::acc_t H[C::FM][C::FN];
        zero_acc<C>(H);

        auto src_of = [&](int pos) {
            const int r = fp.order[pos];
            return make_src(fp.a[r] + (int64_t)m0 * fp.lda[r], fp.lda[r], fp.Mb - m0,
                            fp.b[r] + n0, fp.ldb[r], fp.Nb - n0, fp.Kb);
        };
        const int ntiles = (item.pos1 - item.pos0) * nk;
        Src nxt = src_of(item.pos0);
        Regs<C> Rg;
        load_tile<C, true>(Rg, nxt, 0, tid);
        store_tile<C>(smem, Rg, tid);
        __syncthreads();
        // The tile sequence runs through the group's products back to back:
        // the first tile of the next product is fetched while the last tile
        // of the current one is computed.
        for (int t = 0; t < ntiles; ++t) {
            const int t1 = t + 1;
            const char* cur = smem + (t & 1) * C::STAGE;
            if (t1 < ntiles) {
                const int k1 = t1 % nk;
                if (k1 == 0)
                    nxt = src_of(item.pos0 + t1 / nk);
                load_tile<C, true>(Rg, nxt, k1 * C::BK, tid);
                ktile<C, OBF, true>(cur, smem + (t1 & 1) * C::STAGE, Rg, H, wm, wn, lane, tid);
            } else {
                ktile<C, OBF, false>(cur, nullptr, Rg, H, wm, wn, lane, tid);
            }
            if (t % nk == nk - 1) {
                combine_h<NOUT, C>(fp.w[fp.order[item.pos0 + t / nk]], H, Cacc);
                zero_acc<C>(H);
            }
            __syncthreads();
        }

        fused_epilogue<NOUT, C, CBF>(fp, item, m0, n0, Cacc, tid, wm, wn, lane, &sh_old);
        __syncthreads();
    }
}

// ------------------------------------------------------------------ combine at load
//
// One-level group kernel that forms the combined operands while it stages
// k-tiles, so no pre-pass runs and no combined operand reaches memory
// ("FalconGEMM ...", section "从 LCMA 到 FalconGEMM", combine A/B; here moved
// into the tile loads).  Each operand of a one-level product is one or two
// input blocks with coefficients +-1.  Both blocks' tiles go global -> LDS
// by direct-to-LDS loads three k-tiles ahead (128 KiB ring; four ahead, the
// whole 160 KiB, measured no faster); all threads then fold the second term into the first
// in LDS, one 16-byte chunk of A and one of B per thread and k-tile, before
// the fragment reads.  Adding two bfloat16 values goes through fp32 (4
// unpacks, 2 adds, one packed RNE conversion per 32-bit word); two binary16
// values add with one packed instruction, whose single rounding of the exact
// sum equals rounding their fp32 sum (the fp32 sum of two binary16 values
// is inexact only when the smaller is below a quarter unit of the larger's
// last binary16 place, and then both give the larger).

template <bool BF>
__device__ __forceinline__ u32 add_h2(u32 x, u32 y)
{
    if constexpr (BF) {
        using v2 = __bf16 __attribute__((ext_vector_type(2)));
        return __builtin_bit_cast(u32, __builtin_bit_cast(v2, x) + __builtin_bit_cast(v2, y));
    } else {
        using v2 = _Float16 __attribute__((ext_vector_type(2)));
        return __builtin_bit_cast(u32, __builtin_bit_cast(v2, x) + __builtin_bit_cast(v2, y));
    }
}

// 8 waves of 64 x 32 on the 16x16x32 engine, 128 x 128 group tiles.
using MCFC = m16::Cfg<128, 128, 2, 4, 3>;

template <bool BF>
__global__ void __launch_bounds__(MCFC::NT, 1) k_fused_cal_m16(const FusedParams fp)
{
    using C = MCFC;
    constexpr int NOUT = 4;
    __shared__ __attribute__((aligned(1024))) char smem[C::NSTAGE * 2 * C::STAGE];
    __shared__ int sh_old;
    const int tid = threadIdx.x, lane0 = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / C::WN, wn = wave % C::WN;
    const int w = blockIdx.x;
    const int n_items = sched_count(fp.sp, w);
    const int nk = (fp.Kb + C::BK - 1) / C::BK;
    uint64_t ordw;
    __builtin_memcpy(&ordw, fp.order, sizeof ordw);
    auto order_at = [&](int pos) { return (int)(int8_t)(ordw >> (8 * pos)); };
    for (int it = 0; it < n_items; ++it) {
        // opaque per item: keeps lane-derived addresses from being held in
        // registers across the whole kernel
        int lane = lane0;
        asm volatile("" : "+v"(lane));
        const Item item = sched_item(fp.sp, w, it);
        int p, q;
        tile_coords(item.g, fp.sp.gy, fp.sp.gx, fp.sp.P, fp.sp.raster, &p, &q);
        const int m0 = p * C::BM, n0 = q * C::BN;
        f32x4 Cacc[NOUT][C::FM][C::FN];
#pragma unroll
        for (int o = 0; o < NOUT; ++o)
            zero_acc<C>(Cacc[o]);
        f32x4 H[C::FM][C::FN];
        zero_acc<C>(H);
        const int nprod = item.pos1 - item.pos0;
        const int ntiles = nprod * nk;
        // The engine asks for k-tile sources, folds and finished k-tiles in
        // increasing order, so each walks a cursor and reads a product's
        // parameters (kernel argument arrays) only when the product changes:
        // a dynamically indexed argument read waits for every load in
        // flight, which must not happen once per k-tile.
        struct Prod {
            const u16 *a, *b, *a2, *b2;
            int lda, ldb;
            u32 sa1, sa2, sb1, sb2;
        };
        auto prod = [&](int j) {
            const int r = order_at(item.pos0 + j);
            return Prod{fp.a[r], fp.b[r], fp.a2[r], fp.b2[r], (int)fp.lda[r], (int)fp.ldb[r],
                        fp.sa[r][0], fp.sa[r][1], fp.sb[r][0], fp.sb[r][1]};
        };
        int sj = 0, skt = 0;
        Prod ps = prod(0);
        auto src = [&](int, tiles::TileSrc* s1, tiles::TileSrc* s2) {
            *s1 = tiles::TileSrc{ps.a + (int64_t)m0 * ps.lda, ps.lda, fp.Mb - m0, ps.b + n0, ps.ldb, fp.Nb - n0,
                                 skt * C::BK, fp.Kb};
            *s2 = *s1;
            if (ps.a2)
                s2->a = ps.a2 + (int64_t)m0 * ps.lda;
            else
                s2->a_rows = 0;
            if (ps.b2)
                s2->b = ps.b2 + n0;
            else
                s2->b_cols = 0;
            if (++skt == nk) {
                skt = 0;
                if (++sj < nprod)
                    ps = prod(sj);
            }
        };
        auto fold = [&](char* x, int bytes, bool two, u32 s1, u32 s2) {
            for (int c = tid; c < bytes / 16; c += C::NT) {
                u32x4 v = *reinterpret_cast<const u32x4*>(x + c * 16);
                if (two) {
                    const u32x4 y = *reinterpret_cast<const u32x4*>(x + C::STAGE + c * 16);
#pragma unroll
                    for (int d = 0; d < 4; ++d)
                        v[d] = add_h2<BF>(v[d] ^ s1, y[d] ^ s2);
                } else {
#pragma unroll
                    for (int d = 0; d < 4; ++d)
                        v[d] ^= s1;
                }
                *reinterpret_cast<u32x4*>(x + c * 16) = v;
            }
        };
        int cj = 0, ckt = 0;
        Prod pc = ps;
        auto comb = [&](int, char* stage) {
            if (pc.a2 || pc.sa1)
                fold(stage, C::A_BYTES, pc.a2 != nullptr, pc.sa1, pc.sa2);
            if (pc.b2 || pc.sb1)
                fold(stage + C::A_BYTES, C::B_BYTES, pc.b2 != nullptr, pc.sb1, pc.sb2);
            if (++ckt == nk) {
                ckt = 0;
                if (++cj < nprod)
                    pc = prod(cj);
            }
        };
        int aj = 0, akt = 0;
        auto after = [&](int) {
            if (++akt == nk) {
                akt = 0;
                combine_h<NOUT, C>(fp.w[order_at(item.pos0 + aj)], H, Cacc);
                zero_acc<C>(H);
                ++aj;
            }
        };
        const m16::Addr<C> ad = m16::frag_addr<C>(wm, wn, lane);
        // every term is a block of A or B: one set of grouped-load offsets
        const bool inside = (m0 + C::BM <= fp.Mb) & (n0 + C::BN <= fp.Nb) & (fp.Kb % C::BK == 0);
        if (inside) {
            const tiles::TileSrc st{nullptr, ps.lda, C::BM, nullptr, ps.ldb, C::BN, 0, fp.Kb};
            const q4::Group<C> go = q4::group_offsets<C>(st, wave, lane);
            m16::run_tile_cal<C, BF, true>(smem, ntiles, src, comb, after, wave, lane, ad, go, H);
        } else {
            m16::run_tile_cal<C, BF, false>(smem, ntiles, src, comb, after, wave, lane, ad, q4::Group<C>{}, H);
        }
        __syncthreads();
        fused_epilogue<NOUT, C, BF>(fp, item, m0, n0, Cacc, tid, wm, wn, lane, &sh_old);
        __syncthreads();
    }
}

// One-level fused group kernel on the ping-pong engine (8 waves, 128 x 128
// group tile, 64 x 32 per wave): the product tiles of an item run back to
// back through the DMA ring; after each product's last k-tile every wave folds
// its H sub-tile into its four output sub-tiles.

// Fused one-level group tile: 8 waves of 64 x 32.  A k-tile holds only 8
// MFMAs per wave, so loads run 7 tiles ahead (8-stage ring, 128 KiB) to
// cover the latency of operands that miss L2.
using MCF1 = m16::Cfg<128, 128, 2, 4, 7>;

// Fused one-level group kernel on the 16x16x32 engine: 8 waves (two per
// SIMD) of 64 x 32, each holding four fp32 output sub-tiles plus H (160
// accumulator registers).  The products of a work item stream back to back
// through the same LDS ring (the prefetch runs across product boundaries);
// at each product's last k-tile every wave folds H into its four output
// sub-tiles.
template <bool OBF, bool CBF, bool OUTER>
__global__ void __launch_bounds__(MCF1::NT, 1) k_fused1_m16(const FusedParams fp)
{
    using C = MCF1;
    constexpr int NOUT = 4;
    __shared__ __attribute__((aligned(1024))) char smem[C::LDS];
    __shared__ int sh_old;
    const int tid = threadIdx.x, lane0 = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / C::WN, wn = wave % C::WN;
    const int w = blockIdx.x;
    const int n_items = sched_count(fp.sp, w);
    const int nk = (fp.Kb + C::BK - 1) / C::BK;
    // The 7 order entries as one scalar word: indexing the argument array
    // directly compiles to a vector load, whose wait drains the in-flight
    // tile loads at every product switch.
    uint64_t ordw;
    __builtin_memcpy(&ordw, fp.order, sizeof ordw);
    auto order_at = [&](int pos) { return (int)(int8_t)(ordw >> (8 * pos)); };
    for (int it = 0; it < n_items; ++it) {
        // Opaque per item: keeps lane-derived addresses from being hoisted out
        // of the item loop and held in registers across the whole kernel.
        int lane = lane0;
        asm volatile("" : "+v"(lane));
        const Item item = sched_item(fp.sp, w, it);
        int p, q;
        tile_coords(item.g, fp.sp.gy, fp.sp.gx, fp.sp.P, fp.sp.raster, &p, &q);
        const int m0 = p * C::BM, n0 = q * C::BN;
        f32x4 Cacc[NOUT][C::FM][C::FN];
#pragma unroll
        for (int o = 0; o < NOUT; ++o)
            zero_acc<C>(Cacc[o]);
        f32x4 H[C::FM][C::FN];
        zero_acc<C>(H);
        const int nprod = item.pos1 - item.pos0;
        const int ntiles = nprod * nk;
        // The engine asks for k-tile sources, and reports finished k-tiles, in
        // increasing order, so both walk a cursor; product parameters (kernel
        // argument arrays, read through scalar loads) are fetched only when
        // the product changes.
        auto prod_src = [&](int j) {
            const int r = order_at(item.pos0 + j);
            return tiles::TileSrc{fp.a[r] + (int64_t)m0 * fp.lda[r], (int)fp.lda[r], fp.Mb - m0,
                                  fp.b[r] + n0, (int)fp.ldb[r], fp.Nb - n0, 0, fp.Kb};
        };
        int sj = 0, skt = 0;
        tiles::TileSrc sbase = prod_src(0);
        auto src = [&](int) {
            tiles::TileSrc s = sbase;
            s.k0 = skt * C::BK;
            if (++skt == nk) {
                skt = 0;
                if (++sj < nprod)
                    sbase = prod_src(sj);
            }
            return s;
        };
        int aj = 0, akt = 0;
        auto after = [&](int) {
            if (++akt == nk) {
                akt = 0;
                combine_h<NOUT, C>(fp.w[order_at(item.pos0 + aj)], H, Cacc);
                zero_acc<C>(H);
                ++aj;
            }
        };
        const m16::Addr<C> ad = m16::frag_addr<C>(wm, wn, lane);
        const bool inside = (m0 + C::BM <= fp.Mb) & (n0 + C::BN <= fp.Nb) & (fp.Kb % C::BK == 0);
        // Interior items load through grouped loads; the singleton operands
        // (read in place, with the full matrices' strides) and the combined
        // blocks differ in stride, hence the restriding variant.
        if (inside)
            m16::run_tile<C, OBF, false, true, true>(smem, ntiles, src, after, wave, lane, ad, H);
        else
            m16::run_tile<C, OBF, true, false>(smem, ntiles, src, after, wave, lane, ad, H);
        __syncthreads();
        fused_epilogue<NOUT, C, CBF, OUTER>(fp, item, m0, n0, Cacc, tid, wm, wn, lane, &sh_old);
        __syncthreads();
    }
}

template <bool OBF, bool CBF>
hipError_t launch_fused1_m16(const FusedLaunch& L, hipStream_t st)
{
    if (L.grid <= 0)
        return hipSuccess;
    if (L.outer)
        hipLaunchKernelGGL((k_fused1_m16<OBF, CBF, true>), dim3(L.grid), dim3(MCF1::NT), 0, st, L.p);
    else
        hipLaunchKernelGGL((k_fused1_m16<OBF, CBF, false>), dim3(L.grid), dim3(MCF1::NT), 0, st, L.p);
    return hipGetLastError();
}

template <int LEVELS, bool OBF, bool CBF>
hipError_t launch_fused_t(const FusedLaunch& L, hipStream_t st)
{
    using C = typename FusedCfg<LEVELS>::C;
    if (L.grid <= 0)
        return hipSuccess;
    hipLaunchKernelGGL((k_fused<LEVELS, OBF, CBF>), dim3(L.grid), dim3(C::NT), 0, st, L.p);
    return hipGetLastError();
}

// ------------------------------------------------------------------ padding
//
// Zero-padding of operands to a shape that splits evenly, and the crop of
// the padded product back into C.  Each thread moves 8 consecutive elements
// of one row; rows beyond the grid's y extent are taken in strides.

__global__ void __launch_bounds__(256) k_pad_copy(const u16* __restrict__ src, int64_t lds, int64_t rows,
                                                  int64_t cols, u16* __restrict__ dst, int64_t ldd, int64_t prows,
                                                  int64_t pcols)
{
    const int64_t j0 = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 8;
    if (j0 >= pcols)
        return;
    for (int64_t i = blockIdx.y; i < prows; i += gridDim.y) {
        u16* d = dst + i * ldd;
        const u16* sr = src + i * lds;
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            const int64_t j = j0 + t;
            if (j < pcols)
                d[j] = (i < rows && j < cols) ? sr[j] : (u16)0;
        }
    }
}

// ------------------------------------------------------------------ machine references
//
// Measured ceilings the kernels above are compared against (the published
// peaks are not what the chip holds under load): an MFMA loop and an HBM
// stream copy.

// Random half-precision operands in +-[0.5, 1): random sign and fraction,
// fixed exponent (two values per 32-bit word).
template <bool BF>
__device__ __forceinline__ u32 ref_operand(u32& h)
{
    h ^= h << 13;
    h ^= h >> 17;
    h ^= h << 5;
    return BF ? ((h & 0x807F807Fu) | 0x3F003F00u) : ((h & 0x83FF83FFu) | 0x38003800u);
}

// Eight waves per workgroup, each issuing `iters` rounds of 16 independent
// 16x16x32 MFMAs on operands held in registers; one fp32 sum per thread is
// written so nothing is optimised away.
template <bool BF>
__global__ void __launch_bounds__(512) k_ref_mfma(float* __restrict__ out, int iters)
{
    const u32 gid = blockIdx.x * 512u + threadIdx.x;
    u32 h = gid * 2654435761u + 12345u;
    u32x4 a[4], b[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        a[i] = u32x4{ref_operand<BF>(h), ref_operand<BF>(h), ref_operand<BF>(h), ref_operand<BF>(h)};
        b[i] = u32x4{ref_operand<BF>(h), ref_operand<BF>(h), ref_operand<BF>(h), ref_operand<BF>(h)};
    }
    f32x4 acc[16];
#pragma unroll
    for (int j = 0; j < 16; ++j)
        acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int j = 0; j < 16; ++j)
            acc[j] = mfma<BF>(a[j & 3], b[j >> 2], acc[j]);
    }
    float sum = 0.f;
#pragma unroll
    for (int j = 0; j < 16; ++j)
        sum += acc[j][0] + acc[j][1] + acc[j][2] + acc[j][3];
    out[gid] = sum;
}

// dst = src: each workgroup copies one contiguous chunk of `per` 16-byte
// chunks, four accesses in flight per lane, non-temporal stores (the copy is
// not read back).  Measured faster than grid-stride loops and than torch's
// device copy on MI355X.
__global__ void __launch_bounds__(256) k_ref_copy(const u32x4* __restrict__ src, u32x4* __restrict__ dst, int64_t n,
                                                  int64_t per)
{
    const int64_t b = (int64_t)blockIdx.x * per;
    const int64_t e = b + per < n ? b + per : n;
    for (int64_t i = b + threadIdx.x; i < e; i += 4 * 256) {
        u32x4 v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u)
            if (i + u * 256 < e)
                v[u] = src[i + u * 256];
#pragma unroll
        for (int u = 0; u < 4; ++u)
            if (i + u * 256 < e)
                __builtin_nontemporal_store(v[u], dst + i + u * 256);
    }
}

// Reads src once: each workgroup one contiguous chunk of `per` 16-byte
// chunks, eight loads in flight per lane, folded into one word per lane that
// is stored only when it equals `never` (so the loads stay live and nothing
// is written in practice).
__global__ void __launch_bounds__(256) k_ref_read(const u32x4* __restrict__ src, int64_t n, int64_t per, u32 never,
                                                  u32* __restrict__ out)
{
    const int64_t b = (int64_t)blockIdx.x * per;
    const int64_t e = b + per < n ? b + per : n;
    u32 acc = 0;
    for (int64_t i = b + threadIdx.x; i < e; i += 8 * 256) {
        u32x4 v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u)
            v[u] = i + u * 256 < e ? __builtin_nontemporal_load(src + i + u * 256) : u32x4{0, 0, 0, 0};
#pragma unroll
        for (int u = 0; u < 8; ++u)
            acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    if (acc == never)
        *out = acc;
}

}  // namespace

hipError_t launch_ref_read(const void* src, int64_t chunks, int32_t workgroups, uint32_t never, uint32_t* out,
                           hipStream_t st)
{
    const int64_t per = (chunks + workgroups - 1) / workgroups;
    hipLaunchKernelGGL(k_ref_read, dim3(workgroups), dim3(256), 0, st, (const u32x4*)src, chunks, per, never, out);
    return hipGetLastError();
}

hipError_t launch_ref_mfma(float* out, int32_t workgroups, int32_t iters, int32_t bf16, hipStream_t st)
{
    if (bf16)
        hipLaunchKernelGGL((k_ref_mfma<true>), dim3(workgroups), dim3(512), 0, st, out, iters);
    else
        hipLaunchKernelGGL((k_ref_mfma<false>), dim3(workgroups), dim3(512), 0, st, out, iters);
    return hipGetLastError();
}

hipError_t launch_ref_copy(const void* src, void* dst, int64_t chunks, int32_t workgroups, hipStream_t st)
{
    const int64_t per = (chunks + workgroups - 1) / workgroups;
    hipLaunchKernelGGL(k_ref_copy, dim3(workgroups), dim3(256), 0, st, (const u32x4*)src, (u32x4*)dst, chunks, per);
    return hipGetLastError();
}

hipError_t launch_pad_copy(const void* src, int64_t lds, int64_t rows, int64_t cols, void* dst, int64_t ldd,
                           int64_t prows, int64_t pcols, hipStream_t st)
{
    if (prows <= 0 || pcols <= 0)
        return hipSuccess;
    const dim3 grid((unsigned)((pcols + 2047) / 2048), (unsigned)std::min<int64_t>(prows, 65535));
    hipLaunchKernelGGL(k_pad_copy, grid, dim3(256), 0, st, (const u16*)src, lds, rows, cols, (u16*)dst, ldd, prows,
                       pcols);
    return hipGetLastError();
}

// ------------------------------------------------------------------ host entry points

void classic_tile_dims(int32_t tile, int32_t* bm, int32_t* bn)
{
    switch (tile) {
    case kTile256: *bm = Cfg256::BM; *bn = Cfg256::BN; break;
    case kTile128: *bm = Cfg128::BM; *bn = Cfg128::BN; break;
    default: *bm = Cfg32::BM; *bn = Cfg32::BN; break;
    }
}

hipError_t launch_classic(const ClassicLaunch& L, hipStream_t st)
{
    switch (L.tile) {
    case kTile256:
        if (L.vec && L.split_ws)
            return L.bf16 ? launch_classic_m16_tail_t<MC256, true>(L, st)
                          : launch_classic_m16_tail_t<MC256, false>(L, st);
        if (L.vec)
            return L.bf16 ? launch_classic_m16_t<MC256, true>(L, st) : launch_classic_m16_t<MC256, false>(L, st);
        return launch_classic_c<Cfg256>(L, st);
    case kTile128:
        if (L.vec && L.split_ws)
            return L.bf16 ? launch_classic_m16_split_t<MC128, true>(L, st)
                          : launch_classic_m16_split_t<MC128, false>(L, st);
        if (L.vec && L.K >= kLongK128)
            return L.bf16 ? launch_classic_m16_t<MC128, true>(L, st) : launch_classic_m16_t<MC128, false>(L, st);
        if (L.vec)
            return L.bf16 ? launch_classic_q4_t<QC128, true>(L, st) : launch_classic_q4_t<QC128, false>(L, st);
        return launch_classic_c<Cfg128>(L, st);
    default:
        // with a workspace for the K split (classic plans): 128-column
        // strips, one part of K per workgroup
        if (L.vec && L.M <= 32 && L.split_ws)
            return L.bf16 ? launch_skinny_split_t<sk::CCfg<5, kSplitCols, 32>, true>(L, st)
                          : launch_skinny_split_t<sk::CCfg<5, kSplitCols, 32>, false>(L, st);
        if (L.vec && L.M <= 64 && L.split_ws)
            return L.bf16 ? launch_skinny_split_t<sk::CCfg<5, kSplitCols>, true>(L, st)
                          : launch_skinny_split_t<sk::CCfg<5, kSplitCols>, false>(L, st);
        // M <= 64 with 16-byte aligned operands: the streaming kernels.
        // Up to 32 rows and long K: 64-k stages on two waves.  With more than
        // 128 column strips the waves share one 5-stage ring (1 x 14336 x 4096
        // bf16: 23.1 -> 21.5 us, 16 rows 24.0 -> 22.9 us, 2-7% faster from 160
        // strips up); with fewer strips each compute unit streams more of B and
        // a private 5-stage ring per wave, 4 ahead, keeps more in flight (2-7%
        // faster up to 128 strips).  Short K: 32-k stages on four waves.
        if (L.vec && L.M <= 32 && L.K >= 1024 && (L.N + 63) / 64 > 128)
            return L.bf16 ? launch_skinny_shared_t<sk::CCfg<5, 64, 32>, true>(L, st)
                          : launch_skinny_shared_t<sk::CCfg<5, 64, 32>, false>(L, st);
        if (L.vec && L.M <= 32 && L.K >= 1024)
            return L.bf16 ? launch_skinny_t<sk::SCfg<32, 64, 2, 5>, true>(L, st)
                          : launch_skinny_t<sk::SCfg<32, 64, 2, 5>, false>(L, st);
        if (L.vec && L.M <= 32)
            return L.bf16 ? launch_skinny_t<sk::SCfg<32>, true>(L, st) : launch_skinny_t<sk::SCfg<32>, false>(L, st);
        // 33..64 rows: 64-k stages (A rows of 128 bytes, half the L2 requests
        // per byte of A of 32-k stages) in one 5-stage ring shared by the four
        // waves: measured 28.4 us at 64 x 14336 x 4096 against 29.3 us for a
        // private 4-stage ring per wave on two waves; rings of 3, 6..10 stages
        // and 128-column strips (112 workgroups, 37 us) were slower
        if (L.vec && L.M <= 64)
            return L.bf16 ? launch_skinny_shared_t<sk::CCfg<>, true>(L, st)
                          : launch_skinny_shared_t<sk::CCfg<>, false>(L, st);
        return launch_classic_c<Cfg32>(L, st);
    }
}

hipError_t launch_prepass(const PrepassLaunch& L, hipStream_t st)
{
    const bool all = L.write_all != 0;
    if (L.levels == 1) {
        if (L.in_bf16)
            return L.op_bf16 ? (all ? launch_prepass_t<1, true, true, true>(L, st) : launch_prepass_t<1, true, true, false>(L, st))
                             : launch_prepass_t<1, true, false, true>(L, st);
        return launch_prepass_t<1, false, false, false>(L, st);
    }
    if (L.in_bf16)
        return L.op_bf16 ? (all ? launch_prepass_t<2, true, true, true>(L, st) : launch_prepass_t<2, true, true, false>(L, st))
                         : launch_prepass_t<2, true, false, true>(L, st);
    return launch_prepass_t<2, false, false, false>(L, st);
}

int32_t fused_tile(int32_t levels) { return levels == 1 ? MCF1::BM : FusedCfg<2>::C::BM; }
static_assert(MCF1::BM == MCF1::BN, "fused tiles are square");
static_assert(MCFC::BM == MCF1::BM && MCFC::BN == MCF1::BN,
              "the combine-at-load kernel shares the one-level group geometry");
static_assert(sizeof(FusedParams) <= 4096, "kernel arguments");
static_assert(FusedCfg<2>::C::BM == FusedCfg<2>::C::BN,
              "fused tiles are square");

int64_t fused_partial_bytes(int32_t levels)
{
    if (levels == 1)
        return (int64_t)4 * MCF1::BM * MCF1::BN * 4;
    using C = FusedCfg<2>::C;
    return (int64_t)16 * C::BM * C::BN * 4;
}

void fused_order(int32_t levels, int8_t* order)
{
    // One level: P3, P5, P2, P4, P1, P6, P7 (0-based 2, 4, 1, 3, 0, 5, 6):
    // a split after the first four leaves each piece touching few outputs.
    static const int8_t o1[7] = {2, 4, 1, 3, 0, 5, 6};
    if (levels == 1) {
        for (int i = 0; i < 7; ++i)
            order[i] = o1[i];
        return;
    }
    for (int a = 0; a < 7; ++a)
        for (int b = 0; b < 7; ++b)
            order[a * 7 + b] = (int8_t)(o1[a] * 7 + o1[b]);
}

hipError_t launch_fused(const FusedLaunch& L, hipStream_t st)
{
    if (L.at_load) {
        if (L.levels != 1 || L.outer || L.op_bf16 != L.out_bf16)
            return hipErrorInvalidValue;
        if (L.grid <= 0)
            return hipSuccess;
        if (L.out_bf16)
            hipLaunchKernelGGL((k_fused_cal_m16<true>), dim3(L.grid), dim3(MCFC::NT), 0, st, L.p);
        else
            hipLaunchKernelGGL((k_fused_cal_m16<false>), dim3(L.grid), dim3(MCFC::NT), 0, st, L.p);
        return hipGetLastError();
    }
    if (L.levels == 1 || L.outer) {
        if (L.out_bf16)
            return L.op_bf16 ? launch_fused1_m16<true, true>(L, st) : launch_fused1_m16<false, true>(L, st);
        return launch_fused1_m16<false, false>(L, st);
    }
    if (L.out_bf16)
        return L.op_bf16 ? launch_fused_t<2, true, true>(L, st) : launch_fused_t<2, false, true>(L, st);
    return launch_fused_t<2, false, false>(L, st);
}

hipError_t launch_gen_prepass(const GenPrepassLaunch& L, hipStream_t st)
{
    if (L.in_bf16)
        return L.op_bf16 ? launch_gen_prepass_t<true, true>(L, st) : launch_gen_prepass_t<true, false>(L, st);
    return L.op_bf16 ? launch_gen_prepass_t<false, true>(L, st) : launch_gen_prepass_t<false, false>(L, st);
}

hipError_t launch_gen_group(const GenGroupLaunch& L, hipStream_t st)
{
    if (L.out_bf16)
        return L.op_bf16 ? launch_gen_group_t<true, true>(L, st) : launch_gen_group_t<false, true>(L, st);
    return launch_gen_group_t<false, false>(L, st);
}

// Allocation-free calls: a file-scope device array stands in for the
// caller's workspace.  Each GPU the library runs on holds its own copy until
// the process ends.  In host code `scratch` names a host-side stand-in, not
// device memory, so only the address returned by hipGetSymbolAddress (looked
// up once per device, with that device current) is ever handed to kernels.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

hipError_t scratch_address(void** out)
{
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static void* addr[kMaxDevices] = {};
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return e;
    if (dev < 0 || dev >= kMaxDevices)
        return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess)
            return e;
        if (!p || ((uintptr_t)p % 256) != 0)
            return hipErrorInvalidSymbol;
        addr[dev] = p;
    }
    *out = addr[dev];
    return hipSuccess;
}

hipError_t launch_gen_product(const GenProductLaunch& L, hipStream_t st)
{
    // Products whose 256 x 256 tiles fill the compute units go through the
    // persistent group kernel instead; these use 128 x 128 tiles.
    if (L.out_bf16)
        return L.op_bf16 ? launch_gen_product_t<QC128, true, true>(L, st)
                         : launch_gen_product_t<QC128, false, true>(L, st);
    return launch_gen_product_t<QC128, false, false>(L, st);
}

}  // namespace lcma
