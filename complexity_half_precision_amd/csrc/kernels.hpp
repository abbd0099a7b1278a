// kernels.hpp -- launch interface between the host planner (host.cpp) and the
// gfx950 kernels (kernels.hip).  Internal to the library.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "schedule.hpp"

namespace lcma {

constexpr int kMaxRank = 49;

// Tile shapes of the classic kernel.
enum ClassicTile : int32_t {
    kTile256 = 0,  // 256 x 256 workgroup tile, 8 waves of 128 x 64
    kTile128 = 1,  // 128 x 128: 4 waves of 64 x 64, or 8 waves of 64 x 32 for K >= 2048
    kTile32 = 2    // M <= 64: the streaming kernel (32- or 64-row A, 64-column strips of B)
};

struct ClassicLaunch {
    const void* A; int64_t lda;
    const void* B; int64_t ldb;
    void* C; int64_t ldc;
    int32_t M, N, K;
    int32_t bf16;      // storage type
    int32_t vec;       // 16-byte loads allowed (alignment checked by the caller)
    int32_t vec4;      // 8-byte C stores allowed
    int32_t tile;      // ClassicTile
    int32_t P;         // compute units (for the XCD-aware tile order)
    // M <= 64: K split over split_s (2, 4 or 8) workgroups of each
    // kSplitCols-column strip (split_ws null: no split).  split_ws holds
    // split_ws_bytes(N, split_s, split_rows(M)) bytes (256-byte aligned).
    void* split_ws; int32_t split_s;
};
constexpr int kSplitCols = 128;
inline int split_rows(int64_t M) { return M <= 32 ? 32 : 64; }                 // rows of the tile
inline int64_t split_part_bytes(int rows) { return (int64_t)rows * kSplitCols * 4; }   // one fp32 partial tile
inline int64_t split_strips(int64_t N) { return (N + kSplitCols - 1) / kSplitCols; }
// S partial tiles per strip.
inline int64_t split_ws_bytes(int64_t N, int S, int rows)
{
    return (split_strips(N) * S * split_part_bytes(rows) + 255) / 256 * 256;
}

// Tile edge (rows, cols) of a classic tile shape.
void classic_tile_dims(int32_t tile, int32_t* bm, int32_t* bn);
hipError_t launch_classic(const ClassicLaunch& L, hipStream_t stream);

struct PrepassLaunch {
    const void* A; int64_t lda;
    const void* B; int64_t ldb;
    int32_t Mb, Kb, Nb;         // block sizes
    void* outA; void* outB;     // first combined operand of each side
    int64_t strideA, strideB;   // elements between consecutive combined operands
    int32_t levels;             // 1 or 2
    int32_t in_bf16, op_bf16;   // storage type, combined-operand type
    int32_t write_all;          // also copy single-block operands (operand type differs from storage)
    int32_t* counters; int32_t n_counters;  // split fix-up counters to clear
};
hipError_t launch_prepass(const PrepassLaunch& L, hipStream_t stream);

// Copies the rows x cols window of src (16-bit elements, ld lds) into the
// top-left of the prows x pcols matrix dst (ld ldd) and writes zeros in the
// rest of dst (prows >= rows and pcols >= cols pad; equal sizes crop).
hipError_t launch_pad_copy(const void* src, int64_t lds, int64_t rows, int64_t cols, void* dst, int64_t ldd,
                           int64_t prows, int64_t pcols, hipStream_t stream);

struct FusedParams {
    const uint16_t* a[kMaxRank];   // operand origin (block row 0, col 0) per canonical product
    const uint16_t* b[kMaxRank];
    int64_t lda[kMaxRank];
    int64_t ldb[kMaxRank];
    uint16_t* C; int64_t ldc;
    int32_t Mb, Nb, Kb;
    int32_t vec4;
    SchedParams sp;
    int8_t order[kMaxRank];        // position -> canonical product
    int8_t w[kMaxRank][16];        // W[r][output block] (output blocks row-major)
    float* partial;                // split fix-up partials
    int32_t* counters;             // split fix-up arrival counters
    // Two levels with the outer level in memory: this launch runs the 7 inner
    // products of one outer product r1 over blocks of M/4 x N/4; its inner
    // output (i2, j2) feeds output block (2 i1 + i2, 2 j1 + j2) of every outer
    // output (i1, j1) with omode != kOuterNone, scaled by ow = W1[r1][i1, j1].
    float* acc;                    // fp32 output blocks, 16 of Mb x Nb, block-major (block 4 bi + bj)
    int8_t omode[4];               // OuterMode per outer output (i1, j1), row-major
    float ow[4];
    // Combine at load (one level): a[r] / b[r] are product r's first input
    // block, a2[r] / b2[r] its second (null for a single block, same leading
    // dimension), and sa[r] / sb[r] the sign masks of the two terms
    // (0x80008000 negates both halves of a 32-bit word, 0 keeps them).
    const uint16_t* a2[7];
    const uint16_t* b2[7];
    uint32_t sa[7][2];
    uint32_t sb[7][2];
};

// What one outer product does to an outer output's fp32 blocks: the first
// contributor stores, later ones add, the last adds and rounds into C; an
// output fed by one product only is rounded straight into C.
enum OuterMode : int8_t { kOuterNone = 0, kOuterStore = 1, kOuterAdd = 2, kOuterFinish = 3, kOuterOnly = 4 };

struct FusedLaunch {
    FusedParams p;
    int32_t levels;
    int32_t op_bf16, out_bf16;
    int32_t grid;
    int32_t outer;                 // levels == 2: 1 = one launch of the outer level (one-level kernel + acc)
    int32_t at_load;               // levels == 1: combine the input blocks while staging tiles (no pre-pass)
};
// Workgroup tile edge of the fused kernel for a level (1: 128, 2: 64).
// ---- unfused path for any valid description (one level of it)
constexpr int kGenMaxRank = 64;     // products
constexpr int kGenMaxBlocks = 16;   // blocks per side (ms*ks, ks*ns, ms*ns)

// Combined operands of one side: out_r = sum_b coef[r][b] * X_b (fp32 sum,
// one rounding), for every product r.  Block b of X sits at block row
// b / bcols, block column b % bcols, each rows x cols.
// Tile-packed operand layout (packed = 1; rows a multiple of kPackRows,
// cols of kPackCols; ldo unused): tile row tr and k-tile t form one
// contiguous block of kPackRows x kPackCols elements at element
// (tr * cols + t * kPackCols) * kPackRows; row rr of the block holds its four
// 8-element chunks c at positions c ^ ((rr >> 1) & 3).  That is the A part of
// an LDS stage of the 256 x 256 engine byte for byte, so the persistent
// product kernel reads it with whole-cache-line loads.
constexpr int kPackRows = 256, kPackCols = 32;
struct GenPrepassLaunch {
    const void* X; int64_t ldx;
    int32_t rows, cols, bcols, nblocks, rank;
    int8_t coef[kGenMaxRank * kGenMaxBlocks];
    void* out; int64_t ldo, stride;        // out_r at out + r * stride (elements)
    int32_t in_bf16, op_bf16;
    int32_t packed;                        // 1: write out_r tile-packed (above)
};
hipError_t launch_gen_prepass(const GenPrepassLaunch& L, hipStream_t stream);

// One product H = Ahat * Bhat (M x N x K) whose epilogue folds w[t] * H into
// targets t (each M x N) in place of storing H: the first product feeding an
// output stores its fp32 block, later ones add, the last adds and rounds into
// C, and an output fed once is rounded straight into C.
struct GenProductLaunch {
    const void* A; int64_t lda;
    const void* B; int64_t ldb;
    int32_t M, N, K, op_bf16, P;
    // Targets: fp32 output blocks (ld = ldt) folded with w[t] * H in mode[t]
    // (an OuterMode); the finishing modes round into cdst[t] (ld = ldc) of
    // the storage type (out_bf16).
    float* tgt[kGenMaxBlocks]; float w[kGenMaxBlocks]; int8_t mode[kGenMaxBlocks]; int32_t ntgt; int64_t ldt;
    void* cdst[kGenMaxBlocks]; int64_t ldc; int32_t out_bf16;
};
hipError_t launch_gen_product(const GenProductLaunch& L, hipStream_t stream);

// All products of the unfused path in one persistent launch (256 x 256
// positions, one workgroup per position for every product; same fold modes
// per (product, block)).  Combined operand r: A0 + r * strideA (M x K, ld K),
// B0 + r * strideB (K x N, ld N); fp32 block o at acc + o * M * N (ld N);
// block o of C at row (o / ncols) * M, column (o % ncols) * N.
struct GenGroupLaunch {
    const void* A0; int64_t strideA;       // packed_a = 1: the A operands are tile-packed (GenPrepassLaunch)
    const void* B0; int64_t strideB; int64_t ldb;   // B operands: leading dimension ldb >= N
    int32_t M, N, K, R, op_bf16, out_bf16, P, nout, ncols;
    float* acc;
    void* C; int64_t ldc;
    // Per run j (the products in the order they run): prod[j] is the
    // product, w / mode[j * kGenMaxBlocks + o] its fold into block o, and
    // carry[j] how its accumulators start: 0 = zero, 1 = as the previous
    // run left them, 2 = negated (a chained run continues the partial sum of
    // the one output block it shares with the run before it).
    int8_t w[kGenMaxRank * kGenMaxBlocks];
    int8_t mode[kGenMaxRank * kGenMaxBlocks];
    int8_t prod[kGenMaxRank];
    int8_t carry[kGenMaxRank];
    int32_t packed_a;
};
hipError_t launch_gen_group(const GenGroupLaunch& L, hipStream_t stream);

int32_t fused_tile(int32_t levels);
// Bytes of one split partial (all output blocks of one group, fp32).
int64_t fused_partial_bytes(int32_t levels);
hipError_t launch_fused(const FusedLaunch& L, hipStream_t stream);

// Kernel product order used by the fused kernel (position -> product).
void fused_order(int32_t levels, int8_t* order);

// Machine references: `workgroups` x 8 waves each issuing iters x 16 MFMAs
// (16x16x32, random operands) and writing one float per thread to out; a
// copy of `chunks` 16-byte chunks from src to dst.
hipError_t launch_ref_mfma(float* out, int32_t workgroups, int32_t iters, int32_t bf16, hipStream_t stream);
hipError_t launch_ref_copy(const void* src, void* dst, int64_t chunks, int32_t workgroups, hipStream_t stream);
hipError_t launch_ref_read(const void* src, int64_t chunks, int32_t workgroups, uint32_t never, uint32_t* out,
                           hipStream_t stream);

// Size of the device-resident scratch array of the allocation-free entry
// point (equal to LCMA_SCRATCH_BYTES in lcma.h).
constexpr size_t kScratchBytes = (size_t)64 << 20;
// Device address of the current device's scratch array, looked up once per
// device with that device current and cached.
hipError_t scratch_address(void** out);

}  // namespace lcma
