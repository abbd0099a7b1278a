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
    kTile256 = 0,  // 256 x 256 workgroup tile, 4 waves of 128 x 128
    kTile128 = 1,  // 128 x 128, 4 waves of 64 x 64
    kTile32 = 2    // 32 x 64, 2 waves of 32 x 32 (skinny products)
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
};

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
};

struct FusedLaunch {
    FusedParams p;
    int32_t levels;
    int32_t op_bf16, out_bf16;
    int32_t grid;
};
// Workgroup tile edge of the fused kernel for a level (1: 128, 2: 64).
int32_t fused_tile(int32_t levels);
// Bytes of one split partial (all output blocks of one group, fp32).
int64_t fused_partial_bytes(int32_t levels);
hipError_t launch_fused(const FusedLaunch& L, hipStream_t stream);

// Kernel product order used by the fused kernel (position -> product).
void fused_order(int32_t levels, int8_t* order);

}  // namespace lcma
