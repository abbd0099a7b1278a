// schedule.hpp -- static work schedule of the persistent LCMA kernel, shared
// by the host planner (which exports it for checking) and the device code
// (which evaluates it per worker, so no table travels to the GPU).
//
// Model ("FalconGEMM: Surpassing Hardware Peaks with Lower-Complexity Matrix
// Multiplication", section "从 LCMA 到 FalconGEMM"):
//  * a group is the set of R product tiles that share one output coordinate
//    (p, q); one worker (a workgroup resident on one compute unit)
//    accumulates all of them into the C tiles on chip;
//  * groups are scheduled whole, round after round, over P workers; when the
//    last round is partial, each of its T groups may be split into two
//    pieces (first h products / remaining R-h) on two workers, Stream-K
//    style, the second finisher adding the other's fp32 partial;
//  * pieces are laid out so that the workers of one XCD (the hardware deals
//    workgroups to the 8 XCDs round-robin, and each XCD has its own L2) run
//    the same kind of product at the same time: the two pieces of tail
//    group t go to workers 2t (first half) and 2t+1 (second half), so even
//    XCDs run first halves and odd XCDs second halves.
//  * full rounds map consecutive groups of one XCD to a compact block of
//    output tiles (a grouped raster), so those workers share operand rows
//    and columns in their L2.
#pragma once
#include <stdint.h>

#include "strassen.hpp"

namespace lcma {

enum SplitMode : int32_t { kSplitNone = 0, kSplitTail = 1, kSplitAll = 2 };

struct SchedParams {
    int32_t G;      // groups
    int32_t gy;     // groups along M
    int32_t gx;     // groups along N
    int32_t R;      // products per group
    int32_t P;      // workers (one per compute unit)
    int32_t mode;   // SplitMode actually used
    int32_t h;      // products in the first piece of a split group
    int32_t raster; // rows of tiles per raster band; 0 = plain order (row-major tiles,
                    // split pieces not paired by XCD), the baseline the ordering is measured against
};

struct Item {
    int32_t g;      // group (linear)
    int32_t pos0;   // first product position (in the kernel's product order)
    int32_t pos1;   // one past the last
    int32_t slot;   // split fix-up slot, -1 for a whole group
};

// Number of items of worker w.
LCMA_HD inline int32_t sched_count(const SchedParams& s, int32_t w)
{
    if (s.mode == kSplitTail) {
        const int32_t FR = s.G / s.P, T = s.G % s.P;
        return FR + (w < 2 * T ? 1 : 0);
    }
    if (s.mode == kSplitAll) {
        const int32_t pieces = 2 * s.G;
        return w < pieces ? (pieces - w + s.P - 1) / s.P : 0;
    }
    return w < s.G ? (s.G - w + s.P - 1) / s.P : 0;
}

// Item i of worker w (0 <= i < sched_count(s, w)).
LCMA_HD inline Item sched_item(const SchedParams& s, int32_t w, int32_t i)
{
    Item it;
    if (s.mode == kSplitTail) {
        const int32_t FR = s.G / s.P;
        if (i < FR) {
            it.g = i * s.P + w; it.pos0 = 0; it.pos1 = s.R; it.slot = -1;
        } else {
            const int32_t T = s.G % s.P;
            const int32_t which = s.raster ? (w & 1) : (w >= T), t = s.raster ? (w >> 1) : w - (w >= T) * T;
            it.g = FR * s.P + t;
            it.pos0 = which ? s.h : 0;
            it.pos1 = which ? s.R : s.h;
            it.slot = t;
        }
        return it;
    }
    if (s.mode == kSplitAll) {
        const int32_t piece = w + i * s.P;
        const int32_t which = s.raster ? (piece & 1) : (piece >= s.G), t = s.raster ? (piece >> 1) : piece % s.G;
        it.g = t; it.pos0 = which ? s.h : 0; it.pos1 = which ? s.R : s.h; it.slot = t;
        return it;
    }
    it.g = w + i * s.P; it.pos0 = 0; it.pos1 = s.R; it.slot = -1;
    return it;
}

// Output-tile coordinates of tile / group index g on a gy x gx grid worked
// by P workers.  Within each complete round of P indices the workers of one
// XCD (w % 8) receive consecutive virtual indices; virtual indices then walk
// a raster of bands `raster` tiles tall, column by column inside a band.
// raster = 0 gives the plain row-major order instead.
LCMA_HD inline void tile_coords(int32_t g, int32_t gy, int32_t gx, int32_t P, int32_t raster,
                                int32_t* p, int32_t* q)
{
    const int32_t G = gy * gx;
    if (raster == 0) {
        *p = g / gx;
        *q = g % gx;
        return;
    }
    int32_t v = g;
    if (P % 8 == 0 && P >= 8) {
        const int32_t k = g / P, w = g % P;
        if ((k + 1) * P <= G)
            v = k * P + (w % 8) * (P / 8) + w / 8;
    }
    const int32_t band = raster < gy ? raster : gy;
    const int32_t width = band * gx;
    const int32_t b = v / width, r = v % width;
    const int32_t row0 = b * band;
    const int32_t rows = (gy - row0) < band ? (gy - row0) : band;
    *p = row0 + r % rows;
    *q = r / rows;
}

}  // namespace lcma
