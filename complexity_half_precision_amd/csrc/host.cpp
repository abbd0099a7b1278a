// host.cpp -- C ABI of the library: descriptor checks, the roofline cost
// model, the planner (geometry, persistent schedule, workspace layout) and
// the launch orchestration of the gfx950 kernels.
//
// Sources: "FalconGEMM: Surpassing Hardware Peaks with Lower-Complexity
// Matrix Multiplication" (HyperAI write-up), sections "从 Strassen 出发" (LCMA
// description), "从 LCMA 到 FalconGEMM" (pipeline, groups, split) and
// "从缓存重排到 Cost Model" (a roofline-like model from FLOPs, bytes and the
// target GPU's peak and bandwidth that aims to pick the right algorithm, not
// to predict time); "Kernel 与性能" notes, section "Roofline".
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <new>
#include <vector>

#include "kernels.hpp"
#include "lcma.h"
#include "schedule.hpp"
#include "strassen.hpp"

using namespace lcma;

namespace {

// ---------------------------------------------------------------- descriptors

int8_t g_U1[7 * 4], g_V1[7 * 4], g_W1[7 * 4];
int8_t g_U2[49 * 16], g_V2[49 * 16], g_W2[49 * 16];
std::once_flag g_tables_once;

void init_tables()
{
    for (int r = 0; r < 7; ++r)
        for (int b = 0; b < 4; ++b) {
            g_U1[r * 4 + b] = (int8_t)Scheme<1>::u(r, b / 2, b % 2);
            g_V1[r * 4 + b] = (int8_t)Scheme<1>::v(r, b / 2, b % 2);
            g_W1[r * 4 + b] = (int8_t)Scheme<1>::w(r, b / 2, b % 2);
        }
    for (int r = 0; r < 49; ++r)
        for (int b = 0; b < 16; ++b) {
            g_U2[r * 16 + b] = (int8_t)Scheme<2>::u(r, b / 4, b % 4);
            g_V2[r * 16 + b] = (int8_t)Scheme<2>::v(r, b / 4, b % 4);
            g_W2[r * 16 + b] = (int8_t)Scheme<2>::w(r, b / 4, b % 4);
        }
}

bool desc_shape_ok(const lcma_desc* d)
{
    return d->ms >= 1 && d->ks >= 1 && d->ns >= 1 && d->rank >= 1 && d->ms <= 16 && d->ks <= 16 &&
           d->ns <= 16 && d->rank <= 4096 && d->U && d->V && d->W;
}

// Brent's identity, exact integers: for every (i,k) of A, (k2,j) of B and
// (i2,j2) of C, sum_r U[r][i,k] V[r][k2,j] W[r][i2,j2] = [k==k2][i==i2][j==j2].
bool brent_ok(const lcma_desc* d)
{
    const int ms = d->ms, ks = d->ks, ns = d->ns, R = d->rank;
    for (int x = 0; x < R * ms * ks; ++x)
        if (d->U[x] < -8 || d->U[x] > 8)
            return false;
    for (int x = 0; x < R * ks * ns; ++x)
        if (d->V[x] < -8 || d->V[x] > 8)
            return false;
    for (int x = 0; x < R * ms * ns; ++x)
        if (d->W[x] < -8 || d->W[x] > 8)
            return false;
    for (int i = 0; i < ms; ++i)
        for (int k = 0; k < ks; ++k)
            for (int k2 = 0; k2 < ks; ++k2)
                for (int j = 0; j < ns; ++j)
                    for (int i2 = 0; i2 < ms; ++i2)
                        for (int j2 = 0; j2 < ns; ++j2) {
                            long s = 0;
                            for (int r = 0; r < R; ++r)
                                s += (long)d->U[r * ms * ks + i * ks + k] * d->V[r * ks * ns + k2 * ns + j] *
                                     d->W[r * ms * ns + i2 * ns + j2];
                            if (s != ((k == k2 && i == i2 && j == j2) ? 1 : 0))
                                return false;
                        }
    return true;
}

// 1 / 2 when d is exactly the built-in one- / two-level Strassen scheme, else 0.
int builtin_kind(const lcma_desc* d)
{
    std::call_once(g_tables_once, init_tables);
    if (d->ms == 2 && d->ks == 2 && d->ns == 2 && d->rank == 7 && !memcmp(d->U, g_U1, 28) &&
        !memcmp(d->V, g_V1, 28) && !memcmp(d->W, g_W1, 28))
        return 1;
    if (d->ms == 4 && d->ks == 4 && d->ns == 4 && d->rank == 49 && !memcmp(d->U, g_U2, 784) &&
        !memcmp(d->V, g_V2, 784) && !memcmp(d->W, g_W2, 784))
        return 2;
    return 0;
}

// ---------------------------------------------------------------- device facts

bool log_enabled();

int query_cus(int* out)
{
    static std::mutex mu;
    static int cached[64] = {0};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess || dev < 0 || dev >= 64) {
        if (log_enabled())
            fprintf(stderr, "lcma: hipGetDevice: %s (device %d)\n", hipGetErrorName(e), dev);
        return -1;
    }
    std::lock_guard<std::mutex> lock(mu);
    if (!cached[dev]) {
        int v = 0;
        e = hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess || v <= 0) {
            if (log_enabled())
                fprintf(stderr, "lcma: hipDeviceGetAttribute(CU count): %s (%d)\n", hipGetErrorName(e), v);
            return -1;
        }
        cached[dev] = v;
    }
    *out = cached[dev];
    return 0;
}

bool log_enabled()
{
    static int v = -1;
    if (v < 0) {
        const char* e = getenv("LCMA_LOG");
        v = (e && *e && *e != '0') ? 1 : 0;
    }
    return v == 1;
}

// A HIP call's result as a library status; with LCMA_LOG set, a failure
// prints the HIP error name and the call that returned it.
lcma_status hip_status(hipError_t e, const char* what)
{
    if (e == hipSuccess)
        return LCMA_OK;
    if (log_enabled())
        fprintf(stderr, "lcma: %s: %s (%s)\n", what, hipGetErrorName(e), hipGetErrorString(e));
    return LCMA_E_HIP;
}

// ---------------------------------------------------------------- cost model
//
// t(alg) = sum over its kernels of
//          max( F / (eta_F * peak * q),  B_hbm / (eta_B * bw),  F / (I_tile * bw_L2 * q) )
//          + t_launch
// F: MFMA flops of the kernel; B_hbm: the bytes it must move at least;
// eta_F: the fraction of the MFMA peak the kernel sustains when compute-bound,
// measured per kernel (the classic kernel and the fused kernel at each level
// differ a lot, so one shared factor would misrank them);
// I_tile: flops per byte a workgroup tile draws from L2 (BM*BN/(BM+BN) for a
// BM x BN tile); q: wave-quantisation efficiency = (work units / P) /
// (rounds actually needed).  The first two terms are the roofline of the
// notes page; the L2 term keeps small fused tiles from looking free, and q is
// the tail effect the FalconGEMM write-up measures on coarse groups.

struct Machine {
    double peak, bw, l2bw, launch;
    double eta_mfma, eta_fused1, eta_fused2, eta_cal, eta_bw;
    int P;
};

double quant(double units, int P)
{
    if (units <= 0)
        return 1.0;
    const double rounds = std::ceil(units / P);
    return units / (rounds * P);
}

double kernel_time(double F, double B, double itile, double q, double eta, const Machine& m)
{
    double t = F / (eta * m.peak * q);
    t = std::max(t, B / (m.eta_bw * m.bw));
    if (itile > 0)
        t = std::max(t, F / (itile * m.l2bw * q));
    return t + m.launch;
}

int classic_tile_for(int64_t M, int64_t N, int P)
{
    if (M <= 64)
        return kTile32;
    // Rounds of the compute units each tile size needs.  A round of 128 x 128
    // tiles takes about 0.4 of a round of 256 x 256 tiles (a quarter of the
    // work at a lower rate; measured side by side: 256 x 256 wins by 13-55%
    // with 144-196 tiles of 256 on 256 compute units, 128 x 128 wins by 16%
    // with 128 tiles of 256).
    const int64_t t256 = ((M + 255) / 256) * ((N + 255) / 256);
    const int64_t t128 = ((M + 127) / 128) * ((N + 127) / 128);
    const int64_t r256 = (t256 + P - 1) / P, r128 = (t128 + P - 1) / P;
    return 0.4 * (double)r128 < (double)r256 ? kTile128 : kTile256;
}

double est_classic(int64_t M, int64_t N, int64_t K, const Machine& m)
{
    const double s = 2.0;
    const double F = 2.0 * M * N * K;
    const double B = s * ((double)M * K + (double)K * N + (double)M * N);
    int bm, bn;
    const int tile = classic_tile_for(M, N, m.P);
    classic_tile_dims(tile, &bm, &bn);
    const double tiles = (double)((M + bm - 1) / bm) * ((N + bn - 1) / bn);
    // the 128 x 128 kernel sustains less than the 256 x 256 one (measured
    // 0.34-0.40 of peak against 0.50-0.55)
    const double eta = tile == kTile128 ? m.eta_mfma * 0.7 : m.eta_mfma;
    return kernel_time(F, B, (double)bm * bn / (bm + bn), quant(tiles, m.P), eta, m);
}

// Geometry of an LCMA plan at `levels`.
struct Geo {
    int64_t Mb, Nb, Kb;
    int tile, gy, gx, G, R, S;
};

Geo lcma_geo(int64_t M, int64_t N, int64_t K, int levels)
{
    Geo g;
    g.S = levels == 1 ? 2 : 4;
    g.R = levels == 1 ? 7 : 49;
    g.Mb = M / g.S; g.Nb = N / g.S; g.Kb = K / g.S;
    g.tile = fused_tile(levels);
    g.gy = (int)((g.Mb + g.tile - 1) / g.tile);
    g.gx = (int)((g.Nb + g.tile - 1) / g.tile);
    g.G = g.gy * g.gx;
    return g;
}

int split_mode_for(lcma_split req, int G, int P)
{
    if (req == LCMA_SPLIT_NONE)
        return kSplitNone;
    if (req == LCMA_SPLIT_ALL)
        return kSplitAll;
    const int T = G % P;
    return (T > 0 && 2 * T <= P) ? kSplitTail : kSplitNone;
}

// Number of combined operands the pre-pass writes per side.
void written_counts(int levels, bool write_all, int* nA, int* nB)
{
    std::call_once(g_tables_once, init_tables);
    const int R = levels == 1 ? 7 : 49, SS = levels == 1 ? 4 : 16;
    const int8_t* U = levels == 1 ? g_U1 : g_U2;
    const int8_t* V = levels == 1 ? g_V1 : g_V2;
    *nA = *nB = 0;
    for (int r = 0; r < R; ++r) {
        int a = 0, b = 0;
        for (int x = 0; x < SS; ++x) {
            a += U[r * SS + x] != 0;
            b += V[r * SS + x] != 0;
        }
        *nA += (write_all || a > 1);
        *nB += (write_all || b > 1);
    }
}

// Tiles of the group kernel that runs a plan's products: the one-level
// kernel's (128) for one level and for two levels with the outer level in
// memory (7 launches over the M/4 x N/4 blocks), the on-chip two-level
// kernel's (64) otherwise.
Geo sched_geo(const Geo& g, bool outer)
{
    Geo s = g;
    if (outer) {
        s.tile = fused_tile(1);
        s.R = 7;
        s.gy = (int)((g.Mb + s.tile - 1) / s.tile);
        s.gx = (int)((g.Nb + s.tile - 1) / s.tile);
        s.G = s.gy * s.gx;
    }
    return s;
}

double est_lcma(int64_t M, int64_t N, int64_t K, int levels, int split_req, bool write_all, bool outer,
                const Machine& m, bool at_load = false)
{
    const double s = 2.0;
    const Geo g = lcma_geo(M, N, K, levels);
    const Geo sg = sched_geo(g, levels == 2 && outer);
    int nA, nB;
    written_counts(levels, write_all, &nA, &nB);
    // pre-pass: read A and B once, write the combined operands
    const double Bpre = s * ((double)M * K + (double)K * N) +
                        s * (nA * (double)g.Mb * g.Kb + nB * (double)g.Kb * g.Nb);
    const double t_pre = at_load ? 0.0 : Bpre / (m.eta_bw * m.bw) + m.launch;
    // fused: R products of Mb x Nb x Kb; combining at load reads every
    // nonzero block of U and V instead of one operand per product
    const double F = 2.0 * g.R * (double)g.Mb * g.Nb * g.Kb;
    double rdA = g.R, rdB = g.R;
    if (at_load) {
        rdA = rdB = 0;
        for (int x = 0; x < 7 * 4; ++x) {
            rdA += g_U1[x] != 0;
            rdB += g_V1[x] != 0;
        }
    }
    double Bf = s * (rdA * (double)g.Mb * g.Kb + rdB * (double)g.Kb * g.Nb) + s * (double)M * N;
    const bool out2 = levels == 2 && outer;
    // Outer level in memory: per element of the four M/2 x N/2 outer
    // outputs, 4 bytes stored by the first contributor, 8 read and written by
    // each middle one, 4 read by the last (which writes C): 8c - 6 bytes for
    // c contributors (4, 2, 2, 4 for Strassen), 18 MN bytes in all.
    if (out2)
        Bf += 18.0 * (double)M * N - s * (double)M * N;
    const int mode = split_mode_for((lcma_split)split_req, sg.G, m.P);
    double q;
    if (mode == kSplitTail) {
        const double rounds = (double)(sg.G / m.P) + 0.5;
        q = ((double)sg.G / m.P) / rounds;
    } else {
        q = quant(sg.G, m.P);
    }
    const double eta = at_load ? m.eta_cal : (levels == 1 || out2) ? m.eta_fused1 : m.eta_fused2;
    const double t_f = kernel_time(F, Bf, sg.tile / 2.0, q, eta, m) + (out2 ? 6 * m.launch : 0.0);
    return t_pre + t_f;
}

}  // namespace

// ---------------------------------------------------------------- plan

// Run order of the persistent unfused kernel: run j computes product prod[j]
// starting from zero accumulators (carry 0), from the previous run's
// accumulators (1) or from their negation (2), then folds w[j][o] times its
// accumulators into output block o.
struct RunSchedule {
    int8_t prod[kGenMaxRank];
    int8_t carry[kGenMaxRank];
    int8_t w[kGenMaxRank][kGenMaxBlocks];
    int searched;          // 1: the exhaustive search below found it
};

struct lcma_plan_s {
    int64_t M, N, K;
    lcma_dtype dt;
    lcma_algo chosen;
    int levels;            // 0 = classic
    int op_bf16;           // combined-operand type (LCMA)
    int write_all;         // pre-pass copies single-block operands too
    int classic_tile;
    int split_s;           // classic: workgroups per strip of the K-split kernel (0: none), split_pieces()
    int P;
    Geo geo;
    SchedParams sp;
    int grid;
    int8_t order[kMaxRank];
    int n_slots;
    int64_t offA, offB, offPart, offCtr;
    int outer;             // two levels: inner level fused, outer level accumulated in fp32 memory
    int at_load;           // one level: the group kernel combines the input blocks itself (no pre-pass)
    int8_t order1[7];      // outer level: order of the 7 launches (outer products)
    int64_t offAcc;        // outer level: fp32 output blocks
    int64_t slotA[kMaxRank], slotB[kMaxRank];   // index among written operands, -1 = in place
    int blockA[kMaxRank], blockB[kMaxRank];     // block index of an in-place operand
    size_t ws_bytes;
    double est[4];
    // unfused path (one level of any valid description)
    int unfused;
    int gms, gks, gns, gR;
    int64_t gMb, gKb, gNb;
    int8_t gU[kGenMaxRank * kGenMaxBlocks], gV[kGenMaxRank * kGenMaxBlocks], gW[kGenMaxRank * kGenMaxBlocks];
    int64_t offGA, offGB, offGC;
    int gGroup;            // all products in one persistent launch (enough 256 x 256 positions)
    int gPackA;            // ... with the combined A operands tile-packed (whole 256 x 256 tiles)
    int64_t gLdB;          // leading dimension of the written B operands (Nb, padded in one launch)
    RunSchedule gRuns;     // ... its run order, carries and folds
    // padded plan: a forced LCMA on a shape that does not split evenly runs
    // `inner` on zero-padded Mp x Kp and Kp x Np copies of A and B in the
    // workspace and crops its Mp x Np product into C
    lcma_plan_s* inner = nullptr;
    int64_t Mp, Np, Kp;
    int64_t offPA, offPB, offPC, offIn;
};

static int64_t align_up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }

// The integer a caller passed for an enum argument.  C callers may pass any
// int; reading an out-of-range value through the enum type is undefined in
// C++, so entry points validate the bytes before using the enum.
template <class E>
static int32_t enum_bits(const E* e)
{
    static_assert(sizeof(E) == sizeof(int32_t), "enums of the ABI are 32-bit");
    int32_t v;
    memcpy(&v, e, sizeof v);
    return v;
}

// Kernels address rows through 32-bit buffer offsets re-based at every
// k-tile: a tile spans at most 256 rows of a leading dimension below 2^21.
static constexpr int64_t kMaxLd = (int64_t)1 << 21;

// Wraps `in`, planned for the Mp x Np x Kp product, into a plan for M x N x K
// that copies A and B into zero-padded buffers in the workspace, runs `in`
// there and crops its product into C.  extra_s: estimated seconds of the
// copies.  Takes ownership of `in`.
static lcma_status wrap_padded(lcma_plan_s* in, int64_t M, int64_t N, int64_t K, lcma_dtype dt, lcma_algo chosen,
                               int64_t Mp, int64_t Np, int64_t Kp, const double* est, double extra_s,
                               lcma_plan_s** out)
{
    lcma_plan_s* p = new (std::nothrow) lcma_plan_s();
    if (!p) {
        lcma_plan_destroy(in);
        return LCMA_E_NOMEM;
    }
    p->M = M; p->N = N; p->K = K; p->dt = dt; p->chosen = chosen; p->P = in->P;
    p->levels = in->levels; p->unfused = in->unfused; p->geo = in->geo; p->classic_tile = in->classic_tile;
    p->inner = in;
    p->Mp = Mp; p->Np = Np; p->Kp = Kp;
    p->offPA = 0;
    p->offPB = align_up(p->offPA + Mp * Kp * 2, 256);
    p->offPC = align_up(p->offPB + Kp * Np * 2, 256);
    p->offIn = align_up(p->offPC + Mp * Np * 2, 256);
    p->ws_bytes = (size_t)(p->offIn + (int64_t)in->ws_bytes);
    for (int a = 0; a < 4; ++a)
        p->est[a] = est[a];
    p->est[chosen] = in->est[chosen] + extra_s;
    *out = p;
    return LCMA_OK;
}

extern "C" {

const char* lcma_status_str(lcma_status s)
{
    switch (enum_bits(&s)) {
    case LCMA_OK: return "ok";
    case LCMA_E_INVALID: return "invalid argument";
    case LCMA_E_UNSUPPORTED: return "unsupported shape, alignment or algorithm";
    case LCMA_E_BAD_DESCRIPTOR: return "descriptor fails Brent's identity or is malformed";
    case LCMA_E_WORKSPACE: return "workspace missing, misaligned or too small";
    case LCMA_E_HIP: return "HIP runtime error";
    case LCMA_E_NOMEM: return "out of host memory";
    }
    return "unknown status";
}

lcma_status lcma_desc_builtin(int32_t levels, lcma_desc* out)
{
    if (!out || (levels != 1 && levels != 2))
        return LCMA_E_INVALID;
    std::call_once(g_tables_once, init_tables);
    if (levels == 1)
        *out = lcma_desc{2, 2, 2, 7, g_U1, g_V1, g_W1};
    else
        *out = lcma_desc{4, 4, 4, 49, g_U2, g_V2, g_W2};
    return LCMA_OK;
}

lcma_status lcma_desc_winograd(lcma_desc* out)
{
    if (!out)
        return LCMA_E_INVALID;
    static_assert(sizeof kUw == 28 && sizeof kVw == 28 && sizeof kWw == 28, "rank-7 tables of 2x2 blocks");
    *out = lcma_desc{2, 2, 2, 7, &kUw[0][0], &kVw[0][0], &kWw[0][0]};
    return LCMA_OK;
}

lcma_status lcma_desc_validate(const lcma_desc* d)
{
    if (!d)
        return LCMA_E_INVALID;
    if (!desc_shape_ok(d) || !brent_ok(d))
        return LCMA_E_BAD_DESCRIPTOR;
    return LCMA_OK;
}

namespace {

// Workgroups per 128-column strip of the K-split kernel for classic plans of
// up to 64 rows, 0 for none.  Measured on MI355X (bfloat16; 1, 8, 32 and 64
// rows; 18 shapes each; S in 0, 2, 4, 8): the split pays where few strips
// would leave most compute units idle over a long K, and with many strips
// only for 17 rows and more over a long K, where it halves the A bytes each
// workgroup re-reads.  It costs a second launch and a partial tile per
// piece (1 x 1024 x 14336: 58.5 us unsplit, 18.9 with S = 8; 1 x 4096 x
// 14336: 59.1 unsplit, 26.0 with S = 8; 64 x 14336 x 14336: 93.4 unsplit,
// 81.5 with S = 2; 1 x 14336 x 4096: 21.5 unsplit, 24.5 with S = 2).
int split_pieces(int64_t M, int64_t N, int64_t K)
{
    if (M < 1 || M > 64)
        return 0;
    const int64_t strips = split_strips(N);
    if (strips <= 8)
        return K >= 2048 ? 8 : 0;
    if (strips <= 16)
        return K >= 4096 ? 8 : K >= 2048 ? (M > 32 ? 4 : 8) : 0;
    if (strips <= 32)
        return K >= 4096 ? 8 : K >= 2048 ? 4 : 0;
    if (strips <= 64)
        return K >= 4096 ? 4 : 0;
    if (M > 32)
        return K >= 8192 || (strips > 128 && K >= 4096) ? 2 : 0;
    return M > 16 && K >= 12288 ? 2 : 0;
}

// Pieces of K for the classic kernel beyond 64 rows (128 x 128 tiles): when
// its tiles fill at most half the compute units and K is long, S pieces of K
// per tile write fp32 planes that a second launch adds; S is the largest of
// 2, 4, 8 that keeps tiles x S within the compute units and 768 of K per
// piece.  0 for none.  Measured on MI355X (bfloat16, S in 0, 2, 4, 8): on
// the 26 shapes with K >= 4096 the rule picks the fastest S (4096 x 256 x
// 8192: 52.9 us unsplit, 26.9 with S = 4; 256 x 8192 x 14336: 169.6, 105.2
// with S = 2; 256 x 256 x 16384: 103.6, 22.4 with S = 8; 1024 x 512 x 6144:
// 49.8, 20.8 with S = 8; 2048 x 2048 x 8192, 256 tiles: 63.9 unsplit, 75.8
// with S = 2).  K = 2048 stays unsplit: the split gained up to 11% at
// 1024 x 1024 x 2048 and lost at 4096 x 256 x 2048.
int classic_split_pieces(int64_t M, int64_t N, int64_t K, int P)
{
    if (M <= 64 || N % 8 != 0 || K % 8 != 0)
        return 0;
    const int64_t tiles = ((M + 127) / 128) * ((N + 127) / 128);
    int S = 1;
    if (K < 4096)
        return 0;
    while (S < 8 && tiles * S * 2 <= P && K / (S * 2) >= 768)
        S *= 2;
    return S > 1 ? S : 0;
}

// Pieces of K for the last, partial round of a multi-round classic grid on
// 256 x 256 tiles: its T tiles run as S pieces of K each (T S workgroups
// within one round, at least 1024 of K per piece), writing compact fp32
// partial tiles that a third launch adds.  0 for none.  Measured on MI355X
// (bfloat16, S in 0, 2, 4, 8): the tail round runs faster than a full one,
// so the split pays with one full round before it (3328 x 5120 x 8192,
// T = 4: 324.6 us unsplit, 239.0 with S = 8; 4104^3, T = 33: 187.4, 162.3
// with S = 4), with a small tail (7168^3, T = 16: 614.7, 554.8), or with
// long K (6144 x 6144 x 12288, T = 64: 769.4, 706.0); not with T = 64 after
// six rounds at K = 4096 (10240 x 10240 x 4096: 658.5, 662.6).
int tail_split_pieces(int64_t M, int64_t N, int64_t K, int P)
{
    if (M <= 64 || N % 8 != 0 || K % 8 != 0 || K < 4096)
        return 0;
    const int64_t tiles = ((M + 255) / 256) * ((N + 255) / 256), R = tiles / P, T = tiles % P;
    if (R == 0 || T == 0 || T > 64 || (R > 1 && T > 32 && K < 8192))
        return 0;
    int S = 1;
    while (S < 8 && T * S * 2 <= P && K / (S * 2) >= 1024)
        S *= 2;
    return S > 1 ? S : 0;
}

// Padding of the written B operands' rows in one persistent unfused launch
// (elements): 8192-element rows (16 KB) at a 16 KB + 128 B pitch.  Measured
// at 32768^3 bfloat16: 48.10 -> 46.83 ms (Winograd), 48.37 -> 47.69 ms
// (Strassen); within noise at 8192^3 and 16384^3 (64, 128 and 256 alike).
constexpr int64_t kGenBPad = 64;

// fp32 bytes that the folds of an output block move per element when k runs
// feed it: one run rounds straight into C (2 bytes written); otherwise the
// first stores (4), each middle one reads and writes (8), and the last reads
// and writes C (4 + 2).
int fold_bytes(int k) { return k == 0 ? 0 : k == 1 ? 2 : 8 * k - 6; }

int schedule_fold_bytes(const RunSchedule& s, int R, int nout)
{
    int b = 0;
    for (int o = 0; o < nout; ++o) {
        int k = 0;
        for (int j = 0; j < R; ++j)
            k += s.w[j][o] != 0;
        b += fold_bytes(k);
    }
    return b;
}

// Pairing rule (any description): a product that feeds a single output block
// o with coefficient +-1 runs right after a product that also feeds o with
// coefficient +-1 and continues its accumulators: the first run folds its
// other blocks from the accumulators (which then hold its product alone) and
// carries o; the second starts from them (negated when the two coefficients
// differ in sign) and folds the sum, so o takes one fp32 round trip less.
// The remaining products follow in their own order.
void pair_schedule(const int8_t* W, int R, int nout, RunSchedule* s)
{
    auto w = [&](int r, int o) { return (int)W[r * kGenMaxBlocks + o]; };
    auto single = [&](int r, int* o_out) {
        int n = 0, o1 = -1;
        for (int o = 0; o < nout; ++o)
            if (w(r, o) != 0) {
                ++n;
                o1 = o;
            }
        *o_out = o1;
        return n == 1 && (w(r, o1) == 1 || w(r, o1) == -1);
    };
    bool used[kGenMaxRank] = {};
    int seq[kGenMaxRank], carried[kGenMaxRank], n = 0;   // carried: block a run hands to the next, or -1
    for (int q = 0; q < R; ++q) {
        int o;
        if (used[q] || !single(q, &o))
            continue;
        for (int r = 0; r < R; ++r) {
            if (r == q || used[r] || (w(r, o) != 1 && w(r, o) != -1))
                continue;
            used[r] = used[q] = true;
            seq[n] = r; carried[n] = o; ++n;
            seq[n] = q; carried[n] = -1; ++n;
            break;
        }
    }
    for (int r = 0; r < R; ++r)
        if (!used[r]) {
            seq[n] = r; carried[n] = -1; ++n;
        }
    // the head of a chain does not fold the carried block; the tail folds it
    // with its own coefficient (its accumulators hold that sign times the sum)
    memset(s, 0, sizeof *s);
    for (int j = 0; j < R; ++j) {
        const int r = seq[j];
        const bool tail = j > 0 && carried[j - 1] >= 0;
        s->prod[j] = (int8_t)r;
        s->carry[j] = (int8_t)(!tail ? 0 : (w(r, carried[j - 1]) == w(seq[j - 1], carried[j - 1]) ? 1 : 2));
        for (int o = 0; o < nout; ++o)
            s->w[j][o] = (int8_t)(o == carried[j] ? 0 : w(r, o));
    }
}

// Exhaustive search over run orders and carries (descriptions of up to 7
// products).  After run j the accumulators hold a signed sum of products,
// its snapshot; output block o must be the sum of some snapshots, each taken
// with coefficient +-1, equal to its column of W.  The search keeps the
// schedule whose folds move the fewest fp32 bytes (fold_bytes per block,
// each block written with at most three snapshots).  Chains (maximal runs
// that continue their accumulators) commute, so they are enumerated in the
// order of their first products: about 10^6 candidates at rank 7, 0.2 s.
// A vector over the products is coded as sum_r x_r 7^r.  Snapshots have
// entries in -1..1 and W's columns (checked) in -3..3, so a column minus two
// signed snapshots, compared with a third, differs from it by entries of
// magnitude at most 6: two codes are equal only if the vectors are (base 7).
class RunSearch {
public:
    static constexpr int kMaxRank = 7;

    bool run(const int8_t* W, int R, int nout, RunSchedule* out)
    {
        if (R < 1 || R > kMaxRank || nout < 1 || nout > kGenMaxBlocks)
            return false;
        R_ = R;
        nout_ = nout;
        int p7 = 1;
        for (int r = 0; r < R; ++r) {
            pw_[r] = p7;
            p7 *= 7;
        }
        half_ = p7 / 2;
        for (int o = 0; o < nout; ++o) {
            int t = 0;
            for (int r = 0; r < R; ++r) {
                const int x = W[r * kGenMaxBlocks + o];
                if (x < -3 || x > 3)
                    return false;
                t += x * pw_[r];
            }
            if (t == 0)
                return false;
            tgt_[o] = t;
        }
        map_.assign((size_t)p7, 0);
        best_ = 1 << 30;
        dfs(0, 0, -1, 0);
        if (best_ == 1 << 30)
            return false;
        *out = best_s_;
        out->searched = 1;
        return true;
    }

private:
    int R_ = 0, nout_ = 0, half_ = 0, best_ = 0;
    int pw_[kMaxRank], tgt_[kGenMaxBlocks];
    int seq_[kMaxRank], car_[kMaxRank], snap_[kMaxRank];
    std::vector<int8_t> map_;   // code + half -> +-(1 + run of that snapshot), 0 if none
    RunSchedule best_s_;

    int find(int code) const { return code < -half_ || code > half_ ? 0 : map_[(size_t)(code + half_)]; }

    // fewest snapshots (at most kmax) that write block o; 0 if none
    int rep(int o, int kmax, int* idx, int* coef) const
    {
        const int t = tgt_[o];
        const int e = find(t);
        if (e != 0) {
            idx[0] = std::abs(e) - 1;
            coef[0] = e > 0 ? 1 : -1;
            return 1;
        }
        if (kmax < 2)
            return 0;
        for (int i = 0; i < R_; ++i)
            for (int si = -1; si <= 1; si += 2) {
                const int f = find(t - si * snap_[i]);
                if (f != 0 && std::abs(f) - 1 != i) {
                    idx[0] = i; coef[0] = si;
                    idx[1] = std::abs(f) - 1; coef[1] = f > 0 ? 1 : -1;
                    return 2;
                }
            }
        if (kmax < 3)
            return 0;
        for (int i = 0; i < R_; ++i)
            for (int j = i + 1; j < R_; ++j)
                for (int si = -1; si <= 1; si += 2)
                    for (int sj = -1; sj <= 1; sj += 2) {
                        const int f = find(t - si * snap_[i] - sj * snap_[j]);
                        const int l = std::abs(f) - 1;
                        if (f != 0 && l != i && l != j) {
                            idx[0] = i; coef[0] = si;
                            idx[1] = j; coef[1] = sj;
                            idx[2] = l; coef[2] = f > 0 ? 1 : -1;
                            return 3;
                        }
                    }
        return 0;
    }

    void evaluate()
    {
        for (int j = 0; j < R_; ++j) {
            map_[(size_t)(snap_[j] + half_)] = (int8_t)(1 + j);
            map_[(size_t)(-snap_[j] + half_)] = (int8_t)(-(1 + j));
        }
        int cost = 0, ks[kGenMaxBlocks], idx[kGenMaxBlocks][3], coef[kGenMaxBlocks][3];
        bool ok = true;
        for (int o = 0; o < nout_ && ok; ++o) {
            // the most this block may cost with the schedule still beating the best
            const int room = best_ - 1 - cost - 2 * (nout_ - 1 - o);
            const int kmax = room >= fold_bytes(3) ? 3 : room >= fold_bytes(2) ? 2 : room >= fold_bytes(1) ? 1 : 0;
            ks[o] = kmax > 0 ? rep(o, kmax, idx[o], coef[o]) : 0;
            ok = ks[o] > 0;
            cost += ok ? fold_bytes(ks[o]) : 0;
        }
        for (int j = 0; j < R_; ++j) {
            map_[(size_t)(snap_[j] + half_)] = 0;
            map_[(size_t)(-snap_[j] + half_)] = 0;
        }
        if (!ok)
            return;
        best_ = cost;
        memset(&best_s_, 0, sizeof best_s_);
        for (int j = 0; j < R_; ++j) {
            best_s_.prod[j] = (int8_t)seq_[j];
            best_s_.carry[j] = (int8_t)car_[j];
        }
        for (int o = 0; o < nout_; ++o)
            for (int q = 0; q < ks[o]; ++q)
                best_s_.w[idx[o][q]][o] = (int8_t)coef[o][q];
    }

    void dfs(int j, int used, int head, int acc)
    {
        if (j == R_) {
            evaluate();
            return;
        }
        for (int p = 0; p < R_; ++p) {
            if (used >> p & 1)
                continue;
            for (int c = 0; c < (j == 0 ? 1 : 3); ++c) {
                if (c == 0 && p < head)
                    continue;       // chains in the order of their first products
                const int v = (c == 0 ? 0 : c == 1 ? acc : -acc) + pw_[p];
                seq_[j] = p;
                car_[j] = c;
                snap_[j] = v;
                dfs(j + 1, used | 1 << p, c == 0 ? p : head, v);
            }
        }
    }
};

// The schedule of a description: the searched one when the search applies
// and moves fewer bytes than the pairing rule, else the pairing rule.
// Searches are cached per table (a plan is made once per shape).
void plan_runs(const int8_t* W, int R, int nout, RunSchedule* s)
{
    pair_schedule(W, R, nout, s);
    if (R > RunSearch::kMaxRank)
        return;
    struct Entry {
        int R, nout;
        int8_t W[kGenMaxRank * kGenMaxBlocks];
        RunSchedule s;
        bool found;
    };
    static std::mutex mu;
    static std::vector<Entry> cache;
    std::lock_guard<std::mutex> lock(mu);
    for (const Entry& e : cache)
        if (e.R == R && e.nout == nout && memcmp(e.W, W, sizeof e.W) == 0) {
            if (e.found)
                *s = e.s;
            return;
        }
    Entry e;
    e.R = R;
    e.nout = nout;
    memcpy(e.W, W, sizeof e.W);
    RunSearch search;
    e.found = search.run(W, R, nout, &e.s) &&
              schedule_fold_bytes(e.s, R, nout) < schedule_fold_bytes(*s, R, nout);
    if (cache.size() < 16)
        cache.push_back(e);
    if (e.found)
        *s = e.s;
}

}  // namespace

lcma_status lcma_plan_ex(int64_t M, int64_t N, int64_t K, lcma_dtype dt, const lcma_desc* desc,
                         lcma_algo force, const lcma_options* opts, lcma_plan_t* out)
{
    if (!out)
        return LCMA_E_INVALID;
    *out = nullptr;
    if (M < 0 || N < 0 || K < 0 || M > INT32_MAX || N > INT32_MAX || K > INT32_MAX)
        return LCMA_E_INVALID;
    if (enum_bits(&dt) != LCMA_F16 && enum_bits(&dt) != LCMA_BF16)
        return LCMA_E_INVALID;
    if (enum_bits(&force) < LCMA_ALGO_AUTO || enum_bits(&force) > LCMA_ALGO_L2)
        return LCMA_E_INVALID;
    // lda >= K and ldb, ldc >= N: no call of such a plan could pass the
    // leading-dimension limit of the kernels
    if (M > 0 && N > 0 && K > 0 && (K >= kMaxLd || N >= kMaxLd))
        return LCMA_E_UNSUPPORTED;
    lcma_options o{};
    if (opts)
        o = *opts;
    if (enum_bits(&o.split) < LCMA_SPLIT_AUTO || enum_bits(&o.split) > LCMA_SPLIT_ALL ||
        enum_bits(&o.order) < LCMA_ORDER_AUTO || enum_bits(&o.order) > LCMA_ORDER_PLAIN ||
        enum_bits(&o.combine) < LCMA_COMBINE_AUTO || enum_bits(&o.combine) > LCMA_COMBINE_L2_ON_CHIP || o.num_cus < 0 || o.peak_tflops < 0 || o.hbm_gbps < 0 ||
        o.bf16_ops_f16 < -1 || o.bf16_ops_f16 > 1 || !(o.classic_eff >= 0 && o.classic_eff <= 1) ||
        !(o.fused_eff >= 0 && o.fused_eff <= 1) || o.accuracy_optin < 0 || o.accuracy_optin > 1)
        return LCMA_E_INVALID;

    // Which LCMA levels the description allows.  A description that is not
    // a built-in scheme runs one level of itself through the unfused path.
    bool allow_l1 = true, allow_l2 = true;
    lcma_desc gen{};
    std::call_once(g_tables_once, init_tables);
    if (desc) {
        if (!desc_shape_ok(desc) || !brent_ok(desc))
            return LCMA_E_BAD_DESCRIPTOR;
        const int kind = builtin_kind(desc);
        allow_l2 = kind == 1 || kind == 2;
        if (kind == 1) {
            gen = lcma_desc{2, 2, 2, 7, g_U1, g_V1, g_W1};
        } else if (kind == 0) {
            gen = *desc;
            allow_l1 = desc->rank <= kGenMaxRank && desc->ms * desc->ks <= kGenMaxBlocks &&
                       desc->ks * desc->ns <= kGenMaxBlocks && desc->ms * desc->ns <= kGenMaxBlocks;
        } else {
            allow_l1 = false;   // a two-level table: run it as L2 of the one-level scheme
        }
    } else {
        gen = lcma_desc{2, 2, 2, 7, g_U1, g_V1, g_W1};
    }
    const bool generic = desc && builtin_kind(desc) == 0;
    const bool unfused = generic || o.combine == LCMA_COMBINE_UNFUSED;
    // Combining at load: one level of the built-in scheme, operands of the
    // storage type.
    const bool at_load = o.combine == LCMA_COMBINE_AT_LOAD;
    if (at_load && (generic || force == LCMA_ALGO_L2 || (dt == LCMA_BF16 && o.bf16_ops_f16 == 1)))
        return LCMA_E_UNSUPPORTED;
    // Two levels: the outer level goes through memory unless all 49 products
    // are to accumulate on chip.
    const bool outer2 = o.combine != LCMA_COMBINE_L2_ON_CHIP;
    if (generic && force == LCMA_ALGO_L2)
        return LCMA_E_UNSUPPORTED;

    Machine m;
    m.peak = (o.peak_tflops > 0 ? o.peak_tflops : 2500.0) * 1e12;
    m.bw = (o.hbm_gbps > 0 ? o.hbm_gbps : 8000.0) * 1e9;
    m.l2bw = 8.0 * 2048.0 * 2.4e9;
    m.launch = 4e-6;
    // Sustained fractions of the MFMA peak measured on MI355X (256 CUs) for
    // the kernels as they stand: classic 256x256 tiles 0.50-0.55 over
    // 4096^3..16384^3; fused one-level group kernel about 0.31 (also the
    // inner level of the default two-level path); the on-chip two-level
    // kernel about 0.037; the combine-at-load group kernel about 0.13.
    m.eta_mfma = o.classic_eff > 0 ? o.classic_eff : 0.52;
    m.eta_fused1 = o.fused_eff > 0 ? o.fused_eff : 0.31;
    m.eta_fused2 = o.fused_eff > 0 ? o.fused_eff : 0.037;
    m.eta_cal = o.fused_eff > 0 ? o.fused_eff : 0.13;
    m.eta_bw = 0.8;
    if (o.num_cus > 0) {
        m.P = o.num_cus;
    } else if (query_cus(&m.P) != 0) {
        return LCMA_E_HIP;
    }

    // Operand type of the combined operands (bfloat16 inputs may use binary16).
    auto op_bf16_for = [&](int levels) -> int {
        if (dt == LCMA_F16)
            return 0;
        if (o.bf16_ops_f16 == 1)
            return 0;
        if (o.bf16_ops_f16 == -1)
            return 1;
        return levels == 2 ? 0 : 1;
    };
    // Admissibility: blocks must split evenly and keep 16-byte rows.
    auto admissible = [&](int levels) -> bool {
        const int64_t S = levels == 1 ? 2 : 4;
        if (M % S || N % S || K % S)
            return false;
        const int64_t Mb = M / S, Nb = N / S, Kb = K / S;
        return Mb >= 1 && Nb >= 8 && Kb >= 8 && Nb % 8 == 0 && Kb % 8 == 0 && Nb < kMaxLd && Kb < kMaxLd;
    };

    // One level of the description on the unfused path: even block split,
    // 16-byte rows, and 32-bit offsets into the fp32 output blocks.
    auto admissible_unfused = [&]() -> bool {
        if (M % gen.ms || N % gen.ns || K % gen.ks)
            return false;
        const int64_t Mb = M / gen.ms, Nb = N / gen.ns, Kb = K / gen.ks;
        return Mb >= 1 && Nb >= 8 && Kb >= 8 && Nb % 8 == 0 && Kb % 8 == 0 && Nb <= ((int64_t)1 << 19) &&
               Kb < kMaxLd;
    };

    double est[4] = {-1, -1, -1, -1};
    est[LCMA_ALGO_CLASSIC] = est_classic(M, N, K, m);
    bool ok1 = allow_l1 && (unfused ? admissible_unfused() : admissible(1));
    bool ok2 = allow_l2 && !unfused && !at_load && admissible(2);
    // fp32 fold bytes per element of an output block, summed over the blocks
    // of a description's unfused path: with enough 256 x 256 positions for
    // one persistent launch, those of its run schedule; else each product
    // folds on its own, fold_bytes(c) for a block fed by c products.
    auto unfused_fold_bytes = [&](const lcma_desc& d) -> double {
        const int64_t Mb = M / d.ms, Nb = N / d.ns;
        const int nout = d.ms * d.ns;
        if (((Mb + 255) / 256) * ((Nb + 255) / 256) >= m.P) {
            int8_t Wt[kGenMaxRank * kGenMaxBlocks] = {};
            for (int r = 0; r < d.rank; ++r)
                for (int o = 0; o < nout; ++o)
                    Wt[r * kGenMaxBlocks + o] = d.W[r * nout + o];
            RunSchedule rs;
            plan_runs(Wt, d.rank, nout, &rs);
            return schedule_fold_bytes(rs, d.rank, nout);
        }
        double b = 0;
        for (int o = 0; o < nout; ++o) {
            int c = 0;
            for (int r = 0; r < d.rank; ++r)
                c += d.W[r * nout + o] != 0;
            b += fold_bytes(c);
        }
        return b;
    };
    if (ok1 && unfused) {
        // pre-pass (every operand written), one GEMM per product, fp32 folds
        // into the output blocks (the last one rounds into C)
        const int64_t Mb = M / gen.ms, Nb = N / gen.ns, Kb = K / gen.ks;
        const double pre = 2.0 * ((double)M * K + (double)K * N) + 2.0 * gen.rank * ((double)Mb * Kb + (double)Kb * Nb);
        const double comb = unfused_fold_bytes(gen) * (double)Mb * Nb;
        est[LCMA_ALGO_L1] = (pre + comb) / (m.eta_bw * m.bw) + gen.rank * est_classic(Mb, Nb, Kb, m) + 2 * m.launch;
    } else if (ok1 && at_load) {
        est[LCMA_ALGO_L1] = est_lcma(M, N, K, 1, o.split, false, false, m, true);
    } else if (ok1) {
        est[LCMA_ALGO_L1] = est_lcma(M, N, K, 1, o.split, op_bf16_for(1) != (dt == LCMA_BF16), false, m);
    }
    // One level of the built-in scheme, combine left to the planner: the
    // unfused path when it is estimated faster.  Its products run on the
    // classic kernel's tiles, which wins once the blocks are large (measured
    // at 8192^3 and 16384^3); the fused group kernel wins below.  A split or
    // order request asks for the fused kernel's schedule, so it keeps it.
    bool l1_unfused_auto = false;
    if (ok1 && !unfused && o.combine == LCMA_COMBINE_AUTO && o.split == LCMA_SPLIT_AUTO &&
        o.order == LCMA_ORDER_AUTO && admissible_unfused()) {
        const int64_t Mb = M / 2, Nb = N / 2, Kb = K / 2;
        const double pre = 2.0 * ((double)M * K + (double)K * N) + 2.0 * 7 * ((double)Mb * Kb + (double)Kb * Nb);
        const double comb = unfused_fold_bytes(gen) * (double)Mb * Nb;
        const double t_unf = (pre + comb) / (m.eta_bw * m.bw) + 7 * est_classic(Mb, Nb, Kb, m) + 2 * m.launch;
        if (t_unf < 0.98 * est[LCMA_ALGO_L1]) {
            est[LCMA_ALGO_L1] = t_unf;
            l1_unfused_auto = true;
        }
    }
    if (ok2)
        est[LCMA_ALGO_L2] = est_lcma(M, N, K, 2, o.split, op_bf16_for(2) != (dt == LCMA_BF16), outer2, m);

    // A forced level of the built-in scheme on a shape that does not split
    // evenly: zero-pad M, N, K to multiples of (blocks per side) x 16, plan
    // the padded product and crop it into C (zero-padding non-divisible
    // dimensions to reach an efficient blocking: "CUDA-L2: Surpassing cuBLAS
    // Performance for Matrix Multiplication through Reinforcement Learning",
    // section "核心贡献与发现的技术").  The zero rows and columns add nothing
    // to the product; the padding traffic is part of the estimate.
    const bool forced_lcma = force == LCMA_ALGO_L1 || force == LCMA_ALGO_L2;
    const int64_t pad_g = (force == LCMA_ALGO_L1 ? 2 : 4) * 16;
    auto pad_up = [&](int64_t x) { return (x + pad_g - 1) / pad_g * pad_g; };
    // Padding only changes the shape: an algorithm that is not built for
    // this description or combine mode stays unsupported, and a shape that
    // is already a multiple is never padded (so the padded plan below is
    // always planned without padding).
    if (forced_lcma && !(force == LCMA_ALGO_L1 ? ok1 : ok2) && !generic &&
        (force == LCMA_ALGO_L1 ? allow_l1 : allow_l2 && !unfused) && M > 0 && N > 0 && K > 0 &&
        (pad_up(M) != M || pad_up(N) != N || pad_up(K) != K)) {
        const int64_t Mp = pad_up(M), Np = pad_up(N), Kp = pad_up(K);
        // the padded copies are addressed with leading dimensions Kp and Np
        if (Mp > INT32_MAX || Np >= kMaxLd || Kp >= kMaxLd)
            return LCMA_E_UNSUPPORTED;
        lcma_plan_s* in = nullptr;
        lcma_status s = lcma_plan_ex(Mp, Np, Kp, dt, desc, force, opts, &in);
        if (s != LCMA_OK)
            return s;
        if (in->inner) {   // cannot happen: the padded shape splits evenly
            lcma_plan_destroy(in);
            return LCMA_E_UNSUPPORTED;
        }
        // read A, B; write the padded copies; read the padded C window; write C
        const double pad_bytes = 2.0 * ((double)M * K + (double)K * N + (double)Mp * Kp + (double)Kp * Np) +
                                 4.0 * (double)M * N;
        return wrap_padded(in, M, N, K, dt, force, Mp, Np, Kp, est, pad_bytes / (m.eta_bw * m.bw) + 3 * m.launch,
                           out);
    }

    lcma_algo chosen = force;
    if (force == LCMA_ALGO_L1 && !ok1)
        return LCMA_E_UNSUPPORTED;
    if (force == LCMA_ALGO_L2 && !ok2)
        return LCMA_E_UNSUPPORTED;
    // Accuracy: two levels with combined operands rounded to binary16 from
    // binary16 inputs, or to bfloat16 from bfloat16 inputs, carry about 5.8x
    // the classic kernel's normwise error (fp64 evaluation of the scheme with
    // rounded operands), beyond the 4x this library promises.  Such plans
    // need an explicit opt-in.
    if (force == LCMA_ALGO_L2 && !o.accuracy_optin && (dt == LCMA_F16 || op_bf16_for(2) == 1))
        return LCMA_E_UNSUPPORTED;
    if (force == LCMA_ALGO_AUTO) {
        // Ties (within 2%) go to classic, then to fewer levels.  Two levels
        // with binary16 inputs is never picked automatically: rounding the
        // combined operands to binary16 loses too much accuracy there.
        chosen = LCMA_ALGO_CLASSIC;
        double best = est[LCMA_ALGO_CLASSIC];
        if (ok1 && !unfused && est[LCMA_ALGO_L1] < 0.98 * best) {
            chosen = LCMA_ALGO_L1;
            best = est[LCMA_ALGO_L1];
        }
        if (ok2 && dt == LCMA_BF16 && op_bf16_for(2) == 0 && est[LCMA_ALGO_L2] < 0.98 * best) {
            chosen = LCMA_ALGO_L2;
            best = est[LCMA_ALGO_L2];
        }
    }

    // A classic product whose K or N is not a multiple of 8 cannot use the
    // 16-byte-load kernels.  A plan has a workspace, so it copies A and B
    // into zero-padded buffers with K and N rounded up to 8, runs the fast
    // kernels there and crops C (gemm_classic, which has no workspace, runs
    // the element-load kernel instead).
    if (chosen == LCMA_ALGO_CLASSIC && M > 0 && N > 0 && K > 0 && (K % 8 || N % 8)) {
        const int64_t Np = (N + 7) / 8 * 8, Kp = (K + 7) / 8 * 8;
        if (Np >= kMaxLd || Kp >= kMaxLd)
            return LCMA_E_UNSUPPORTED;
        lcma_plan_s* in = nullptr;
        lcma_status s = lcma_plan_ex(M, Np, Kp, dt, nullptr, LCMA_ALGO_CLASSIC, &o, &in);
        if (s != LCMA_OK)
            return s;
        const double pad_bytes = 2.0 * ((double)M * K + (double)K * N + (double)M * Kp + (double)Kp * Np) +
                                 2.0 * (2.0 * (double)M * Np + (double)M * N);
        return wrap_padded(in, M, N, K, dt, LCMA_ALGO_CLASSIC, M, Np, Kp, est,
                           pad_bytes / (m.eta_bw * m.bw) + 3 * m.launch, out);
    }

    lcma_plan_s* p = new (std::nothrow) lcma_plan_s();
    if (!p)
        return LCMA_E_NOMEM;
    p->M = M; p->N = N; p->K = K; p->dt = dt; p->chosen = chosen; p->P = m.P;
    for (int a = 0; a < 4; ++a)
        p->est[a] = est[a];
    p->classic_tile = classic_tile_for(M, N, m.P);
    p->levels = chosen == LCMA_ALGO_L1 ? 1 : chosen == LCMA_ALGO_L2 ? 2 : 0;
    p->ws_bytes = 0;
    p->n_slots = 0;
    // K splits of classic plans (none with LCMA_SPLIT_NONE, which keeps
    // classic plans free of workspace): decode shapes on the streaming
    // kernels; beyond 64 rows, few tiles on 128 x 128 tiles, or the last,
    // partial round of a multi-round 256 x 256 grid
    const bool ksplit = p->levels == 0 && o.split != LCMA_SPLIT_NONE;
    p->split_s = ksplit ? split_pieces(M, N, K) : 0;
    if (p->split_s)
        p->ws_bytes = (size_t)split_ws_bytes(N, p->split_s, split_rows(M));
    if (ksplit && M > 64) {
        if ((p->split_s = classic_split_pieces(M, N, K, m.P)) != 0) {
            p->classic_tile = kTile128;
            p->ws_bytes = (size_t)((p->split_s * M * N * 4 + 255) / 256 * 256);
        } else if (p->classic_tile == kTile256 && (p->split_s = tail_split_pieces(M, N, K, m.P)) != 0) {
            const int64_t T = ((M + 255) / 256) * ((N + 255) / 256) % m.P;
            p->ws_bytes = (size_t)((p->split_s * T * 256 * 256 * 4 + 255) / 256 * 256);
        }
    }
    p->unfused = p->levels == 1 && (unfused || l1_unfused_auto);
    if (p->unfused) {
        p->op_bf16 = op_bf16_for(1);
        p->gms = gen.ms; p->gks = gen.ks; p->gns = gen.ns; p->gR = gen.rank;
        p->gMb = M / gen.ms; p->gKb = K / gen.ks; p->gNb = N / gen.ns;
        memset(p->gU, 0, sizeof p->gU);
        memset(p->gV, 0, sizeof p->gV);
        memset(p->gW, 0, sizeof p->gW);
        for (int r = 0; r < gen.rank; ++r) {
            for (int x = 0; x < gen.ms * gen.ks; ++x)
                p->gU[r * kGenMaxBlocks + x] = gen.U[r * gen.ms * gen.ks + x];
            for (int x = 0; x < gen.ks * gen.ns; ++x)
                p->gV[r * kGenMaxBlocks + x] = gen.V[r * gen.ks * gen.ns + x];
            for (int x = 0; x < gen.ms * gen.ns; ++x)
                p->gW[r * kGenMaxBlocks + x] = gen.W[r * gen.ms * gen.ns + x];
        }
        // geometry of the one level (for lcma_plan_operand)
        p->geo.Mb = p->gMb; p->geo.Kb = p->gKb; p->geo.Nb = p->gNb; p->geo.R = gen.rank; p->geo.S = 0;
        p->gLdB = p->gNb + ((((p->gMb + 255) / 256) * ((p->gNb + 255) / 256) >= p->P) ? kGenBPad : 0);
        int64_t off = 0;
        p->offGA = off;
        off = align_up(off + (int64_t)gen.rank * p->gMb * p->gKb * 2, 256);
        p->offGB = off;
        off = align_up(off + (int64_t)gen.rank * p->gKb * p->gLdB * 2, 256);
        p->offGC = off;
        off = align_up(off + (int64_t)gen.ms * gen.ns * p->gMb * p->gNb * 4, 256);
        p->ws_bytes = (size_t)off;
        // Enough 256 x 256 output positions for a round of the compute units:
        // every product in one persistent launch.  Whole tiles there: the
        // pre-pass writes the A operands in the engine's stage layout.
        p->gGroup = ((p->gMb + 255) / 256) * ((p->gNb + 255) / 256) >= p->P;
        p->gPackA = p->gGroup && p->gMb % kPackRows == 0 && p->gNb % 256 == 0 && p->gKb % kPackCols == 0;
        if (p->gGroup)
            plan_runs(p->gW, gen.rank, gen.ms * gen.ns, &p->gRuns);
    } else if (p->levels > 0) {
        const int L = p->levels;
        p->op_bf16 = op_bf16_for(L);
        p->write_all = p->op_bf16 != (dt == LCMA_BF16 ? 1 : 0);
        p->outer = L == 2 && outer2;
        p->at_load = L == 1 && at_load;
        p->geo = lcma_geo(M, N, K, L);
        const Geo& g = p->geo;
        const Geo sg = sched_geo(g, p->outer);
        SchedParams& sp = p->sp;
        sp.G = sg.G; sp.gy = sg.gy; sp.gx = sg.gx; sp.R = sg.R; sp.P = m.P;
        sp.mode = split_mode_for(o.split, sg.G, m.P);
        sp.h = (sg.R + 1) / 2;
        sp.raster = o.order == LCMA_ORDER_PLAIN ? 0 : 8;
        if (sp.mode == kSplitTail) {
            p->n_slots = sg.G % m.P;
            p->grid = sg.G / m.P > 0 ? m.P : 2 * (sg.G % m.P);
        } else if (sp.mode == kSplitAll) {
            p->n_slots = sg.G;
            p->grid = std::min(2 * sg.G, m.P);
        } else {
            p->grid = std::min(sg.G, m.P);
        }
        fused_order(p->outer ? 1 : L, p->order);
        fused_order(1, p->order1);
        // workspace layout
        std::call_once(g_tables_once, init_tables);
        const int SS = g.S * g.S;
        const int8_t* U = L == 1 ? g_U1 : g_U2;
        const int8_t* V = L == 1 ? g_V1 : g_V2;
        int nA = 0, nB = 0;
        for (int r = 0; r < g.R; ++r) {
            int na = 0, nb = 0, ba = -1, bb = -1, ca = 0, cb = 0;
            for (int x = 0; x < SS; ++x) {
                if (U[r * SS + x]) { ++na; ba = x; ca = U[r * SS + x]; }
                if (V[r * SS + x]) { ++nb; bb = x; cb = V[r * SS + x]; }
            }
            // Same rule as the pre-pass kernel: a single-block operand is read
            // in place (the built-in schemes give it coefficient +1).
            (void)ca; (void)cb;
            const bool wa = !p->at_load && (p->write_all || na > 1);
            const bool wb = !p->at_load && (p->write_all || nb > 1);
            p->slotA[r] = wa ? nA++ : -1;
            p->slotB[r] = wb ? nB++ : -1;
            p->blockA[r] = ba;
            p->blockB[r] = bb;
        }
        int64_t off = 0;
        p->offA = off;
        off = align_up(off + (int64_t)nA * g.Mb * g.Kb * 2, 256);
        p->offB = off;
        off = align_up(off + (int64_t)nB * g.Kb * g.Nb * 2, 256);
        p->offPart = off;
        off = align_up(off + (int64_t)p->n_slots * 2 * fused_partial_bytes(p->outer ? 1 : L), 256);
        p->offCtr = off;
        off = align_up(off + (int64_t)p->n_slots * 4, 256);
        p->offAcc = off;
        if (p->outer)
            off = align_up(off + (int64_t)16 * g.Mb * g.Nb * 4, 256);
        p->ws_bytes = (size_t)off;
    }
    if (log_enabled())
        fprintf(stderr, "[lcma] plan M=%lld N=%lld K=%lld %s: est classic=%.3g L1=%.3g L2=%.3g s -> %s (ws %zu B)\n",
                (long long)M, (long long)N, (long long)K, dt == LCMA_BF16 ? "bf16" : "f16", est[1], est[2],
                est[3], chosen == LCMA_ALGO_CLASSIC ? "classic" : chosen == LCMA_ALGO_L1 ? "L1" : "L2",
                p->ws_bytes);
    *out = p;
    return LCMA_OK;
}

lcma_status lcma_plan(int64_t M, int64_t N, int64_t K, lcma_dtype dt, const lcma_desc* desc, lcma_algo force,
                      lcma_plan_t* out)
{
    return lcma_plan_ex(M, N, K, dt, desc, force, nullptr, out);
}

lcma_status lcma_plan_info(lcma_plan_t p, lcma_algo* chosen, size_t* ws, double* est)
{
    if (!p)
        return LCMA_E_INVALID;
    if (chosen)
        *chosen = p->chosen;
    if (ws)
        *ws = p->ws_bytes;
    if (est)
        *est = p->est[p->chosen];
    return LCMA_OK;
}

lcma_status lcma_plan_estimate(lcma_plan_t p, lcma_algo algo, double* est)
{
    if (!p || !est || enum_bits(&algo) < LCMA_ALGO_CLASSIC || enum_bits(&algo) > LCMA_ALGO_L2)
        return LCMA_E_INVALID;
    *est = p->est[algo];
    return LCMA_OK;
}

lcma_status lcma_plan_operand(lcma_plan_t p, int32_t side, int32_t r, int64_t* offset, int64_t* ld,
                              lcma_dtype* dtype)
{
    if (!p || p->levels == 0 || side < 0 || side > 1 || r < 0 || r >= p->geo.R)
        return LCMA_E_INVALID;
    if (p->at_load)
        return LCMA_E_INVALID;   // no combined operand is ever written
    if (p->inner) {
        const lcma_status s = lcma_plan_operand(p->inner, side, r, offset, ld, dtype);
        if (s == LCMA_OK && offset && *offset >= 0)
            *offset += p->offIn;
        return s;
    }
    if (p->unfused) {
        if (offset)
            *offset = side == 0 ? p->offGA + (int64_t)r * p->gMb * p->gKb * 2 : p->offGB + (int64_t)r * p->gKb * p->gLdB * 2;
        if (ld)
            *ld = side == 0 ? (p->gPackA ? 0 : p->gKb) : p->gLdB;
        if (dtype)
            *dtype = p->op_bf16 ? LCMA_BF16 : LCMA_F16;
        return LCMA_OK;
    }
    const int64_t slot = side == 0 ? p->slotA[r] : p->slotB[r];
    if (offset)
        *offset = slot < 0 ? -1
                           : (side == 0 ? p->offA + slot * p->geo.Mb * p->geo.Kb * 2
                                        : p->offB + slot * p->geo.Kb * p->geo.Nb * 2);
    if (ld)
        *ld = side == 0 ? p->geo.Kb : p->geo.Nb;
    if (dtype)
        *dtype = p->op_bf16 ? LCMA_BF16 : LCMA_F16;
    return LCMA_OK;
}

lcma_status lcma_plan_runs(lcma_plan_t p, int32_t run, int32_t* product, int32_t* carry, int8_t* fold)
{
    if (p && p->inner)
        return lcma_plan_runs(p->inner, run, product, carry, fold);
    if (!p || !p->unfused || !p->gGroup || run < 0 || run >= p->gR || !product || !carry || !fold)
        return LCMA_E_INVALID;
    *product = p->gRuns.prod[run];
    *carry = p->gRuns.carry[run];
    for (int o = 0; o < p->gms * p->gns; ++o)
        fold[o] = p->gRuns.w[run][o];
    return LCMA_OK;
}

lcma_status lcma_plan_schedule(lcma_plan_t p, int32_t* items, int64_t cap, int64_t* count, int32_t* order)
{
    if (p && p->inner)
        return lcma_plan_schedule(p->inner, items, cap, count, order);
    if (!p || p->levels == 0 || p->unfused || !count || (cap > 0 && !items))
        return LCMA_E_INVALID;
    int64_t n = 0;
    for (int w = 0; w < p->grid; ++w) {
        const int c = sched_count(p->sp, w);
        for (int i = 0; i < c; ++i, ++n) {
            if (n < cap) {
                const Item it = sched_item(p->sp, w, i);
                int32_t* o = items + 5 * n;
                o[0] = w; o[1] = it.g; o[2] = it.pos0; o[3] = it.pos1; o[4] = it.slot;
            }
        }
    }
    *count = n;
    if (order)
        for (int r = 0; r < p->sp.R; ++r)
            order[r] = p->order[r];
    return LCMA_OK;
}

void lcma_plan_destroy(lcma_plan_t p)
{
    if (p)
        lcma_plan_destroy(p->inner);
    delete p;
}

}  // extern "C"

// ---------------------------------------------------------------- launching

namespace {

struct Io {
    bool vec, vec4;
};

lcma_status check_io(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* B, int64_t ldb,
                     const void* C, int64_t ldc, Io* io, bool check_c = true)
{
    if (M < 0 || N < 0 || K < 0)
        return LCMA_E_INVALID;
    if (check_c && M > 0 && N > 0 && (!C || ldc < std::max<int64_t>(N, 1)))
        return LCMA_E_INVALID;
    if (M > 0 && N > 0 && K > 0) {
        if (!A || !B || lda < K || ldb < N)
            return LCMA_E_INVALID;
    }
    // 32-bit buffer offsets: a tile spans at most 256 rows of a leading dimension.
    if (lda >= kMaxLd || ldb >= kMaxLd || (check_c && ldc >= kMaxLd))
        return LCMA_E_UNSUPPORTED;
    const auto al = [](const void* x, uintptr_t a) { return ((uintptr_t)x % a) == 0; };
    io->vec = al(A, 16) && al(B, 16) && lda % 8 == 0 && ldb % 8 == 0 && K % 8 == 0 && N % 8 == 0;
    io->vec4 = check_c ? (al(C, 8) && ldc % 4 == 0 && N % 4 == 0) : false;
    return LCMA_OK;
}

lcma_status run_classic(int64_t M, int64_t N, int64_t K, lcma_dtype dt, const void* A, int64_t lda, const void* B,
                        int64_t ldb, void* C, int64_t ldc, const Io& io, int tile, int P, hipStream_t st,
                        void* split_ws = nullptr, int split_s = 0)
{
    if (M == 0 || N == 0)
        return LCMA_OK;
    ClassicLaunch L;
    L.A = A; L.lda = lda; L.B = B; L.ldb = ldb; L.C = C; L.ldc = ldc;
    L.M = (int32_t)M; L.N = (int32_t)N; L.K = (int32_t)K;
    L.bf16 = dt == LCMA_BF16; L.vec = io.vec; L.vec4 = io.vec4; L.tile = tile; L.P = P;
    L.split_ws = split_s ? split_ws : nullptr;
    L.split_s = split_s;
    return hip_status(launch_classic(L, st), "launch_classic");
}

lcma_status check_ws(const lcma_plan_s* p, void* ws, size_t ws_bytes)
{
    if (p->ws_bytes == 0)
        return LCMA_OK;
    if (!ws || ws_bytes < p->ws_bytes || ((uintptr_t)ws % 256) != 0)
        return LCMA_E_WORKSPACE;
    return LCMA_OK;
}

// Padded plans.  The element-wise pad and crop kernels take any alignment,
// so only the arguments' validity and the workspace are checked here.
lcma_status check_padded_call(const lcma_plan_s* p, const void* A, int64_t lda, const void* B, int64_t ldb,
                              const void* C, int64_t ldc, void* ws, size_t ws_bytes, bool need_c)
{
    Io io;
    const lcma_status s = check_io(p->M, p->N, p->K, A, lda, B, ldb, C, ldc, &io, need_c);
    return s != LCMA_OK ? s : check_ws(p, ws, ws_bytes);
}

lcma_status pad_operands(const lcma_plan_s* p, const void* A, int64_t lda, const void* B, int64_t ldb, void* ws,
                         hipStream_t st)
{
    char* w = (char*)ws;
    if (hip_status(launch_pad_copy(A, lda, p->M, p->K, w + p->offPA, p->Kp, p->Mp, p->Kp, st), "pad A") != LCMA_OK ||
        hip_status(launch_pad_copy(B, ldb, p->K, p->N, w + p->offPB, p->Np, p->Kp, p->Np, st), "pad B") != LCMA_OK)
        return LCMA_E_HIP;
    return LCMA_OK;
}

lcma_status crop_output(const lcma_plan_s* p, void* C, int64_t ldc, void* ws, hipStream_t st)
{
    return hip_status(launch_pad_copy((char*)ws + p->offPC, p->Np, p->M, p->N, C, ldc, p->M, p->N, st), "crop C");
}

lcma_status do_prepass(const lcma_plan_s* p, const void* A, int64_t lda, const void* B, int64_t ldb, void* ws,
                       hipStream_t st)
{
    PrepassLaunch L;
    L.A = A; L.lda = lda; L.B = B; L.ldb = ldb;
    L.Mb = (int32_t)p->geo.Mb; L.Kb = (int32_t)p->geo.Kb; L.Nb = (int32_t)p->geo.Nb;
    L.outA = (char*)ws + p->offA;
    L.outB = (char*)ws + p->offB;
    L.strideA = p->geo.Mb * p->geo.Kb;
    L.strideB = p->geo.Kb * p->geo.Nb;
    L.levels = p->levels;
    L.in_bf16 = p->dt == LCMA_BF16;
    L.op_bf16 = p->op_bf16;
    L.write_all = p->write_all;
    L.counters = (int32_t*)((char*)ws + p->offCtr);
    L.n_counters = p->n_slots;
    return hip_status(launch_prepass(L, st), "launch_prepass");
}

// Operand pointers of canonical product r into position j of the kernel
// arguments: the pre-pass output, or the block of A / B read in place.
void set_operands(const lcma_plan_s* p, const void* A, int64_t lda, const void* B, int64_t ldb, void* ws, int r,
                  int j, FusedParams& fp)
{
    const Geo& g = p->geo;
    if (p->slotA[r] >= 0) {
        fp.a[j] = (const uint16_t*)((char*)ws + p->offA) + p->slotA[r] * g.Mb * g.Kb;
        fp.lda[j] = g.Kb;
    } else {
        const int bi = p->blockA[r] / g.S, bk = p->blockA[r] % g.S;
        fp.a[j] = (const uint16_t*)A + bi * g.Mb * lda + bk * g.Kb;
        fp.lda[j] = lda;
    }
    if (p->slotB[r] >= 0) {
        fp.b[j] = (const uint16_t*)((char*)ws + p->offB) + p->slotB[r] * g.Kb * g.Nb;
        fp.ldb[j] = g.Nb;
    } else {
        const int bk = p->blockB[r] / g.S, bj = p->blockB[r] % g.S;
        fp.b[j] = (const uint16_t*)B + bk * g.Kb * ldb + bj * g.Nb;
        fp.ldb[j] = ldb;
    }
}

lcma_status do_fused(const lcma_plan_s* p, const void* A, int64_t lda, const void* B, int64_t ldb, void* C,
                     int64_t ldc, const Io& io, void* ws, hipStream_t st)
{
    FusedLaunch L;
    memset(&L, 0, sizeof L);
    const Geo& g = p->geo;
    L.p.C = (uint16_t*)C;
    L.p.ldc = ldc;
    L.p.Mb = (int32_t)g.Mb; L.p.Nb = (int32_t)g.Nb; L.p.Kb = (int32_t)g.Kb;
    L.p.vec4 = io.vec4;
    L.p.sp = p->sp;
    L.p.partial = (float*)((char*)ws + p->offPart);
    L.p.counters = (int32_t*)((char*)ws + p->offCtr);
    L.levels = p->levels;
    L.op_bf16 = p->op_bf16;
    L.out_bf16 = p->dt == LCMA_BF16;
    L.grid = p->grid;
    if (p->at_load) {
        // Each operand is one or two input blocks (block order), read in
        // place with the inputs' leading dimensions; a coefficient of -1
        // becomes a sign mask on the loaded halves.
        L.at_load = 1;
        // no pre-pass clears the split fix-up counters here: a fill kernel
        // does (no memset node, so the call stays capturable)
        if (p->n_slots > 0 &&
            hip_status(launch_pad_copy(L.p.counters, 0, 0, 0, L.p.counters, 2 * p->n_slots, 1, 2 * p->n_slots, st),
                       "launch_pad_copy (split counters)") != LCMA_OK)
            return LCMA_E_HIP;
        for (int r = 0; r < 7; ++r) {
            int na = 0, nb = 0;
            for (int x = 0; x < 4; ++x) {
                const int bi = x / 2, bk = x % 2;
                if (g_U1[r * 4 + x]) {
                    const uint16_t* ptr = (const uint16_t*)A + bi * g.Mb * lda + bk * g.Kb;
                    (na == 0 ? L.p.a[r] : L.p.a2[r]) = ptr;
                    L.p.sa[r][na++] = g_U1[r * 4 + x] < 0 ? 0x80008000u : 0u;
                }
                const int kb = x / 2, bj = x % 2;
                if (g_V1[r * 4 + x]) {
                    const uint16_t* ptr = (const uint16_t*)B + kb * g.Kb * ldb + bj * g.Nb;
                    (nb == 0 ? L.p.b[r] : L.p.b2[r]) = ptr;
                    L.p.sb[r][nb++] = g_V1[r * 4 + x] < 0 ? 0x80008000u : 0u;
                }
            }
            if (na < 1 || na > 2 || nb < 1 || nb > 2)
                return LCMA_E_UNSUPPORTED;   // not a Strassen-shaped row
            L.p.lda[r] = lda;
            L.p.ldb[r] = ldb;
            L.p.order[r] = p->order[r];
            for (int o = 0; o < 4; ++o)
                L.p.w[r][o] = g_W1[r * 4 + o];
        }
        return hip_status(launch_fused(L, st), "launch_fused (combine at load)");
    }
    if (!p->outer) {
        const int8_t* W = p->levels == 1 ? g_W1 : g_W2;
        for (int r = 0; r < g.R; ++r) {
            set_operands(p, A, lda, B, ldb, ws, r, r, L.p);
            L.p.order[r] = p->order[r];
            for (int o = 0; o < g.S * g.S; ++o)
                L.p.w[r][o] = W[r * g.S * g.S + o];
        }
        return hip_status(launch_fused(L, st), "launch_fused");
    }
    // Two levels, outer level in memory: one launch per outer product r1 (in
    // the order order1), each running the inner products (r1, r2) = r1*7 + r2
    // of the flattened scheme.  Outer output (i1, j1) is fed by every r1 with
    // W1[r1][i1, j1] != 0: the first in launch order stores its fp32 blocks,
    // the last adds and rounds into C.
    L.outer = 1;
    L.p.acc = (float*)((char*)ws + p->offAcc);
    int first[4], last[4], uses[4];
    for (int o = 0; o < 4; ++o) {
        first[o] = last[o] = -1;
        uses[o] = 0;
        for (int k = 0; k < 7; ++k)
            if (g_W1[p->order1[k] * 4 + o] != 0) {
                if (first[o] < 0)
                    first[o] = k;
                last[o] = k;
                ++uses[o];
            }
    }
    for (int r2 = 0; r2 < 7; ++r2) {
        L.p.order[r2] = p->order[r2];
        for (int o = 0; o < 4; ++o)
            L.p.w[r2][o] = g_W1[r2 * 4 + o];
    }
    for (int k = 0; k < 7; ++k) {
        const int r1 = p->order1[k];
        for (int r2 = 0; r2 < 7; ++r2)
            set_operands(p, A, lda, B, ldb, ws, r1 * 7 + r2, r2, L.p);
        for (int o = 0; o < 4; ++o) {
            const int c = g_W1[r1 * 4 + o];
            L.p.ow[o] = (float)c;
            L.p.omode[o] = c == 0             ? kOuterNone
                           : uses[o] == 1     ? kOuterOnly
                           : k == first[o]    ? kOuterStore
                           : k == last[o]     ? kOuterFinish
                                              : kOuterAdd;
        }
        if (hip_status(launch_fused(L, st), "launch_fused (outer level)") != LCMA_OK)
            return LCMA_E_HIP;
    }
    return LCMA_OK;
}

// Unfused path, pre-pass half: every combined operand of both sides.
lcma_status do_gen_prepass(const lcma_plan_s* p, const void* A, int64_t lda, const void* B, int64_t ldb, void* ws,
                           hipStream_t st)
{
    GenPrepassLaunch L;
    memset(&L, 0, sizeof L);
    L.in_bf16 = p->dt == LCMA_BF16;
    L.op_bf16 = p->op_bf16;
    L.rank = p->gR;
    // side A: blocks (i, k) of Mb x Kb
    L.X = A; L.ldx = lda; L.rows = (int32_t)p->gMb; L.cols = (int32_t)p->gKb; L.bcols = p->gks;
    L.nblocks = p->gms * p->gks;
    memcpy(L.coef, p->gU, sizeof L.coef);
    L.out = (char*)ws + p->offGA; L.ldo = p->gKb; L.stride = p->gMb * p->gKb;
    L.packed = p->gPackA;
    if (hip_status(launch_gen_prepass(L, st), "launch_gen_prepass") != LCMA_OK)
        return LCMA_E_HIP;
    L.packed = 0;
    // side B: blocks (k, j) of Kb x Nb
    L.X = B; L.ldx = ldb; L.rows = (int32_t)p->gKb; L.cols = (int32_t)p->gNb; L.bcols = p->gns;
    L.nblocks = p->gks * p->gns;
    memcpy(L.coef, p->gV, sizeof L.coef);
    L.out = (char*)ws + p->offGB; L.ldo = p->gLdB; L.stride = p->gKb * p->gLdB;
    return hip_status(launch_gen_prepass(L, st), "launch_gen_prepass");
}

// Unfused path, product half: one GEMM per product, whose epilogue folds
// W[r][i,j] * H_r into output block (i, j).  The first product feeding a
// block stores its fp32 sum in the workspace, later ones add, and the last
// one rounds it into C (a block fed by one product goes straight to C), so
// no fill or final rounding pass is needed.  Brent's identity gives every
// output block at least one product.
// The persistent launch runs the plan's run schedule; fold modes (store,
// add, finish, only) follow from the order of the runs that fold into each
// block.
void gen_group_runs(const lcma_plan_s* p, int nout, GenGroupLaunch* G)
{
    const RunSchedule& s = p->gRuns;
    for (int j = 0; j < p->gR; ++j) {
        G->prod[j] = s.prod[j];
        G->carry[j] = s.carry[j];
    }
    for (int o = 0; o < nout; ++o) {
        int f = -1, l = -1, c = 0;
        for (int j = 0; j < p->gR; ++j)
            if (s.w[j][o] != 0) {
                f = f < 0 ? j : f;
                l = j;
                ++c;
            }
        for (int j = 0; j < p->gR; ++j) {
            const int w = s.w[j][o];
            G->w[j * kGenMaxBlocks + o] = (int8_t)w;
            G->mode[j * kGenMaxBlocks + o] = w == 0  ? kOuterNone
                                             : c == 1 ? kOuterOnly
                                             : j == f ? kOuterStore
                                             : j == l ? kOuterFinish
                                                      : kOuterAdd;
        }
    }
}

lcma_status do_gen_products(const lcma_plan_s* p, void* C, int64_t ldc, void* ws, hipStream_t st)
{
    float* acc = (float*)((char*)ws + p->offGC);
    const int nout = p->gms * p->gns;
    int first[kGenMaxBlocks], last[kGenMaxBlocks], uses[kGenMaxBlocks];
    for (int o = 0; o < nout; ++o) {
        first[o] = last[o] = -1;
        uses[o] = 0;
        for (int r = 0; r < p->gR; ++r)
            if (p->gW[r * kGenMaxBlocks + o] != 0) {
                if (first[o] < 0)
                    first[o] = r;
                last[o] = r;
                ++uses[o];
            }
        if (uses[o] == 0)
            return LCMA_E_BAD_DESCRIPTOR;
    }
    // Every product in one persistent launch, each position owned by one
    // workgroup throughout.
    if (p->gGroup) {
        GenGroupLaunch G;
        memset(&G, 0, sizeof G);
        G.A0 = (const char*)ws + p->offGA; G.strideA = p->gMb * p->gKb;
        G.B0 = (const char*)ws + p->offGB; G.strideB = p->gKb * p->gLdB; G.ldb = p->gLdB;
        G.M = (int32_t)p->gMb; G.N = (int32_t)p->gNb; G.K = (int32_t)p->gKb; G.R = p->gR;
        G.op_bf16 = p->op_bf16; G.out_bf16 = p->dt == LCMA_BF16; G.P = p->P;
        G.nout = nout; G.ncols = p->gns;
        G.acc = acc; G.C = C; G.ldc = ldc;
        G.packed_a = p->gPackA;
        gen_group_runs(p, nout, &G);
        return hip_status(launch_gen_group(G, st), "launch_gen_group");
    }
    for (int r = 0; r < p->gR; ++r) {
        GenProductLaunch L;
        memset(&L, 0, sizeof L);
        L.A = (const char*)ws + p->offGA + (int64_t)r * p->gMb * p->gKb * 2; L.lda = p->gKb;
        L.B = (const char*)ws + p->offGB + (int64_t)r * p->gKb * p->gLdB * 2; L.ldb = p->gLdB;
        L.M = (int32_t)p->gMb; L.N = (int32_t)p->gNb; L.K = (int32_t)p->gKb;
        L.op_bf16 = p->op_bf16; L.P = p->P; L.ldt = p->gNb;
        L.ldc = ldc; L.out_bf16 = p->dt == LCMA_BF16;
        for (int o = 0; o < nout; ++o) {
            const int w = p->gW[r * kGenMaxBlocks + o];
            if (w != 0) {
                const int bi = o / p->gns, bj = o % p->gns;
                L.tgt[L.ntgt] = acc + (int64_t)o * p->gMb * p->gNb;
                L.cdst[L.ntgt] = (uint16_t*)C + bi * p->gMb * ldc + bj * p->gNb;
                L.w[L.ntgt] = (float)w;
                L.mode[L.ntgt] = uses[o] == 1 ? kOuterOnly
                                 : r == first[o] ? kOuterStore
                                 : r == last[o]  ? kOuterFinish
                                                 : kOuterAdd;
                ++L.ntgt;
            }
        }
        if (L.ntgt == 0)
            continue;
        if (hip_status(launch_gen_product(L, st), "launch_gen_product") != LCMA_OK)
            return LCMA_E_HIP;
    }
    return LCMA_OK;
}

lcma_status check_lcma_call(const lcma_plan_s* p, const void* A, int64_t lda, const void* B, int64_t ldb,
                            const void* C, int64_t ldc, void* ws, size_t ws_bytes, bool need_c, Io* io)
{
    lcma_status s = check_io(p->M, p->N, p->K, A, lda, B, ldb, C, ldc, io, need_c);
    if (s != LCMA_OK)
        return s;
    // LCMA paths use 16-byte operand loads and 8-byte C stores only.
    if (!io->vec || (need_c && !io->vec4))
        return LCMA_E_UNSUPPORTED;
    return check_ws(p, ws, ws_bytes);
}

}  // namespace

extern "C" {

lcma_status gemm_classic(int64_t M, int64_t N, int64_t K, lcma_dtype dt, const void* A, int64_t lda, const void* B,
                         int64_t ldb, void* C, int64_t ldc, void* stream)
{
    if (enum_bits(&dt) != LCMA_F16 && enum_bits(&dt) != LCMA_BF16)
        return LCMA_E_INVALID;
    if (M > INT32_MAX || N > INT32_MAX || K > INT32_MAX)
        return LCMA_E_INVALID;
    Io io;
    lcma_status s = check_io(M, N, K, A, lda, B, ldb, C, ldc, &io);
    if (s != LCMA_OK)
        return s;
    if (M == 0 || N == 0)
        return LCMA_OK;
    int P = 0;
    if (query_cus(&P) != 0)
        return LCMA_E_HIP;
    return run_classic(M, N, K, dt, A, lda, B, ldb, C, ldc, io, classic_tile_for(M, N, P), P, (hipStream_t)stream);
}

lcma_status lcma_gemm(lcma_plan_t p, const void* A, int64_t lda, const void* B, int64_t ldb, void* C, int64_t ldc,
                      void* ws, size_t ws_bytes, void* stream)
{
    if (!p)
        return LCMA_E_INVALID;
    hipStream_t st = (hipStream_t)stream;
    if (p->inner) {
        lcma_status s = check_padded_call(p, A, lda, B, ldb, C, ldc, ws, ws_bytes, true);
        if (s != LCMA_OK)
            return s;
        char* w = (char*)ws;
        s = pad_operands(p, A, lda, B, ldb, ws, st);
        if (s == LCMA_OK)
            s = lcma_gemm(p->inner, w + p->offPA, p->Kp, w + p->offPB, p->Np, w + p->offPC, p->Np, w + p->offIn,
                          p->inner->ws_bytes, stream);
        return s != LCMA_OK ? s : crop_output(p, C, ldc, ws, st);
    }
    if (p->levels == 0) {
        Io io;
        lcma_status s = check_io(p->M, p->N, p->K, A, lda, B, ldb, C, ldc, &io);
        if (s == LCMA_OK)
            s = check_ws(p, ws, ws_bytes);
        if (s != LCMA_OK)
            return s;
        return run_classic(p->M, p->N, p->K, p->dt, A, lda, B, ldb, C, ldc, io, p->classic_tile, p->P, st, ws,
                           p->split_s);
    }
    Io io;
    lcma_status s = check_lcma_call(p, A, lda, B, ldb, C, ldc, ws, ws_bytes, true, &io);
    if (s != LCMA_OK)
        return s;
    if (p->unfused) {
        s = do_gen_prepass(p, A, lda, B, ldb, ws, st);
        return s != LCMA_OK ? s : do_gen_products(p, C, ldc, ws, st);
    }
    if (!p->at_load) {
        s = do_prepass(p, A, lda, B, ldb, ws, st);
        if (s != LCMA_OK)
            return s;
    }
    return do_fused(p, A, lda, B, ldb, C, ldc, io, ws, st);
}

lcma_status lcma_measure_mfma(float* out, int32_t workgroups, int32_t iters, lcma_dtype dt, void* stream)
{
    if (!out || workgroups < 1 || workgroups > (1 << 16) || iters < 1 || iters > (1 << 24) ||
        (enum_bits(&dt) != LCMA_F16 && enum_bits(&dt) != LCMA_BF16))
        return LCMA_E_INVALID;
    return hip_status(launch_ref_mfma(out, workgroups, iters, dt == LCMA_BF16, (hipStream_t)stream), "launch_ref_mfma");
}

lcma_status lcma_measure_copy(const void* src, void* dst, size_t bytes, void* stream)
{
    if (bytes == 0)
        return LCMA_OK;
    if (!src || !dst)
        return LCMA_E_INVALID;
    if ((uintptr_t)src % 16 || (uintptr_t)dst % 16 || bytes % 16)
        return LCMA_E_UNSUPPORTED;
    int P = 0;
    if (query_cus(&P) != 0)
        return LCMA_E_HIP;
    // 64 workgroups per compute unit (measured best of 4..64 on MI355X)
    return hip_status(launch_ref_copy(src, dst, (int64_t)(bytes / 16), 64 * P, (hipStream_t)stream), "launch_ref_copy");
}

lcma_status lcma_measure_read(const void* src, size_t bytes, uint32_t* out, void* stream)
{
    if (bytes == 0)
        return LCMA_OK;
    if (!src || !out)
        return LCMA_E_INVALID;
    if ((uintptr_t)src % 16 || bytes % 16)
        return LCMA_E_UNSUPPORTED;
    int P = 0;
    if (query_cus(&P) != 0)
        return LCMA_E_HIP;
    // 16 workgroups per compute unit: eight 16-byte loads in flight per lane
    return hip_status(launch_ref_read(src, (int64_t)(bytes / 16), 16 * P, 0x9e3779b9u, out, (hipStream_t)stream),
                      "launch_ref_read");
}

lcma_status lcma_gemm_noalloc(lcma_plan_t p, const void* A, int64_t lda, const void* B, int64_t ldb, void* C,
                              int64_t ldc, void* stream)
{
    static_assert(kScratchBytes == LCMA_SCRATCH_BYTES, "scratch size in lcma.h and kernels.hpp");
    if (!p)
        return LCMA_E_INVALID;
    if (p->ws_bytes > kScratchBytes) {
        if (log_enabled())
            fprintf(stderr, "lcma: lcma_gemm_noalloc: the plan needs %zu workspace bytes, more than the %zu of the "
                            "static scratch array\n", p->ws_bytes, kScratchBytes);
        return LCMA_E_WORKSPACE;
    }
    void* ws = nullptr;
    if (p->ws_bytes > 0 && hip_status(scratch_address(&ws), "hipGetSymbolAddress(scratch)") != LCMA_OK)
        return LCMA_E_HIP;
    return lcma_gemm(p, A, lda, B, ldb, C, ldc, ws, p->ws_bytes, stream);
}

lcma_status lcma_prepass(lcma_plan_t p, const void* A, int64_t lda, const void* B, int64_t ldb, void* ws,
                         size_t ws_bytes, void* stream)
{
    if (!p || p->levels == 0)
        return LCMA_E_INVALID;
    if (p->inner) {
        lcma_status s = check_padded_call(p, A, lda, B, ldb, nullptr, 0, ws, ws_bytes, false);
        if (s == LCMA_OK)
            s = pad_operands(p, A, lda, B, ldb, ws, (hipStream_t)stream);
        char* w = (char*)ws;
        return s != LCMA_OK ? s
                            : lcma_prepass(p->inner, w + p->offPA, p->Kp, w + p->offPB, p->Np, w + p->offIn,
                                           p->inner->ws_bytes, stream);
    }
    Io io;
    lcma_status s = check_lcma_call(p, A, lda, B, ldb, nullptr, 0, ws, ws_bytes, false, &io);
    if (s != LCMA_OK)
        return s;
    if (p->unfused)
        return do_gen_prepass(p, A, lda, B, ldb, ws, (hipStream_t)stream);
    if (p->at_load)
        return LCMA_OK;   // the group kernel combines the blocks itself
    return do_prepass(p, A, lda, B, ldb, ws, (hipStream_t)stream);
}

lcma_status lcma_fused(lcma_plan_t p, const void* A, int64_t lda, const void* B, int64_t ldb, void* C, int64_t ldc,
                       void* ws, size_t ws_bytes, void* stream)
{
    if (!p || p->levels == 0)
        return LCMA_E_INVALID;
    if (p->inner) {
        // the padded operands were written by lcma_prepass on this workspace
        lcma_status s = check_padded_call(p, A, lda, B, ldb, C, ldc, ws, ws_bytes, true);
        char* w = (char*)ws;
        if (s == LCMA_OK)
            s = lcma_fused(p->inner, w + p->offPA, p->Kp, w + p->offPB, p->Np, w + p->offPC, p->Np, w + p->offIn,
                           p->inner->ws_bytes, stream);
        return s != LCMA_OK ? s : crop_output(p, C, ldc, ws, (hipStream_t)stream);
    }
    Io io;
    lcma_status s = check_lcma_call(p, A, lda, B, ldb, C, ldc, ws, ws_bytes, true, &io);
    if (s != LCMA_OK)
        return s;
    if (p->unfused)
        return do_gen_products(p, C, ldc, ws, (hipStream_t)stream);
    return do_fused(p, A, lda, B, ldb, C, ldc, io, ws, (hipStream_t)stream);
}

}  // extern "C"
