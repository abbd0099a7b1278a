// strassen.hpp -- the built-in LCMA schemes of the library, usable from host
// and device code.
//
// One level: Strassen's 1969 rank-7 scheme for a 2x2 block product
// ("FalconGEMM: Surpassing Hardware Peaks with Lower-Complexity Matrix
// Multiplication", section "从 Strassen 出发": 8 block products become 7).
// Blocks are ordered [11, 12, 21, 22]; product r uses
//   Ahat = sum U1[r][b] A_b,  Bhat = sum V1[r][b] B_b,  C_b += W1[r][b] Ahat*Bhat.
// Written from the formulas
//   P1 = (A11+A22)(B11+B22), P2 = (A21+A22)B11, P3 = A11(B12-B22),
//   P4 = A22(B21-B11), P5 = (A11+A12)B22, P6 = (A21-A11)(B11+B12),
//   P7 = (A12-A22)(B21+B22);
//   C11 = P1+P4-P5+P7, C12 = P3+P5, C21 = P2+P4, C22 = P1-P2+P3+P6.
//
// Two levels (same section: 64 block products become 49) is the scheme
// applied inside each block product, flattened: product (r1, r2) -> r1*7+r2
// and a 4x4 block index (2*outer + inner) in each dimension.
#pragma once
#include <stdint.h>

#if defined(__HIPCC__)
#define LCMA_HD __host__ __device__
#else
#define LCMA_HD
#endif

namespace lcma {

constexpr int8_t kU1[7][4] = {{1, 0, 0, 1}, {0, 0, 1, 1}, {1, 0, 0, 0}, {0, 0, 0, 1},
                              {1, 1, 0, 0}, {-1, 0, 1, 0}, {0, 1, 0, -1}};
constexpr int8_t kV1[7][4] = {{1, 0, 0, 1}, {1, 0, 0, 0}, {0, 1, 0, -1}, {-1, 0, 1, 0},
                              {0, 0, 0, 1}, {1, 1, 0, 0}, {0, 0, 1, 1}};
constexpr int8_t kW1[7][4] = {{1, 0, 0, 1}, {0, 0, 1, -1}, {0, 1, 0, 1}, {1, 0, 1, 0},
                              {-1, 1, 0, 0}, {0, 0, 0, 1}, {1, 0, 0, 0}};

// Coefficient of block (i, j) of a two-level table built from a one-level
// table T (2x2 blocks): i = 2*i1 + i2, j = 2*j1 + j2, r = r1*7 + r2.
LCMA_HD constexpr int coef2(const int8_t (&T)[7][4], int r, int i, int j)
{
    return T[r / 7][(i >> 1) * 2 + (j >> 1)] * T[r % 7][(i & 1) * 2 + (j & 1)];
}

// Coefficient accessors: levels 1 (2x2 blocks, 7 products) or 2 (4x4, 49).
template <int LEVELS> struct Scheme;

template <> struct Scheme<1> {
    static constexpr int S = 2;   // blocks per dimension
    static constexpr int R = 7;
    LCMA_HD static constexpr int u(int r, int i, int k) { return kU1[r][i * 2 + k]; }
    LCMA_HD static constexpr int v(int r, int k, int j) { return kV1[r][k * 2 + j]; }
    LCMA_HD static constexpr int w(int r, int i, int j) { return kW1[r][i * 2 + j]; }
};

template <> struct Scheme<2> {
    static constexpr int S = 4;
    static constexpr int R = 49;
    LCMA_HD static constexpr int u(int r, int i, int k) { return coef2(kU1, r, i, k); }
    LCMA_HD static constexpr int v(int r, int k, int j) { return coef2(kV1, r, k, j); }
    LCMA_HD static constexpr int w(int r, int i, int j) { return coef2(kW1, r, i, j); }
};

// Winograd's variant of the one-level scheme (rank 7, the same 2x2 split;
// a textbook description, not one of the pages'), written from its shared
// sums S1 = A21 + A22, S2 = S1 - A11, S3 = A11 - A21, S4 = A12 - S2 and
// T1 = B12 - B11, T2 = B22 - T1, T3 = B22 - B12, T4 = T2 - B21:
//   M1 = A11 B11, M2 = A12 B21, M3 = S4 B22, M4 = A22 T4, M5 = S1 T1,
//   M6 = S2 T2, M7 = S3 T3;
//   C11 = M1 + M2, C12 = M1 + M6 + M5 + M3, C21 = M1 + M6 + M7 - M4,
//   C22 = M1 + M6 + M7 + M5.
// Three products on each side take a single input block, and its output
// sums nest, which lets the unfused path's run schedule carry
// accumulators from product to product.
constexpr int8_t kUw[7][4] = {{1, 0, 0, 0}, {0, 1, 0, 0}, {1, 1, -1, -1}, {0, 0, 0, 1},
                              {0, 0, 1, 1}, {-1, 0, 1, 1}, {1, 0, -1, 0}};
constexpr int8_t kVw[7][4] = {{1, 0, 0, 0}, {0, 0, 1, 0}, {0, 0, 0, 1}, {1, -1, -1, 1},
                              {-1, 1, 0, 0}, {1, -1, 0, 1}, {0, -1, 0, 1}};
constexpr int8_t kWw[7][4] = {{1, 1, 1, 1}, {1, 0, 0, 0}, {0, 1, 0, 0}, {0, 0, -1, 0},
                              {0, 1, 0, 1}, {0, 1, 1, 1}, {0, 0, 1, 1}};

}  // namespace lcma
