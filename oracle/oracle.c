/*
 * oracle.c -- plain, slow, obviously-correct CPU oracle for half-precision
 * GEMM and for low-complexity (LCMA / Strassen-type) matrix multiplication.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file; only the tests, the smoke check and the CPU-baseline leg of
 * the benchmark do.  It shares no code, header, table or helper with the HIP
 * library.
 *
 * Sources (cited by page title and section):
 *   [FG]  "FalconGEMM: Surpassing Hardware Peaks with Lower-Complexity Matrix
 *         Multiplication" (HyperAI write-up of the talk).
 *         S1 = section "从 Strassen 出发" (starting from Strassen),
 *         S2 = section "从 LCMA 到 FalconGEMM" (from LCMA to FalconGEMM),
 *         S3 = section "从缓存重排到 Cost Model" (cache reordering, cost model,
 *              numerics).
 *   [CL2] "CUDA-L2: Surpassing cuBLAS Performance for Matrix Multiplication
 *         through Reinforcement Learning" (gist.science explanation),
 *         section "系统架构与训练" (validation against an FP32 CPU truth,
 *         exact match on binary inputs).
 *
 * Everything is fp64 unless a function says otherwise.  Half-precision
 * values (IEEE binary16 and bfloat16) are decoded exactly into fp64; fp64
 * products of two such values are exact.
 *
 * Parity pins for every function live in tests/test_oracle.py (brute force
 * in exact rational arithmetic, library routines, algebraic identities,
 * product counts).
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* Host threads the product loops use (timing the oracle on a given number of
 * cores; no effect on any result: each element's summation order is fixed). */
void oracle_set_threads(int n)
{
    if (n > 0)
        omp_set_num_threads(n);
}

int oracle_max_threads(void)
{
    return omp_get_max_threads();
}

/* ------------------------------------------------------------------------ */
/* Half-precision encodings, written from the format definitions.            */
/* binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits.        */
/* bfloat16: 1 sign bit, 8 exponent bits (bias 127), 7 fraction bits.        */
/* Rounding: round to nearest, ties to even (the IEEE default; the pages do  */
/* not name a mode), applied once to the exact fp64 value.                   */
/* ------------------------------------------------------------------------ */

/* Generic decoder for a format with `ebits` exponent and `fbits` fraction
 * bits: value = (-1)^s * 2^(e-bias) * (1 + f/2^fbits) for normal numbers,
 * (-1)^s * 2^(1-bias) * (f/2^fbits) for subnormals. */
static double decode_bits(uint32_t bits, int ebits, int fbits)
{
    const uint32_t fmask = (1u << fbits) - 1u;
    const uint32_t emask = (1u << ebits) - 1u;
    const int bias = (1 << (ebits - 1)) - 1;
    const uint32_t s = (bits >> (ebits + fbits)) & 1u;
    const uint32_t e = (bits >> fbits) & emask;
    const uint32_t f = bits & fmask;
    double v;
    if (e == emask) {
        v = (f == 0) ? INFINITY : NAN;
    } else if (e == 0) {
        v = ldexp((double)f, 1 - bias - fbits);
    } else {
        v = ldexp((double)(f | (1u << fbits)), (int)e - bias - fbits);
    }
    return s ? -v : v;
}

/* Generic RNE encoder.  The quantum (spacing of representable numbers) at
 * |x| is 2^(E - fbits) with E = max(floor(log2|x|), 1 - bias); dividing by
 * the quantum and rounding to the nearest integer (ties to even: rint in the
 * default rounding mode) gives the significand count.  Results beyond the
 * largest finite value become infinity. */
static uint32_t encode_bits(double x, int ebits, int fbits)
{
    const int bias = (1 << (ebits - 1)) - 1;
    const uint32_t emask = (1u << ebits) - 1u;
    const uint32_t sign = signbit(x) ? (1u << (ebits + fbits)) : 0u;
    if (isnan(x))
        return sign | (emask << fbits) | (1u << (fbits - 1));
    double a = fabs(x);
    if (isinf(a))
        return sign | (emask << fbits);
    if (a == 0.0)
        return sign;
    int e2;
    (void)frexp(a, &e2);          /* a = m * 2^e2, m in [0.5, 1) */
    int E = e2 - 1;               /* floor(log2 a) */
    if (E < 1 - bias)
        E = 1 - bias;             /* subnormal range shares the smallest quantum */
    double q = ldexp(1.0, E - fbits);
    double n = rint(a / q);       /* exact division by a power of two */
    /* n in [0, 2^(fbits+1)]; n == 2^(fbits+1) means rounding carried into
     * the next binade. */
    if (n >= ldexp(1.0, fbits + 1)) {
        n = n / 2.0;
        E += 1;
    }
    if (E > bias)                 /* above the largest finite binade */
        return sign | (emask << fbits);
    uint32_t ni = (uint32_t)n;
    if (ni < (1u << fbits))       /* subnormal (only possible when E == 1-bias) */
        return sign | ni;
    return sign | ((uint32_t)(E + bias) << fbits) | (ni - (1u << fbits));
}

double oracle_f16_to_f64(uint16_t h) { return decode_bits(h, 5, 10); }
double oracle_bf16_to_f64(uint16_t h) { return decode_bits(h, 8, 7); }
uint16_t oracle_f64_to_f16(double x) { return (uint16_t)encode_bits(x, 5, 10); }
uint16_t oracle_f64_to_bf16(double x) { return (uint16_t)encode_bits(x, 8, 7); }

/* dtype: 0 = binary16, 1 = bfloat16. */
void oracle_encode(int dtype, const double* x, uint16_t* out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = dtype == 0 ? oracle_f64_to_f16(x[i]) : oracle_f64_to_bf16(x[i]);
}

void oracle_decode(int dtype, const uint16_t* h, double* out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = dtype == 0 ? oracle_f16_to_f64(h[i]) : oracle_bf16_to_f64(h[i]);
}

/* Value of x after one RNE rounding to the dtype (decode(encode(x))). */
static double round_to(int dtype, double x)
{
    return dtype == 0 ? oracle_f16_to_f64(oracle_f64_to_f16(x))
                      : oracle_bf16_to_f64(oracle_f64_to_bf16(x));
}

/* ------------------------------------------------------------------------ */
/* Classic product: C[i][j] = sum_{k=0}^{K-1} A[i][k] * B[k][j], row-major,  */
/* accumulated in fp64 with k ascending for every element (the definition   */
/* of the matrix product; [CL2] validates against exactly such a CPU truth). */
/* The loop order i-k-j visits, for each element, the k terms in ascending  */
/* order, so the per-element summation order is that of the naive triple     */
/* loop.  Rows are independent and split across OpenMP threads.              */
/* ------------------------------------------------------------------------ */
void oracle_gemm_f64(int64_t M, int64_t N, int64_t K,
                     const double* A, int64_t lda,
                     const double* B, int64_t ldb,
                     double* C, int64_t ldc)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < M; ++i) {
        double* c = C + i * ldc;
        for (int64_t j = 0; j < N; ++j)
            c[j] = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            const double a = A[i * lda + k];
            const double* b = B + k * ldb;
            for (int64_t j = 0; j < N; ++j)
                c[j] += a * b[j];
        }
    }
}

/* Row slice of the classic product: rows [r0, r1) only (used to time and to
 * check very large shapes on a bounded sample). */
void oracle_gemm_rows_f64(int64_t r0, int64_t r1, int64_t N, int64_t K,
                          const double* A, int64_t lda,
                          const double* B, int64_t ldb,
                          double* C, int64_t ldc)
{
    oracle_gemm_f64(r1 - r0, N, K, A + r0 * lda, lda, B, ldb, C, ldc);
}

/* ------------------------------------------------------------------------ */
/* LCMA descriptors ([FG] S1: an LCMA states which sub-blocks of the inputs  */
/* are combined, how many block products are run, and how the products are  */
/* combined into the output).                                                */
/*                                                                           */
/* A is split into ms x ks blocks, B into ks x ns, C into ms x ns.  For      */
/* product r (0-based):                                                      */
/*   Ahat_r = sum_{i,k} U[r][i*ks+k] * A_{ik}                                */
/*   Bhat_r = sum_{k,j} V[r][k*ns+j] * B_{kj}                                */
/*   H_r    = Ahat_r * Bhat_r                                                */
/*   C_{ij} = sum_r W[r][i*ns+j] * H_r                                       */
/* ------------------------------------------------------------------------ */

/* Strassen's 1969 scheme for a 2x2 block product with 7 products ([FG] S1:
 * 8 block products become 7).  Block order within each table row is
 * [11, 12, 21, 22].  The products are
 *   P1 = (A11 + A22)(B11 + B22)    P2 = (A21 + A22) B11
 *   P3 = A11 (B12 - B22)           P4 = A22 (B21 - B11)
 *   P5 = (A11 + A12) B22           P6 = (A21 - A11)(B11 + B12)
 *   P7 = (A12 - A22)(B21 + B22)
 * and C11 = P1 + P4 - P5 + P7, C12 = P3 + P5, C21 = P2 + P4,
 *     C22 = P1 - P2 + P3 + P6. */
static const int8_t STRASSEN_U[7][4] = {
    {1, 0, 0, 1}, {0, 0, 1, 1}, {1, 0, 0, 0}, {0, 0, 0, 1},
    {1, 1, 0, 0}, {-1, 0, 1, 0}, {0, 1, 0, -1}};
static const int8_t STRASSEN_V[7][4] = {
    {1, 0, 0, 1}, {1, 0, 0, 0}, {0, 1, 0, -1}, {-1, 0, 1, 0},
    {0, 0, 0, 1}, {1, 1, 0, 0}, {0, 0, 1, 1}};
static const int8_t STRASSEN_W[7][4] = {
    {1, 0, 0, 1}, {0, 0, 1, -1}, {0, 1, 0, 1}, {1, 0, 1, 0},
    {-1, 1, 0, 0}, {0, 0, 0, 1}, {1, 0, 0, 0}};

/* Writes the one-level Strassen tables (rank 7, 2x2x2) into caller buffers
 * of at least 28 entries each.  Returns the rank. */
int oracle_strassen_tables(int8_t* U, int8_t* V, int8_t* W)
{
    memcpy(U, STRASSEN_U, sizeof STRASSEN_U);
    memcpy(V, STRASSEN_V, sizeof STRASSEN_V);
    memcpy(W, STRASSEN_W, sizeof STRASSEN_W);
    return 7;
}

/* The plain block product as an LCMA (rank ms*ks*ns): product (i,k,j)
 * takes A_ik and B_kj and adds into C_ij.  Used to count the 8 (resp. 64)
 * block products of the classic scheme against Strassen's 7 (resp. 49). */
int oracle_naive_tables(int ms, int ks, int ns, int8_t* U, int8_t* V, int8_t* W)
{
    int r = 0;
    const int R = ms * ks * ns;
    memset(U, 0, (size_t)R * ms * ks);
    memset(V, 0, (size_t)R * ks * ns);
    memset(W, 0, (size_t)R * ms * ns);
    for (int i = 0; i < ms; ++i)
        for (int k = 0; k < ks; ++k)
            for (int j = 0; j < ns; ++j, ++r) {
                U[r * ms * ks + i * ks + k] = 1;
                V[r * ks * ns + k * ns + j] = 1;
                W[r * ms * ns + i * ns + j] = 1;
            }
    return R;
}

/* Two-level scheme as one level of the Kronecker product of two schemes
 * ([FG] S1: applying Strassen recursively turns 64 block products of a 4x4
 * block product into 49).  Blocks of the composite split are indexed
 * outer-major: composite block row i = i1*ms2 + i2 where i1 is the block
 * row at the outer level and i2 the block row inside that block (same for
 * columns); product index r = r1*R2 + r2.  Output buffers must hold
 * R1*R2 * (ms1*ms2)*(ks1*ks2) (etc.) entries. */
void oracle_kron_tables(int ms1, int ks1, int ns1, int R1,
                        const int8_t* U1, const int8_t* V1, const int8_t* W1,
                        int ms2, int ks2, int ns2, int R2,
                        const int8_t* U2, const int8_t* V2, const int8_t* W2,
                        int8_t* U, int8_t* V, int8_t* W)
{
    const int ms = ms1 * ms2, ks = ks1 * ks2, ns = ns1 * ns2;
    for (int r1 = 0; r1 < R1; ++r1)
        for (int r2 = 0; r2 < R2; ++r2) {
            const int r = r1 * R2 + r2;
            for (int i1 = 0; i1 < ms1; ++i1)
                for (int i2 = 0; i2 < ms2; ++i2)
                    for (int k1 = 0; k1 < ks1; ++k1)
                        for (int k2 = 0; k2 < ks2; ++k2)
                            U[r * ms * ks + (i1 * ms2 + i2) * ks + (k1 * ks2 + k2)] =
                                (int8_t)(U1[r1 * ms1 * ks1 + i1 * ks1 + k1] *
                                         U2[r2 * ms2 * ks2 + i2 * ks2 + k2]);
            for (int k1 = 0; k1 < ks1; ++k1)
                for (int k2 = 0; k2 < ks2; ++k2)
                    for (int j1 = 0; j1 < ns1; ++j1)
                        for (int j2 = 0; j2 < ns2; ++j2)
                            V[r * ks * ns + (k1 * ks2 + k2) * ns + (j1 * ns2 + j2)] =
                                (int8_t)(V1[r1 * ks1 * ns1 + k1 * ns1 + j1] *
                                         V2[r2 * ks2 * ns2 + k2 * ns2 + j2]);
            for (int i1 = 0; i1 < ms1; ++i1)
                for (int i2 = 0; i2 < ms2; ++i2)
                    for (int j1 = 0; j1 < ns1; ++j1)
                        for (int j2 = 0; j2 < ns2; ++j2)
                            W[r * ms * ns + (i1 * ms2 + i2) * ns + (j1 * ns2 + j2)] =
                                (int8_t)(W1[r1 * ms1 * ns1 + i1 * ns1 + j1] *
                                         W2[r2 * ms2 * ns2 + i2 * ns2 + j2]);
        }
}

/* Brent's identity: the scheme computes the block product for every input
 * iff, for all block indices,
 *   sum_r U[r][i,k] * V[r][k',j] * W[r][i',j'] = [k==k'] [i==i'] [j==j'].
 * (Expanding C_{i'j'} = sum_r W[r][i'j'] (sum U A)(sum V B) and matching the
 * coefficient of A_{ik} B_{k'j} against the definition of the product.)
 * Exact integer arithmetic.  Returns the number of index tuples where the
 * identity fails (0 = valid scheme). */
int64_t oracle_brent_violations(int ms, int ks, int ns, int R,
                                const int8_t* U, const int8_t* V, const int8_t* W)
{
    int64_t bad = 0;
    for (int i = 0; i < ms; ++i)
        for (int k = 0; k < ks; ++k)
            for (int k2 = 0; k2 < ks; ++k2)
                for (int j = 0; j < ns; ++j)
                    for (int i2 = 0; i2 < ms; ++i2)
                        for (int j2 = 0; j2 < ns; ++j2) {
                            int64_t s = 0;
                            for (int r = 0; r < R; ++r)
                                s += (int64_t)U[r * ms * ks + i * ks + k] *
                                     V[r * ks * ns + k2 * ns + j] *
                                     W[r * ms * ns + i2 * ns + j2];
                            const int64_t want = (k == k2 && i == i2 && j == j2) ? 1 : 0;
                            if (s != want)
                                ++bad;
                        }
    return bad;
}

/* ------------------------------------------------------------------------ */
/* Scalar LCMA evaluator ([FG] S1 and S2): combine the input blocks, run R   */
/* block products (recursively for levels > 1), combine the products into C. */
/*                                                                           */
/* round_dtype < 0: every step exact in fp64 (for small-integer inputs the   */
/*   result is exact; Strassen is algebraically the classic product, [FG]    */
/*   S1).                                                                    */
/* round_dtype = 0 / 1: the combined operands Ahat, Bhat are rounded once    */
/*   (RNE) to binary16 / bfloat16 before their product, as they are when the  */
/*   combined operands feed a half-precision matrix unit ([FG] S2: the       */
/*   combined inputs are the operands of the batched GEMMs; [FG] S3: the     */
/*   casts, not the fp32 accumulation, are the significant error source).   */
/*   Products and the output combination stay fp64 (standing in for the      */
/*   fp32 on-chip accumulation, [FG] S3); C is left unrounded.               */
/*                                                                           */
/* Block sizes must divide exactly: M % ms^levels == 0 etc.  *count is       */
/* incremented once per base-case (level 0) block product.                   */
/* Returns 0 on success, -1 on a shape that does not split evenly, -2 when   */
/* out of memory.                                                            */
/* ------------------------------------------------------------------------ */
static int lcma_rec(int ms, int ks, int ns, int R,
                    const int8_t* U, const int8_t* V, const int8_t* W,
                    int levels, int64_t M, int64_t N, int64_t K,
                    const double* A, int64_t lda, const double* B, int64_t ldb,
                    double* C, int64_t ldc, int round_dtype, int64_t* count)
{
    if (levels == 0) {
        oracle_gemm_f64(M, N, K, A, lda, B, ldb, C, ldc);
        if (count)
            ++*count;
        return 0;
    }
    if (M % ms || K % ks || N % ns)
        return -1;
    const int64_t bm = M / ms, bk = K / ks, bn = N / ns;
    double* Ah = (double*)malloc(sizeof(double) * (size_t)(bm * bk > 0 ? bm * bk : 1));
    double* Bh = (double*)malloc(sizeof(double) * (size_t)(bk * bn > 0 ? bk * bn : 1));
    double* H = (double*)malloc(sizeof(double) * (size_t)(bm * bn > 0 ? bm * bn : 1));
    if (!Ah || !Bh || !H) {
        free(Ah); free(Bh); free(H);
        return -2;
    }
    for (int64_t i = 0; i < M; ++i)
        for (int64_t j = 0; j < N; ++j)
            C[i * ldc + j] = 0.0;
    int rc = 0;
    for (int r = 0; r < R && rc == 0; ++r) {
        /* Ahat_r = sum_{i,k} U[r][i*ks+k] * A_ik */
        for (int64_t x = 0; x < bm * bk; ++x)
            Ah[x] = 0.0;
        for (int bi = 0; bi < ms; ++bi)
            for (int bkk = 0; bkk < ks; ++bkk) {
                const int u = U[r * ms * ks + bi * ks + bkk];
                if (!u)
                    continue;
                for (int64_t i = 0; i < bm; ++i)
                    for (int64_t k = 0; k < bk; ++k)
                        Ah[i * bk + k] += u * A[(bi * bm + i) * lda + bkk * bk + k];
            }
        /* Bhat_r = sum_{k,j} V[r][k*ns+j] * B_kj */
        for (int64_t x = 0; x < bk * bn; ++x)
            Bh[x] = 0.0;
        for (int bkk = 0; bkk < ks; ++bkk)
            for (int bj = 0; bj < ns; ++bj) {
                const int v = V[r * ks * ns + bkk * ns + bj];
                if (!v)
                    continue;
                for (int64_t k = 0; k < bk; ++k)
                    for (int64_t j = 0; j < bn; ++j)
                        Bh[k * bn + j] += v * B[(bkk * bk + k) * ldb + bj * bn + j];
            }
        if (round_dtype >= 0) {
            for (int64_t x = 0; x < bm * bk; ++x)
                Ah[x] = round_to(round_dtype, Ah[x]);
            for (int64_t x = 0; x < bk * bn; ++x)
                Bh[x] = round_to(round_dtype, Bh[x]);
        }
        /* H_r = Ahat_r * Bhat_r (recursively) */
        rc = lcma_rec(ms, ks, ns, R, U, V, W, levels - 1, bm, bn, bk,
                      Ah, bk, Bh, bn, H, bn, round_dtype, count);
        /* C_ij += W[r][i*ns+j] * H_r */
        for (int bi = 0; bi < ms && rc == 0; ++bi)
            for (int bj = 0; bj < ns; ++bj) {
                const int w = W[r * ms * ns + bi * ns + bj];
                if (!w)
                    continue;
                for (int64_t i = 0; i < bm; ++i)
                    for (int64_t j = 0; j < bn; ++j)
                        C[(bi * bm + i) * ldc + bj * bn + j] += w * H[i * bn + j];
            }
    }
    free(Ah);
    free(Bh);
    free(H);
    return rc;
}

int oracle_lcma_eval(int ms, int ks, int ns, int R,
                     const int8_t* U, const int8_t* V, const int8_t* W,
                     int levels, int64_t M, int64_t N, int64_t K,
                     const double* A, int64_t lda, const double* B, int64_t ldb,
                     double* C, int64_t ldc, int round_dtype, int64_t* count)
{
    if (levels < 0 || ms < 1 || ks < 1 || ns < 1 || R < 1)
        return -1;
    if (count)
        *count = 0;
    return lcma_rec(ms, ks, ns, R, U, V, W, levels, M, N, K, A, lda, B, ldb,
                    C, ldc, round_dtype, count);
}

/* Combined operand of one product, exact sum then (optionally) one RNE
 * rounding: out = round(sum_{i,k} coef[i*cs+k] * X_ik) where X is split into
 * rs x cs blocks of size (rows/rs) x (cols/cs).  Used to check a combine
 * pre-pass block by block. */
int oracle_combine_block(int rs, int cs, const int8_t* coef,
                         int64_t rows, int64_t cols, const double* X, int64_t ldx,
                         double* out, int round_dtype)
{
    if (rows % rs || cols % cs)
        return -1;
    const int64_t br = rows / rs, bc = cols / cs;
    for (int64_t i = 0; i < br; ++i)
        for (int64_t j = 0; j < bc; ++j) {
            double s = 0.0;
            for (int a = 0; a < rs; ++a)
                for (int b = 0; b < cs; ++b) {
                    const int c = coef[a * cs + b];
                    if (c)
                        s += c * X[(a * br + i) * ldx + b * bc + j];
                }
            out[i * bc + j] = round_dtype >= 0 ? round_to(round_dtype, s) : s;
        }
    return 0;
}
