/*
 * lcma.h -- C ABI of the MI355X (gfx950) half-precision GEMM library:
 * a classic MFMA GEMM and low-complexity (LCMA / Strassen-type) products.
 *
 * Operation (all entry points): C = A * B, C overwritten (no alpha/beta).
 *   A: M x K, B: K x N, C: M x N, row-major with leading dimensions
 *   lda >= K, ldb >= N, ldc >= N (elements).  A, B and C share one storage
 *   type (binary16 or bfloat16).  Products accumulate in fp32 and C is
 *   rounded once, to nearest even, to the storage type.  NaN/Inf propagate
 *   as IEEE arithmetic makes them; nothing is checked.
 *
 * Sources (cited by page title and section):
 *   [FG] "FalconGEMM: Surpassing Hardware Peaks with Lower-Complexity Matrix
 *        Multiplication" (HyperAI write-up of the talk):
 *        "从 Strassen 出发" -- Strassen 8 -> 7, two levels 64 -> 49, the LCMA
 *            description (which input blocks are combined, how many
 *            products, how products combine into C);
 *        "从 LCMA 到 FalconGEMM" -- combine A/B, 7 batched products, combine
 *            H; spatial groups on one compute unit with on-chip accumulation
 *            into C; split of a group over two compute units; reordering for
 *            L2 locality; persistent kernel;
 *        "从缓存重排到 Cost Model" -- roofline-like cost model that picks the
 *            algorithm per shape; fp32 on-chip combination with one final
 *            cast.
 *   [KP] "Kernel 与性能" notes page, section "Roofline" (I = FLOPs / bytes,
 *        F <= min(F_max, I * B_max)).
 *   [CL2] "CUDA-L2: Surpassing cuBLAS Performance for Matrix Multiplication
 *        through Reinforcement Learning", section "核心贡献与发现的技术" --
 *            zero-padding of dimensions that do not divide the blocking.
 *
 * Memory ownership: the caller owns A, B, C and the workspace (device
 * memory).  The library never allocates device memory.  A plan owns only
 * host memory.  A plan is immutable after lcma_plan() and may be used from
 * several threads, each with its own workspace.
 *
 * Streams: launching calls only enqueue work on `stream` (a hipStream_t; 0
 * is the null stream) and never synchronise.  Launch failures are reported
 * as LCMA_E_HIP (from hipGetLastError).
 *
 * Errors: every call returns an lcma_status; no exception crosses the ABI.
 * All argument checks run before any device call, so invalid calls never
 * touch the GPU.
 */
#ifndef LCMA_H_
#define LCMA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { LCMA_F16 = 0, LCMA_BF16 = 1 } lcma_dtype;

typedef enum {
    LCMA_ALGO_AUTO = 0,     /* cost model picks */
    LCMA_ALGO_CLASSIC = 1,  /* one tiled MFMA GEMM */
    LCMA_ALGO_L1 = 2,       /* one-level Strassen: 7 block products */
    LCMA_ALGO_L2 = 3        /* two-level Strassen: 49 block products */
} lcma_algo;

typedef enum {
    LCMA_OK = 0,
    LCMA_E_INVALID = 1,        /* bad argument (negative size, null pointer, ld too small, ...) */
    LCMA_E_UNSUPPORTED = 2,    /* valid but not implemented (alignment, forced algo on an unsplittable shape) */
    LCMA_E_BAD_DESCRIPTOR = 3, /* descriptor fails Brent's identity or is malformed */
    LCMA_E_WORKSPACE = 4,      /* workspace missing or smaller than lcma_plan_info() reports */
    LCMA_E_HIP = 5,            /* a HIP runtime call failed */
    LCMA_E_NOMEM = 6           /* host allocation failed */
} lcma_status;

/* How a tail group may be split over two compute units ([FG] "从 LCMA 到
 * FalconGEMM": a group is split over two compute units when needed). */
typedef enum {
    LCMA_SPLIT_AUTO = 0,  /* split the last, partial round of groups when that shortens it */
    LCMA_SPLIT_NONE = 1,  /* never split (nor split K in classic plans) */
    LCMA_SPLIT_ALL = 2    /* split every group (testing the fix-up path) */
} lcma_split;

/* Order in which the persistent LCMA kernel deals output groups and split
 * pieces to compute units ([FG] "从 LCMA 到 FalconGEMM": tiles of one product
 * type run together, which keeps the cache hit rate and the clock up). */
typedef enum {
    LCMA_ORDER_AUTO = 0,  /* locality order: the compute units of one XCD (own L2) take a compact
                             block of output groups; the two pieces of a split group go to adjacent
                             workers, so even XCDs run first halves and odd XCDs second halves */
    LCMA_ORDER_PLAIN = 1  /* row-major groups; first halves of split groups on workers 0..T-1,
                             second halves on T..2T-1 (every XCD mixes both halves): the baseline
                             the locality order is measured against */
} lcma_order;

/* How the combined operands reach the fused kernel, and (two levels) where
 * the products of one output coordinate accumulate. */
typedef enum {
    LCMA_COMBINE_AUTO = 0,    /* one level of a built-in scheme: PREPASS, or UNFUSED when the cost model
                                 estimates it at least 2% faster (large blocks) and split and order are left
                                 at their defaults; two levels: PREPASS */
    LCMA_COMBINE_PREPASS = 1, /* a separate bandwidth-bound pass writes each combined operand to the workspace.
                                 Two levels: the 7 inner products of each outer product run fused as one
                                 level (their 4 outputs accumulate on chip), one launch per outer product,
                                 and each launch folds W1[r1][i1,j1] * (its inner outputs) into fp32 output
                                 blocks in the workspace; the last contributor to an output rounds it into C */
    LCMA_COMBINE_AT_LOAD = 2, /* one level of the built-in scheme: no pre-pass; the group kernel loads the one
                                 or two input blocks of each operand, adds them in fp32 (binary16: one packed
                                 add, the same single rounding) and rounds once to the operand type while
                                 staging each k-tile (both blocks go to LDS, then all threads fold them in
                                 place), so no combined operand is written and the workspace is empty.
                                 Operands keep the storage type: with LCMA_ALGO_L2, a generic description
                                 or bf16_ops_f16 = 1 on bfloat16 inputs, lcma_plan_ex returns
                                 LCMA_E_UNSUPPORTED.  The workspace holds only the split fix-up partials and
                                 counters (none without a split).  lcma_prepass does nothing and lcma_fused
                                 runs the whole product (it clears the counters first); lcma_plan_operand is
                                 LCMA_E_INVALID */
    LCMA_COMBINE_UNFUSED = 3, /* one level only: every combined operand is written; each product's epilogue adds
                                 W[r][i,j] * H_r into fp32 output blocks in the workspace (H_r is never stored)
                                 and the last contributor to a block rounds it into C.  Blocks with enough
                                 256 x 256 positions for every compute unit run all products in one persistent
                                 launch (each position owned by one workgroup; on whole tiles the pre-pass
                                 writes the A operands tile-packed, see lcma_plan_operand); smaller ones run
                                 one launch per product.  The path for descriptions that are not a built-in scheme, and
                                 the unfused form of the built-in one */
    LCMA_COMBINE_L2_ON_CHIP = 4 /* two levels only (pre-pass as above): all 49 products of an output coordinate
                                 run in one group on one workgroup and the 16 outputs accumulate on chip.  The
                                 register file holds 17 accumulator tiles only at 64 x 64 group tiles, so this
                                 runs far below the default; kept as the literal form of the fused group */
} lcma_combine;

/*
 * An LCMA description ([FG] "从 Strassen 出发").  A is split into ms x ks
 * blocks, B into ks x ns, C into ms x ns; product r (0-based) is
 *   Ahat_r = sum_{i,k} U[r*ms*ks + i*ks + k] * A_ik
 *   Bhat_r = sum_{k,j} V[r*ks*ns + k*ns + j] * B_kj
 *   H_r    = Ahat_r * Bhat_r
 *   C_ij   = sum_r W[r*ms*ns + i*ns + j] * H_r
 * Tables are row-major int8, rank rows each.  Block (i, k) of a two-level
 * split uses i = 2*i_outer + i_inner (outer-major).
 */
typedef struct {
    int32_t ms, ks, ns, rank;
    const int8_t* U;
    const int8_t* V;
    const int8_t* W;
} lcma_desc;

/* Optional planning knobs; pass NULL to lcma_plan_ex for the defaults
 * (all-zero fields mean "default"). */
typedef struct {
    lcma_split split;
    lcma_combine combine;
    int32_t bf16_ops_f16;   /* bfloat16 inputs only: 1 = combined operands are rounded to
                               binary16 (3 more fraction bits; requires |combinations| < 65504),
                               0 = default (binary16 operands for two-level, bfloat16 for one-level),
                               -1 = always bfloat16 operands */
    int32_t num_cus;        /* 0 = query the current device; >0 = plan for that many compute units
                               (host-only planning and tests) */
    double peak_tflops;     /* 0 = 2500 (published dense fp16/bf16 MFMA peak of MI355X) */
    double hbm_gbps;        /* 0 = 8000 */
    double classic_eff;     /* fraction of peak_tflops the classic kernel sustains when compute-bound;
                               0 = 0.52 (measured on MI355X at 4096^3 .. 16384^3) */
    double fused_eff;       /* the same for the fused group kernel (both levels);
                               0 = 0.31 for one level and for two levels with the outer level in
                               memory, 0.037 for LCMA_COMBINE_L2_ON_CHIP, 0.13 for
                               LCMA_COMBINE_AT_LOAD (measured) */
    lcma_order order;       /* persistent fused kernel's work order (LCMA_ORDER_AUTO by default) */
    int32_t accuracy_optin; /* 1 = accept a forced algorithm whose error exceeds 4x the classic kernel's
                               on the same inputs (see "Accuracy" at lcma_plan); 0 = refuse it with
                               LCMA_E_UNSUPPORTED */
} lcma_options;

typedef struct lcma_plan_s* lcma_plan_t;

/* Built-in Strassen schemes: levels = 1 (2x2x2, rank 7) or 2 (4x4x4, rank
 * 49, the Kronecker square of the one-level scheme).  The tables are static
 * storage owned by the library (do not free).
 * Errors: LCMA_E_INVALID (levels not 1 or 2, out == NULL).
 * Source: [FG] "从 Strassen 出发" (Strassen's 7 products of a 2x2 block split;
 * applied twice, 49 products instead of 64; the U/V/W description). */
lcma_status lcma_desc_builtin(int32_t levels, lcma_desc* out);

/* Winograd's variant of the one-level scheme (2x2x2, rank 7; a textbook
 * description, not from the pages), for the unfused path that runs any valid
 * description: M1 = A11 B11, M2 = A12 B21, M3 = (A11 + A12 - A21 - A22) B22,
 * M4 = A22 (B11 - B12 - B21 + B22), M5 = (A21 + A22)(B12 - B11),
 * M6 = (A21 + A22 - A11)(B11 - B12 + B22), M7 = (A11 - A21)(B22 - B12);
 * C11 = M1 + M2, C12 = M1 + M3 + M5 + M6, C21 = M1 - M4 + M6 + M7,
 * C22 = M1 + M5 + M6 + M7.  Its output sums nest, so the run schedule of a
 * persistent unfused plan moves 32 fp32 fold bytes per output block element
 * against Strassen's 56 (see lcma_plan_runs).  Accuracy: with operands of
 * the input type its normwise error is about 3.8x that of the classic
 * product (Strassen's about 2.8x), within the 4x gate; bfloat16 inputs with
 * binary16 operands (bf16_ops_f16 = 1) about 1.03x.  Static storage owned
 * by the library.  Errors: LCMA_E_INVALID (out == NULL).
 * Source: [FG] "从 LCMA 到 FalconGEMM" (a scheme is its U/V/W description;
 * the same kernels run any of them). */
lcma_status lcma_desc_winograd(lcma_desc* out);

/* Checks a description: positive sizes, coefficients in [-8, 8], and
 * Brent's identity sum_r U[r][i,k] V[r][k',j] W[r][i',j'] =
 * [k==k'][i==i'][j==j'] (exact integers).  LCMA_OK or LCMA_E_BAD_DESCRIPTOR
 * (LCMA_E_INVALID for NULL).
 * Source: [FG] "从 Strassen 出发" (a scheme is a set of coefficient tables that
 * must reproduce the exact product); the identity itself is the textbook
 * condition for such tables. */
lcma_status lcma_desc_validate(const lcma_desc* desc);

/* Plans C = A * B for an M x N x K product of storage type dt.
 * Source: [FG] "从缓存重排到 Cost Model" (a roofline-like cost model from
 * FLOPs, bytes and the device's peak and bandwidth picks the algorithm per
 * shape; it aims to pick, not to predict) and [KP] "Roofline"; the product
 * forms come from [FG] "从 LCMA 到 FalconGEMM".
 *   desc:  NULL = built-in Strassen schemes; otherwise validated
 *          (LCMA_E_BAD_DESCRIPTOR) and deep-copied.  A description that is
 *          not one of the built-in schemes runs one level of itself through
 *          the unfused path (LCMA_COMBINE_UNFUSED) when LCMA_ALGO_L1 is
 *          forced (up to 64 products and 16 blocks per side; larger ones are
 *          LCMA_E_UNSUPPORTED); LCMA_ALGO_AUTO picks classic for it, and
 *          LCMA_ALGO_L2 is LCMA_E_UNSUPPORTED.  One level of a description
 *          (ms, ks, ns) needs M, K, N divisible by ms, ks, ns.
 *   force: LCMA_ALGO_AUTO lets the roofline cost model pick among the
 *          admissible algorithms (ties go to classic); shapes that do not
 *          split evenly are left to classic.
 *          A forced L1/L2 of the built-in scheme on a shape that does not
 *          split evenly is zero-padded: M, N, K are rounded up to multiples
 *          of 32 (L1) or 64 (L2), A and B are copied into zero-padded
 *          buffers in the workspace, the padded product runs there and its
 *          M x N window is copied into C (any alignment and leading
 *          dimensions).  Other forced combinations that do not fit return
 *          LCMA_E_UNSUPPORTED.
 * Accuracy: an LCMA result may carry at most 4x the error of the classic
 * kernel on the same inputs (e_nw = ||C - C_ref||_F / (||A||_F ||B||_F)).
 * Measured by evaluating the schemes with rounded combined operands in fp64
 * (uniform / normal inputs, 512..1024 per side): one level 2.8x; two levels
 * with combined operands of the input type 5.8-5.9x; two levels of bfloat16
 * inputs with binary16 operands (the default) 1.1x.  So LCMA_ALGO_L2 on
 * binary16 inputs, and on bfloat16 inputs with bf16_ops_f16 = -1, returns
 * LCMA_E_UNSUPPORTED unless opts->accuracy_optin = 1 (AUTO never picks them).
 * Two levels with binary16 operands need every combination of up to four
 * bfloat16 input entries to stay below 65520 in magnitude: a larger sum
 * rounds to +-Inf, which then propagates into C as IEEE arithmetic makes it
 * (nothing is checked on the device).
 * Leading dimensions: every buffer the plan addresses (the inputs, the
 * combined operands and, for padded plans, the zero-padded copies) must have
 * a leading dimension below 2^21 elements; a plan that would need a larger
 * one returns LCMA_E_UNSUPPORTED (AUTO falls back to classic when it can).
 * Sizes: M, N, K >= 0 (negative: LCMA_E_INVALID).  Zero-sized products are
 * valid (K = 0 writes C = 0).  Performs no device work; the only HIP call
 * is a device-property query when opts->num_cus is 0.
 * On success *out receives a plan to free with lcma_plan_destroy. */
lcma_status lcma_plan(int64_t M, int64_t N, int64_t K, lcma_dtype dt,
                      const lcma_desc* desc, lcma_algo force, lcma_plan_t* out);
lcma_status lcma_plan_ex(int64_t M, int64_t N, int64_t K, lcma_dtype dt,
                         const lcma_desc* desc, lcma_algo force,
                         const lcma_options* opts, lcma_plan_t* out);

/* What the plan chose: algorithm, workspace bytes the caller must pass to
 * lcma_gemm, and the cost model's time estimate in seconds (any output
 * pointer may be NULL).  LCMA_E_INVALID for a NULL plan.
 * Source: [FG] "从缓存重排到 Cost Model" (the algorithm picked per shape). */
lcma_status lcma_plan_info(lcma_plan_t plan, lcma_algo* chosen, size_t* workspace_bytes,
                           double* est_seconds);

/* Cost-model estimate (seconds) the plan computed for one algorithm;
 * a negative value means the algorithm was not admissible for the shape.
 * Per kernel the model takes max(F / (eta * peak * q), B / (0.8 * bw),
 * F / (I_tile * bw_L2 * q)) + 4 us, with bw_L2 = 8 * 2048 B * 2.4 GHz,
 * I_tile = BM * BN / (BM + BN), q the wave-quantisation efficiency and eta
 * the kernel's sustained fraction of the peak.
 * Source: [FG] "从缓存重排到 Cost Model"; [KP] "Roofline". */
lcma_status lcma_plan_estimate(lcma_plan_t plan, lcma_algo algo, double* est_seconds);

/* Runs the planned product on `stream`.  A, B, C: device pointers as above.
 * Source: [FG] "从 LCMA 到 FalconGEMM" (combine A/B, the block products,
 * combine H accumulated in fp32 on chip, one final cast) for LCMA plans;
 * [CL2] "核心贡献与发现的技术" (staged, coalesced tile loads) for classic
 * plans.
 * Fast path: pointers 16-byte aligned and lda, ldb multiples of 8; classic
 * and padded LCMA plans accept any alignment (slower element loads, resp.
 * element-wise padding copies), other LCMA plans require it
 * (LCMA_E_UNSUPPORTED otherwise).  workspace: device memory of at least
 * the planned size (may be NULL when that size is 0), 256-byte aligned; it
 * must not be used by two calls that can overlap.  Classic plans of up to
 * 64 rows whose K is long against their number of 128-column strips
 * (N <= 4096: K >= 2048; N <= 8192: K >= 4096; wider N: 33..64 rows with
 * K >= 8192, or K >= 4096 when N > 16384, and 17..32 rows with K >= 12288)
 * have a workspace: 2, 4 or 8
 * workgroups per strip each take a part of K and write an fp32 partial tile
 * (the rows below M of 32 or 64 x 128) there, and a second kernel on the
 * same stream adds the partials in a fixed order and rounds into C ([KP]
 * "GEMM 形状": such products stream B; the split cuts the bytes of A each
 * workgroup re-reads and fills the chip when the strips are few).  The
 * workspace needs no clearing and keeps nothing between calls.  Classic
 * plans beyond 64 rows whose 128 x 128 tiles fill at most half the compute
 * units, with K >= 4096, split K the same way into S fp32 planes of M x N
 * (S = 2, 4 or 8); multi-round plans on 256 x 256 tiles split the K of the
 * last round's T tiles (up to 64) into S compact 256 x 256 fp32 tiles each
 * (S * T * 256 KiB, at most 64 MiB).  LCMA_SPLIT_NONE in lcma_options turns
 * every K split off (classic plans then need no workspace).  Without 16-byte
 * alignment the unsplit kernels run instead.
 * Errors: LCMA_E_INVALID (NULL pointers with nonzero sizes, ld too small),
 * LCMA_E_WORKSPACE, LCMA_E_UNSUPPORTED, LCMA_E_HIP. */
lcma_status lcma_gemm(lcma_plan_t plan, const void* A, int64_t lda, const void* B, int64_t ldb,
                      void* C, int64_t ldc, void* workspace, size_t workspace_bytes,
                      void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): lcma_gemm
 * with the workspace taken from a static device array of LCMA_SCRATCH_BYTES
 * that the library holds on each GPU it runs on until the process ends.
 * The first call on a device looks the array's address up (once per device,
 * with that device current); no call allocates or frees device memory.
 * The caller still passes A, B and C.  Every call on one GPU shares that
 * GPU's array and finds the last call's contents there (the kernels clear
 * what must start at zero), so calls that can overlap on one GPU -- on two
 * streams, or from two threads -- race and must not be issued.
 * Errors: LCMA_E_WORKSPACE when the plan's workspace (lcma_plan_info) is
 * larger than LCMA_SCRATCH_BYTES; LCMA_E_HIP if the address lookup fails;
 * otherwise those of lcma_gemm. */
#define LCMA_SCRATCH_BYTES ((size_t)64 << 20)
lcma_status lcma_gemm_noalloc(lcma_plan_t plan, const void* A, int64_t lda, const void* B, int64_t ldb,
                              void* C, int64_t ldc, void* stream);

/* Source: [FG] "从 LCMA 到 FalconGEMM" (the combine-A/B pass and the
 * persistent group kernel as two stages of the pipeline).
 * The two halves of lcma_gemm for an LCMA plan using the pre-pass, exposed
 * so each kernel can be checked and timed on its own: lcma_prepass writes
 * the combined operands (and clears the split counters) in the workspace;
 * lcma_fused then runs the persistent group kernel from them.  Calling
 * lcma_prepass then lcma_fused on one stream equals lcma_gemm.  Unfused
 * plans: lcma_prepass writes every combined operand, lcma_fused runs the
 * products and their folds.  Padded plans: lcma_prepass also writes the
 * zero-padded copies of A and B, lcma_fused also crops the padded product
 * into C.  Classic plans: LCMA_E_INVALID. */
lcma_status lcma_prepass(lcma_plan_t plan, const void* A, int64_t lda, const void* B, int64_t ldb,
                         void* workspace, size_t workspace_bytes, void* stream);
lcma_status lcma_fused(lcma_plan_t plan, const void* A, int64_t lda, const void* B, int64_t ldb,
                       void* C, int64_t ldc, void* workspace, size_t workspace_bytes,
                       void* stream);

/* Source: [FG] "从 LCMA 到 FalconGEMM" (combined operands of the products).
 * Where the pre-pass puts the combined operand of product r (0-based) in the
 * workspace: side 0 = A (an (M/ms) x (K/ks) matrix), side 1 = B (a (K/ks) x
 * (N/ns) matrix).  *offset_bytes receives its byte offset and *ld its
 * leading dimension; *offset_bytes = -1 when the operand is a single input
 * block read in place (not copied).  *dtype receives the operand type.
 * *ld = 0 marks a tile-packed A operand: an unfused plan whose products run
 * in one persistent launch on whole 256 x 256 tiles (Mb and Nb multiples of
 * 256, Kb of 32) stores each combined A operand as consecutive blocks of
 * 256 rows x 32 columns, block (tr, t) (rows 256 tr.., columns 32 t..) at
 * element (tr * Kb + 32 t) * 256; row rr of a block is 32 elements whose four
 * 8-element chunks c sit at positions c ^ ((rr >> 1) & 3).
 * A padded plan reports the operands of its padded product (blocks of the
 * padded shape).  LCMA_E_INVALID for a plan that combines at load (it
 * writes no combined operand). */
lcma_status lcma_plan_operand(lcma_plan_t plan, int32_t side, int32_t r, int64_t* offset_bytes,
                              int64_t* ld, lcma_dtype* dtype);

/* Source: [FG] "从 LCMA 到 FalconGEMM" (groups on compute units, the split of
 * a group over two compute units, locality-aware ordering).
 * Schedule of the persistent kernel, for host-side checking.  Fills up to
 * `cap` work items, 5 int32 each: worker, group, first product position,
 * end product position (in the kernel's product order), split slot (-1 for
 * a whole group).  *count receives the total number of items (call with
 * cap = 0 to size).  *order (if not NULL, `rank` entries) receives the
 * kernel's product order.  LCMA_E_INVALID for a classic plan and for an
 * unfused one (it has no persistent schedule).  A padded plan reports the
 * schedule of its padded product. */
lcma_status lcma_plan_schedule(lcma_plan_t plan, int32_t* items, int64_t cap, int64_t* count,
                               int32_t* order);

/* Source: [FG] "从 LCMA 到 FalconGEMM" (each output block is the W-weighted
 * sum of the products; the products of a position accumulate on chip).
 * Run schedule of an unfused plan whose products run in one persistent
 * launch, for host-side checking.  Run j (0 <= j < rank) computes product
 * *product starting from zero accumulators (*carry = 0), from the previous
 * run's accumulators (1) or from their negation (2), then adds fold[o]
 * times its accumulators into output block o (ms * ns entries, row-major
 * block order; 0 = no fold).  Each block is the sum of its folds.  For
 * descriptions of up to 7 products the planner searches every run order and
 * carry for the schedule whose fp32 folds move the fewest bytes (a block fed
 * by k runs moves 2 bytes per element for k = 1, else 8k - 6), which takes
 * up to about 0.2 s at plan creation (once per table; later plans reuse
 * it); otherwise a product feeding a single block continues the
 * accumulators of another product feeding that block.  LCMA_E_INVALID for
 * any other plan, a run outside 0..rank-1 or NULL outputs.  A padded plan
 * reports the schedule of its padded product. */
lcma_status lcma_plan_runs(lcma_plan_t plan, int32_t run, int32_t* product, int32_t* carry, int8_t* fold);

/* Classic MFMA GEMM without a plan (enqueues one kernel on `stream`).
 * Same layout, alignment and error rules as lcma_gemm; K or N not a
 * multiple of 8, or unaligned operands, take the element-load kernel.
 * Source: [CL2] "核心贡献与发现的技术" (multi-stage staging of A/B tiles,
 * wide epilogue stores, block swizzling); [KP] "Roofline" (compute-bound
 * when FLOPs per byte exceed the ridge point). */
lcma_status gemm_classic(int64_t M, int64_t N, int64_t K, lcma_dtype dt, const void* A, int64_t lda,
                         const void* B, int64_t ldb, void* C, int64_t ldc, void* stream);

/* Measured machine references, the ceilings the kernels are compared with
 * beside the published peaks.
 * lcma_measure_mfma: `workgroups` workgroups of 8 waves, each wave issuing
 *   iters x 16 independent 16x16x32 MFMAs (dt operands, random values held
 *   in registers, fp32 accumulate); out receives one float per thread
 *   (workgroups * 512 floats, device memory).  Work per launch:
 *   workgroups * 8 * iters * 16 * 16384 flops.  LCMA_E_INVALID for a NULL
 *   out, workgroups outside 1..65536 or iters outside 1..2^24.
 * lcma_measure_copy: dst = src over `bytes` (device memory, 16-byte aligned,
 *   a multiple of 16 bytes: else LCMA_E_UNSUPPORTED); reads and writes each
 *   byte once, so HBM traffic is 2 * bytes when both exceed the caches.
 * lcma_measure_read: reads `bytes` of src once (same alignment rules), the
 *   ceiling of read-dominated kernels such as decode products; out is one
 *   device uint32 that the kernel may write (its value is unspecified).
 *   LCMA_E_INVALID for a NULL src or out with nonzero bytes.
 * All only enqueue on `stream`.
 * Source: [KP] "Roofline" (F <= min(F_max, I * B_max): the peaks the
 * roofline is drawn against) and "Benchmark 纪律" (measure, do not assume). */
lcma_status lcma_measure_mfma(float* out, int32_t workgroups, int32_t iters, lcma_dtype dt, void* stream);
lcma_status lcma_measure_copy(const void* src, void* dst, size_t bytes, void* stream);
lcma_status lcma_measure_read(const void* src, size_t bytes, uint32_t* out, void* stream);

/* Frees a plan (NULL is a no-op).  Plans own host memory only.
 * Source: none on the pages (plan lifetime is this library's interface). */
void lcma_plan_destroy(lcma_plan_t plan);

/* Static text for a status code.
 * Source: none on the pages (error reporting is this library's interface). */
const char* lcma_status_str(lcma_status s);

#ifdef __cplusplus
}
#endif

#endif /* LCMA_H_ */
