/*
 * w4g.h -- C ABI of the MI355X (gfx950) library for 4-bit affine group-64
 * quantized matrix products and the greedy vocabulary argmax.
 *
 * Operations (what each computes, and where the sources define it):
 *
 *   qmm_gemv / qmm_gemm:  y[m][n] = sum_k x[m][k] * w[n][k], fp32 result,
 *     with w[n][k] = q[n][k] * s[n][k/64] + b[n][k/64].
 *     - 4-bit affine quantization with group size 64: TensorFold PR #1437
 *       ("qwen27: document two-Mac 27B serving and the seam's known tie"),
 *       Receipt.
 *     - fp32 accumulation and an fp32 store: the same PR, commit "Add the
 *       pair seam and register its kernels with the kernel contract".
 *     - Within a kernel family (qmm_gemv_ex) the K reduction order is a
 *       function of the matrix width K alone, never of N, the batch, the
 *       grid or timing: TensorFold PR #1433, step-2 description (a rank's K
 *       tree is its own full matrix's; the split is keyed on the whole
 *       matrix, not on a slice).  qmm_gemv's own choice of family is a
 *       function of K and of the whole matrix's row count only, never of the
 *       batch size, so a row has the same bits at every batch size and in
 *       every row slice that names its whole matrix: a request served beside
 *       others gets the bits it gets alone (TensorFold PR #1437, Checklist).
 *     qmm_gemv is the decode path (1 <= B <= 8 activation rows); qmm_gemm is
 *     the prompt path (any M >= 1, matrix cores).
 *
 *   vocab_argmax:  ids[r] = the greedy token of logit row r.  A row holding any
 *     NaN, +Inf or -Inf yields W4G_SENTINEL (0xFFFFFFFF); otherwise the largest
 *     value wins and exact ties go to the lowest id (-0.0 ties +0.0).
 *     TensorFold PR #1433, step-1 description (pair_argmax flags a non-finite
 *     row with bit 31 of its id word, pair_pick turns the flag into the
 *     maxInt(u32) sentinel, and a pick that ties to the higher id is a planted
 *     failure) and step-2 description (the session reads the sentinel as a
 *     failure, never as a logit).
 *
 * Data layout (all row-major, all device memory):
 *   wq      [N][K/8]  uint32: element k = 8i+j of row n is bits [4j, 4j+4) of
 *                     word wq[n][i] (low nibble first), an unsigned code 0..15.
 *   scales  [N][K/64] bf16 (passed as uint16 bit patterns).
 *   biases  [N][K/64] bf16.
 *   x       [B][K] or [M][K] bf16.
 *   y       [B][N] or [M][N] fp32 (qmm_gemm_ex: fp32 or bf16).
 *   logits  [rows][ld] fp32 or bf16; row r occupies elements [r*ld, r*ld+vocab).
 *   ids     [rows] uint32.
 *
 * Ownership and behaviour common to every entry point:
 *   - Every pointer is a device pointer owned by the caller.  No call
 *     allocates, frees or synchronizes; the library keeps no state between
 *     calls.  Work is enqueued on `stream` (a hipStream_t; NULL is the null
 *     stream) and completes asynchronously.
 *   - All arguments are validated on the host before any HIP call; a call that
 *     fails validation enqueues nothing and returns a nonzero W4G_E* status.
 *   - Outputs must not overlap inputs or the workspace.
 *   - Non-finite logits are data, not an error: the row's id is the sentinel.
 *   - Device faults surface at the caller's next synchronization.
 *   - Calls that share one workspace buffer must be ordered on one stream.
 */
#ifndef W4G_H
#define W4G_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define W4G_ABI_VERSION 3
#define W4G_SENTINEL 0xFFFFFFFFu
#define W4G_MAX_GEMV_BATCH 8

/* status codes */
#define W4G_OK 0
#define W4G_EINVAL_PTR 1  /* a required pointer is NULL */
#define W4G_ESHAPE 2      /* a size is out of range (K % 64, B, N, M, vocab, ld) */
#define W4G_EALIGN 3      /* a buffer below its alignment (16 bytes: wq, x, y, logits, the
                             product workspace; 8: the argmax workspace; 4: ids; 2: tables) */
#define W4G_EWORKSPACE 4  /* workspace missing or smaller than qmm_workspace_bytes */
#define W4G_EDTYPE 5      /* unknown logits dtype or op code */
#define W4G_ELAUNCH 6     /* the HIP runtime refused a launch */
#define W4G_EALIAS 7      /* an output overlaps an input or the workspace */
#define W4G_ESCRATCH 8    /* the sizes need more than the library's static scratch */

/* logits dtypes */
#define W4G_F32 0
#define W4G_BF16 1

/* op codes for qmm_workspace_bytes */
#define W4G_OP_GEMV 0
#define W4G_OP_GEMM 1
#define W4G_OP_ARGMAX 2
#define W4G_OP_GEMV_ARGMAX 3
#define W4G_OP_ARGMAX_TOP2 4
#define W4G_OP_GEMV_BITS_ARGMAX 5

/*
 * Decode product, 1 <= B <= 8 activation rows.
 *   wq, scales, biases: the quantized matrix (N rows, K columns), see layout.
 *   x [B][K] bf16, y [B][N] fp32.  N >= 1; K >= 64 and K % 64 == 0.
 *   wq, x and y must be 16-byte aligned.
 *   workspace: at least qmm_workspace_bytes(W4G_OP_GEMV, B, N, K) bytes
 *   (may be NULL when that is 0).
 * Reduction order (a function of K only): K is cut into chunks of 1024
 * elements (the last may be shorter); within a chunk, lane j of a 32-lane
 * group owns elements [32j, 32j+32), half of one 64-group, and forms
 * s*D + (b - 128*s)*X, where D is the dot of x with (128 + q) taken over
 * bf16 pairs in ascending pair order and X the fp32 sum of those 32 x; each
 * lane adds its chunk terms in ascending chunk order, and the 32 lane sums
 * meet in a fixed tree: lanes j and j ^ 16 are added (a permlane16 swap),
 * then, within 16 lanes, lane j adds lane 15 - j (DPP row_mirror), within 8
 * lanes lane 7 - j (row_half_mirror), then lane j ^ 2 and lane j ^ 1
 * (quad_perm), leaving the sum in every lane.  That is the order of the
 * vector-ALU family, which qmm_gemv runs for every shape: the choice is
 * qmm_gemv_ex's W4G_GEMV_AUTO with whole = N, a function of (K, N) only, so
 * row m of a B-row call has the bits of that row computed alone, at every B.
 */
int qmm_gemv(const uint32_t* wq, const uint16_t* scales, const uint16_t* biases,
             const uint16_t* x, float* y, int64_t B, int64_t N, int64_t K,
             void* workspace, size_t workspace_bytes, void* stream);

/*
 * Decode product with codes of another width.  Same arguments, layout and
 * result as qmm_gemv, plus `bits` in {2, 4, 8} (else W4G_EDTYPE): wq is
 * [N][K*bits/32] uint32, element (32/bits) i + j of a row in bits
 * [bits j, bits j + bits) of word i (low field first), an unsigned code
 * 0 .. 2^bits - 1, with the same bf16 scale and bias per (row, 64-group):
 * w = q*s + b.  bits = 4 is exactly qmm_gemv.  The pages' kernel takes widths
 * other than 4 bits in its simd_qmm_bits variant (TensorFold PR #1433, review
 * of step 2) and the B70 page serves an INT8 LM head with bf16 scales
 * (b70-optimization-lab, "Reproduce Qwen3.6 27B AutoRound Bring-Up", current
 * best profile); reading: the same affine group-64 format at those widths.
 * Widths 2 and 8 run on the vector ALUs with x staged in LDS, so one row of x
 * must fit: 2.125 * K bytes <= 152 KiB, K <= 72,704 (else W4G_ESHAPE); a batch
 * whose rows do not fit together runs in parts that do (each reading the
 * weights once), with the same bits per row.  Order per row, K only:
 * as qmm_gemv's, with each lane's 32-element segment taken as its code words
 * in order; 2-bit: within a word fields (j, j + 8) form one bf16 pair
 * (128 + q), j ascending; 8-bit: a code is its two nibbles, Dl over the low
 * and Dh over the high nibbles (each 128 + nibble, pairs (q0, q2), (q1, q3)
 * per word), the segment's term is fma(16, Dh, Dl), and the constant part
 * folds into b - 2176 s.
 */
int qmm_gemv_bits(const uint32_t* wq, const uint16_t* scales, const uint16_t* biases,
                  const uint16_t* x, float* y, int64_t B, int64_t N, int64_t K, int bits,
                  void* workspace, size_t workspace_bytes, void* stream);

/* kernel families for qmm_gemv_ex */
#define W4G_GEMV_AUTO 0   /* the library's choice, by K and the whole matrix's rows only (qmm_gemv's) */
#define W4G_GEMV_VALU 1   /* vector-ALU dot2 kernel (the order documented for qmm_gemv) */
#define W4G_GEMV_MFMA 2   /* matrix-core kernel (order documented below) */
#define W4G_GEMV_VALU_REGS 3  /* vector-ALU family, register-staged variant (same bits as 1) */
#define W4G_GEMV_MFMA_STEP 4  /* matrix-core family, step-staged variant (same bits as 2) */

/*
 * qmm_gemv with an explicit kernel family.  Same arguments and results as
 * qmm_gemv; `kernel` is one of W4G_GEMV_*, else W4G_EDTYPE.
 * `whole`: the row count of the whole matrix that these N rows are a slice of
 * (0 means N; else N <= whole < 2^31, W4G_ESHAPE otherwise).  W4G_GEMV_AUTO
 * picks the family from (K, whole) alone, so a row slice of a matrix runs the
 * family the whole matrix runs and its rows have the whole matrix's bits, as
 * the pages' kernel keeps the K split of the whole width for a rank holding a
 * slice (TensorFold PR #1433, step-1 description: chunks(n, whole)).  Today
 * that choice is the vector-ALU family for every (K, whole).  The vector-ALU
 * family stages x in LDS when B * 2.125 * K bytes fit in 152 KiB; a batch
 * whose x does not fit runs in parts of two rows or more that do (the weights
 * read once per part), and x is staged in registers where not even two rows
 * fit; W4G_GEMV_VALU_REGS forces the register variant (for checking that all
 * of these give the same bits).
 * The matrix-core family (W4G_GEMV_MFMA) feeds the codes to the matrix cores
 * as exact bf16 values 128 + q; per 64-group it adds s*P_g and
 * (b - 128 s)*X_g in fp32 (P_g the matrix-core group product from zero, X_g
 * the fp32 group sum of x).  One workgroup per CU on v_mfma_f32_16x16x32_bf16
 * (two instructions per group), the CU's rows in 16-row tiles: W = min(8, NI)
 * waves, NI = ceil(K / 128) items of two groups, wave w summing items
 * [w NI / W, (w + 1) NI / W) in ascending order, the W wave sums added in
 * ascending order.  x is held whole in LDS where eight rows of it fit (K up
 * to about 9,000) and staged one step of items at a time otherwise
 * (W4G_GEMV_MFMA_STEP forces the latter, for checking that both give the
 * same bits); the choice depends on K alone.
 * Within one family, row m of a B-row call is bitwise equal to the same row
 * computed alone; the two families agree within fp32 rounding, not bitwise.
 */
int qmm_gemv_ex(const uint32_t* wq, const uint16_t* scales, const uint16_t* biases,
                const uint16_t* x, float* y, int64_t B, int64_t N, int64_t K,
                void* workspace, size_t workspace_bytes, void* stream, int kernel,
                int64_t whole);

/*
 * Prompt product on the matrix cores, any M >= 1 rows.
 *   Same layout and constraints as qmm_gemv with M in place of B.
 *   workspace: at least qmm_workspace_bytes(W4G_OP_GEMM, M, N, K) bytes,
 *   16-byte aligned.
 * Each code enters the bf16 matrix cores as the exact value 2 + q/8; a
 * 64-group's partial P_g is scaled by 8s in fp32 and added to the running sum
 * in ascending group order; the remaining affine term sum_g (b - 16 s) X_g
 * (X_g the fp32 group sum of x, split exactly into three bf16 parts X1..X3) is
 * accumulated on the matrix cores after the last group, block of 16 groups by
 * block in ascending order, each block as b X1, b X2, b X3, -16s X1, -16s X2,
 * -16s X3.  Row m of the result does not depend on M or on the other rows.
 */
int qmm_gemm(const uint32_t* wq, const uint16_t* scales, const uint16_t* biases,
             const uint16_t* x, float* y, int64_t M, int64_t N, int64_t K,
             void* workspace, size_t workspace_bytes, void* stream);

/*
 * qmm_gemm with a choice of output dtype.
 *   y_dtype: W4G_F32 (y is float [M][N], exactly qmm_gemm) or W4G_BF16 (y is
 *   bf16 [M][N], passed as uint16 bit patterns); anything else is W4G_EDTYPE.
 *   y must be 16-byte aligned either way.
 * The bf16 store rounds the fp32 result that qmm_gemm would have stored to
 * nearest-even (a NaN stays a quiet NaN of its sign; a finite value beyond
 * the bf16 range becomes +-Inf, as that rounding gives).  The pages' kernel
 * has a store in the activation dtype, to which TensorFold PR #1437 (commit
 * "Add the pair seam and register its kernels with the kernel contract") adds
 * the fp32-out variant; reading: that original store is bf16.
 */
int qmm_gemm_ex(const uint32_t* wq, const uint16_t* scales, const uint16_t* biases,
                const uint16_t* x, void* y, int64_t M, int64_t N, int64_t K,
                void* workspace, size_t workspace_bytes, void* stream, int y_dtype);

/*
 * Greedy argmax of `rows` logit rows of `vocab` entries (row pitch `ld`).
 *   dtype: W4G_F32 or W4G_BF16 (bf16 is widened to fp32 exactly).
 *   1 <= vocab < 2^31 (bit 31 of an id word is the non-finite flag),
 *   ld >= vocab, rows >= 1.  logits must be 16-byte aligned.
 *   ids [rows] uint32: the winning id, or W4G_SENTINEL for a row holding NaN
 *   or +-Inf.
 *   workspace: at least qmm_workspace_bytes(W4G_OP_ARGMAX, rows, vocab, 0),
 *   8-byte aligned.
 * Two passes: pass 1 reduces blocks of 1024 ids to (value, id | flag) records,
 * pass 2 combines a row's records; both keep the lowest id among equal
 * values and propagate the flag.
 */
int vocab_argmax(const void* logits, int dtype, int64_t rows, int64_t vocab, int64_t ld,
                 uint32_t* ids, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Decode product followed by the greedy argmax of each batch row, with the
 * argmax's first pass fused into the product's epilogue, so the logits need not
 * be written and read back.  The pages split the head the same way: each part
 * reduces its own rows to one (value, id word) pair with the non-finite flag in
 * bit 31, and a final pick combines the pairs (TensorFold PR #1433, step-1
 * description: pair_argmax and pair_pick; step-2 description: the head over
 * the whole vocabulary).
 *   wq, scales, biases, x, B, N, K: as qmm_gemv (N is the vocabulary size,
 *   N < 2^31).
 *   logits [B][N] fp32, or NULL: when given, receives exactly the bits
 *   qmm_gemv writes for the same (B, N, K) (the same kernel family, chosen
 *   the same way: from (K, N) alone, so a row's logit and the ids do not
 *   depend on the batch size).
 *   ids [B] uint32: per batch row the id of the largest logit, the lowest id
 *   among equal values (-0.0 ties +0.0), or W4G_SENTINEL if any logit of the
 *   row is NaN or +-Inf; always equal to vocab_argmax over those logits.
 *   workspace: at least qmm_workspace_bytes(W4G_OP_GEMV_ARGMAX, B, N, K)
 *   bytes, 8-byte aligned: one (value, id | flag) record per workgroup of the
 *   product and batch row.
 * Order of the logits: that of the family qmm_gemv picks (see qmm_gemv).
 */
int qmm_gemv_argmax(const uint32_t* wq, const uint16_t* scales, const uint16_t* biases,
                    const uint16_t* x, float* logits, uint32_t* ids, int64_t B, int64_t N,
                    int64_t K, void* workspace, size_t workspace_bytes, void* stream);

/*
 * qmm_gemv_argmax at another code width: the greedy head over a 2- or 8-bit
 * affine group-64 matrix (the B70 page, "Reproduce Qwen3.6 27B AutoRound
 * Bring-Up", serves its target model's vocabulary projection with 8-bit
 * integer weights; other widths take their own kernel variant, TensorFold PR
 * #1433, owner's review of step 2), with the argmax's first pass fused into
 * the product's epilogue as in qmm_gemv_argmax.
 *   wq, scales, biases, x, B, N, K, bits: as qmm_gemv_bits (bits 2, 4 or 8,
 *   else W4G_EDTYPE; 4 is qmm_gemv_argmax); N < 2^31.
 *   logits [B][N] fp32, or NULL: when given, exactly the bits qmm_gemv_bits
 *   writes for the same (B, N, K, bits).
 *   ids [B] uint32: as qmm_gemv_argmax, always equal to vocab_argmax over
 *   those logits.
 *   workspace: at least qmm_workspace_bytes(W4G_OP_GEMV_BITS_ARGMAX, B, N, K)
 *   bytes (the same for 2 and 8 bits), 8-byte aligned.
 * W4G_ESHAPE where qmm_gemv_bits refuses the shape (one row of x must fit in
 * LDS: K <= 72,704).
 */
int qmm_gemv_bits_argmax(const uint32_t* wq, const uint16_t* scales, const uint16_t* biases,
                         const uint16_t* x, float* logits, uint32_t* ids, int64_t B, int64_t N, int64_t K,
                         int bits, void* workspace, size_t workspace_bytes, void* stream);

/*
 * qmm_gemv_argmax for callers that cannot allocate (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * arguments without a workspace, the same results bit for bit (logits and
 * ids).  The per-workgroup records live in a static device array of the
 * library, 1 MiB (131,072 records) on each GPU the library runs on, held until
 * the process ends; sizes that need more, B * (records per batch row) above
 * 131,072 (qmm_workspace_bytes(W4G_OP_GEMV_ARGMAX, B, N, K) / 8), return
 * W4G_ESCRATCH before any launch.  The call allocates and frees nothing.
 * Every call on one GPU shares that GPU's array: calls that overlap in time on
 * one GPU (on different streams, or from several threads) race and may return
 * wrong ids; order them on one stream.  Nothing in the array needs clearing:
 * each call writes every record it reads.
 */
int qmm_gemv_argmax_noalloc(const uint32_t* wq, const uint16_t* scales, const uint16_t* biases,
                            const uint16_t* x, float* logits, uint32_t* ids, int64_t B, int64_t N,
                            int64_t K, void* stream);

/*
 * Top two of each logit row: the winner and the runner-up of the argmax's own
 * ordering (value descending, lowest id first among equal values, -0.0 equal
 * to +0.0) and the gap between them, so that a greedy pick that differs
 * between two computations of the logits can be told apart from a near tie.
 * (Reading: the pages' session keeps the two best candidates of each block
 * and merges them for its tie test, TensorFold PR #1433, step-1 description;
 * no format is given.)
 *   logits, dtype, rows, ld: as vocab_argmax; 2 <= vocab < 2^31.
 *   ids2 [rows][2] uint32: winner, runner-up (ids2[r][0] equals vocab_argmax's
 *   id); both W4G_SENTINEL if the row holds NaN or +-Inf.
 *   gaps [rows] fp32: v(winner) - v(runner-up) rounded to fp32, with either
 *   zero taken as +0.0 (so never -0.0); NaN for a non-finite row.
 *   workspace: at least qmm_workspace_bytes(W4G_OP_ARGMAX_TOP2, rows, vocab, 0)
 *   bytes, 16-byte aligned.
 * Two passes as in vocab_argmax, each keeping the two largest candidates.
 */
int vocab_argmax_top2(const void* logits, int dtype, int64_t rows, int64_t vocab, int64_t ld,
                      uint32_t* ids2, float* gaps, void* workspace, size_t workspace_bytes,
                      void* stream);

/*
 * Bytes of workspace an operation needs for the given sizes; 0 when none.
 *   op W4G_OP_GEMV: rows = B, n = N, k = K.
 *   op W4G_OP_GEMM: rows = M, n = N, k = K.
 *   op W4G_OP_ARGMAX: rows = rows, n = vocab, k ignored.
 *   op W4G_OP_GEMV_ARGMAX: rows = B, n = N, k = K.
 *   op W4G_OP_ARGMAX_TOP2: rows = rows, n = vocab (>= 2), k ignored.
 *   op W4G_OP_GEMV_BITS_ARGMAX: rows = B, n = N, k = K (2- and 8-bit codes).
 * Returns (size_t)-1 for an unknown op or sizes out of range.
 */
size_t qmm_workspace_bytes(int op, int64_t rows, int64_t n, int64_t k);

/* Static, NUL-terminated description of a status code (never NULL). */
const char* w4g_status_string(int status);

/* W4G_ABI_VERSION of the loaded library. */
int w4g_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* W4G_H */
