/*
 * w4g_oracle.c -- plain, slow CPU oracle for the W4 g64 matrix products and the
 * greedy vocabulary argmax.
 *
 * TEST INFRASTRUCTURE ONLY.  The product path (the HIP library) never calls,
 * links or loads this file; only the test suite, the smoke check and the CPU
 * baseline leg of the benchmark do.  It shares no code, header, table or
 * helper with the HIP kernels.
 *
 * What it computes, and where the sources state it:
 *
 *  - Weight format: 4-bit affine quantization with group size 64 (TensorFold
 *    PR #1437, "Receipt": the served checkpoint is "4-bit affine with group
 *    64").  Readings taken where the pages are silent: each weight is an
 *    unsigned code q in 0..15; eight codes are packed per uint32 along K with
 *    element 8i+j in bits [4j, 4j+4) of word i (low nibble first); one bf16
 *    scale s and one bf16 bias b per (output row, 64-element K group); the
 *    dequantized weight is w = q*s + b.
 *
 *  - Other widths: the pages' kernel takes widths other than 4 bits in a
 *    separate variant (TensorFold PR #1433, review of step 2: other widths
 *    take simd_qmm_bits), and the B70 page serves an INT8 LM head with bf16
 *    scales.  Reading: the same affine group-64 format with b-bit unsigned
 *    codes, b in {2, 4, 8}: 32/b codes per uint32, element (32/b) i + j in
 *    bits [b j, b j + b) of word i, K b / 32 words per row, the same bf16
 *    scale and bias tables.
 *
 *  - Products: y[m][n] = sum_k x[m][k] * w[n][k], with an fp32 result (the
 *    seam's payload is fp32, "the seam's accumulation", and simd_qmm gains an
 *    fp32-out store: TensorFold PR #1437, commit "Add the pair seam and
 *    register its kernels with the kernel contract").  The oracle forms each
 *    w exactly as fp32 (q*s is exact, so a single rounding happens in the
 *    add), multiplies by x exactly in fp64, sums in fp64 in ascending k and
 *    rounds once to fp32.  This is the plain definition with a wider
 *    accumulator; its own error is about 1e-16 relative, far below any
 *    tolerance the GPU path is held to.
 *
 *  - Greedy head: the argmax over a full logit row.  A row holding any NaN,
 *    +Inf or -Inf fails: its id is the sentinel maxInt(u32) = 0xFFFFFFFF
 *    (TensorFold PR #1433, step-1 description: one machine fails a row holding
 *    any NaN or +-Inf, pair_argmax flags such a row with bit 31 of its id word
 *    and pair_pick turns the flag into the id sentinel; step-2 description:
 *    the session reads the maxInt(u32) sentinel as a failure, never as a
 *    logit).  Otherwise the largest value wins and an exact tie goes to the
 *    lowest id (the same step-1 description lists, among the controls that
 *    must fail, an argmax and a pick that resolve a tie to the larger id).  Comparison is
 *    IEEE float comparison, so -0.0 and +0.0 tie and denormals compare
 *    exactly.  bf16 logits are widened to fp32 exactly first.
 *
 *  - Top two: the winner and the runner-up of the same ordering (value
 *    descending, id ascending), that is the argmax and then the argmax over
 *    the other ids, with the gap v(winner) - v(runner-up) in fp32, zeros
 *    counted as +0.0 so the gap is never -0.0.  A row holding a non-finite
 *    value gives the sentinel for both and a NaN gap.  (Reading: the pages'
 *    session merges "the top two" across blocks for its tie test, TensorFold
 *    PR #1433, step-1 description; the pages fix no format for it.)
 *
 *  - bf16 store: a product's fp32 result rounded to bf16 to nearest, ties to
 *    the even last bit (8 significant bits, the fp32 exponent range; a value
 *    at or beyond the midpoint between the largest bf16 and 2^128 becomes
 *    infinity); a NaN stays a quiet NaN of its sign.  (Reading: the pages'
 *    kernel stores in the activation dtype, and TensorFold PR #1437, commit
 *    "Add the pair seam and register its kernels with the kernel contract",
 *    adds the fp32-out variant beside it; the pages name no rounding, and
 *    nearest-even is the IEEE default.)
 *
 * Parallelism: optional OpenMP over independent output elements only.  Every
 * single dot product is computed by one thread in ascending k, so the result
 * does not depend on the thread count.
 *
 * Planted mistakes (for the test that proves the pins catch them): building
 * with -DW4O_PLANT=<n> compiles one deliberate error into this file.  The
 * default build has none.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#ifndef W4O_PLANT
#define W4O_PLANT 0
#endif
/* planted mistakes: 1 high nibble first, 2 bias dropped, 3 group of 32,
   4 tie to the higher id, 5 no non-finite flag, 6 bias sign flipped,
   7 scale/bias tables read as [G][N], 8 -0.0 ordered below +0.0,
   9 fp32 accumulation, 10 activation row picked by the output row's stride,
   11 last K group dropped, 12 runner-up tie to the higher id,
   13 bf16 store ties rounded away from zero, 14 high field first in a word
   for widths other than 4, 15 8-bit rows read at the 4-bit pitch */

/* bf16 -> fp32 is exact: the bf16 bits are the top half of the fp32 bits. */
static float o_bf16_to_f32(uint16_t h) {
  uint32_t u = ((uint32_t)h) << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return f;
}

static int o_bits = 4; /* code width of the call in progress */

/* code of element k in packed row `row` (K*bits/32 words). */
static uint32_t o_code(const uint32_t* row, int64_t k) {
  if (o_bits == 4) {
#if W4O_PLANT == 1
    return (row[k >> 3] >> (4 * (7 - (k & 7)))) & 0xFu;
#else
    return (row[k >> 3] >> (4 * (k & 7))) & 0xFu;
#endif
  }
  const int64_t per = 32 / o_bits; /* codes per word */
  const uint32_t mask = (1u << o_bits) - 1u;
#if W4O_PLANT == 14
  const int64_t j = per - 1 - (k % per);
#else
  const int64_t j = k % per;
#endif
  return (row[k / per] >> (o_bits * j)) & mask;
}

/* words per packed row */
static int64_t o_row_words(int64_t K) {
#if W4O_PLANT == 15
  return o_bits == 8 ? K / 8 : K * o_bits / 32; /* half the 8-bit pitch: stays in bounds */
#else
  return K * o_bits / 32;
#endif
}

static int64_t o_groups = 1; /* K/64 of the call in progress (planted mistake 3 only) */
static int64_t o_group(int64_t k) {
#if W4O_PLANT == 3
  return (k >> 5) % o_groups; /* stays inside the table */
#else
  return k >> 6;
#endif
}

/* Dequantized weight w[n][k] = q*s + b, exact product then one fp32 rounding. */
static float o_weight(const uint32_t* wq, const uint16_t* scales, const uint16_t* biases,
                      int64_t N, int64_t K, int64_t n, int64_t k) {
  const int64_t G = K / 64;
  float q = (float)o_code(wq + n * o_row_words(K), k);
#if W4O_PLANT == 7
  float s = o_bf16_to_f32(scales[(o_group(k) * N + n) % (N * G)]);
  float b = o_bf16_to_f32(biases[(o_group(k) * N + n) % (N * G)]);
#else
  float s = o_bf16_to_f32(scales[n * G + o_group(k)]);
  float b = o_bf16_to_f32(biases[n * G + o_group(k)]);
#endif
  (void)N;
#if W4O_PLANT == 2
  b = 0.0f;
#endif
#if W4O_PLANT == 6
  b = -b;
#endif
  float prod = q * s; /* exact: at most 8 x 8 significant bits */
  return prod + b;    /* the only rounding */
}

/* Dequantize a whole matrix to fp32, w[n][k] row-major. */
void w4o_dequant(const uint32_t* wq, const uint16_t* scales, const uint16_t* biases,
                 int64_t N, int64_t K, float* w) {
  o_bits = 4;
  o_groups = K / 64;
  for (int64_t n = 0; n < N; ++n)
    for (int64_t k = 0; k < K; ++k) w[n * K + k] = o_weight(wq, scales, biases, N, K, n, k);
}

/* Start of activation row m in the [M][K] activation matrix. */
static int64_t o_xrow(int64_t m, int64_t M, int64_t N, int64_t K) {
#if W4O_PLANT == 10
  int64_t r = m * N; /* clipped so the planted read stays inside x */
  return r < (M - 1) * K ? r : (M - 1) * K;
#else
  (void)M;
  (void)N;
  return m * K;
#endif
}

/* One output element: fl32( sum_k x[k] * w[n][k] ), fp64 ascending-k sum. */
static float o_dot(const uint32_t* wq, const uint16_t* scales, const uint16_t* biases,
                   const uint16_t* xrow, int64_t N, int64_t K, int64_t n) {
#if W4O_PLANT == 11
  const int64_t kend = K - 64;
#else
  const int64_t kend = K;
#endif
#if W4O_PLANT == 9
  float acc = 0.0f;
  for (int64_t k = 0; k < kend; ++k)
    acc += o_bf16_to_f32(xrow[k]) * o_weight(wq, scales, biases, N, K, n, k);
  return acc;
#else
  double acc = 0.0;
  for (int64_t k = 0; k < kend; ++k)
    acc += (double)o_bf16_to_f32(xrow[k]) * (double)o_weight(wq, scales, biases, N, K, n, k);
  return (float)acc;
#endif
}

/* y[m][n] for all m < M and n < N.  x is [M][K] bf16, y is [M][N] fp32. */
void w4o_qmm(const uint32_t* wq, const uint16_t* scales, const uint16_t* biases,
             const uint16_t* x, float* y, int64_t M, int64_t N, int64_t K, int threads) {
  o_bits = 4;
  o_groups = K / 64;
#ifdef _OPENMP
  if (threads < 1) threads = omp_get_max_threads();
#pragma omp parallel for collapse(2) schedule(static) num_threads(threads)
#else
  (void)threads;
#endif
  for (int64_t m = 0; m < M; ++m)
    for (int64_t n = 0; n < N; ++n)
      y[m * N + n] = o_dot(wq, scales, biases, x + o_xrow(m, M, N, K), N, K, n);
}

/* Selected output rows only: y[m][j] = output (m, rows[j]), y is [M][nrows]. */
void w4o_qmm_rows(const uint32_t* wq, const uint16_t* scales, const uint16_t* biases,
                  const uint16_t* x, float* y, int64_t M, int64_t N, int64_t K,
                  const int64_t* rows, int64_t nrows, int threads) {
  o_bits = 4;
  o_groups = K / 64;
#ifdef _OPENMP
  if (threads < 1) threads = omp_get_max_threads();
#pragma omp parallel for collapse(2) schedule(static) num_threads(threads)
#else
  (void)threads;
#endif
  for (int64_t m = 0; m < M; ++m)
    for (int64_t j = 0; j < nrows; ++j)
      y[m * nrows + j] = o_dot(wq, scales, biases, x + o_xrow(m, M, N, K), N, K, rows[j]);
}

/* The same three products at code width `bits` (2, 4 or 8; anything else
   returns 1 and computes nothing). */
int w4o_dequant_bits(const uint32_t* wq, const uint16_t* scales, const uint16_t* biases,
                     int64_t N, int64_t K, int bits, float* w) {
  if (bits != 2 && bits != 4 && bits != 8) return 1;
  o_groups = K / 64;
  o_bits = bits;
  for (int64_t n = 0; n < N; ++n)
    for (int64_t k = 0; k < K; ++k) w[n * K + k] = o_weight(wq, scales, biases, N, K, n, k);
  o_bits = 4;
  return 0;
}

int w4o_qmm_bits(const uint32_t* wq, const uint16_t* scales, const uint16_t* biases,
                 const uint16_t* x, float* y, int64_t M, int64_t N, int64_t K, int bits, int threads) {
  if (bits != 2 && bits != 4 && bits != 8) return 1;
  o_groups = K / 64;
  o_bits = bits;
#ifdef _OPENMP
  if (threads < 1) threads = omp_get_max_threads();
#pragma omp parallel for collapse(2) schedule(static) num_threads(threads)
#else
  (void)threads;
#endif
  for (int64_t m = 0; m < M; ++m)
    for (int64_t n = 0; n < N; ++n)
      y[m * N + n] = o_dot(wq, scales, biases, x + o_xrow(m, M, N, K), N, K, n);
  o_bits = 4;
  return 0;
}

int w4o_qmm_rows_bits(const uint32_t* wq, const uint16_t* scales, const uint16_t* biases,
                      const uint16_t* x, float* y, int64_t M, int64_t N, int64_t K,
                      const int64_t* rows, int64_t nrows, int bits, int threads) {
  if (bits != 2 && bits != 4 && bits != 8) return 1;
  o_groups = K / 64;
  o_bits = bits;
#ifdef _OPENMP
  if (threads < 1) threads = omp_get_max_threads();
#pragma omp parallel for collapse(2) schedule(static) num_threads(threads)
#else
  (void)threads;
#endif
  for (int64_t m = 0; m < M; ++m)
    for (int64_t j = 0; j < nrows; ++j)
      y[m * nrows + j] = o_dot(wq, scales, biases, x + o_xrow(m, M, N, K), N, K, rows[j]);
  o_bits = 4;
  return 0;
}

static int o_finite(float v) {
#if W4O_PLANT == 5
  (void)v;
  return 1;
#else
  return isfinite(v);
#endif
}

/* Greedy pick over one row of fp32 values: linear scan in ascending id. */
static uint32_t o_argmax_f32(const float* v, int64_t V) {
  for (int64_t i = 0; i < V; ++i)
    if (!o_finite(v[i])) return 0xFFFFFFFFu;
  int64_t best = 0;
  for (int64_t i = 1; i < V; ++i) {
#if W4O_PLANT == 4
    if (v[i] >= v[best]) best = i;
#elif W4O_PLANT == 8
    if (v[i] > v[best] || (v[i] == v[best] && signbit(v[best]) && !signbit(v[i]))) best = i;
#else
    if (v[i] > v[best]) best = i;
#endif
  }
  return (uint32_t)best;
}

/* The runner-up: the argmax over every id but `skip`, same rules.  V >= 2. */
static uint32_t o_argmax_skip_f32(const float* v, int64_t V, int64_t skip) {
  int64_t best = skip == 0 ? 1 : 0;
  for (int64_t i = best + 1; i < V; ++i) {
    if (i == skip) continue;
#if W4O_PLANT == 12
    if (v[i] >= v[best]) best = i;
#else
    if (v[i] > v[best]) best = i;
#endif
  }
  return (uint32_t)best;
}

static float o_plus_zero(float v) { return v == 0.0f ? 0.0f : v; }

static void o_top2_f32(const float* v, int64_t V, uint32_t* ids2, float* gap) {
  const uint32_t a = o_argmax_f32(v, V);
  if (a == 0xFFFFFFFFu) {
    ids2[0] = ids2[1] = 0xFFFFFFFFu;
    *gap = NAN;
    return;
  }
  const uint32_t b = o_argmax_skip_f32(v, V, (int64_t)a);
  ids2[0] = a;
  ids2[1] = b;
  *gap = o_plus_zero(v[a]) - o_plus_zero(v[b]);
}

/* Top two per row (V >= 2): ids2[r][0..1], gaps[r]. */
int w4o_argmax_top2(const void* logits, int dtype, int64_t rows, int64_t V, int64_t ld,
                    uint32_t* ids2, float* gaps, float* scratch) {
  if (V < 2 || ld < V || rows < 0) return 1;
  for (int64_t r = 0; r < rows; ++r) {
    if (dtype == 0) {
      o_top2_f32((const float*)logits + r * ld, V, ids2 + 2 * r, gaps + r);
    } else if (dtype == 1) {
      const uint16_t* row = (const uint16_t*)logits + r * ld;
      for (int64_t i = 0; i < V; ++i) scratch[i] = o_bf16_to_f32(row[i]);
      o_top2_f32(scratch, V, ids2 + 2 * r, gaps + r);
    } else {
      return 2;
    }
  }
  return 0;
}

/* dtype 0: fp32 logits; dtype 1: bf16 logits.  Row r starts at element r*ld. */
int w4o_argmax(const void* logits, int dtype, int64_t rows, int64_t V, int64_t ld,
               uint32_t* ids, float* scratch) {
  if (V < 1 || ld < V || rows < 0) return 1;
  for (int64_t r = 0; r < rows; ++r) {
    if (dtype == 0) {
      ids[r] = o_argmax_f32((const float*)logits + r * ld, V);
    } else if (dtype == 1) {
      const uint16_t* row = (const uint16_t*)logits + r * ld;
      for (int64_t i = 0; i < V; ++i) scratch[i] = o_bf16_to_f32(row[i]);
      ids[r] = o_argmax_f32(scratch, V);
    } else {
      return 2;
    }
  }
  return 0;
}

/* fp32 value of fp32 bit pattern u */
static double o_f32_bits(uint32_t u) {
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/* One fp32 value to bf16 bits, nearest-even.  The two candidates are the bf16
   magnitudes just below and just above |f| (the fp32 bits with the low 16 bits
   cleared, and the next bf16 up, 2^128 standing in for infinity); the nearer
   one wins, a tie goes to the one whose last bit is 0.  The distances are
   exact in double. */
static uint16_t o_to_bf16(float f) {
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  if (isnan(f)) return (uint16_t)((u >> 16) | 0x0040u);
  const uint32_t sign = u & 0x80000000u, mag = u & 0x7FFFFFFFu;
  const uint32_t lo = mag & 0xFFFF0000u;
  if (lo == mag) return (uint16_t)((sign | mag) >> 16); /* already a bf16 value (0, inf too) */
  const uint32_t hi = lo + 0x00010000u;
  const double v = o_f32_bits(mag);
  const double dlo = v - o_f32_bits(lo);
  const double dhi = (hi == 0x7F800000u ? ldexp(1.0, 128) : o_f32_bits(hi)) - v;
  uint32_t pick;
  if (dlo < dhi)
    pick = lo;
  else if (dhi < dlo)
    pick = hi;
  else
#if W4O_PLANT == 13
    pick = hi;
#else
    pick = ((lo >> 16) & 1u) ? hi : lo;
#endif
  return (uint16_t)((sign | pick) >> 16);
}

/* bf16 store of n fp32 values. */
void w4o_to_bf16(const float* in, uint16_t* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = o_to_bf16(in[i]);
}

int w4o_plant(void) { return W4O_PLANT; }

int w4o_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
