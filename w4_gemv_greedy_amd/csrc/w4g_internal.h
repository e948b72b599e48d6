// Internal declarations shared by the library's own translation units only.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w4g {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

// Workgroups of the one-workgroup-per-CU layouts: the current device's compute
// unit count (queried once per device), at most kMaxCUs, the MI355X's 256.  A
// layout only decides which workgroup computes which rows; no result depends on
// it.  Workspace sizes are computed with kMaxCUs, an upper bound for any device.
constexpr int kMaxCUs = 256;
int cu_count();

// Kernel launchers.  Arguments are already validated; each returns the
// hipError_t of its launch(es).
hipError_t launch_gemv(const uint32_t* wq, const uint16_t* scales, const uint16_t* biases,
                       const uint16_t* x, float* y, int B, int64_t N, int64_t K, bool force_regs,
                       hipStream_t stream);
// step: run the step-staged per-CU kernel whatever K is (same bits as the
// whole-x kernel; for checking that)
hipError_t launch_gemv_mfma(const uint32_t* wq, const uint16_t* scales, const uint16_t* biases,
                            const uint16_t* x, float* y, int B, int64_t N, int64_t K, bool step,
                            hipStream_t stream);
// y: fp32 [M][N], or bf16 [M][N] (nearest-even from the fp32 result) when y_bf16
hipError_t launch_gemm(const uint32_t* wq, const uint16_t* scales, const uint16_t* biases,
                       const uint16_t* x, void* y, bool y_bf16, int64_t M, int64_t N, int64_t K,
                       void* workspace, hipStream_t stream);
// Decode product with 2-, 4- or 8-bit codes (32/bits per uint32, low field
// first); widths other than 4 run the vector-ALU shared-memory variant only,
// which needs gemv_bits_fits(B, K).
hipError_t launch_gemv_bits(const uint32_t* wq, const uint16_t* scales, const uint16_t* biases,
                            const uint16_t* x, float* y, int B, int64_t N, int64_t K, int bits,
                            hipStream_t stream);
bool gemv_bits_fits(int B, int64_t K);
// The fused head at 2 or 8 bits: launch_gemv_bits's kernels with the argmax's
// pass 1 as their epilogue (one record per workgroup and batch row), so the
// logits are launch_gemv_bits's bit for bit; y may be null.
hipError_t launch_gemv_bits_argmax(const uint32_t* wq, const uint16_t* scales, const uint16_t* biases,
                                   const uint16_t* x, float* y, uint2* rec, int B, int64_t N, int64_t K,
                                   int bits, hipStream_t stream);
int64_t gemv_bits_argmax_records(int B, int64_t N, int64_t K);
int64_t gemv_bits_argmax_records_max(int B, int64_t N, int64_t K);
// Kernel family qmm_gemv runs (1 = vector ALU, 2 = matrix cores): a function
// of the whole matrix's row count and of K only, never of the batch size.
int gemv_auto_family(int64_t whole, int64_t K);
size_t gemm_workspace_bytes(int64_t M, int64_t N, int64_t K);
hipError_t launch_argmax(const void* logits, int dtype, int64_t rows, int64_t vocab, int64_t ld,
                         uint32_t* ids, void* workspace, hipStream_t stream);
size_t argmax_workspace_bytes(int64_t rows, int64_t vocab);
// Top two per row: ids2[r][0..1] (winner, runner-up) and gaps[r].
hipError_t launch_argmax_top2(const void* logits, int dtype, int64_t rows, int64_t vocab, int64_t ld,
                              uint32_t* ids2, float* gaps, void* workspace, hipStream_t stream);
size_t argmax_top2_workspace_bytes(int64_t rows, int64_t vocab);
// Pass 2 alone: combines `nrec` (value, id | flag) records per row into ids.
hipError_t launch_argmax_combine(const uint2* rec, int64_t rows, int64_t nrec, uint32_t* ids,
                                 hipStream_t stream);
// Decode product with the argmax's pass 1 as its epilogue, in the family
// gemv_auto_family picks: each workgroup writes one record per batch row
// (`nrec` per row, see gemv_argmax_records) instead of needing the logits read
// back; `y` may be null.  The logits' bits are those of that family's product.
hipError_t launch_gemv_argmax(const uint32_t* wq, const uint16_t* scales, const uint16_t* biases,
                              const uint16_t* x, float* y, uint2* rec, int B, int64_t N, int64_t K,
                              hipStream_t stream);
int64_t gemv_argmax_records(int B, int64_t N, int64_t K);
// An upper bound of gemv_argmax_records on any device (for workspace sizes).
int64_t gemv_argmax_records_max(int B, int64_t N, int64_t K);
// The matrix-core family's epilogue variant: one record per workgroup (one
// workgroup per CU share, whether x is held whole or staged step by step).
hipError_t launch_gemv_mfma_argmax(const uint32_t* wq, const uint16_t* scales, const uint16_t* biases,
                                   const uint16_t* x, float* y, uint2* rec, int B, int64_t N, int64_t K,
                                   hipStream_t stream);
int64_t gemv_mfma_argmax_records(int B, int64_t N, int64_t K, int cus);

// Loads of the packed codes, the stream that is read exactly once per call:
// non-temporal, so the lines pass through the caches with the streaming
// policy.  Measured on MI355X, a read-only stream of 2 GiB moves 7.0-7.1 TB/s
// with non-temporal 16-byte loads against 6.0-6.3 TB/s with plain ones, and
// the vector-ALU decode sweep runs 8% faster with them.  (The scale and bias
// tables keep plain loads: a row's table line is read in pieces, one per
// 1024-element chunk, and the products ran as fast or slower with the
// streaming policy on them (gate-up alone 18.3 against 19.8-20.7 us); the
// matrix-core decode keeps plain loads too: it ran slower with non-temporal
// ones.)
__device__ __forceinline__ uint4 ld_stream(const uint4* p) {
  typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ uint2 ld_stream(const uint2* p) {
  typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
  const u32x2_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(p));
  return make_uint2(v[0], v[1]);
}

constexpr int kArgmaxBlock = 1024;  // ids per pass-1 record
constexpr uint32_t kArgmaxFlag = 0x80000000u;  // non-finite bit of a record's id word

// Argmax ordering.  Each finite fp32 value maps to an unsigned key that orders
// exactly as IEEE comparison does, with -0.0 and +0.0 given the same key, so
// denormals compare exactly whatever the float denormal mode.  A candidate is
// the 64-bit word (key << 32) | (0xFFFFFFFF - id); the maximum word is the
// largest value with the lowest id, so every reduction step is an unsigned max
// and no result depends on the reduction tree.
__device__ __forceinline__ uint32_t order_key(uint32_t u) {
  if ((u & 0x7FFFFFFFu) == 0) return 0x80000000u;  // +0 and -0 tie
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ uint32_t key_bits(uint32_t k) {
  return (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
}
__device__ __forceinline__ bool finite_bits(uint32_t u) {
  return (u & 0x7F800000u) != 0x7F800000u;
}
__device__ __forceinline__ uint64_t cand(uint32_t bits, uint32_t id) {
  return ((uint64_t)order_key(bits) << 32) | (uint64_t)(0xFFFFFFFFu - id);
}
__device__ __forceinline__ uint64_t umax64(uint64_t a, uint64_t b) { return a > b ? a : b; }
// The pass-1 record of a candidate: value bits and id, or the flag if any
// value was not finite.
__device__ __forceinline__ uint2 make_record(uint64_t best, bool bad, uint32_t first_id) {
  uint2 r;
  if (bad) {
    r.x = 0x7FC00000u;
    r.y = kArgmaxFlag | first_id;
  } else {
    r.x = key_bits((uint32_t)(best >> 32));
    r.y = 0xFFFFFFFFu - (uint32_t)best;
  }
  return r;
}

}  // namespace w4g
