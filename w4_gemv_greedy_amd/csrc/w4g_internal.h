// Internal declarations shared by the library's own translation units only.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w4g {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

// Kernel launchers.  Arguments are already validated; each returns the
// hipError_t of its launch(es).
hipError_t launch_gemv(const uint32_t* wq, const uint16_t* scales, const uint16_t* biases,
                       const uint16_t* x, float* y, int B, int64_t N, int64_t K, bool force_regs,
                       hipStream_t stream);
hipError_t launch_gemv_mfma(const uint32_t* wq, const uint16_t* scales, const uint16_t* biases,
                            const uint16_t* x, float* y, int B, int64_t N, int64_t K,
                            hipStream_t stream);
hipError_t launch_gemm(const uint32_t* wq, const uint16_t* scales, const uint16_t* biases,
                       const uint16_t* x, float* y, int64_t M, int64_t N, int64_t K,
                       void* workspace, hipStream_t stream);
// Kernel family qmm_gemv runs for a shape (1 = vector ALU, 2 = matrix cores);
// a function of (B, N, K) only.
inline int gemv_auto_family(int B, int64_t N, int64_t K) {
  (void)N;
  (void)K;
  return B >= 5 ? 2 : 1;  // measured: the vector ALUs keep up to B = 4
}
size_t gemm_workspace_bytes(int64_t M, int64_t N, int64_t K);
hipError_t launch_argmax(const void* logits, int dtype, int64_t rows, int64_t vocab, int64_t ld,
                         uint32_t* ids, void* workspace, hipStream_t stream);
size_t argmax_workspace_bytes(int64_t rows, int64_t vocab);

constexpr int kArgmaxBlock = 1024;  // ids per pass-1 record

}  // namespace w4g
