// Decode product y[b][n] = sum_k x[b][k] * (q*s + b)[n][k] for 1 <= B <= 8,
// 4-bit affine codes with one bf16 scale and bias per 64-group (TensorFold
// PR #1437, Receipt: "4-bit affine with group 64"; fp32 result: same PR,
// commit "Add the pair seam and register its kernels with the kernel
// contract").
//
// Work split: a 32-lane half wave owns R output rows.  It walks K in chunks of
// 1024 elements; in each chunk lane j owns elements [32j, 32j+32), i.e. half
// of one 64-group, and reads them as one 128-bit load per row (the half wave
// reads 512 contiguous bytes of each row).  The four code words are expanded
// in registers to bf16 pairs (128 + q) by OR-ing the nibble into the exponent
// pattern of 128.0, and v_dot2 against bf16 pairs of x accumulates
// D = sum x*(128 + q) in fp32.  The lane then adds s*D + (b - 128 s)*X, X the
// fp32 sum of its 32 x values, so the group's affine map is applied once per
// half group instead of once per weight.  After the last chunk the 32 lane
// sums meet in an xor butterfly.  The order of every floating-point step
// depends on K alone, so a row's bits do not change with N, B or the grid
// (TensorFold PR #1433, step-2 description: the K reduction tree is the full
// matrix's).
#include "w4g_internal.h"

namespace w4g {
namespace {

constexpr int kChunk = 1024;
constexpr uint32_t kMagic128 = 0x43004300u;  // bf16 pair (128.0, 128.0)
constexpr uint32_t kOnes = 0x3F803F80u;      // bf16 pair (1.0, 1.0)

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

// (x[j], x[j+4]) pairs of an 8-element block held as natural pairs
// n0 = (x0,x1), n1 = (x2,x3), n2 = (x4,x5), n3 = (x6,x7).
__device__ __forceinline__ void pair_x(uint32_t n0, uint32_t n1, uint32_t n2, uint32_t n3,
                                       uint32_t* p) {
  p[0] = __builtin_amdgcn_perm(n2, n0, 0x05040100u);  // (x0, x4)
  p[1] = __builtin_amdgcn_perm(n2, n0, 0x07060302u);  // (x1, x5)
  p[2] = __builtin_amdgcn_perm(n3, n1, 0x05040100u);  // (x2, x6)
  p[3] = __builtin_amdgcn_perm(n3, n1, 0x07060302u);  // (x3, x7)
}

// (128 + q[j], 128 + q[j+4]) bf16 pairs of one code word, j = 0..3.
__device__ __forceinline__ void pair_q(uint32_t w, uint32_t* p) {
  p[0] = (w & 0x000F000Fu) | kMagic128;
  p[1] = ((w >> 4) & 0x000F000Fu) | kMagic128;
  p[2] = ((w >> 8) & 0x000F000Fu) | kMagic128;
  p[3] = ((w >> 12) & 0x000F000Fu) | kMagic128;
}

__device__ __forceinline__ float bf16_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

template <int B, int R>
__global__ __launch_bounds__(64) void gemv_valu_kernel(const uint32_t* __restrict__ wq,
                                                       const uint16_t* __restrict__ scales,
                                                       const uint16_t* __restrict__ biases,
                                                       const uint16_t* __restrict__ x,
                                                       float* __restrict__ y, int64_t N,
                                                       int64_t K) {
  const int lane = threadIdx.x & 31;
  const int64_t row0 = ((int64_t)blockIdx.x * 2 + (threadIdx.x >> 5)) * R;
  const int64_t G = K >> 6;
  const int64_t K8 = K >> 3;
  float acc[R][B];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int b = 0; b < B; ++b) acc[r][b] = 0.0f;

  int64_t rows[R];
#pragma unroll
  for (int r = 0; r < R; ++r) rows[r] = (row0 + r < N) ? row0 + r : N - 1;

  const int64_t nchunks = (K + kChunk - 1) / kChunk;
  for (int64_t c = 0; c < nchunks; ++c) {
    const int64_t kb = c * kChunk + (int64_t)lane * 32;
    if (kb < K) {
      uint4 wv[R];
      uint32_t sv[R], bv[R];
#pragma unroll
      for (int r = 0; r < R; ++r) {
        wv[r] = *reinterpret_cast<const uint4*>(wq + rows[r] * K8 + (kb >> 3));
        sv[r] = scales[rows[r] * G + (kb >> 6)];
        bv[r] = biases[rows[r] * G + (kb >> 6)];
      }
      uint32_t xp[B][16];
      float xh[B];
#pragma unroll
      for (int b = 0; b < B; ++b) {
        const uint4* xs = reinterpret_cast<const uint4*>(x + (int64_t)b * K + kb);
        uint4 v0 = xs[0], v1 = xs[1], v2 = xs[2], v3 = xs[3];
        pair_x(v0.x, v0.y, v0.z, v0.w, &xp[b][0]);
        pair_x(v1.x, v1.y, v1.z, v1.w, &xp[b][4]);
        pair_x(v2.x, v2.y, v2.z, v2.w, &xp[b][8]);
        pair_x(v3.x, v3.y, v3.z, v3.w, &xp[b][12]);
        float h = 0.0f;
#pragma unroll
        for (int j = 0; j < 16; ++j) h = dot2(xp[b][j], kOnes, h);
        xh[b] = h;
      }
#pragma unroll
      for (int r = 0; r < R; ++r) {
        uint32_t qp[16];
        pair_q(wv[r].x, &qp[0]);
        pair_q(wv[r].y, &qp[4]);
        pair_q(wv[r].z, &qp[8]);
        pair_q(wv[r].w, &qp[12]);
        const float s = bf16_to_f32(sv[r]);
        const float cb = __builtin_fmaf(-128.0f, s, bf16_to_f32(bv[r]));
#pragma unroll
        for (int b = 0; b < B; ++b) {
          float d = 0.0f;
#pragma unroll
          for (int j = 0; j < 16; ++j) d = dot2(qp[j], xp[b][j], d);
          acc[r][b] = __builtin_fmaf(s, d, acc[r][b]);
          acc[r][b] = __builtin_fmaf(cb, xh[b], acc[r][b]);
        }
      }
    }
  }
#pragma unroll
  for (int r = 0; r < R; ++r) {
#pragma unroll
    for (int b = 0; b < B; ++b) {
      float v = acc[r][b];
      v += __shfl_xor(v, 16);
      v += __shfl_xor(v, 8);
      v += __shfl_xor(v, 4);
      v += __shfl_xor(v, 2);
      v += __shfl_xor(v, 1);
      acc[r][b] = v;
    }
  }
  if (lane == 0) {
#pragma unroll
    for (int r = 0; r < R; ++r)
      if (row0 + r < N)
#pragma unroll
        for (int b = 0; b < B; ++b) y[(int64_t)b * N + row0 + r] = acc[r][b];
  }
}

template <int B, int R>
hipError_t launch_b(const uint32_t* wq, const uint16_t* scales, const uint16_t* biases,
                    const uint16_t* x, float* y, int64_t N, int64_t K, hipStream_t stream) {
  const int64_t rows_per_block = 2 * R;
  const int64_t blocks = (N + rows_per_block - 1) / rows_per_block;
  hipLaunchKernelGGL((gemv_valu_kernel<B, R>), dim3((unsigned)blocks), dim3(64), 0, stream, wq,
                     scales, biases, x, y, N, K);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemv(const uint32_t* wq, const uint16_t* scales, const uint16_t* biases,
                       const uint16_t* x, float* y, int B, int64_t N, int64_t K,
                       hipStream_t stream) {
  switch (B) {
    case 1: return launch_b<1, 4>(wq, scales, biases, x, y, N, K, stream);
    case 2: return launch_b<2, 4>(wq, scales, biases, x, y, N, K, stream);
    case 3: return launch_b<3, 2>(wq, scales, biases, x, y, N, K, stream);
    case 4: return launch_b<4, 2>(wq, scales, biases, x, y, N, K, stream);
    case 5: return launch_b<5, 2>(wq, scales, biases, x, y, N, K, stream);
    case 6: return launch_b<6, 2>(wq, scales, biases, x, y, N, K, stream);
    case 7: return launch_b<7, 2>(wq, scales, biases, x, y, N, K, stream);
    case 8: return launch_b<8, 2>(wq, scales, biases, x, y, N, K, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace w4g
