// Prompt product Y[m][n] = sum_k X[m][k] * (q*s + b)[n][k] on the bf16 matrix
// cores of gfx950, for the 4-bit affine group-64 format (TensorFold PR #1437,
// Receipt) with an fp32 result (same PR, commit "Add the pair seam and
// register its kernels with the kernel contract").
//
// Exactness: a code enters the matrix core as the bf16 value 2 + q/8 (the
// nibble OR-ed into the top four mantissa bits of 2.0), which is exact, and
// each product with a bf16 activation is exact in fp32.  Per 64-group the
// matrix core forms P_g = sum_{k in g} x*(2 + q/8); the group's scale is
// applied in fp32, T += (8 s_g) * P_g, in ascending group order.  What remains
// of the affine map, sum_g (b_g - 16 s_g) * X_g with X_g the fp32 group sum of
// x, runs on the matrix cores after the last group: X_g is split exactly into
// three bf16 parts (X = X1 + X2 + X3) and both b_g and -16 s_g are exact bf16
// values, so all six partial products are exact and only the fp32
// accumulation rounds.  Placing the nibble in the top mantissa bits keeps the
// constant part of the expanded code (2 per unit of q/8, a ratio of 16) small,
// so little is lost when it cancels against the -16 s_g X_g term.
// The K order (groups ascending, then the six bias passes) depends on K alone
// (TensorFold PR #1433, step-2 description: prompt rows keep the whole
// matrix's reduction tree).
//
// Tiling: a 256-thread workgroup owns a 128 x 128 tile of Y; each of its four
// waves owns 64 x 64 as 2 x 2 tiles of v_mfma_f32_32x32x16_bf16.  Per group
// the workgroup stages its 128 activation rows (64 bf16 each, permuted into
// the lane order of the code expansion) and its 128 code rows (32 bytes each)
// in LDS; global loads for the next group are issued before the current
// group's matrix-core work.
#include "w4g_internal.h"

namespace w4g {
namespace {

constexpr int kTM = 128, kTN = 128, kThreads = 256;
constexpr int kXPitch = 144;  // bytes per staged activation row (64 bf16 + 16 pad)
constexpr int kCPitch = 32;   // bytes per staged code row (64 codes)
constexpr uint32_t kMagic2 = 0x40004000u;  // bf16 pair (2.0, 2.0)
constexpr uint32_t kOnes = 0x3F803F80u;

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}
__device__ __forceinline__ float bf16_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// Round fp32 to bf16 bits, nearest-even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Natural bf16 pairs (x0,x1),(x2,x3),(x4,x5),(x6,x7) -> (x0,x4),(x1,x5),(x2,x6),(x3,x7),
// the element order of the code expansion below.
__device__ __forceinline__ uint4 permute_block(uint4 v) {
  uint4 p;
  p.x = __builtin_amdgcn_perm(v.z, v.x, 0x05040100u);
  p.y = __builtin_amdgcn_perm(v.z, v.x, 0x07060302u);
  p.z = __builtin_amdgcn_perm(v.w, v.y, 0x05040100u);
  p.w = __builtin_amdgcn_perm(v.w, v.y, 0x07060302u);
  return p;
}

// One code word (8 codes) -> 8 bf16 values 2 + q/8 (q in mantissa bits 3..6)
// in the order q0,q4,q1,q5,q2,q6,q3,q7.
__device__ __forceinline__ bf16x8_t expand_codes(uint32_t w) {
  uint4 p;
  p.x = ((w << 3) & 0x00780078u) | kMagic2;
  p.y = ((w >> 1) & 0x00780078u) | kMagic2;
  p.z = ((w >> 5) & 0x00780078u) | kMagic2;
  p.w = ((w >> 9) & 0x00780078u) | kMagic2;
  return __builtin_bit_cast(bf16x8_t, p);
}

// Group sums of x, split exactly into three bf16 parts:
// xs[m][p*G16 + g] for p = 0, 1, 2 (zero for G <= g < G16).
__global__ __launch_bounds__(kThreads) void xsum_kernel(const uint16_t* __restrict__ x,
                                                        uint16_t* __restrict__ xs, int64_t M,
                                                        int64_t K, int64_t G16) {
  const int64_t G = K >> 6;
  const int64_t t = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (t >= M * G16) return;
  const int64_t m = t / G16, g = t % G16;
  uint32_t parts[3] = {0u, 0u, 0u};
  if (g < G) {
    const uint4* src = reinterpret_cast<const uint4*>(x + m * K + g * 64);
    float h = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint4 v = src[i];
      h = dot2(v.x, kOnes, h);
      h = dot2(v.y, kOnes, h);
      h = dot2(v.z, kOnes, h);
      h = dot2(v.w, kOnes, h);
    }
    const uint32_t a = f32_to_bf16_rne(h);
    const float r1 = h - bf16_to_f32(a);
    const uint32_t b = f32_to_bf16_rne(r1);
    const float r2 = r1 - bf16_to_f32(b);
    parts[0] = a;
    parts[1] = b;
    parts[2] = __float_as_uint(r2) >> 16;  // exact: at most 8 significant bits remain
  }
  uint16_t* dst = xs + m * 3 * G16 + g;
  dst[0] = (uint16_t)parts[0];
  dst[G16] = (uint16_t)parts[1];
  dst[2 * G16] = (uint16_t)parts[2];
}

__global__ __launch_bounds__(kThreads) void gemm_kernel(
    const uint32_t* __restrict__ wq, const uint16_t* __restrict__ scales,
    const uint16_t* __restrict__ biases, const uint16_t* __restrict__ x,
    const uint16_t* __restrict__ xs, float* __restrict__ y, int64_t M, int64_t N, int64_t K,
    int64_t G16) {
  __shared__ __attribute__((aligned(16))) unsigned char s_x[kTM * kXPitch];
  __shared__ __attribute__((aligned(16))) unsigned char s_c[kTN * kCPitch];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave & 1, wn = wave >> 1;
  const int l32 = lane & 31, h = lane >> 5;
  const int64_t m0 = (int64_t)blockIdx.y * kTM;
  const int64_t n0 = (int64_t)blockIdx.x * kTN;
  const int64_t G = K >> 6;
  const int64_t K8 = K >> 3;

  // staging assignment: 4 activation blocks of 16 B and 1 code block of 16 B per thread
  int xrow[4], xcol[4];
  bool xok[4];
  const uint16_t* xsrc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int blk = tid + i * kThreads;
    xrow[i] = blk >> 3;
    xcol[i] = blk & 7;
    xok[i] = (m0 + xrow[i]) < M;
    xsrc[i] = x + (xok[i] ? (m0 + xrow[i]) : 0) * K + xcol[i] * 8;
  }
  const int crow = tid >> 1, chalf = tid & 1;
  const int64_t cn = (n0 + crow < N) ? n0 + crow : N - 1;
  const uint32_t* csrc = wq + cn * K8 + chalf * 4;

  // this lane's output columns (clamped for reads) and their scale rows
  int64_t ncol[2];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const int64_t n = n0 + wn * 64 + nt * 32 + l32;
    ncol[nt] = n < N ? n : N - 1;
  }

  f32x16_t tot[2][2];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int v = 0; v < 16; ++v) tot[mt][nt][v] = 0.0f;

  uint4 px[4], pc;
  const uint4 zero4 = make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
  for (int i = 0; i < 4; ++i) px[i] = xok[i] ? *reinterpret_cast<const uint4*>(xsrc[i]) : zero4;
  pc = *reinterpret_cast<const uint4*>(csrc);

  for (int64_t g = 0; g < G; ++g) {
    __syncthreads();  // previous group's LDS reads are done
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *reinterpret_cast<uint4*>(s_x + xrow[i] * kXPitch + xcol[i] * 16) = permute_block(px[i]);
    *reinterpret_cast<uint4*>(s_c + crow * kCPitch + chalf * 16) = pc;
    __syncthreads();
    if (g + 1 < G) {  // prefetch the next group into registers
#pragma unroll
      for (int i = 0; i < 4; ++i)
        px[i] = xok[i] ? *reinterpret_cast<const uint4*>(xsrc[i] + (g + 1) * 64) : zero4;
      pc = *reinterpret_cast<const uint4*>(csrc + (g + 1) * 8);
    }
    float s[2];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) s[nt] = 8.0f * bf16_to_f32(scales[ncol[nt] * G + g]);

    uint4 cw[2];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
      cw[nt] = *reinterpret_cast<const uint4*>(s_c + (wn * 64 + nt * 32 + l32) * kCPitch + h * 16);
    f32x16_t part[2][2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
#pragma unroll
        for (int v = 0; v < 16; ++v) part[mt][nt][v] = 0.0f;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      bf16x8_t bop[2];
      bop[0] = expand_codes(t == 0 ? cw[0].x : t == 1 ? cw[0].y : t == 2 ? cw[0].z : cw[0].w);
      bop[1] = expand_codes(t == 0 ? cw[1].x : t == 1 ? cw[1].y : t == 2 ? cw[1].z : cw[1].w);
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        const uint4 av = *reinterpret_cast<const uint4*>(
            s_x + (wm * 64 + mt * 32 + l32) * kXPitch + h * 64 + t * 16);
        const bf16x8_t aop = __builtin_bit_cast(bf16x8_t, av);
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
          part[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aop, bop[nt], part[mt][nt], 0, 0, 0);
      }
    }
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
#pragma unroll
        for (int v = 0; v < 16; ++v)
          tot[mt][nt][v] = __builtin_fmaf(s[nt], part[mt][nt][v], tot[mt][nt][v]);
  }

  // bias passes: sum over g of (b_g - 16 s_g) * (X1 + X2 + X3)_g, six exact bf16 products
  for (int p = 0; p < 6; ++p) {
    for (int64_t kk = 0; kk < G16; kk += 16) {
      bf16x8_t aop[2], bop[2];
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        const int64_t m = m0 + wm * 64 + mt * 32 + l32;
        uint4 av = zero4;
        if (m < M)
          av = *reinterpret_cast<const uint4*>(xs + m * 3 * G16 + (p % 3) * G16 + kk + h * 8);
        aop[mt] = __builtin_bit_cast(bf16x8_t, av);
      }
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        uint32_t e[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int64_t g = kk + h * 8 + j;
          uint32_t bits = 0u;
          if (g < G) {
            if (p < 3) {
              bits = biases[ncol[nt] * G + g];
            } else {
              const float v = -16.0f * bf16_to_f32(scales[ncol[nt] * G + g]);
              bits = __float_as_uint(v) >> 16;  // exact: a power-of-two multiple of a bf16
            }
          }
          e[j] = bits;
        }
        uint4 bv;
        bv.x = e[0] | (e[1] << 16);
        bv.y = e[2] | (e[3] << 16);
        bv.z = e[4] | (e[5] << 16);
        bv.w = e[6] | (e[7] << 16);
        bop[nt] = __builtin_bit_cast(bf16x8_t, bv);
      }
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
          tot[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aop[mt], bop[nt], tot[mt][nt], 0, 0, 0);
    }
  }

  // store: lane holds rows 8*(v/4) + 4*h + v%4 of column l32 of each 32 x 32 tile
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      const int64_t n = n0 + wn * 64 + nt * 32 + l32;
      if (n >= N) continue;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int64_t m = m0 + wm * 64 + mt * 32 + 8 * (v >> 2) + 4 * h + (v & 3);
        if (m < M) y[m * N + n] = tot[mt][nt][v];
      }
    }
}

int64_t g16_of(int64_t K) { return (((K >> 6) + 15) / 16) * 16; }

}  // namespace

size_t gemm_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  (void)N;
  return (size_t)(M * 3 * g16_of(K)) * sizeof(uint16_t);
}

hipError_t launch_gemm(const uint32_t* wq, const uint16_t* scales, const uint16_t* biases,
                       const uint16_t* x, float* y, int64_t M, int64_t N, int64_t K,
                       void* workspace, hipStream_t stream) {
  const int64_t G16 = g16_of(K);
  uint16_t* xs = reinterpret_cast<uint16_t*>(workspace);
  const int64_t nt = M * G16;
  hipLaunchKernelGGL(xsum_kernel, dim3((unsigned)((nt + kThreads - 1) / kThreads)), dim3(kThreads),
                     0, stream, x, xs, M, K, G16);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 grid((unsigned)((N + kTN - 1) / kTN), (unsigned)((M + kTM - 1) / kTM));
  hipLaunchKernelGGL(gemm_kernel, grid, dim3(kThreads), 0, stream, wq, scales, biases, x, xs, y, M,
                     N, K, G16);
  return hipGetLastError();
}

}  // namespace w4g
