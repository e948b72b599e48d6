// Decode product on the matrix cores for 1 <= B <= 8 activation rows.
//
// Same format and result as the vector-ALU decode kernel (4-bit affine,
// group 64: TensorFold PR #1437, Receipt; fp32 result: same PR, commit "Add
// the pair seam and register its kernels with the kernel contract"), for
// batches where the vector ALUs cannot keep up with HBM: a 32 x 32 x 16 bf16
// matrix-core instruction multiplies 16 K-elements of 32 weight rows by up to
// 32 activation rows, so every code is expanded once whatever B is.
//
// Operands: A = the activations (rows b < B, the rest zero), B = the codes of
// 32 weight rows, expanded to the exact bf16 values 128 + q.  Lane (h, n) of
// the wave loads 16 bytes of row n: half h of one 64-group, which feeds the
// four instructions of that group (one 32-bit code word each).  The
// activations are staged in LDS per 1024-element chunk, permuted once into
// the order the expansion produces.
//
// Arithmetic per (row n, batch row b): for each group g the matrix core forms
// P = sum_{k in g} x*(128 + q) from zero; the lane then adds s*P and
// (b_g - 128 s) * X_g, X_g the fp32 sum of the group's activations, in fp32.
// X_g is the sum of the group's two 32-element halves, each summed over its
// natural bf16 pairs in ascending order.  Wave w of the workgroup takes the
// groups g = w (mod W) in ascending order; the W wave sums are added in
// ascending wave order at the end.  The order
// depends on K alone (TensorFold PR #1433, step-2 description), and every
// batch row is computed independently of the others.
#include "w4g_internal.h"

namespace w4g {
namespace {

constexpr int kStageGroups = 16;  // groups per staged activation chunk (1024 elements)
constexpr int kXRows = 10;        // LDS rows per activation block
constexpr uint32_t kMagic128 = 0x43004300u;
constexpr uint32_t kOnes = 0x3F803F80u;

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}
__device__ __forceinline__ float bf16_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

__device__ __forceinline__ uint4 permute_block(uint4 v) {
  uint4 p;
  p.x = __builtin_amdgcn_perm(v.z, v.x, 0x05040100u);
  p.y = __builtin_amdgcn_perm(v.z, v.x, 0x07060302u);
  p.z = __builtin_amdgcn_perm(v.w, v.y, 0x05040100u);
  p.w = __builtin_amdgcn_perm(v.w, v.y, 0x07060302u);
  return p;
}

// (a & m) | g in one instruction (the compiler would emit two with literals)
__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t m, uint32_t g) {
  uint32_t d;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(d) : "v"(a), "s"(m), "v"(g));
  return d;
}

// The largest 64-bit word over the 32 lanes of each half wave, in every lane
// of that half: partners across the two 16-lane rows, then within a row by
// mirrors and quad swaps (each step pairs every lane with one whose set of
// covered lanes is disjoint from its own, so the last step covers all 32).
template <int CTRL>
__device__ __forceinline__ uint64_t dpp_max64(uint64_t c) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)c, CTRL, 0xF, 0xF, false);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)(c >> 32), CTRL, 0xF, 0xF, false);
  return umax64(c, ((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ uint64_t half_wave_max64(uint64_t c) {
  const auto l = __builtin_amdgcn_permlane16_swap((uint32_t)c, (uint32_t)c, false, false);
  const auto h = __builtin_amdgcn_permlane16_swap((uint32_t)(c >> 32), (uint32_t)(c >> 32), false, false);
  c = umax64(((uint64_t)h[0] << 32) | l[0], ((uint64_t)h[1] << 32) | l[1]);
  c = dpp_max64<0x140>(c);  // row_mirror
  c = dpp_max64<0x141>(c);  // row_half_mirror
  c = dpp_max64<0x4E>(c);   // quad_perm [2,3,0,1]
  c = dpp_max64<0xB1>(c);   // quad_perm [1,0,3,2]
  return c;
}

// 8 codes -> bf16 values 128 + q in the order q0,q4,q1,q5,q2,q6,q3,q7
__device__ __forceinline__ bf16x8_t expand128(uint32_t w, uint32_t m, uint32_t g) {
  uint4 p;
  p.x = and_or(w, m, g);
  p.y = and_or(w >> 4, m, g);
  p.z = and_or(w >> 8, m, g);
  p.w = and_or(w >> 12, m, g);
  return __builtin_bit_cast(bf16x8_t, p);
}

__device__ __forceinline__ uint32_t word(const uint4& v, int t) {
  return t == 0 ? v.x : t == 1 ? v.y : t == 2 ? v.z : v.w;
}

// Codes, scales and biases of one stage of one wave.  VEC: the scales and
// biases come as one 16-byte vector per lane (lane (h, n): groups 8h .. 8h + 7
// of the stage for row n; a 2-byte load per group and row would cost an L1
// tag lookup per lane), else one 2-byte load per group.
template <int GPS, bool VEC>
struct Ring {
  uint4 c[GPS];
  uint32_t s[VEC ? 1 : GPS], b[VEC ? 1 : GPS];
  uint4 sv, bv;
};

__device__ __forceinline__ uint32_t bf16_at(const uint4& v, int i) {
  const uint32_t w = i >> 1 == 0 ? v.x : i >> 1 == 1 ? v.y : i >> 1 == 2 ? v.z : v.w;
  return (w >> ((i & 1) * 16)) & 0xFFFFu;
}

// The workgroup's four waves split the K groups round robin; each stage of 16
// groups gives every wave GPS = 16 / W of them.  The activations of a stage are
// staged in one of two LDS buffers while the other feeds the matrix cores.
//
// AM adds the argmax's pass 1 as an epilogue: per batch row, the best (value,
// lowest row) of the workgroup's 32 rows, or the non-finite flag, goes to
// rec[b][blockIdx.x] (one record per 32 rows); y may then be null.
template <int W, bool VEC, bool AM>
__global__ __launch_bounds__(64 * W) void gemv_mfma_kernel(const uint32_t* __restrict__ wq,
                                                           const uint16_t* __restrict__ scales,
                                                           const uint16_t* __restrict__ biases,
                                                           const uint16_t* __restrict__ x,
                                                           float* __restrict__ y, int B, int64_t N,
                                                           int64_t K, uint2* __restrict__ rec) {
  constexpr int GPS = kStageGroups / W;
  // [buf][8-element block][slot]: slots 0..7 hold the batch rows (row r of
  // block k at slot r ^ ((k >> 3) & 7), so the staging writes of different
  // groups land in different banks), slot 8 zeros, slot 9 padding so the two
  // half-group reads of a wave fall in different banks
  __shared__ uint4 s_x[2][kStageGroups * 8][kXRows];
  __shared__ float s_X[2][8][kStageGroups];      // [buf][b][group]: group sums
  __shared__ float s_red[W][4][64];              // wave sums

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int l32 = lane & 31, h = lane >> 5;
  const int arow = l32 < 8 ? l32 : 8;  // activation row this lane feeds; rows >= B are zero
  const uint32_t m = 0x000F000Fu, g = kMagic128;
  const int64_t n0 = (int64_t)blockIdx.x * 32;
  const int64_t n = (n0 + l32 < N) ? n0 + l32 : N - 1;
  const int64_t G = K >> 6;
  const int nstage = (int)((G + kStageGroups - 1) / kStageGroups);
  const uint32_t* wrow = wq + n * (K >> 3);
  const uint16_t* srow = scales + n * G;
  const uint16_t* brow = biases + n * G;

  // codes of stage st for this wave (groups past the end reread the row's last
  // group, a cache hit, so no other rows are pulled in)
  auto issue = [&](Ring<GPS, VEC>& r, int st) {
#pragma unroll
    for (int j = 0; j < GPS; ++j) {
      int64_t g = (int64_t)st * kStageGroups + wave + W * j;
      g = g < G ? g : G - 1;
      r.c[j] = *reinterpret_cast<const uint4*>(wrow + g * 8 + h * 4);
      if constexpr (!VEC) {
        r.s[j] = srow[g];
        r.b[j] = brow[g];
      }
    }
    if constexpr (VEC) {  // G % 8 == 0: clamp the block start to the row's last 8 groups
      int64_t g8 = (int64_t)st * kStageGroups + 8 * h;
      g8 = g8 <= G - 8 ? g8 : G - 8;
      r.sv = *reinterpret_cast<const uint4*>(srow + g8);
      r.bv = *reinterpret_cast<const uint4*>(brow + g8);
    }
  };

  // activation staging: thread -> (row xb, group xg, half xh) of a stage, 32 elements
  const int xb = tid >> 5, xg = (tid & 31) >> 1, xhalf = tid & 1;
  const bool xload = (64 * W >= 256) && xb < B;
  uint4 xr[4];
  auto load_x = [&](int st) {
    const int64_t g = (int64_t)st * kStageGroups + xg;
    const bool ok = xload && st < nstage && g < G;
    const uint4* src = reinterpret_cast<const uint4*>(x + (ok ? (int64_t)xb * K + g * 64 + xhalf * 32 : 0));
#pragma unroll
    for (int i = 0; i < 4; ++i) xr[i] = ok ? src[i] : make_uint4(0u, 0u, 0u, 0u);
  };
  auto store_x = [&](int buf) {
    float part = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      s_x[buf][xg * 8 + xhalf * 4 + i][xb ^ (xg & 7)] = permute_block(xr[i]);
      part = dot2(xr[i].x, kOnes, part);
      part = dot2(xr[i].y, kOnes, part);
      part = dot2(xr[i].z, kOnes, part);
      part = dot2(xr[i].w, kOnes, part);
    }
    const float other = __shfl_xor(part, 1);
    if (xhalf == 0) s_X[buf][xb][xg] = part + other;  // first half + second half
  };

  float tot[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  // The stage's GPS groups run their four-instruction matrix-core chains side
  // by side (instruction t of every group, then t + 1), so the chains overlap;
  // each group's partial is still its own, and the groups are added to the
  // running sums in ascending order.
  auto compute = [&](const Ring<GPS, VEC>& r, int st, int buf) {
    f32x16_t p[GPS];
    bf16x8_t bop[GPS][4];
    uint4 av[GPS][4];
#pragma unroll
    for (int j = 0; j < GPS; ++j) {
      const int gl = wave + W * j;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        av[j][t] = s_x[buf][gl * 8 + h * 4 + t][arow < 8 ? arow ^ (gl & 7) : 8];
        bop[j][t] = expand128(word(r.c[j], t), m, g);
      }
#pragma unroll
      for (int v = 0; v < 16; ++v) p[j][v] = 0.0f;
    }
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int j = 0; j < GPS; ++j)
        p[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, av[j][t]),
                                                       bop[j][t], p[j], 0, 0, 0);
#pragma unroll
    for (int j = 0; j < GPS; ++j) {
      const int gl = wave + W * j;
      if ((int64_t)st * kStageGroups + gl < G) {
        uint32_t sbits, bbits;
        if constexpr (VEC) {
          // this lane's vector holds the group when gl / 8 == h, else its partner's does
          const uint32_t so = bf16_at(r.sv, gl & 7), bo = bf16_at(r.bv, gl & 7);
          const uint32_t sp = __shfl_xor(so, 32), bp = __shfl_xor(bo, 32);
          sbits = (gl >> 3) == h ? so : sp;
          bbits = (gl >> 3) == h ? bo : bp;
        } else {
          sbits = r.s[j];
          bbits = r.b[j];
        }
        const float sc = bf16_to_f32(sbits);
        const float cb = __builtin_fmaf(-128.0f, sc, bf16_to_f32(bbits));
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          tot[v] = __builtin_fmaf(sc, p[j][v], tot[v]);
          tot[v] = __builtin_fmaf(cb, s_X[buf][4 * h + v][gl], tot[v]);
        }
      }
    }
  };

  // the zero slot that lanes 8..31 read as their activation operand
  for (int i = tid; i < 2 * kStageGroups * 8; i += 64 * W)
    s_x[i / (kStageGroups * 8)][i % (kStageGroups * 8)][8] = make_uint4(0u, 0u, 0u, 0u);

  // Per half step: activations of stage st + 2 load first, then its codes, so
  // the wait for stage st + 1's activations (issued a half step earlier) does
  // not also wait for codes that are only needed later.
  Ring<GPS, VEC> ra, rb;
  load_x(0);
  issue(ra, 0);
  store_x(0);
  load_x(1);
  issue(rb, 1);
  __syncthreads();
  for (int st = 0; st < nstage; st += 2) {
    // xr holds stage st + 1
    compute(ra, st, 0);
    store_x(1);  // stage st + 1 (zeros past the end)
    load_x(st + 2);
    issue(ra, st + 2);
    __syncthreads();
    compute(rb, st + 1, 1);  // no-op past the last stage
    store_x(0);  // stage st + 2
    load_x(st + 3);
    issue(rb, st + 3);
    __syncthreads();
  }

#pragma unroll
  for (int v = 0; v < 4; ++v) s_red[wave][v][lane] = tot[v];
  __syncthreads();
  {
    // wave v finishes column v of every lane: batch row b = 4 h + v, weight row
    // n0 + l32 (the wave sums added in ascending wave order)
    static_assert(W == 4, "one output column per wave");
    const int v = wave;
    float acc = s_red[0][v][lane];
#pragma unroll
    for (int w = 1; w < W; ++w) acc += s_red[w][v][lane];
    const int b = 4 * h + v;
    const bool valid = n0 + l32 < N;
    if (b < B && valid && (!AM || y != nullptr)) y[(int64_t)b * N + n0 + l32] = acc;
    if constexpr (AM) {
      // the best candidate over the 32 rows of this half wave's batch row
      const uint32_t u = __float_as_uint(acc);
      const bool bad = valid && !finite_bits(u);
      const uint64_t c = half_wave_max64((valid && !bad) ? cand(u, (uint32_t)(n0 + l32)) : 0);
      const uint64_t badm = __ballot(bad);
      const bool half_bad = ((badm >> (32 * h)) & 0xFFFFFFFFull) != 0;
      if (l32 == 0 && b < B)
        rec[(int64_t)b * gridDim.x + blockIdx.x] = make_record(c, half_bad, (uint32_t)n0);
    }
  }
}

template <bool AM>
hipError_t launch(const uint32_t* wq, const uint16_t* scales, const uint16_t* biases,
                  const uint16_t* x, float* y, uint2* rec, int B, int64_t N, int64_t K,
                  hipStream_t stream) {
  const int64_t blocks = (N + 31) / 32;
  const bool vec = ((K >> 6) % 8) == 0 && ((reinterpret_cast<uintptr_t>(scales) |
                                             reinterpret_cast<uintptr_t>(biases)) & 15u) == 0;
  if (vec)
    hipLaunchKernelGGL((gemv_mfma_kernel<4, true, AM>), dim3((unsigned)blocks), dim3(256), 0, stream, wq,
                       scales, biases, x, y, B, N, K, rec);
  else
    hipLaunchKernelGGL((gemv_mfma_kernel<4, false, AM>), dim3((unsigned)blocks), dim3(256), 0, stream, wq,
                       scales, biases, x, y, B, N, K, rec);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemv_mfma(const uint32_t* wq, const uint16_t* scales, const uint16_t* biases,
                            const uint16_t* x, float* y, int B, int64_t N, int64_t K,
                            hipStream_t stream) {
  return launch<false>(wq, scales, biases, x, y, nullptr, B, N, K, stream);
}

int64_t gemv_mfma_argmax_records(int64_t N) { return (N + 31) / 32; }

hipError_t launch_gemv_mfma_argmax(const uint32_t* wq, const uint16_t* scales, const uint16_t* biases,
                                   const uint16_t* x, float* y, uint2* rec, int B, int64_t N, int64_t K,
                                   hipStream_t stream) {
  return launch<true>(wq, scales, biases, x, y, rec, B, N, K, stream);
}

}  // namespace w4g
