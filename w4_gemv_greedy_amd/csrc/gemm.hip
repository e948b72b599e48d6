// Prompt product Y[m][n] = sum_k X[m][k] * (q*s + b)[n][k] on the bf16 matrix
// cores of gfx950, for the 4-bit affine group-64 format (TensorFold PR #1437,
// Receipt) with an fp32 result (same PR, commit "Add the pair seam and
// register its kernels with the kernel contract").
//
// Exactness: a code enters the matrix core as the bf16 value 2 + q/8 (the
// nibble OR-ed into the top four mantissa bits of 2.0), which is exact, and
// each product with a bf16 activation is exact in fp32.  Per 64-group the
// matrix core forms P_g = sum_{k in g} x*(2 + q/8) from zero (four
// v_mfma_f32_32x32x16_bf16); the group's scale is applied in fp32,
// T += (8 s_g) * P_g, in ascending group order.  What remains of the affine
// map, sum_g (b_g - 16 s_g) * X_g with X_g the fp32 group sum of x, runs on the
// matrix cores after the last group: X_g is split exactly into three bf16
// parts (X = X1 + X2 + X3) and both b_g and -16 s_g are exact bf16 values, so
// all six partial products are exact and only the fp32 accumulation rounds.
// Placing the nibble in the top mantissa bits keeps the constant part of the
// expanded code (2 per unit of q/8, a ratio of 16) small, so little is lost
// when it cancels against the -16 s_g X_g term.  The K order (groups
// ascending; then, for each block of 16 groups in ascending order, the bias
// products b X1, b X2, b X3, -16s X1, -16s X2, -16s X3) depends on K alone
// (TensorFold PR #1433, step-2 description: prompt rows keep the whole
// matrix's reduction tree), and no output depends on M, on the other rows or
// on which of the two kernels below ran.
//
// Work split: a pre-pass writes x permuted into the element order of the code
// expansion, and the exact three-part group sums.  A workgroup of four waves
// owns a 128 x 128 tile of Y, each wave 64 x 64 (2 x 2 matrix-core tiles); the
// tile's activations, codes and scales go through LDS one or two groups at a
// time.  Two main loops share that arithmetic: one stages the operands
// through registers (small enough for two workgroups per CU), the other loads
// them straight into a three-stage LDS ring (one workgroup per CU, deeper
// prefetch), taken when the grid is too small to place two workgroups per CU.
#include <algorithm>

#include "w4g_internal.h"

namespace w4g {
namespace {

constexpr int kThreads = 256;
constexpr uint32_t kMagic2 = 0x40004000u;  // bf16 pair (2.0, 2.0)
constexpr uint32_t kOnes = 0x3F803F80u;

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}
__device__ __forceinline__ float bf16_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// (a & m) | g in one instruction (the compiler would emit two with literals)
__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t m, uint32_t g) {
  uint32_t d;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(d) : "v"(a), "s"(m), "v"(g));
  return d;
}

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
__device__ __forceinline__ bf16x8_t expand_codes(uint32_t w, uint32_t m, uint32_t g) {
  uint4 p;
  p.x = and_or(w << 3, m, g);
  p.y = and_or(w >> 1, m, g);
  p.z = and_or(w >> 5, m, g);
  p.w = and_or(w >> 9, m, g);
  return __builtin_bit_cast(bf16x8_t, p);
}

__device__ __forceinline__ uint32_t word(const uint4& v, int t) {
  return t == 0 ? v.x : t == 1 ? v.y : t == 2 ? v.z : v.w;
}

// Pre-pass, one thread per (row m, group g):
//   xp[m][g*64 + ...] = the group's 64 activations permuted block by block;
//   xs[m][p*G16 + g]  = part p of the group sum (zero for G <= g < G16).
__global__ __launch_bounds__(kThreads) void xprep_kernel(const uint16_t* __restrict__ x,
                                                         uint16_t* __restrict__ xp,
                                                         uint16_t* __restrict__ xs, int64_t M,
                                                         int64_t K, int64_t G16) {
  const int64_t G = K >> 6;
  const int64_t t = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (t >= M * G16) return;
  const int64_t m = t / G16, g = t % G16;
  uint32_t parts[3] = {0u, 0u, 0u};
  if (g < G) {
    const uint4* src = reinterpret_cast<const uint4*>(x + m * K + g * 64);
    uint4* dst = reinterpret_cast<uint4*>(xp + m * K + g * 64);
    float h = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint4 v = src[i];
      dst[i] = permute_block(v);
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

// The affine remainder and the store, shared by both main loops: for each block of 16
// groups (ascending), b X1, b X2, b X3, (-16 s) X1, (-16 s) X2, (-16 s) X3, each an
// exact bf16 product on the matrix cores; `vec` (G % 8 == 0 and 16-byte aligned scale
// and bias tables) allows 16-byte loads.  The wave's tile starts at row mw, column nw.
template <int TI, int TJ>
__device__ __forceinline__ void bias_and_store(f32x16_t (&tot)[TI][TJ], const uint16_t* __restrict__ scales,
                                               const uint16_t* __restrict__ biases,
                                               const uint16_t* __restrict__ xs, float* __restrict__ y,
                                               int64_t M, int64_t N, int64_t G, int64_t G16, int64_t ldy,
                                               int64_t mw, int64_t nw, int l32, int h, bool vec) {
  for (int64_t kk = 0; kk < G16; kk += 16) {
    uint4 ax[TI][3];
#pragma unroll
    for (int i = 0; i < TI; ++i) {
      const int64_t m = mw + i * 32 + l32;
#pragma unroll
      for (int q = 0; q < 3; ++q) {
        ax[i][q] = make_uint4(0u, 0u, 0u, 0u);
        if (m < M)
          ax[i][q] = *reinterpret_cast<const uint4*>(xs + m * 3 * G16 + q * G16 + kk + h * 8);
      }
    }
    bf16x8_t bb[TJ], bs[TJ];
#pragma unroll
    for (int j = 0; j < TJ; ++j) {
      int64_t n = nw + j * 32 + l32;
      n = n < N ? n : N - 1;
      const int64_t g0 = kk + h * 8;
      uint32_t eb[8], es[8];
      if (vec && g0 + 8 <= G) {
        const uint4 rb = *reinterpret_cast<const uint4*>(biases + n * G + g0);
        const uint4 rs = *reinterpret_cast<const uint4*>(scales + n * G + g0);
        const uint32_t wb[4] = {rb.x, rb.y, rb.z, rb.w};
        const uint32_t ws[4] = {rs.x, rs.y, rs.z, rs.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          eb[2 * q] = wb[q] & 0xFFFFu;
          eb[2 * q + 1] = wb[q] >> 16;
          es[2 * q] = ws[q] & 0xFFFFu;
          es[2 * q + 1] = ws[q] >> 16;
        }
      } else {
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const bool in = g0 + q < G;
          eb[q] = in ? (uint32_t)biases[n * G + g0 + q] : 0u;
          es[q] = in ? (uint32_t)scales[n * G + g0 + q] : 0u;
        }
      }
#pragma unroll
      for (int q = 0; q < 8; ++q)  // -16 s, exact: a power-of-two multiple of a bf16
        es[q] = __float_as_uint(-16.0f * bf16_to_f32(es[q])) >> 16;
      uint4 vb, vs;
      vb.x = eb[0] | (eb[1] << 16);
      vb.y = eb[2] | (eb[3] << 16);
      vb.z = eb[4] | (eb[5] << 16);
      vb.w = eb[6] | (eb[7] << 16);
      vs.x = es[0] | (es[1] << 16);
      vs.y = es[2] | (es[3] << 16);
      vs.z = es[4] | (es[5] << 16);
      vs.w = es[6] | (es[7] << 16);
      bb[j] = __builtin_bit_cast(bf16x8_t, vb);
      bs[j] = __builtin_bit_cast(bf16x8_t, vs);
    }
#pragma unroll
    for (int pass = 0; pass < 6; ++pass)
#pragma unroll
      for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int j = 0; j < TJ; ++j)
          tot[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              __builtin_bit_cast(bf16x8_t, ax[i][pass % 3]), pass < 3 ? bb[j] : bs[j], tot[i][j],
              0, 0, 0);
  }

  // store: lane holds rows 8*(v/4) + 4*h + v%4 of column l32 of each 32 x 32 tile
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j) {
      const int64_t n = nw + j * 32 + l32;
      if (n >= N) continue;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int64_t m = mw + i * 32 + 8 * (v >> 2) + 4 * h + (v & 3);
        if (m < M) y[m * ldy + n] = tot[i][j][v];
      }
    }
}

// Workgroup tile 128 x 128 of Y, four waves in a 2 x 2 grid, each owning 64 x 64
// (2 x 2 matrix-core tiles).  Per 64-group one stage holds in LDS
//   A: 128 rows x 64 permuted activations (16-byte chunk c of row r stored at
//      chunk c ^ (r & 7), so a wave's reads of one chunk column spread over
//      the banks),
//   B: the 128 columns' code halves, [half][column] x 16 bytes,
//   S: the 128 columns' scales.
// Global loads run two groups ahead in registers, and LDS is double-buffered,
// with one barrier per group.
constexpr int kTM = 128, kTN = 128;
constexpr int kAStage = kTM * 128;
constexpr int kBStage = 2 * kTN * 16;
constexpr int kSStage = kTN * 2;
constexpr int kStage = kAStage + kBStage + kSStage;
constexpr int kRsrcWord3 = 0x00020000;  // buffer descriptor word 3 (gfx9 family): raw dword data

typedef uint32_t v4u __attribute__((ext_vector_type(4)));  // plain vector: copies stay in registers

// one group's activations for the workgroup tile (this thread's share) ...
struct StagedA {
  v4u a[4];
};
// ... and its codes and scales, which come from HBM and are fetched a group earlier
struct StagedB {
  v4u b;
  uint16_t s;
};

__global__ __launch_bounds__(256) void gemm_kernel(
    const uint32_t* __restrict__ wq, const uint16_t* __restrict__ scales,
    const uint16_t* __restrict__ biases, const uint16_t* __restrict__ xp,
    const uint16_t* __restrict__ xs, float* __restrict__ y, int64_t M, int64_t N, int64_t K,
    int64_t ldy, int64_t G16, int64_t NT, int64_t tiles, int64_t per, bool vec) {
  __shared__ __attribute__((aligned(16))) unsigned char smem[2 * kStage];
  const int tid = threadIdx.x;
  // tiles are numbered row-major; consecutive workgroups go to different XCDs,
  // so hand each XCD a contiguous run of tiles (shared activation rows in its L2)
  const int b = blockIdx.x;
  const int tile = (b & 7) * (int)per + (b >> 3);
  if (tile >= (int)tiles) return;
  // wave-uniform by construction; readfirstlane keeps the descriptors in SGPRs
  const int mt = __builtin_amdgcn_readfirstlane(tile / (int)NT);
  const int nt = __builtin_amdgcn_readfirstlane(tile - mt * (int)NT);
  const int64_t m0 = (int64_t)mt * kTM, n0 = (int64_t)nt * kTN;
  const int64_t G = K >> 6;
  const int64_t K8 = K >> 3;

  // staging: thread tid moves A chunk (tid & 7) of rows (tid >> 3) + 32 i, the
  // code half (tid & 1) of column tid >> 1, and the scale of column tid & 127.
  // Buffer loads: the per-lane offsets stay fixed, the group offset is scalar,
  // and reads past a buffer's end (rows >= M, columns >= N, groups >= G of the
  // last row) return zero instead of faulting; the host keeps every buffer
  // below 2^31 bytes.
  const int srow = tid >> 3, sch = tid & 7;
  const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(xp + m0 * K), (short)0, (int)((M - m0) * K * 2), kRsrcWord3);
  const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint32_t*>(wq + n0 * K8), (short)0, (int)((N - n0) * K8 * 4), kRsrcWord3);
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(scales + n0 * G), (short)0, (int)((N - n0) * G * 2), kRsrcWord3);
  const int xa_off = (int)(srow * K * 2) + sch * 16;  // + 32 i rows
  const int xa_step = (int)(32 * K * 2);
  const int bcol = tid >> 1, bh = tid & 1;
  const int wb_off = (int)(bcol * K8 * 4) + bh * 16;
  const int scol = tid & (kTN - 1);
  const int ws_off = (int)(scol * G * 2);
  const int a_w = srow * 128 + ((sch ^ (srow & 7)) << 4);  // + 32 i * 128
  const int b_w = kAStage + bh * (kTN * 16) + bcol * 16;
  const int s_w = kAStage + kBStage + scol * 2;

  auto gload_a = [&](StagedA& r, int g) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      r.a[i] = __builtin_amdgcn_raw_buffer_load_b128(rx, xa_off + i * xa_step, g * 128, 0);
  };
  auto gload_b = [&](StagedB& r, int g) __attribute__((always_inline)) {
    r.b = __builtin_amdgcn_raw_buffer_load_b128(rw, wb_off, g * 32, 0);
    r.s = __builtin_amdgcn_raw_buffer_load_b16(rs, ws_off, g * 2, 0);
  };
  auto sstore = [&](const StagedA& ra, const StagedB& rb, int buf) __attribute__((always_inline)) {
    unsigned char* base = smem + buf * kStage;
#pragma unroll
    for (int i = 0; i < 4; ++i) *reinterpret_cast<v4u*>(base + a_w + i * 32 * 128) = ra.a[i];
    *reinterpret_cast<v4u*>(base + b_w) = rb.b;
    if (tid < kTN) *reinterpret_cast<uint16_t*>(base + s_w) = rb.s;
  };

  // compute: wave (wm, wn), lane (h, l32)
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int lane = tid & 63, l32 = lane & 31, h = lane >> 5;
  int a_r[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int t = 0; t < 4; ++t)
      a_r[i][t] = (wm * 64 + i * 32 + l32) * 128 + ((((t + 4 * h) ^ (l32 & 7))) << 4);
  int b_r[2], s_r[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    b_r[j] = kAStage + h * (kTN * 16) + (wn * 64 + j * 32 + l32) * 16;
    s_r[j] = kAStage + kBStage + (wn * 64 + j * 32 + l32) * 2;
  }
  const uint32_t msk = 0x00780078u, mg = kMagic2;

  f32x16_t tot[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) tot[i][j][v] = 0.0f;

  auto compute = [&](int buf) __attribute__((always_inline)) {
    const unsigned char* base = smem + buf * kStage;
    bf16x8_t bop[2][4];
    float s8[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const v4u c = *reinterpret_cast<const v4u*>(base + b_r[j]);
      s8[j] = 8.0f * bf16_to_f32(*reinterpret_cast<const uint16_t*>(base + s_r[j]));
      bop[j][0] = expand_codes(c.x, msk, mg);
      bop[j][1] = expand_codes(c.y, msk, mg);
      bop[j][2] = expand_codes(c.z, msk, mg);
      bop[j][3] = expand_codes(c.w, msk, mg);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      v4u a[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) a[t] = *reinterpret_cast<const v4u*>(base + a_r[i][t]);
      f32x16_t p[2];
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) p[j][v] = 0.0f;
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          p[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a[t]),
                                                         bop[j][t], p[j], 0, 0, 0);
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) tot[i][j][v] = __builtin_fmaf(s8[j], p[j][v], tot[i][j][v]);
    }
  };

  // pipeline: LDS buffer g % 2 holds group g while the activations of group g + 1
  // and the codes of groups g + 1 and g + 2 are in flight in registers
  const int Gi = (int)G;
  StagedA ra;
  StagedB rb0, rb1;
  gload_a(ra, 0);
  gload_b(rb0, 0);
  gload_b(rb1, 1);
  sstore(ra, rb0, 0);
  __syncthreads();
  for (int g = 0; g < Gi; g += 2) {
    gload_a(ra, g + 1);
    gload_b(rb0, g + 2);
    __builtin_amdgcn_sched_barrier(0);
    compute(0);
    __builtin_amdgcn_sched_barrier(0);
    sstore(ra, rb1, 1);
    __syncthreads();
    if (g + 1 >= Gi) break;
    gload_a(ra, g + 2);
    gload_b(rb1, g + 3);
    __builtin_amdgcn_sched_barrier(0);
    compute(1);
    __builtin_amdgcn_sched_barrier(0);
    sstore(ra, rb0, 0);
    __syncthreads();
  }

  bias_and_store<2, 2>(tot, scales, biases, xs, y, M, N, G, G16, ldy, m0 + wm * 64, n0 + wn * 64, l32,
                       h, vec);
}

// The same tile walk with the operands moved by buffer loads straight into LDS
// (no staging registers), two groups per stage and three stages in flight, so a
// stage's loads are issued two stages before it is used.  Used when G is even
// (whole stages) and the scale table is 4-byte aligned (one dword per column
// carries a stage's two scales).  Per stage, in LDS:
//   A: 128 rows x 256 bytes, 16-byte chunk c (of the two groups' 16) of row r
//      at position c ^ (r & 15);
//   B: 128 columns x 64 bytes (group-in-stage, half) pieces, piece q of column n
//      at position q ^ ((n >> 2) & 3);
//   S: 128 columns x the two groups' scales.
// Every wave issues exactly 11 of these loads per stage, so waiting for all but
// the newest 11 completes the older stage.  Per output the arithmetic and its
// order are those of gemm_kernel: both kernels give the same bits.
constexpr int kDStageA = kTM * 256;
constexpr int kDStageB = kTN * 64;
constexpr int kDStageS = kTN * 4;
constexpr int kDStage = kDStageA + kDStageB + kDStageS;
constexpr int kDStages = 3;
constexpr int kCUs = 256;  // compute units of the MI355X

// Buffer load of 16 bytes per lane into LDS at m0 + 16 * lane.
__device__ __forceinline__ void dma16(uint32_t lds, uint32_t voff, __amdgpu_buffer_rsrc_t r, uint32_t soff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :: "s"(lds), "v"(voff), "s"(r), "s"(soff) : "memory");
}
// Buffer load of 4 bytes per lane into LDS at m0 + 4 * lane.
__device__ __forceinline__ void dma4(uint32_t lds, uint32_t voff, __amdgpu_buffer_rsrc_t r, uint32_t soff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, %3 offen lds"
               :: "s"(lds), "v"(voff), "s"(r), "s"(soff) : "memory");
}

__global__ __launch_bounds__(256) void gemm_dma_kernel(
    const uint32_t* __restrict__ wq, const uint16_t* __restrict__ scales,
    const uint16_t* __restrict__ biases, const uint16_t* __restrict__ xp,
    const uint16_t* __restrict__ xs, float* __restrict__ y, int64_t M, int64_t N, int64_t K,
    int64_t ldy, int64_t G16, int64_t NT, int64_t tiles, int64_t per, bool vec) {
  __shared__ __attribute__((aligned(16))) unsigned char smem[kDStages * kDStage];
  const int tid = threadIdx.x;
  const int b = blockIdx.x;
  const int tile = (b & 7) * (int)per + (b >> 3);
  if (tile >= (int)tiles) return;
  const int mt = __builtin_amdgcn_readfirstlane(tile / (int)NT);
  const int nt = __builtin_amdgcn_readfirstlane(tile - mt * (int)NT);
  const int64_t m0 = (int64_t)mt * kTM, n0 = (int64_t)nt * kTN;
  const int G = (int)(K >> 6);
  const int K8 = (int)(K >> 3);
  const int ns = G >> 1;
  const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(xp + m0 * K), (short)0, (int)((M - m0) * K * 2), kRsrcWord3);
  const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint32_t*>(wq + n0 * K8), (short)0, (int)((N - n0) * K8 * 4), kRsrcWord3);
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(scales + n0 * G), (short)0, (int)((N - n0) * G * 2), kRsrcWord3);

  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  // loads: lane offsets per instruction (rows 4 blk .. 4 blk + 3 of A, columns
  // 16 blk .. 16 blk + 15 of B, columns 32 wave + lane of S for lanes < 32)
  uint32_t va[8], vb[2];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int rr = 32 * wave + 4 * i + (lane >> 4);
    const int c = (lane & 15) ^ (rr & 15);
    va[i] = (uint32_t)(rr * K * 2 + c * 16);
  }
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int col = 16 * (2 * wave + j) + (lane >> 2);
    const int q = (lane & 3) ^ ((col >> 2) & 3);
    vb[j] = (uint32_t)(col * (K8 * 4) + q * 16);
  }
  const uint32_t vsc = (uint32_t)((32 * wave + (lane & 31)) * G * 2);
  const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) unsigned char*)smem;
  auto issue = [&](int s) __attribute__((always_inline)) {
    const uint32_t base = lds0 + (uint32_t)((s % kDStages) * kDStage);
#pragma unroll
    for (int i = 0; i < 8; ++i)
      dma16(__builtin_amdgcn_readfirstlane(base + (8 * wave + i) * 1024), va[i], rx, (uint32_t)(s * 256));
#pragma unroll
    for (int j = 0; j < 2; ++j)
      dma16(__builtin_amdgcn_readfirstlane(base + kDStageA + (2 * wave + j) * 1024), vb[j], rw,
            (uint32_t)(s * 64));
    const uint32_t sbase = __builtin_amdgcn_readfirstlane(base + kDStageA + kDStageB + wave * 128);
    if (lane < 32) dma4(sbase, vsc, rs, (uint32_t)(s * 4));
  };

  // compute: wave (wm, wn) owns rows 64 wm.., columns 64 wn.. of the tile; lane
  // (h, l32) feeds row l32 of a row tile and column l32 of a column tile, half h
  // of each 16-element step
  const int wm = wave >> 1, wn = wave & 1;
  const int l32 = lane & 31, h = lane >> 5;
  int ar[2][4], br[2];
#pragma unroll
  for (int gi = 0; gi < 2; ++gi) {
#pragma unroll
    for (int t = 0; t < 4; ++t)
      ar[gi][t] = (wm * 64 + l32) * 256 + (((gi * 8 + t + 4 * h) ^ (l32 & 15)) << 4);
    br[gi] = kDStageA + (wn * 64 + l32) * 64 + (((gi * 2 + h) ^ ((l32 >> 2) & 3)) << 4);
  }
  const int sr = kDStageA + kDStageB + (wn * 64 + l32) * 4;
  const uint32_t msk = 0x00780078u, mg = kMagic2;

  f32x16_t tot[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) tot[i][j][v] = 0.0f;

  auto compute = [&](const unsigned char* base, int gi) __attribute__((always_inline)) {
    bf16x8_t bop[2][4];
    float s8[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const v4u c = *reinterpret_cast<const v4u*>(base + br[gi] + j * 2048);
      s8[j] = 8.0f * bf16_to_f32(*reinterpret_cast<const uint16_t*>(base + sr + j * 128 + gi * 2));
      bop[j][0] = expand_codes(c.x, msk, mg);
      bop[j][1] = expand_codes(c.y, msk, mg);
      bop[j][2] = expand_codes(c.z, msk, mg);
      bop[j][3] = expand_codes(c.w, msk, mg);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      v4u a[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) a[t] = *reinterpret_cast<const v4u*>(base + ar[gi][t] + i * 8192);
      f32x16_t p[2];
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) p[j][v] = 0.0f;
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          p[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a[t]),
                                                         bop[j][t], p[j], 0, 0, 0);
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) tot[i][j][v] = __builtin_fmaf(s8[j], p[j][v], tot[i][j][v]);
    }
  };

  issue(0);
  if (ns > 1) issue(1);
  for (int st = 0; st < ns; ++st) {
    if (st + 1 < ns)
      asm volatile("s_waitcnt vmcnt(11)" ::: "memory");
    else
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (st + 2 < ns) issue(st + 2);
    const unsigned char* base = smem + (st % kDStages) * kDStage;
    compute(base, 0);
    compute(base, 1);
  }

  bias_and_store<2, 2>(tot, scales, biases, xs, y, M, N, G, G16, ldy, m0 + wm * 64, n0 + wn * 64, l32,
                       h, vec);
}

int64_t g16_of(int64_t K) { return (((K >> 6) + 15) / 16) * 16; }

}  // namespace

size_t gemm_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  (void)N;
  return (size_t)(M * K) * sizeof(uint16_t) + (size_t)(M * 3 * g16_of(K)) * sizeof(uint16_t);
}

hipError_t launch_gemm(const uint32_t* wq, const uint16_t* scales, const uint16_t* biases,
                       const uint16_t* x, float* y, int64_t M, int64_t N, int64_t K,
                       void* workspace, hipStream_t stream) {
  const int64_t G16 = g16_of(K);
  uint16_t* xp = reinterpret_cast<uint16_t*>(workspace);
  uint16_t* xs = xp + M * K;
  const int64_t nt = M * G16;
  hipLaunchKernelGGL(xprep_kernel, dim3((unsigned)((nt + kThreads - 1) / kThreads)), dim3(kThreads),
                     0, stream, x, xp, xs, M, K, G16);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const bool vec = ((K >> 6) & 7) == 0 && ((reinterpret_cast<uintptr_t>(scales) |
                                             reinterpret_cast<uintptr_t>(biases)) & 15u) == 0;
  // every buffer the main loop reads stays below 2^31 bytes: cut M and N into slices
  const int64_t G = K >> 6;
  // whole two-group stages and 4-byte aligned scale pairs: the LDS-load kernel
  const bool dma = (G % 2) == 0 && (reinterpret_cast<uintptr_t>(scales) & 3u) == 0;
  const int64_t max_rows_x = std::max<int64_t>(kTM, (((int64_t)1 << 31) - 1) / (K * 2) / kTM * kTM);
  const int64_t max_cols_w = std::max<int64_t>(kTN, (((int64_t)1 << 31) - 1) / (K / 2) / kTN * kTN);
  for (int64_t ms = 0; ms < M; ms += max_rows_x) {
    const int64_t Ms = std::min(M - ms, max_rows_x);
    for (int64_t ns = 0; ns < N; ns += max_cols_w) {
      const int64_t Ns = std::min(N - ns, max_cols_w);
      const int64_t MT = (Ms + kTM - 1) / kTM, NT = (Ns + kTN - 1) / kTN;
      const int64_t tiles = MT * NT, per = (tiles + 7) / 8;
      // the register-staged kernel fits two workgroups per CU, the LDS-load kernel one:
      // take the latter only when the grid leaves CUs without a second workgroup
      if (dma && tiles < 2 * kCUs)
        hipLaunchKernelGGL(gemm_dma_kernel, dim3((unsigned)(8 * per)), dim3(256), 0, stream,
                           wq + ns * (K / 8), scales + ns * G, biases + ns * G, xp + ms * K,
                           xs + ms * 3 * G16, y + ms * N + ns, Ms, Ns, K, N, G16, NT, tiles, per, vec);
      else
        hipLaunchKernelGGL(gemm_kernel, dim3((unsigned)(8 * per)), dim3(256), 0, stream, wq + ns * (K / 8),
                           scales + ns * G, biases + ns * G, xp + ms * K, xs + ms * 3 * G16,
                           y + ms * N + ns, Ms, Ns, K, N, G16, NT, tiles, per, vec);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  }
  return hipGetLastError();
}

}  // namespace w4g
