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
// owns a tile of Y; its activations, codes and scales go through LDS one or two
// groups at a time.  Four main loops share that arithmetic: 128 x 128 tiles
// (each wave 64 x 64, 2 x 2 matrix-core tiles) with the operands staged
// through registers (two workgroups per CU) when there are tiles enough for
// that; tiles loaded straight into an LDS ring when fewer: 128 x 128 (one
// workgroup per CU) while they cover the CUs, 64 x 128 (each wave 32 x 64,
// two workgroups per CU) where they cover half of them, and 64 x 64 (each wave
// one 32 x 32 matrix-core tile) for short prompts and small grids (64 x 128
// again past 32 rows where 64 x 64 tiles would outnumber the CUs).  Prompts of
// at most 32 rows over narrow matrices take a fourth loop that deals each
// tile's groups to eight waves and passes the group products on through LDS
// (a tile's K chain would otherwise run on one wave).  The bias terms and the
// store follow the main loop; the result is fp32, or bf16 rounded to
// nearest-even from it.
#include <algorithm>

#include "w4g_internal.h"

namespace w4g {
namespace {

constexpr int kThreads = 256;
constexpr uint32_t kMagic2 = 0x40004000u;  // bf16 pair (2.0, 2.0)
constexpr int kRsrcWord3 = 0x00020000;  // buffer descriptor word 3 (gfx9 family): raw dword data

typedef uint32_t v4u __attribute__((ext_vector_type(4)));  // plain vector: copies stay in registers
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

// The stored value: fp32 as computed, or bf16 rounded to nearest-even from it
// (a NaN stays a quiet NaN of the same sign; a finite value past the bf16
// range rounds to infinity, as nearest-even rounding does).
__device__ __forceinline__ void put(float* y, int64_t i, float v) { y[i] = v; }
__device__ __forceinline__ void put(uint16_t* y, int64_t i, float v) {
  const uint32_t u = __float_as_uint(v);
  y[i] = (uint16_t)((u & 0x7FFFFFFFu) > 0x7F800000u ? (u >> 16) | 0x0040u : f32_to_bf16_rne(v));
}

// The affine remainder and the store, shared by the main loops: for each block of 16
// groups (ascending), b X1, b X2, b X3, (-16 s) X1, (-16 s) X2, (-16 s) X3, each an
// exact bf16 product on the matrix cores.  The wave's tile starts at row mw, column
// nw; lane (h, l32) feeds row l32 of a row tile and column l32 of a column tile,
// groups 8h .. 8h + 7 of each block.
//
// The operands of the next PF blocks are in flight while a block is multiplied
// (a ring of registers).  Rows at or past M read zero sums (a buffer load past
// the end of the slice's rows); columns past N read row N - 1 and store nothing;
// groups at or past G (the padding of the last block) get zero biases and scales
// and have zero sums.  VEC (G % 8 == 0 and 16-byte aligned tables): one 16-byte
// load per lane for the block's eight biases or scales, else eight 2-byte loads.
struct BiasCols {
  uint32_t b[4], s[4];  // bf16 pairs: groups 8h + 2q, 8h + 2q + 1 in word q
};

template <bool VEC>
__device__ __forceinline__ void load_cols(BiasCols& o, const uint16_t* __restrict__ scales,
                                          const uint16_t* __restrict__ biases, int64_t n, int64_t G,
                                          int64_t g0) {
  if constexpr (VEC) {
    const int64_t gc = g0 <= G - 8 ? g0 : G - 8;  // a valid 8-group block; masked if past G
    const uint4 rb = *reinterpret_cast<const uint4*>(biases + n * G + gc);
    const uint4 rs = *reinterpret_cast<const uint4*>(scales + n * G + gc);
    const uint32_t keep = g0 < G ? 0xFFFFFFFFu : 0u;
    o.b[0] = rb.x & keep, o.b[1] = rb.y & keep, o.b[2] = rb.z & keep, o.b[3] = rb.w & keep;
    o.s[0] = rs.x & keep, o.s[1] = rs.y & keep, o.s[2] = rs.z & keep, o.s[3] = rs.w & keep;
  } else {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int64_t g = g0 + 2 * q;
      const uint32_t b0 = g < G ? biases[n * G + g] : 0u, b1 = g + 1 < G ? biases[n * G + g + 1] : 0u;
      const uint32_t s0 = g < G ? scales[n * G + g] : 0u, s1 = g + 1 < G ? scales[n * G + g + 1] : 0u;
      o.b[q] = b0 | (b1 << 16);
      o.s[q] = s0 | (s1 << 16);
    }
  }
}

template <int TI, int TJ>
struct BiasOps {
  v4u ax[TI][3];
  BiasCols c[TJ];
};

template <int TI, int TJ, bool VEC, int PF, typename OUT>
__device__ __forceinline__ void bias_and_store(f32x16_t (&tot)[TI][TJ], const uint16_t* __restrict__ scales,
                                               const uint16_t* __restrict__ biases,
                                               const uint16_t* __restrict__ xs, OUT* __restrict__ y,
                                               int64_t M, int64_t N, int64_t G, int64_t G16, int64_t ldy,
                                               int64_t mw, int64_t nw, int l32, int h) {
  // sums: rows mw.. of xs ([M][3][G16] bf16) through a buffer descriptor, so rows
  // past M read zero
  const int64_t rows = M > mw ? M - mw : 0;
  const __amdgpu_buffer_rsrc_t rxs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(xs + (rows ? mw : 0) * 3 * G16), (short)0, (int)(rows * 3 * G16 * 2),
      kRsrcWord3);
  int xoff[TI];
#pragma unroll
  for (int i = 0; i < TI; ++i) xoff[i] = (int)((i * 32 + l32) * 3 * G16 * 2 + h * 16);
  int64_t ncol[TJ];
#pragma unroll
  for (int j = 0; j < TJ; ++j) {
    const int64_t n = nw + j * 32 + l32;
    ncol[j] = n < N ? n : N - 1;
  }
  const int nb = (int)(G16 / 16);
  auto load = [&](BiasOps<TI, TJ>& o, int blk) __attribute__((always_inline)) {
    blk = blk < nb ? blk : nb - 1;  // past the last block: reload it (never used)
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
      for (int q = 0; q < 3; ++q)
        o.ax[i][q] = __builtin_amdgcn_raw_buffer_load_b128(rxs, xoff[i] + q * (int)G16 * 2, blk * 32, 0);
#pragma unroll
    for (int j = 0; j < TJ; ++j) load_cols<VEC>(o.c[j], scales, biases, ncol[j], G, (int64_t)blk * 16 + h * 8);
  };
  auto consume = [&](const BiasOps<TI, TJ>& o) __attribute__((always_inline)) {
    bf16x8_t bb[TJ], bs[TJ];
#pragma unroll
    for (int j = 0; j < TJ; ++j) {
      uint4 vb, vs;
      uint32_t ws[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {  // -16 s, exact: a power-of-two multiple of a bf16
        const uint32_t lo = __float_as_uint(-16.0f * bf16_to_f32(o.c[j].s[q] & 0xFFFFu)) >> 16;
        const uint32_t hi = __float_as_uint(-16.0f * bf16_to_f32(o.c[j].s[q] >> 16)) >> 16;
        ws[q] = lo | (hi << 16);
      }
      vb = make_uint4(o.c[j].b[0], o.c[j].b[1], o.c[j].b[2], o.c[j].b[3]);
      vs = make_uint4(ws[0], ws[1], ws[2], ws[3]);
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
              __builtin_bit_cast(bf16x8_t, o.ax[i][pass % 3]), pass < 3 ? bb[j] : bs[j], tot[i][j],
              0, 0, 0);
  };

  BiasOps<TI, TJ> ring[PF];
#pragma unroll
  for (int p = 0; p < PF; ++p) load(ring[p], p);
  // every iteration consumes PF blocks and loads the PF after them (loads past
  // the last block reread it, so the number in flight never changes)
  for (int b = 0; b < nb; b += PF) {
#pragma unroll
    for (int p = 0; p < PF; ++p) {
      if (b + p < nb) consume(ring[p]);
      load(ring[p], b + p + PF);
    }
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
        if (m < M) put(y, m * ldy + n, tot[i][j][v]);
      }
    }
}

template <int TI, int TJ, int PF, typename OUT>
__device__ __forceinline__ void bias_and_store_any(f32x16_t (&tot)[TI][TJ], const uint16_t* __restrict__ scales,
                                                   const uint16_t* __restrict__ biases,
                                                   const uint16_t* __restrict__ xs, OUT* __restrict__ y,
                                                   int64_t M, int64_t N, int64_t G, int64_t G16,
                                                   int64_t ldy, int64_t mw, int64_t nw, int l32, int h,
                                                   bool vec) {
  if (vec)
    bias_and_store<TI, TJ, true, PF, OUT>(tot, scales, biases, xs, y, M, N, G, G16, ldy, mw, nw, l32, h);
  else  // the uncommon layouts: one block in flight
    bias_and_store<TI, TJ, false, 1, OUT>(tot, scales, biases, xs, y, M, N, G, G16, ldy, mw, nw, l32, h);
}

// Workgroup tile 128 x 128 of Y, four waves in a 2 x 2 grid, each owning 64 x 64
// (2 x 2 matrix-core tiles).  Per 64-group one stage holds in LDS
//   A: 128 rows x 64 permuted activations (16-byte chunk c of row r stored at
//      chunk c ^ ((r >> 1) & 7): sixteen consecutive rows' chunk c, which one
//      16-lane LDS pass reads, land in sixteen distinct 16-byte bank slots),
//   B: the 128 columns' code halves, [half][column] x 16 bytes,
//   S: the 128 columns' scales.
// Global loads run two groups ahead in registers, and LDS is double-buffered,
// with one barrier per group.
constexpr int kTM = 128, kTN = 128;
constexpr int kAStage = kTM * 128;
constexpr int kBStage = 2 * kTN * 16;
constexpr int kSStage = kTN * 2;
constexpr int kStage = kAStage + kBStage + kSStage;

// one group's activations for the workgroup tile (this thread's share) ...
struct StagedA {
  v4u a[4];
};
// ... and its codes and scales, which come from HBM and are fetched a group earlier
struct StagedB {
  v4u b;
  uint16_t s;
};

template <typename OUT>
__global__ __launch_bounds__(256) void gemm_kernel(
    const uint32_t* __restrict__ wq, const uint16_t* __restrict__ scales,
    const uint16_t* __restrict__ biases, const uint16_t* __restrict__ xp,
    const uint16_t* __restrict__ xs, OUT* __restrict__ y, int64_t M, int64_t N, int64_t K,
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
  const int a_w = srow * 128 + ((sch ^ ((srow >> 1) & 7)) << 4);  // + 32 i * 128
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
      a_r[i][t] = (wm * 64 + i * 32 + l32) * 128 + ((((t + 4 * h) ^ ((l32 >> 1) & 7))) << 4);
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

  bias_and_store_any<2, 2, 2, OUT>(tot, scales, biases, xs, y, M, N, G, G16, ldy, m0 + wm * 64,
                                   n0 + wn * 64, l32, h, vec);
}

// The same arithmetic with the operands moved by buffer loads straight into
// LDS (no staging registers), two groups per stage and NS stages in a ring, so
// a stage's loads are issued NS - 1 stages before it is used.  The tile is
// (32 TI WM) x (32 TJ WN): four waves in a WM x WN grid, each owning
// (32 TI) x (32 TJ).  Used when G is even (whole stages) and the scale table is
// 4-byte aligned (one dword per column carries a stage's two scales).  Per
// stage, in LDS:
//   A: TM rows x 256 bytes, 16-byte chunk c (of the two groups' 16) of row r
//      at position c ^ (r & 15);
//   B: TN columns x 64 bytes (group-in-stage, half) pieces, piece q of column n
//      at position q ^ ((n >> 2) & 3);
//   S: TN columns x the two groups' scales.
// Every wave issues the same number of these loads per stage (TM / 16 + TN / 64
// + 1), so waiting for all but the newest stages' loads completes the oldest.
// Per output the arithmetic and its order are those of gemm_kernel, whatever
// the tile: every variant gives the same bits.
// (the loop choice below is a matter of speed only: the four loops give the
// same bits; it is keyed on this device's compute units)

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
// Wait until at most N of this wave's vector-memory loads are outstanding.
template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory");
}
// Workgroup barrier for data exchanged through LDS by the waves themselves (the
// buffer loads in flight are not waited for).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
}
// ... with N = ahead * L for a run-time ahead in [0, A] (the immediate is fixed
// per instruction)
template <int L, int A>
__device__ __forceinline__ void wait_stages(int ahead) {
  if constexpr (A > 0) {
    if (ahead >= A) {
      wait_vm<A * L>();
      return;
    }
    wait_stages<L, A - 1>(ahead);
  } else {
    wait_vm<0>();
  }
}

template <int TI, int TJ, int WM, int WN, int NS, typename OUT>
__global__ __launch_bounds__(256) void gemm_dma_kernel(
    const uint32_t* __restrict__ wq, const uint16_t* __restrict__ scales,
    const uint16_t* __restrict__ biases, const uint16_t* __restrict__ xp,
    const uint16_t* __restrict__ xs, OUT* __restrict__ y, int64_t M, int64_t N, int64_t K,
    int64_t ldy, int64_t G16, int64_t NT, int64_t tiles, int64_t per, bool vec) {
  static_assert(WM * WN == 4, "four waves");
  constexpr int TM = 32 * TI * WM, TN = 32 * TJ * WN;
  constexpr int SA = TM * 256, SB = TN * 64, SS = TN * 4, STAGE = SA + SB + SS;
  constexpr int LA = TM / 16, LB = TN / 64, SL = TN / 4;  // per wave and stage
  constexpr int L = LA + LB + 1;
  static_assert(LA >= 1 && LB >= 1 && SL <= 64 && (NS - 2) * L <= 63, "tile");
  __shared__ __attribute__((aligned(16))) unsigned char smem[NS * STAGE];
  const int tid = threadIdx.x;
  const int b = blockIdx.x;
  const int tile = (b & 7) * (int)per + (b >> 3);
  if (tile >= (int)tiles) return;
  const int mt = __builtin_amdgcn_readfirstlane(tile / (int)NT);
  const int nt = __builtin_amdgcn_readfirstlane(tile - mt * (int)NT);
  const int64_t m0 = (int64_t)mt * TM, n0 = (int64_t)nt * TN;
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
  // loads: lane offsets per instruction (rows 4 (LA wave + i) + lane / 16 of A,
  // columns 16 (LB wave + j) + lane / 4 of B, columns SL wave + lane of S for
  // lanes < SL)
  uint32_t va[LA], vb[LB];
#pragma unroll
  for (int i = 0; i < LA; ++i) {
    const int rr = 4 * (LA * wave + i) + (lane >> 4);
    const int c = (lane & 15) ^ (rr & 15);
    va[i] = (uint32_t)(rr * K * 2 + c * 16);
  }
#pragma unroll
  for (int j = 0; j < LB; ++j) {
    const int col = 16 * (LB * wave + j) + (lane >> 2);
    const int q = (lane & 3) ^ ((col >> 2) & 3);
    vb[j] = (uint32_t)(col * (K8 * 4) + q * 16);
  }
  const uint32_t vsc = (uint32_t)((SL * wave + (lane & (SL - 1))) * G * 2);
  const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) unsigned char*)smem;
  auto issue = [&](int s) __attribute__((always_inline)) {
    const uint32_t base = lds0 + (uint32_t)((s % NS) * STAGE);
#pragma unroll
    for (int i = 0; i < LA; ++i)
      dma16(__builtin_amdgcn_readfirstlane(base + (LA * wave + i) * 1024), va[i], rx, (uint32_t)(s * 256));
#pragma unroll
    for (int j = 0; j < LB; ++j)
      dma16(__builtin_amdgcn_readfirstlane(base + SA + (LB * wave + j) * 1024), vb[j], rw,
            (uint32_t)(s * 64));
    const uint32_t sbase = __builtin_amdgcn_readfirstlane(base + SA + SB + wave * SL * 4);
    if (lane < SL) dma4(sbase, vsc, rs, (uint32_t)(s * 4));
  };

  // compute: wave (wm, wn) owns rows 32 TI wm.., columns 32 TJ wn.. of the tile;
  // lane (h, l32) feeds row l32 of a row tile and column l32 of a column tile,
  // half h of each 16-element step
  const int wm = wave / WN, wn = wave % WN;
  const int l32 = lane & 31, h = lane >> 5;
  int ar[2][4], br[2];
#pragma unroll
  for (int gi = 0; gi < 2; ++gi) {
#pragma unroll
    for (int t = 0; t < 4; ++t)
      ar[gi][t] = (wm * 32 * TI + l32) * 256 + (((gi * 8 + t + 4 * h) ^ (l32 & 15)) << 4);
    br[gi] = SA + (wn * 32 * TJ + l32) * 64 + (((gi * 2 + h) ^ ((l32 >> 2) & 3)) << 4);
  }
  const int sr = SA + SB + (wn * 32 * TJ + l32) * 4;
  const uint32_t msk = 0x00780078u, mg = kMagic2;

  f32x16_t tot[TI][TJ];
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) tot[i][j][v] = 0.0f;

  auto compute = [&](const unsigned char* base, int gi) __attribute__((always_inline)) {
    bf16x8_t bop[TJ][4];
    float s8[TJ];
#pragma unroll
    for (int j = 0; j < TJ; ++j) {
      const v4u c = *reinterpret_cast<const v4u*>(base + br[gi] + j * 2048);
      s8[j] = 8.0f * bf16_to_f32(*reinterpret_cast<const uint16_t*>(base + sr + j * 128 + gi * 2));
      bop[j][0] = expand_codes(c.x, msk, mg);
      bop[j][1] = expand_codes(c.y, msk, mg);
      bop[j][2] = expand_codes(c.z, msk, mg);
      bop[j][3] = expand_codes(c.w, msk, mg);
    }
#pragma unroll
    for (int i = 0; i < TI; ++i) {
      v4u a[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) a[t] = *reinterpret_cast<const v4u*>(base + ar[gi][t] + i * 8192);
      f32x16_t p[TJ];
#pragma unroll
      for (int j = 0; j < TJ; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) p[j][v] = 0.0f;
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int j = 0; j < TJ; ++j)
          p[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a[t]),
                                                         bop[j][t], p[j], 0, 0, 0);
#pragma unroll
      for (int j = 0; j < TJ; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) tot[i][j][v] = __builtin_fmaf(s8[j], p[j][v], tot[i][j][v]);
    }
  };

  // one wave tile (TI = TJ = 1): the stage's two group products are independent
  // matrix-core chains, so they run side by side; the scaled sums still enter
  // the total in group order
  auto compute_pair = [&](const unsigned char* base) __attribute__((always_inline)) {
    bf16x8_t bop[2][4];
    float s8[2];
    v4u a[2][4];
#pragma unroll
    for (int gi = 0; gi < 2; ++gi) {
      const v4u c = *reinterpret_cast<const v4u*>(base + br[gi]);
      s8[gi] = 8.0f * bf16_to_f32(*reinterpret_cast<const uint16_t*>(base + sr + gi * 2));
      bop[gi][0] = expand_codes(c.x, msk, mg);
      bop[gi][1] = expand_codes(c.y, msk, mg);
      bop[gi][2] = expand_codes(c.z, msk, mg);
      bop[gi][3] = expand_codes(c.w, msk, mg);
#pragma unroll
      for (int t = 0; t < 4; ++t) a[gi][t] = *reinterpret_cast<const v4u*>(base + ar[gi][t]);
    }
    f32x16_t p[2];
#pragma unroll
    for (int gi = 0; gi < 2; ++gi)
#pragma unroll
      for (int v = 0; v < 16; ++v) p[gi][v] = 0.0f;
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int gi = 0; gi < 2; ++gi)
        p[gi] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a[gi][t]),
                                                        bop[gi][t], p[gi], 0, 0, 0);
#pragma unroll
    for (int gi = 0; gi < 2; ++gi)
#pragma unroll
      for (int v = 0; v < 16; ++v) tot[0][0][v] = __builtin_fmaf(s8[gi], p[gi][v], tot[0][0][v]);
  };

  auto compute_stage = [&](const unsigned char* base) __attribute__((always_inline)) {
    if constexpr (TI == 1 && TJ == 1) {
      compute_pair(base);
    } else {
      compute(base, 0);
      compute(base, 1);
    }
  };

#pragma unroll
  for (int s = 0; s < NS - 1; ++s)
    if (s < ns) issue(s);
  // Stage st waits until only the stages issued after it are in flight, then
  // (all waves past the barrier) its buffer's predecessor is free for stage
  // st + NS - 1.  Steady state, unrolled by NS so every buffer offset is a
  // constant: NS - 2 stages ahead, and the next issue exists.
  int st = 0;
  for (; st + NS - 1 <= ns - NS; st += NS) {
#pragma unroll
    for (int u = 0; u < NS; ++u) {
      wait_vm<(NS - 2) * L>();
      __syncthreads();
      issue(st + u + NS - 1);
      compute_stage(smem + u * STAGE);
    }
  }
  for (; st < ns; ++st) {
    const int ahead = ns - 1 - st < NS - 2 ? ns - 1 - st : NS - 2;
    wait_stages<L, NS - 2>(ahead);
    __syncthreads();
    if (st + NS - 1 < ns) issue(st + NS - 1);
    compute_stage(smem + (st % NS) * STAGE);
  }

  bias_and_store_any<TI, TJ, TI * TJ == 1 ? 6 : 2, OUT>(tot, scales, biases, xs, y, M, N, G, G16, ldy,
                                                         m0 + wm * 32 * TI, n0 + wn * 32 * TJ, l32, h,
                                                         vec);
}

// Short prompts: a workgroup of NW waves owns a tile of MR (16 or 32) rows x 32
// columns of Y, small enough that the tiles of a few-row prompt cover the CUs.
// The tile's 64-groups go in rounds of NW: in round j wave w forms P_g of group
// g = NW j + w on the matrix cores, with the operands and the four
// instructions of the tiled loops (a 32 x 32 matrix-core tile; with MR = 16 its
// rows 16..31 are zero), and passes it on through LDS with the group's scales
// 8 s_g; then every wave runs the fp32 chain T += 8 s_g P_g over the round's
// groups in ascending order for its share of the tile's outputs (wave r keeps
// values NV r .. NV (r + 1) - 1, NV = MR / (2 NW), of each lane position's
// sixteen: only rows below MR).  Each output therefore gets the tiled loops'
// arithmetic in their order, and the same bits.  A round's codes (32 columns x
// 32 NW bytes) and activations (MR rows x 128 NW bytes) are loaded whole-line
// by the waves, D rounds ahead into registers, and staged through LDS into the
// matrix-core layout; products are formed two rounds before they go out, so
// the matrix cores' latency stays off a round's path.  After the last round
// wave 0 gathers the tile and adds the bias terms as the tiled loops do,
// storing only the tile's own rows.
template <int MR>
struct ChainOps {
  v4u c;             // 16 bytes of the round's codes
  v4u a[MR / 8];     // 16 bytes each of the round's activations
  uint16_t s;        // scale of column l32, group NW j + w (bf16)
};

template <int MR, int NW, int D, typename OUT>
__global__ __launch_bounds__(64 * NW) void gemm_chain_kernel(
    const uint32_t* __restrict__ wq, const uint16_t* __restrict__ scales,
    const uint16_t* __restrict__ biases, const uint16_t* __restrict__ xp,
    const uint16_t* __restrict__ xs, OUT* __restrict__ y, int64_t M, int64_t N, int64_t K,
    int64_t ldy, int64_t G16, int64_t MT, int64_t tiles, int64_t per, bool vec) {
  static_assert(MR == 16 || MR == 32, "tile rows");
  static_assert(NW == 4 || NW == 8, "waves");
  constexpr int NV = MR / (2 * NW);                  // chain values per lane
  constexpr int XI = MR / 8;                         // activation loads per wave and round
  constexpr int CS = 2 * NW;                         // 16-byte code slots per column and round
  constexpr int XS = 8 * NW;                         // 16-byte activation slots per row and round
  constexpr int XP_G = NW * 64 * NV * 4;             // one group's products: [reader][lane][NV]
  constexpr int XS_G = 64 * 4;                       // one group's scales: [lane]
  constexpr int XCH = NW * (XP_G + XS_G);            // one round's exchange
  constexpr int SC = 32 * CS * 16, SX = MR * XS * 16;  // one round's staged codes, activations
  constexpr int ST = SC + SX;
  __shared__ __attribute__((aligned(16))) unsigned char smem[2 * XCH + 2 * ST];
  const int tid = threadIdx.x;
  const int b = blockIdx.x;
  const int tile = (b & 7) * (int)per + (b >> 3);
  if (tile >= (int)tiles) return;
  // row tiles fastest: the row tiles of one column tile share its codes in L2
  const int nt = __builtin_amdgcn_readfirstlane(tile / (int)MT);
  const int mt = __builtin_amdgcn_readfirstlane(tile - nt * (int)MT);
  const int64_t m0 = (int64_t)mt * MR, n0 = (int64_t)nt * 32;
  const int G = (int)(K >> 6);
  const int K8 = (int)(K >> 3);
  const int R = (G + NW - 1) / NW;
  const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(xp + m0 * K), (short)0, (int)((M - m0) * K * 2), kRsrcWord3);
  const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint32_t*>(wq + n0 * K8), (short)0, (int)((N - n0) * K8 * 4), kRsrcWord3);
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(scales + n0 * G), (short)0, (int)((N - n0) * G * 2), kRsrcWord3);

  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, l32 = lane & 31, h = lane >> 5;
  // loads: 16-byte piece cp of column cr's round segment (32 NW bytes), and
  // piece xq_i of row xr_i's (128 NW bytes)
  const int cr = (64 * wave + lane) / CS, cp = (64 * wave + lane) % CS;
  const int vc = cr * K8 * 4 + cp * 16;
  int vx[XI], xw[XI];
  // LDS slots are swizzled so that both the whole-line writes and the
  // matrix-core reads are free of bank conflicts: codes [column][CS slots],
  // slot p ^ (column & (CS - 1)); activations [row][XS slots], slot q ^ (row & 15)
  const int cw = cr * CS * 16 + ((cp ^ (cr & (CS - 1))) << 4);
#pragma unroll
  for (int i = 0; i < XI; ++i) {
    const int f = (i * NW + wave) * 64 + lane;
    const int xr = f / XS, xq = f % XS;
    vx[i] = xr * (int)K * 2 + xq * 16;
    xw[i] = SC + xr * XS * 16 + ((xq ^ (xr & 15)) << 4);
  }
  const int vs = l32 * G * 2;
  // matrix-core reads: lane (h, l32) takes codes piece 2w + h of column l32 and
  // activation chunks 4h + t (t = 0..3) of its group, row l32 (a 16-row tile's
  // rows 16..31 are zeros held in registers; their lanes read nothing)
  const int crd = l32 * CS * 16 + (((2 * wave + h) ^ (l32 & (CS - 1))) << 4);
  int xrd[4];
#pragma unroll
  for (int t = 0; t < 4; ++t)
    xrd[t] = SC + (l32 & (MR - 1)) * XS * 16 + (((8 * wave + 4 * h + t) ^ (l32 & 15)) << 4);

  // rounds past the last reload the last one (cached), so every round loads alike
  auto load = [&](ChainOps<MR>& o, int r) __attribute__((always_inline)) {
    r = r < R ? r : R - 1;
    o.c = __builtin_amdgcn_raw_buffer_load_b128(rw, vc, r * (32 * NW), 0);
#pragma unroll
    for (int i = 0; i < XI; ++i) o.a[i] = __builtin_amdgcn_raw_buffer_load_b128(rx, vx[i], r * (128 * NW), 0);
    o.s = __builtin_amdgcn_raw_buffer_load_b16(rs, vs, (NW * r + wave) * 2, 0);
  };
  auto stage = [&](const ChainOps<MR>& o, int par) __attribute__((always_inline)) {
    unsigned char* base = smem + 2 * XCH + par * ST;
    *reinterpret_cast<v4u*>(base + cw) = o.c;
#pragma unroll
    for (int i = 0; i < XI; ++i) *reinterpret_cast<v4u*>(base + xw[i]) = o.a[i];
  };
  const uint32_t msk = 0x00780078u, mg = kMagic2;
  auto compute_p = [&](int par) __attribute__((always_inline)) -> f32x16_t {
    const unsigned char* base = smem + 2 * XCH + par * ST;
    const v4u c = *reinterpret_cast<const v4u*>(base + crd);
    v4u a[4];
    if (MR == 16 && l32 >= 16) {
#pragma unroll
      for (int t = 0; t < 4; ++t) a[t] = v4u{0u, 0u, 0u, 0u};
    } else {
#pragma unroll
      for (int t = 0; t < 4; ++t) a[t] = *reinterpret_cast<const v4u*>(base + xrd[t]);
    }
    f32x16_t p;
#pragma unroll
    for (int v = 0; v < 16; ++v) p[v] = 0.0f;
    p = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a[0]), expand_codes(c.x, msk, mg), p, 0, 0, 0);
    p = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a[1]), expand_codes(c.y, msk, mg), p, 0, 0, 0);
    p = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a[2]), expand_codes(c.z, msk, mg), p, 0, 0, 0);
    p = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a[3]), expand_codes(c.w, msk, mg), p, 0, 0, 0);
    return p;
  };
  // this wave's group product of a round -> reader r's slots, and its scales
  auto put_p = [&](const f32x16_t& p, float s8, int par) __attribute__((always_inline)) {
    unsigned char* base = smem + par * XCH + wave * XP_G + lane * NV * 4;
#pragma unroll
    for (int r = 0; r < NW; ++r) {
      if constexpr (NV == 4)
        *reinterpret_cast<float4*>(base + r * 64 * NV * 4) = make_float4(p[4 * r], p[4 * r + 1], p[4 * r + 2], p[4 * r + 3]);
      else if constexpr (NV == 2)
        *reinterpret_cast<float2*>(base + r * 64 * NV * 4) = make_float2(p[2 * r], p[2 * r + 1]);
      else
        *reinterpret_cast<float*>(base + r * 64 * NV * 4) = p[r];
    }
    *reinterpret_cast<float*>(smem + par * XCH + NW * XP_G + wave * XS_G + lane * 4) = s8;
  };
  float tot[NV];
#pragma unroll
  for (int e = 0; e < NV; ++e) tot[e] = 0.0f;
  // the chain over round j's groups, ascending
  auto chain = [&](int j) __attribute__((always_inline)) {
    const unsigned char* xr_ = smem + (j & 1) * XCH + (wave * 64 + lane) * NV * 4;
    const float* xsr = reinterpret_cast<const float*>(smem + (j & 1) * XCH + NW * XP_G) + lane;
    float pv[NW][NV], s8[NW];
#pragma unroll
    for (int gq = 0; gq < NW; ++gq) {
      const float* f = reinterpret_cast<const float*>(xr_ + gq * XP_G);
#pragma unroll
      for (int e = 0; e < NV; ++e) pv[gq][e] = f[e];
      s8[gq] = xsr[gq * 64];
    }
    if (NW * (j + 1) <= G) {
#pragma unroll
      for (int gq = 0; gq < NW; ++gq)
#pragma unroll
        for (int e = 0; e < NV; ++e) tot[e] = __builtin_fmaf(s8[gq], pv[gq][e], tot[e]);
    } else {  // the last round of a ragged G
      const int ng = G - NW * j;
#pragma unroll
      for (int gq = 0; gq < NW; ++gq)
        if (gq < ng)
#pragma unroll
          for (int e = 0; e < NV; ++e) tot[e] = __builtin_fmaf(s8[gq], pv[gq][e], tot[e]);
    }
  };

  ChainOps<MR> ring[D];
#pragma unroll
  for (int u = 0; u < D; ++u) load(ring[u], u);
  stage(ring[0], 0);
  float sc = 8.0f * bf16_to_f32(ring[0].s);
  load(ring[0], D);
  float sc1 = sc;
  if (R > 1) {
    stage(ring[1], 1);
    sc1 = 8.0f * bf16_to_f32(ring[1].s);
  }
  load(ring[1], D + 1);
  lds_barrier();
  f32x16_t pc = compute_p(0);
  f32x16_t pc1 = pc;
  if (R > 1) pc1 = compute_p(1);
  // round j: its product goes out with its scales and round j + 2's operands
  // are staged (ring slot (j + 2) % D, then refilled with round j + 2 + D);
  // after the barrier round j + 2's product is started and the chain takes
  // round j's products
  auto round = [&](int j, ChainOps<MR>& nxt) __attribute__((always_inline)) {
    put_p(pc, sc, j & 1);
    float sn = sc1;
    if (j + 2 < R) {
      stage(nxt, j & 1);
      sn = 8.0f * bf16_to_f32(nxt.s);
    }
    load(nxt, j + 2 + D);
    lds_barrier();
    f32x16_t pn = pc1;
    if (j + 2 < R) pn = compute_p(j & 1);
    chain(j);
    pc = pc1;
    sc = sc1;
    pc1 = pn;
    sc1 = sn;
  };
  int j0 = 0;
  for (; j0 + D <= R; j0 += D) {
#pragma unroll
    for (int u = 0; u < D; ++u) round(j0 + u, ring[(u + 2) % D]);
  }
#pragma unroll
  for (int u = 0; u < D - 1; ++u)
    if (j0 + u < R) round(j0 + u, ring[(u + 2) % D]);

  // wave 0 gathers the tile (the exchange area is free after this barrier)
  lds_barrier();
  float* gat = reinterpret_cast<float*>(smem) + (wave * 64 + lane) * NV;
#pragma unroll
  for (int e = 0; e < NV; ++e) gat[e] = tot[e];
  lds_barrier();
  if (wave != 0) return;
  f32x16_t t16[1][1];
#pragma unroll
  for (int v = 0; v < 16; ++v) t16[0][0][v] = 0.0f;
#pragma unroll
  for (int r = 0; r < NW; ++r) {
    const float* src = reinterpret_cast<const float*>(smem) + (r * 64 + lane) * NV;
#pragma unroll
    for (int e = 0; e < NV; ++e) t16[0][0][NV * r + e] = src[e];
  }
  const int64_t mlim = M < m0 + MR ? M : m0 + MR;
  bias_and_store_any<1, 1, 6, OUT>(t16, scales, biases, xs, y, mlim, N, G, G16, ldy, m0, n0, l32, h, vec);
}

int64_t g16_of(int64_t K) { return (((K >> 6) + 15) / 16) * 16; }

// The short-prompt kernel takes prompts of at most 32 rows whose 32-column
// tiles number at most two per CU (wider matrices keep the tiled loops, which
// stream them as fast)
bool chain_tiles(int64_t M, int64_t N) { return M <= 32 && (N + 31) / 32 <= 2 * cu_count(); }

// Where the 64 x 64 tiles take over (rows of the slice, 128 x 128 tiles it makes)
bool small_tiles(int64_t M, int64_t tiles128) {
  const int cus = cu_count();
  return tiles128 < cus / 2 || (M <= 128 && tiles128 < 2 * cus);
}


}  // namespace

size_t gemm_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  (void)N;
  return (size_t)(M * K) * sizeof(uint16_t) + (size_t)(M * 3 * g16_of(K)) * sizeof(uint16_t);
}

namespace {

// One launch per slice of rows and columns; every buffer a slice reads stays
// below 2^31 bytes.  The variant follows from the shape and the pointers:
//   the register-staged loop with 128 x 128 tiles when there are enough tiles
//   for two workgroups per CU (or when the LDS-load kernel does not apply),
//   the LDS-load loop with 128 x 128 tiles while they still cover every CU,
//   with 64 x 128 tiles (two workgroups per CU) where they cover half of them
//   or more, and with 64 x 64 tiles (a deeper ring) below that, except past 32
//   rows where those would outnumber the CUs (64 x 128 again).
template <typename OUT>
hipError_t launch_main(const uint32_t* wq, const uint16_t* scales, const uint16_t* biases,
                       const uint16_t* xp, const uint16_t* xs, OUT* y, int64_t M, int64_t N,
                       int64_t K, int64_t G16, bool vec, bool dma, hipStream_t stream) {
  const int64_t G = K >> 6;
  const int64_t max_rows_x = std::max<int64_t>(kTM, (((int64_t)1 << 31) - 1) / (K * 2) / kTM * kTM);
  const int64_t max_cols_w = std::max<int64_t>(kTN, (((int64_t)1 << 31) - 1) / (K / 2) / kTN * kTN);
  for (int64_t ms = 0; ms < M; ms += max_rows_x) {
    const int64_t Ms = std::min(M - ms, max_rows_x);
    for (int64_t ns = 0; ns < N; ns += max_cols_w) {
      const int64_t Ns = std::min(N - ns, max_cols_w);
      const uint32_t* w_s = wq + ns * (K / 8);
      const uint16_t *s_s = scales + ns * G, *b_s = biases + ns * G;
      const uint16_t *xp_s = xp + ms * K, *xs_s = xs + ms * 3 * G16;
      OUT* y_s = y + ms * N + ns;
      const int64_t tiles128 = ((Ms + kTM - 1) / kTM) * ((Ns + kTN - 1) / kTN);
      if (dma && chain_tiles(Ms, Ns)) {
        // few rows over a narrow matrix: MR x 32 tiles, each column tile's groups
        // dealt to eight waves
        const int64_t NT = (Ns + 31) / 32;
        if (Ms <= 16) {
          const int64_t tiles = NT, per = (tiles + 7) / 8;
          hipLaunchKernelGGL((gemm_chain_kernel<16, 8, 3, OUT>), dim3((unsigned)(8 * per)), dim3(512), 0,
                             stream, w_s, s_s, b_s, xp_s, xs_s, y_s, Ms, Ns, K, N, G16, (int64_t)1, tiles, per,
                             vec);
        } else {
          const int64_t MT = (Ms + 31) / 32, tiles = MT * NT, per = (tiles + 7) / 8;
          hipLaunchKernelGGL((gemm_chain_kernel<32, 8, 3, OUT>), dim3((unsigned)(8 * per)), dim3(512), 0,
                             stream, w_s, s_s, b_s, xp_s, xs_s, y_s, Ms, Ns, K, N, G16, MT, tiles, per, vec);
        }
      } else if (dma && small_tiles(Ms, tiles128)) {
        // 64 x 64 tiles: a 4-stage ring (83 KiB, one workgroup per CU) while the
        // tiles fit on the CUs once, else 3 stages (62 KiB) so two share a CU;
        // past 32 rows, where they outnumber the CUs, 64 x 128 tiles (half as
        // many, two per CU: gate-up at 128 rows 107 -> 102 us, at 64 rows 72.2 ->
        // 71.3; at 16 and 32 rows, whose second half-tile of rows is empty,
        // they were slower)
        const int64_t NT = (Ns + 63) / 64, tiles = ((Ms + 63) / 64) * NT, per = (tiles + 7) / 8;
        if (tiles > cu_count() && Ms > 32) {
          const int64_t NT2 = (Ns + 127) / 128, tiles2 = ((Ms + 63) / 64) * NT2, per2 = (tiles2 + 7) / 8;
          hipLaunchKernelGGL((gemm_dma_kernel<1, 2, 2, 2, 3, OUT>), dim3((unsigned)(8 * per2)), dim3(256), 0,
                             stream, w_s, s_s, b_s, xp_s, xs_s, y_s, Ms, Ns, K, N, G16, NT2, tiles2, per2, vec);
        } else if (tiles <= cu_count())
          hipLaunchKernelGGL((gemm_dma_kernel<1, 1, 2, 2, 4, OUT>), dim3((unsigned)(8 * per)), dim3(256), 0,
                             stream, w_s, s_s, b_s, xp_s, xs_s, y_s, Ms, Ns, K, N, G16, NT, tiles, per, vec);
        else
          hipLaunchKernelGGL((gemm_dma_kernel<1, 1, 2, 2, 3, OUT>), dim3((unsigned)(8 * per)), dim3(256), 0,
                             stream, w_s, s_s, b_s, xp_s, xs_s, y_s, Ms, Ns, K, N, G16, NT, tiles, per, vec);
      } else if (!dma || tiles128 >= 2 * cu_count()) {
        const int64_t NT = (Ns + kTN - 1) / kTN, per = (tiles128 + 7) / 8;
        hipLaunchKernelGGL(gemm_kernel<OUT>, dim3((unsigned)(8 * per)), dim3(256), 0, stream, w_s, s_s,
                           b_s, xp_s, xs_s, y_s, Ms, Ns, K, N, G16, NT, tiles128, per, vec);
      } else if (tiles128 < cu_count()) {
        // 128 x 128 tiles would leave CUs idle: 64 x 128 tiles, a 3-stage ring
        // (74 KiB) so two share a CU (o_proj and down at 512 rows, 160 tiles of
        // 128 x 128: 67 -> 64 and 202 -> 195 us)
        const int64_t NT = (Ns + 127) / 128, tiles = ((Ms + 63) / 64) * NT, per = (tiles + 7) / 8;
        hipLaunchKernelGGL((gemm_dma_kernel<1, 2, 2, 2, 3, OUT>), dim3((unsigned)(8 * per)), dim3(256), 0,
                           stream, w_s, s_s, b_s, xp_s, xs_s, y_s, Ms, Ns, K, N, G16, NT, tiles, per, vec);
      } else {
        const int64_t NT = (Ns + kTN - 1) / kTN, per = (tiles128 + 7) / 8;
        hipLaunchKernelGGL((gemm_dma_kernel<2, 2, 2, 2, 3, OUT>), dim3((unsigned)(8 * per)), dim3(256), 0,
                           stream, w_s, s_s, b_s, xp_s, xs_s, y_s, Ms, Ns, K, N, G16, NT, tiles128, per,
                           vec);
      }
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  }
  return hipSuccess;
}

}  // namespace

hipError_t launch_gemm(const uint32_t* wq, const uint16_t* scales, const uint16_t* biases,
                       const uint16_t* x, void* y, bool y_bf16, int64_t M, int64_t N, int64_t K,
                       void* workspace, hipStream_t stream) {
  const int64_t G16 = g16_of(K);
  uint16_t* xp = reinterpret_cast<uint16_t*>(workspace);
  uint16_t* xs = xp + M * K;
  const int64_t nt = M * G16;
  hipLaunchKernelGGL(xprep_kernel, dim3((unsigned)((nt + kThreads - 1) / kThreads)), dim3(kThreads),
                     0, stream, x, xp, xs, M, K, G16);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const bool vec = ((K >> 6) & 7) == 0 && ((reinterpret_cast<uintptr_t>(scales) |
                                             reinterpret_cast<uintptr_t>(biases)) & 15u) == 0;
  // whole two-group stages and 4-byte aligned scale pairs: the LDS-load kernels apply
  const bool dma = ((K >> 6) % 2) == 0 && (reinterpret_cast<uintptr_t>(scales) & 3u) == 0;
  if (y_bf16)
    return launch_main(wq, scales, biases, xp, xs, reinterpret_cast<uint16_t*>(y), M, N, K, G16, vec, dma,
                       stream);
  return launch_main(wq, scales, biases, xp, xs, reinterpret_cast<float*>(y), M, N, K, G16, vec, dma,
                     stream);
}

}  // namespace w4g
