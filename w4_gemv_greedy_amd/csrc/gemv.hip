// Decode product y[b][n] = sum_k x[b][k] * (q*s + b)[n][k] on the vector ALUs,
// 4-bit affine codes with one bf16 scale and bias per 64-group (TensorFold
// PR #1437, Receipt: "4-bit affine with group 64"; fp32 result: same PR,
// commit "Add the pair seam and register its kernels with the kernel
// contract").
//
// Arithmetic, per output row and batch row (the order depends on K alone, so a
// row's bits do not change with N, B or the grid: TensorFold PR #1433, step-2
// description, the K reduction tree is the full matrix's):
//   K is cut into chunks of 1024 elements; in chunk c, lane l of a 32-lane
//   half wave owns elements [32l, 32l + 32), half of one 64-group.  The lane
//   expands its four code words to bf16 pairs (128 + q[i], 128 + q[i+4]) by
//   OR-ing each nibble into the bit pattern of 128.0, and v_dot2 against the
//   matching pairs (x[i], x[i+4]) accumulates D = sum x*(128 + q) in fp32,
//   word by word and pair by pair.  X is the fp32 sum of the same 32 x, taken
//   over the same pairs in the same order against (1, 1).  The lane then adds
//   s*D and (b - 128 s)*X to its running sum with fused multiply-adds
//   (b - 128 s itself one fused multiply-add), chunk after chunk in ascending
//   order.  After the last chunk the 32 lane sums meet in a fixed tree: the
//   two 16-lane rows add lane by lane, then each row folds by mirror
//   (i, 15 - i), half mirror (i, 7 - i), and quad swaps (i, i ^ 2), (i, i ^ 1).
//
// Memory: a half wave owns whole rows; in each chunk lane l reads one 16-byte
// code vector at byte 16l (a non-temporal load: the codes are read once), so a wave-wide load covers 512 contiguous bytes of
// each of two rows.  A work item is one chunk of R consecutive rows; P items
// are in flight while one is consumed.  The activations are paired and summed
// once per workgroup into LDS, laid out so that a half wave's reads are
// contiguous, and each item's R rows share them; their loads go out before the
// first codes', so staging does not wait behind the code stream.  Rows are
// dealt out in equal shares: at B = 1 one workgroup per CU for the layer
// widths (every CU streams the same bytes, no trailing second round), short
// workgroups of 8 R rows elsewhere.
#include "w4g_internal.h"

namespace w4g {
namespace {

constexpr int kChunk = 1024;
constexpr int kThreads = 256;
constexpr int kHalfWaves = kThreads / 32;
// LDS one workgroup may take here: most of the CU's 160 KiB (above 64 KiB the
// kernel asks for it with hipFuncSetAttribute); one such workgroup per CU still
// streams faster than the register-staged variant (measured: down at B=4,
// 148 KiB, 29 us against 46 us)
constexpr size_t kMaxLds = 152 * 1024;
constexpr size_t kDefaultLds = 64 * 1024;
constexpr uint32_t kMagic128 = 0x43004300u;  // bf16 pair (128.0, 128.0)
constexpr uint32_t kOnes = 0x3F803F80u;      // bf16 pair (1.0, 1.0)
constexpr uint32_t kNibbles = 0x000F000Fu;

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

// (a & m) | g in one instruction (the compiler would emit two with literals)
__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t m, uint32_t g) {
  uint32_t d;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(d) : "v"(a), "s"(m), "v"(g));
  return d;
}

// (x[i], x[i+4]) pairs of an 8-element block held as natural pairs
// (x0,x1), (x2,x3), (x4,x5), (x6,x7).
__device__ __forceinline__ uint4 pair_x(uint4 v) {
  uint4 p;
  p.x = __builtin_amdgcn_perm(v.z, v.x, 0x05040100u);  // (x0, x4)
  p.y = __builtin_amdgcn_perm(v.z, v.x, 0x07060302u);  // (x1, x5)
  p.z = __builtin_amdgcn_perm(v.w, v.y, 0x05040100u);  // (x2, x6)
  p.w = __builtin_amdgcn_perm(v.w, v.y, 0x07060302u);  // (x3, x7)
  return p;
}

// D += the 8 codes of one word against 4 x pairs
__device__ __forceinline__ float dot_word(uint32_t w, uint4 xp, float d, uint32_t m, uint32_t g) {
  d = dot2(and_or(w, m, g), xp.x, d);
  d = dot2(and_or(w >> 4, m, g), xp.y, d);
  d = dot2(and_or(w >> 8, m, g), xp.z, d);
  d = dot2(and_or(w >> 12, m, g), xp.w, d);
  return d;
}

__device__ __forceinline__ float bf16_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// Sum over the 32 lanes of each half wave, the same bits in every lane:
// the two 16-lane rows add lane by lane (v_permlane16_swap), then each row
// folds onto itself by mirror (lane i with 15 - i), half mirror (i with
// 7 - i within 8) and the two quad swaps (i with i ^ 2, then i ^ 1).  Every
// step adds a pair of equal-order partners, so all lanes end equal.
template <int CTRL>
__device__ __forceinline__ float dpp_add(float v) {
  const int o = __builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, false);
  return v + __int_as_float(o);
}
__device__ __forceinline__ float half_wave_sum(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  v = dpp_add<0x140>(v);  // row_mirror
  v = dpp_add<0x141>(v);  // row_half_mirror
  v = dpp_add<0x4E>(v);   // quad_perm [2,3,0,1]
  v = dpp_add<0xB1>(v);   // quad_perm [1,0,3,2]
  return v;
}

// The same tree for NB values at once (NB = 2, 4 or 8; batch rows past B
// enter as zeros), transposed: each step adds the same pairs of lanes as
// half_wave_sum, in the same operand order, but a lane keeps only half of the
// values it holds, the half its partner does not keep.  The 16-lane row swap
// leaves value 2k's pair sums in row 0 and value 2k + 1's in row 1 (one
// v_permlane16_swap per pair of values); mirror and half mirror then split by
// lane bits 3 and 2 the same way; the quad swaps add what is left.  So every
// value's total has the bits half_wave_sum gives it, and lane i of the half
// wave ends with the total of value half_wave_index<NB>(i): NB / 2 row swaps
// and about 2 NB instructions in all, against 10 NB for NB separate trees.
template <int NB>
__device__ __forceinline__ int half_wave_index(int lane) {
  int t = (lane >> 4) & 1;
  if constexpr (NB >= 4) t |= ((lane >> 3) & 1) << 1;
  if constexpr (NB >= 8) t |= ((lane >> 2) & 1) << 2;
  return t;
}
// lanes of a half wave that hold value t: the first of each group of 32 / NB
template <int NB>
__device__ __forceinline__ bool half_wave_first(int lane) {
  return (lane & (32 / NB - 1)) == 0;
}
template <int CTRL>
__device__ __forceinline__ float dpp_keep_add(float lo_keep, float hi_keep, bool hi) {
  // keep one of two values and add the partner's copy of the same value
  const float keep = hi ? hi_keep : lo_keep;
  const float send = hi ? lo_keep : hi_keep;
  const int o = __builtin_amdgcn_mov_dpp(__float_as_int(send), CTRL, 0xF, 0xF, false);
  return keep + __int_as_float(o);
}
template <int NB>
__device__ __forceinline__ float half_wave_sums(const float (&v)[NB], int lane) {
  static_assert(NB == 2 || NB == 4 || NB == 8, "2, 4 or 8 values");
  float a[NB / 2];
#pragma unroll
  for (int k = 0; k < NB / 2; ++k) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v[2 * k]), __float_as_uint(v[2 * k + 1]),
                                                    false, false);
    a[k] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
  float t;
  if constexpr (NB == 2) {
    t = dpp_add<0x140>(a[0]);
    t = dpp_add<0x141>(t);
  } else if constexpr (NB == 4) {
    t = dpp_keep_add<0x140>(a[0], a[1], (lane & 8) != 0);
    t = dpp_add<0x141>(t);
  } else {
    const float b0 = dpp_keep_add<0x140>(a[0], a[1], (lane & 8) != 0);
    const float b1 = dpp_keep_add<0x140>(a[2], a[3], (lane & 8) != 0);
    t = dpp_keep_add<0x141>(b0, b1, (lane & 4) != 0);
  }
  t = dpp_add<0x4E>(t);
  t = dpp_add<0xB1>(t);
  return t;
}
constexpr int sums_width(int B) { return B <= 2 ? 2 : B <= 4 ? 4 : 8; }

// Other code widths (2 and 8 bits: 32/bits codes per uint32, low field first).
// 2-bit: word t of a lane's 32 elements covers elements 16t .. 16t + 15; field j
// and field j + 8 go to one bf16 pair (128 + q[j], 128 + q[j + 8]) with one
// v_and_or_b32, against the x pair (x[j], x[j + 8]).
__device__ __forceinline__ float dot_word2(uint32_t w, uint4 xa, uint4 xb, float d, uint32_t g) {
  const uint32_t m2 = 0x00030003u;
  d = dot2(and_or(w, m2, g), xa.x, d);
  d = dot2(and_or(w >> 2, m2, g), xa.y, d);
  d = dot2(and_or(w >> 4, m2, g), xa.z, d);
  d = dot2(and_or(w >> 6, m2, g), xa.w, d);
  d = dot2(and_or(w >> 8, m2, g), xb.x, d);
  d = dot2(and_or(w >> 10, m2, g), xb.y, d);
  d = dot2(and_or(w >> 12, m2, g), xb.z, d);
  d = dot2(and_or(w >> 14, m2, g), xb.w, d);
  return d;
}
// 8-bit: a code q = 16 h + l is taken as its two nibbles; word t covers
// elements 4t .. 4t + 3; pairs (l[0], l[2]), (l[1], l[3]) against (x0, x2),
// (x1, x3) accumulate Dl, the high nibbles likewise Dh (each 128 + nibble).
__device__ __forceinline__ void dot_word8(uint32_t w, uint32_t p0, uint32_t p1, float& dl, float& dh,
                                          uint32_t m, uint32_t g) {
  dl = dot2(and_or(w, m, g), p0, dl);
  dl = dot2(and_or(w >> 8, m, g), p1, dl);
  dh = dot2(and_or(w >> 4, m, g), p0, dh);
  dh = dot2(and_or(w >> 12, m, g), p1, dh);
}
// x pairs for those orders, from natural pairs: 2-bit, a 16-element block
// (a, b) -> (x[j], x[j + 8]) for j = 0..3 and 4..7; 8-bit, each 4-element
// block -> (x0, x2), (x1, x3).
__device__ __forceinline__ void pair_x2(uint4 a, uint4 b, uint4& lo, uint4& hi) {
  lo.x = __builtin_amdgcn_perm(b.x, a.x, 0x05040100u);
  lo.y = __builtin_amdgcn_perm(b.x, a.x, 0x07060302u);
  lo.z = __builtin_amdgcn_perm(b.y, a.y, 0x05040100u);
  lo.w = __builtin_amdgcn_perm(b.y, a.y, 0x07060302u);
  hi.x = __builtin_amdgcn_perm(b.z, a.z, 0x05040100u);
  hi.y = __builtin_amdgcn_perm(b.z, a.z, 0x07060302u);
  hi.z = __builtin_amdgcn_perm(b.w, a.w, 0x05040100u);
  hi.w = __builtin_amdgcn_perm(b.w, a.w, 0x07060302u);
}
__device__ __forceinline__ uint4 pair_x8(uint4 v) {
  uint4 p;
  p.x = __builtin_amdgcn_perm(v.y, v.x, 0x05040100u);  // (x0, x2)
  p.y = __builtin_amdgcn_perm(v.y, v.x, 0x07060302u);  // (x1, x3)
  p.z = __builtin_amdgcn_perm(v.w, v.z, 0x05040100u);  // (x4, x6)
  p.w = __builtin_amdgcn_perm(v.w, v.z, 0x07060302u);  // (x5, x7)
  return p;
}

// One lane's codes of one row and chunk: 32 codes = 4 BITS bytes, loaded as
// VPL vectors of type V.
template <int BITS>
struct CodeVec {
  typedef uint4 V;
  static constexpr int VPL = BITS / 4;
};
template <>
struct CodeVec<2> {
  typedef uint2 V;
  static constexpr int VPL = 1;
};

template <int R, int BITS = 4>
struct Item {
  typename CodeVec<BITS>::V w[R][CodeVec<BITS>::VPL];
  uint16_t s[R], b[R];  // kept 16-bit so no widening copy waits on the loads
};

// LDS: paired activations [B][C][4][32] uint4 (chunk, vector, lane), then lane
// sums [B][C][32] float.  P items are in flight per half wave (a ring of P
// buffers).  Workgroup b owns rows [b rpw, (b + 1) rpw) (fewer at the end of
// the matrix), taken as groups of R consecutive rows: half wave h of H owns
// groups h, h + H, h + 2H, ...  Both half waves of a wave run as many groups as
// the first of them (the second repeats its last valid row and stores
// nothing), so every branch in the stream is wave-uniform.  A lane past the
// end of a short last chunk reads lane 0 of chunk 0 (always staged, so finite)
// and adds exact zeros.
//
// AM adds the argmax's pass 1 as an epilogue, in any layout: as each group of
// rows finishes, its candidates (value, lowest row) go into the workgroup's
// per-batch-row maximum in LDS (an atomic max), and the last half wave to
// finish writes the workgroup's record, or the non-finite flag, to
// rec[bb][blockIdx.x]; y may then be null.
template <int B, int R, int P, bool RAGGED, bool AM, int MAXT = kThreads, int BITS = 4>
__global__ __launch_bounds__(MAXT) void gemv_valu_kernel(const uint32_t* __restrict__ wq,
                                                         const uint16_t* __restrict__ scales,
                                                         const uint16_t* __restrict__ biases,
                                                         const uint16_t* __restrict__ x,
                                                         float* __restrict__ y, int64_t N,
                                                         int64_t K, int64_t rpw,
                                                         uint2* __restrict__ rec) {
  extern __shared__ uint4 s_mem[];
  typedef typename CodeVec<BITS>::V V;
  constexpr int VPL = CodeVec<BITS>::VPL;
  const int64_t KW = K * BITS / 32, K32 = K >> 5, G = K >> 6;  // KW: code words per row
  const int C = (int)((K + kChunk - 1) / kChunk);
  uint4* s_xp = s_mem;                                                   // [B][C][4][32]
  float* s_xh = reinterpret_cast<float*>(s_mem + (int64_t)B * C * 128);  // [B][C][32]

  const int tid = threadIdx.x;
  const int lane = tid & 31;
  const int H = (int)(blockDim.x >> 5), hwi = tid >> 5;
  const int64_t wg_begin = (int64_t)blockIdx.x * rpw;
  const int64_t wg_end = N - wg_begin < rpw ? N : wg_begin + rpw;
  const int64_t wg_groups = (wg_end - wg_begin + R - 1) / R;
  const int lead = hwi & ~1;  // the wave's first half wave sets the group count
  const int64_t ng = wg_groups > lead ? (wg_groups - lead + H - 1) / H : 0;
  const int64_t row_begin = wg_begin + (int64_t)hwi * R;
  const int64_t row_step = (int64_t)H * R;
  const int64_t n_items = ng * C;
  const int last_lanes = (int)((K - (int64_t)(C - 1) * kChunk) >> 5);  // active lanes, chunk C-1
  const uint32_t m = kNibbles, g = kMagic128;

  // this lane's position in the rows of the group being loaded (set once per
  // group); an item adds the chunk's offset to each
  const V* pw[R];
  const uint16_t* ps[R];
  const uint16_t* pb[R];
  int64_t prow = row_begin;
  auto set_rows = [&]() {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int64_t row = prow + r < wg_end ? prow + r : wg_end - 1;
      pw[r] = reinterpret_cast<const V*>(wq + row * KW) + VPL * lane;
      ps[r] = scales + row * G + (lane >> 1);
      pb[r] = biases + row * G + (lane >> 1);
    }
  };
  set_rows();
  int pc = 0;  // chunk of the next item to load
  // Loads the next item.  The stream below never asks for an item past the
  // last one, except in the prologue when a half wave has fewer than P items;
  // those loads read clamped, valid rows and are never consumed.
  auto issue = [&](Item<R, BITS>& it) {
    int vo = pc * 32 * VPL, go = pc * 16;  // vector and group offsets of the chunk
    if (RAGGED && pc == C - 1 && lane >= last_lanes) {  // past the end: lane 0's data
      vo = -VPL * lane;
      go = -(lane >> 1);
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
#pragma unroll
      for (int v = 0; v < VPL; ++v) it.w[r][v] = ld_stream(pw[r] + vo + v);
      it.s[r] = ps[r][go];
      it.b[r] = pb[r][go];
    }
    if (++pc == C) {
      pc = 0;
      prow += row_step;
      set_rows();
    }
  };
  // ---- stage x: pair each 8-element block, and sum each 32-element lane segment.
  // The first XPRE segments of each thread are loaded before the first P items'
  // codes are issued, so that waiting for them does not also wait for the codes.
  constexpr int XPRE = 2;
  const int64_t nseg = B * K32;
  auto put_seg = [&](int64_t seg, const uint4 (&raw)[4]) {
    const int bb = (int)(seg / K32);
    const int64_t sg = seg % K32;
    const int64_t c = sg >> 5, l = sg & 31;
    float h = 0.0f;
    uint4 pr[4];
    if constexpr (BITS == 2) {
      pair_x2(raw[0], raw[1], pr[0], pr[1]);
      pair_x2(raw[2], raw[3], pr[2], pr[3]);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint4 p = BITS == 4 ? pair_x(raw[i]) : BITS == 8 ? pair_x8(raw[i]) : pr[i];
      s_xp[((int64_t)bb * C + c) * 128 + i * 32 + l] = p;
      h = dot2(p.x, kOnes, h);
      h = dot2(p.y, kOnes, h);
      h = dot2(p.z, kOnes, h);
      h = dot2(p.w, kOnes, h);
    }
    s_xh[((int64_t)bb * C + c) * 32 + l] = h;
  };
  auto load_seg = [&](int64_t seg, uint4 (&raw)[4]) {
    const int bb = (int)(seg / K32);
    const int64_t sg = seg % K32;
    const uint4* src = reinterpret_cast<const uint4*>(x + (int64_t)bb * K + sg * 32);
#pragma unroll
    for (int i = 0; i < 4; ++i) raw[i] = src[i];
  };
  uint4 pre[XPRE][4];
#pragma unroll
  for (int q = 0; q < XPRE; ++q) {
    const int64_t seg = tid + (int64_t)q * blockDim.x;
    if (seg < nseg) load_seg(seg, pre[q]);
  }

  Item<R, BITS> ring[P];
#pragma unroll
  for (int sl = 0; sl < P; ++sl) issue(ring[sl]);

  // argmax epilogue: the workgroup's best candidate so far per batch row, a bit
  // per batch row for a non-finite value, and the count of half waves done
  // (cleared before the barrier that ends the staging of x)
  __shared__ uint64_t s_best[AM ? B : 1];
  __shared__ uint32_t s_bad, s_done;
  if (AM && tid == 0) {
#pragma unroll
    for (int bb = 0; bb < B; ++bb) s_best[bb] = 0;
    s_bad = 0;
    s_done = 0;
  }

#pragma unroll
  for (int q = 0; q < XPRE; ++q) {
    const int64_t seg = tid + (int64_t)q * blockDim.x;
    if (seg < nseg) put_seg(seg, pre[q]);
  }
  for (int64_t seg = tid + (int64_t)XPRE * blockDim.x; seg < nseg; seg += blockDim.x) {
    uint4 raw[4];
    load_seg(seg, raw);
    put_seg(seg, raw);
  }
  __syncthreads();

  // ---- stream
  float acc[R][B];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int bb = 0; bb < B; ++bb) acc[r][bb] = 0.0f;
  int64_t crow = row_begin;
  int cc = 0;

  const uint4* xlane = s_xp + lane;
  const float* hlane = s_xh + lane;
  auto consume = [&](const Item<R, BITS>& it, int64_t item) {
    if (item < n_items) {
      // a lane past the end of a short last chunk reads lane 0 of chunk 0
      // (always staged, so finite) and scales it by exact zeros
      bool active = true;
      int xo = cc * 128, ho = cc * 32;
      if (RAGGED && cc == C - 1 && lane >= last_lanes) {
        active = false;
        xo = -lane;
        ho = -lane;
      }
      float sc[R], cb[R];
#pragma unroll
      for (int r = 0; r < R; ++r) {
        sc[r] = bf16_to_f32(it.s[r]);
        // the constant part of the expanded codes: 128 per code, 128 + 16 * 128
        // per 8-bit code (two nibbles)
        cb[r] = __builtin_fmaf(BITS == 8 ? -2176.0f : -128.0f, sc[r], bf16_to_f32(it.b[r]));
        if (RAGGED && !active) sc[r] = cb[r] = 0.0f;
      }
#pragma unroll
      for (int bb = 0; bb < B; ++bb) {
        const uint4* xv = xlane + (int64_t)bb * C * 128 + xo;
        const uint4 x0 = xv[0], x1 = xv[32], x2 = xv[64], x3 = xv[96];
        const float xh = hlane[(int64_t)bb * C * 32 + ho];
#pragma unroll
        for (int r = 0; r < R; ++r) {
          float d = 0.0f;
          if constexpr (BITS == 4) {
            d = dot_word(it.w[r][0].x, x0, d, m, g);
            d = dot_word(it.w[r][0].y, x1, d, m, g);
            d = dot_word(it.w[r][0].z, x2, d, m, g);
            d = dot_word(it.w[r][0].w, x3, d, m, g);
          } else if constexpr (BITS == 2) {
            d = dot_word2(it.w[r][0].x, x0, x1, d, g);
            d = dot_word2(it.w[r][0].y, x2, x3, d, g);
          } else {
            float dl = 0.0f, dh = 0.0f;
            dot_word8(it.w[r][0].x, x0.x, x0.y, dl, dh, m, g);
            dot_word8(it.w[r][0].y, x0.z, x0.w, dl, dh, m, g);
            dot_word8(it.w[r][0].z, x1.x, x1.y, dl, dh, m, g);
            dot_word8(it.w[r][0].w, x1.z, x1.w, dl, dh, m, g);
            dot_word8(it.w[r][1].x, x2.x, x2.y, dl, dh, m, g);
            dot_word8(it.w[r][1].y, x2.z, x2.w, dl, dh, m, g);
            dot_word8(it.w[r][1].z, x3.x, x3.y, dl, dh, m, g);
            dot_word8(it.w[r][1].w, x3.z, x3.w, dl, dh, m, g);
            d = __builtin_fmaf(16.0f, dh, dl);  // sum x q = Dl + 16 Dh - 2176 X
          }
          acc[r][bb] = __builtin_fmaf(sc[r], d, acc[r][bb]);
          acc[r][bb] = __builtin_fmaf(cb[r], xh, acc[r][bb]);
        }
      }
      if (++cc == C) {
        // B = 1: every lane holds the sum and lane 0 stores it; B >= 2: the
        // transposed tree leaves batch row bq's sum in lanes of its own, and
        // the first of them stores it, so the stores and the argmax fold of a
        // group are one branch, not one per (row, batch row)
        float mine[R];
        int bq = 0;
        bool st = lane == 0;
        if constexpr (B == 1) {
#pragma unroll
          for (int r = 0; r < R; ++r) {
            mine[r] = half_wave_sum(acc[r][0]);
            acc[r][0] = 0.0f;
          }
        } else {
          constexpr int NB = sums_width(B);
          bq = half_wave_index<NB>(lane);
          st = half_wave_first<NB>(lane) && bq < B;
#pragma unroll
          for (int r = 0; r < R; ++r) {
            float v[NB];
#pragma unroll
            for (int bb = 0; bb < NB; ++bb) v[bb] = bb < B ? acc[r][bb < B ? bb : 0] : 0.0f;
            mine[r] = half_wave_sums<NB>(v, lane);
#pragma unroll
            for (int bb = 0; bb < B; ++bb) acc[r][bb] = 0.0f;
          }
        }
        if (st) {
          uint64_t best = 0;
          bool bad = false;
#pragma unroll
          for (int r = 0; r < R; ++r) {
            if (crow + r < wg_end) {
              if (!AM || y != nullptr) y[(int64_t)bq * N + crow + r] = mine[r];
              if constexpr (AM) {
                const uint32_t u = __float_as_uint(mine[r]);
                if (!finite_bits(u)) bad = true;
                else best = umax64(best, cand(u, (uint32_t)(crow + r)));
              }
            }
          }
          if constexpr (AM) {
            // (a candidate word is never 0: every finite value's key is above 0)
            if (bad) __hip_atomic_fetch_or(&s_bad, 1u << bq, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            if (best)
              __hip_atomic_fetch_max(&s_best[bq], best, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
          }
        }
        cc = 0;
        crow += row_step;
      }
    }
  };
  // steady state: every issued item exists; the loads stay unconditional so
  // each wait counts exactly the loads of the items still in flight
  int64_t it = 0;
  for (; it + 2 * P - 1 < n_items; it += P) {
#pragma unroll
    for (int sl = 0; sl < P; ++sl) {
      consume(ring[sl], it + sl);
      issue(ring[sl]);
    }
  }
  // the last items (fewer than 2P)
#pragma unroll
  for (int sl = 0; sl < P; ++sl) {
    consume(ring[sl], it + sl);
    if (it + sl + P < n_items) issue(ring[sl]);
  }
#pragma unroll
  for (int sl = 0; sl < P; ++sl) consume(ring[sl], it + P + sl);

  if constexpr (AM) {
    // The last half wave to finish writes the workgroup's record per batch row:
    // the best (value, lowest row), or the non-finite flag.  A maximum, so it
    // does not depend on which half wave took which rows or finished first; no
    // barrier, so finished waves leave at once as in the plain product.  (The
    // count's release orders each half wave's maxima before it; the last one's
    // acquire sees them all.)
    if (lane == 0 &&
        __hip_atomic_fetch_add(&s_done, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_WORKGROUP) == (uint32_t)H - 1) {
      const uint32_t bad = __hip_atomic_load(&s_bad, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
#pragma unroll
      for (int bb = 0; bb < B; ++bb)
        rec[(int64_t)bb * gridDim.x + blockIdx.x] =
            make_record(__hip_atomic_load(&s_best[bb], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP),
                        ((bad >> bb) & 1u) != 0, (uint32_t)wg_begin);
    }
  }
}

// Workgroup barrier for data exchanged through LDS only (the loads in flight
// are not waited for).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
}

// Step-staged variant for batches whose paired activations exceed LDS, and for
// one row of long activations, where a CU's share is at most 24 rows: the
// workgroup's first waves compute (R rows
// per half wave, every half wave taking its rows' chunks in ascending order,
// all in step), the last ceil(B / 2) waves only stage the activations of the
// batch, one chunk at a time, into two LDS buffers (chunk c + 1 is stored
// while chunk c is used; one barrier per chunk).  Two kinds of waves keep the
// staging registers apart from the compute registers.  Per row the arithmetic
// and its order are gemv_valu_kernel's (the same chunk loop into one
// accumulator per batch row, the same lane tree; a lane past the end of a
// short last chunk reads lane 0 of chunk 0, kept in LDS for the purpose, and
// adds exact zeros), so the bits are the same, and the weights are read once
// for the whole batch; the codes stream from the first chunk on instead of
// after all of x is staged.  P: items of codes in flight per half wave; PS:
// chunks of activations in flight per staging lane.
// AM: the argmax epilogue as in gemv_valu_kernel.
template <int B, int R, int P, int PS, bool RAGGED, bool AM, int BITS = 4>
__global__ __launch_bounds__(B == 1 ? 1024 : 512) void gemv_valu_step_kernel(const uint32_t* __restrict__ wq,
                                                             const uint16_t* __restrict__ scales,
                                                             const uint16_t* __restrict__ biases,
                                                             const uint16_t* __restrict__ x,
                                                             float* __restrict__ y, int64_t N,
                                                             int64_t K, int64_t rpw, int ncw,
                                                             uint2* __restrict__ rec) {
  extern __shared__ uint4 s_mem[];
  typedef typename CodeVec<BITS>::V V;
  constexpr int VPL = CodeVec<BITS>::VPL;
  const int64_t KW = K * BITS / 32, G = K >> 6;
  const int C = (int)((K + kChunk - 1) / kChunk);
  // two chunk buffers, then (RAGGED) a copy of chunk 0 for the lanes past the
  // end of the short last chunk: [3][B][4][32] pairs, then [3][B][32] sums
  constexpr int NBUF = RAGGED ? 3 : 2;
  uint4* s_xp = s_mem;
  float* s_xh = reinterpret_cast<float*>(s_mem + NBUF * B * 128);
  __shared__ uint64_t s_best[AM ? B : 1];
  __shared__ uint32_t s_bad;

  const int tid = threadIdx.x;
  const int lane = tid & 31;
  const int64_t wg_begin = (int64_t)blockIdx.x * rpw;
  const int64_t wg_end = N - wg_begin < rpw ? N : wg_begin + rpw;
  if (AM && tid == 0) {
#pragma unroll
    for (int bb = 0; bb < B; ++bb) s_best[bb] = 0;
    s_bad = 0;
  }

  if (__builtin_amdgcn_readfirstlane(tid >> 6) >= ncw) {
    // staging lane: segment `lane` of batch row sbb (an odd batch's last half
    // wave repeats row B - 1: the same values to the same places).  A segment
    // past the end of a short last chunk loads the chunk's first segment; its
    // slots are never read.
    const int st = tid - 64 * ncw;
    const int sbb = (st >> 5) < B ? (st >> 5) : B - 1;
    auto load_chunk = [&](int c, uint4 (&raw)[4]) {
      if (c > C - 1) c = C - 1;
      int64_t e = (int64_t)c * kChunk + (int64_t)lane * 32;
      if (e >= K) e = (int64_t)c * kChunk;
      const uint4* src = reinterpret_cast<const uint4*>(x + (int64_t)sbb * K + e);
#pragma unroll
      for (int i = 0; i < 4; ++i) raw[i] = src[i];
    };
    auto put_chunk = [&](int c, const uint4 (&raw)[4]) {
      const int buf = c & 1;
      float h = 0.0f;
      uint4 pr[4];
      if constexpr (BITS == 2) {
        pair_x2(raw[0], raw[1], pr[0], pr[1]);
        pair_x2(raw[2], raw[3], pr[2], pr[3]);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint4 q = BITS == 4 ? pair_x(raw[i]) : BITS == 8 ? pair_x8(raw[i]) : pr[i];
        s_xp[(buf * B + sbb) * 128 + i * 32 + lane] = q;
        if (RAGGED && c == 0) s_xp[(2 * B + sbb) * 128 + i * 32 + lane] = q;
        h = dot2(q.x, kOnes, h);
        h = dot2(q.y, kOnes, h);
        h = dot2(q.z, kOnes, h);
        h = dot2(q.w, kOnes, h);
      }
      s_xh[(buf * B + sbb) * 32 + lane] = h;
      if (RAGGED && c == 0) s_xh[(2 * B + sbb) * 32 + lane] = h;
    };
    // chunk k in raw[k % PS]; chunk 0 stored before the first barrier, chunk
    // c + 1 after barrier c, then chunk c + 1 + PS loaded in its place
    // (the loads stay unconditional, past the last chunk rereading it, so that
    // each store waits for its own chunk only)
    uint4 raw[PS][4];
#pragma unroll
    for (int k = 0; k < PS; ++k) load_chunk(k, raw[k]);
    put_chunk(0, raw[0]);
    load_chunk(PS, raw[0]);
    int c = 0;
    for (; c + PS < C; c += PS) {
#pragma unroll
      for (int k = 0; k < PS; ++k) {
        lds_barrier();
        put_chunk(c + k + 1, raw[(k + 1) % PS]);
        load_chunk(c + k + 1 + PS, raw[(k + 1) % PS]);
      }
    }
#pragma unroll
    for (int k = 0; k < PS; ++k) {
      if (c + k < C) {
        lds_barrier();
        if (c + k + 1 < C) put_chunk(c + k + 1, raw[(k + 1) % PS]);
      }
    }
    if constexpr (AM) __syncthreads();
    return;
  }

  const int hwi = tid >> 5;
  const int64_t row0 = wg_begin + (int64_t)hwi * R;  // this half wave's rows (past the share: valid rows, not stored)
  const int last_lanes = (int)((K - (int64_t)(C - 1) * kChunk) >> 5);
  const uint32_t m = kNibbles, g = kMagic128;

  const V* pw[R];
  const uint16_t* ps[R];
  const uint16_t* pb[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int64_t lrow = row0 + r < wg_end ? row0 + r : wg_end - 1;
    pw[r] = reinterpret_cast<const V*>(wq + lrow * KW) + VPL * lane;
    ps[r] = scales + lrow * G + (lane >> 1);
    pb[r] = biases + lrow * G + (lane >> 1);
  }
  int pc = 0;  // chunk of the next item to load (past the last: the last again, never consumed)
  auto issue = [&](Item<R, BITS>& it) {
    const int c = pc < C ? pc : C - 1;
    int vo = c * 32 * VPL, go = c * 16;
    if (RAGGED && c == C - 1 && lane >= last_lanes) {
      vo = -VPL * lane;
      go = -(lane >> 1);
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
#pragma unroll
      for (int v = 0; v < VPL; ++v) it.w[r][v] = ld_stream(pw[r] + vo + v);
      it.s[r] = ps[r][go];
      it.b[r] = pb[r][go];
    }
    ++pc;
  };
  Item<R, BITS> ring[P];
#pragma unroll
  for (int k = 0; k < P; ++k) issue(ring[k]);

  float acc[R][B];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int bb = 0; bb < B; ++bb) acc[r][bb] = 0.0f;
  // item c: chunk c of this half wave's rows
  auto consume = [&](const Item<R, BITS>& it, int c) {
    // all half waves are done with chunk c - 1 and chunk c is staged (nothing
    // of this item is moved above the barrier, where it would wait for loads
    // issued after the ones the previous item needs)
    lds_barrier();
    __builtin_amdgcn_sched_barrier(0);
    bool active = true;
    if (RAGGED && c == C - 1 && lane >= last_lanes) active = false;
    float sc[R], cb[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      sc[r] = bf16_to_f32(it.s[r]);
      cb[r] = __builtin_fmaf(BITS == 8 ? -2176.0f : -128.0f, sc[r], bf16_to_f32(it.b[r]));
      if (RAGGED && !active) sc[r] = cb[r] = 0.0f;
    }
#pragma unroll
    for (int bb = 0; bb < B; ++bb) {
      // (a lane past the end of a short last chunk: lane 0 of the chunk-0 copy)
      const int xb = (!RAGGED || active) ? ((c & 1) * B + bb) : (2 * B + bb);
      const int xl = (!RAGGED || active) ? lane : 0;
      const uint4* xv = s_xp + xb * 128 + xl;
      const uint4 x0 = xv[0], x1 = xv[32], x2 = xv[64], x3 = xv[96];
      const float xh = s_xh[xb * 32 + xl];
#pragma unroll
      for (int r = 0; r < R; ++r) {
        float d = 0.0f;
        if constexpr (BITS == 4) {
          d = dot_word(it.w[r][0].x, x0, d, m, g);
          d = dot_word(it.w[r][0].y, x1, d, m, g);
          d = dot_word(it.w[r][0].z, x2, d, m, g);
          d = dot_word(it.w[r][0].w, x3, d, m, g);
        } else if constexpr (BITS == 2) {
          d = dot_word2(it.w[r][0].x, x0, x1, d, g);
          d = dot_word2(it.w[r][0].y, x2, x3, d, g);
        } else {
          float dl = 0.0f, dh = 0.0f;
          dot_word8(it.w[r][0].x, x0.x, x0.y, dl, dh, m, g);
          dot_word8(it.w[r][0].y, x0.z, x0.w, dl, dh, m, g);
          dot_word8(it.w[r][0].z, x1.x, x1.y, dl, dh, m, g);
          dot_word8(it.w[r][0].w, x1.z, x1.w, dl, dh, m, g);
          dot_word8(it.w[r][1].x, x2.x, x2.y, dl, dh, m, g);
          dot_word8(it.w[r][1].y, x2.z, x2.w, dl, dh, m, g);
          dot_word8(it.w[r][1].z, x3.x, x3.y, dl, dh, m, g);
          dot_word8(it.w[r][1].w, x3.z, x3.w, dl, dh, m, g);
          d = __builtin_fmaf(16.0f, dh, dl);
        }
        acc[r][bb] = __builtin_fmaf(sc[r], d, acc[r][bb]);
        acc[r][bb] = __builtin_fmaf(cb[r], xh, acc[r][bb]);
      }
    }
  };
  // every half wave has exactly C items; the loads stay unconditional (past
  // the last chunk they reread it and are never consumed)
  int c = 0;
  for (; c + 2 * P - 1 < C; c += P) {
#pragma unroll
    for (int k = 0; k < P; ++k) {
      consume(ring[k], c + k);
      issue(ring[k]);
    }
  }
#pragma unroll
  for (int k = 0; k < P; ++k) {
    if (c + k < C) consume(ring[k], c + k);
    if (c + k + P < C) issue(ring[k]);
  }
#pragma unroll
  for (int k = 0; k < P; ++k)
    if (c + P + k < C) consume(ring[k], c + P + k);

  // the rows' sums: B = 1, every lane holds them and lane 0 stores; B >= 2,
  // the transposed tree leaves batch row bq's in lanes of its own
  float mine[R];
  int bq = 0;
  bool st = lane == 0;
  if constexpr (B == 1) {
#pragma unroll
    for (int r = 0; r < R; ++r) mine[r] = half_wave_sum(acc[r][0]);
  } else {
    constexpr int NB = sums_width(B);
    bq = half_wave_index<NB>(lane);
    st = half_wave_first<NB>(lane) && bq < B;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      float v[NB];
#pragma unroll
      for (int bb = 0; bb < NB; ++bb) v[bb] = bb < B ? acc[r][bb < B ? bb : 0] : 0.0f;
      mine[r] = half_wave_sums<NB>(v, lane);
    }
  }
  if (st) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int64_t row = row0 + r;
      if (row < wg_end) {
        if (!AM || y != nullptr) y[(int64_t)bq * N + row] = mine[r];
        if constexpr (AM) {
          const uint32_t u = __float_as_uint(mine[r]);
          if (!finite_bits(u))
            __hip_atomic_fetch_or(&s_bad, 1u << bq, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
          else
            __hip_atomic_fetch_max(&s_best[bq], cand(u, (uint32_t)row), __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_WORKGROUP);
        }
      }
    }
  }
  if constexpr (AM) {
    __syncthreads();
    if (tid < B)
      rec[(int64_t)tid * gridDim.x + blockIdx.x] =
          make_record(s_best[tid], ((s_bad >> tid) & 1u) != 0, (uint32_t)wg_begin);
  }
}

// Register-staged variant of the same arithmetic, for shapes whose paired
// activations do not fit in LDS (B * 2.125 * K bytes above the limit): each
// 64-lane workgroup owns 2R rows, a half wave R of them, and reads the x pairs
// of a chunk straight into registers.  Every floating-point step, and its
// order, is the one described at the top of this file, so both variants give
// the same bits.
// AM: the argmax epilogue as in gemv_valu_kernel (one record per batch row per
// 64-lane workgroup).
template <int B, int R, bool AM>
__global__ __launch_bounds__(64) void gemv_valu_regs_kernel(const uint32_t* __restrict__ wq,
                                                            const uint16_t* __restrict__ scales,
                                                            const uint16_t* __restrict__ biases,
                                                            const uint16_t* __restrict__ x,
                                                            float* __restrict__ y, int64_t N,
                                                            int64_t K, uint2* __restrict__ rec) {
  const int lane = threadIdx.x & 31;
  const int64_t row0 = ((int64_t)blockIdx.x * 2 + (threadIdx.x >> 5)) * R;
  const int64_t G = K >> 6;
  const int64_t K8 = K >> 3;
  const uint32_t m = kNibbles, g = kMagic128;
  float acc[R][B];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int bb = 0; bb < B; ++bb) acc[r][bb] = 0.0f;
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
        wv[r] = ld_stream(reinterpret_cast<const uint4*>(wq + rows[r] * K8 + (kb >> 3)));
        sv[r] = scales[rows[r] * G + (kb >> 6)];
        bv[r] = biases[rows[r] * G + (kb >> 6)];
      }
#pragma unroll
      for (int bb = 0; bb < B; ++bb) {
        const uint4* xs = reinterpret_cast<const uint4*>(x + (int64_t)bb * K + kb);
        uint4 xp[4];
        float xh = 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          xp[i] = pair_x(xs[i]);
          xh = dot2(xp[i].x, kOnes, xh);
          xh = dot2(xp[i].y, kOnes, xh);
          xh = dot2(xp[i].z, kOnes, xh);
          xh = dot2(xp[i].w, kOnes, xh);
        }
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const float sc = bf16_to_f32(sv[r]);
          const float cb = __builtin_fmaf(-128.0f, sc, bf16_to_f32(bv[r]));
          float d = 0.0f;
          d = dot_word(wv[r].x, xp[0], d, m, g);
          d = dot_word(wv[r].y, xp[1], d, m, g);
          d = dot_word(wv[r].z, xp[2], d, m, g);
          d = dot_word(wv[r].w, xp[3], d, m, g);
          acc[r][bb] = __builtin_fmaf(sc, d, acc[r][bb]);
          acc[r][bb] = __builtin_fmaf(cb, xh, acc[r][bb]);
        }
      }
    }
  }
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int bb = 0; bb < B; ++bb) acc[r][bb] = half_wave_sum(acc[r][bb]);
  if (lane == 0 && (!AM || y != nullptr)) {
#pragma unroll
    for (int r = 0; r < R; ++r)
      if (row0 + r < N)
#pragma unroll
        for (int bb = 0; bb < B; ++bb) y[(int64_t)bb * N + row0 + r] = acc[r][bb];
  }
  if constexpr (AM) {
#pragma unroll
    for (int bb = 0; bb < B; ++bb) {
      uint64_t best = 0;
      bool bad = false;
#pragma unroll
      for (int r = 0; r < R; ++r) {
        if (row0 + r < N) {
          const uint32_t u = __float_as_uint(acc[r][bb]);
          if (!finite_bits(u)) bad = true;
          else best = umax64(best, cand(u, (uint32_t)(row0 + r)));
        }
      }
      // the two half waves meet in lane 0
      const uint32_t lo = __shfl((uint32_t)best, 32), hi = __shfl((uint32_t)(best >> 32), 32);
      const int bad2 = __shfl(bad ? 1 : 0, 32);
      if (threadIdx.x == 0)
        rec[(int64_t)bb * gridDim.x + blockIdx.x] =
            make_record(umax64(best, ((uint64_t)hi << 32) | lo), bad || bad2 != 0,
                        (uint32_t)((int64_t)blockIdx.x * 2 * R));
    }
  }
}

size_t lds_bytes(int B, int64_t K) {
  const int64_t C = (K + kChunk - 1) / kChunk;
  return (size_t)B * (size_t)C * (128 * 16 + 32 * 4);
}

// Few rows (N below 16 per-item groups of 1024) take one row per item and a
// deeper ring in the short layout.
bool few_rows(int64_t N) { return N < (int64_t)kHalfWaves * 2 * 1024; }
int regs_rows(int B) { return B <= 2 ? 4 : 2; }
bool use_regs(int B, int64_t K, bool force_regs) { return force_regs || lds_bytes(B, K) > kMaxLds; }

template <int B, int R, int P, bool AM, int MAXT = kThreads, int BITS = 4>
hipError_t launch_lds(const uint32_t* wq, const uint16_t* scales, const uint16_t* biases,
                      const uint16_t* x, float* y, uint2* rec, int64_t N, int64_t K, int64_t rpw,
                      int threads, hipStream_t stream) {
  const bool ragged = (K % kChunk) != 0;
  const int64_t blocks = (N + rpw - 1) / rpw;
  const size_t lds = lds_bytes(B, K);
  const void* fn = ragged ? reinterpret_cast<const void*>(&gemv_valu_kernel<B, R, P, true, AM, MAXT, BITS>)
                          : reinterpret_cast<const void*>(&gemv_valu_kernel<B, R, P, false, AM, MAXT, BITS>);
  if (lds > kDefaultLds) {
    // a host-side attribute of the kernel, set before each such launch (not a
    // stream operation, so it is also fine while a graph is being captured)
    const hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)kMaxLds);
    if (e != hipSuccess) return e;
  }
  if (ragged)
    hipLaunchKernelGGL((gemv_valu_kernel<B, R, P, true, AM, MAXT, BITS>), dim3((unsigned)blocks), dim3(threads),
                       lds, stream, wq, scales, biases, x, y, N, K, rpw, rec);
  else
    hipLaunchKernelGGL((gemv_valu_kernel<B, R, P, false, AM, MAXT, BITS>), dim3((unsigned)blocks), dim3(threads),
                       lds, stream, wq, scales, biases, x, y, N, K, rpw, rec);
  return hipGetLastError();
}

// 256 threads, short_groups() groups of R rows per half wave: many short
// workgroups, which the dispatcher spreads over the CUs as they free up
// Groups of R rows per half wave in the short layout: two (32-row workgroups
// for R = 2; measured on the vocabulary-wide head at B = 1 on three GPUs: as
// fast as one group or up to 5% faster, and half the fused head's records).
int short_groups() { return 2; }

template <int B, int R, int P, bool AM, int BITS = 4>
hipError_t launch_short(const uint32_t* wq, const uint16_t* scales, const uint16_t* biases,
                        const uint16_t* x, float* y, uint2* rec, int64_t N, int64_t K,
                        hipStream_t stream) {
  return launch_lds<B, R, P, AM, kThreads, BITS>(wq, scales, biases, x, y, rec, N, K,
                                                 (int64_t)kHalfWaves * R * short_groups(), kThreads, stream);
}

// One workgroup per CU, each with an equal share of the rows (so every CU
// streams the same number of bytes and no second round of workgroups
// trails; x is staged once per CU): up to 32 rows per CU one row per half
// wave, else 16 half waves striding through the share, R rows per item.
// (Launch bounds: 640 threads for shares of at most 20 groups of R rows, one
// group per half wave; else 512 threads, 16 half waves striding.)
int64_t per_cu_rows(int64_t N, int cus) { return (N + cus - 1) / cus; }
int64_t per_cu_rows(int64_t N) { return per_cu_rows(N, cu_count()); }

template <int R, int P, int BITS = 4, int B = 1, bool AM = false>
hipError_t launch_per_cu(const uint32_t* wq, const uint16_t* scales, const uint16_t* biases,
                         const uint16_t* x, float* y, int64_t N, int64_t K, hipStream_t stream,
                         uint2* rec = nullptr) {
  const int64_t rpw = per_cu_rows(N);
  // (R >= 2 at B >= 2 runs only for shares above 40 rows, so that it never
  // takes the 640-thread variant, which is not built for it; nor are 8-bit
  // codes at B >= 7, whose registers exceed the 640-thread budget)
  if constexpr (!(R >= 2 && B >= 2) && !(BITS == 8 && B >= 7)) {
    if (rpw <= 20 * R)
      return launch_lds<B, R, P, AM, 640, BITS>(wq, scales, biases, x, y, rec, N, K, rpw,
                                                64 * (int)((rpw + 2 * R - 1) / (2 * R)), stream);
  }
  return launch_lds<B, R, P, AM, 512, BITS>(wq, scales, biases, x, y, rec, N, K, rpw, 512, stream);
}

// The layer widths (a CU's share below 512 rows) take the per-CU layout at
// B = 1; the vocabulary-wide head keeps the short workgroups there.
// (keyed on the MI355X's CU count whatever the device, so that the workspace
// bound of the fused head, computed with kMaxCUs, holds on any device)
bool b1_per_cu(int64_t N) { return per_cu_rows(N, kMaxCUs) < 2 * 16 * 16; }

template <int B, int R, bool AM>
hipError_t launch_regs(const uint32_t* wq, const uint16_t* scales, const uint16_t* biases,
                       const uint16_t* x, float* y, uint2* rec, int64_t N, int64_t K,
                       hipStream_t stream) {
  const int64_t blocks = (N + 2 * R - 1) / (2 * R);
  hipLaunchKernelGGL((gemv_valu_regs_kernel<B, R, AM>), dim3((unsigned)blocks), dim3(64), 0, stream,
                     wq, scales, biases, x, y, N, K, rec);
  return hipGetLastError();
}

// The one dispatch both entry points share: the kernel, R and P are functions
// of (B, N, K) and force_regs only, and the workgroup count follows from them.
// The largest batch whose activations fit in the shared-memory variant's LDS
// (0 if not even one row's do).
int lds_rows(int64_t K) {
  int b = 0;
  while (b < 8 && !use_regs(b + 1, K, false)) ++b;
  return b;
}

// The per-CU layout for any batch (1..8): R = 2 over more than 40 rows per CU
// at B >= 2, R = 4 over more than 512 (the vocabulary-wide head: each pass of
// the activations through LDS feeds twice the rows; measured at B = 2..8,
// 3-11% faster than R = 2).  Every batch size takes the same workgroups, so the
// batch can be cut into parts that write their records side by side.
template <bool AM>
hipError_t launch_per_cu_any(const uint32_t* wq, const uint16_t* scales, const uint16_t* biases,
                             const uint16_t* x, float* y, uint2* rec, int B, int64_t N, int64_t K,
                             hipStream_t stream) {
  if (B == 1) return launch_per_cu<1, 4, 4, 1, AM>(wq, scales, biases, x, y, N, K, stream, rec);
  const int64_t rows = per_cu_rows(N);
  const bool two = rows > 40, four = rows > 512;  // (R >= 2 then always strides: 512 threads)
  switch (B) {
#define W4G_PER_CU(BB)                                                                               \
    case BB:                                                                                         \
      return four  ? launch_per_cu<4, 2, 4, BB, AM>(wq, scales, biases, x, y, N, K, stream, rec)     \
             : two ? launch_per_cu<2, 2, 4, BB, AM>(wq, scales, biases, x, y, N, K, stream, rec)     \
                   : launch_per_cu<1, 2, 4, BB, AM>(wq, scales, biases, x, y, N, K, stream, rec);
    W4G_PER_CU(2) W4G_PER_CU(3) W4G_PER_CU(4) W4G_PER_CU(5) W4G_PER_CU(6) W4G_PER_CU(7) W4G_PER_CU(8)
#undef W4G_PER_CU
    default: return hipErrorInvalidValue;
  }
}

// Where the activations of the whole batch do not fit in LDS but those of two
// rows or more do (down_proj, K = 17,408, from B = 5), the batch is cut into
// the fewest equal parts that fit, each a launch of the per-CU layout: the
// weights are read once per part, which measured faster than the
// register-staged variant (down at B = 8: two parts of 4 rows, about 40 us,
// against 70 us).  Every row has the bits it has alone, in any part.
int batch_parts(int B, int64_t K) {
  const int b = lds_rows(K);
  return b >= 2 && B > b ? (B + b - 1) / b : 1;
}

// Where a CU's share is at most 24 rows (decided with the MI355X's CU count,
// so that the records of the fused head stay within the bound computed the
// same way) the step-staged kernel serves every batch of three rows or more:
// it reads the weights once for the whole batch where the batch's activations
// do not fit in LDS (down at B = 8: 40 us in two parts before), and where they
// do, staging them a chunk at a time while the codes stream beats staging them
// whole first (o_proj at B = 3 / 8: 8.1 -> 7.7 / 11.9 -> 11.5 us, down at
// B = 3 / 4: 17.5 -> 16.0 / 19.8 -> 18.7 us; B = 2 gains nothing certain).
// Four computing waves of 2 x 3 rows (one per SIMD).  At B = 1 it takes shares
// of at most 20 rows whose x spans 8 chunks or more, one row per half wave, so
// that the codes stream while x is staged (down at B = 1: 11.8 -> 10.4 us;
// o_proj, 5 chunks, gains nothing).
constexpr int64_t kStepRows = 24;
constexpr int step_r(int B) { return B == 1 ? 1 : 3; }
bool use_step(int B, int64_t N, int64_t K) {
  const int64_t r = per_cu_rows(N, kMaxCUs);
  if (B == 1 && r <= 20 && K >= 8 * kChunk) return true;
  if (B >= 3 && r <= kStepRows) return true;
  return (batch_parts(B, K) > 1 || use_regs(B, K, false)) && r <= kStepRows;
}
int64_t step_rows(int64_t N, int cus) {
  const int64_t r = per_cu_rows(N, cus);
  return r < kStepRows ? r : kStepRows;
}
size_t step_lds_bytes(int B, bool ragged) {
  const size_t nbuf = ragged ? 3 : 2;
  return nbuf * (size_t)B * (128 * 16 + 32 * 4);
}

template <bool AM, int BITS = 4>
hipError_t launch_step(const uint32_t* wq, const uint16_t* scales, const uint16_t* biases,
                       const uint16_t* x, float* y, uint2* rec, int B, int64_t N, int64_t K,
                       hipStream_t stream) {
  const int64_t rpw = step_rows(N, cu_count());
  const int64_t blocks = (N + rpw - 1) / rpw;
  const int ncw = (int)((rpw + 2 * step_r(B) - 1) / (2 * step_r(B)));  // computing waves
  const int threads = 64 * (ncw + (B + 1) / 2);                        // then the staging waves
  const bool ragged = (K % kChunk) != 0;
  const size_t lds = step_lds_bytes(B, ragged);
  switch (B) {
#define W4G_STEP(BB)                                                                                        \
    case BB:                                                                                                \
      if (ragged)                                                                                           \
        hipLaunchKernelGGL((gemv_valu_step_kernel<BB, step_r(BB), 2, BB == 1 ? 5 : 3, true, AM, BITS>),       \
                           dim3((unsigned)blocks),                                                          \
                           dim3(threads), lds, stream, wq, scales, biases, x, y, N, K, rpw, ncw, rec);      \
      else                                                                                                  \
        hipLaunchKernelGGL((gemv_valu_step_kernel<BB, step_r(BB), 2, BB == 1 ? 5 : 3, false, AM, BITS>),      \
                           dim3((unsigned)blocks),                                                          \
                           dim3(threads), lds, stream, wq, scales, biases, x, y, N, K, rpw, ncw, rec);      \
      return hipGetLastError();
    W4G_STEP(1) W4G_STEP(2) W4G_STEP(3) W4G_STEP(4) W4G_STEP(5) W4G_STEP(6) W4G_STEP(7) W4G_STEP(8)
#undef W4G_STEP
    default: return hipErrorInvalidValue;
  }
}

// The one dispatch both entry points share: the kernel, R and P are functions
// of (B, N, K) and force_regs only, and the workgroup count follows from them.
template <bool AM>
hipError_t dispatch(const uint32_t* wq, const uint16_t* scales, const uint16_t* biases,
                    const uint16_t* x, float* y, uint2* rec, int B, int64_t N, int64_t K,
                    bool force_regs, hipStream_t stream) {
  if (!force_regs && use_step(B, N, K))
    return launch_step<AM>(wq, scales, biases, x, y, rec, B, N, K, stream);
  const int parts = force_regs ? 1 : batch_parts(B, K);
  if (parts > 1) {
    const int64_t grid = (N + per_cu_rows(N) - 1) / per_cu_rows(N);
    for (int p = 0, b0 = 0; p < parts; ++p) {
      const int bp = B / parts + (p < B % parts ? 1 : 0);
      const hipError_t e = launch_per_cu_any<AM>(wq, scales, biases, x + (int64_t)b0 * K,
                                                 y ? y + (int64_t)b0 * N : nullptr,
                                                 rec ? rec + (int64_t)b0 * grid : nullptr, bp, N, K, stream);
      if (e != hipSuccess) return e;
      b0 += bp;
    }
    return hipSuccess;
  }
  if (use_regs(B, K, force_regs)) {
    switch (B) {
      case 1: return launch_regs<1, 4, AM>(wq, scales, biases, x, y, rec, N, K, stream);
      case 2: return launch_regs<2, 4, AM>(wq, scales, biases, x, y, rec, N, K, stream);
      case 3: return launch_regs<3, 2, AM>(wq, scales, biases, x, y, rec, N, K, stream);
      case 4: return launch_regs<4, 2, AM>(wq, scales, biases, x, y, rec, N, K, stream);
      case 5: return launch_regs<5, 2, AM>(wq, scales, biases, x, y, rec, N, K, stream);
      case 6: return launch_regs<6, 2, AM>(wq, scales, biases, x, y, rec, N, K, stream);
      case 7: return launch_regs<7, 2, AM>(wq, scales, biases, x, y, rec, N, K, stream);
      case 8: return launch_regs<8, 2, AM>(wq, scales, biases, x, y, rec, N, K, stream);
      default: return hipErrorInvalidValue;
    }
  }
  if (B == 1) {
    // measured in the decode sweep
    if (b1_per_cu(N)) return launch_per_cu<1, 4, 4, 1, AM>(wq, scales, biases, x, y, N, K, stream, rec);
    return few_rows(N) ? launch_short<1, 1, 4, AM>(wq, scales, biases, x, y, rec, N, K, stream)
                       : launch_short<1, 2, 2, AM>(wq, scales, biases, x, y, rec, N, K, stream);
  }
  // B >= 2: the per-CU layout too, also for the head (measured: down at B = 4
  // 36 -> 22 us, gate-up at B = 8 90 -> 47 us, lm_head at B = 8 581 -> 322 us),
  // two rows per item when a CU's share exceeds 40 rows
  return launch_per_cu_any<AM>(wq, scales, biases, x, y, rec, B, N, K, stream);
}

// 2- and 8-bit codes: the shared-memory variant only (the caller checks that x
// fits), with the 4-bit layouts (per CU, short workgroups for the B = 1 head).
// AM: the argmax's pass 1 as the epilogue, one record per workgroup and batch
// row at rec (as for 4-bit codes).
template <int BITS, bool AM = false>
hipError_t dispatch_bits_lds(const uint32_t* wq, const uint16_t* scales, const uint16_t* biases,
                             const uint16_t* x, float* y, uint2* rec, int B, int64_t N, int64_t K, bool per_cu,
                             hipStream_t stream) {
  if (B == 1) {
    if (per_cu || b1_per_cu(N)) return launch_per_cu<1, 4, BITS, 1, AM>(wq, scales, biases, x, y, N, K, stream, rec);
    return launch_short<1, 2, 2, AM, BITS>(wq, scales, biases, x, y, rec, N, K, stream);
  }
  const bool two = per_cu_rows(N) > 40;
  switch (B) {
#define W4G_PER_CU(BB)                                                                                  \
    case BB:                                                                                            \
      return two ? launch_per_cu<2, 2, BITS, BB, AM>(wq, scales, biases, x, y, N, K, stream, rec)       \
                 : launch_per_cu<1, 2, BITS, BB, AM>(wq, scales, biases, x, y, N, K, stream, rec);
    W4G_PER_CU(2) W4G_PER_CU(3) W4G_PER_CU(4) W4G_PER_CU(5) W4G_PER_CU(6) W4G_PER_CU(7) W4G_PER_CU(8)
#undef W4G_PER_CU
    default: return hipErrorInvalidValue;
  }
}

// Other widths run the shared-memory variant only: where the batch's
// activations do not fit in LDS, the batch is cut into parts that do, as for
// 4-bit codes (the weights are read once per part), each part writing its
// records beside the others'; from B = 3 where a CU's share is at most 24 rows,
// and where the batch's activations exceed LDS (down_proj at K = 17,408 from
// B = 5), the step-staged kernel reads the weights once for the whole batch.
// The caller checks gemv_bits_fits.
template <int BITS, bool AM = false>
hipError_t dispatch_bits(const uint32_t* wq, const uint16_t* scales, const uint16_t* biases,
                         const uint16_t* x, float* y, uint2* rec, int B, int64_t N, int64_t K,
                         hipStream_t stream) {
  if (use_step(B, N, K)) return launch_step<AM, BITS>(wq, scales, biases, x, y, rec, B, N, K, stream);
  if (lds_rows(K) < 1) return hipErrorInvalidValue;
  const int parts = B > lds_rows(K) ? (B + lds_rows(K) - 1) / lds_rows(K) : 1;
  const int64_t grid = (N + per_cu_rows(N) - 1) / per_cu_rows(N);  // per-CU workgroups, when in parts
  for (int p = 0, b0 = 0; p < parts; ++p) {
    const int bp = B / parts + (p < B % parts ? 1 : 0);
    const hipError_t e = dispatch_bits_lds<BITS, AM>(wq, scales, biases, x + (int64_t)b0 * K,
                                                     y ? y + (int64_t)b0 * N : nullptr,
                                                     rec ? rec + (int64_t)b0 * grid : nullptr, bp, N, K,
                                                     parts > 1, stream);
    if (e != hipSuccess) return e;
    b0 += bp;
  }
  return hipSuccess;
}

// the workgroups of the layout dispatch_bits launches on a device with `cus`
// compute units, one record each
int64_t bits_records(int B, int64_t N, int64_t K, int cus) {
  if (use_step(B, N, K)) return (N + step_rows(N, cus) - 1) / step_rows(N, cus);
  const int parts = lds_rows(K) >= 1 && B > lds_rows(K) ? (B + lds_rows(K) - 1) / lds_rows(K) : 1;
  if (B == 1 && parts == 1 && !b1_per_cu(N)) {
    const int64_t rpw = (int64_t)kHalfWaves * 2 * short_groups();
    return (N + rpw - 1) / rpw;
  }
  return (N + per_cu_rows(N, cus) - 1) / per_cu_rows(N, cus);
}

}  // namespace

bool gemv_bits_fits(int B, int64_t K) { return B >= 1 && lds_rows(K) >= 1; }

hipError_t launch_gemv_bits(const uint32_t* wq, const uint16_t* scales, const uint16_t* biases,
                            const uint16_t* x, float* y, int B, int64_t N, int64_t K, int bits,
                            hipStream_t stream) {
  switch (bits) {
    case 2: return dispatch_bits<2>(wq, scales, biases, x, y, nullptr, B, N, K, stream);
    case 8: return dispatch_bits<8>(wq, scales, biases, x, y, nullptr, B, N, K, stream);
    default: return launch_gemv(wq, scales, biases, x, y, B, N, K, false, stream);
  }
}

int64_t gemv_bits_argmax_records(int B, int64_t N, int64_t K) { return bits_records(B, N, K, cu_count()); }
int64_t gemv_bits_argmax_records_max(int B, int64_t N, int64_t K) { return bits_records(B, N, K, kMaxCUs); }

hipError_t launch_gemv_bits_argmax(const uint32_t* wq, const uint16_t* scales, const uint16_t* biases,
                                   const uint16_t* x, float* y, uint2* rec, int B, int64_t N, int64_t K,
                                   int bits, hipStream_t stream) {
  switch (bits) {
    case 2: return dispatch_bits<2, true>(wq, scales, biases, x, y, rec, B, N, K, stream);
    case 8: return dispatch_bits<8, true>(wq, scales, biases, x, y, rec, B, N, K, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_gemv(const uint32_t* wq, const uint16_t* scales, const uint16_t* biases,
                       const uint16_t* x, float* y, int B, int64_t N, int64_t K, bool force_regs,
                       hipStream_t stream) {
  return dispatch<false>(wq, scales, biases, x, y, nullptr, B, N, K, force_regs, stream);
}

namespace {
// the workgroups of the layout dispatch() launches on a device with `cus`
// compute units, one record each
int64_t valu_records(int B, int64_t N, int64_t K, int cus) {
  if (use_step(B, N, K)) return (N + step_rows(N, cus) - 1) / step_rows(N, cus);
  if (batch_parts(B, K) > 1) return (N + per_cu_rows(N, cus) - 1) / per_cu_rows(N, cus);
  if (use_regs(B, K, false)) {
    const int R = regs_rows(B);
    return (N + 2 * R - 1) / (2 * R);
  }
  const int64_t rpw = (B >= 2 || b1_per_cu(N)) ? per_cu_rows(N, cus)
                                               : (int64_t)kHalfWaves * (few_rows(N) ? 1 : 2) * short_groups();
  return (N + rpw - 1) / rpw;
}
}  // namespace

int64_t gemv_argmax_records(int B, int64_t N, int64_t K) {
  if (gemv_auto_family(N, K) == 2) return gemv_mfma_argmax_records(B, N, K, cu_count());
  return valu_records(B, N, K, cu_count());
}

int64_t gemv_argmax_records_max(int B, int64_t N, int64_t K) {
  if (gemv_auto_family(N, K) == 2) return gemv_mfma_argmax_records(B, N, K, kMaxCUs);
  return valu_records(B, N, K, kMaxCUs);
}

hipError_t launch_gemv_argmax(const uint32_t* wq, const uint16_t* scales, const uint16_t* biases,
                              const uint16_t* x, float* y, uint2* rec, int B, int64_t N, int64_t K,
                              hipStream_t stream) {
  if (gemv_auto_family(N, K) == 2)
    return launch_gemv_mfma_argmax(wq, scales, biases, x, y, rec, B, N, K, stream);
  return dispatch<true>(wq, scales, biases, x, y, rec, B, N, K, false, stream);
}

// The family qmm_gemv runs: a function of the matrix width K and of the row
// count of the whole matrix only, never of the batch size or of the rows one
// call covers, so a row keeps its bits at every batch size and in every row
// slice (the pages key the K reduction on the whole matrix and ask that a
// request served beside others get the bits it gets alone).  Every (K, whole)
// takes the vector-ALU family: it is the faster one at B = 1 for every shape
// here (o_proj, gate-up, down and the vocabulary head), and the matrix-core
// family, faster from B = 3..7 depending on the shape, gives other bits.
int gemv_auto_family(int64_t whole, int64_t K) {
  (void)whole;
  (void)K;
  return 1;
}

}  // namespace w4g
