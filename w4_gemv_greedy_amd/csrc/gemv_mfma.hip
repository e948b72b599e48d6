// Decode product on the matrix cores for 1 <= B <= 8 activation rows.
//
// Same format and result as the vector-ALU decode kernel (4-bit affine,
// group 64: TensorFold PR #1437, Receipt; fp32 result: same PR, commit "Add
// the pair seam and register its kernels with the kernel contract"), for
// batches where the vector ALUs cannot keep up with HBM: a 16 x 16 x 32 bf16
// matrix-core instruction multiplies 32 K-elements of 16 weight rows by up to
// 16 activation rows, so every code is expanded once whatever B is.
//
// Two kernels with one arithmetic and one order, so the same bits: one that
// holds the activations of the batch whole in LDS (where eight rows of them
// fit) and one that stages them step by step (larger K).  Which one runs is a
// function of K alone, and neither's order depends on N, B, the grid or
// timing (TensorFold PR #1433, step-2 description: the K reduction of a row is
// its full matrix's, whatever slice of rows a call covers).
#include "w4g_internal.h"

namespace w4g {
namespace {

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

// 8 codes -> bf16 values 128 + q in the order q0,q4,q1,q5,q2,q6,q3,q7
__device__ __forceinline__ bf16x8_t expand128(uint32_t w, uint32_t m, uint32_t g) {
  uint4 p;
  p.x = and_or(w, m, g);
  p.y = and_or(w >> 4, m, g);
  p.z = and_or(w >> 8, m, g);
  p.w = and_or(w >> 12, m, g);
  return __builtin_bit_cast(bf16x8_t, p);
}

// ---- One workgroup per CU (the per-CU matrix-core layout) ----
//
// Workgroup b owns rows [b * rpw, (b + 1) * rpw) (rpw = ceil(N / 256)) as tiles
// of 16 rows, and stages the activations of its batch rows once, whole, in LDS
// (used where eight rows' activations fit, whatever B is).  Its W
// waves (W = min(8, NI), NI = ceil(G / 2) items of two consecutive groups
// (2i, 2i + 1)) split the items of every tile into contiguous ranges: wave w
// takes items [w NI / W, (w + 1) NI / W) of each tile in ascending order, the
// tiles one after the other, through a ring of P items in flight.  Where a CU
// has two tiles or more, two such sets of W waves run side by side, set s
// taking tiles s, s + 2, ... (four waves per SIMD instead of two, for latency
// hiding); a tile's items, their split and the order of its wave sums are the
// same whichever set runs it.
//
// v_mfma_f32_16x16x32_bf16: A = activations (batch row m = lane & 15, rows
// m >= B zero), B = codes of the tile's 16 rows expanded to 128 + q (row
// lane & 15); the K quarter q = lane >> 4 of an instruction is one code word.
// Lane l loads 16 bytes of row l / 4 (part p = l % 4: for p < 2 words 4p ..
// 4p + 3 of group 2i, for p >= 2 the same words of group 2i + 1), so four
// adjacent lanes read one row's 64 contiguous bytes and the L1 sees one access
// per row; a ds_bpermute moves them to lane (n = row, q = p) of the
// instruction's layout, and one v_permlane32_swap per word pair then gives
// every quarter two words of each group (quarter 0: words 0,1; 1: words 4,5;
// 2: words 2,3; 3: words 6,7), the first for the group's first instruction and
// the second for its second.  The activations are staged in that order.  The
// scale and bias pairs of a row come the same way: with an even group count
// once per four items, lane 4n + p loading row n's pairs of the p-th of them;
// with an odd one each lane loads those of the row it loads codes of, per item.
//
// Arithmetic per (row n, batch row b): for each group g the matrix core forms
// P_g = sum_{k in g} x*(128 + q) from zero over two instructions; the wave
// then adds s*P_g and (b_g - 128 s)*X_g in fp32 (X_g the fp32 sum of the
// group's activations: the sum of its two 32-element halves, each summed over
// its natural bf16 pairs in ascending order).
// Wave w's sum covers its range of groups in ascending order; the W wave sums
// are added in ascending wave order.  The order depends on K alone (W and the
// ranges are functions of K), and each batch row is its own.  Activation rows
// past the batch read row B - 1: they only reach result rows that are never
// read.
//
// Tiles run in batches of TB (as many as LDS holds partial sums for): each
// wave writes its partial sums of a tile to LDS when it finishes its share,
// and after the batch, at one barrier, the wave sums are added.  The results
// stay in LDS until the stream ends where they fit beside the rest (hold), so
// no global store sits among the code loads in flight (a store there makes
// the next waits for loads wait for it too); else each batch's are stored as
// it is reduced.  AM folds the results into the workgroup's argmax record per
// batch row instead of or beside the store.  The activations, their group
// sums and one tile's partial sums must fit: a function of K alone, so
// whether this kernel applies depends on K alone; where the results go does
// not change them.

constexpr int kCuRows = 16;      // rows per tile
constexpr int kCuMaxWaves = 8;   // waves per set (the order's wave split)
constexpr int kCuSets = 2;       // sets of waves per workgroup (whole-x kernel)

// LDS barrier for data exchanged through LDS only: the loads in flight are not
// waited for
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
}

template <bool EVENG>
struct CuItem {
  uint4 c;  // 16 bytes of codes, as loaded (see above)
  // EVENG: the scale pair and the bias pair (bf16 x 2) of the item's groups for
  // the row this lane loaded codes of; else this lane's row's one by one
  uint32_t s[EVENG ? 1 : 2], b[EVENG ? 1 : 2];
};

template <bool EVENG, bool AM, int P>
__global__ __launch_bounds__(64 * kCuMaxWaves * kCuSets) void gemv_mfma_cu_kernel(
    const uint32_t* __restrict__ wq, const uint16_t* __restrict__ scales, const uint16_t* __restrict__ biases,
    const uint16_t* __restrict__ x, float* __restrict__ y, int B, int64_t N, int64_t K, int64_t rpw,
    int TB, bool hold, uint2* __restrict__ rec, int S) {
  extern __shared__ uint4 s_mem[];
  __shared__ uint64_t s_best[AM ? 8 : 1];
  __shared__ uint32_t s_bad;
  const int tid = threadIdx.x, lane = tid & 63;
  // S sets of W waves; set s takes tiles s, s + S, ... (every set splits a
  // tile's items the same way, so which set runs a tile changes nothing)
  const int W = (int)(blockDim.x >> 6) / S;
  const int set = __builtin_amdgcn_readfirstlane((tid >> 6) / W);
  const int wave = __builtin_amdgcn_readfirstlane((tid >> 6) - set * W);
  const int n16 = lane & 15, q = lane >> 4;
  const int G = (int)(K >> 6), NI = (G + 1) >> 1;
  const int64_t KW = K >> 3;
  const int64_t r0 = (int64_t)blockIdx.x * rpw;
  const int64_t r1 = N - r0 < rpw ? N : r0 + rpw;
  const int nrows = (int)(r1 - r0);
  const int T = (nrows + kCuRows - 1) / kCuRows;
  // this wave's items of every tile: [ist, iend) (contiguous, >= 1 since W <= NI)
  const int ist = (int)((int64_t)wave * NI / W), iend = (int)((int64_t)(wave + 1) * NI / W);
  const int cnt = iend - ist;
  const int my_tiles = set < T ? (T - set + S - 1) / S : 0;
  const int n_items = my_tiles * cnt;

  const int XS = B > 4 ? 8 : 4;                                      // batch slots per group sum
  uint4* s_x = s_mem;                                                // [G][2][4][B]
  float* s_X = reinterpret_cast<float*>(s_mem + (int64_t)G * 8 * B);  // [G][XS]
  float* s_red = s_X + (int64_t)G * XS;                              // [TB][W][32][4]
  float* s_y = s_red + TB * W * 128;                                 // [B][rpw] when hold

  // Per-lane LDS offsets.  Lanes whose activation row m = n16 is past the batch
  // read row B - 1: they only feed result rows m >= B, which are never used.
  const int lane_a = q * B + (n16 < B ? n16 : B - 1);  // uint4, within a (group, half) block
  const int stride_g = 8 * B;                           // uint4 per group
  const int xq = XS == 8 ? 4 * (q & 1) : 0;             // first batch row of this lane's results

  // ---- item issue.  Codes: lane l reads 16 bytes of row l / 4 of the tile
  // (four adjacent lanes read one row's 64 bytes, so the L1 sees one access per
  // row, not one per lane); part p = l % 4 is words 4 (p % 2) .. + 3 of group
  // g0 + p / 2.  The consumer moves each lane's 16 bytes to lane
  // (row, quarter p), the matrix-core layout, through the LDS crossbar.
  const int pc = lane & 3;
  int it_t = set, it_i = ist;
  const uint32_t* cptr;
  const uint16_t *sptr = scales, *bptr = biases;
  auto set_tile = [&]() {
    const int64_t rt = r0 + (int64_t)it_t * kCuRows;
    int64_t rc = rt + (lane >> 2);
    rc = rc < r1 ? rc : r1 - 1;
    cptr = wq + rc * KW + (pc & 1) * 4 + (pc >> 1) * 8;
    if constexpr (!EVENG) {  // (EVENG: the pair loads below)
      int64_t rn = rt + n16;
      rn = rn < r1 ? rn : r1 - 1;
      sptr = scales + rn * G;
      bptr = biases + rn * G;
    }
  };
  set_tile();
  auto issue = [&](CuItem<EVENG>& it) {
    const int g0 = 2 * it_i;
    int off = g0 * 8;
    if (!EVENG && g0 + 1 >= G && pc >= 2) off -= 8;  // an odd last group: parts 2, 3 reread it (unused)
    it.c = *reinterpret_cast<const uint4*>(cptr + off);
    if constexpr (!EVENG) {
      const int g1 = g0 + 1 < G ? g0 + 1 : g0;
      it.s[0] = sptr[g0];
      it.s[1] = sptr[g1];
      it.b[0] = bptr[g0];
      it.b[1] = bptr[g1];
    }
    if (++it_i == iend) {
      it_i = ist;
      it_t += S;
      set_tile();
    }
  };
  // EVENG: the scale and bias pairs come once per P = 4 items: for the k-th
  // such load, lane 4n + p reads row n's pairs of item 4k + p of the wave's
  // sequence (one load per table per four items instead of one per item:
  // B = 8 gate-up 31 against 35 us, lm_head 172 against 188), each lane
  // following its own item through the tiles
  static_assert(!EVENG || P == 4, "one pair load per four items");
  int qt = set, qi = ist;  // this lane's item of the next pair load: tile, item within the tile
  auto q_adv = [&](int k) {
    qi += k;
    while (qi >= iend) {
      qi -= cnt;
      qt += S;
    }
  };
  if constexpr (EVENG) q_adv(pc);
  uint32_t sqa = 0, bqa = 0, sqb = 0, bqb = 0;  // pairs of the even / odd groups of four items
  auto issue_pairs = [&](uint32_t& sw, uint32_t& bw) {
    int64_t row = r0 + (int64_t)qt * kCuRows + (lane >> 2);
    row = row < r1 ? row : r1 - 1;  // past the last tile: a valid row, never used
    sw = *reinterpret_cast<const uint32_t*>(scales + row * G + 2 * qi);
    bw = *reinterpret_cast<const uint32_t*>(biases + row * G + 2 * qi);
    q_adv(P);
  };

  // ---- stage x: segment (b, g) = 64 activations -> 8 blocks in the quarter
  // order above, and the group sum X_g (two 32-element halves over natural pairs)
  const int nseg = B * G;
  auto load_seg = [&](int seg, uint4 (&v)[8]) {
    const int g = seg / B, bb = seg - g * B;  // batch row fastest: conflict-free LDS writes
    const uint4* src = reinterpret_cast<const uint4*>(x + (int64_t)bb * K + (int64_t)g * 64);
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = src[j];
  };
  auto put_seg = [&](int seg, const uint4 (&v)[8]) {
    const int g = seg / B, bb = seg - g * B;
    float h0 = 0.0f, h1 = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int qq = ((j >> 1) & 1) * 2 + (j >> 2), hh = j & 1;
      s_x[g * stride_g + hh * 4 * B + qq * B + bb] = permute_block(v[j]);
      float& h = j < 4 ? h0 : h1;
      h = dot2(v[j].x, kOnes, h);
      h = dot2(v[j].y, kOnes, h);
      h = dot2(v[j].z, kOnes, h);
      h = dot2(v[j].w, kOnes, h);
    }
    s_X[g * XS + bb] = h0 + h1;
  };
  uint4 pre[8];
  const bool has_pre = tid < nseg;
  if (has_pre) load_seg(tid, pre);

  CuItem<EVENG> ring[P];
#pragma unroll
  for (int sl = 0; sl < P; ++sl) issue(ring[sl]);
  if constexpr (EVENG) issue_pairs(sqa, bqa);

  if (has_pre) put_seg(tid, pre);
  for (int seg = tid + (int)blockDim.x; seg < nseg; seg += (int)blockDim.x) {
    uint4 v[8];
    load_seg(seg, v);
    put_seg(seg, v);
  }
  for (int i = tid; i < XS * G; i += (int)blockDim.x)  // the unused batch slots of the group sums
    if ((i & (XS - 1)) >= B) s_X[i] = 0.0f;
  if (AM && tid < 8) s_best[tid] = 0;
  if (AM && tid == 0) s_bad = 0;
  __syncthreads();

  // ---- stream, TB tiles at a time: each wave writes its partial sums of a
  // tile to LDS as it finishes its share (from a register that holds the
  // address, so nothing on that path waits for the loads in flight), and when
  // a batch of tiles is done the wave sums are added, at two barriers
  const uint32_t m = 0x000F000Fu, gm = kMagic128;
  f32x4_t tot = {0.0f, 0.0f, 0.0f, 0.0f};
  int ci = ist, tb0 = 0, ct = set;  // ct: the tile being consumed
  float* const red_base = s_red + (wave * 32 + lane) * 4;
  auto group = [&](int g, uint32_t w0, uint32_t w1, uint32_t sb, uint32_t bb) {
    const int ab = lane_a + g * stride_g;
    const bf16x8_t a0 = __builtin_bit_cast(bf16x8_t, s_x[ab]);
    const bf16x8_t a1 = __builtin_bit_cast(bf16x8_t, s_x[ab + 4 * B]);
    const float4 xs = *reinterpret_cast<const float4*>(s_X + g * XS + xq);
    f32x4_t pg = {0.0f, 0.0f, 0.0f, 0.0f};
    pg = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, expand128(w0, m, gm), pg, 0, 0, 0);
    pg = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, expand128(w1, m, gm), pg, 0, 0, 0);
    const float sc = bf16_to_f32(sb);
    const float cb = __builtin_fmaf(-128.0f, sc, bf16_to_f32(bb));
    tot[0] = __builtin_fmaf(cb, xs.x, __builtin_fmaf(sc, pg[0], tot[0]));
    tot[1] = __builtin_fmaf(cb, xs.y, __builtin_fmaf(sc, pg[1], tot[1]));
    tot[2] = __builtin_fmaf(cb, xs.z, __builtin_fmaf(sc, pg[2], tot[2]));
    tot[3] = __builtin_fmaf(cb, xs.w, __builtin_fmaf(sc, pg[3], tot[3]));
  };
  // the result of (batch row bq, workgroup row `row`): kept in LDS until the
  // stream ends (hold), else stored and with AM folded into the workgroup's
  // argmax record for bq at once
  auto put_result = [&](int bq, int row, float v) {
    if (hold) {
      s_y[bq * (int)rpw + row] = v;
      return;
    }
    if (!AM || y != nullptr) y[(int64_t)bq * N + r0 + row] = v;
    if constexpr (AM) {
      const uint32_t u = __float_as_uint(v);
      if (!finite_bits(u))
        __hip_atomic_fetch_or(&s_bad, 1u << bq, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      else
        __hip_atomic_fetch_max(&s_best[bq], cand(u, (uint32_t)(r0 + row)), __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_WORKGROUP);
    }
  };
  auto reduce_batch = [&]() {
    // add the wave sums of the batch's bt tiles in ascending wave order (rows
    // fastest across threads, so the stores of a batch row are contiguous)
    const int bt = T - tb0 < TB ? T - tb0 : TB;
    lds_barrier();
    const int nout = bt * kCuRows * B;
    for (int o = tid; o < nout; o += (int)blockDim.x) {
      const int tb = o / (kCuRows * B), rem = o - tb * (kCuRows * B);
      const int bq = rem / kCuRows, n = rem - bq * kCuRows;
      const int row = (tb0 + tb) * kCuRows + n;
      if (row < nrows) {
        const float* pr = s_red + (tb * W * 32 + n + 16 * (bq >> 2)) * 4 + (bq & 3);
        float acc = pr[0];
        for (int w = 1; w < W; ++w) acc += pr[w * 128];
        put_result(bq, row, acc);
      }
    }
    lds_barrier();
  };
  const int src_lane = ((n16 << 2) | q) << 2;  // byte address of lane 4 n + q
  auto consume = [&](const CuItem<EVENG>& it, int sl, uint32_t sq, uint32_t bq) {
    // lane (n, q) takes the 16 bytes lane 4 n + q loaded
    const uint32_t c0 = (uint32_t)__builtin_amdgcn_ds_bpermute(src_lane, (int)it.c.x);
    const uint32_t c1 = (uint32_t)__builtin_amdgcn_ds_bpermute(src_lane, (int)it.c.y);
    const uint32_t c2 = (uint32_t)__builtin_amdgcn_ds_bpermute(src_lane, (int)it.c.z);
    const uint32_t c3 = (uint32_t)__builtin_amdgcn_ds_bpermute(src_lane, (int)it.c.w);
    // quarters 0,1 hold group 2i's words, 2,3 group 2i + 1's: swap word pairs across
    const auto sx = __builtin_amdgcn_permlane32_swap(c0, c2, false, false);
    const auto sy = __builtin_amdgcn_permlane32_swap(c1, c3, false, false);
    const int g0 = 2 * ci;
    if constexpr (EVENG) {
      // the scale and bias pairs of row n for this item (slot sl of four):
      // lane 4n + sl loaded them
      const int src_q = ((n16 << 2) | sl) << 2;
      const uint32_t sp = (uint32_t)__builtin_amdgcn_ds_bpermute(src_q, (int)sq);
      const uint32_t bp = (uint32_t)__builtin_amdgcn_ds_bpermute(src_q, (int)bq);
      group(g0, sx[0], sy[0], sp & 0xFFFFu, bp & 0xFFFFu);
      group(g0 + 1, sx[1], sy[1], sp >> 16, bp >> 16);
    } else {
      group(g0, sx[0], sy[0], it.s[0], it.b[0]);
      if (g0 + 1 < G) group(g0 + 1, sx[1], sy[1], it.s[1], it.b[1]);
    }
    if (++ci == iend) {  // this wave's share of a tile is done: its partial sums to LDS
      ci = ist;
      if (lane < 32) *reinterpret_cast<f32x4_t*>(red_base + (ct - tb0) * W * 32 * 4) = tot;
      tot = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
      ct += S;
      // every batch whose tiles of this set are all done is reduced (all sets
      // take part in every batch's reduction, in batch order)
      while (tb0 < T && (ct >= tb0 + TB || ct >= T)) {
        reduce_batch();
        tb0 += TB;
      }
    }
  };
  // steady state (every issued item exists), two groups of P items per
  // iteration so the pairs of the even and odd groups keep registers of their
  // own (with EVENG the next group's pairs are loaded beside the first of its
  // codes), then the last items (fewer than 3P)
  int j = 0;
  for (; j + 3 * P - 1 < n_items; j += 2 * P) {
#pragma unroll
    for (int sl = 0; sl < P; ++sl) {
      consume(ring[sl], sl, sqa, bqa);
      issue(ring[sl]);
      if (EVENG && sl == 0) issue_pairs(sqb, bqb);
    }
#pragma unroll
    for (int sl = 0; sl < P; ++sl) {
      consume(ring[sl], sl, sqb, bqb);
      issue(ring[sl]);
      if (EVENG && sl == 0) issue_pairs(sqa, bqa);
    }
  }
#pragma unroll
  for (int sl = 0; sl < P; ++sl) {
    if (j + sl < n_items) consume(ring[sl], sl, sqa, bqa);
    if (j + sl + P < n_items) {
      issue(ring[sl]);
      if (EVENG && sl == 0) issue_pairs(sqb, bqb);
    }
  }
#pragma unroll
  for (int sl = 0; sl < P; ++sl) {
    if (j + P + sl < n_items) consume(ring[sl], sl, sqb, bqb);
    if (j + 2 * P + sl < n_items) {
      issue(ring[sl]);
      if (EVENG && sl == 0) issue_pairs(sqa, bqa);
    }
  }
#pragma unroll
  for (int sl = 0; sl < P; ++sl)
    if (j + 2 * P + sl < n_items) consume(ring[sl], sl, sqa, bqa);

  // a set without tiles in the last batches still takes part in their reductions
  while (tb0 < T) {
    reduce_batch();
    tb0 += TB;
  }

  // ---- held results out (the last reduction ended with a barrier), then the record
  if (hold) {
    const int nout = B * nrows;
    for (int o = tid; o < nout; o += (int)blockDim.x) {
      const int bq = o / nrows, row = o - bq * nrows;
      const float v = s_y[bq * (int)rpw + row];
      if (!AM || y != nullptr) y[(int64_t)bq * N + r0 + row] = v;
      if constexpr (AM) {
        const uint32_t u = __float_as_uint(v);
        if (!finite_bits(u))
          __hip_atomic_fetch_or(&s_bad, 1u << bq, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        else
          __hip_atomic_fetch_max(&s_best[bq], cand(u, (uint32_t)(r0 + row)), __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_WORKGROUP);
      }
    }
    if constexpr (AM) __syncthreads();
  }
  if constexpr (AM) {
    if (tid < B)
      rec[(int64_t)tid * gridDim.x + blockIdx.x] = make_record(s_best[tid], ((s_bad >> tid) & 1u) != 0, (uint32_t)r0);
  }
}

// ---- The per-CU layout where x does not fit in LDS (the down projection) ----
//
// Same rows, tiles, waves, items and arithmetic as gemv_mfma_cu_kernel (so the
// same bits), with the activations staged step by step instead of whole: the
// workgroup takes its tiles TT at a time (one or two), and for each such pair
// the waves advance through their item ranges in lockstep, one item per tile
// per step, step s's activations (each wave's two groups, all batch rows)
// sitting in one of two LDS buffers.  Threads load the activations of step
// s + SPB as the step starts (SPB steps ahead, as the codes are) and store
// them into the free buffer when the next step's turn comes, then all meet at
// one barrier per step.  Each wave keeps one running sum per tile; the wave
// sums of a pair are added when its steps are done.  A CU with more than two
// tiles runs the pairs one after the other, staging the activations again for
// each (they come from L2).
template <bool EVENG, bool AM, int TT>
__global__ __launch_bounds__(64 * kCuMaxWaves) void gemv_mfma_cuk_kernel(
    const uint32_t* __restrict__ wq, const uint16_t* __restrict__ scales, const uint16_t* __restrict__ biases,
    const uint16_t* __restrict__ x, float* __restrict__ y, int B, int64_t N, int64_t K, int64_t rpw,
    uint2* __restrict__ rec) {
  static_assert(TT == 1 || TT == 2, "one or two tiles at a time (activations loaded two or more steps ahead)");
  constexpr int SPB = 4 / TT;  // steps per unrolled body (code items in flight: P = TT * SPB = 4)
  constexpr int P = TT * SPB;
  extern __shared__ uint4 s_mem[];
  __shared__ uint64_t s_best[AM ? 8 : 1];
  __shared__ uint32_t s_bad;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int W = (int)(blockDim.x >> 6);
  const int n16 = lane & 15, q = lane >> 4;
  const int G = (int)(K >> 6), NI = (G + 1) >> 1;
  const int64_t KW = K >> 3;
  const int64_t r0 = (int64_t)blockIdx.x * rpw;
  const int64_t r1 = N - r0 < rpw ? N : r0 + rpw;
  const int nrows = (int)(r1 - r0);
  const int ist = (int)((int64_t)wave * NI / W), iend = (int)((int64_t)(wave + 1) * NI / W);
  const int cnt = iend - ist;
  const int S = (NI + W - 1) / W;  // steps: the most items any wave has per tile
  const int T = (nrows + kCuRows - 1) / kCuRows;  // tiles of this workgroup

  const int XS = B > 4 ? 8 : 4;
  uint4* s_xs = s_mem;                                                     // [2][W][2][2][4][B]
  float* s_Xs = reinterpret_cast<float*>(s_mem + 2 * W * 16 * B);          // [2][W][2][XS]
  float* s_red = s_Xs + 2 * W * 2 * XS;                                    // [TT][W][32][4]
  const int stride_buf = W * 16 * B;  // uint4 per buffer

  // ---- codes: as in gemv_mfma_cu_kernel; tile t of the current pair is
  // workgroup tile tp + t (a tile past the last reads the last row, and its
  // results are not kept)
  const int pc = lane & 3;
  const uint32_t* cptr[TT];
  const uint16_t* sptr[TT];
  const uint16_t* bptr[TT];
  auto set_tiles = [&](int tp) {
#pragma unroll
    for (int t = 0; t < TT; ++t) {
      const int64_t rt = r0 + (int64_t)(tp + t) * kCuRows;
      int64_t rc = rt + (lane >> 2);
      rc = rc < r1 ? rc : r1 - 1;
      cptr[t] = wq + rc * KW + (pc & 1) * 4 + (pc >> 1) * 8;
      if constexpr (EVENG) {
        sptr[t] = scales + rc * G;
        bptr[t] = biases + rc * G;
      } else {
        int64_t rn = rt + n16;
        rn = rn < r1 ? rn : r1 - 1;
        sptr[t] = scales + rn * G;
        bptr[t] = biases + rn * G;
      }
    }
  };
  // item (step s, tile t): item index ist + s, clamped to the wave's last (loads
  // stay unconditional so the waits count exactly; a clamped item is not consumed)
  auto issue = [&](CuItem<EVENG>& it, int s, int t) {
    const int i = ist + (s < cnt ? s : cnt - 1);
    const int g0 = 2 * i;
    int off = g0 * 8;
    if (!EVENG && g0 + 1 >= G && pc >= 2) off -= 8;
    it.c = *reinterpret_cast<const uint4*>(cptr[t] + off);
    if constexpr (!EVENG) {
      const int g1 = g0 + 1 < G ? g0 + 1 : g0;
      it.s[0] = sptr[t][g0];
      it.s[1] = sptr[t][g1];
      it.b[0] = bptr[t][g0];
      it.b[1] = bptr[t][g1];
    }
  };
  // EVENG: a tile's scale and bias pairs come once per four steps (a group),
  // a group ahead: lane 4n + p reads row n's pairs of step 4k + p (clamped to
  // the wave's last item, as the codes are); even and odd groups keep
  // registers of their own
  uint32_t psq[2][TT], pbq[2][TT];
  auto issue_pairs = [&](int k, int set) {
    int st = 4 * k + pc;
    st = st < cnt ? st : cnt - 1;
    const int g0 = 2 * (ist + st);
#pragma unroll
    for (int t = 0; t < TT; ++t) {
      psq[set][t] = *reinterpret_cast<const uint32_t*>(sptr[t] + g0);
      pbq[set][t] = *reinterpret_cast<const uint32_t*>(bptr[t] + g0);
    }
  };

  // ---- activations of a step: half-segment h = (wave w, group gg, row bb,
  // half) of 32 elements per staging thread (the two halves of a group in
  // adjacent lanes, whose sums meet over a lane swap)
  const int H = W * 2 * B * 2;
  const int xhalf = tid & 1, xrest = tid >> 1;
  const int xbb = xrest % B, xgg = (xrest / B) & 1, xw = xrest / (2 * B);
  const int xist = (int)((int64_t)xw * NI / W), xcnt = (int)((int64_t)(xw + 1) * NI / W) - xist;
  auto x_load = [&](int s, uint4 (&v)[4]) {
    const int g = 2 * (xist + s) + xgg;
    const bool ok = tid < H && s < xcnt && g < G;
    const uint4* src = reinterpret_cast<const uint4*>(x + (ok ? (int64_t)xbb * K + (int64_t)g * 64 + xhalf * 32 : 0));
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = ok ? src[i] : make_uint4(0u, 0u, 0u, 0u);
  };
  auto x_store = [&](const uint4 (&v)[4], int buf) {
    float h = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      h = dot2(v[i].x, kOnes, h);
      h = dot2(v[i].y, kOnes, h);
      h = dot2(v[i].z, kOnes, h);
      h = dot2(v[i].w, kOnes, h);
    }
    const float other = __shfl_xor(h, 1);
    if (tid < H) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int j = xhalf * 4 + i;  // block of the group
        const int qq = ((j >> 1) & 1) * 2 + (j >> 2), hh = j & 1;
        s_xs[buf * stride_buf + (((xw * 2 + xgg) * 2 + hh) * 4 + qq) * B + xbb] = permute_block(v[i]);
      }
      if (xhalf == 0) s_Xs[((buf * W + xw) * 2 + xgg) * XS + xbb] = h + other;  // first half + second
    }
  };

  // ---- per-lane LDS offsets (as in gemv_mfma_cu_kernel)
  const int lane_a = q * B + (n16 < B ? n16 : B - 1);
  const int xq = XS == 8 ? 4 * (q & 1) : 0;
  const int src_lane = ((n16 << 2) | q) << 2;
  const uint32_t m = 0x000F000Fu, gm = kMagic128;
  f32x4_t tot[TT];
#pragma unroll
  for (int t = 0; t < TT; ++t) tot[t] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  auto group = [&](f32x4_t& acc, int buf, int gg, int g, uint32_t w0, uint32_t w1, uint32_t sb, uint32_t bb) {
    const int ab = buf * stride_buf + ((wave * 2 + gg) * 2) * 4 * B + lane_a;
    const bf16x8_t a0 = __builtin_bit_cast(bf16x8_t, s_xs[ab]);
    const bf16x8_t a1 = __builtin_bit_cast(bf16x8_t, s_xs[ab + 4 * B]);
    const float4 xs = *reinterpret_cast<const float4*>(s_Xs + ((buf * W + wave) * 2 + gg) * XS + xq);
    f32x4_t pg = {0.0f, 0.0f, 0.0f, 0.0f};
    pg = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, expand128(w0, m, gm), pg, 0, 0, 0);
    pg = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, expand128(w1, m, gm), pg, 0, 0, 0);
    const float sc = bf16_to_f32(sb);
    const float cb = __builtin_fmaf(-128.0f, sc, bf16_to_f32(bb));
    acc[0] = __builtin_fmaf(cb, xs.x, __builtin_fmaf(sc, pg[0], acc[0]));
    acc[1] = __builtin_fmaf(cb, xs.y, __builtin_fmaf(sc, pg[1], acc[1]));
    acc[2] = __builtin_fmaf(cb, xs.z, __builtin_fmaf(sc, pg[2], acc[2]));
    acc[3] = __builtin_fmaf(cb, xs.w, __builtin_fmaf(sc, pg[3], acc[3]));
    (void)g;
  };
  auto consume = [&](const CuItem<EVENG>& it, f32x4_t& acc, int s, int buf, uint32_t sq, uint32_t bq) {
    const uint32_t c0 = (uint32_t)__builtin_amdgcn_ds_bpermute(src_lane, (int)it.c.x);
    const uint32_t c1 = (uint32_t)__builtin_amdgcn_ds_bpermute(src_lane, (int)it.c.y);
    const uint32_t c2 = (uint32_t)__builtin_amdgcn_ds_bpermute(src_lane, (int)it.c.z);
    const uint32_t c3 = (uint32_t)__builtin_amdgcn_ds_bpermute(src_lane, (int)it.c.w);
    const auto sx = __builtin_amdgcn_permlane32_swap(c0, c2, false, false);
    const auto sy = __builtin_amdgcn_permlane32_swap(c1, c3, false, false);
    const int g0 = 2 * (ist + s);
    if constexpr (EVENG) {
      // this step's pairs of row n: lane 4n + (s % 4) loaded them
      const int src_q = ((n16 << 2) | (s & 3)) << 2;
      const uint32_t sp = (uint32_t)__builtin_amdgcn_ds_bpermute(src_q, (int)sq);
      const uint32_t bp = (uint32_t)__builtin_amdgcn_ds_bpermute(src_q, (int)bq);
      group(acc, buf, 0, g0, sx[0], sy[0], sp & 0xFFFFu, bp & 0xFFFFu);
      group(acc, buf, 1, g0 + 1, sx[1], sy[1], sp >> 16, bp >> 16);
    } else {
      group(acc, buf, 0, g0, sx[0], sy[0], it.s[0], it.b[0]);
      if (g0 + 1 < G) group(acc, buf, 1, g0 + 1, sx[1], sy[1], it.s[1], it.b[1]);
    }
  };

  if (AM && tid < 8) s_best[tid] = 0;
  if (AM && tid == 0) s_bad = 0;
  for (int tp = 0; tp < T; tp += TT) {
    set_tiles(tp);
#pragma unroll
    for (int t = 0; t < TT; ++t) tot[t] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};

    // ---- prologue: the first SPB steps' activations, the first P code items
    // (the barrier also ends the previous pair's reads of the partial sums)
    uint4 xr[SPB][4];
#pragma unroll
    for (int u = 0; u < SPB; ++u) x_load(u, xr[u]);
    CuItem<EVENG> ring[P];
#pragma unroll
    for (int u = 0; u < SPB; ++u)
#pragma unroll
      for (int t = 0; t < TT; ++t) issue(ring[u * TT + t], u, t);
    if constexpr (EVENG) issue_pairs(0, 0);
    x_store(xr[0], 0);
    __syncthreads();

    // ---- steps, eight per unrolled body (two groups of four, so every ring
    // slot, activation register and pair set is a constant): step s consumes
    // buffer s % 2; the activations of step s + 1 (loaded SPB - 1 steps
    // earlier) go into the other buffer before the step's barrier, and those
    // of step s + SPB are loaded; with EVENG the first step of a group loads
    // the next group's pairs
    for (int s0 = 0; s0 < S; s0 += 8) {
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int s = s0 + u;
        const int ur = u % SPB, set = (u >> 2) & 1;
        if (s < S) {
          const int buf = s & 1;
          if (EVENG && (u & 3) == 0) issue_pairs((s >> 2) + 1, set ^ 1);
          if (s < cnt) {
#pragma unroll
            for (int t = 0; t < TT; ++t) {
              consume(ring[ur * TT + t], tot[t], s, buf, psq[set][t], pbq[set][t]);
              issue(ring[ur * TT + t], s + SPB, t);
            }
          } else {
#pragma unroll
            for (int t = 0; t < TT; ++t) issue(ring[ur * TT + t], s + SPB, t);
          }
          if (s + 1 < S) x_store(xr[(ur + 1) % SPB], buf ^ 1);
          x_load(s + SPB, xr[ur]);
          lds_barrier();
        }
      }
    }

    // ---- the pair's wave sums, in ascending wave order, stored (rows fastest
    // across threads) and with AM folded into the workgroup's record
    if (lane < 32) {
#pragma unroll
      for (int t = 0; t < TT; ++t) *reinterpret_cast<f32x4_t*>(s_red + ((t * W + wave) * 32 + lane) * 4) = tot[t];
    }
    __syncthreads();
    for (int o = tid; o < TT * kCuRows * B; o += (int)blockDim.x) {
      const int tb = o / (kCuRows * B), rem = o - tb * (kCuRows * B);
      const int bq = rem / kCuRows, n = rem - bq * kCuRows;
      const int row = (tp + tb) * kCuRows + n;
      if (row < nrows) {
        const float* pr = s_red + (tb * W * 32 + n + 16 * (bq >> 2)) * 4 + (bq & 3);
        float acc = pr[0];
        for (int w = 1; w < W; ++w) acc += pr[w * 128];
        if (!AM || y != nullptr) y[(int64_t)bq * N + r0 + row] = acc;
        if constexpr (AM) {
          const uint32_t uv = __float_as_uint(acc);
          if (!finite_bits(uv))
            __hip_atomic_fetch_or(&s_bad, 1u << bq, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
          else
            __hip_atomic_fetch_max(&s_best[bq], cand(uv, (uint32_t)(r0 + row)), __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_WORKGROUP);
        }
      }
    }
  }
  if constexpr (AM) {
    __syncthreads();
    if (tid < B)
      rec[(int64_t)tid * gridDim.x + blockIdx.x] = make_record(s_best[tid], ((s_bad >> tid) & 1u) != 0, (uint32_t)r0);
  }
}

constexpr int kMaxBatch = 8;               // decode batch rows at most
constexpr size_t kCuMaxLds = 152 * 1024;   // dynamic LDS asked for (of 160 KiB per CU)

// rows per workgroup of the one-workgroup-per-CU layout on this device
int64_t cu_rows(int64_t N, int cus) { return (N + cus - 1) / cus; }
int64_t cu_rows(int64_t N) { return cu_rows(N, cu_count()); }
int cu_waves(int64_t K) {
  const int64_t NI = ((K >> 6) + 1) >> 1;
  return NI < kCuMaxWaves ? (int)NI : kCuMaxWaves;
}
int cu_tiles(int64_t N) { return (int)((cu_rows(N) + kCuRows - 1) / kCuRows); }
// two sets of waves where a CU has two tiles or more (and a batch of
// reductions holds two), else one
int cu_sets(int64_t N, int64_t K);
// LDS of the whole-x kernel: the activations and group sums of Bc batch rows,
// then the partial sums of a batch of tiles
size_t cu_lds_fixed(int Bc, int64_t K) {
  const int64_t G = K >> 6;
  return (size_t)(G * 8 * Bc) * 16 + (size_t)G * (Bc > 4 ? 8 : 4) * 4;
}
size_t cu_tile_bytes(int64_t K) { return (size_t)cu_waves(K) * 32 * 4 * 4; }
// The whole-x kernel runs where the activations of the largest batch (8 rows)
// and one tile's partial sums fit in its LDS (K up to about 9,000), so one
// choice serves any B; the step-staged kernel otherwise.  A function of K
// alone; both kernels give the same bits in any case.
bool use_cu(int64_t K) { return cu_lds_fixed(kMaxBatch, K) + cu_tile_bytes(K) <= kCuMaxLds; }
// whether the whole-x kernel holds its results in LDS until the end: where
// they fit beside one tile's partial sums
size_t cu_held_bytes(int Bc, int64_t N) { return (size_t)Bc * cu_rows(N) * 4; }
bool cu_hold(int Bc, int64_t N, int64_t K) {
  return cu_lds_fixed(Bc, K) + cu_held_bytes(Bc, N) + cu_tile_bytes(K) <= kCuMaxLds;
}
// tiles per reduction batch of the whole-x kernel: as many as the LDS left
// holds partial sums for (at least one where use_cu holds)
int cu_batch_tiles(int Bc, int64_t N, int64_t K) {
  const size_t fixed = cu_lds_fixed(Bc, K) + (cu_hold(Bc, N, K) ? cu_held_bytes(Bc, N) : 0);
  const int64_t t = (int64_t)((kCuMaxLds - fixed) / cu_tile_bytes(K));
  return t < cu_tiles(N) ? (int)t : cu_tiles(N);
}
int cu_sets(int64_t N, int64_t K) {
  return cu_tiles(N) >= 2 && cu_batch_tiles(kMaxBatch, N, K) >= 2 ? kCuSets : 1;
}
size_t cu_lds_bytes(int Bc, int64_t N, int64_t K) {
  return cu_lds_fixed(Bc, K) + (cu_hold(Bc, N, K) ? cu_held_bytes(Bc, N) : 0) +
         (size_t)cu_batch_tiles(Bc, N, K) * cu_tile_bytes(K);
}
// the step-staged kernel takes a CU's tiles two at a time (one where it has one)
int cuk_pair(int64_t N) { return cu_tiles(N) == 1 ? 1 : 2; }
size_t cuk_lds_bytes(int B, int64_t N, int64_t K) {
  const int W = cu_waves(K), XS = B > 4 ? 8 : 4;
  return (size_t)2 * W * 16 * B * 16 + (size_t)2 * W * 2 * XS * 4 + (size_t)cuk_pair(N) * W * 128 * 4;
}

template <bool EVENG, bool AM>
hipError_t launch_cuk(const uint32_t* wq, const uint16_t* scales, const uint16_t* biases,
                      const uint16_t* x, float* y, uint2* rec, int B, int64_t N, int64_t K,
                      hipStream_t stream) {
  const int64_t rpw = cu_rows(N);
  const int64_t blocks = (N + rpw - 1) / rpw;
  const size_t lds = cuk_lds_bytes(B, N, K);
  if (cuk_pair(N) == 1) {
    hipLaunchKernelGGL((gemv_mfma_cuk_kernel<EVENG, AM, 1>), dim3((unsigned)blocks), dim3(64 * cu_waves(K)), lds,
                       stream, wq, scales, biases, x, y, B, N, K, rpw, rec);
  } else {
    hipLaunchKernelGGL((gemv_mfma_cuk_kernel<EVENG, AM, 2>), dim3((unsigned)blocks), dim3(64 * cu_waves(K)), lds,
                       stream, wq, scales, biases, x, y, B, N, K, rpw, rec);
  }
  return hipGetLastError();
}

template <bool EVENG, bool AM>
hipError_t launch_cu_pass(const uint32_t* wq, const uint16_t* scales, const uint16_t* biases,
                          const uint16_t* x, float* y, uint2* rec, int B, int64_t N, int64_t K,
                          hipStream_t stream) {
  const int64_t rpw = cu_rows(N);
  const int64_t blocks = (N + rpw - 1) / rpw;
  const size_t lds = cu_lds_bytes(B, N, K);
  const void* fn = reinterpret_cast<const void*>(&gemv_mfma_cu_kernel<EVENG, AM, 4>);
  if (lds > 64 * 1024) {
    // a host-side attribute of the kernel (not a stream operation)
    const hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)kCuMaxLds);
    if (e != hipSuccess) return e;
  }
  const int sets = cu_sets(N, K);
  hipLaunchKernelGGL((gemv_mfma_cu_kernel<EVENG, AM, 4>), dim3((unsigned)blocks), dim3(64 * cu_waves(K) * sets),
                     lds, stream, wq, scales, biases, x, y, B, N, K, rpw, cu_batch_tiles(B, N, K), cu_hold(B, N, K),
                     rec, sets);
  return hipGetLastError();
}

// step: the step-staged kernel whatever K is (it needs two groups or more;
// below that the whole-x kernel runs, with the same bits)
template <bool AM>
hipError_t launch(const uint32_t* wq, const uint16_t* scales, const uint16_t* biases,
                  const uint16_t* x, float* y, uint2* rec, int B, int64_t N, int64_t K, bool step,
                  hipStream_t stream) {
  const bool eveng = ((K >> 6) % 2) == 0 && ((reinterpret_cast<uintptr_t>(scales) |
                                               reinterpret_cast<uintptr_t>(biases)) & 3u) == 0;
  if (use_cu(K) && !(step && (K >> 6) >= 2))
    return eveng ? launch_cu_pass<true, AM>(wq, scales, biases, x, y, rec, B, N, K, stream)
                 : launch_cu_pass<false, AM>(wq, scales, biases, x, y, rec, B, N, K, stream);
  return eveng ? launch_cuk<true, AM>(wq, scales, biases, x, y, rec, B, N, K, stream)
               : launch_cuk<false, AM>(wq, scales, biases, x, y, rec, B, N, K, stream);
}

}  // namespace

hipError_t launch_gemv_mfma(const uint32_t* wq, const uint16_t* scales, const uint16_t* biases,
                            const uint16_t* x, float* y, int B, int64_t N, int64_t K, bool step,
                            hipStream_t stream) {
  return launch<false>(wq, scales, biases, x, y, nullptr, B, N, K, step, stream);
}

int64_t gemv_mfma_argmax_records(int B, int64_t N, int64_t K, int cus) {
  (void)B;
  (void)K;
  return (N + cu_rows(N, cus) - 1) / cu_rows(N, cus);
}

hipError_t launch_gemv_mfma_argmax(const uint32_t* wq, const uint16_t* scales, const uint16_t* biases,
                                   const uint16_t* x, float* y, uint2* rec, int B, int64_t N, int64_t K,
                                   hipStream_t stream) {
  return launch<true>(wq, scales, biases, x, y, rec, B, N, K, false, stream);
}

}  // namespace w4g
