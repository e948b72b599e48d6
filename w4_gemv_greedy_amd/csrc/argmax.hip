// Greedy vocabulary argmax in two passes.
//
// Rules (TensorFold PR #1433, step-1 description): a row holding any NaN,
// +Inf or -Inf fails; pass 1 reports such a block with bit 31 set in its id
// word (and NaN in its value word), and pass 2 turns any flag in the row into
// the sentinel 0xFFFFFFFF.  Otherwise the largest value wins and equal values
// go to the lowest id (a pick that ties to the higher id is one of the planted
// failures there).  The session reads the sentinel as a failure, never as a
// logit (step-2 description).
//
// Comparison: the ordering helpers of w4g_internal.h (an unsigned key per
// value, -0.0 and +0.0 equal, and a 64-bit candidate word whose maximum is the
// largest value with the lowest id).
#include "w4g_internal.h"

namespace w4g {
namespace {

constexpr int kThreads = 256;
constexpr uint32_t kFlag = kArgmaxFlag;

// Block-wide reduction of (best, bad) over NT threads; returns the result in
// every thread.
template <int NT = kThreads>
__device__ __forceinline__ void block_reduce(uint64_t& best, bool& bad) {
  __shared__ uint64_t s_best[NT / 64];
  __shared__ int s_bad[NT / 64];
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    uint32_t lo = (uint32_t)best, hi = (uint32_t)(best >> 32);
    lo = __shfl_xor(lo, off);
    hi = __shfl_xor(hi, off);
    best = umax64(best, ((uint64_t)hi << 32) | lo);
  }
  const bool any_bad = __any(bad);
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    s_best[wave] = best;
    s_bad[wave] = any_bad ? 1 : 0;
  }
  __syncthreads();
  best = s_best[0];
  int b = s_bad[0];
#pragma unroll
  for (int w = 1; w < NT / 64; ++w) {
    best = umax64(best, s_best[w]);
    b |= s_bad[w];
  }
  bad = b != 0;
}

// Widened element bits: fp32 as is, bf16 shifted into the top half (exact).
template <int DT>
__device__ __forceinline__ uint32_t elem_bits(const void* p, int64_t i) {
  if (DT == 0) return reinterpret_cast<const uint32_t*>(p)[i];
  return ((uint32_t)reinterpret_cast<const uint16_t*>(p)[i]) << 16;
}

template <int DT>
__global__ __launch_bounds__(kThreads) void argmax_pass1(const void* __restrict__ logits,
                                                         int64_t ld, int64_t vocab, int nblk,
                                                         uint2* __restrict__ rec) {
  const int64_t row = blockIdx.y;
  const int64_t blk = blockIdx.x;
  const int64_t i0 = blk * kArgmaxBlock + (int64_t)threadIdx.x * 4;
  const int64_t base = row * ld;
  uint32_t u[4];
  const bool vec = ((ld & 3) == 0) && (i0 + 3 < vocab);
  if (vec) {
    if (DT == 0) {
      const uint4 v = *reinterpret_cast<const uint4*>(
          reinterpret_cast<const uint32_t*>(logits) + base + i0);
      u[0] = v.x; u[1] = v.y; u[2] = v.z; u[3] = v.w;
    } else {
      const uint2 v = *reinterpret_cast<const uint2*>(
          reinterpret_cast<const uint16_t*>(logits) + base + i0);
      u[0] = v.x << 16; u[1] = v.x & 0xFFFF0000u; u[2] = v.y << 16; u[3] = v.y & 0xFFFF0000u;
    }
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) u[j] = (i0 + j < vocab) ? elem_bits<DT>(logits, base + i0 + j) : 0u;
  }
  uint64_t best = 0;  // below every finite candidate
  bool bad = false;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if (i0 + j < vocab) {
      if (!finite_bits(u[j])) bad = true;
      else best = umax64(best, cand(u[j], (uint32_t)(i0 + j)));
    }
  }
  block_reduce(best, bad);
  if (threadIdx.x == 0) rec[row * nblk + blk] = make_record(best, bad, (uint32_t)(blk * kArgmaxBlock));
}

// One workgroup of NT threads per row; each thread folds its records with U
// loads in flight at a time (all of a row's records in one round when there
// are at most NT * U of them).
template <int NT, int U>
__global__ __launch_bounds__(NT) void argmax_pass2(const uint2* __restrict__ rec, int64_t nblk,
                                                   uint32_t* __restrict__ ids) {
  const int64_t row = blockIdx.x;
  const uint2* r0 = rec + row * nblk;
  uint64_t best = 0;
  bool bad = false;
  for (int64_t i0 = threadIdx.x; i0 < nblk; i0 += (int64_t)NT * U) {
    uint2 r[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t i = i0 + (int64_t)u * NT;
      r[u] = i < nblk ? r0[i] : make_uint2(0u, 0u);  // (+0.0, id 0): below any real candidate's id
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (i0 + (int64_t)u * NT >= nblk) continue;
      if (r[u].y & kFlag) bad = true;
      else best = umax64(best, cand(r[u].x, r[u].y));
    }
  }
  block_reduce<NT>(best, bad);
  if (threadIdx.x == 0) ids[row] = bad ? 0xFFFFFFFFu : 0xFFFFFFFFu - (uint32_t)best;
}

// ---- top two.  A pair (a, b) holds the two largest candidate words seen, a > b
// (0 = none; candidates of distinct ids never tie).  A row's non-finite value
// sets its pass-1 record's a to ~0, which no finite candidate reaches.

__device__ __forceinline__ void top2_push(uint64_t& a, uint64_t& b, uint64_t c) {
  if (c > a) {
    b = a;
    a = c;
  } else if (c > b) {
    b = c;
  }
}
// (a, b) <- the top two of {a, b, c, d}, given a >= b and c >= d
__device__ __forceinline__ void top2_merge(uint64_t& a, uint64_t& b, uint64_t c, uint64_t d) {
  const uint64_t lo = a > c ? c : a;
  a = umax64(a, c);
  b = umax64(lo, umax64(b, d));
}
__device__ __forceinline__ uint64_t shfl_xor64(uint64_t v, int off) {
  const uint32_t lo = __shfl_xor((uint32_t)v, off), hi = __shfl_xor((uint32_t)(v >> 32), off);
  return ((uint64_t)hi << 32) | lo;
}
// Block-wide top two of (a, b) and the non-finite flag; the result in every thread.
__device__ __forceinline__ void block_top2(uint64_t& a, uint64_t& b, bool& bad) {
  __shared__ uint64_t s_a[kThreads / 64], s_b[kThreads / 64];
  __shared__ int s_bad[kThreads / 64];
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const uint64_t c = shfl_xor64(a, off), d = shfl_xor64(b, off);
    top2_merge(a, b, c, d);
  }
  const bool any_bad = __any(bad);
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    s_a[wave] = a;
    s_b[wave] = b;
    s_bad[wave] = any_bad ? 1 : 0;
  }
  __syncthreads();
  a = s_a[0];
  b = s_b[0];
  int f = s_bad[0];
#pragma unroll
  for (int w = 1; w < kThreads / 64; ++w) {
    top2_merge(a, b, s_a[w], s_b[w]);
    f |= s_bad[w];
  }
  bad = f != 0;
}

// pass 1: one block of 1024 ids per workgroup -> record (a, b) as four words
template <int DT>
__global__ __launch_bounds__(kThreads) void top2_pass1(const void* __restrict__ logits, int64_t ld,
                                                       int64_t vocab, int nblk,
                                                       uint4* __restrict__ rec) {
  const int64_t row = blockIdx.y;
  const int64_t blk = blockIdx.x;
  const int64_t i0 = blk * kArgmaxBlock + (int64_t)threadIdx.x * 4;
  const int64_t base = row * ld;
  uint64_t a = 0, b = 0;
  bool bad = false;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if (i0 + j < vocab) {
      const uint32_t u = elem_bits<DT>(logits, base + i0 + j);
      if (!finite_bits(u)) bad = true;
      else top2_push(a, b, cand(u, (uint32_t)(i0 + j)));
    }
  }
  block_top2(a, b, bad);
  if (threadIdx.x == 0) {
    if (bad) {
      a = ~0ull;
      b = 0;
    }
    rec[row * nblk + blk] = make_uint4((uint32_t)a, (uint32_t)(a >> 32), (uint32_t)b, (uint32_t)(b >> 32));
  }
}

// pass 2: one workgroup per row combines the row's records
__global__ __launch_bounds__(kThreads) void top2_pass2(const uint4* __restrict__ rec, int64_t nblk,
                                                       uint32_t* __restrict__ ids2,
                                                       float* __restrict__ gaps) {
  const int64_t row = blockIdx.x;
  uint64_t a = 0, b = 0;
  bool bad = false;
  for (int64_t i = threadIdx.x; i < nblk; i += kThreads) {
    const uint4 r = rec[row * nblk + i];
    const uint64_t ra = ((uint64_t)r.y << 32) | r.x, rb = ((uint64_t)r.w << 32) | r.z;
    if (ra == ~0ull) bad = true;
    else top2_merge(a, b, ra, rb);
  }
  block_top2(a, b, bad);
  if (threadIdx.x == 0) {
    if (bad) {
      ids2[2 * row] = ids2[2 * row + 1] = 0xFFFFFFFFu;
      gaps[row] = __uint_as_float(0x7FC00000u);
    } else {
      ids2[2 * row] = 0xFFFFFFFFu - (uint32_t)a;
      ids2[2 * row + 1] = 0xFFFFFFFFu - (uint32_t)b;
      // key_bits gives +0.0 for either zero, so the gap is never -0.0
      gaps[row] = __uint_as_float(key_bits((uint32_t)(a >> 32))) -
                  __uint_as_float(key_bits((uint32_t)(b >> 32)));
    }
  }
}

}  // namespace

size_t argmax_top2_workspace_bytes(int64_t rows, int64_t vocab) {
  const int64_t nblk = (vocab + kArgmaxBlock - 1) / kArgmaxBlock;
  return (size_t)(rows * nblk) * sizeof(uint4);
}

hipError_t launch_argmax_top2(const void* logits, int dtype, int64_t rows, int64_t vocab, int64_t ld,
                              uint32_t* ids2, float* gaps, void* workspace, hipStream_t stream) {
  const int nblk = (int)((vocab + kArgmaxBlock - 1) / kArgmaxBlock);
  uint4* rec = reinterpret_cast<uint4*>(workspace);
  const dim3 g1((unsigned)nblk, (unsigned)rows);
  if (dtype == 0)
    hipLaunchKernelGGL(top2_pass1<0>, g1, dim3(kThreads), 0, stream, logits, ld, vocab, nblk, rec);
  else
    hipLaunchKernelGGL(top2_pass1<1>, g1, dim3(kThreads), 0, stream, logits, ld, vocab, nblk, rec);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(top2_pass2, dim3((unsigned)rows), dim3(kThreads), 0, stream, rec, (int64_t)nblk,
                     ids2, gaps);
  return hipGetLastError();
}

size_t argmax_workspace_bytes(int64_t rows, int64_t vocab) {
  const int64_t nblk = (vocab + kArgmaxBlock - 1) / kArgmaxBlock;
  return (size_t)(rows * nblk) * sizeof(uint2);
}

hipError_t launch_argmax(const void* logits, int dtype, int64_t rows, int64_t vocab, int64_t ld,
                         uint32_t* ids, void* workspace, hipStream_t stream) {
  const int nblk = (int)((vocab + kArgmaxBlock - 1) / kArgmaxBlock);
  uint2* rec = reinterpret_cast<uint2*>(workspace);
  const dim3 g1((unsigned)nblk, (unsigned)rows);
  if (dtype == 0)
    hipLaunchKernelGGL(argmax_pass1<0>, g1, dim3(kThreads), 0, stream, logits, ld, vocab, nblk, rec);
  else
    hipLaunchKernelGGL(argmax_pass1<1>, g1, dim3(kThreads), 0, stream, logits, ld, vocab, nblk, rec);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_argmax_combine(rec, rows, nblk, ids, stream);
}

hipError_t launch_argmax_combine(const uint2* rec, int64_t rows, int64_t nrec, uint32_t* ids,
                                 hipStream_t stream) {
  if (nrec > 4 * kThreads)
    hipLaunchKernelGGL((argmax_pass2<1024, 16>), dim3((unsigned)rows), dim3(1024), 0, stream, rec, nrec,
                       ids);
  else
    hipLaunchKernelGGL((argmax_pass2<kThreads, 4>), dim3((unsigned)rows), dim3(kThreads), 0, stream, rec,
                       nrec, ids);
  return hipGetLastError();
}

}  // namespace w4g
