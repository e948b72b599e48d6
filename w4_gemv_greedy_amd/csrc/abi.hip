// C ABI of the library (declared in include/w4g.h): argument validation on the
// host, then dispatch to the kernels on the caller's stream.  Validation never
// touches the HIP runtime, so every rejection path runs without a GPU.
#include <stdint.h>
#include <string.h>

#include <atomic>

#include "../../include/w4g.h"
#include "w4g_internal.h"

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned2(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 1u) == 0; }

// [p, p + bytes) and [q, q + qbytes) overlap (empty ranges never do)
bool overlap(const void* p, size_t bytes, const void* q, size_t qbytes) {
  if (!p || !q || bytes == 0 || qbytes == 0) return false;
  const uintptr_t a = reinterpret_cast<uintptr_t>(p), b = reinterpret_cast<uintptr_t>(q);
  return a < b + qbytes && b < a + bytes;
}

constexpr int64_t kMaxDim = (int64_t)1 << 31;  // rows, columns and batch below 2^31

int check_qmm(const uint32_t* wq, const uint16_t* scales, const uint16_t* biases,
              const uint16_t* x, const void* y, int64_t rows, int64_t N, int64_t K,
              const void* workspace, size_t workspace_bytes, size_t need, size_t ysize = 4,
              int bits = 4) {
  if (!wq || !scales || !biases || !x || !y) return W4G_EINVAL_PTR;
  if (rows < 1 || rows >= kMaxDim || N < 1 || N >= kMaxDim || K < 64 || K >= kMaxDim || K % 64)
    return W4G_ESHAPE;
  if (!aligned16(wq) || !aligned16(x) || !aligned16(y) || !aligned2(scales) || !aligned2(biases))
    return W4G_EALIGN;
  if (need > 0 && (!workspace || workspace_bytes < need)) return W4G_EWORKSPACE;
  if (need > 0 && !aligned16(workspace)) return W4G_EALIGN;
  const size_t ybytes = (size_t)rows * (size_t)N * ysize;
  const size_t wbytes = (size_t)N * (size_t)(K * bits / 32) * sizeof(uint32_t);
  const size_t gbytes = (size_t)N * (size_t)(K / 64) * sizeof(uint16_t);
  const size_t xbytes = (size_t)rows * (size_t)K * sizeof(uint16_t);
  if (overlap(y, ybytes, wq, wbytes) || overlap(y, ybytes, scales, gbytes) ||
      overlap(y, ybytes, biases, gbytes) || overlap(y, ybytes, x, xbytes) ||
      overlap(y, ybytes, workspace, need))
    return W4G_EALIAS;
  if (need > 0 && (overlap(workspace, need, wq, wbytes) || overlap(workspace, need, x, xbytes) ||
                   overlap(workspace, need, scales, gbytes) ||
                   overlap(workspace, need, biases, gbytes)))
    return W4G_EALIAS;
  return W4G_OK;
}

int from_hip(hipError_t e) { return e == hipSuccess ? W4G_OK : W4G_ELAUNCH; }

size_t gemv_argmax_bytes(int64_t B, int64_t N, int64_t K) {
  return (size_t)B * (size_t)w4g::gemv_argmax_records_max((int)B, N, K) * sizeof(uint2);
}
size_t gemv_bits_argmax_bytes(int64_t B, int64_t N, int64_t K) {
  return (size_t)B * (size_t)w4g::gemv_bits_argmax_records_max((int)B, N, K) * sizeof(uint2);
}

}  // namespace

namespace w4g {

// Compute units of the current device, queried once per device and kept (a
// device attribute, the same every time it is read); 1..kMaxCUs.  Where the
// query fails the layouts assume kMaxCUs.
int cu_count() {
  constexpr int kDevices = 64;
  static std::atomic<int> cached[kDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kDevices) return kMaxCUs;
  int v = cached[dev].load(std::memory_order_relaxed);
  if (v > 0) return v;
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1) n = kMaxCUs;
  v = n < kMaxCUs ? n : kMaxCUs;
  cached[dev].store(v, std::memory_order_relaxed);
  return v;
}

}  // namespace w4g

namespace {

// The fused head's records for callers that cannot allocate: a file-scope
// device array (zero at load, one copy per GPU, kept until the process ends).
// Host code never passes `scratch` itself to a kernel (on the host the name is
// a stand-in, not a device address): each device's address is taken once with
// hipGetSymbolAddress, with that device current, and kept.
constexpr int64_t kScratchRecords = 131072;  // 1 MiB of (value, id | flag) records
__device__ __align__(256) uint2 scratch[kScratchRecords];

std::atomic<uintptr_t> g_scratch_ptr[64];

// this device's address of `scratch`, or 0 if it cannot be had
uint2* scratch_ptr() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  uintptr_t p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p) return reinterpret_cast<uint2*>(p);
  void* q = nullptr;
  if (hipGetSymbolAddress(&q, HIP_SYMBOL(scratch)) != hipSuccess || !q) return nullptr;
  g_scratch_ptr[dev].store(reinterpret_cast<uintptr_t>(q), std::memory_order_release);
  return reinterpret_cast<uint2*>(q);
}

}  // namespace

extern "C" {

int w4g_abi_version(void) { return W4G_ABI_VERSION; }

const char* w4g_status_string(int status) {
  switch (status) {
    case W4G_OK: return "ok";
    case W4G_EINVAL_PTR: return "a required pointer is NULL";
    case W4G_ESHAPE: return "a size is out of range";
    case W4G_EALIGN: return "a buffer is below its required alignment";
    case W4G_EWORKSPACE: return "workspace missing or too small";
    case W4G_EDTYPE: return "unknown dtype or op";
    case W4G_ELAUNCH: return "the HIP runtime refused a launch";
    case W4G_EALIAS: return "an output overlaps an input or the workspace";
    case W4G_ESCRATCH: return "the sizes need more than the library's static scratch";
    default: return "unknown status";
  }
}

size_t qmm_workspace_bytes(int op, int64_t rows, int64_t n, int64_t k) {
  switch (op) {
    case W4G_OP_GEMV:
      if (rows < 1 || rows > W4G_MAX_GEMV_BATCH || n < 1 || n >= kMaxDim || k < 64 ||
          k >= kMaxDim || k % 64)
        return (size_t)-1;
      return 0;
    case W4G_OP_GEMM:
      if (rows < 1 || rows >= kMaxDim || n < 1 || n >= kMaxDim || k < 64 || k >= kMaxDim || k % 64)
        return (size_t)-1;
      return w4g::gemm_workspace_bytes(rows, n, k);
    case W4G_OP_ARGMAX:
      if (rows < 1 || rows > 65535 || n < 1 || n >= kMaxDim) return (size_t)-1;
      return w4g::argmax_workspace_bytes(rows, n);
    case W4G_OP_ARGMAX_TOP2:
      if (rows < 1 || rows > 65535 || n < 2 || n >= kMaxDim) return (size_t)-1;
      return w4g::argmax_top2_workspace_bytes(rows, n);
    case W4G_OP_GEMV_ARGMAX:
      if (rows < 1 || rows > W4G_MAX_GEMV_BATCH || n < 1 || n >= kMaxDim || k < 64 ||
          k >= kMaxDim || k % 64)
        return (size_t)-1;
      return gemv_argmax_bytes(rows, n, k);
    case W4G_OP_GEMV_BITS_ARGMAX:
      if (rows < 1 || rows > W4G_MAX_GEMV_BATCH || n < 1 || n >= kMaxDim || k < 64 ||
          k >= kMaxDim || k % 64 || !w4g::gemv_bits_fits((int)rows, k))
        return (size_t)-1;
      return gemv_bits_argmax_bytes(rows, n, k);
    default:
      return (size_t)-1;
  }
}

int qmm_gemv_ex(const uint32_t* wq, const uint16_t* scales, const uint16_t* biases,
                const uint16_t* x, float* y, int64_t B, int64_t N, int64_t K, void* workspace,
                size_t workspace_bytes, void* stream, int kernel, int64_t whole) {
  if (kernel != W4G_GEMV_AUTO && kernel != W4G_GEMV_VALU && kernel != W4G_GEMV_MFMA &&
      kernel != W4G_GEMV_VALU_REGS && kernel != W4G_GEMV_MFMA_STEP)
    return W4G_EDTYPE;
  if (B < 1 || B > W4G_MAX_GEMV_BATCH)
    return (!wq || !scales || !biases || !x || !y) ? W4G_EINVAL_PTR : W4G_ESHAPE;
  const int rc = check_qmm(wq, scales, biases, x, y, B, N, K, workspace, workspace_bytes, 0);
  if (rc) return rc;
  if (whole == 0) whole = N;
  if (whole < N || whole >= kMaxDim) return W4G_ESHAPE;
  if (kernel == W4G_GEMV_AUTO) kernel = w4g::gemv_auto_family(whole, K);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (kernel == W4G_GEMV_MFMA || kernel == W4G_GEMV_MFMA_STEP)
    return from_hip(w4g::launch_gemv_mfma(wq, scales, biases, x, y, (int)B, N, K,
                                          kernel == W4G_GEMV_MFMA_STEP, s));
  return from_hip(w4g::launch_gemv(wq, scales, biases, x, y, (int)B, N, K,
                                   kernel == W4G_GEMV_VALU_REGS, s));
}

int qmm_gemv_bits(const uint32_t* wq, const uint16_t* scales, const uint16_t* biases,
                  const uint16_t* x, float* y, int64_t B, int64_t N, int64_t K, int bits,
                  void* workspace, size_t workspace_bytes, void* stream) {
  if (bits != 2 && bits != 4 && bits != 8) return W4G_EDTYPE;
  if (bits == 4)
    return qmm_gemv_ex(wq, scales, biases, x, y, B, N, K, workspace, workspace_bytes, stream,
                       W4G_GEMV_AUTO, 0);
  if (B < 1 || B > W4G_MAX_GEMV_BATCH)
    return (!wq || !scales || !biases || !x || !y) ? W4G_EINVAL_PTR : W4G_ESHAPE;
  const int rc = check_qmm(wq, scales, biases, x, y, B, N, K, workspace, workspace_bytes, 0, 4, bits);
  if (rc) return rc;
  if (!w4g::gemv_bits_fits((int)B, K)) return W4G_ESHAPE;
  return from_hip(w4g::launch_gemv_bits(wq, scales, biases, x, y, (int)B, N, K, bits,
                                        reinterpret_cast<hipStream_t>(stream)));
}

int qmm_gemv(const uint32_t* wq, const uint16_t* scales, const uint16_t* biases,
             const uint16_t* x, float* y, int64_t B, int64_t N, int64_t K, void* workspace,
             size_t workspace_bytes, void* stream) {
  return qmm_gemv_ex(wq, scales, biases, x, y, B, N, K, workspace, workspace_bytes, stream,
                     W4G_GEMV_AUTO, 0);
}

int qmm_gemm_ex(const uint32_t* wq, const uint16_t* scales, const uint16_t* biases,
                const uint16_t* x, void* y, int64_t M, int64_t N, int64_t K, void* workspace,
                size_t workspace_bytes, void* stream, int y_dtype) {
  if (y_dtype != W4G_F32 && y_dtype != W4G_BF16) return W4G_EDTYPE;
  if (M < 1 || M >= kMaxDim || N < 1 || N >= kMaxDim || K < 64 || K >= kMaxDim || K % 64)
    return (!wq || !scales || !biases || !x || !y) ? W4G_EINVAL_PTR : W4G_ESHAPE;
  const size_t need = w4g::gemm_workspace_bytes(M, N, K);
  const int rc = check_qmm(wq, scales, biases, x, y, M, N, K, workspace, workspace_bytes, need,
                           y_dtype == W4G_BF16 ? 2 : 4);
  if (rc) return rc;
  return from_hip(w4g::launch_gemm(wq, scales, biases, x, y, y_dtype == W4G_BF16, M, N, K, workspace,
                                   reinterpret_cast<hipStream_t>(stream)));
}

int qmm_gemm(const uint32_t* wq, const uint16_t* scales, const uint16_t* biases,
             const uint16_t* x, float* y, int64_t M, int64_t N, int64_t K, void* workspace,
             size_t workspace_bytes, void* stream) {
  return qmm_gemm_ex(wq, scales, biases, x, y, M, N, K, workspace, workspace_bytes, stream, W4G_F32);
}

}  // extern "C"

namespace {

// Checks shared by the fused head's entry points: pointers, sizes, alignment
// and, with `alias`, that no output overlaps an input or another output (the
// records' `need` bytes at `workspace`, when one is given, among the outputs).
int check_gemv_argmax(const uint32_t* wq, const uint16_t* scales, const uint16_t* biases,
                      const uint16_t* x, const float* logits, const uint32_t* ids, int64_t B, int64_t N,
                      int64_t K, const void* workspace, size_t need, bool alias = true, int bits = 4) {
  if (!wq || !scales || !biases || !x || !ids) return W4G_EINVAL_PTR;
  if (B < 1 || B > W4G_MAX_GEMV_BATCH || N < 1 || N >= kMaxDim || K < 64 || K >= kMaxDim || K % 64)
    return W4G_ESHAPE;
  if (!aligned16(wq) || !aligned16(x) || (logits && !aligned16(logits)) || !aligned2(scales) ||
      !aligned2(biases) || (reinterpret_cast<uintptr_t>(ids) & 3u))
    return W4G_EALIGN;
  if (!alias) return W4G_OK;
  const size_t wbytes = (size_t)N * (size_t)(K * bits / 32) * sizeof(uint32_t);
  const size_t gbytes = (size_t)N * (size_t)(K / 64) * sizeof(uint16_t);
  const size_t xbytes = (size_t)B * (size_t)K * sizeof(uint16_t);
  const size_t lbytes = logits ? (size_t)B * (size_t)N * sizeof(float) : 0;
  const size_t ibytes = (size_t)B * sizeof(uint32_t);
  const void* outs[3] = {logits, ids, workspace};
  const size_t osz[3] = {lbytes, ibytes, workspace ? need : 0};
  for (int i = 0; i < 3; ++i) {
    if (overlap(outs[i], osz[i], wq, wbytes) || overlap(outs[i], osz[i], scales, gbytes) ||
        overlap(outs[i], osz[i], biases, gbytes) || overlap(outs[i], osz[i], x, xbytes))
      return W4G_EALIAS;
    for (int j = i + 1; j < 3; ++j)
      if (overlap(outs[i], osz[i], outs[j], osz[j])) return W4G_EALIAS;
  }
  return W4G_OK;
}

int run_gemv_argmax(const uint32_t* wq, const uint16_t* scales, const uint16_t* biases, const uint16_t* x,
                    float* logits, uint32_t* ids, int64_t B, int64_t N, int64_t K, uint2* rec,
                    hipStream_t s) {
  const hipError_t e = w4g::launch_gemv_argmax(wq, scales, biases, x, logits, rec, (int)B, N, K, s);
  if (e != hipSuccess) return W4G_ELAUNCH;
  return from_hip(w4g::launch_argmax_combine(rec, B, w4g::gemv_argmax_records((int)B, N, K), ids, s));
}

}  // namespace

extern "C" {

int qmm_gemv_argmax(const uint32_t* wq, const uint16_t* scales, const uint16_t* biases,
                    const uint16_t* x, float* logits, uint32_t* ids, int64_t B, int64_t N, int64_t K,
                    void* workspace, size_t workspace_bytes, void* stream) {
  int rc = check_gemv_argmax(wq, scales, biases, x, logits, ids, B, N, K, nullptr, 0, false);
  if (rc) return rc;
  const size_t need = gemv_argmax_bytes(B, N, K);
  if (!workspace || workspace_bytes < need) return W4G_EWORKSPACE;
  if (reinterpret_cast<uintptr_t>(workspace) & 7u) return W4G_EALIGN;
  rc = check_gemv_argmax(wq, scales, biases, x, logits, ids, B, N, K, workspace, need);
  if (rc) return rc;
  return run_gemv_argmax(wq, scales, biases, x, logits, ids, B, N, K, reinterpret_cast<uint2*>(workspace),
                         reinterpret_cast<hipStream_t>(stream));
}

int qmm_gemv_bits_argmax(const uint32_t* wq, const uint16_t* scales, const uint16_t* biases,
                         const uint16_t* x, float* logits, uint32_t* ids, int64_t B, int64_t N, int64_t K,
                         int bits, void* workspace, size_t workspace_bytes, void* stream) {
  if (bits != 2 && bits != 4 && bits != 8) return W4G_EDTYPE;
  if (bits == 4)
    return qmm_gemv_argmax(wq, scales, biases, x, logits, ids, B, N, K, workspace, workspace_bytes, stream);
  int rc = check_gemv_argmax(wq, scales, biases, x, logits, ids, B, N, K, nullptr, 0, false, bits);
  if (rc) return rc;
  if (!w4g::gemv_bits_fits((int)B, K)) return W4G_ESHAPE;
  const size_t need = gemv_bits_argmax_bytes(B, N, K);
  if (!workspace || workspace_bytes < need) return W4G_EWORKSPACE;
  if (reinterpret_cast<uintptr_t>(workspace) & 7u) return W4G_EALIGN;
  rc = check_gemv_argmax(wq, scales, biases, x, logits, ids, B, N, K, workspace, need, true, bits);
  if (rc) return rc;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  uint2* rec = reinterpret_cast<uint2*>(workspace);
  const hipError_t e = w4g::launch_gemv_bits_argmax(wq, scales, biases, x, logits, rec, (int)B, N, K, bits, s);
  if (e != hipSuccess) return W4G_ELAUNCH;
  return from_hip(w4g::launch_argmax_combine(rec, B, w4g::gemv_bits_argmax_records((int)B, N, K), ids, s));
}

int qmm_gemv_argmax_noalloc(const uint32_t* wq, const uint16_t* scales, const uint16_t* biases,
                            const uint16_t* x, float* logits, uint32_t* ids, int64_t B, int64_t N,
                            int64_t K, void* stream) {
  const int rc = check_gemv_argmax(wq, scales, biases, x, logits, ids, B, N, K, nullptr, 0);
  if (rc) return rc;
  if (gemv_argmax_bytes(B, N, K) > (size_t)kScratchRecords * sizeof(uint2)) return W4G_ESCRATCH;
  uint2* rec = scratch_ptr();
  if (!rec) return W4G_ELAUNCH;
  return run_gemv_argmax(wq, scales, biases, x, logits, ids, B, N, K, rec, reinterpret_cast<hipStream_t>(stream));
}

int vocab_argmax_top2(const void* logits, int dtype, int64_t rows, int64_t vocab, int64_t ld,
                      uint32_t* ids2, float* gaps, void* workspace, size_t workspace_bytes,
                      void* stream) {
  if (!logits || !ids2 || !gaps) return W4G_EINVAL_PTR;
  if (dtype != W4G_F32 && dtype != W4G_BF16) return W4G_EDTYPE;
  if (rows < 1 || rows > 65535 || vocab < 2 || vocab >= kMaxDim || ld < vocab || ld >= ((int64_t)1 << 40))
    return W4G_ESHAPE;
  if (!aligned16(logits) || (reinterpret_cast<uintptr_t>(ids2) & 3u) ||
      (reinterpret_cast<uintptr_t>(gaps) & 3u))
    return W4G_EALIGN;
  const size_t need = w4g::argmax_top2_workspace_bytes(rows, vocab);
  if (!workspace || workspace_bytes < need) return W4G_EWORKSPACE;
  if (!aligned16(workspace)) return W4G_EALIGN;
  const size_t esz = dtype == W4G_F32 ? 4 : 2;
  const size_t lbytes = ((size_t)(rows - 1) * (size_t)ld + (size_t)vocab) * esz;
  const void* outs[3] = {ids2, gaps, workspace};
  const size_t osz[3] = {(size_t)rows * 8, (size_t)rows * 4, need};
  for (int i = 0; i < 3; ++i) {
    if (overlap(outs[i], osz[i], logits, lbytes)) return W4G_EALIAS;
    for (int j = i + 1; j < 3; ++j)
      if (overlap(outs[i], osz[i], outs[j], osz[j])) return W4G_EALIAS;
  }
  return from_hip(w4g::launch_argmax_top2(logits, dtype, rows, vocab, ld, ids2, gaps, workspace,
                                          reinterpret_cast<hipStream_t>(stream)));
}

int vocab_argmax(const void* logits, int dtype, int64_t rows, int64_t vocab, int64_t ld,
                 uint32_t* ids, void* workspace, size_t workspace_bytes, void* stream) {
  if (!logits || !ids) return W4G_EINVAL_PTR;
  if (dtype != W4G_F32 && dtype != W4G_BF16) return W4G_EDTYPE;
  if (rows < 1 || rows > 65535 || vocab < 1 || vocab >= kMaxDim || ld < vocab || ld >= ((int64_t)1 << 40))
    return W4G_ESHAPE;
  if (!aligned16(logits) || (reinterpret_cast<uintptr_t>(ids) & 3u)) return W4G_EALIGN;
  const size_t need = w4g::argmax_workspace_bytes(rows, vocab);
  if (!workspace || workspace_bytes < need) return W4G_EWORKSPACE;
  if (reinterpret_cast<uintptr_t>(workspace) & 7u) return W4G_EALIGN;
  const size_t esz = dtype == W4G_F32 ? 4 : 2;
  const size_t lbytes = ((size_t)(rows - 1) * (size_t)ld + (size_t)vocab) * esz;
  if (overlap(ids, (size_t)rows * 4, logits, lbytes) || overlap(ids, (size_t)rows * 4, workspace, need) ||
      overlap(workspace, need, logits, lbytes))
    return W4G_EALIAS;
  return from_hip(w4g::launch_argmax(logits, dtype, rows, vocab, ld, ids, workspace,
                                     reinterpret_cast<hipStream_t>(stream)));
}

}  // extern "C"
