"""ctypes view of libw4g.so (the C ABI declared in include/w4g.h)."""
import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libw4g.so")

# status codes and constants, as in include/w4g.h
OK, EINVAL_PTR, ESHAPE, EALIGN, EWORKSPACE, EDTYPE, ELAUNCH, EALIAS, ESCRATCH = range(9)
F32, BF16 = 0, 1
OP_GEMV, OP_GEMM, OP_ARGMAX, OP_GEMV_ARGMAX, OP_ARGMAX_TOP2, OP_GEMV_BITS_ARGMAX = 0, 1, 2, 3, 4, 5
SENTINEL = 0xFFFFFFFF
MAX_GEMV_BATCH = 8
ABI_VERSION = 3

GEMV_AUTO, GEMV_VALU, GEMV_MFMA, GEMV_VALU_REGS, GEMV_MFMA_STEP = 0, 1, 2, 3, 4

EXPORTS = ["qmm_gemv", "qmm_gemv_ex", "qmm_gemv_bits", "qmm_gemm", "qmm_gemm_ex", "qmm_gemv_argmax", "qmm_gemv_bits_argmax", "qmm_gemv_argmax_noalloc", "vocab_argmax",
           "vocab_argmax_top2", "qmm_workspace_bytes", "w4g_status_string", "w4g_abi_version"]

_lib = None


class W4GError(RuntimeError):
    def __init__(self, fn, status, msg):
        super().__init__(f"{fn}: status {status} ({msg})")
        self.status = status


def load(path=None):
    """Load the library (once).  Raises if it has not been built: there is no fallback."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"{p} is missing: build it with `python -m w4_gemv_greedy_amd.build`")
    lib = ctypes.CDLL(p)
    P, I64, I, SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t
    lib.qmm_gemv.argtypes = [P, P, P, P, P, I64, I64, I64, P, SZ, P]
    lib.qmm_gemv.restype = I
    lib.qmm_gemv_ex.argtypes = [P, P, P, P, P, I64, I64, I64, P, SZ, P, I, I64]
    lib.qmm_gemv_ex.restype = I
    lib.qmm_gemv_bits.argtypes = [P, P, P, P, P, I64, I64, I64, I, P, SZ, P]
    lib.qmm_gemv_bits.restype = I
    lib.qmm_gemm.argtypes = [P, P, P, P, P, I64, I64, I64, P, SZ, P]
    lib.qmm_gemm.restype = I
    lib.qmm_gemm_ex.argtypes = [P, P, P, P, P, I64, I64, I64, P, SZ, P, I]
    lib.qmm_gemm_ex.restype = I
    lib.qmm_gemv_argmax.argtypes = [P, P, P, P, P, P, I64, I64, I64, P, SZ, P]
    lib.qmm_gemv_argmax.restype = I
    lib.qmm_gemv_bits_argmax.argtypes = [P, P, P, P, P, P, I64, I64, I64, I, P, SZ, P]
    lib.qmm_gemv_bits_argmax.restype = I
    lib.qmm_gemv_argmax_noalloc.argtypes = [P, P, P, P, P, P, I64, I64, I64, P]
    lib.qmm_gemv_argmax_noalloc.restype = I
    lib.vocab_argmax_top2.argtypes = [P, I, I64, I64, I64, P, P, P, SZ, P]
    lib.vocab_argmax_top2.restype = I
    lib.vocab_argmax.argtypes = [P, I, I64, I64, I64, P, P, SZ, P]
    lib.vocab_argmax.restype = I
    lib.qmm_workspace_bytes.argtypes = [I, I64, I64, I64]
    lib.qmm_workspace_bytes.restype = SZ
    lib.w4g_status_string.argtypes = [I]
    lib.w4g_status_string.restype = ctypes.c_char_p
    lib.w4g_abi_version.argtypes = []
    lib.w4g_abi_version.restype = I
    if lib.w4g_abi_version() != ABI_VERSION:
        raise RuntimeError(f"{p}: ABI version {lib.w4g_abi_version()}, expected {ABI_VERSION}")
    if path is None:
        _lib = lib
    return lib


def check(fn, status):
    if status != OK:
        raise W4GError(fn, status, load().w4g_status_string(status).decode())
