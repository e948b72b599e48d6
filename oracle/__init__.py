"""CPU oracle for the W4 g64 products and the greedy vocabulary argmax.

TEST INFRASTRUCTURE ONLY: imported by the test suite, by the smoke check and by
the benchmark's CPU-baseline leg, never by the product path.  It shares no code
with the HIP library.  The arithmetic lives in ``w4g_oracle.c`` (plain C, built
with gcc); this module compiles it, loads it with ctypes and marshals numpy
arrays.  bf16 tensors travel as their uint16 bit patterns.

Definitions followed (see the C file for the full statement and citations):
  * weights: 4-bit affine, group 64 (TensorFold PR #1437, "Receipt"),
    w = q*s + b with q in 0..15 packed low nibble first, 8 per uint32 along K;
    other widths (2 and 8 bits, reading of the pages' simd_qmm_bits variant and
    the B70 page's INT8 LM head): the same format with 32/bits codes per word;
  * products: fp32 result of sum_k x*w (TensorFold PR #1437, commit "Add the
    pair seam ...": fp32 payload and fp32-out store), summed in fp64;
  * argmax: any non-finite value in a row gives 0xFFFFFFFF, else the largest
    value with ties to the lowest id (TensorFold PR #1433, step-1 description);
  * bf16 store: fp32 result rounded to bf16 nearest-even, NaN kept (reading of
    the pages' activation-dtype store beside the fp32-out variant).
"""
import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "w4g_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")
SENTINEL = 0xFFFFFFFF

_libs = {}


def build(plant=0, out=None, quiet=True, sanitize=False):
    """Compile the oracle (optionally with planted mistake ``plant``, or with
    AddressSanitizer and UndefinedBehaviorSanitizer for a checking run) and
    return the path."""
    out = out or (LIB if plant == 0 else os.path.join(HERE, f"liboracle_plant{plant}.so"))
    opt = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all"] if sanitize else ["-O2"]
    cmd = ["gcc"] + opt + ["-std=c99", "-fopenmp", "-ffp-contract=off", "-fPIC", "-shared",
                           f"-DW4O_PLANT={int(plant)}", SRC, "-o", out + ".tmp", "-lm"]
    subprocess.run(cmd, check=True, capture_output=quiet)
    os.replace(out + ".tmp", out)
    return out


def load(path=None):
    path = path or LIB
    if path in _libs:
        return _libs[path]
    if path == LIB and (not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC)):
        build()
    lib = ctypes.CDLL(path)
    P, I64, I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    lib.w4o_dequant.argtypes = [P, P, P, I64, I64, P]
    lib.w4o_dequant.restype = None
    lib.w4o_qmm.argtypes = [P, P, P, P, P, I64, I64, I64, I]
    lib.w4o_qmm.restype = None
    lib.w4o_qmm_rows.argtypes = [P, P, P, P, P, I64, I64, I64, P, I64, I]
    lib.w4o_qmm_rows.restype = None
    lib.w4o_argmax.argtypes = [P, I, I64, I64, I64, P, P]
    lib.w4o_argmax.restype = I
    lib.w4o_argmax_top2.argtypes = [P, I, I64, I64, I64, P, P, P]
    lib.w4o_argmax_top2.restype = I
    lib.w4o_dequant_bits.argtypes = [P, P, P, I64, I64, I, P]
    lib.w4o_dequant_bits.restype = I
    lib.w4o_qmm_bits.argtypes = [P, P, P, P, P, I64, I64, I64, I, I]
    lib.w4o_qmm_bits.restype = I
    lib.w4o_qmm_rows_bits.argtypes = [P, P, P, P, P, I64, I64, I64, P, I64, I, I]
    lib.w4o_qmm_rows_bits.restype = I
    lib.w4o_to_bf16.argtypes = [P, P, I64]
    lib.w4o_to_bf16.restype = None
    lib.w4o_plant.restype = I
    lib.w4o_threads.restype = I
    _libs[path] = lib
    return lib


def _c(a, dtype):
    a = np.ascontiguousarray(a)
    if a.dtype != dtype:
        raise TypeError(f"expected {dtype}, got {a.dtype}")
    return a


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def _shapes(wq, scales, biases, x, bits=4):
    if bits not in (2, 4, 8):
        raise ValueError("bits must be 2, 4 or 8")
    N, words = wq.shape
    K = words * 32 // bits
    if K % 64 or scales.shape != (N, K // 64) or biases.shape != (N, K // 64):
        raise ValueError("bad weight/scale/bias shapes")
    if x.ndim != 2 or x.shape[1] != K:
        raise ValueError("x must be [M][K]")
    return x.shape[0], N, K


def dequant(wq, scales, biases, lib=None, bits=4):
    """fp32 [N][K] matrix of w = q*s + b (codes of `bits` bits, 32/bits per word)."""
    lib = lib or load()
    wq, scales, biases = _c(wq, np.uint32), _c(scales, np.uint16), _c(biases, np.uint16)
    N, K = wq.shape[0], wq.shape[1] * 32 // bits
    w = np.empty((N, K), np.float32)
    if bits == 4:
        lib.w4o_dequant(_ptr(wq), _ptr(scales), _ptr(biases), N, K, _ptr(w))
    elif lib.w4o_dequant_bits(_ptr(wq), _ptr(scales), _ptr(biases), N, K, int(bits), _ptr(w)):
        raise ValueError("bits must be 2, 4 or 8")
    return w


def qmm(wq, scales, biases, x, threads=0, lib=None, bits=4):
    """y [M][N] fp32 = x [M][K] (bf16 bits) times dequantized W^T."""
    lib = lib or load()
    wq, scales, biases, x = (_c(wq, np.uint32), _c(scales, np.uint16), _c(biases, np.uint16),
                             _c(x, np.uint16))
    M, N, K = _shapes(wq, scales, biases, x, bits)
    y = np.empty((M, N), np.float32)
    if bits == 4:
        lib.w4o_qmm(_ptr(wq), _ptr(scales), _ptr(biases), _ptr(x), _ptr(y), M, N, K, int(threads))
    else:
        lib.w4o_qmm_bits(_ptr(wq), _ptr(scales), _ptr(biases), _ptr(x), _ptr(y), M, N, K, int(bits),
                         int(threads))
    return y


def qmm_rows(wq, scales, biases, x, rows, threads=0, lib=None, bits=4):
    """y [M][len(rows)]: only the listed output rows."""
    lib = lib or load()
    wq, scales, biases, x = (_c(wq, np.uint32), _c(scales, np.uint16), _c(biases, np.uint16),
                             _c(x, np.uint16))
    M, N, K = _shapes(wq, scales, biases, x, bits)
    rows = _c(np.asarray(rows, dtype=np.int64), np.int64)
    if rows.size and (rows.min() < 0 or rows.max() >= N):
        raise IndexError("row out of range")
    y = np.empty((M, rows.size), np.float32)
    if bits == 4:
        lib.w4o_qmm_rows(_ptr(wq), _ptr(scales), _ptr(biases), _ptr(x), _ptr(y), M, N, K,
                         _ptr(rows), rows.size, int(threads))
    else:
        lib.w4o_qmm_rows_bits(_ptr(wq), _ptr(scales), _ptr(biases), _ptr(x), _ptr(y), M, N, K,
                              _ptr(rows), rows.size, int(bits), int(threads))
    return y


def argmax(logits, lib=None):
    """ids [rows] uint32 of a [rows][V] fp32 array, or of bf16 bits given as uint16."""
    lib = lib or load()
    logits = np.ascontiguousarray(logits)
    if logits.ndim == 1:
        logits = logits[None, :]
    if logits.dtype == np.float32:
        dtype = 0
    elif logits.dtype == np.uint16:
        dtype = 1
    else:
        raise TypeError("logits must be float32 or bf16 bits (uint16)")
    rows, V = logits.shape
    ids = np.empty(rows, np.uint32)
    scratch = np.empty(max(V, 1), np.float32)
    rc = lib.w4o_argmax(_ptr(logits), dtype, rows, V, V, _ptr(ids), _ptr(scratch))
    if rc:
        raise ValueError(f"oracle argmax rejected its arguments ({rc})")
    return ids


def argmax_top2(logits, lib=None):
    """(ids [rows][2] uint32, gaps [rows] fp32): winner and runner-up of each row
    (value descending, id ascending), gap = v(winner) - v(runner-up) with zeros as
    +0.0; the sentinel twice and a NaN gap for a row holding a non-finite value.
    logits: [rows][V >= 2] fp32, or bf16 bits as uint16."""
    lib = lib or load()
    logits = np.ascontiguousarray(logits)
    if logits.ndim == 1:
        logits = logits[None, :]
    if logits.dtype == np.float32:
        dtype = 0
    elif logits.dtype == np.uint16:
        dtype = 1
    else:
        raise TypeError("logits must be float32 or bf16 bits (uint16)")
    rows, V = logits.shape
    ids = np.empty((rows, 2), np.uint32)
    gaps = np.empty(rows, np.float32)
    scratch = np.empty(max(V, 1), np.float32)
    rc = lib.w4o_argmax_top2(_ptr(logits), dtype, rows, V, V, _ptr(ids), _ptr(gaps), _ptr(scratch))
    if rc:
        raise ValueError(f"oracle top-2 rejected its arguments ({rc})")
    return ids, gaps


def to_bf16(y, lib=None):
    """bf16 bits (uint16, same shape) of fp32 values rounded to nearest-even."""
    lib = lib or load()
    y = _c(np.asarray(y, np.float32), np.float32)
    out = np.empty(y.shape, np.uint16)
    lib.w4o_to_bf16(_ptr(y), _ptr(out), y.size)
    return out


def threads(lib=None):
    return (lib or load()).w4o_threads()
