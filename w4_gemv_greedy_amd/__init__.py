"""W4 g64 quantized GEMV/GEMM and greedy vocabulary argmax for MI355X (gfx950).

A thin binding over the C ABI of ``libw4g.so`` (include/w4g.h): it checks
tensor dtypes, devices and shapes, then passes raw device pointers and the
current HIP stream.  Every step of the computation runs in the library's HIP
kernels; there is no Python or CPU fallback, and a missing library raises.

Tensors (all on one GPU, contiguous):
  wq      [N][K/8]  int32/uint32  packed 4-bit codes, element 8i+j in bits [4j, 4j+4)
  scales  [N][K/64] bfloat16
  biases  [N][K/64] bfloat16
  x       [B or M][K] bfloat16
  returns y [B or M][N] float32
"""
import ctypes

from . import _lib
from ._lib import (BF16, F32, GEMV_AUTO, GEMV_MFMA, GEMV_MFMA_STEP, GEMV_VALU, GEMV_VALU_REGS,  # noqa: F401
                   MAX_GEMV_BATCH,
                   OP_ARGMAX, OP_ARGMAX_TOP2, OP_GEMM, OP_GEMV, OP_GEMV_ARGMAX, OP_GEMV_BITS_ARGMAX, SENTINEL,
                   W4GError)

__all__ = ["qmm_gemv", "qmm_gemm", "qmm_gemv_argmax", "qmm_gemv_argmax_noalloc", "vocab_argmax",
           "vocab_argmax_top2",
           "workspace_bytes", "SENTINEL", "W4GError"]


_TORCH = None


def _torch():
    global _TORCH
    if _TORCH is None:
        import torch
        _TORCH = torch
    return _TORCH


def _stream(t):
    """The current stream of t's GPU (as torch.cuda.current_stream(t.device))."""
    return ctypes.c_void_p(_torch()._C._cuda_getCurrentRawStream(t.get_device()))


def _need(t, name, dtypes, ndim, device):
    """device: a GPU index (or torch.device) t must be on, or None for any GPU.
    Every check runs on every call; they read only cheap tensor attributes."""
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype not in dtypes:
        raise TypeError(f"{name}: dtype {t.dtype} not in {dtypes}")
    if t.dim() != ndim:
        raise ValueError(f"{name}: expected {ndim} dims, got {tuple(t.shape)}")
    d = t.get_device()
    if d < 0 or (device is not None and d != (device if isinstance(device, int) else device.index)):
        raise ValueError(f"{name} must be on the same GPU as the weights")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _check_qmm(wq, scales, biases, x, bits=4):
    torch = _torch()
    _need(wq, "wq", (torch.int32, torch.uint32), 2, None)
    dev = wq.get_device()
    _need(scales, "scales", (torch.bfloat16, torch.int16, torch.uint16), 2, dev)
    _need(biases, "biases", (torch.bfloat16, torch.int16, torch.uint16), 2, dev)
    _need(x, "x", (torch.bfloat16, torch.int16, torch.uint16), 2, dev)
    if bits not in (2, 4, 8):
        raise ValueError("bits must be 2, 4 or 8")
    N, K = wq.shape[0], wq.shape[1] * 32 // bits
    if tuple(scales.shape) != (N, K // 64) or tuple(biases.shape) != (N, K // 64):
        raise ValueError("scales and biases must be [N][K/64]")
    if x.shape[1] != K:
        raise ValueError(f"x must be [rows][{K}]")
    return N, K


def workspace_bytes(op, rows, n, k):
    v = _lib.load().qmm_workspace_bytes(op, rows, n, k)
    if v == ctypes.c_size_t(-1).value:
        raise ValueError("sizes out of range for this op")
    return v


def _workspace(op, rows, n, k, device, workspace):
    """The workspace for op: a new one when none is given, else the caller's,
    checked like every other tensor argument (on the inputs' GPU, contiguous,
    large enough) before its address reaches a kernel."""
    need = workspace_bytes(op, rows, n, k)
    if need == 0:
        return None, 0
    torch = _torch()
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=device)
    if not isinstance(workspace, torch.Tensor):
        raise TypeError("workspace must be a torch.Tensor")
    d = workspace.get_device()
    if d < 0 or d != (device if isinstance(device, int) else device.index):
        raise ValueError("workspace must be on the same GPU as the inputs")
    if not workspace.is_contiguous():
        raise ValueError("workspace must be contiguous")
    if workspace.numel() * workspace.element_size() < need:
        raise ValueError(f"workspace needs {need} bytes")
    return workspace, need


def _call_qmm(fn, op, wq, scales, biases, x, y, workspace, extra=(), y_dtypes=None):
    torch = _torch()
    N, K = _check_qmm(wq, scales, biases, x)
    rows = x.shape[0]
    y_dtypes = y_dtypes or (torch.float32,)
    if y is None:
        y = torch.empty((rows, N), dtype=y_dtypes[0], device=wq.device)
    _need(y, "y", y_dtypes, 2, wq.get_device())
    if y.shape[0] != rows or y.shape[1] != N:
        raise ValueError(f"y must be [{rows}][{N}]")
    # the decode products take no workspace (the library checks B itself)
    ws, nbytes = (None, 0) if op == OP_GEMV else _workspace(op, rows, N, K, wq.device, workspace)
    lib = _lib.load()
    status = getattr(lib, fn)(wq.data_ptr(), scales.data_ptr(), biases.data_ptr(), x.data_ptr(),
                              y.data_ptr(), rows, N, K, ws.data_ptr() if ws is not None else None,
                              nbytes if ws is not None else 0, _stream(wq), *extra)
    _lib.check(fn, status)
    return y


def qmm_gemv(wq, scales, biases, x, y=None, workspace=None, kernel=GEMV_AUTO, bits=4, whole=None):
    """Decode product for 1 <= B <= 8 rows of x; returns y [B][N] fp32.

    kernel: GEMV_AUTO (the library's choice, a function of K and `whole` only,
    never of B), GEMV_VALU, GEMV_MFMA, GEMV_VALU_REGS (the register-staged
    variant of the vector-ALU family) or GEMV_MFMA_STEP (the step-staged
    variant of the matrix-core family).
    whole: the row count of the whole matrix when wq holds a row slice of it
    (None: N), so that the slice's rows get the whole matrix's bits.
    bits: code width, 4 (the default) or 2 or 8 (wq [N][K*bits/32], low field
    first; the library's choice of kernel only).
    """
    if x.dim() == 2 and not 1 <= x.shape[0] <= MAX_GEMV_BATCH:
        raise ValueError(f"qmm_gemv takes 1..{MAX_GEMV_BATCH} rows")
    if bits != 4:
        if kernel != GEMV_AUTO or whole is not None:
            raise ValueError("other code widths take the library's kernel choice only")
        torch = _torch()
        N, K = _check_qmm(wq, scales, biases, x, bits)
        rows = x.shape[0]
        if y is None:
            y = torch.empty((rows, N), dtype=torch.float32, device=wq.device)
        _need(y, "y", (torch.float32,), 2, wq.device)
        if tuple(y.shape) != (rows, N):
            raise ValueError(f"y must be [{rows}][{N}]")
        status = _lib.load().qmm_gemv_bits(wq.data_ptr(), scales.data_ptr(), biases.data_ptr(), x.data_ptr(),
                                           y.data_ptr(), rows, N, K, int(bits), None, 0, _stream(wq))
        _lib.check("qmm_gemv_bits", status)
        return y
    if kernel == GEMV_AUTO and whole is None:
        return _call_qmm("qmm_gemv", OP_GEMV, wq, scales, biases, x, y, workspace)
    return _call_qmm("qmm_gemv_ex", OP_GEMV, wq, scales, biases, x, y, workspace,
                     (int(kernel), int(whole or 0)))


def qmm_gemm(wq, scales, biases, x, y=None, workspace=None, out_dtype=None):
    """Prompt product for any M >= 1 rows of x (matrix cores); returns y [M][N].

    out_dtype: torch.float32 (the default) or torch.bfloat16, the fp32 result
    rounded to nearest-even in the kernel's store.  A given y sets the dtype.
    """
    torch = _torch()
    if out_dtype is None:
        out_dtype = y.dtype if y is not None else torch.float32
    if out_dtype == torch.float32:
        return _call_qmm("qmm_gemm", OP_GEMM, wq, scales, biases, x, y, workspace)
    if out_dtype != torch.bfloat16:
        raise TypeError(f"out_dtype must be float32 or bfloat16, not {out_dtype}")
    return _call_qmm("qmm_gemm_ex", OP_GEMM, wq, scales, biases, x, y, workspace, (BF16,),
                     y_dtypes=(torch.bfloat16,))


def qmm_gemv_argmax(wq, scales, biases, x, logits=None, ids=None, workspace=None, want_logits=True, bits=4):
    """Decode product and greedy argmax per batch row, the argmax's first pass
    fused into the product; returns (ids, logits).  The logits are bitwise
    those of qmm_gemv (the same kernel family; with bits 2 or 8, those of
    qmm_gemv(..., bits=bits)).

    ids: int32 tensor [B] holding uint32 bits (0xFFFFFFFF = a non-finite logit
    in the row).  logits: [B][N] fp32, allocated when not given and
    want_logits is true; with want_logits false and no tensor given the
    logits are never written and None is returned in their place.
    """
    torch = _torch()
    N, K = _check_qmm(wq, scales, biases, x, bits)
    rows = x.shape[0]
    if not 1 <= rows <= MAX_GEMV_BATCH:
        raise ValueError(f"qmm_gemv_argmax takes 1..{MAX_GEMV_BATCH} rows")
    if logits is None and want_logits:
        logits = torch.empty((rows, N), dtype=torch.float32, device=wq.device)
    if logits is not None:
        _need(logits, "logits", (torch.float32,), 2, wq.device)
        if tuple(logits.shape) != (rows, N):
            raise ValueError(f"logits must be [{rows}][{N}]")
    if ids is None:
        ids = torch.empty(rows, dtype=torch.int32, device=wq.device)
    _need(ids, "ids", (torch.int32, torch.uint32), 1, wq.device)
    if ids.shape[0] != rows:
        raise ValueError("ids must have one entry per row")
    lib = _lib.load()
    if bits != 4:
        ws, nbytes = _workspace(OP_GEMV_BITS_ARGMAX, rows, N, K, wq.device, workspace)
        status = lib.qmm_gemv_bits_argmax(wq.data_ptr(), scales.data_ptr(), biases.data_ptr(), x.data_ptr(),
                                          logits.data_ptr() if logits is not None else None, ids.data_ptr(),
                                          rows, N, K, int(bits), ws.data_ptr(), nbytes, _stream(wq))
        _lib.check("qmm_gemv_bits_argmax", status)
        return ids, logits
    ws, nbytes = _workspace(OP_GEMV_ARGMAX, rows, N, K, wq.device, workspace)
    status = lib.qmm_gemv_argmax(wq.data_ptr(), scales.data_ptr(), biases.data_ptr(), x.data_ptr(),
                                 logits.data_ptr() if logits is not None else None, ids.data_ptr(),
                                 rows, N, K, ws.data_ptr(), nbytes, _stream(wq))
    _lib.check("qmm_gemv_argmax", status)
    return ids, logits


def qmm_gemv_argmax_noalloc(wq, scales, biases, x, ids, logits=None):
    """qmm_gemv_argmax for callers that cannot allocate: the caller passes every
    output (ids [B] int32/uint32, logits [B][N] fp32 or None to skip them); the
    library keeps the per-workgroup records in a static device array of its
    own (1 MiB per GPU), so nothing is allocated at any level.  Calls that
    overlap on one GPU race (one static array per GPU).  Returns ids."""
    torch = _torch()
    N, K = _check_qmm(wq, scales, biases, x)
    rows = x.shape[0]
    if not 1 <= rows <= MAX_GEMV_BATCH:
        raise ValueError(f"qmm_gemv_argmax_noalloc takes 1..{MAX_GEMV_BATCH} rows")
    _need(ids, "ids", (torch.int32, torch.uint32), 1, wq.device)
    if ids.shape[0] != rows:
        raise ValueError("ids must have one entry per row")
    if logits is not None:
        _need(logits, "logits", (torch.float32,), 2, wq.device)
        if tuple(logits.shape) != (rows, N):
            raise ValueError(f"logits must be [{rows}][{N}]")
    status = _lib.load().qmm_gemv_argmax_noalloc(
        wq.data_ptr(), scales.data_ptr(), biases.data_ptr(), x.data_ptr(),
        logits.data_ptr() if logits is not None else None, ids.data_ptr(), rows, N, K, _stream(wq))
    _lib.check("qmm_gemv_argmax_noalloc", status)
    return ids


def vocab_argmax(logits, ids=None, workspace=None, vocab=None):
    """Greedy ids [rows] (int32 tensor holding uint32 bits; 0xFFFFFFFF = non-finite row)."""
    torch = _torch()
    _need(logits, "logits", (torch.float32, torch.bfloat16), 2, None)
    rows, ld = logits.shape
    vocab = ld if vocab is None else vocab
    dtype = F32 if logits.dtype == torch.float32 else BF16
    if ids is None:
        ids = torch.empty(rows, dtype=torch.int32, device=logits.device)
    _need(ids, "ids", (torch.int32, torch.uint32), 1, logits.device)
    if ids.shape[0] != rows:
        raise ValueError("ids must have one entry per row")
    ws, nbytes = _workspace(OP_ARGMAX, rows, vocab, 0, logits.device, workspace)
    lib = _lib.load()
    status = lib.vocab_argmax(logits.data_ptr(), dtype, rows, vocab, ld, ids.data_ptr(),
                              ws.data_ptr(), nbytes, _stream(logits))
    _lib.check("vocab_argmax", status)
    return ids


def vocab_argmax_top2(logits, ids2=None, gaps=None, workspace=None, vocab=None):
    """Winner and runner-up per row and their gap: returns (ids2 [rows][2] int32
    holding uint32 bits, gaps [rows] fp32); a non-finite row gives the sentinel
    twice and a NaN gap."""
    torch = _torch()
    _need(logits, "logits", (torch.float32, torch.bfloat16), 2, None)
    rows, ld = logits.shape
    vocab = ld if vocab is None else vocab
    dtype = F32 if logits.dtype == torch.float32 else BF16
    if ids2 is None:
        ids2 = torch.empty((rows, 2), dtype=torch.int32, device=logits.device)
    if gaps is None:
        gaps = torch.empty(rows, dtype=torch.float32, device=logits.device)
    _need(ids2, "ids2", (torch.int32, torch.uint32), 2, logits.device)
    _need(gaps, "gaps", (torch.float32,), 1, logits.device)
    if tuple(ids2.shape) != (rows, 2) or gaps.shape[0] != rows:
        raise ValueError("ids2 must be [rows][2] and gaps [rows]")
    ws, nbytes = _workspace(OP_ARGMAX_TOP2, rows, vocab, 0, logits.device, workspace)
    lib = _lib.load()
    status = lib.vocab_argmax_top2(logits.data_ptr(), dtype, rows, vocab, ld, ids2.data_ptr(),
                                   gaps.data_ptr(), ws.data_ptr(), nbytes, _stream(logits))
    _lib.check("vocab_argmax_top2", status)
    return ids2, gaps
