"""The C ABI on the CPU: the library loads, exports every function the header
declares, agrees with the binding's constants, and rejects bad arguments with
the documented status before any HIP call (no GPU is touched here)."""
import ctypes
import os
import re
import subprocess

import pytest

from w4_gemv_greedy_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "w4g.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        from w4_gemv_greedy_amd import build
        build.build(quiet=True)
    return _lib.load()


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\**(\w+)\(", text, flags=re.M)))


def test_exports_every_declared_function(lib):
    names = _declared_functions()
    assert set(names) >= {"qmm_gemv", "qmm_gemv_ex", "qmm_gemv_bits", "qmm_gemm", "qmm_gemm_ex", "qmm_gemv_argmax", "vocab_argmax",
                          "vocab_argmax_top2",
                          "qmm_workspace_bytes", "w4g_status_string", "w4g_abi_version"}
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if line.strip()}
    missing = [n for n in names if n not in exported]
    assert not missing, f"declared but not exported: {missing}"
    for n in names:
        getattr(lib, n)


def test_constants_match_header(lib):
    defs = dict(re.findall(r"#define\s+(W4G_\w+)\s+(\S+)", open(HEADER).read()))
    val = lambda k: int(defs[k].rstrip("u"), 0)
    assert val("W4G_ABI_VERSION") == _lib.ABI_VERSION == lib.w4g_abi_version()
    assert val("W4G_SENTINEL") == _lib.SENTINEL
    assert val("W4G_MAX_GEMV_BATCH") == _lib.MAX_GEMV_BATCH
    for k, v in (("W4G_OK", _lib.OK), ("W4G_EINVAL_PTR", _lib.EINVAL_PTR), ("W4G_ESHAPE", _lib.ESHAPE),
                 ("W4G_EALIGN", _lib.EALIGN), ("W4G_EWORKSPACE", _lib.EWORKSPACE),
                 ("W4G_EDTYPE", _lib.EDTYPE), ("W4G_ELAUNCH", _lib.ELAUNCH), ("W4G_EALIAS", _lib.EALIAS),
                 ("W4G_ESCRATCH", _lib.ESCRATCH),
                 ("W4G_F32", _lib.F32), ("W4G_BF16", _lib.BF16), ("W4G_OP_GEMV", _lib.OP_GEMV),
                 ("W4G_OP_GEMM", _lib.OP_GEMM), ("W4G_OP_ARGMAX", _lib.OP_ARGMAX),
                 ("W4G_OP_GEMV_ARGMAX", _lib.OP_GEMV_ARGMAX), ("W4G_OP_ARGMAX_TOP2", _lib.OP_ARGMAX_TOP2),
                 ("W4G_OP_GEMV_BITS_ARGMAX", _lib.OP_GEMV_BITS_ARGMAX),
                 ("W4G_GEMV_AUTO", _lib.GEMV_AUTO), ("W4G_GEMV_VALU", _lib.GEMV_VALU),
                 ("W4G_GEMV_MFMA", _lib.GEMV_MFMA), ("W4G_GEMV_VALU_REGS", _lib.GEMV_VALU_REGS)):
        assert val(k) == v, k


def test_status_strings(lib):
    for s in range(9):
        msg = lib.w4g_status_string(s)
        assert msg and msg != b"unknown status"
    assert lib.w4g_status_string(99) == b"unknown status"


# fake but aligned, distinct device addresses: validation never dereferences them
A = 1 << 40
WQ, SC, BI, X, Y, WS, LOG, IDS = (A + i * (1 << 36) for i in range(8))


def gemv(lib, wq=WQ, sc=SC, bi=BI, x=X, y=Y, B=1, N=64, K=128, ws=None, wsb=0, kernel=None, whole=0):
    if kernel is None:
        return lib.qmm_gemv(wq, sc, bi, x, y, B, N, K, ws, wsb, None)
    return lib.qmm_gemv_ex(wq, sc, bi, x, y, B, N, K, ws, wsb, None, kernel, whole)


def test_gemv_rejects(lib):
    assert gemv(lib, wq=None) == _lib.EINVAL_PTR
    assert gemv(lib, y=None) == _lib.EINVAL_PTR
    assert gemv(lib, B=0) == _lib.ESHAPE
    assert gemv(lib, B=9) == _lib.ESHAPE
    assert gemv(lib, N=0) == _lib.ESHAPE
    assert gemv(lib, K=96) == _lib.ESHAPE
    assert gemv(lib, K=0) == _lib.ESHAPE
    assert gemv(lib, K=1 << 31) == _lib.ESHAPE
    assert gemv(lib, wq=WQ + 4) == _lib.EALIGN
    assert gemv(lib, x=X + 8) == _lib.EALIGN
    assert gemv(lib, y=Y + 4) == _lib.EALIGN
    assert gemv(lib, sc=SC + 1) == _lib.EALIGN
    # y overlapping x, the codes, or the scales
    assert gemv(lib, y=X) == _lib.EALIAS
    assert gemv(lib, y=WQ + 64) == _lib.EALIAS
    assert gemv(lib, y=SC) == _lib.EALIAS
    assert gemv(lib, kernel=5) == _lib.EDTYPE
    assert gemv(lib, kernel=7) == _lib.EDTYPE
    assert gemv(lib, kernel=-1) == _lib.EDTYPE
    # the whole matrix has at least the call's rows, and fewer than 2^31
    assert gemv(lib, kernel=0, whole=63) == _lib.ESHAPE
    assert gemv(lib, kernel=0, whole=-1) == _lib.ESHAPE
    assert gemv(lib, kernel=1, whole=1 << 31) == _lib.ESHAPE


def test_gemv_bits_rejects(lib):
    call = lambda **k: lib.qmm_gemv_bits(k.get("wq", WQ), SC, BI, X, k.get("y", Y), k.get("B", 1),
                                         k.get("N", 64), k.get("K", 128), k.get("bits", 8), None, 0, None)
    assert call(bits=3) == _lib.EDTYPE
    assert call(bits=16) == _lib.EDTYPE
    assert call(wq=None) == _lib.EINVAL_PTR
    assert call(B=0) == _lib.ESHAPE
    assert call(B=9) == _lib.ESHAPE
    assert call(K=96) == _lib.ESHAPE
    assert call(wq=WQ + 4) == _lib.EALIGN
    assert call(y=X) == _lib.EALIAS
    # an 8-bit table is twice a 4-bit one: y just past the 4-bit extent still overlaps it
    assert call(y=WQ + 64 * (128 // 8) * 4) == _lib.EALIAS
    assert call(bits=2, y=WQ + 64 * (128 // 16) * 4 - 16) == _lib.EALIAS
    # one row of x must fit in LDS at widths other than 4 (2.125 * K bytes <= 152 KiB:
    # K up to 72 chunks of 1024 less one, 72,704); larger batches run in parts
    assert call(K=73728) == _lib.ESHAPE
    assert call(bits=2, B=8, K=73728) == _lib.ESHAPE


def test_gemm_rejects(lib):
    need = lib.qmm_workspace_bytes(_lib.OP_GEMM, 16, 64, 128)
    assert 0 < need < (1 << 20)
    call = lambda **k: lib.qmm_gemm(k.get("wq", WQ), SC, BI, X, k.get("y", Y), k.get("M", 16), 64,
                                    k.get("K", 128), k.get("ws", WS), k.get("wsb", need), None)
    assert call(wq=None) == _lib.EINVAL_PTR
    assert call(M=0) == _lib.ESHAPE
    assert call(K=100) == _lib.ESHAPE
    assert call(ws=None) == _lib.EWORKSPACE
    assert call(wsb=need - 1) == _lib.EWORKSPACE
    assert call(ws=WS + 8) == _lib.EALIGN
    assert call(ws=X) == _lib.EALIAS
    assert call(y=WS) == _lib.EALIAS
    ex = lambda **k: lib.qmm_gemm_ex(WQ, SC, BI, X, k.get("y", Y), 16, 64, 128, WS, need, None,
                                     k.get("dt", _lib.BF16))
    assert ex(dt=2) == _lib.EDTYPE
    assert ex(dt=-1) == _lib.EDTYPE
    assert ex(y=None) == _lib.EINVAL_PTR
    assert ex(y=Y + 2) == _lib.EALIGN
    assert ex(y=WS) == _lib.EALIAS
    assert ex(y=X + 16 * 128 * 2 - 16) == _lib.EALIAS   # the last bytes of x


def test_argmax_rejects(lib):
    need = lib.qmm_workspace_bytes(_lib.OP_ARGMAX, 2, 5000, 0)
    assert need == 2 * 5 * 8
    call = lambda **k: lib.vocab_argmax(k.get("lg", LOG), k.get("dt", _lib.F32), k.get("rows", 2),
                                        k.get("V", 5000), k.get("ld", 5000), k.get("ids", IDS),
                                        k.get("ws", WS), k.get("wsb", need), None)
    assert call(lg=None) == _lib.EINVAL_PTR
    assert call(ids=None) == _lib.EINVAL_PTR
    assert call(dt=2) == _lib.EDTYPE
    assert call(rows=0) == _lib.ESHAPE
    assert call(rows=65536) == _lib.ESHAPE
    assert call(V=0) == _lib.ESHAPE
    assert call(V=1 << 31, ld=1 << 31) == _lib.ESHAPE
    assert call(ld=4999) == _lib.ESHAPE
    assert call(lg=LOG + 4) == _lib.EALIGN
    assert call(ids=IDS + 2) == _lib.EALIGN
    assert call(ws=WS + 4) == _lib.EALIGN
    assert call(ws=None) == _lib.EWORKSPACE
    assert call(wsb=need - 8) == _lib.EWORKSPACE
    assert call(ids=LOG + 64) == _lib.EALIAS
    assert call(ws=LOG) == _lib.EALIAS


def test_gemv_argmax_rejects(lib):
    need = lib.qmm_workspace_bytes(_lib.OP_GEMV_ARGMAX, 2, 5000, 1024)
    assert need > 0 and need % 16 == 0
    call = lambda **k: lib.qmm_gemv_argmax(k.get("wq", WQ), SC, BI, X, k.get("lg", Y),
                                           k.get("ids", IDS), k.get("B", 2), k.get("N", 5000),
                                           k.get("K", 1024), k.get("ws", WS), k.get("wsb", need), None)
    assert call(wq=None) == _lib.EINVAL_PTR
    assert call(ids=None) == _lib.EINVAL_PTR
    assert call(B=0) == _lib.ESHAPE
    assert call(B=9) == _lib.ESHAPE
    assert call(K=1000) == _lib.ESHAPE
    assert call(N=1 << 31) == _lib.ESHAPE
    assert call(lg=Y + 4) == _lib.EALIGN
    assert call(ids=IDS + 2) == _lib.EALIGN
    assert call(ws=WS + 4) == _lib.EALIGN
    assert call(ws=None) == _lib.EWORKSPACE
    assert call(wsb=need - 8) == _lib.EWORKSPACE
    assert call(lg=X) == _lib.EALIAS
    assert call(ids=WQ + 64) == _lib.EALIAS
    assert call(ws=Y) == _lib.EALIAS
    assert call(ids=WS) == _lib.EALIAS


def test_gemv_bits_argmax_rejects(lib):
    """The fused head at 2 and 8 bits validates like qmm_gemv_argmax, with the
    code table sized by the width, and refuses widths other than 2, 4, 8 and K
    whose one row of x does not fit in LDS, all before any HIP call."""
    need = lib.qmm_workspace_bytes(_lib.OP_GEMV_BITS_ARGMAX, 2, 5000, 1024)
    assert need > 0 and need % 16 == 0
    call = lambda **k: lib.qmm_gemv_bits_argmax(k.get("wq", WQ), SC, BI, X, k.get("lg", Y),
                                                k.get("ids", IDS), k.get("B", 2), k.get("N", 5000),
                                                k.get("K", 1024), k.get("bits", 8), k.get("ws", WS),
                                                k.get("wsb", need), None)
    for bits in (0, 1, 3, 16):
        assert call(bits=bits) == _lib.EDTYPE
    assert call(wq=None) == _lib.EINVAL_PTR
    assert call(ids=None) == _lib.EINVAL_PTR
    assert call(B=0) == _lib.ESHAPE
    assert call(B=9) == _lib.ESHAPE
    assert call(K=1000) == _lib.ESHAPE
    assert call(K=80000) == _lib.ESHAPE  # one row of x (80,000 activations) exceeds LDS
    assert call(lg=Y + 4) == _lib.EALIGN
    assert call(ids=IDS + 2) == _lib.EALIGN
    assert call(ws=WS + 4) == _lib.EALIGN
    assert call(ws=None) == _lib.EWORKSPACE
    assert call(wsb=need - 8) == _lib.EWORKSPACE
    assert call(lg=X) == _lib.EALIAS
    assert call(ws=Y) == _lib.EALIAS
    # the code table of 5000 rows x 1024 codes: 5,120,000 bytes at 8 bits, 1,280,000 at 2
    assert call(ids=WQ + 5_000_000) == _lib.EALIAS
    assert call(bits=2, ids=WQ + 1_279_996) == _lib.EALIAS


def test_gemv_argmax_noalloc_rejects(lib):
    """The no-allocation head validates like qmm_gemv_argmax, and refuses sizes
    whose records exceed its 1 MiB static scratch, all before any HIP call."""
    call = lambda **k: lib.qmm_gemv_argmax_noalloc(k.get("wq", WQ), SC, BI, X, k.get("lg", Y),
                                                   k.get("ids", IDS), k.get("B", 2), k.get("N", 5000),
                                                   k.get("K", 1024), None)
    assert call(wq=None) == _lib.EINVAL_PTR
    assert call(ids=None) == _lib.EINVAL_PTR
    assert call(B=0) == _lib.ESHAPE
    assert call(B=9) == _lib.ESHAPE
    assert call(K=1000) == _lib.ESHAPE
    assert call(lg=Y + 4) == _lib.EALIGN
    assert call(ids=IDS + 2) == _lib.EALIGN
    assert call(lg=X) == _lib.EALIAS
    assert call(ids=WQ + 64) == _lib.EALIAS
    # records beyond 131,072: the B = 1 head in 32-row workgroups above 4.19 M rows,
    # and x staged in registers (4 rows per workgroup: K = 40,960 holds one row of
    # x in LDS, not two) at B = 8 over 600,000 rows
    assert lib.qmm_workspace_bytes(_lib.OP_GEMV_ARGMAX, 1, 5_000_000, 64) > (1 << 20)
    assert call(B=1, N=5_000_000, K=64) == _lib.ESCRATCH
    assert call(B=8, N=600_000, K=40960) == _lib.ESCRATCH
    # the full vocabulary head fits at every batch size
    for B in range(1, 9):
        assert lib.qmm_workspace_bytes(_lib.OP_GEMV_ARGMAX, B, 248320, 5120) <= (1 << 20)


def test_top2_rejects(lib):
    need = lib.qmm_workspace_bytes(_lib.OP_ARGMAX_TOP2, 2, 5000, 0)
    assert need == 2 * 5 * 16
    assert lib.qmm_workspace_bytes(_lib.OP_ARGMAX_TOP2, 2, 1, 0) == ctypes.c_size_t(-1).value
    GP = IDS + (1 << 20)
    call = lambda **k: lib.vocab_argmax_top2(k.get("lg", LOG), k.get("dt", _lib.F32), k.get("rows", 2),
                                             k.get("V", 5000), k.get("ld", 5000), k.get("ids", IDS),
                                             k.get("gp", GP), k.get("ws", WS), k.get("wsb", need), None)
    assert call(gp=None) == _lib.EINVAL_PTR
    assert call(dt=3) == _lib.EDTYPE
    assert call(V=1, ld=1) == _lib.ESHAPE
    assert call(gp=GP + 2) == _lib.EALIGN
    assert call(ws=WS + 8) == _lib.EALIGN
    assert call(wsb=need - 16) == _lib.EWORKSPACE
    assert call(gp=IDS + 8) == _lib.EALIAS
    assert call(ws=LOG) == _lib.EALIAS


def test_workspace_sizes(lib):
    size_max = ctypes.c_size_t(-1).value
    assert lib.qmm_workspace_bytes(_lib.OP_GEMV, 8, 5120, 5120) == 0
    assert lib.qmm_workspace_bytes(_lib.OP_GEMV, 9, 5120, 5120) == size_max
    assert lib.qmm_workspace_bytes(_lib.OP_GEMM, 512, 5120, 5120) == 512 * 5120 * 2 + 512 * 3 * 80 * 2
    assert lib.qmm_workspace_bytes(_lib.OP_GEMM, 512, 5120, 17408) == 512 * 17408 * 2 + 512 * 3 * 272 * 2
    assert lib.qmm_workspace_bytes(_lib.OP_ARGMAX, 1, 248320, 0) == 243 * 8
    # fused head: one record per product workgroup and batch row, in the layout
    # of qmm_gemv's own choice, the vector-ALU family for every shape: 32 rows
    # per workgroup for the vocabulary-wide head at B = 1, one workgroup per CU
    # where x fits in LDS, also where a batch too large for it is cut into parts
    # that fit, one per CU share of at most 24 rows for the step-staged kernel
    # (o_proj and down from B = 3), 4 rows per 64-lane workgroup where not even
    # two rows of x fit (x staged in registers)
    assert lib.qmm_workspace_bytes(_lib.OP_GEMV_ARGMAX, 1, 248320, 5120) == 7760 * 8
    assert lib.qmm_workspace_bytes(_lib.OP_GEMV_ARGMAX, 1, 5120, 5120) == 256 * 8
    assert lib.qmm_workspace_bytes(_lib.OP_GEMV_ARGMAX, 4, 248320, 5120) == 4 * 256 * 8
    assert lib.qmm_workspace_bytes(_lib.OP_GEMV_ARGMAX, 3, 248320, 5120) == 3 * 256 * 8
    assert lib.qmm_workspace_bytes(_lib.OP_GEMV_ARGMAX, 3, 34816, 5120) == 3 * 256 * 8
    assert lib.qmm_workspace_bytes(_lib.OP_GEMV_ARGMAX, 2, 5120, 17408) == 2 * 256 * 8
    assert lib.qmm_workspace_bytes(_lib.OP_GEMV_ARGMAX, 8, 248320, 5120) == 8 * 256 * 8
    assert lib.qmm_workspace_bytes(_lib.OP_GEMV_ARGMAX, 4, 5120, 17408) == 4 * 256 * 8
    assert lib.qmm_workspace_bytes(_lib.OP_GEMV_ARGMAX, 5, 5120, 17408) == 5 * 256 * 8
    assert lib.qmm_workspace_bytes(_lib.OP_GEMV_ARGMAX, 8, 5120, 17408) == 8 * 256 * 8
    # x too long for LDS over at most 24 rows per CU: the step-staged kernel, one
    # record per CU share (2 rows here); also at B = 1 where x spans 8 chunks or more
    assert lib.qmm_workspace_bytes(_lib.OP_GEMV_ARGMAX, 3, 300, 73728) == 3 * 150 * 8
    assert lib.qmm_workspace_bytes(_lib.OP_GEMV_ARGMAX, 1, 3000, 17408) == 1 * 250 * 8
    assert lib.qmm_workspace_bytes(_lib.OP_GEMV_ARGMAX, 1, 3000, 5120) == 1 * 250 * 8
    assert lib.qmm_workspace_bytes(_lib.OP_GEMV_ARGMAX, 8, 9000, 10240) == 8 * 250 * 8
    assert lib.qmm_workspace_bytes(_lib.OP_GEMV_ARGMAX, 8, 600000, 40960) == 8 * 150000 * 8
    assert lib.qmm_workspace_bytes(_lib.OP_GEMV_ARGMAX, 9, 248320, 5120) == size_max
    # the fused head at 2 and 8 bits: the same layouts (32-row workgroups for the
    # vocabulary-wide head at B = 1, one workgroup per CU share elsewhere, the
    # step-staged kernel over at most 24 rows per CU from B = 3 or where x does
    # not fit); K whose one row of x exceeds LDS is out of range
    assert lib.qmm_workspace_bytes(_lib.OP_GEMV_BITS_ARGMAX, 1, 248320, 5120) == 7760 * 8
    assert lib.qmm_workspace_bytes(_lib.OP_GEMV_BITS_ARGMAX, 8, 248320, 5120) == 8 * 256 * 8
    assert lib.qmm_workspace_bytes(_lib.OP_GEMV_BITS_ARGMAX, 1, 5120, 5120) == 256 * 8
    assert lib.qmm_workspace_bytes(_lib.OP_GEMV_BITS_ARGMAX, 8, 5120, 17408) == 8 * 256 * 8
    assert lib.qmm_workspace_bytes(_lib.OP_GEMV_BITS_ARGMAX, 3, 300, 5120) == 3 * 150 * 8
    assert lib.qmm_workspace_bytes(_lib.OP_GEMV_BITS_ARGMAX, 1, 5120, 80000) == size_max
    assert lib.qmm_workspace_bytes(_lib.OP_GEMV_BITS_ARGMAX, 9, 5120, 5120) == size_max
    assert lib.qmm_workspace_bytes(7, 1, 1, 64) == size_max


def test_binding_fails_loudly_without_library(tmp_path):
    with pytest.raises(RuntimeError, match="missing"):
        _lib.load(str(tmp_path / "libw4g.so"))


def test_binding_checks_a_given_workspace(lib):
    """A caller's workspace is checked like the other tensors before its
    address can reach a kernel: on the inputs' GPU, contiguous, large enough
    (a host tensor would otherwise be read as a device address)."""
    import torch
    import w4_gemv_greedy_amd as w4g
    need = w4g.workspace_bytes(_lib.OP_GEMM, 70, 320, 1088)
    assert need > 0
    with pytest.raises(ValueError, match="same GPU"):
        w4g._workspace(_lib.OP_GEMM, 70, 320, 1088, 0, torch.empty(need, dtype=torch.uint8))
    with pytest.raises(TypeError):
        w4g._workspace(_lib.OP_GEMM, 70, 320, 1088, 0, bytearray(need))
