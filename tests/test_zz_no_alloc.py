"""The no-allocation fused head (qmm_gemv_argmax_noalloc), called through the
C ABI: its logits and ids equal those of qmm_gemv_argmax (the entry point it
is a variant of) bit for bit, on two calls in a row, the second smaller, so a
call never reads what the one before it left in the library's static scratch."""
import ctypes

import numpy as np
import pytest

from gpu_util import down, ids_down, up_bf16, up_u32
from w4_gemv_greedy_amd import _lib, synth

pytestmark = pytest.mark.gpu


def _call_noalloc(lib, W, X, logits, ids, B, N, K):
    import torch
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    st = lib.qmm_gemv_argmax_noalloc(W[0].data_ptr(), W[1].data_ptr(), W[2].data_ptr(), X.data_ptr(),
                                     logits.data_ptr() if logits is not None else None, ids.data_ptr(),
                                     B, N, K, stream)
    assert st == _lib.OK, lib.w4g_status_string(st)


@pytest.mark.parametrize("first,second", [((8, 248320, 5120), (1, 248320, 5120)),   # the vocabulary head
                                          ((8, 5120, 17408), (3, 4099, 1088)),      # x in registers, then LDS
                                          ((1, 40000, 8192), (1, 777, 64))])
def test_noalloc_head_matches_workspace_head(first, second):
    import torch
    import w4_gemv_greedy_amd as w4g
    lib = _lib.load()
    for i, (B, N, K) in enumerate((first, second)):
        wq, sc, bi = synth.weights(N, K, workload=90 + i)
        x = synth.activations(B, K, workload=90 + i)
        W = (up_u32(wq), up_bf16(sc), up_bf16(bi))
        X = up_bf16(x)
        ids_ref, lg_ref = w4g.qmm_gemv_argmax(*W, X)
        ids = torch.full((B,), -1, dtype=torch.int32, device=X.device)
        lg = torch.full((B, N), float("nan"), dtype=torch.float32, device=X.device)
        _call_noalloc(lib, W, X, lg, ids, B, N, K)
        assert np.array_equal(ids_down(ids), ids_down(ids_ref)), f"call {i}: ids differ"
        assert np.array_equal(down(lg).view(np.uint32), down(lg_ref).view(np.uint32)), f"call {i}: logits differ"
        ids2 = torch.full((B,), -1, dtype=torch.int32, device=X.device)
        _call_noalloc(lib, W, X, None, ids2, B, N, K)  # ids only
        assert np.array_equal(ids_down(ids2), ids_down(ids_ref)), f"call {i}: ids-only call differs"
        ids3 = w4g.qmm_gemv_argmax_noalloc(*W, X, torch.empty(B, dtype=torch.int32, device=X.device))
        assert np.array_equal(ids_down(ids3), ids_down(ids_ref)), f"call {i}: binding differs"
