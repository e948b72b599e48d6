"""Helpers for the GPU tests: upload seeded numpy inputs, compare with the oracle."""
import numpy as np

TOL = 2e-3        # the parity bar: per-row normwise relative error against the oracle
TIGHT = 2e-5      # the accuracy the fp32 paths are expected to reach (derived in the design notes)


def torch_mod():
    import torch
    return torch


def dev():
    return torch_mod().device("cuda:0")


def up_u32(a):
    torch = torch_mod()
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int32)).to(dev())


def up_bf16(a):
    torch = torch_mod()
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev()).view(torch.bfloat16)


def up_f32(a):
    torch = torch_mod()
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev())


def down(t):
    torch = torch_mod()
    torch.cuda.synchronize()
    return t.cpu().numpy()


def ids_down(t):
    return down(t).view(np.uint32)


def normwise(y, ref):
    """max over rows of max|y - ref| / max|ref| (rows with ref == 0 use absolute error)."""
    y = np.asarray(y, np.float64)
    ref = np.asarray(ref, np.float64)
    num = np.max(np.abs(y - ref), axis=1)
    den = np.max(np.abs(ref), axis=1)
    den = np.where(den == 0, 1.0, den)
    return float(np.max(num / den))


def assert_close(y, ref, what, tol=TOL, tight=TIGHT):
    assert y.shape == ref.shape, (y.shape, ref.shape)
    assert np.all(np.isfinite(y)), f"{what}: non-finite output"
    e = normwise(y, ref)
    assert e <= tol, f"{what}: normwise error {e:.3e} > bar {tol:.1e}"
    assert e <= tight, f"{what}: normwise error {e:.3e} > expected fp32 accuracy {tight:.1e}"
    return e
