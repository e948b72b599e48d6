"""Host-side checks of bench.py (CPU only): the byte counts behind its GB/s
figures, the traffic field's source check, and its refusal of several GPUs."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402  (module level holds no GPU work)


def _format_bytes(N, K, B):
    # the 4-bit affine group-64 format: half a byte per code, one bf16 scale
    # and one bf16 bias per 64 codes; x is B rows of bf16, y B rows of fp32
    codes = N * K // 2
    tables = 2 * (2 * N * (K // 64))
    return codes + tables + 2 * B * K + 4 * B * N


@pytest.mark.parametrize("N,K", [(5120, 5120), (34816, 5120), (5120, 17408), (248320, 5120)])
@pytest.mark.parametrize("B", [1, 4, 8])
def test_gemv_bytes_follow_the_format(N, K, B):
    assert bench.gemv_bytes(N, K, B) == _format_bytes(N, K, B)


def test_step_bytes_decode_sweep():
    # 16 layers of o_proj, gate-up and down, then the lm_head and the argmax's
    # read of the logits (counted as the two-pass argmax would read them)
    per_layer = _format_bytes(5120, 5120, 1) + _format_bytes(34816, 5120, 1) + _format_bytes(5120, 17408, 1)
    want = 16 * per_layer + _format_bytes(248320, 5120, 1) + 4 * 248320
    assert bench.step_bytes(1) == want == 3_363_338_240
    assert bench.gemv_bytes(34816, 5120, 1) == 100_419_584


def test_counted_traffic_tracks_the_kernel_source(tmp_path, monkeypatch):
    text = open(bench.PROFILE).read()
    # the committed summary matches the committed source
    assert bench.counted_traffic() is not None
    # a changed source voids it
    src = tmp_path / "gemv.hip"
    src.write_bytes(open(bench.GEMV_SRC, "rb").read() + b"\n")
    monkeypatch.setattr(bench, "GEMV_SRC", str(src))
    assert bench.counted_traffic() is None
    # so does a summary without the hash
    prof = tmp_path / "p.txt"
    prof.write_text("\n".join(l for l in text.splitlines() if not l.startswith("source_sha256")))
    monkeypatch.setattr(bench, "PROFILE", str(prof))
    assert bench.counted_traffic() is None


def test_bench_refuses_several_gpus():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""
