"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

The oracle (plain C) is rebuilt with both sanitizers and runs every pin; the
library's C ABI is rebuilt with both sanitizers on its host code (the GPU
code is untouched) and runs every argument-validation check of the ABI tests.
Each runs in a child process with the sanitizer runtime preloaded (the Python
interpreter itself is not instrumented) and must finish cleanly: any
sanitizer report fails the test."""
import glob
import os
import shutil
import subprocess
import sys

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
TESTS = os.path.join(ROOT, "tests")
BUILD = os.path.join(ROOT, "w4_gemv_greedy_amd", "_build")
REPORTS = ("ERROR: AddressSanitizer", "runtime error:", "ERROR: LeakSanitizer")


def _run(code, preload):
    env = dict(os.environ, LD_PRELOAD=preload, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", PYTHONPATH=f"{ROOT}:{TESTS}")
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, env=env, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0 and not any(m in out for m in REPORTS), out[-4000:]
    return out


def test_oracle_pins_under_sanitizers(tmp_path):
    lib = oracle.build(out=str(tmp_path / "liboracle_san.so"), sanitize=True)
    asan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    if not os.path.isabs(asan):
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    out = _run("import oracle, pins\n"
               f"lib = oracle.load({lib!r})\n"
               "[p(lib) for p in pins.ALL_PINS]\n"
               "print('pins', len(pins.ALL_PINS))\n", asan)
    assert "pins" in out


def test_abi_validation_under_sanitizers(tmp_path):
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    objs = [os.path.join(BUILD, f) for f in ("gemv.o", "gemv_mfma.o", "gemm.o", "argmax.o")]
    rts = sorted(glob.glob("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not shutil.which(hipcc) and not os.path.exists(hipcc):
        pytest.skip("hipcc is not available")
    if not all(os.path.exists(o) for o in objs) or not rts:
        pytest.skip("the library's objects (built by build()) or clang's sanitizer runtime are missing")
    src = os.path.join(ROOT, "w4_gemv_greedy_amd", "csrc", "abi.hip")
    obj, so = str(tmp_path / "abi_san.o"), str(tmp_path / "libw4g_san.so")
    # sanitizers on the host code only: each -fsanitize flag goes to the host pass
    host_san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                "-Xarch_host", "-fno-omit-frame-pointer"]
    subprocess.run([hipcc, "-O1", "-g", "-std=c++17", "-fPIC", "--offload-arch=gfx950", "-Wno-unused-result"]
                   + host_san + ["-c", src, "-o", obj], check=True, capture_output=True)
    subprocess.run([hipcc, "-shared", "-fPIC", "--offload-arch=gfx950"] + host_san + [obj] + objs + ["-o", so],
                   check=True, capture_output=True)
    out = _run("import inspect\n"
               "from w4_gemv_greedy_amd import _lib\n"
               f"lib = _lib.load({so!r})\n"
               "import test_abi_cpu as t\n"
               "n = 0\n"
               "for name in dir(t):\n"
               "    f = getattr(t, name)\n"
               "    if name.startswith('test_') and list(inspect.signature(f).parameters) == ['lib']:\n"
               "        f(lib); n += 1\n"
               "print('abi checks', n)\n", rts[-1])
    assert "abi checks" in out
