"""The C ABI's host-side validation layer under AddressSanitizer and
UndefinedBehaviorSanitizer, on the CPU: api.hip is compiled with both sanitizers on its
host pass only (device code is unchanged), linked with the library's other objects into
a separate copy, and tests/test_boundary.py runs against that copy in a subprocess with
the sanitizer runtime preloaded; any report aborts the run.  Skipped where hipcc or the
runtime is missing."""
import glob
import os
import subprocess
import sys

import pytest

from ternary_weight_linear_token_amd import build as bw_build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def asan_runtime():
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


def test_boundary_under_host_sanitizers(tmp_path):
    rt = asan_runtime()
    if not os.path.exists(bw_build.HIPCC) or rt is None:
        pytest.skip("hipcc or the sanitizer runtime is not installed")
    if not bw_build.is_current():
        bw_build.build()
    api = os.path.join(bw_build.CSRC, "api.hip")
    others = [os.path.join(bw_build.BUILD_DIR, os.path.basename(s) + ".o")
              for s in bw_build.sources() if s.endswith(".hip") and s != api]
    assert all(os.path.exists(o) for o in others)
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-omit-frame-pointer"]
    obj = str(tmp_path / "api_san.o")
    lib = str(tmp_path / "libbitnet_w2a8_san.so")
    flags = [f for f in bw_build.FLAGS if f != "-O3"] + ["-O1", "-g"]
    subprocess.run([bw_build.HIPCC] + flags + san + ["-c", api, "-o", obj], check=True,
                   capture_output=True)
    subprocess.run([bw_build.HIPCC, f"--offload-arch={bw_build.ARCH}", "-shared", "-fPIC"] + san +
                   ["-o", lib, obj] + others, check=True, capture_output=True)
    env = dict(os.environ, BITNET_LIBRARY=lib, LD_PRELOAD=rt,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                          os.path.join(ROOT, "tests", "test_boundary.py")],
                         cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert res.returncode == 0, res.stdout[-3000:] + res.stderr[-3000:]
    assert "passed" in res.stdout
