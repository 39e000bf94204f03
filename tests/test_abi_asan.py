"""The C ABI's host code under AddressSanitizer (CPU only).

The library is built a second time with the host side instrumented
(``-fsanitize=address`` on the host compilation only; the gfx950 code is
built as usual), and the CPU checks of ``tests/test_abi.py`` -- every entry
point's argument validation, the route and size queries, the property-based
defect combinations -- run against it in a child process with the sanitizer
runtime preloaded. Any invalid read or write, use after free or buffer
overflow in the validation and host paths aborts the child and fails here.
"""

import glob
import os
import subprocess
import sys

import pytest

from stream_hyper_connections_amd import build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _asan_runtime():
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    hits = sorted(glob.glob(os.path.join(rocm, "llvm", "lib", "clang", "*", "lib", "linux",
                                         "libclang_rt.asan-x86_64.so")))
    return hits[-1] if hits else None


@pytest.mark.timeout(600)
def test_abi_checks_pass_under_address_sanitizer(tmp_path):
    hipcc = build.hipcc()
    runtime = _asan_runtime()
    if not os.path.exists(hipcc) or runtime is None:
        pytest.skip("no hipcc or no sanitizer runtime")
    lib = tmp_path / "libmhc_asan.so"
    cmd = [hipcc, f"--offload-arch={build.ARCH}", "-O1", "-g", "-std=c++17", "-fPIC", "-shared",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-shared-libasan",
           "-Xarch_host", "-fno-omit-frame-pointer", "-I", build.INCLUDE, build.SRC,
           "-o", str(lib)]
    res = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert res.returncode == 0, res.stderr[-2000:]
    env = dict(os.environ, MHC_LIBRARY=str(lib), LD_PRELOAD=runtime,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=1")
    run = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                          os.path.join(ROOT, "tests", "test_abi.py"), "-k", "not c_and_links"],
                         capture_output=True, text=True, timeout=600, cwd=ROOT, env=env)
    out = run.stdout + run.stderr
    assert "AddressSanitizer" not in out, out[-4000:]
    assert run.returncode == 0, out[-4000:]
    assert " passed" in out
