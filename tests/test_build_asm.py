"""The gfx950 code of both libraries, compiled to assembly with the build's
flags, holds no scalar-cache writes (scalar stores, scalar atomics, scalar
cache write-back or discard) and no packed fp32 add / multiply / fma
instructions: every store of the kernels goes through the vector memory path,
and fp32 arithmetic is scalar per lane (the build turns packed fp32 off).
CPU only: hipcc cross-compiles for gfx950 without a device."""

import os
import re
import subprocess

import pytest

from stream_hyper_connections_amd import build

SOURCES = [build.SRC, build.PROBE_SRC]
FORBIDDEN = re.compile(r"^\s+(s_store|s_atomic|s_dcache_wb|s_dcache_discard|s_scratch_store|"
                       r"s_buffer_store|v_pk_add_f32|v_pk_mul_f32|v_pk_fma_f32)\b", re.M)


@pytest.mark.parametrize("src", SOURCES, ids=os.path.basename)
def test_device_code_has_no_scalar_stores_or_packed_fp32(src, tmp_path):
    hipcc = build.hipcc()
    if not os.path.exists(hipcc) and hipcc == "hipcc":
        pytest.skip("no hipcc")
    out = tmp_path / "k.s"
    cmd = [hipcc, f"--offload-arch={build.ARCH}", "-O3", "-std=c++17", "-Xclang",
           "-target-feature", "-Xclang", "-packed-fp32-ops", "-I", build.INCLUDE,
           "--cuda-device-only", "-S", src, "-o", str(out)]
    res = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert res.returncode == 0, res.stderr[-2000:]
    text = out.read_text()
    assert "s_endpgm" in text   # kernels were emitted
    bad = FORBIDDEN.findall(text)
    assert not bad, sorted(set(bad))
