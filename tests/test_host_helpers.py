"""The reorder kernels' host-side index arithmetic (taco_internal.h), built
with hipcc and run on the CPU by tests/host_helpers.cpp: the span-row
division by a multiply is exact over every span index a tensor can have, and
the staged-unit rule gives whole tiles within the largest unit and the LDS a
CU has."""

import os
import subprocess
import tempfile

import pytest

from tests.conftest import ROOT

HIPCC = "/opt/rocm/bin/hipcc"


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not installed")
def test_reorder_index_arithmetic_on_the_host():
    csrc = os.path.join(ROOT, "quantized_compression_tensor_amd", "csrc")
    with tempfile.TemporaryDirectory() as tmp:
        exe = os.path.join(tmp, "host_helpers")
        b = subprocess.run([HIPCC, "--offload-arch=gfx950", "-O2", "-std=c++17", "-x", "hip",
                            f"-I{os.path.join(ROOT, 'include')}", f"-I{csrc}",
                            os.path.join(ROOT, "tests", "host_helpers.cpp"), "-o", exe],
                           capture_output=True, text=True, timeout=600)
        assert b.returncode == 0, b.stdout[-3000:] + b.stderr[-3000:]
        r = subprocess.run([exe], capture_output=True, text=True, timeout=300,
                           env=dict(os.environ, HIP_VISIBLE_DEVICES=""))
        assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
        assert "every staged width checked" in r.stdout
