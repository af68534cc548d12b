"""Build the HIP library (libtaco.so) in-tree for gfx950 with hipcc.

    python -m quantized_compression_tensor_amd.build

Every call recompiles all sources. The result lands in
``quantized_compression_tensor_amd/lib/libtaco.so`` (written atomically).
"""

import os
import shutil
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIBDIR = os.path.join(PKG, "lib")
LIB = os.path.join(LIBDIR, "libtaco.so")

SOURCES = ["taco_abi.hip", "fp8_hadamard.hip", "codecs.hip", "reorder.hip", "dequant_gemm.hip"]
ARCH = "gfx950"

# -ffp-contract=off: no fused multiply-adds except the explicit fmaf calls,
# so every product and sum rounds once, as the codec definitions require.
# Correctly rounded float32 division; float32 denormals kept.
# Packed FP32 instructions are switched off. Atomics stay as written (every
# one is issued by a single lane): the wave-aggregating rewrite would consume
# an atomic's result right after issuing it, so the wave would wait for the
# round trip before issuing the loads that follow.
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-ffp-contract=off", "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-fno-gpu-flush-denormals-to-zero",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-mllvm", "-amdgpu-atomic-optimizer-strategy=None",
    "-Wno-unused-command-line-argument",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def hipcc():
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def _run(cmd):
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in p.stdout.splitlines() if "is not a recognized feature" not in l)
    if p.returncode != 0:
        raise RuntimeError("command failed: " + " ".join(cmd) + "\n" + out)
    return out


def build(verbose=False, extra_flags=(), out=None):
    cc = hipcc()
    os.makedirs(LIBDIR, exist_ok=True)
    with tempfile.TemporaryDirectory(dir=LIBDIR) as tmp:
        def compile_one(src):
            obj = os.path.join(tmp, src.replace(".hip", ".o"))
            _run([cc, *FLAGS, *extra_flags, "-c", os.path.join(CSRC, src), "-o", obj])
            return obj
        with ThreadPoolExecutor(len(SOURCES)) as ex:
            objs = list(ex.map(compile_one, SOURCES))
        tmp_lib = os.path.join(tmp, "libtaco.so")
        _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp_lib])
        os.replace(tmp_lib, out or LIB)
    if verbose:
        print("built", out or LIB)
    return out or LIB


if __name__ == "__main__":
    build(verbose=True, extra_flags=sys.argv[1:])
