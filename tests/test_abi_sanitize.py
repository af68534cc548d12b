"""The ABI's host code built with AddressSanitizer and UndefinedBehavior-
Sanitizer (host pass only; the device code is built as usual) and driven by
tests/abi_sanitize.cpp on the CPU: layouts, status strings, the launch cap and
the argument checks, with any sanitizer report failing the test."""

import os
import subprocess
import tempfile

import pytest

from tests.conftest import ROOT

CSRC = os.path.join(ROOT, "quantized_compression_tensor_amd", "csrc")


def _library_sources():
    """The library's source list, from its build script (one list to keep)."""
    import importlib.util
    spec = importlib.util.spec_from_file_location(
        "taco_build", os.path.join(ROOT, "quantized_compression_tensor_amd", "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return list(mod.SOURCES)


SOURCES = _library_sources()
HIPCC = "/opt/rocm/bin/hipcc"


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not installed")
def test_abi_host_code_under_sanitizers():
    from concurrent.futures import ThreadPoolExecutor
    flags = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17",
             "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
             "-ffp-contract=off", "-fhip-fp32-correctly-rounded-divide-sqrt", "-fno-gpu-flush-denormals-to-zero",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wno-unused-command-line-argument", f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}"]
    srcs = [os.path.join(CSRC, s) for s in SOURCES] + [os.path.join(ROOT, "tests", "abi_sanitize.cpp")]
    with tempfile.TemporaryDirectory() as tmp:
        exe = os.path.join(tmp, "abi_sanitize")

        def compile_one(src):
            obj = os.path.join(tmp, os.path.basename(src) + ".o")
            lang = ["-x", "hip"] if src.endswith(".cpp") else []
            return obj, subprocess.run([HIPCC, *flags, *lang, "-c", src, "-o", obj], capture_output=True,
                                       text=True, timeout=600)

        with ThreadPoolExecutor(len(srcs)) as ex:
            built = list(ex.map(compile_one, srcs))
        for obj, b in built:
            assert b.returncode == 0, b.stdout[-3000:] + b.stderr[-3000:]
        b = subprocess.run([HIPCC, "--offload-arch=gfx950", "-Xarch_host", "-fsanitize=address", "-Xarch_host",
                            "-fsanitize=undefined", *[o for o, _ in built], "-o", exe],
                           capture_output=True, text=True, timeout=600)
        assert b.returncode == 0, b.stdout[-3000:] + b.stderr[-3000:]
        env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
                   UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", HIP_VISIBLE_DEVICES="")
        r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
        assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
        assert "all checks passed" in r.stdout
        assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr[-3000:]
