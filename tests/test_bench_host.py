"""Host-side checks of the bench (no GPU): the one-GPU contract and the
algorithmic bytes its roofline divides by."""

import os
import subprocess
import sys

import pytest

import bench
import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True, timeout=300)
    assert p.returncode == 2
    assert "one GPU" in p.stderr
    assert p.stdout.strip() == ""


# Bytes per element each kernel must move, from the formats: bf16 input 2 B;
# FP8 code 1 B + one int8 exponent per 128; INT8 symmetric 1 B + one float32
# scale per 64; asymmetric codes (INT4: 1/2 B, INT8: 1 B) + a float32 scale and
# a uint8 zero point per 128. A reduce reads N shards and writes one
# re-quantized output (or a float32 sum).
PER_ELEMENT = {
    "taco-tiny": (2 + 1 + 1 / 128, 2 * (1 + 1 / 128) + 4),
    "gpt-tp": (2 + 1 + 1 / 128, 4 * (1 + 1 / 128) + (1 + 1 / 128)),
    "equarx": (2 + 1 + 4 / 64, 8 * (1 + 4 / 64) + (1 + 4 / 64)),
    "flashcomm": (2 + 0.5 + 5 / 128, 8 * (0.5 + 5 / 128) + (1 + 5 / 128)),
    "qwen-tp": (2 + 1 + 1 / 128, 8 * (1 + 1 / 128) + (1 + 1 / 128)),
}


@pytest.mark.parametrize("name", sorted(PER_ELEMENT))
def test_algorithmic_bytes_per_element(name):
    w = W.WORKLOADS[name]
    comp, red = bench.algorithmic_bytes(w)
    want_c, want_r = PER_ELEMENT[name]
    # FP8 buffers also carry a 16-byte tensor-scale header: at most 16 B per
    # shard, far below one part in 10^5 of these sizes
    assert comp == pytest.approx(want_c * w.n, rel=1e-5, abs=16)
    assert red == pytest.approx(want_r * w.n, rel=1e-5, abs=16 * (w.shards + 1))


def test_trace_stats_leave_out_launches_beside_a_gemm(tmp_path):
    """Per-kernel statistics from a kernel trace drop every dispatch that ran at
    the same time as a library GEMM, keep the GEMM's own dispatches, and can
    split a kernel by grid size."""
    import bench
    rows = [("Cijk_gemm", 100, 200, 65536), ("Cijk_gemm", 300, 400, 4096),
            ("taco::k_reduce", 50, 90, 1024),      # before the first GEMM: kept
            ("taco::k_reduce", 150, 170, 1024),    # inside it: dropped
            ("taco::k_reduce", 190, 260, 1024),    # overlaps its end: dropped
            ("taco::k_reduce", 200, 300, 1024),    # touches both ends only: kept
            ("taco::k_reduce", 410, 450, 1024)]    # after the last: kept
    lines = ['"Kernel_Name","Start_Timestamp","End_Timestamp","Grid_Size_X"']
    lines += [f'"{n}",{a},{b},{g}' for n, a, b, g in rows]
    (tmp_path / "run_kernel_trace.csv").write_text("\n".join(lines) + "\n")
    st = bench._trace_stats(str(tmp_path), concurrent_with=("Cijk",))
    assert st["taco::k_reduce"]["Calls"] == 3
    assert st["taco::k_reduce"]["AverageNs"] == (40 + 100 + 40) / 3
    assert st["Cijk_gemm"]["Calls"] == 2
    split = bench._trace_stats(str(tmp_path), concurrent_with=(), by_grid=("Cijk",))
    assert split["Cijk_gemm [grid 65536]"]["Calls"] == 1 and split["Cijk_gemm [grid 4096]"]["Calls"] == 1
    assert split["taco::k_reduce"]["Calls"] == 5


def test_summarize_trace_lists_this_librarys_kernels(tmp_path, monkeypatch):
    """The generic trace summary keeps this library's kernels only (slowest
    first), leaves out launches beside a library GEMM and records the command
    and the kernel-source hash."""
    import bench
    rows = [("Cijk_gemm", 100, 200), ("taco::k_quantize<2>", 0, 30), ("taco::k_quantize<2>", 150, 160),
            ("taco::k_dequantize<2>", 300, 360), ("other_kernel", 400, 500)]
    trace = tmp_path / "trace"
    trace.mkdir()
    lines = ['"Kernel_Name","Start_Timestamp","End_Timestamp"'] + [f'"{n}",{a},{b}' for n, a, b in rows]
    (trace / "run_kernel_trace.csv").write_text("\n".join(lines) + "\n")
    (tmp_path / "profiles").mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "abc123")
    bench.summarize_trace(str(trace), "demo", "the command")
    text = (tmp_path / "profiles" / "kernels_demo_trace.txt").read_text().splitlines()
    assert text[1] == "# command: the command" and text[2] == "source_hash: abc123"
    body = text[4:]
    assert len(body) == 2 and "k_dequantize" in body[0] and "k_quantize" in body[1]
    assert body[1].split()[0] == "1"      # the launch beside the GEMM is left out
    assert float(body[0].split()[1]) == 0.06
