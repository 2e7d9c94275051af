"""The plan's work-block tables on the CPU: tests/table_check.cpp (g++, no HIP) builds them as
ob_plan_create does for every workload's chunking and many random ones, at six block sizes, and checks
what the kernels assume of them (ob_tables.h's check_block_table, which ob_plan_create also runs);
for uniform chunks, the no-allocation kernel's per-block formula must reproduce every block.  It also
checks the chunk groups the compressed step's passes run over (greedy, covering, with each group's
block ranges those of its chunks in both tables; the no-allocation path's uniform groups too)."""
import os
import subprocess
import tempfile

import numpy as np

from adam_ob_compress_amd import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _shapes():
    lines = []
    for w in synth.WORKLOADS.values():
        if w.offsets is not None:
            off = w.chunk_offsets()
            lines.append(f"{w.n} {off.size - 1} " + " ".join(str(int(o)) for o in off))
        elif w.n < (1 << 31):                       # the large uniform ones: geometry below
            lines.append(f"u {w.n} {w.chunk}")
    for n, c in ((1, 64), (63, 64), (64, 64), (65, 64), (1000, 128), (4097, 1024), (100_003, 1 << 14),
                 (17_000_003, 17_000_003), (1_052_772, 1 << 16), (5_000_000, 1 << 14), (300_037, 300_037),
                 (1 << 28, 1 << 20), (1_557_611_200, 1 << 24)):
        lines.append(f"u {n} {c}")
    rng = np.random.default_rng(11)
    for _ in range(40):
        K = int(rng.integers(1, 60))
        sizes = rng.integers(1, 200_000, K) // 64 * 64 + 64
        sizes[-1] = int(rng.integers(1, 100_000))          # the last chunk may be ragged
        off = np.concatenate([[0], np.cumsum(sizes)])
        lines.append(f"{int(off[-1])} {K} " + " ".join(str(int(o)) for o in off))
    return "\n".join(lines) + "\n"


def test_block_tables_hold_what_the_kernels_assume():
    with tempfile.TemporaryDirectory() as d:
        exe = os.path.join(d, "table_check")
        subprocess.run(["g++", "-std=c++17", "-O2", "-Wall", "-Wextra", "-Werror",
                        "-I", os.path.join(ROOT, "adam_ob_compress_amd", "csrc"),
                        os.path.join(ROOT, "tests", "table_check.cpp"), "-o", exe], check=True)
        r = subprocess.run([exe], input=_shapes(), capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr
    assert r.stdout.startswith("table_check ok"), r.stdout
    assert "planted mistakes rejected" in r.stdout and "group sets" in r.stdout
