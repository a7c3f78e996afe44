"""Host-side checks of the benchmark: the one-GPU rule and the algorithmic
bytes/FLOPs that the roofline numerator uses (no GPU needed)."""
from __future__ import annotations

import json
import subprocess
import sys
from pathlib import Path

import numpy as np

import workloads as W

ROOT = Path(__file__).resolve().parent.parent


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, str(ROOT / "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    msg = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in msg["error"]


def test_algorithmic_work_of_the_decode_workload():
    """Reads: 132 B per live fp8 position (128 codes + 4-byte scale), per row the
    16 KiB query, 256 B of weights and a 4-byte length, 4 B per live page of
    table; writes: 4 B for every output slot (live or -inf); 2*64*128 FLOPs per
    live position.  Counted here from the workload's own lengths."""
    sys.path.insert(0, str(ROOT))
    import bench

    wl = W.config(3)
    L = np.clip(wl.seqlens.astype(np.int64), 0, wl.table_width * W.PAGE)
    live = int(L.sum())
    pages = int(((L + W.PAGE - 1) // W.PAGE).sum())
    reads = live * (W.HEAD_DIM + 4) + wl.rows * (W.NUM_HEADS * W.HEAD_DIM * 2 + W.NUM_HEADS * 4 + 4) + 4 * pages
    writes = wl.rows * wl.table_width * W.PAGE * 4
    flops = 2 * W.NUM_HEADS * W.HEAD_DIM * live
    assert bench.algorithmic_work(wl) == (reads, writes, flops)
    # the figures the benchmark line reports for this workload
    assert (live, pages) == (983136, 15389)
    assert reads + writes == 198025972
