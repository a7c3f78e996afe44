"""Multi-request prefill (rows mapped to per-request page tables) on the GPU
against the CPU oracle, through the C ABI.

Bar as for the other logits tests (max |d| <= 2e-2, rel <= 5e-3, exact -inf
and NaN patterns); equalities between two library paths that run the same
arithmetic are bit-exact.
"""
from __future__ import annotations

import dataclasses
import sys

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from helpers import assert_parity, mask_of

pytestmark = pytest.mark.gpu


def announce(msg: str) -> None:
    sys.__stderr__.write(f"[gpu] {msg}\n")
    sys.__stderr__.flush()


def run(lib, wl) -> np.ndarray:
    announce(f"varlen {wl.key_kind} rows={wl.rows} tables={wl.num_tables} width={wl.table_width} "
             f"({wl.name})")
    dw = W.to_device(wl)
    W.run_library(dw, lib)
    torch.cuda.synchronize()
    return dw.out.cpu().numpy()


@pytest.mark.parametrize("kind", ["fp8", "bf16"])
@pytest.mark.parametrize("interleave", [False, True])
def test_varlen_small(lib, kind, interleave):
    """Requests whose row counts do not fill 4-row blocks (blocks straddle
    requests), causal lengths, one request longer than the others."""
    wl = W.varlen_workload(50 + interleave, kind, tokens=[3, 5, 2, 7], contexts=[700, 64, 1500, 2900],
                           table_width=50, num_pages=300, interleave=interleave)
    got = run(lib, wl)
    st = assert_parity(got, oracle.paged_mqa_logits(wl), mask_of(wl), label=f"varlen {kind}")
    announce(str(st))


@pytest.mark.parametrize("kind", ["fp8", "bf16"])
def test_varlen_matches_expanded_tables_bit_exact(lib, kind):
    """The same rows with each row given a copy of its request's table (the
    per-row-table entry point) give the same bits."""
    wl = W.varlen_workload(52, kind, tokens=[6, 1, 9], contexts=[1200, 300, 2000], table_width=40,
                           num_pages=200)
    tabs = wl.page_table.reshape(wl.num_tables, wl.pt_stride)
    per_row = dataclasses.replace(wl, page_table=tabs[wl.row_table].reshape(-1).copy(), row_table=None,
                                  num_tables=0)
    assert np.array_equal(run(lib, wl).view(np.uint32), run(lib, per_row).view(np.uint32))


def test_varlen_one_request_matches_shared_table_bit_exact(lib):
    wl = W.varlen_workload(53, "bf16", tokens=[37], contexts=[2500], table_width=45, num_pages=100)
    shared = dataclasses.replace(wl, pt_stride=0, row_table=None, num_tables=0)
    assert np.array_equal(run(lib, wl).view(np.uint32), run(lib, shared).view(np.uint32))


def test_varlen_invalid_table_index_gives_nan(lib):
    wl = W.varlen_workload(54, "fp8", tokens=[4, 4], contexts=[500, 900], table_width=20,
                           num_pages=64)
    wl = dataclasses.replace(wl, row_table=wl.row_table.copy())
    wl.row_table[1] = 2      # past the two tables
    wl.row_table[6] = -3
    got = run(lib, wl)
    m = mask_of(wl)
    for b in range(wl.rows):
        bad = b in (1, 6)
        assert np.all(np.isnan(got[b][~m[b]]) == bad) and np.all(np.isneginf(got[b][m[b]]))
    ref = oracle.paged_mqa_logits(wl)
    assert_parity(got, ref, m, label="varlen invalid")


def test_varlen_full_size_sampled(lib):
    """The multi-request prefill of the benchmark: four requests, 4096 rows;
    sampled rows, including both sides of every request boundary."""
    wl = W.varlen_config()
    got = run(lib, wl)
    m = mask_of(wl)
    assert np.array_equal(np.isneginf(got), m) and np.isfinite(got[~m]).all()
    edges = np.flatnonzero(np.diff(wl.row_table)) if wl.rows > 1 else np.array([], dtype=np.int64)
    rows = sorted({0, wl.rows - 1, *edges.tolist(), *(edges + 1).tolist(), 777, 2222})
    ref = oracle.paged_mqa_logits(wl, rows=rows)
    st = assert_parity(got[rows], ref, m[rows], label="varlen full")
    announce(f"rows {rows}: {st}")
