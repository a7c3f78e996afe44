"""Top-k over logits rows on the GPU against the CPU oracle, through the C ABI.

The selection itself is integer work: given the same float32 logits, the
library's indices must equal the oracle's exactly (ties by lower position,
+0 equal to -0, NaN last) and the returned values must be the selected logits
bit for bit.  For the fused call (logits, then top-k) the logits are also
compared with the oracle's float64 logits: an index may differ from the
oracle's selection only where the oracle's values of both positions lie within
the logits tolerance of the oracle's k-th value.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from helpers import ATOL, mask_of

pytestmark = pytest.mark.gpu

P = W.PAGE


def announce(msg: str) -> None:
    sys.__stderr__.write(f"[gpu] {msg}\n")
    sys.__stderr__.flush()


def values_of(rng, kind, rows, ncols):
    if kind == "ties":
        return np.round(rng.standard_normal((rows, ncols)) * 3, 1).astype(np.float32)
    if kind == "normal":
        return (rng.standard_normal((rows, ncols)) * 7).astype(np.float32)
    if kind == "equal":
        v = np.full((rows, ncols), 1.5, dtype=np.float32)
        v[:, ::97] = 2.0
        return v
    if kind == "zeros":
        # +0 and -0 (equal values) among small numbers, no NaN: the selected
        # zeros must come back with their own sign bits
        v = np.round(rng.standard_normal((rows, ncols)) * 0.8).astype(np.float32)
        v[v == 0] = np.where(rng.random(int((v == 0).sum())) < 0.5, np.float32(-0.0), np.float32(0.0))
        return v
    if kind in ("sample_low", "sample_high"):
        # every 8th position far below / above the rest: a guess taken from
        # those positions alone misplaces the k-th value (or finds it there)
        v = (rng.standard_normal((rows, ncols)) * 7).astype(np.float32)
        v[:, ::8] = -1000.0 if kind == "sample_low" else 1000.0
        return v
    pool = np.array([0.0, -0.0, 1.0, -1.0, 2.5, np.nan, np.inf, -np.inf, 3.0e38, -1e-45],
                    dtype=np.float32)
    return pool[rng.integers(0, len(pool), size=(rows, ncols))]


def lengths_for(rng, rows, ncols, k):
    special = [0, -3, k - 1, k, k + 1, ncols, ncols + 10, 1]
    out = [special[i] if i < len(special) else int(rng.integers(0, ncols + 1)) for i in range(rows)]
    return np.array(out, dtype=np.int32)


def check_selection(lib, vals, seqlens, k, row_stride=None):
    rows, ncols = vals.shape
    announce(f"topk rows={rows} ncols={ncols} k={k}")
    x = torch.from_numpy(vals).cuda()
    if row_stride is not None:  # rows inside a wider buffer, NaN in the gaps
        buf = torch.full((rows, row_stride), float("nan"), device="cuda")
        buf[:, :ncols] = x
        x = buf[:, :ncols]
    idx = torch.full((rows, k), -7, dtype=torch.int32, device="cuda")
    val = torch.full((rows, k), 123.0, dtype=torch.float32, device="cuda")
    lib.idx_topk_logits(x, torch.from_numpy(seqlens).cuda(), idx, val, ncols=ncols)
    torch.cuda.synchronize()
    got, got_v = idx.cpu().numpy(), val.cpu().numpy()
    want = oracle.topk(vals, seqlens, k)
    assert np.array_equal(got, want)
    sel = np.where(want >= 0, vals[np.arange(rows)[:, None], np.maximum(want, 0)], -np.inf)
    assert np.array_equal(got_v.view(np.uint32), sel.astype(np.float32).view(np.uint32))


@pytest.mark.parametrize("rows,ncols,k,kind", [
    (1, 8, 4, "special"), (9, 300, 1, "ties"), (9, 5000, 2048, "ties"), (9, 5000, 2048, "normal"),
    (9, 9000, 2048, "special"), (9, 4100, 2048, "equal"), (64, 40000, 2048, "normal"),
    (9, 12288, 4096, "ties"), (9, 70000, 3, "normal"),
    (5, 30000, 2048, "equal"),   # first digit holds more keys than the candidate list
    (5, 6144, 700, "equal"), (6, 20000, 2048, "sample_low"), (6, 20000, 2048, "sample_high"),
    (6, 5000, 2048, "sample_low"), (6, 5000, 300, "sample_high"),
    (6, 3000, 2000, "zeros"), (6, 9000, 7000, "zeros"),
    (6, 9000, 300, "zeros"), (6, 20000, 700, "ties"),  # sparse rows: per-thread bit words
    (8, 36000, 3000, "special"),  # NaN, +-0, +-inf in rows longer than the LDS stage
    (300, 6200, 64, "normal"),   # more rows than one-per-CU workgroups: taken last first
    (1100, 700, 200, "ties")])   # more rows than four-per-CU workgroups: taken last first
def test_topk_bit_exact(lib, rows, ncols, k, kind):
    rng = np.random.default_rng(rows * 7 + ncols + k)
    vals = values_of(rng, kind, rows, ncols)
    check_selection(lib, vals, lengths_for(rng, rows, ncols, k), k)


@pytest.mark.parametrize("k", [1, 2048])
@pytest.mark.parametrize("kind", ["normal", "special", "equal"])
def test_topk_sparse_row_boundaries(lib, k, kind):
    """The 1024-thread kernel finishes a staged row that takes at most a
    quarter of its keys from per-thread 32-position bit words: lengths just
    below, at and above 4k, a partial last word, and the full 32,768-key
    stage (every word whole)."""
    rng = np.random.default_rng(k * 3 + len(kind))
    ncols = 32768
    lens = [4 * k - 1, 4 * k, 4 * k + 1, 4 * k + 33, 32767, 32768, 20000 + 17]
    vals = values_of(rng, kind, len(lens), ncols)
    check_selection(lib, vals, np.array(lens, dtype=np.int32), k)


def test_topk_reads_only_live_positions(lib):
    """Values past each row's length (+inf here) and past the row (NaN in a
    wider buffer) are never selected."""
    rng = np.random.default_rng(31)
    rows, ncols, k = 6, 3000, 512
    vals = values_of(rng, "normal", rows, ncols)
    seqlens = np.array([2999, 1500, 600, 513, 100, 3000], dtype=np.int32)
    for b in range(rows):
        vals[b, seqlens[b]:] = np.inf
    check_selection(lib, vals, seqlens, k, row_stride=3072)


@pytest.mark.parametrize("ncols,list_cap", [(6144, 1024), (20000, 4096)])
@pytest.mark.parametrize("extra", [-1, 0, 1])
def test_topk_first_digit_at_list_capacity(lib, ncols, list_cap, extra):
    """Rows whose first 11-bit digit (sign, exponent and two mantissa bits)
    holds list_cap - 1, list_cap or list_cap + 1 keys: the kernel's candidate
    list for that row size (256-thread rows up to 6144 wide, 1024-thread rows
    above) is just filled or just overflows into the full-row passes.  Keys in
    the digit are distinct values in [5, 5.5) plus repeats, so the later
    digits and the tie rule both decide."""
    rng = np.random.default_rng(ncols + extra)
    rows, k = 3, 3000 if ncols > 6144 else 700
    n_in = list_cap + extra
    vals = np.full((rows, ncols), -1.0, dtype=np.float32)
    for b in range(rows):
        pos = rng.permutation(ncols)
        high = k // 3                                           # a higher digit: all taken
        digit = (5.0 + rng.integers(0, n_in // 3, size=n_in) * 1e-4).astype(np.float32)
        assert np.all((digit.view(np.uint32) >> 21) == (np.float32(5.0).view(np.uint32) >> 21))
        vals[b, pos[:high]] = 100.0
        vals[b, pos[high:high + n_in]] = digit
    seqlens = np.full(rows, ncols, dtype=np.int32)
    seqlens[2] = ncols - 5
    check_selection(lib, vals, seqlens, k)


def fused(lib, wl, k, canary=7.0):
    announce(f"fused topk {wl.key_kind} rows={wl.rows} width={wl.table_width} k={k} "
             f"pt_stride={wl.pt_stride} ({wl.name})")
    dw = W.to_device(wl, out_fill=canary)
    idx = torch.full((wl.rows, k), -7, dtype=torch.int32, device="cuda")
    val = torch.full((wl.rows, k), 123.0, dtype=torch.float32, device="cuda")
    W.run_library_topk(dw, lib, idx, val)
    torch.cuda.synchronize()
    return dw.out.cpu().numpy(), idx.cpu().numpy(), val.cpu().numpy()


def full_logits(lib, wl):
    dw = W.to_device(wl)
    W.run_library(dw, lib)
    torch.cuda.synchronize()
    return dw.out.cpu().numpy()


def check_fused(lib, wl, k, ref_rows=None):
    """Fused call == separate logits call + oracle top-k over those float32
    logits (exact), and == oracle top-k over the oracle's float64 logits up to
    swaps at the threshold (sampled rows)."""
    logits, idx, val = fused(lib, wl, k)
    full = full_logits(lib, wl)
    L = wl.lengths()
    live = ~mask_of(wl)
    assert np.array_equal(logits[live].view(np.uint32), full[live].view(np.uint32))
    want = oracle.topk(full, wl.seqlens, k)
    assert np.array_equal(idx, want)
    sel = np.where(want >= 0, full[np.arange(wl.rows)[:, None], np.maximum(want, 0)], -np.inf)
    assert np.array_equal(val.view(np.uint32), sel.astype(np.float32).view(np.uint32))
    rows = range(wl.rows) if ref_rows is None else ref_rows
    ref = oracle.paged_mqa_logits(wl, rows=list(rows))
    for j, b in enumerate(rows):
        assert_topk_near_threshold(idx[b], ref[j, :L[b]], k)
    return idx


def assert_topk_near_threshold(sel_row, ref, k, tol=ATOL):
    """The library's selection for one row vs the oracle's selection over its
    float64 logits: any position in one and not the other has an oracle value
    within tol of the oracle's k-th largest value."""
    L = len(ref)
    m = min(k, L)
    sel = sel_row[:m]
    assert np.all(sel_row[m:] == -1)
    assert np.all(np.diff(sel) > 0) and (m == 0 or (sel[0] >= 0 and sel[-1] < L))
    if m == 0:
        return
    ora = oracle.topk(ref[None, :], [L], k)[0][:m]
    kth = np.sort(ref)[::-1][m - 1]
    swapped = np.setxor1d(sel, ora)
    assert np.all(np.abs(ref[swapped] - kth) <= tol), (len(swapped), kth)


@pytest.mark.parametrize("kind", ["fp8", "bf16"])
@pytest.mark.parametrize("shared", [False, True])
def test_fused_topk_small(lib, kind, shared):
    rows = 13 if shared else 9
    seqlens = [0, 1, 63, 64, 65, 700, 1000, 1600, 3000][:rows] + [1234, 2000, 777, 3200][:rows - 9]
    wl = W.random_workload(40 + shared, kind, rows=rows, table_width=50, num_pages=120,
                           seqlens=seqlens, shared_table=shared)
    check_fused(lib, wl, k=512)


@pytest.mark.parametrize("k", [0, 1, 64, 5000])
def test_fused_topk_k_edges(lib, k):
    wl = W.random_workload(44, "fp8", rows=5, table_width=40, num_pages=64,
                           seqlens=[0, 64, 1000, 2560, 4000])
    if k == 0:
        logits, idx, _ = fused(lib, wl, 0)
        live = ~mask_of(wl)
        assert np.array_equal(logits[live].view(np.uint32), full_logits(lib, wl)[live].view(np.uint32))
        assert idx.shape == (5, 0)
    else:
        check_fused(lib, wl, k)


def test_fused_topk_zero_width(lib):
    wl = W.random_workload(45, "fp8", rows=3, table_width=0, num_pages=4, seqlens=[5, 0, 9])
    dw = W.to_device(wl)
    idx = torch.full((3, 16), 9, dtype=torch.int32, device="cuda")
    W.run_library_topk(dw, lib, idx)
    torch.cuda.synchronize()
    assert np.all(idx.cpu().numpy() == -1)


def test_fused_topk_decode_full_size(lib):
    """The 4097-page decode batch (64 rows) with k = 2048."""
    wl = W.config(3)
    check_fused(lib, wl, 2048, ref_rows=[0, 17, 63])


def test_fused_topk_prefill_full_size(lib):
    """The 4096-token prefill (shared table) with k = 2048."""
    wl = W.config(4)
    check_fused(lib, wl, 2048, ref_rows=[0, 1500, 2047, 2048, 4095])


def test_fused_topk_fp8_prefill_full_size(lib):
    """The 4096-token prefill with e4m3 keys: whole-table units of 88 pages,
    so each wave's logits buffer flushes inside the unit, with the fused
    call's ordinary stores."""
    wl = W.config("4f")
    check_fused(lib, wl, 2048, ref_rows=[3, 2049, 4095])


def test_fused_topk_bf16_decode(lib):
    """The 128-page bf16-key decode batch (64 rows), k = 2048: the bf16 decode
    path with the fill off."""
    wl = W.config("2b")
    check_fused(lib, wl, 2048, ref_rows=[0, 31, 63])


def test_fused_topk_graph_replay(lib):
    """Captured fused call: every replay gives the eager result."""
    wl = W.random_workload(46, "fp8", rows=16, table_width=64, num_pages=300)
    dw = W.to_device(wl)
    k = 300
    idx = torch.full((wl.rows, k), -7, dtype=torch.int32, device="cuda")
    W.run_library_topk(dw, lib, idx)
    torch.cuda.synchronize()
    eager = idx.cpu().numpy().copy()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        W.run_library_topk(dw, lib, idx)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        W.run_library_topk(dw, lib, idx)
    for _ in range(3):
        idx.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(idx.cpu().numpy(), eager)
