"""Parity of the HIP library against the CPU oracle, called through the C ABI.

Bar (finite logits): max |d| <= 2e-2 and max |d| / max |oracle| <= 5e-3; the
-inf pattern, NaN pattern and finiteness must match exactly.  Integer/index
facts (mask, page indirection, invariances) are checked bit-exactly.
"""
from __future__ import annotations

import dataclasses
import sys

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from helpers import (CODE_ONE, assert_parity, compare, make_workload, mask_of,
                     read_golden_rows)

pytestmark = pytest.mark.gpu

H, D, P = W.NUM_HEADS, W.HEAD_DIM, W.PAGE


def announce(msg: str) -> None:
    sys.__stderr__.write(f"[gpu] {msg}\n")
    sys.__stderr__.flush()


def run(lib, wl, stream=None, out_fill=float("nan")) -> np.ndarray:
    announce(f"{wl.key_kind} rows={wl.rows} width={wl.table_width} pages={wl.num_pages} "
             f"pt_stride={wl.pt_stride} ({wl.name})")
    dw = W.to_device(wl, out_fill=out_fill)
    W.run_library(dw, lib, stream=stream)
    torch.cuda.synchronize()
    return dw.out.cpu().numpy()


def check_full(lib, wl, label=""):
    got = run(lib, wl)
    ref = oracle.paged_mqa_logits(wl)
    return assert_parity(got, ref, mask_of(wl), label=label or wl.name)


# ---------------------------------------------------------------------------
# the specified configurations

@pytest.mark.parametrize("cfg", [0, 1, 2, "2b"])
def test_config_full(lib, cfg):
    st = check_full(lib, W.config(cfg))
    announce(f"config {cfg}: {st}")


def _sample_rows(wl, n, seed):
    L = wl.lengths()
    rng = np.random.default_rng(seed)
    pick = {int(np.argmin(L)), int(np.argmax(L)), 0, wl.rows - 1}
    pick |= set(int(x) for x in rng.choice(wl.rows, size=min(n, wl.rows), replace=False))
    return sorted(pick)


@pytest.mark.parametrize("cfg", [3, "3c", 4, "4f"])
def test_config_sampled_rows(lib, cfg):
    """Full-size configurations in the benchmark's launch shape: every output's
    mask checked; sampled rows checked against the oracle element by element.
    The 4096-row prefills (bf16 and fp8 keys) run whole-table units of 88
    pages, so each wave's 24-page logits buffer is written out mid-unit."""
    wl = W.config(cfg)
    got = run(lib, wl)
    m = mask_of(wl)
    assert np.array_equal(np.isneginf(got), m)
    assert np.isfinite(got[~m]).all()
    prefill = cfg in (4, "4f")
    rows = _sample_rows(wl, 40 if prefill else 6, seed=5)
    if prefill:  # rows on both sides of 4-row block edges
        rows = sorted(set(rows) | {1, 2, 3, 4, 5, 2047, 2048, 4092, 4093, 4094})
    ref = oracle.paged_mqa_logits(wl, rows=rows)
    st = assert_parity(got[rows], ref, m[rows], label=str(cfg))
    announce(f"config {cfg} rows {rows}: {st}")


def test_wide_table_matches_narrow_table(lib):
    """Config 3 at width 4097 and its 513-slot control give identical scores."""
    a = run(lib, W.config(3))
    b = run(lib, W.config("3c"))
    n = b.shape[1]
    assert np.array_equal(a[:, :n], b)
    assert np.all(np.isneginf(a[:, n:]))


# ---------------------------------------------------------------------------
# the pages' own test shapes (B, pages, max seqlen), reported in their format

@pytest.mark.parametrize("row", read_golden_rows("pages_accuracy.txt"),
                         ids=lambda r: f"B{int(r[0])}-p{int(r[1])}")
def test_pages_test_shapes(lib, row):
    B, pages, smax = int(row[0]), int(row[1]), int(row[2])
    wl = W.random_workload(2000 + B, "fp8", rows=B, table_width=pages, num_pages=B * pages,
                           seqlens=np.random.default_rng(B).integers(1, smax + 1, size=B))
    st = check_full(lib, wl)
    announce(f"B={B} H=64 pages={pages} seqlen<= {smax}: finite max|d|={st['max_abs']:.3e} "
             f"rel={st['rel']:.3e} inf-pattern-match={st['inf_pattern_match']}")


# ---------------------------------------------------------------------------
# both kernels x both key formats x both scale layouts

@pytest.mark.parametrize("kind", ["fp8", "bf16"])
@pytest.mark.parametrize("shared", [False, True])
def test_kernel_variants(lib, kind, shared):
    rows = 13 if shared else 9
    wl = W.random_workload(40 + shared, kind, rows=rows, table_width=21, num_pages=30,
                           shared_table=shared)
    check_full(lib, wl, label=f"{kind} shared={shared}")


@pytest.mark.parametrize("shared", [False, True])
def test_split_scale_layout(lib, shared):
    wl = W.random_workload(50, "fp8", rows=6, table_width=11, num_pages=70, layout="split",
                           shared_table=shared)
    check_full(lib, wl)


def test_prefill_shape_fp8_keys(lib):
    """fp8 keys through the shared-table kernel at a prefill-like shape."""
    T, width = 260, 13
    seq = ((width * P * (np.arange(T) + 1) + T - 1) // T).astype(np.int32)
    wl = W.random_workload(51, "fp8", rows=T, table_width=width, num_pages=width,
                           shared_table=True, seqlens=seq)
    check_full(lib, wl)


@pytest.mark.parametrize("kind", ["fp8", "bf16"])
def test_prefill_units_past_logits_buffer(lib, kind):
    """Shared-table units longer than a wave's 24-page logits buffer, checked
    in full: 4096 rows (1024 row blocks, so every unit is the whole 40-page
    table), most rows short and every 97th row block long (28..40 pages), so
    the buffer is written out in the middle of a unit and again at its end."""
    rows, width = 4096, 40
    rng = np.random.default_rng(98)
    seq = rng.integers(1, 2 * P + 1, size=rows)
    for rb in range(0, rows // 4, 97):
        seq[4 * rb: 4 * rb + 4] = rng.integers(27 * P + 1, width * P + 1, size=4)
    seq[-1] = width * P
    wl = W.random_workload(98, kind, rows=rows, table_width=width, num_pages=width + 9,
                           seqlens=seq, shared_table=True)
    assert int(wl.lengths().max()) > 24 * P
    st = check_full(lib, wl, label=f"prefill units > buffer {kind}")
    announce(f"prefill units past the logits buffer {kind}: {st}")


def test_decode_shape_bf16_keys(lib):
    wl = W.random_workload(52, "bf16", rows=24, table_width=40, num_pages=24 * 40,
                           seqlens=np.random.default_rng(3).integers(1, 40 * P, size=24))
    check_full(lib, wl)


# ---------------------------------------------------------------------------
# edge cases

EDGE_SEQ = [0, 1, 63, 64, 65, 127, 128, 129, 5 * P - 1, 5 * P, 5 * P + 9, -3,
            2 ** 31 - 1, -2 ** 31]


@pytest.mark.parametrize("kind", ["fp8", "bf16"])
@pytest.mark.parametrize("shared", [False, True])
def test_edge_lengths(lib, kind, shared):
    wl = W.random_workload(60, kind, rows=len(EDGE_SEQ), table_width=5, num_pages=80,
                           seqlens=EDGE_SEQ, shared_table=shared, pad=-1)
    check_full(lib, wl, label=f"edge {kind} shared={shared}")


def test_zero_rows_and_zero_width_touch_nothing(lib):
    out = torch.full((4, 64), 7.0, device="cuda")
    dummy = torch.zeros(64, dtype=torch.int32, device="cuda")
    q = torch.zeros((1, H, D), dtype=torch.bfloat16, device="cuda")
    kv = torch.zeros(8448, dtype=torch.uint8, device="cuda")
    w = torch.zeros((1, H), device="cuda")
    for rows, width in ((0, 1), (1, 0)):
        st = lib.idx_paged_mqa_logits_fp8(q, kv, kv.data_ptr() + 8192, dummy, dummy, w, out,
                                          rows=rows, table_width=width, num_pages=1,
                                          page_table_row_stride=1)
        assert st == 0
    torch.cuda.synchronize()
    assert torch.all(out == 7.0)


@pytest.mark.parametrize("shared", [False, True])
def test_poisoned_tail_and_padding(lib, shared):
    """NaN keys and scales past seqlen inside the last live page, table padding -1:
    the tail must come out -inf (a select, not a multiply) and padding is never read."""
    rows, width = 5, 6
    wl = W.random_workload(61, "fp8", rows=rows, table_width=width, num_pages=rows * width,
                           seqlens=[1, 70, 130, 200, 383], shared_table=shared, pad=-1)
    L = wl.lengths()
    perm = np.random.default_rng(6).permutation(wl.num_pages).astype(np.int32)
    tab = np.full((1 if shared else rows, width), -1, dtype=np.int32)
    lens = [int(L.max())] if shared else [int(x) for x in L]
    for r, Lr in enumerate(lens):                 # disjoint pages per row
        nlive = (Lr + P - 1) // P
        tab[r, :nlive] = perm[r * width: r * width + nlive]
    wl = dataclasses.replace(wl, page_table=tab.reshape(-1).copy())
    kv = wl.kv.reshape(wl.num_pages, wl.kv_stride)
    nan_bytes = np.frombuffer(np.float32(np.nan).tobytes(), np.uint8)
    for r, Lr in enumerate(lens):
        j_last = (Lr - 1) // P
        g = int(tab[r, j_last])
        for i in range(Lr - j_last * P, P):
            kv[g, i * D:(i + 1) * D] = 0x7F                        # NaN codes
            kv[g, 8192 + 4 * i: 8192 + 4 * i + 4] = nan_bytes       # NaN scale
    got = run(lib, wl)
    ref = oracle.paged_mqa_logits(wl)
    m = mask_of(wl)
    assert np.isfinite(ref[~m]).all()
    assert_parity(got, ref, m, label=f"poison shared={shared}")


@pytest.mark.parametrize("shared", [False, True])
def test_invalid_page_ids_give_nan(lib, shared):
    wl = W.random_workload(62, "fp8", rows=3, table_width=4, num_pages=12,
                           seqlens=[256, 200, 150], shared_table=shared)
    if shared:
        wl.page_table[2] = 12
    else:
        wl.page_table[1] = 12
        wl.page_table[4 + 3] = -5
        wl.page_table[8 + 0] = 2 ** 31 - 1
    check_full(lib, wl, label=f"bad ids shared={shared}")


@pytest.mark.parametrize("kind,shared", [("fp8", False), ("fp8", True), ("bf16", False)])
def test_pool_size_past_int32(lib, kind, shared):
    """A declared pool of 2^31 + 7 pages (more than a 32-bit signed id can name):
    every non-negative id is then in the pool, negative ids still give NaN.  The
    table names only pages of the small pool actually allocated, so nothing past
    it is read; the oracle sees the real pool size, under which the same ids are
    valid and invalid."""
    wl = W.random_workload(65, kind, rows=3, table_width=4, num_pages=12,
                           seqlens=[256, 200, 150], shared_table=shared)
    wl.page_table[1] = -5
    if not shared:
        wl.page_table[4 + 2] = -1
    ref = oracle.paged_mqa_logits(wl)
    dw = W.to_device(wl)
    dw.wl = dataclasses.replace(wl, num_pages=2 ** 31 + 7)
    W.run_library(dw, lib)
    torch.cuda.synchronize()
    got = dw.out.cpu().numpy()
    m = mask_of(wl)
    assert np.array_equal(np.isnan(got), np.isnan(ref)), "NaN pattern"
    assert_parity(got, ref, m, label=f"pool 2^31+7 {kind} shared={shared}")


def test_all_256_fp8_codes(lib):
    """Every e4m3fn code reaches the logits exactly: key code c at dim 0 of one
    position, q = e_0 for head 0, w = e_0, s = +1 -> ReLU(dec(c)); s = -1 -> ReLU(-dec(c))."""
    codes = np.zeros((4, P, D), dtype=np.uint8)
    codes.reshape(256, D)[:, 0] = np.arange(256, dtype=np.uint8)
    q = np.zeros((2, H, D), dtype=np.float32)
    q[:, 0, 0] = 1.0
    w = np.zeros((2, H), dtype=np.float32)
    w[:, 0] = 1.0
    for sign in (1.0, -1.0):
        scales = np.full((4, P), sign, dtype=np.float32)
        wl = make_workload("fp8", q, w, codes, [[0, 1, 2, 3], [3, 2, 1, 0]], [256, 256], scales)
        got = run(lib, wl)
        ref = oracle.paged_mqa_logits(wl)
        assert np.array_equal(np.isnan(got), np.isnan(ref))
        ok = ~np.isnan(ref)
        assert np.array_equal(got[ok], ref[ok].astype(np.float32)), sign


def test_zero_weights_and_identical_keys(lib):
    wl = W.random_workload(63, "fp8", rows=4, table_width=3, num_pages=12)
    wl.weights[:] = 0.0
    got = run(lib, wl)
    m = mask_of(wl)
    assert np.all(got[~m] == 0.0) and np.all(np.isneginf(got[m]))
    wl = W.random_workload(64, "bf16", rows=3, table_width=3, num_pages=4)
    kv = wl.kv.reshape(wl.num_pages, P, 2 * D)
    kv[:] = kv[0, 0]
    got = run(lib, wl)
    for b in range(wl.rows):
        live = got[b][~mask_of(wl)[b]]
        if live.size:
            assert np.all(live == live[0])


# ---------------------------------------------------------------------------
# invariances (bit-exact on the GPU)

def test_pool_permutation_bit_exact(lib):
    wl = W.random_workload(70, "fp8", rows=8, table_width=9, num_pages=80)
    perm = np.random.default_rng(1).permutation(wl.num_pages)
    blocks = wl.kv.reshape(wl.num_pages, wl.kv_stride)
    nb = np.empty_like(blocks)
    nb[perm] = blocks
    kv2 = nb.reshape(-1)
    tab = wl.page_table.copy()
    tab[tab >= 0] = perm[tab[tab >= 0]]
    wl2 = dataclasses.replace(wl, kv=kv2, ks=kv2, page_table=tab)
    assert np.array_equal(run(lib, wl), run(lib, wl2))


def test_batch_and_width_invariance_bit_exact(lib):
    wl = W.random_workload(71, "fp8", rows=10, table_width=7, num_pages=80)
    full = run(lib, wl)
    sub_rows = [7, 2, 9]
    sub = dataclasses.replace(
        wl, rows=3, q=wl.q[sub_rows], weights=wl.weights[sub_rows],
        page_table=wl.page_table.reshape(10, 7)[sub_rows].reshape(-1).copy(),
        seqlens=wl.seqlens[sub_rows])
    assert np.array_equal(run(lib, sub), full[sub_rows])
    wide_tab = np.full((10, 30), -1, dtype=np.int32)
    wide_tab[:, :7] = wl.page_table.reshape(10, 7)
    wide = dataclasses.replace(wl, table_width=30, page_table=wide_tab.reshape(-1), pt_stride=30)
    gw = run(lib, wide)
    assert np.array_equal(gw[:, :7 * P], full) and np.all(np.isneginf(gw[:, 7 * P:]))


def test_shared_kernel_matches_rowwise_bit_exact(lib):
    """A shared table (stride 0) and explicit per-row copies run different kernels
    with the same per-page arithmetic."""
    for kind in ("fp8", "bf16"):
        wl = W.random_workload(72, kind, rows=11, table_width=10, num_pages=10,
                               shared_table=True)
        tab = np.tile(wl.page_table[:10], 11)
        copy = dataclasses.replace(wl, page_table=tab, pt_stride=10)
        assert np.array_equal(run(lib, wl), run(lib, copy)), kind


# ---------------------------------------------------------------------------
# launch plumbing

def test_no_write_outside_output(lib):
    wl = W.random_workload(80, "fp8", rows=5, table_width=9, num_pages=50)
    dw = W.to_device(wl)
    big = torch.full((wl.rows * wl.ncols + 4096,), 123.0, device="cuda")
    dw.out = big[:wl.rows * wl.ncols].view(wl.rows, wl.ncols)
    announce("canary")
    W.run_library(dw, lib)
    torch.cuda.synchronize()
    assert torch.all(big[wl.rows * wl.ncols:] == 123.0)
    assert_parity(dw.out.cpu().numpy(), oracle.paged_mqa_logits(wl), mask_of(wl))


def test_side_stream(lib):
    wl = W.random_workload(81, "bf16", rows=7, table_width=6, num_pages=42)
    dw = W.to_device(wl)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    announce("side stream")
    with torch.cuda.stream(s):
        W.run_library(dw, lib, stream=s)
    s.synchronize()
    assert_parity(dw.out.cpu().numpy(), oracle.paged_mqa_logits(wl), mask_of(wl))


@pytest.mark.parametrize("shared", [False, True])
def test_graph_capture_replay(lib, shared):
    """One launch captured in a HIP graph; lengths and page table mutated in place
    between replays, with eager work in between; every replay checked."""
    wl = W.random_workload(82, "fp8", rows=6, table_width=8, num_pages=48,
                           shared_table=shared, seqlens=[100, 512, 3, 0, 300, 64])
    dw = W.to_device(wl)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):                      # warm-up launch outside capture
        W.run_library(dw, lib, stream=s)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    announce(f"graph capture shared={shared}")
    with torch.cuda.graph(g):
        W.run_library(dw, lib)
    rng = np.random.default_rng(5)
    for it in range(4):
        seq = rng.integers(-5, wl.ncols + 40, size=wl.rows).astype(np.int32)
        tab = wl.page_table.copy()
        rows_t = 1 if shared else wl.rows
        for r in range(rows_t):
            tab[r * (wl.pt_stride or 0): r * (wl.pt_stride or 0) + wl.table_width] = \
                rng.permutation(wl.num_pages)[:wl.table_width]
        wl2 = dataclasses.replace(wl, seqlens=seq, page_table=tab)
        dw.seqlens.copy_(torch.from_numpy(seq))
        dw.page_table.copy_(torch.from_numpy(tab))
        dw.out.fill_(float("nan"))
        _ = (torch.ones(1000, device="cuda") * it).sum().item()   # eager work between replays
        g.replay()
        torch.cuda.synchronize()
        assert_parity(dw.out.cpu().numpy(), oracle.paged_mqa_logits(wl2), mask_of(wl2),
                      label=f"replay {it}")


def test_grid_stride_beyond_grid_cap(lib):
    """More work units than the launch grid holds: the grid-stride loop covers them."""
    rows, width = 2048, 4100
    rng = np.random.default_rng(90)
    seq = rng.integers(0, 3 * P, size=rows)
    seq[-1] = width * P                                 # last row fully live
    wl = W.random_workload(90, "fp8", rows=rows, table_width=width, num_pages=4100,
                           seqlens=seq, pad=-1)
    got = run(lib, wl)
    m = mask_of(wl)
    assert np.array_equal(np.isneginf(got), m)
    sample = [0, 1, 1023, 2046, 2047]
    assert_parity(got[sample], oracle.paged_mqa_logits(wl, rows=sample), m[sample])


@pytest.mark.parametrize("kind", ["fp8", "bf16"])
def test_long_live_shares(lib, kind):
    """Enough live pages that each wave of the decode grid scores more pages
    than its logits buffer holds (12), so the buffer is written out in the
    middle of a row segment as well as at its end; segments also cross rows."""
    rows, width = 64, 600
    rng = np.random.default_rng(95)
    seq = rng.integers(width * P - 2 * P, width * P + 1, size=rows)
    seq[3] = 0                                          # an empty row between full ones
    wl = W.random_workload(95, kind, rows=rows, table_width=width, num_pages=256,
                           seqlens=seq, pad=-1)
    assert wl.live_pages() > 12 * 4 * 512               # > 12 pages per wave at any grid
    got = run(lib, wl)
    m = mask_of(wl)
    assert np.array_equal(np.isneginf(got), m)
    assert np.isfinite(got[~m]).all()
    sample = [0, 2, 3, 4, 31, 62, 63]
    st = assert_parity(got[sample], oracle.paged_mqa_logits(wl, rows=sample), m[sample],
                       label=f"long shares {kind}")
    announce(f"long shares {kind}: {st}")


@pytest.mark.parametrize("kind", ["bf16", "fp8"])
def test_prefill_row_blocks_past_resident_grid(lib, kind):
    """A shared-table prefill with more 4-row blocks (725) than resident
    workgroups and not a multiple of them: with bf16 keys the blocks are dealt in
    passes (long and short blocks paired, the last pass partial); every row is
    scored exactly once."""
    rows, width = 2900, 24
    t = np.arange(rows)
    seq = (width * P * (t + 1) + rows - 1) // rows           # causal limits, 1 .. width*64
    wl = W.random_workload(97, kind, rows=rows, table_width=width, num_pages=40,
                           seqlens=seq, shared_table=True)
    got = run(lib, wl)
    m = mask_of(wl)
    assert np.array_equal(np.isneginf(got), m)
    assert np.isfinite(got[~m]).all()
    sample = [0, 1, 3, 4, 511 * 4, 512 * 4 + 1, 724 * 4, 2047, 2048, rows - 1]
    st = assert_parity(got[sample], oracle.paged_mqa_logits(wl, rows=sample), m[sample],
                       label=f"prefill 725 blocks {kind}")
    announce(f"prefill 725 row blocks {kind}: {st}")


def test_binding_rejects_bad_arguments(lib):
    q = torch.zeros((2, 32, D), dtype=torch.bfloat16, device="cuda")
    kv = torch.zeros(8448, dtype=torch.uint8, device="cuda")
    pt = torch.zeros((2, 1), dtype=torch.int32, device="cuda")
    sl = torch.zeros(2, dtype=torch.int32, device="cuda")
    w = torch.zeros((2, H), device="cuda")
    out = torch.zeros((2, 64), device="cuda")
    with pytest.raises(lib.IdxError):
        lib.idx_paged_mqa_logits_fp8(q, kv, kv.data_ptr() + 8192, pt, sl, w, out, num_pages=1)
    st = lib.idx_paged_mqa_logits_fp8(q, kv, kv.data_ptr() + 8192, pt, sl, w, out, num_pages=1,
                                      check=False)
    assert st == -2


@pytest.mark.parametrize("seed", range(6))
def test_random_shapes(lib, seed):
    """Seeded random problems: rows, width, pool, lengths (including <= 0 and
    past the table), key format, table sharing and scale layout drawn per seed."""
    rng = np.random.default_rng(900 + seed)
    kind = ["fp8", "bf16"][seed % 2]
    shared = bool(rng.integers(0, 2))
    rows = int(rng.integers(1, 40))
    width = int(rng.integers(1, 90))
    pool = int(rng.integers(width, 3 * width + 2))
    seq = rng.integers(-70, width * P + 140, size=rows)
    layout = "split" if (kind == "fp8" and seed % 3 == 0) else "fused"
    wl = W.random_workload(1200 + seed, kind, rows=rows, table_width=width, num_pages=pool,
                           seqlens=seq, shared_table=shared, layout=layout)
    st = check_full(lib, wl, label=f"random {seed}")
    announce(f"random seed {seed} {kind} rows={rows} width={width} shared={shared} {layout}: {st}")
