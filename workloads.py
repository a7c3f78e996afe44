"""Seeded synthetic inputs for the paged MQA-logits indexer.

Shared by the tests (oracle side), the benchmark and the smoke check (library
side).  This module holds no part of the indexer's arithmetic: it draws
random numbers, rounds them to the storage formats (bf16 for queries and bf16
keys, e4m3fn codes with a per-position fp32 scale for fp8 keys) and lays the
bytes out as the library expects.  Both sides then read the very same bytes.

Recipe (all draws from numpy ``Generator(PCG64(seed))`` in this order):
  1. q        standard normal float32 [rows, 64, 128] -> bf16 (round to nearest even)
  2. weights  standard normal float32 [rows, 64] / 8
  3. keys     standard normal float32, page by page in chunks of 1024 pages,
              [pages, 64, 128]; fp8: scale = amax_d |k| / 448 per position,
              code = e4m3fn(k / scale) (nearest even, clamped to +-448);
              bf16: rounded to nearest even
  4. page table, 5. seqlens  (per configuration)

The five configurations follow the workloads the indexer is specified on
(fp8 decode at three batch/width points, the O(actual) wide-table decode and a
bf16 prefill of one 4096-token request); seeds are 1000 + configuration index.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np
import torch

NUM_HEADS = 64
HEAD_DIM = 128
PAGE = 64
FP8_KEY_BYTES = PAGE * HEAD_DIM          # 8192 per page
FP8_SCALE_BYTES = PAGE * 4               # 256 per page
FP8_FUSED_STRIDE = FP8_KEY_BYTES + FP8_SCALE_BYTES  # 8448
BF16_PAGE_BYTES = PAGE * HEAD_DIM * 2    # 16384
E4M3_MAX = 448.0
KEY_CHUNK_PAGES = 1024


@dataclasses.dataclass
class Workload:
    name: str
    key_kind: str            # "fp8" or "bf16"
    rows: int
    table_width: int
    num_pages: int
    q: np.ndarray            # uint16 bf16 bits [rows, 64, 128]
    weights: np.ndarray      # float32 [rows, 64]
    kv: np.ndarray           # uint8, num_pages * kv_stride bytes (+ slack)
    kv_stride: int
    ks: np.ndarray | None    # uint8 buffer holding the scales (may be ``kv`` itself)
    ks_offset: int
    ks_stride: int
    page_table: np.ndarray   # int32, flat
    pt_stride: int
    seqlens: np.ndarray      # int32 [rows]
    row_table: np.ndarray | None = None  # int32 [rows]: page-table row of each row (multi-request)
    num_tables: int = 0

    @property
    def ncols(self) -> int:
        return self.table_width * PAGE

    @property
    def fused(self) -> bool:
        return self.ks is not None and self.ks is self.kv

    def lengths(self) -> np.ndarray:
        """Row lengths clamped to [0, table_width*64] (positions that get a score)."""
        return np.clip(self.seqlens.astype(np.int64), 0, self.ncols)

    def live_positions(self) -> int:
        return int(self.lengths().sum())

    def live_pages(self) -> int:
        return int(((self.lengths() + PAGE - 1) // PAGE).sum())


# --------------------------------------------------------------------------
# storage-format rounding (library routines; input preparation only)

def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def quantize_fp8(k: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Per-position e4m3fn codes and fp32 scales for keys k [..., 64, 128]."""
    k = np.ascontiguousarray(k, dtype=np.float32)
    amax = np.abs(k).max(axis=-1)
    scale = np.where(amax > 0, amax / np.float32(E4M3_MAX), np.float32(1.0)).astype(np.float32)
    y = np.clip(k / scale[..., None], -E4M3_MAX, E4M3_MAX).astype(np.float32)
    codes = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()
    return codes, scale


def keys_from_normal(rng: np.random.Generator, num_pages: int, key_kind: str,
                     layout: str = "fused") -> tuple[np.ndarray, int, np.ndarray | None, int, int]:
    """Draw keys page-chunk by page-chunk and lay them out.

    Returns (kv, kv_stride, ks, ks_offset, ks_stride).  fp8 layouts: "fused"
    (8448-byte blocks, scales at +8192) or "split" (8192-byte key pages and a
    separate 256-byte-per-page scale buffer).
    """
    if key_kind == "fp8":
        if layout == "fused":
            kv = np.zeros(num_pages * FP8_FUSED_STRIDE, dtype=np.uint8)
            blocks = kv.reshape(num_pages, FP8_FUSED_STRIDE)
            ks, ks_offset, ks_stride, kv_stride = kv, FP8_KEY_BYTES, FP8_FUSED_STRIDE, FP8_FUSED_STRIDE
        elif layout == "split":
            kv = np.zeros(num_pages * FP8_KEY_BYTES, dtype=np.uint8)
            ks = np.zeros(num_pages * FP8_SCALE_BYTES, dtype=np.uint8)
            ks_offset, ks_stride, kv_stride = 0, FP8_SCALE_BYTES, FP8_KEY_BYTES
        else:
            raise ValueError(layout)
        for p0 in range(0, num_pages, KEY_CHUNK_PAGES):
            n = min(KEY_CHUNK_PAGES, num_pages - p0)
            k = rng.standard_normal((n, PAGE, HEAD_DIM), dtype=np.float32)
            codes, scale = quantize_fp8(k)
            if layout == "fused":
                blocks[p0:p0 + n, :FP8_KEY_BYTES] = codes.reshape(n, -1)
                blocks[p0:p0 + n, FP8_KEY_BYTES:] = scale.view(np.uint8).reshape(n, -1)
            else:
                kv.reshape(num_pages, -1)[p0:p0 + n] = codes.reshape(n, -1)
                ks.reshape(num_pages, -1)[p0:p0 + n] = scale.view(np.uint8).reshape(n, -1)
        return kv, kv_stride, ks, ks_offset, ks_stride
    if key_kind == "bf16":
        kv = np.zeros(num_pages * BF16_PAGE_BYTES, dtype=np.uint8)
        pages = kv.view(np.uint16).reshape(num_pages, PAGE * HEAD_DIM)
        for p0 in range(0, num_pages, KEY_CHUNK_PAGES):
            n = min(KEY_CHUNK_PAGES, num_pages - p0)
            k = rng.standard_normal((n, PAGE, HEAD_DIM), dtype=np.float32)
            pages[p0:p0 + n] = to_bf16_bits(k).reshape(n, -1)
        return kv, BF16_PAGE_BYTES, None, 0, 0
    raise ValueError(key_kind)


def draw_q_w(rng: np.random.Generator, rows: int) -> tuple[np.ndarray, np.ndarray]:
    q = to_bf16_bits(rng.standard_normal((rows, NUM_HEADS, HEAD_DIM), dtype=np.float32))
    w = (rng.standard_normal((rows, NUM_HEADS), dtype=np.float32) / np.float32(8.0)).astype(np.float32)
    return q, w


# --------------------------------------------------------------------------
# the five specified configurations

CONFIG_NAMES = {
    0: "fp8 decode B=1 width=8",
    1: "fp8 decode B=16 width=32",
    2: "fp8 decode B=64 width=128",
    3: "fp8 decode O(actual) B=64 width=4097",
    "3c": "fp8 decode B=64 width=513 (same rows as width=4097)",
    4: "bf16 prefill T=4096 width=88",
    "2b": "bf16-key decode B=64 width=128",
    "4f": "fp8-key prefill T=4096 width=88",
}


def config(idx, layout: str = "fused") -> Workload:
    """Seeded workload of one configuration: 0-4; "3c" = the 4097-wide decode's
    rows in a 513-slot table; "2b" / "4f" = the 128-page decode with bf16 keys /
    the prefill with fp8 keys (same shapes, lengths and tables)."""
    base = {"3c": 3, "2b": 2, "4f": 4}.get(idx, idx)
    base = int(base)
    rng = np.random.Generator(np.random.PCG64(1000 + base))
    if base == 0:
        rows, width, pool, kind = 1, 8, 8, "fp8"
    elif base == 1:
        rows, width, pool, kind = 16, 32, 512, "fp8"
    elif base == 2:
        rows, width, pool, kind = 64, 128, 8192, "fp8"
    elif base == 3:
        rows, width, pool, kind = 64, 4097, 64 * 512, "fp8"
    elif base == 4:
        rows, width, pool, kind = 4096, 88, 88, "bf16"
    else:
        raise ValueError(idx)
    if idx in ("2b", "4f"):
        kind = "bf16" if idx == "2b" else "fp8"
    q, w = draw_q_w(rng, rows)
    kv, kv_stride, ks, ks_off, ks_stride = keys_from_normal(rng, pool, kind, layout)

    if base == 0:
        table = rng.permutation(pool).astype(np.int32).reshape(1, width)
        seqlens = rng.integers(1, 512 + 1, size=rows).astype(np.int32)
        pt_stride = width
    elif base == 1:
        table = rng.permutation(pool).astype(np.int32).reshape(rows, width)
        seqlens = rng.integers(1, 2048 + 1, size=rows).astype(np.int32)
        pt_stride = width
    elif base == 2:
        table = rng.permutation(pool).astype(np.int32).reshape(rows, width)
        seqlens = rng.integers(256, 8192 + 1, size=rows).astype(np.int32)
        pt_stride = width
    elif base == 3:
        live = rng.permutation(pool).astype(np.int32).reshape(rows, 512)
        seqlens = rng.integers(512, 32768 + 1, size=rows).astype(np.int32)
        if idx == "3c":
            width = 513
        table = np.full((rows, width), -1, dtype=np.int32)
        table[:, :512] = live
        pt_stride = width
    else:  # 4: one request's prefill; token t sees ceil(5632 (t+1) / 4096) positions
        table = rng.permutation(pool).astype(np.int32).reshape(1, width)
        t = np.arange(rows, dtype=np.int64)
        seqlens = ((5632 * (t + 1) + 4095) // 4096).astype(np.int32)
        pt_stride = 0
    return Workload(name=CONFIG_NAMES[idx], key_kind=kind, rows=rows, table_width=width,
                    num_pages=pool, q=q, weights=w, kv=kv, kv_stride=kv_stride, ks=ks,
                    ks_offset=ks_off, ks_stride=ks_stride, page_table=table.reshape(-1).copy(),
                    pt_stride=pt_stride, seqlens=seqlens)


def random_workload(seed: int, key_kind: str, rows: int, table_width: int, num_pages: int,
                    seqlens=None, shared_table: bool = False, layout: str = "fused",
                    pad: int = -1, pt_stride: int | None = None) -> Workload:
    """Small seeded workload with random tables (tests).

    Row tables draw distinct pages from the pool when it is large enough
    (else with replacement); slots past each row's live pages hold ``pad``.
    ``seqlens`` may be given (any int32, even negative or past the width).
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    q, w = draw_q_w(rng, rows)
    kv, kv_stride, ks, ks_off, ks_stride = keys_from_normal(rng, num_pages, key_kind, layout)
    trows = 1 if shared_table else rows
    if seqlens is None:
        seqlens = rng.integers(0, table_width * PAGE + 1, size=rows)
    seqlens = np.asarray(seqlens, dtype=np.int64).astype(np.int32)
    stride = (0 if shared_table else table_width) if pt_stride is None else pt_stride
    tab_rows = trows if stride == 0 else rows
    table = np.full((tab_rows, max(stride, table_width)), pad, dtype=np.int32)
    for r in range(tab_rows):
        if num_pages >= table_width:
            ids = rng.permutation(num_pages)[:table_width]
        else:
            ids = rng.integers(0, max(num_pages, 1), size=table_width)
        if stride == 0:
            L = int(np.clip(seqlens.astype(np.int64), 0, table_width * PAGE).max()) if rows else 0
        else:
            L = int(np.clip(int(seqlens[r]), 0, table_width * PAGE))
        nlive = (L + PAGE - 1) // PAGE
        table[r, :nlive] = ids[:nlive]
    return Workload(name=f"random seed={seed}", key_kind=key_kind, rows=rows,
                    table_width=table_width, num_pages=num_pages, q=q, weights=w, kv=kv,
                    kv_stride=kv_stride, ks=ks, ks_offset=ks_off, ks_stride=ks_stride,
                    page_table=table.reshape(-1).copy(), pt_stride=stride, seqlens=seqlens)


def varlen_workload(seed: int, key_kind: str, tokens, contexts, table_width: int, num_pages: int,
                    interleave: bool = False, layout: str = "fused") -> Workload:
    """Seeded prefill batch of several requests (tests and benchmark).

    Request r contributes tokens[r] query rows and owns contexts[r] cached
    positions; its token t (0-based) sees ceil(contexts[r] * (t+1) / tokens[r])
    of them (causal growth, as in the single-request prefill).  Each request
    has its own table (row r of page_table, stride table_width) of distinct
    pool pages, -1 past its live pages; row_table maps each row to its
    request.  Rows are grouped by request, or dealt round-robin over the
    requests with ``interleave``.
    Draws: q, weights, keys (as random_workload), then the tables.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    tokens = [int(t) for t in tokens]
    contexts = [int(c) for c in contexts]
    rows = sum(tokens)
    q, w = draw_q_w(rng, rows)
    kv, kv_stride, ks, ks_off, ks_stride = keys_from_normal(rng, num_pages, key_kind, layout)
    R = len(tokens)
    table = np.full((R, table_width), -1, dtype=np.int32)
    for r in range(R):
        nlive = min(table_width, (contexts[r] + PAGE - 1) // PAGE)
        table[r, :nlive] = rng.permutation(num_pages)[:nlive]
    req_rows = [(r, t) for r in range(R) for t in range(tokens[r])]
    if interleave:
        req_rows = []
        for t in range(max(tokens) if tokens else 0):
            req_rows += [(r, t) for r in range(R) if t < tokens[r]]
    row_table = np.array([r for r, _ in req_rows], dtype=np.int32)
    seqlens = np.array([(contexts[r] * (t + 1) + tokens[r] - 1) // tokens[r] for r, t in req_rows],
                       dtype=np.int64).astype(np.int32)
    return Workload(name=f"varlen seed={seed} requests={R}", key_kind=key_kind, rows=rows,
                    table_width=table_width, num_pages=num_pages, q=q, weights=w, kv=kv,
                    kv_stride=kv_stride, ks=ks, ks_offset=ks_off, ks_stride=ks_stride,
                    page_table=table.reshape(-1).copy(), pt_stride=table_width, seqlens=seqlens,
                    row_table=row_table, num_tables=R)


VARLEN_NAME = "bf16 multi-request prefill, 4 requests, 4096 rows, width=128"


def varlen_config() -> Workload:
    """Multi-request prefill at the single-request prefill's scale: 4096 query
    rows from four requests (1024, 512, 2048 and 512 tokens) over contexts of
    5632, 2048, 8192 and 1024 positions, bf16 keys, tables of 128 pages."""
    wl = varlen_workload(1005, "bf16", tokens=[1024, 512, 2048, 512],
                         contexts=[5632, 2048, 8192, 1024], table_width=128, num_pages=512)
    wl.name = VARLEN_NAME
    return wl


# --------------------------------------------------------------------------
# device placement (plumbing for the library side)

@dataclasses.dataclass
class DeviceWorkload:
    wl: Workload
    q: torch.Tensor
    weights: torch.Tensor
    kv: torch.Tensor
    ks: torch.Tensor | None
    kscale_addr: int | None
    page_table: torch.Tensor
    seqlens: torch.Tensor
    out: torch.Tensor
    row_table: torch.Tensor | None = None


def to_device(wl: Workload, device="cuda", out_fill: float = float("nan")) -> DeviceWorkload:
    dev = torch.device(device)
    q = torch.from_numpy(wl.q.view(np.int16)).to(dev).view(torch.bfloat16)
    w = torch.from_numpy(wl.weights).to(dev)
    kv = torch.from_numpy(wl.kv).to(dev)
    ks = None
    kscale_addr = None
    if wl.key_kind == "fp8":
        if wl.fused:
            kscale_addr = kv.data_ptr() + wl.ks_offset
        else:
            ks = torch.from_numpy(wl.ks).to(dev)
            kscale_addr = ks.data_ptr() + wl.ks_offset
    pt = torch.from_numpy(wl.page_table).to(dev)
    sl = torch.from_numpy(wl.seqlens).to(dev)
    out = torch.full((wl.rows, wl.ncols), out_fill, dtype=torch.float32, device=dev)
    rt = None if wl.row_table is None else torch.from_numpy(wl.row_table).to(dev)
    return DeviceWorkload(wl, q, w, kv, ks, kscale_addr, pt, sl, out, rt)


def run_library(dw: DeviceWorkload, lib_module, stream=None, check: bool = True) -> int:
    """Call the library entry point matching the workload's key kind (the
    multi-request entry points when rows map to request tables)."""
    wl = dw.wl
    if wl.row_table is not None:
        fn = (lib_module.idx_paged_mqa_logits_varlen_fp8 if wl.key_kind == "fp8"
              else lib_module.idx_paged_mqa_logits_varlen_bf16)
        return fn(dw.q, dw.kv, dw.kscale_addr if wl.key_kind == "fp8" else None, dw.page_table,
                  dw.row_table, dw.seqlens, dw.weights, dw.out, num_tables=wl.num_tables,
                  num_pages=wl.num_pages, table_width=wl.table_width,
                  page_table_row_stride=wl.pt_stride, kv_page_stride=wl.kv_stride,
                  kscale_page_stride=wl.ks_stride if wl.key_kind == "fp8" else 0,
                  rows=wl.rows, stream=stream, check=check)
    if wl.key_kind == "fp8":
        return lib_module.idx_paged_mqa_logits_fp8(
            dw.q, dw.kv, dw.kscale_addr, dw.page_table, dw.seqlens, dw.weights, dw.out,
            rows=wl.rows, table_width=wl.table_width, num_pages=wl.num_pages,
            kv_page_stride=wl.kv_stride, kscale_page_stride=wl.ks_stride,
            page_table_row_stride=wl.pt_stride, stream=stream, check=check)
    return lib_module.idx_paged_mqa_logits_bf16(
        dw.q, dw.kv, None, dw.page_table, dw.seqlens, dw.weights, dw.out, rows=wl.rows,
        table_width=wl.table_width, num_pages=wl.num_pages, kv_page_stride=wl.kv_stride,
        kscale_page_stride=0, page_table_row_stride=wl.pt_stride, stream=stream, check=check)


def run_library_topk(dw: DeviceWorkload, lib_module, topk_idx, topk_val=None, stream=None,
                     check: bool = True) -> int:
    """Call the fused logits + top-k entry point of the workload's key kind; the
    logits go to dw.out (defined only at positions below each row's length)."""
    wl = dw.wl
    if wl.key_kind == "fp8":
        return lib_module.idx_paged_mqa_topk_fp8(
            dw.q, dw.kv, dw.kscale_addr, dw.page_table, dw.seqlens, dw.weights, dw.out, topk_idx,
            topk_val, rows=wl.rows, table_width=wl.table_width, num_pages=wl.num_pages,
            kv_page_stride=wl.kv_stride, kscale_page_stride=wl.ks_stride,
            page_table_row_stride=wl.pt_stride, stream=stream, check=check)
    return lib_module.idx_paged_mqa_topk_bf16(
        dw.q, dw.kv, None, dw.page_table, dw.seqlens, dw.weights, dw.out, topk_idx, topk_val,
        rows=wl.rows, table_width=wl.table_width, num_pages=wl.num_pages,
        kv_page_stride=wl.kv_stride, kscale_page_stride=0, page_table_row_stride=wl.pt_stride,
        stream=stream, check=check)
