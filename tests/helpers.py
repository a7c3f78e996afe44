"""Builders for hand-made workloads and comparison utilities shared by tests."""
from __future__ import annotations

import math
from pathlib import Path

import numpy as np
import torch

import workloads as W

GOLDEN = Path(__file__).resolve().parent / "golden"

CODE_ONE = 0x38        # e4m3fn 1.0
CODE_ZERO = 0x00

# Parity bar on finite logits (max |d| and max |d| / max |oracle|).
ATOL = 2e-2
RTOL = 5e-3


def bf16_bits(x) -> np.ndarray:
    """bf16 bits of values that must already be exactly representable in bf16."""
    x = np.asarray(x, dtype=np.float32)
    bits = W.to_bf16_bits(x)
    back = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).float().numpy()
    ok = (back == x) | (np.isnan(back) & np.isnan(x))
    assert ok.all(), "value not representable in bf16"
    return bits


def make_workload(key_kind: str, q: np.ndarray, weights: np.ndarray, keys: np.ndarray,
                  table: np.ndarray, seqlens, scales: np.ndarray | None = None,
                  layout: str = "fused", pt_stride: int | None = None,
                  num_pages: int | None = None, width: int | None = None) -> W.Workload:
    """Workload from explicit contents.

    q        float [rows, 64, 128] (bf16-exact values)
    weights  float32 [rows, 64]
    keys     fp8: uint8 codes [pages, 64, 128]; bf16: float (bf16-exact) [pages, 64, 128]
    scales   fp8 only: float32 [pages, 64]
    table    int32 [rows or 1, >= width] (row stride = its second dim unless given)
    """
    q = np.asarray(q, dtype=np.float32)
    rows = q.shape[0]
    table = np.asarray(table, dtype=np.int32)
    if table.ndim == 1:
        table = table[None, :]
    pages = keys.shape[0]
    if key_kind == "fp8":
        codes = np.asarray(keys, dtype=np.uint8).reshape(pages, -1)
        sc = np.asarray(scales, dtype=np.float32).reshape(pages, W.PAGE)
        if layout == "fused":
            kv = np.zeros((pages, W.FP8_FUSED_STRIDE), dtype=np.uint8)
            kv[:, :W.FP8_KEY_BYTES] = codes
            kv[:, W.FP8_KEY_BYTES:] = sc.view(np.uint8).reshape(pages, -1)
            kv = kv.reshape(-1)
            ks, ks_off, ks_stride, kv_stride = kv, W.FP8_KEY_BYTES, W.FP8_FUSED_STRIDE, W.FP8_FUSED_STRIDE
        else:
            kv = codes.reshape(-1).copy()
            ks = sc.view(np.uint8).reshape(-1).copy()
            ks_off, ks_stride, kv_stride = 0, W.FP8_SCALE_BYTES, W.FP8_KEY_BYTES
    else:
        kv = bf16_bits(keys).reshape(-1).view(np.uint8).copy()
        ks, ks_off, ks_stride, kv_stride = None, 0, 0, W.BF16_PAGE_BYTES
    if pt_stride is None:
        pt_stride = 0 if (table.shape[0] == 1 and rows > 1) else table.shape[1]
    if width is None:
        width = table.shape[1]
    return W.Workload(name="hand", key_kind=key_kind, rows=rows, table_width=width,
                      num_pages=pages if num_pages is None else num_pages,
                      q=bf16_bits(q), weights=np.asarray(weights, dtype=np.float32),
                      kv=kv, kv_stride=kv_stride, ks=ks, ks_offset=ks_off, ks_stride=ks_stride,
                      page_table=table.reshape(-1).copy(), pt_stride=pt_stride,
                      seqlens=np.asarray(seqlens, dtype=np.int64).astype(np.int32))


def with_width(wl: W.Workload, width: int) -> W.Workload:
    import dataclasses
    return dataclasses.replace(wl, table_width=width)


def read_golden_pairs(name: str) -> dict[str, int]:
    out = {}
    for line in (GOLDEN / name).read_text().splitlines():
        line = line.strip()
        if line and not line.startswith("#"):
            k, v = line.split()
            out[k] = int(v)
    return out


def read_golden_rows(name: str) -> list[list[float]]:
    rows = []
    for line in (GOLDEN / name).read_text().splitlines():
        line = line.strip()
        if line and not line.startswith("#"):
            rows.append([float(x) for x in line.split()])
    return rows


def mask_of(wl: W.Workload) -> np.ndarray:
    """Expected -inf pattern: True where position >= clamp(seqlen)."""
    p = np.arange(wl.ncols)[None, :]
    return p >= wl.lengths()[:, None]


def compare(got: np.ndarray, ref: np.ndarray, mask: np.ndarray | None = None):
    """Parity statistics of library output vs oracle output (same shape).

    Returns dict with max_abs, rel, inf_pattern_match, nan_match, bad_inf.
    """
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    ref_ninf = np.isneginf(ref)
    got_ninf = np.isneginf(got)
    ref_nan = np.isnan(ref)
    got_nan = np.isnan(got)
    fin = np.isfinite(ref)
    both = fin & np.isfinite(got)
    diff = np.abs(got[both] - ref[both])
    max_abs = float(diff.max()) if diff.size else 0.0
    ref_max = float(np.abs(ref[fin]).max()) if fin.any() else 0.0
    return {
        "max_abs": max_abs,
        "rel": max_abs / ref_max if ref_max > 0 else 0.0,
        "inf_pattern_match": bool(np.array_equal(ref_ninf, got_ninf)),
        "mask_match": True if mask is None else bool(np.array_equal(got_ninf, mask)),
        "nan_match": bool(np.array_equal(ref_nan, got_nan)),
        "finite_match": bool(np.array_equal(fin, np.isfinite(got))),
        "posinf": bool(np.isposinf(got).any()),
        "n_finite": int(fin.sum()),
    }


def assert_parity(got, ref, mask=None, atol=ATOL, rtol=RTOL, label=""):
    st = compare(got, ref, mask)
    msg = f"{label}: {st}"
    assert st["inf_pattern_match"], msg
    assert st["mask_match"], msg
    assert st["nan_match"], msg
    assert st["finite_match"], msg
    assert not st["posinf"], msg
    assert st["max_abs"] <= atol, msg
    assert st["rel"] <= rtol, msg
    return st


def random_slot_workload(rng, rows: int, width: int, num_pages: int):
    """fp8 workload whose pool is left empty for the key store to fill.

    Returns (workload, keys as bf16 bits [n, 128], slots [n]) with one key for
    every slot of the pool in a random order; q, w, tables and lengths are
    random (tables draw distinct pages per row).
    """
    q = W.to_bf16_bits(rng.standard_normal((rows, W.NUM_HEADS, W.HEAD_DIM), dtype=np.float32))
    w = (rng.standard_normal((rows, W.NUM_HEADS)) / 8).astype(np.float32)
    table = np.stack([rng.permutation(num_pages)[:width] for _ in range(rows)]).astype(np.int32)
    seqlens = rng.integers(1, width * W.PAGE + 1, size=rows).astype(np.int32)
    n = num_pages * W.PAGE
    bits = W.to_bf16_bits(rng.standard_normal((n, W.HEAD_DIM), dtype=np.float32))
    slots = rng.permutation(n).astype(np.int64)
    kv = np.zeros(num_pages * W.FP8_FUSED_STRIDE, dtype=np.uint8)
    wl = W.Workload(name="stored keys", key_kind="fp8", rows=rows, table_width=width,
                    num_pages=num_pages, q=q, weights=w, kv=kv, kv_stride=W.FP8_FUSED_STRIDE,
                    ks=kv, ks_offset=W.FP8_KEY_BYTES, ks_stride=W.FP8_FUSED_STRIDE,
                    page_table=table.reshape(-1).copy(), pt_stride=width, seqlens=seqlens)
    return wl, bits, slots
