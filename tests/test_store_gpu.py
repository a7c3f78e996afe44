"""Paged key store on the GPU against the CPU oracle, called through the C ABI.

The fp8 store is checked byte for byte: its codes and scales are integer /
bit-pattern results of a float32 recipe, so the library must reproduce the
oracle's bytes exactly.  Slots that are skipped (negative or past the pool)
must leave the pool untouched.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from helpers import assert_parity, mask_of, random_slot_workload

pytestmark = pytest.mark.gpu

D, P = W.HEAD_DIM, W.PAGE
FUSED = W.FP8_FUSED_STRIDE


def announce(msg: str) -> None:
    sys.__stderr__.write(f"[gpu] {msg}\n")
    sys.__stderr__.flush()


def keys_bits(rng, n):
    """bf16 keys [n, 128] over several magnitudes, with zero keys, -0 values and
    bf16 subnormals mixed in."""
    k = rng.standard_normal((n, D), dtype=np.float32)
    k *= np.float32(10.0) ** rng.integers(-30, 30, size=(n, 1)).astype(np.float32)
    k[rng.random(n) < 0.03] = 0.0
    neg0 = rng.random((n, D)) < 0.01
    k[neg0] = -0.0
    sub = rng.random((n, D)) < 0.01
    k[sub] = (rng.standard_normal(int(sub.sum())) * 1e-39).astype(np.float32)
    return torch.from_numpy(k).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def expected_pool(pool0, codes, scales, slots, num_pages, kv_stride, ks_pool=None, ks_stride=None,
                  ks_offset=0):
    """Host copy of the pool after storing: oracle bytes at every valid slot."""
    pool = pool0.copy()
    ks = pool if ks_pool is None else ks_pool.copy()
    for t, s in enumerate(slots):
        if s < 0 or s >= num_pages * P:
            continue
        g, i = divmod(int(s), P)
        pool[g * kv_stride + i * D: g * kv_stride + (i + 1) * D] = codes[t]
        o = ks_offset + g * ks_stride + 4 * i
        ks[o:o + 4] = np.frombuffer(scales[t:t + 1].tobytes(), dtype=np.uint8)
    return pool, (None if ks_pool is None else ks)


def store_fp8(lib, bits, slots, num_pages, pool0, kv_stride=FUSED, ks0=None, ks_stride=FUSED,
              ks_offset=P * D):
    keys = torch.from_numpy(bits.view(np.int16).copy()).cuda().view(torch.bfloat16)
    sl = torch.from_numpy(np.asarray(slots, dtype=np.int64)).cuda()
    pool = torch.from_numpy(pool0.copy()).cuda()
    if ks0 is None:
        ks_addr, ks_t = pool.data_ptr() + ks_offset, None
    else:
        ks_t = torch.from_numpy(ks0.copy()).cuda()
        ks_addr = ks_t.data_ptr() + ks_offset
    lib.idx_store_keys_fp8(keys, sl, pool, ks_addr, num_pages=num_pages, kv_page_stride=kv_stride,
                           kscale_page_stride=ks_stride)
    torch.cuda.synchronize()
    return pool.cpu().numpy(), (None if ks_t is None else ks_t.cpu().numpy())


@pytest.mark.parametrize("n,num_pages,seed", [(1, 1, 0), (3, 2, 1), (1000, 40, 2), (5000, 90, 3)])
def test_store_fp8_bit_exact(lib, n, num_pages, seed):
    rng = np.random.default_rng(seed)
    announce(f"store fp8 n={n} pages={num_pages}")
    bits = keys_bits(rng, n)
    cap = num_pages * P
    slots = rng.permutation(cap)[:n].astype(np.int64) if n <= cap else rng.integers(0, cap, n)
    if n > 4:  # skipped keys: padding (-1) and slots past the pool
        slots[rng.random(n) < 0.05] = -1
        slots[rng.random(n) < 0.02] = cap + rng.integers(0, 1000)
    pool0 = rng.integers(0, 256, size=num_pages * FUSED, dtype=np.uint8)  # canary bytes
    got, _ = store_fp8(lib, bits, slots, num_pages, pool0)
    codes, scales = oracle.quantize_keys_fp8(bits)
    want, _ = expected_pool(pool0, codes, scales, slots, num_pages, FUSED, ks_stride=FUSED,
                            ks_offset=P * D)
    assert np.array_equal(got, want)


def test_store_fp8_scale_ranges_bit_exact(lib):
    """Keys whose scale (amax/448) falls below 2^-60, inside [2^-60, 2^100] and
    above 2^100 (largest bf16 magnitudes), and keys whose values are exact
    fractions of their maximum (quotients on e4m3fn rounding ties): the codes
    and scales equal the oracle's bytes."""
    rng = np.random.default_rng(21)
    n = 1536
    k = rng.standard_normal((n, D), dtype=np.float32)
    mags = np.array([1e-35, 1e-20, 1e-16, 1e-3, 1.0, 1e5, 1e29, 3e30, 1e34, 1e38], dtype=np.float32)
    with np.errstate(over="ignore"):
        k = np.clip(k * mags[rng.integers(0, len(mags), size=(n, 1))], -3.3e38, 3.3e38)
    ties = rng.random(n) < 0.25                       # values = (m/256) * amax
    amax = np.abs(k).max(axis=1, keepdims=True)
    frac = rng.integers(-256, 257, size=(n, D)).astype(np.float32) / np.float32(256.0)
    k[ties] = (frac * amax)[ties]
    assert np.isfinite(k).all()
    bits = torch.from_numpy(k).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    num_pages = 24
    slots = rng.permutation(num_pages * P)[:n].astype(np.int64)
    pool0 = rng.integers(0, 256, size=num_pages * FUSED, dtype=np.uint8)
    got, _ = store_fp8(lib, bits, slots, num_pages, pool0)
    codes, scales = oracle.quantize_keys_fp8(bits)
    assert np.isfinite(scales).all()
    assert (scales < 2.0 ** -60).any() and (scales > 2.0 ** 100).any()
    want, _ = expected_pool(pool0, codes, scales, slots, num_pages, FUSED, ks_stride=FUSED,
                            ks_offset=P * D)
    assert np.array_equal(got, want)


def test_store_fp8_split_layout(lib):
    rng = np.random.default_rng(11)
    n, num_pages = 700, 16
    bits = keys_bits(rng, n)
    slots = rng.permutation(num_pages * P)[:n].astype(np.int64)
    kv_stride, ks_stride = P * D + 128, 512  # padded key pages, strided scale rows
    pool0 = rng.integers(0, 256, size=num_pages * kv_stride, dtype=np.uint8)
    ks0 = rng.integers(0, 256, size=num_pages * ks_stride + 64, dtype=np.uint8)
    got, got_ks = store_fp8(lib, bits, slots, num_pages, pool0, kv_stride=kv_stride, ks0=ks0,
                            ks_stride=ks_stride, ks_offset=64)
    codes, scales = oracle.quantize_keys_fp8(bits)
    want, want_ks = expected_pool(pool0, codes, scales, slots, num_pages, kv_stride, ks_pool=ks0,
                                  ks_stride=ks_stride, ks_offset=64)
    assert np.array_equal(got, want)
    assert np.array_equal(got_ks, want_ks)


def test_store_bf16_copies(lib):
    rng = np.random.default_rng(12)
    n, num_pages = 900, 20
    bits = keys_bits(rng, n)
    slots = rng.permutation(num_pages * P)[:n].astype(np.int64)
    slots[::50] = -1
    stride = P * D * 2
    pool0 = rng.integers(0, 256, size=num_pages * stride, dtype=np.uint8)
    keys = torch.from_numpy(bits.view(np.int16).copy()).cuda().view(torch.bfloat16)
    pool = torch.from_numpy(pool0.copy()).cuda()
    lib.idx_store_keys_bf16(keys, torch.from_numpy(slots).cuda(), pool, num_pages=num_pages)
    torch.cuda.synchronize()
    want = pool0.copy()
    for t, s in enumerate(slots):
        if s >= 0:
            g, i = divmod(int(s), P)
            want[g * stride + i * 2 * D: g * stride + (i + 1) * 2 * D] = bits[t].view(np.uint8)
    assert np.array_equal(pool.cpu().numpy(), want)


def test_store_then_score_round_trip(lib):
    """Keys stored by the library and then scored by the library match the
    oracle scoring the oracle-quantised pool (the same bytes)."""
    rng = np.random.default_rng(13)
    wl, bits, slots = random_slot_workload(rng, rows=8, width=12, num_pages=96)
    announce(f"store + score rows={wl.rows} width={wl.table_width}")
    codes, scales = oracle.quantize_keys_fp8(bits)
    pool0 = np.zeros(wl.num_pages * FUSED, dtype=np.uint8)
    want_pool, _ = expected_pool(pool0, codes, scales, slots, wl.num_pages, FUSED, ks_stride=FUSED,
                                 ks_offset=P * D)
    got_pool, _ = store_fp8(lib, bits, slots, wl.num_pages, pool0)
    assert np.array_equal(got_pool, want_pool)
    wl.kv = want_pool
    wl.ks = want_pool
    dw = W.to_device(wl)
    W.run_library(dw, lib)
    torch.cuda.synchronize()
    assert_parity(dw.out.cpu().numpy(), oracle.paged_mqa_logits(wl), mask_of(wl), label="round trip")


def test_store_fp8_large_sampled(lib):
    """The benchmark's size: every slot of a 32,768-page pool written once;
    a sample of keys checked byte for byte."""
    rng = np.random.default_rng(14)
    num_pages = 32768
    n = num_pages * P
    announce(f"store fp8 n={n} (sampled)")
    bits = keys_bits(rng, n)
    slots = rng.permutation(n).astype(np.int64)
    got, _ = store_fp8(lib, bits, slots, num_pages, np.zeros(num_pages * FUSED, dtype=np.uint8))
    pick = rng.choice(n, size=4000, replace=False)
    codes, scales = oracle.quantize_keys_fp8(bits[pick])
    for j, t in enumerate(pick):
        g, i = divmod(int(slots[t]), P)
        assert np.array_equal(got[g * FUSED + i * D: g * FUSED + (i + 1) * D], codes[j])
        o = g * FUSED + P * D + 4 * i
        assert got[o:o + 4].tobytes() == scales[j:j + 1].tobytes()
