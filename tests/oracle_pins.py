"""Pins of the CPU oracle: facts fixed by the pages and by mathematics.

Every pin takes an oracle object (``oracle.Oracle``) so the same checks also
run against deliberately broken oracle builds (tests/test_oracle_mutants.py),
which shows each plausible mistake is caught by at least one pin.

None of these pins retypes the oracle's formula: each one checks a closed
form that a special input reduces the method to, a library routine, an
invariant of the definition, exact rational arithmetic, or a number the
pages print.
"""
from __future__ import annotations

import math
from fractions import Fraction

import numpy as np
import torch

import workloads as W
from helpers import (CODE_ONE, CODE_ZERO, make_workload, mask_of, read_golden_pairs,
                     read_golden_rows, with_width)

H, D, P = W.NUM_HEADS, W.HEAD_DIM, W.PAGE


def _bf16_round(x):
    """Round float32 values to bf16-representable float32 values (library rounding)."""
    return torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.bfloat16).float().numpy()


def _rand_q(rng, rows):
    return _bf16_round(rng.standard_normal((rows, H, D), dtype=np.float32))


def _torch_e4m3(codes) -> np.ndarray:
    """Library decode of e4m3fn codes (torch.float8_e4m3fn -> float64)."""
    t = torch.from_numpy(np.asarray(codes, dtype=np.uint8)).view(torch.float8_e4m3fn)
    return t.to(torch.float64).numpy()


# ---------------------------------------------------------------------------
# storage formats

def pin_e4m3fn_matches_library_decode(ora):
    """All 256 codes agree with torch.float8_e4m3fn (a library routine)."""
    lib = _torch_e4m3(np.arange(256))
    mine = np.array([ora.e4m3fn_value(c) for c in range(256)])
    assert np.array_equal(np.isnan(mine), np.isnan(lib))
    ok = ~np.isnan(lib)
    assert np.array_equal(mine[ok], lib[ok])
    assert np.array_equal(np.signbit(mine[ok]), np.signbit(lib[ok]))


def pin_e4m3fn_spec_values(ora):
    """Closed-form values of the OCP E4M3 format."""
    cases = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6,
             0x38: 1.0, 0x3F: 1.875, 0x40: 2.0, 0x7E: 448.0, 0xFE: -448.0, 0xB8: -1.0,
             0x81: -(2.0 ** -9)}
    for code, val in cases.items():
        assert ora.e4m3fn_value(code) == val, hex(code)
    assert math.copysign(1.0, ora.e4m3fn_value(0x80)) == -1.0 and ora.e4m3fn_value(0x80) == 0.0
    assert math.isnan(ora.e4m3fn_value(0x7F)) and math.isnan(ora.e4m3fn_value(0xFF))
    finite = [abs(ora.e4m3fn_value(c)) for c in range(256) if not math.isnan(ora.e4m3fn_value(c))]
    assert max(finite) == 448.0                              # largest finite value
    assert len(finite) == 254                                # no infinities, 2 NaN codes


def pin_bf16_matches_library_decode(ora):
    rng = np.random.default_rng(7)
    bits = rng.integers(0, 1 << 16, size=4000).astype(np.uint16)
    bits[:6] = [0x0000, 0x8000, 0x3F80, 0x7F80, 0xFF80, 0x0001]
    lib = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    mine = np.array([ora.bf16_value(int(b)) for b in bits])
    nan = np.isnan(lib)
    assert np.array_equal(np.isnan(mine), nan)
    assert np.array_equal(mine[~nan], lib[~nan])
    assert ora.bf16_value(0x3F80) == 1.0 and ora.bf16_value(0xC000) == -2.0


# ---------------------------------------------------------------------------
# closed forms

def pin_one_hot_key_selects_one_product(ora):
    """Key = e_d, w = c*e_h, s = 1/2: logit = c * ReLU(q[h,d] / 2) exactly, 0 for zero keys.

    One row per (h, d, c), each with its own query, weights and page, covering
    the first and last head and dimension, so a dropped term, a transposed
    query, a wrong head/dim/row index shows."""
    rng = np.random.default_rng(11)
    cases = [(0, 0, 3.0), (63, 127, 1.5), (17, 93, -2.0), (40, 5, 0.25), (1, 126, 1.0)]
    rows = len(cases)
    q = _rand_q(rng, rows)
    w = np.zeros((rows, H), dtype=np.float32)
    keys = np.zeros((rows + 1, P, D), dtype=np.uint8)      # page 0 stays all-zero
    for r, (h, d, c) in enumerate(cases):
        q[r, h, d] = 1.5 if c > 0 else -1.25
        w[r, h] = c
        keys[r + 1, 37, d] = CODE_ONE
    scales = np.full((rows + 1, P), 0.5, dtype=np.float32)
    table = [[r + 1, 0] for r in range(rows)]
    wl = make_workload("fp8", q, w, keys, table, [2 * P] * rows, scales)
    out = ora.paged_mqa_logits(wl)
    for r, (h, d, c) in enumerate(cases):
        expect = np.zeros(2 * P)
        expect[37] = c * max(0.5 * float(q[r, h, d]), 0.0)
        assert np.array_equal(out[r], expect), (h, d, c)


def pin_relu_before_weight_and_after_scale(ora):
    """Signs: w*ReLU(s*x).  x=+3,w=-2 -> -6; x=-3,w=-2 -> 0; s=-1/2,x=-4 -> w*2."""
    keys = np.zeros((1, P, D), dtype=np.uint8)
    keys[0, :, 0] = CODE_ONE
    q = np.zeros((3, H, D), dtype=np.float32)
    q[0, 0, 0], q[1, 0, 0], q[2, 0, 0] = 3.0, -3.0, -4.0
    w = np.zeros((3, H), dtype=np.float32)
    w[:, 0] = -2.0
    scales = np.ones((1, P), dtype=np.float32)
    wl = make_workload("fp8", q[:2], w[:2], keys, [[0], [0]], [P, P], scales)
    out = ora.paged_mqa_logits(wl)
    assert np.all(out[0] == -6.0) and np.all(out[1] == 0.0)
    scales_neg = np.full((1, P), -0.5, dtype=np.float32)
    wl = make_workload("fp8", q[2:], w[2:], keys, [[0]], [P], scales_neg)
    assert np.all(ora.paged_mqa_logits(wl)[0] == -4.0)


def pin_negative_dots_give_exact_zero(ora):
    rng = np.random.default_rng(3)
    keys = rng.integers(0x08, 0x70, size=(2, P, D)).astype(np.uint8)   # positive normal codes
    q = -np.abs(_rand_q(rng, 2)) - 0.125                                  # every entry < 0
    w = rng.standard_normal((2, H)).astype(np.float32)
    scales = rng.uniform(0.01, 2.0, size=(2, P)).astype(np.float32)
    wl = make_workload("fp8", _bf16_round(q), w, keys, [[0, 1], [1, 0]], [2 * P, 2 * P], scales)
    out = ora.paged_mqa_logits(wl)
    assert np.all(out == 0.0)


def pin_zero_weights_give_positive_zero(ora):
    wl = W.random_workload(5, "fp8", rows=3, table_width=3, num_pages=9)
    wl.weights[:] = 0.0
    out = ora.paged_mqa_logits(wl)
    m = mask_of(wl)
    assert np.all(out[~m] == 0.0) and not np.signbit(out[~m]).any()
    assert np.all(np.isneginf(out[m]))


def pin_single_head_is_relu_of_matvec(ora):
    """w = e_h reduces the method to ReLU(s * K q_h): checked against numpy's float64 matmul."""
    rng = np.random.default_rng(21)
    for kind in ("fp8", "bf16"):
        wl = W.random_workload(31, kind, rows=2, table_width=3, num_pages=6,
                               seqlens=[3 * P, 2 * P + 17])
        h = 45
        wl.weights[:] = 0.0
        wl.weights[:, h] = 1.0
        out = ora.paged_mqa_logits(wl)
        qf = torch.from_numpy(wl.q.view(np.int16)).view(torch.bfloat16).double().numpy()
        for b in range(wl.rows):
            L = int(wl.lengths()[b])
            for j in range((L + P - 1) // P):
                g = int(wl.page_table[b * wl.pt_stride + j])
                if kind == "fp8":
                    blk = wl.kv[g * wl.kv_stride: g * wl.kv_stride + W.FP8_KEY_BYTES]
                    K = _torch_e4m3(blk).reshape(P, D)
                    s = wl.ks[wl.ks_offset + g * wl.ks_stride:][:W.FP8_SCALE_BYTES].view(np.float32)
                else:
                    blk = wl.kv[g * wl.kv_stride: g * wl.kv_stride + W.BF16_PAGE_BYTES]
                    K = torch.from_numpy(blk.view(np.int16).copy()).view(torch.bfloat16).double().numpy().reshape(P, D)
                    s = np.ones(P)
                ref = np.maximum(s.astype(np.float64) * (K @ qf[b, h]), 0.0)
                n = min(P, L - j * P)
                got = out[b, j * P: j * P + n]
                assert np.allclose(got, ref[:n], rtol=1e-13, atol=1e-13), (kind, b, j)


def pin_exact_rational_brute_force(ora):
    """Tiny input against exact rational arithmetic (every input is a dyadic rational)."""
    for kind in ("fp8", "bf16"):
        wl = W.random_workload(77, kind, rows=1, table_width=2, num_pages=3, seqlens=[P + 9])
        out = ora.paged_mqa_logits(wl)[0]
        qf = torch.from_numpy(wl.q.view(np.int16)).view(torch.bfloat16).double().numpy()[0]
        for j in range(2):
            g = int(wl.page_table[j])
            for i in (0, 1, 2, 31, 62, 63) if j == 0 else (0, 7, 8, 9, 10, 63):
                p = j * P + i
                if p >= P + 9:
                    assert np.isneginf(out[p])
                    continue
                if kind == "fp8":
                    codes = wl.kv[g * wl.kv_stride + i * D: g * wl.kv_stride + (i + 1) * D]
                    k = [Fraction(float(v)) for v in _torch_e4m3(codes)]
                    off = wl.ks_offset + g * wl.ks_stride + 4 * i
                    s = Fraction(float(wl.ks[off:off + 4].view(np.float32)[0]))
                else:
                    base = g * wl.kv_stride + i * 2 * D
                    bits = wl.kv[base: base + 2 * D].view(np.int16).copy()
                    k = [Fraction(float(v)) for v in torch.from_numpy(bits).view(torch.bfloat16).double().numpy()]
                    s = Fraction(1)
                acc = Fraction(0)
                for h in range(H):
                    dot = sum((Fraction(float(qf[h, d])) * k[d] for d in range(D)), Fraction(0))
                    x = s * dot
                    acc += Fraction(float(wl.weights[0, h])) * (x if x > 0 else Fraction(0))
                exact = float(acc)
                assert abs(out[p] - exact) <= 1e-12 * max(1.0, abs(exact)), (kind, p, out[p], exact)


# ---------------------------------------------------------------------------
# indexing, masking, layout

def pin_position_tags_follow_page_table(ora):
    """Key e_0 with scale tag(g, i) = (64 g + i + 1) / 2^16, q_0 = e_0, w = e_0:
    logit[b, 64 j + i] = tag(page_table[b][j], i) exactly.  Several rows, a
    table stride wider than the table, fused and split scale layouts."""
    rng = np.random.default_rng(9)
    pages, rows, width, stride = 7, 3, 4, 6
    keys = np.zeros((pages, P, D), dtype=np.uint8)
    keys[:, :, 0] = CODE_ONE
    g_idx, i_idx = np.meshgrid(np.arange(pages), np.arange(P), indexing="ij")
    tags = ((P * g_idx + i_idx + 1) / 2.0 ** 16).astype(np.float32)
    q = np.zeros((rows, H, D), dtype=np.float32)
    q[:, 0, 0] = 1.0
    w = np.zeros((rows, H), dtype=np.float32)
    w[:, 0] = 1.0
    table = np.full((rows, stride), 99, dtype=np.int32)
    for b in range(rows):
        table[b, :width] = rng.permutation(pages)[:width]
    seq = [width * P, 2 * P + 5, P - 1]
    for layout in ("fused", "split"):
        wl = make_workload("fp8", q, w, keys, table, seq, tags, layout=layout,
                           pt_stride=stride, width=width)
        out = ora.paged_mqa_logits(wl)
        for b in range(rows):
            for j in range(width):
                for i in range(P):
                    p = j * P + i
                    want = float(tags[table[b, j], i]) if p < seq[b] else -np.inf
                    assert out[b, p] == want, (layout, b, j, i)


def pin_shared_table_equals_copies(ora):
    base = W.random_workload(12, "bf16", rows=5, table_width=3, num_pages=4,
                             shared_table=True, seqlens=[1, 64, 65, 130, 192])
    import dataclasses
    tab = np.tile(base.page_table[:3], 5)
    copy = dataclasses.replace(base, page_table=tab, pt_stride=3)
    assert np.array_equal(ora.paged_mqa_logits(base), ora.paged_mqa_logits(copy), equal_nan=True)


def pin_request_map_equals_expanded_tables(ora):
    """Rows mapped to request tables score exactly as rows given copies of
    their request's table; an index outside the tables gives NaN at the
    row's live positions."""
    import dataclasses
    base = W.varlen_workload(14, "fp8", tokens=[3, 1, 4], contexts=[150, 64, 260], table_width=5,
                             num_pages=16, interleave=True)
    tabs = base.page_table.reshape(3, 5)
    copy = dataclasses.replace(base, page_table=tabs[base.row_table].reshape(-1).copy(), pt_stride=5,
                               row_table=None, num_tables=0)
    got = ora.paged_mqa_logits(base)
    assert np.array_equal(got, ora.paged_mqa_logits(copy), equal_nan=True)
    assert np.all(np.isfinite(got[~mask_of(base)]))
    # only tables 0 and 1 declared (table 2 stays in the buffer): rows of
    # request 2 and a negative index are outside
    bad = dataclasses.replace(base, row_table=base.row_table.copy(), num_tables=2)
    bad.row_table[0] = -1
    out = ora.paged_mqa_logits(bad)
    m = mask_of(bad)
    for b in range(bad.rows):
        want_nan = bad.row_table[b] < 0 or bad.row_table[b] >= 2
        assert np.all(np.isnan(out[b][~m[b]]) == want_nan) and np.all(np.isneginf(out[b][m[b]]))
    assert (bad.row_table == 2).sum() == 4 and bad.lengths()[0] > 0


def pin_mask_edges(ora):
    """-inf exactly at p >= clamp(seqlen, 0, 64*width); finite below; padding never read."""
    seq = [0, 1, 63, 64, 65, 3 * P - 1, 3 * P, 3 * P + 5, -3, 2 ** 31 - 1, -2 ** 31]
    wl = W.random_workload(4, "fp8", rows=len(seq), table_width=3, num_pages=40, seqlens=seq,
                           pad=-1)
    out = ora.paged_mqa_logits(wl)
    m = mask_of(wl)
    assert np.array_equal(np.isneginf(out), m)
    assert np.all(np.isfinite(out[~m]))
    L = wl.lengths()
    assert list(L) == [0, 1, 63, 64, 65, 191, 192, 192, 0, 192, 0]


def pin_invalid_page_id_gives_nan(ora):
    wl = W.random_workload(8, "fp8", rows=2, table_width=3, num_pages=4, seqlens=[150, 150])
    wl.page_table[1] = 4            # row 0, slot 1: one past the pool
    wl.page_table[3 + 2] = -7       # row 1, slot 2: negative
    out = ora.paged_mqa_logits(wl)
    assert np.all(np.isnan(out[0, 64:128])) and np.all(np.isfinite(out[0, :64]))
    assert np.all(np.isnan(out[1, 128:150])) and np.all(np.isneginf(out[1, 150:]))
    assert np.all(np.isfinite(out[1, :128])) and np.all(np.isfinite(out[0, 128:150]))


def pin_nan_key_code_propagates(ora):
    wl = W.random_workload(13, "fp8", rows=1, table_width=1, num_pages=1, seqlens=[P])
    blk = wl.kv.reshape(1, -1)
    blk[0, 5 * D + 77] = 0x7F       # position 5, dim 77 -> NaN
    out = ora.paged_mqa_logits(wl)[0]
    assert np.isnan(out[5]) and np.isfinite(np.delete(out, 5)).all()


# ---------------------------------------------------------------------------
# invariants

def pin_linearity_in_weights(ora):
    wl = W.random_workload(14, "fp8", rows=3, table_width=2, num_pages=6)
    import dataclasses
    rng = np.random.default_rng(1)
    w1 = rng.standard_normal((3, H)).astype(np.float32)
    w2 = rng.standard_normal((3, H)).astype(np.float32)
    o1 = ora.paged_mqa_logits(dataclasses.replace(wl, weights=w1))
    o2 = ora.paged_mqa_logits(dataclasses.replace(wl, weights=w2))
    o12 = ora.paged_mqa_logits(dataclasses.replace(wl, weights=(w1 + w2)))  # float32 sum
    w12 = w1.astype(np.float64) + w2.astype(np.float64)
    exact_sum = (w1 + w2).astype(np.float64) == w12
    m = mask_of(wl)
    assert np.array_equal(np.isneginf(o12), m)
    if exact_sum.all():
        scale = np.abs(o1[~m]).max() + np.abs(o2[~m]).max()
        assert np.abs(o12[~m] - (o1[~m] + o2[~m])).max() <= 1e-12 * scale
    o4 = ora.paged_mqa_logits(dataclasses.replace(wl, weights=(w1 * 4).astype(np.float32)))
    assert np.array_equal(o4[~m], 4 * o1[~m])


def pin_power_of_two_scale_homogeneity(ora):
    wl = W.random_workload(15, "fp8", rows=2, table_width=2, num_pages=5, layout="split")
    import dataclasses
    ks2 = (wl.ks.view(np.float32) * np.float32(4.0)).view(np.uint8)
    o1 = ora.paged_mqa_logits(wl)
    o4 = ora.paged_mqa_logits(dataclasses.replace(wl, ks=ks2))
    m = mask_of(wl)
    assert np.array_equal(o4[~m], 4 * o1[~m])


def pin_pool_permutation_invariance(ora):
    import dataclasses
    for kind in ("fp8", "bf16"):
        wl = W.random_workload(16, kind, rows=4, table_width=3, num_pages=12)
        perm = np.random.default_rng(2).permutation(wl.num_pages)   # new slot of page g
        stride = wl.kv_stride
        blocks = wl.kv.reshape(wl.num_pages, stride)
        new_blocks = np.empty_like(blocks)
        new_blocks[perm] = blocks
        kv2 = new_blocks.reshape(-1)
        tab = wl.page_table.copy()
        live = tab >= 0
        tab[live] = perm[tab[live]]
        wl2 = dataclasses.replace(wl, kv=kv2, ks=(kv2 if wl.ks is not None else None),
                                  page_table=tab)
        assert np.array_equal(ora.paged_mqa_logits(wl), ora.paged_mqa_logits(wl2))


def pin_width_and_row_subset_invariance(ora):
    import dataclasses
    wl = W.random_workload(17, "fp8", rows=4, table_width=3, num_pages=12)
    out = ora.paged_mqa_logits(wl)
    wide_tab = np.full((4, 7), -1, dtype=np.int32)
    wide_tab[:, :3] = wl.page_table.reshape(4, 3)
    wide = dataclasses.replace(wl, table_width=7, page_table=wide_tab.reshape(-1), pt_stride=7)
    ow = ora.paged_mqa_logits(wide)
    assert np.array_equal(ow[:, :3 * P], out)
    assert np.all(np.isneginf(ow[:, 3 * P:]))
    sub = ora.paged_mqa_logits(wl, rows=[3, 1])
    assert np.array_equal(sub, out[[3, 1]])


def pin_fp8_and_bf16_agree_on_representable_keys(ora):
    """fp8 keys with s = 1 and the same values stored as bf16 give identical logits."""
    rng = np.random.default_rng(19)
    codes = rng.integers(0, 0x7F, size=(2, P, D)).astype(np.uint8)
    codes |= (rng.integers(0, 2, size=codes.shape) << 7).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x10
    vals = _torch_e4m3(codes).astype(np.float32)
    q = _rand_q(rng, 2)
    w = rng.standard_normal((2, H)).astype(np.float32)
    seq = [2 * P, P + 3]
    a = make_workload("fp8", q, w, codes, [[0, 1], [1, 0]], seq, np.ones((2, P), np.float32))
    b = make_workload("bf16", q, w, vals, [[0, 1], [1, 0]], seq)
    assert np.array_equal(ora.paged_mqa_logits(a), ora.paged_mqa_logits(b))


# ---------------------------------------------------------------------------
# numbers printed on the pages

def pin_pages_block_layout(ora):
    g = read_golden_pairs("pages_layout.txt")
    assert g["block_bytes"] == g["block_positions"] * (g["block_values_per_position"]
                                                         + g["block_scale_bytes"])
    assert g["block_positions"] == P and g["block_values_per_position"] == D
    assert g["block_bytes"] == W.FP8_FUSED_STRIDE
    assert g["block_fp8_bytes_per_position"] * g["block_positions"] == W.FP8_KEY_BYTES
    assert g["bf16_bytes_per_position"] * P == W.BF16_PAGE_BYTES
    assert g["width_full_pages"] * P == g["width_full_positions"]
    assert g["width_capped_pages"] * P == g["width_capped_positions"]
    # a hand-assembled 8448-byte block read through the fused layout
    keys = np.zeros((1, P, D), dtype=np.uint8)
    keys[0, 63, 127] = 0x40                      # 2.0 at the last value of the last position
    scales = np.zeros((1, P), dtype=np.float32)
    scales[0, 63] = 0.75
    q = np.zeros((1, H, D), dtype=np.float32)
    q[0, 9, 127] = 1.0
    w = np.zeros((1, H), dtype=np.float32)
    w[0, 9] = 1.0
    wl = make_workload("fp8", q, w, keys, [[0]], [P], scales)
    blk = wl.kv.reshape(-1)
    assert blk.size == g["block_bytes"]
    assert blk[63 * D + 127] == 0x40 and blk[8192 + 4 * 63: 8192 + 4 * 64].view(np.float32)[0] == 0.75
    out = ora.paged_mqa_logits(wl)[0]
    assert out[63] == 1.5 and np.all(out[:63] == 0.0)
    # full-width table of the pages: 4097 slots -> 262,208 columns, -inf after the length
    wl = W.random_workload(18, "fp8", rows=1, table_width=g["width_full_pages"], num_pages=2,
                           seqlens=[100])
    out = ora.paged_mqa_logits(wl)
    assert out.shape == (1, g["width_full_positions"])
    assert np.all(np.isfinite(out[0, :100])) and np.all(np.isneginf(out[0, 100:]))


def pin_pages_accuracy_bar(ora):
    """The parity bar admits the agreement the pages report for their own kernel."""
    from helpers import ATOL, RTOL
    rows = read_golden_rows("pages_accuracy.txt")
    assert len(rows) == 5
    for b, pages, smax, max_abs, rel in rows:
        assert max_abs <= ATOL and rel <= RTOL
        assert smax == pages * P


# --- key store (fp8 quantiser) ----------------------------------------------

def _keys_bits(rng, n, scale=1.0):
    k = (rng.standard_normal((n, D), dtype=np.float32) * np.float32(scale))
    return torch.from_numpy(k).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _bits_to_f32(bits):
    return (np.asarray(bits, dtype=np.uint32) << 16).view(np.float32)


def pin_e4m3fn_encode_matches_library_cast(ora):
    """Nearest-even encoding equals torch's float8_e4m3fn cast over a dense
    sweep of [-448, 448] that includes every tie between neighbouring codes."""
    vals = np.array([ora.e4m3fn_value(c) for c in range(0x7F)], dtype=np.float64)
    mids = (vals[:-1] + vals[1:]) / 2  # ties: exactly representable in float32
    ys = np.concatenate([mids, -mids, vals, -vals,
                         np.linspace(-448, 448, 4001),
                         np.arange(-64, 65) * 2.0 ** -12]).astype(np.float32)
    ref = torch.from_numpy(ys).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([ora.e4m3fn_encode(float(y)) for y in ys], dtype=np.uint8)
    assert np.array_equal(got, ref)


def pin_e4m3fn_encode_round_trips_every_code(ora):
    """Every finite code decodes to a value that encodes back to the same code."""
    for c in list(range(0x7F)) + list(range(0x80, 0xFF)):
        assert ora.e4m3fn_encode(ora.e4m3fn_value(c)) == c, hex(c)


def pin_quantiser_matches_library_recipe(ora):
    """Codes and scales equal the library route: scale = amax/448 in float32,
    torch's e4m3fn cast of the clamped quotient (the generators' recipe)."""
    rng = np.random.Generator(np.random.PCG64(7))
    bits = np.concatenate([_keys_bits(rng, 200), _keys_bits(rng, 40, 1e-3), _keys_bits(rng, 40, 300.0)])
    codes, scales = ora.quantize_keys_fp8(bits)
    ref_codes, ref_scales = W.quantize_fp8(_bits_to_f32(bits))
    assert np.array_equal(scales.view(np.uint32), ref_scales.view(np.uint32))
    assert np.array_equal(codes, ref_codes)


def pin_quantiser_closed_forms(ora):
    """amax element -> +-448; one-hot key -> one code; zero key -> scale 1 and
    codes 0; keys that are scale * (an e4m3fn value) come back exactly."""
    one_hot = np.zeros((1, D), dtype=np.float32)
    one_hot[0, 17] = -3.5
    zero = np.zeros((1, D), dtype=np.float32)
    rng = np.random.Generator(np.random.PCG64(8))
    codes_in = rng.integers(0, 0x7F, size=(1, D))
    codes_in[0, 5] = 0x7E  # 448 present: amax / 448 is exactly the scale
    vals = np.array([ora.e4m3fn_value(int(c)) for c in codes_in[0]], dtype=np.float32)
    exact = (vals * np.float32(0.25))[None, :]  # a power-of-two scale keeps bf16 exactness
    k = np.concatenate([one_hot, zero, exact])
    bits = torch.from_numpy(k).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(_bits_to_f32(bits), k)  # every input is exactly bf16
    codes, scales = ora.quantize_keys_fp8(bits)
    assert scales[0] == np.float32(3.5) / np.float32(448.0)
    assert codes[0, 17] == 0xFE and np.all(np.delete(codes[0], 17) == 0)
    assert scales[1] == 1.0 and np.all(codes[1] == 0)
    assert scales[2] == np.float32(0.25) and np.array_equal(codes[2], codes_in[0].astype(np.uint8))


# ---------------------------------------------------------------------------
# top-k over the logits

def _brute_topk(vals, L, k):
    """Exhaustive search over every index set of size min(k, L) in [0, L):
    keep the sets whose values, listed largest first (NaN below every number),
    form the largest sequence, and of those the set whose sorted positions form
    the smallest sequence."""
    import itertools

    def desc(ix):
        return sorted(((0, 0.0) if math.isnan(vals[i]) else (1, float(vals[i])) for i in ix),
                      reverse=True)

    m = min(k, max(L, 0))
    best = None
    for ix in itertools.combinations(range(max(L, 0)), m):
        key = desc(ix)
        if best is None or key > best[0] or (key == best[0] and list(ix) < best[1]):
            best = (key, list(ix))
    return best[1] + [-1] * (k - m)


def pin_topk_brute_force_tiny(ora):
    """Rows of at most 8 values drawn from a small set (repeats, +-0, NaN,
    +-inf), any length and k: the oracle equals exhaustive search."""
    rng = np.random.Generator(np.random.PCG64(21))
    pool = np.array([0.0, -0.0, 1.0, -1.0, 2.5, np.nan, np.inf, -np.inf], dtype=np.float32)
    for _ in range(400):
        ncols = int(rng.integers(1, 9))
        k = int(rng.integers(0, 7))
        vals = pool[rng.integers(0, len(pool), size=(1, ncols))]
        L = int(rng.integers(-2, ncols + 3))
        got = ora.topk(vals, [L], k)[0].tolist()
        want = _brute_topk(vals[0], min(L, ncols), k)
        assert got == want, (vals.tolist(), L, k, got, want)


def pin_topk_matches_library_topk(ora):
    """Distinct values: the set equals torch.topk's (a library routine), in
    ascending position order; rows shorter than k return every position."""
    rng = np.random.Generator(np.random.PCG64(22))
    rows, ncols, k = 6, 5000, 2048
    vals = rng.permutation(rows * ncols).reshape(rows, ncols).astype(np.float32) - 7000.0
    seqlens = np.array([5000, 4000, 2049, 2048, 100, 0], dtype=np.int32)
    got = ora.topk(vals, seqlens, k)
    for b in range(rows):
        L = int(seqlens[b])
        if L >= k:
            ref = torch.topk(torch.from_numpy(vals[b, :L]), k).indices.sort().values.numpy()
            assert np.array_equal(got[b], ref)
        else:
            assert np.array_equal(got[b, :L], np.arange(L)) and np.all(got[b, L:] == -1)


def pin_topk_closed_forms(ora):
    """Equal values -> the first k positions; increasing -> the last k of
    [0, L); decreasing -> the first k; L <= 0 -> all -1; seqlen past the row
    clamps to it; +0 and -0 tie; NaN ranks below -inf."""
    n, k = 50, 7
    eq = np.full((1, n), 3.0, dtype=np.float32)
    inc = np.arange(n, dtype=np.float32)[None, :]
    assert ora.topk(eq, [n], k)[0].tolist() == list(range(k))
    assert ora.topk(inc, [30], k)[0].tolist() == list(range(23, 30))
    assert ora.topk(-inc, [30], k)[0].tolist() == list(range(k))
    assert ora.topk(inc, [0], k)[0].tolist() == [-1] * k
    assert ora.topk(inc, [-5], k)[0].tolist() == [-1] * k
    assert ora.topk(inc, [10 ** 6], 3)[0].tolist() == [n - 3, n - 2, n - 1]
    zeros = np.array([[-0.0, 0.0, -0.0, 0.0]], dtype=np.float32)
    assert ora.topk(zeros, [4], 2)[0].tolist() == [0, 1]
    nan = np.array([[np.nan, 1.0, np.nan, -np.inf]], dtype=np.float32)
    assert ora.topk(nan, [4], 2)[0].tolist() == [1, 3]
    assert ora.topk(nan, [4], 3)[0].tolist() == [0, 1, 3]
    assert ora.topk(nan, [4], 0).shape == (1, 0)


def pin_topk_threshold_split(ora):
    """Large rows with many ties: every selected value is >= every candidate
    left out, and of the values equal to the k-th largest the selected ones
    are those at the lowest positions."""
    rng = np.random.Generator(np.random.PCG64(23))
    rows, ncols, k = 4, 20000, 2048
    vals = np.round(rng.standard_normal((rows, ncols)) * 3, 1).astype(np.float32)
    seqlens = np.array([20000, 15000, 3000, 2100], dtype=np.int32)
    got = ora.topk(vals, seqlens, k)
    for b in range(rows):
        L = int(seqlens[b])
        sel = got[b]
        assert np.all(np.diff(sel) > 0) and sel[0] >= 0 and sel[-1] < L
        mask = np.zeros(L, dtype=bool)
        mask[sel] = True
        v = vals[b, :L]
        kth = np.sort(v)[::-1][k - 1]
        assert v[mask].min() == kth and v[~mask].max() <= kth
        tied = np.flatnonzero(v == kth)
        n_above = int((v > kth).sum())
        assert np.array_equal(np.flatnonzero(mask & (v == kth)), tied[:k - n_above])


# cheap pins first; the exact rational brute force last
ALL_PINS = sorted((v for k, v in globals().items() if k.startswith("pin_")),
                  key=lambda f: (f is pin_exact_rational_brute_force, f.__name__))
