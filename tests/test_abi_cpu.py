"""The C-ABI library loads on the CPU host and exports what the header declares.

No kernel is launched here: only entry points whose arguments fail host-side
validation are called, and those return before any HIP call.
"""
import ctypes
import re
import subprocess
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parent.parent
HEADER = ROOT / "include" / "paged_mqa_logits.h"
LIB = ROOT / "paged_mqa_logits_idx_amd" / "libidx_paged_mqa.so"

IDX_OK, IDX_ERR_NULL, IDX_ERR_UNSUPPORTED, IDX_ERR_SHAPE, IDX_ERR_ALIGN = 0, -1, -2, -3, -4


def declared_functions():
    text = HEADER.read_text()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(idx_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not LIB.exists():
        pytest.fail(f"{LIB} not built (run __graft_entry__.build())")
    l = ctypes.CDLL(str(LIB))
    args = [ctypes.c_void_p] * 7 + [ctypes.c_int32] * 4 + [ctypes.c_int64] * 4 + [ctypes.c_void_p]
    for name in ("idx_paged_mqa_logits_fp8", "idx_paged_mqa_logits_bf16"):
        getattr(l, name).argtypes = args
        getattr(l, name).restype = ctypes.c_int
    l.idx_store_keys_fp8.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                                     ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                     ctypes.c_void_p]
    l.idx_store_keys_fp8.restype = ctypes.c_int
    l.idx_store_keys_bf16.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                                      ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p]
    l.idx_store_keys_bf16.restype = ctypes.c_int
    l.idx_topk_logits.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int32,
                                  ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p,
                                  ctypes.c_void_p]
    l.idx_topk_logits.restype = ctypes.c_int
    for name in ("idx_paged_mqa_logits_varlen_fp8", "idx_paged_mqa_logits_varlen_bf16"):
        getattr(l, name).argtypes = args[:4] + [ctypes.c_void_p, ctypes.c_int32] + args[4:]
        getattr(l, name).restype = ctypes.c_int
    for name in ("idx_paged_mqa_topk_fp8", "idx_paged_mqa_topk_bf16"):
        getattr(l, name).argtypes = args[:-1] + [ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p,
                                                 ctypes.c_void_p]
        getattr(l, name).restype = ctypes.c_int
    l.idx_status_string.restype = ctypes.c_char_p
    l.idx_status_string.argtypes = [ctypes.c_int]
    return l


def test_header_declares_the_entry_points():
    assert declared_functions() == sorted([
        "idx_abi_version", "idx_paged_mqa_logits_bf16", "idx_paged_mqa_logits_fp8",
        "idx_paged_mqa_logits_varlen_bf16", "idx_paged_mqa_logits_varlen_fp8",
        "idx_paged_mqa_topk_bf16", "idx_paged_mqa_topk_fp8", "idx_status_string",
        "idx_store_keys_bf16", "idx_store_keys_fp8", "idx_topk_logits"])


def test_every_declared_symbol_is_exported(lib):
    dyn = subprocess.run(["nm", "-D", "--defined-only", str(LIB)], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (idx_[a-z0-9_]+)$", dyn, flags=re.M))
    for name in declared_functions():
        assert name in exported, name
        assert hasattr(lib, name)


def test_version_and_status_strings(lib):
    assert lib.idx_abi_version() == 1
    for st in (IDX_OK, IDX_ERR_NULL, IDX_ERR_UNSUPPORTED, IDX_ERR_SHAPE, IDX_ERR_ALIGN, -5, 99):
        assert isinstance(lib.idx_status_string(st), bytes) and lib.idx_status_string(st)


def _call(lib, name, **kw):
    a = dict(q=16, kv=16, ks=16, pt=4, sl=4, w=16, out=16, rows=1, heads=64, dim=128, width=1,
             num_pages=1, kv_stride=8448, ks_stride=8448, pt_stride=1)
    if name.endswith("bf16"):
        a.update(ks=None, kv_stride=16384, ks_stride=0)
    a.update(kw)
    fn = getattr(lib, name)
    return fn(a["q"], a["kv"], a["ks"], a["pt"], a["sl"], a["w"], a["out"], a["rows"],
              a["heads"], a["dim"], a["width"], a["num_pages"], a["kv_stride"], a["ks_stride"],
              a["pt_stride"], None)


FP8, BF16 = "idx_paged_mqa_logits_fp8", "idx_paged_mqa_logits_bf16"


@pytest.mark.parametrize("name,kw,status", [
    (FP8, dict(heads=32), IDX_ERR_UNSUPPORTED),
    (FP8, dict(dim=64), IDX_ERR_UNSUPPORTED),
    (BF16, dict(heads=128), IDX_ERR_UNSUPPORTED),
    (FP8, dict(rows=-1), IDX_ERR_SHAPE),
    (FP8, dict(width=-1), IDX_ERR_SHAPE),
    (FP8, dict(width=(1 << 24) + 1), IDX_ERR_SHAPE),
    (FP8, dict(num_pages=-1), IDX_ERR_SHAPE),
    (FP8, dict(pt_stride=-1), IDX_ERR_SHAPE),
    (FP8, dict(kv_stride=8191), IDX_ERR_SHAPE),
    (FP8, dict(ks_stride=255), IDX_ERR_SHAPE),
    (BF16, dict(kv_stride=8448), IDX_ERR_SHAPE),
    (FP8, dict(rows=0, q=None, kv=None), IDX_OK),          # nothing to do: no launch
    (FP8, dict(width=0, out=None), IDX_OK),
    (FP8, dict(q=None), IDX_ERR_NULL),
    (FP8, dict(kv=None), IDX_ERR_NULL),
    (FP8, dict(ks=None), IDX_ERR_NULL),
    (FP8, dict(pt=None), IDX_ERR_NULL),
    (FP8, dict(sl=None), IDX_ERR_NULL),
    (FP8, dict(w=None), IDX_ERR_NULL),
    (FP8, dict(out=None), IDX_ERR_NULL),
    (BF16, dict(ks=16), IDX_ERR_NULL),                       # bf16 takes no scales
    (FP8, dict(q=8), IDX_ERR_ALIGN),
    (FP8, dict(kv=32 + 4), IDX_ERR_ALIGN),
    (FP8, dict(out=4), IDX_ERR_ALIGN),
    (FP8, dict(w=20), IDX_ERR_ALIGN),
    (FP8, dict(pt=2), IDX_ERR_ALIGN),
    (FP8, dict(sl=6), IDX_ERR_ALIGN),
    (FP8, dict(ks=18), IDX_ERR_ALIGN),
    (FP8, dict(kv_stride=8456), IDX_ERR_ALIGN),
    (FP8, dict(ks_stride=8450), IDX_ERR_ALIGN),
])
def test_host_validation(lib, name, kw, status):
    assert _call(lib, name, **kw) == status


def _store(lib, name, **kw):
    a = dict(keys=16, slots=8, n=1, kv=16, ks=16, num_pages=1, kv_stride=8448, ks_stride=8448)
    if name.endswith("bf16"):
        a.update(kv_stride=16384)
    a.update(kw)
    if name.endswith("bf16"):
        return lib.idx_store_keys_bf16(a["keys"], a["slots"], a["n"], a["kv"], a["num_pages"],
                                       a["kv_stride"], None)
    return lib.idx_store_keys_fp8(a["keys"], a["slots"], a["n"], a["kv"], a["ks"], a["num_pages"],
                                  a["kv_stride"], a["ks_stride"], None)


SF, SB = "idx_store_keys_fp8", "idx_store_keys_bf16"


@pytest.mark.parametrize("name,kw,status", [
    (SF, dict(n=-1), IDX_ERR_SHAPE),
    (SF, dict(num_pages=-1), IDX_ERR_SHAPE),
    (SF, dict(kv_stride=8191), IDX_ERR_SHAPE),
    (SF, dict(ks_stride=255), IDX_ERR_SHAPE),
    (SB, dict(kv_stride=8448), IDX_ERR_SHAPE),
    (SF, dict(n=0, keys=None, slots=None, kv=None, ks=None), IDX_OK),   # nothing to store
    (SF, dict(keys=None), IDX_ERR_NULL),
    (SF, dict(slots=None), IDX_ERR_NULL),
    (SF, dict(kv=None), IDX_ERR_NULL),
    (SF, dict(ks=None), IDX_ERR_NULL),
    (SB, dict(kv=None), IDX_ERR_NULL),
    (SF, dict(keys=8), IDX_ERR_ALIGN),
    (SF, dict(slots=4), IDX_ERR_ALIGN),
    (SF, dict(kv=20), IDX_ERR_ALIGN),
    (SF, dict(ks=18), IDX_ERR_ALIGN),
    (SF, dict(kv_stride=8456), IDX_ERR_ALIGN),
    (SF, dict(ks_stride=8450), IDX_ERR_ALIGN),
])
def test_store_host_validation(lib, name, kw, status):
    assert _store(lib, name, **kw) == status


def _topk(lib, **kw):
    a = dict(logits=16, row_stride=64, sl=4, rows=1, ncols=64, k=8, idx=4, val=None)
    a.update(kw)
    return lib.idx_topk_logits(a["logits"], a["row_stride"], a["sl"], a["rows"], a["ncols"], a["k"],
                               a["idx"], a["val"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(rows=-1), IDX_ERR_SHAPE),
    (dict(ncols=-1), IDX_ERR_SHAPE),
    (dict(k=-1), IDX_ERR_SHAPE),
    (dict(row_stride=60), IDX_ERR_SHAPE),             # shorter than a row
    (dict(rows=0, logits=None, sl=None, idx=None), IDX_OK),
    (dict(k=0, logits=None, sl=None, idx=None), IDX_OK),
    (dict(logits=None), IDX_ERR_NULL),
    (dict(sl=None), IDX_ERR_NULL),
    (dict(idx=None), IDX_ERR_NULL),
    (dict(logits=20), IDX_ERR_ALIGN),
    (dict(row_stride=66), IDX_ERR_ALIGN),
    (dict(sl=2), IDX_ERR_ALIGN),
    (dict(idx=6), IDX_ERR_ALIGN),
    (dict(val=2), IDX_ERR_ALIGN),
])
def test_topk_host_validation(lib, kw, status):
    assert _topk(lib, **kw) == status


def _fused(lib, name, k=8, idx=4, val=None, **kw):
    a = dict(q=16, kv=16, ks=16, pt=4, sl=4, w=16, out=16, rows=1, heads=64, dim=128, width=1,
             num_pages=1, kv_stride=8448, ks_stride=8448, pt_stride=1)
    if name.endswith("bf16"):
        a.update(ks=None, kv_stride=16384, ks_stride=0)
    a.update(kw)
    return getattr(lib, name)(a["q"], a["kv"], a["ks"], a["pt"], a["sl"], a["w"], a["out"], a["rows"],
                              a["heads"], a["dim"], a["width"], a["num_pages"], a["kv_stride"],
                              a["ks_stride"], a["pt_stride"], k, idx, val, None)


TF, TB = "idx_paged_mqa_topk_fp8", "idx_paged_mqa_topk_bf16"


@pytest.mark.parametrize("name,kw,status", [
    (TF, dict(heads=32), IDX_ERR_UNSUPPORTED),
    (TF, dict(kv_stride=8191), IDX_ERR_SHAPE),
    (TF, dict(k=-1), IDX_ERR_SHAPE),
    (TB, dict(k=-1), IDX_ERR_SHAPE),
    (TF, dict(rows=0, q=None, idx=None), IDX_OK),             # nothing to do
    (TF, dict(q=None), IDX_ERR_NULL),
    (TF, dict(idx=None), IDX_ERR_NULL),
    (TB, dict(ks=16), IDX_ERR_NULL),
    (TF, dict(out=4), IDX_ERR_ALIGN),
    (TF, dict(idx=2), IDX_ERR_ALIGN),
    (TB, dict(val=6), IDX_ERR_ALIGN),
])
def test_fused_topk_host_validation(lib, name, kw, status):
    assert _fused(lib, name, **kw) == status


def _varlen(lib, name, rt=4, ntab=2, **kw):
    a = dict(q=16, kv=16, ks=16, pt=4, sl=4, w=16, out=16, rows=1, heads=64, dim=128, width=1,
             num_pages=1, kv_stride=8448, ks_stride=8448, pt_stride=1)
    if name.endswith("bf16"):
        a.update(ks=None, kv_stride=16384, ks_stride=0)
    a.update(kw)
    return getattr(lib, name)(a["q"], a["kv"], a["ks"], a["pt"], rt, ntab, a["sl"], a["w"], a["out"],
                              a["rows"], a["heads"], a["dim"], a["width"], a["num_pages"],
                              a["kv_stride"], a["ks_stride"], a["pt_stride"], None)


VF, VB = "idx_paged_mqa_logits_varlen_fp8", "idx_paged_mqa_logits_varlen_bf16"


@pytest.mark.parametrize("name,kw,status", [
    (VF, dict(heads=32), IDX_ERR_UNSUPPORTED),
    (VF, dict(ntab=-1), IDX_ERR_SHAPE),
    (VB, dict(kv_stride=8448), IDX_ERR_SHAPE),
    (VF, dict(rows=0, rt=None, q=None), IDX_OK),              # nothing to do
    (VF, dict(rt=None), IDX_ERR_NULL),
    (VF, dict(q=None), IDX_ERR_NULL),
    (VB, dict(ks=16), IDX_ERR_NULL),
    (VF, dict(rt=2), IDX_ERR_ALIGN),
    (VF, dict(out=4), IDX_ERR_ALIGN),
])
def test_varlen_host_validation(lib, name, kw, status):
    assert _varlen(lib, name, **kw) == status


def test_binding_checks_tensor_layouts():
    """The binding refuses tensors whose element type or layout differs from
    what the kernels read, before any call into the library."""
    import torch

    import paged_mqa_logits_idx_amd as b

    b._check("q", torch.zeros((2, 64, 128), dtype=torch.bfloat16), torch.bfloat16)
    with pytest.raises(ValueError, match="q must be torch.bfloat16"):
        b._check("q", torch.zeros((2, 64, 128), dtype=torch.float32), torch.bfloat16)
    with pytest.raises(ValueError, match="contiguous"):
        b._check("weights", torch.zeros((64, 2)).t(), torch.float32)
    with pytest.raises(ValueError, match="topk_idx must be torch.int32"):
        b._check("topk_idx", torch.zeros((2, 8), dtype=torch.int64), torch.int32)
    # tables and logits carry their own row stride: only the last dim must be dense
    b._check("logits", torch.zeros((4, 100))[:, :64], torch.float32, dense_rows=True)
    with pytest.raises(ValueError, match="unit-stride"):
        b._check("logits", torch.zeros((100, 4)).t(), torch.float32, dense_rows=True)
    b._check("kscale", 12345, torch.float32)  # raw addresses pass through
