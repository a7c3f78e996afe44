"""Python binding of the paged MQA-logits indexer library (libidx_paged_mqa.so).

Argument marshalling only: every step of the computation runs in the library's
HIP kernels.  The functions carry the C-ABI names and argument order; they
accept torch device tensors (or raw device addresses as ints) and pass their
addresses and sizes through ctypes.  torch supplies device memory and streams.

The library must be built in-tree first (``python paged_mqa_logits_idx_amd/_build.py``
or ``__graft_entry__.build()``); importing this module without it raises.
"""
from __future__ import annotations

import ctypes
from pathlib import Path

import torch  # loads the HIP runtime the library binds to (same soname)

LIB_PATH = Path(__file__).resolve().parent / "libidx_paged_mqa.so"

NUM_HEADS = 64
HEAD_DIM = 128
PAGE_POSITIONS = 64
FP8_PAGE_KEY_BYTES = PAGE_POSITIONS * HEAD_DIM          # 8192
FP8_PAGE_SCALE_BYTES = PAGE_POSITIONS * 4               # 256
FP8_FUSED_PAGE_BYTES = FP8_PAGE_KEY_BYTES + FP8_PAGE_SCALE_BYTES  # 8448
BF16_PAGE_BYTES = PAGE_POSITIONS * HEAD_DIM * 2         # 16384

IDX_OK = 0
IDX_ERR_NULL = -1
IDX_ERR_UNSUPPORTED = -2
IDX_ERR_SHAPE = -3
IDX_ERR_ALIGN = -4
IDX_ERR_LAUNCH = -5

_SYMBOLS = (
    "idx_paged_mqa_logits_fp8",
    "idx_paged_mqa_logits_bf16",
    "idx_paged_mqa_logits_varlen_fp8",
    "idx_paged_mqa_logits_varlen_bf16",
    "idx_topk_logits",
    "idx_paged_mqa_topk_fp8",
    "idx_paged_mqa_topk_bf16",
    "idx_store_keys_fp8",
    "idx_store_keys_bf16",
    "idx_status_string",
    "idx_abi_version",
)


class IdxError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{msg} (status {status})")
        self.status = status


def _load() -> ctypes.CDLL:
    if not LIB_PATH.exists():
        raise ImportError(
            f"{LIB_PATH} is missing: build the HIP library first "
            "(python paged_mqa_logits_idx_amd/_build.py)")
    lib = ctypes.CDLL(str(LIB_PATH))
    argtypes = [
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
        ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
        ctypes.c_void_p,
    ]
    for name in ("idx_paged_mqa_logits_fp8", "idx_paged_mqa_logits_bf16"):
        fn = getattr(lib, name)
        fn.argtypes = argtypes
        fn.restype = ctypes.c_int
    for name in ("idx_paged_mqa_logits_varlen_fp8", "idx_paged_mqa_logits_varlen_bf16"):
        fn = getattr(lib, name)
        fn.argtypes = argtypes[:4] + [ctypes.c_void_p, ctypes.c_int32] + argtypes[4:]
        fn.restype = ctypes.c_int
    lib.idx_topk_logits.argtypes = [
        ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
        ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    lib.idx_topk_logits.restype = ctypes.c_int
    for name in ("idx_paged_mqa_topk_fp8", "idx_paged_mqa_topk_bf16"):
        fn = getattr(lib, name)
        fn.argtypes = argtypes[:-1] + [ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p,
                                       ctypes.c_void_p]
        fn.restype = ctypes.c_int
    lib.idx_store_keys_fp8.argtypes = [
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p]
    lib.idx_store_keys_fp8.restype = ctypes.c_int
    lib.idx_store_keys_bf16.argtypes = [
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int64,
        ctypes.c_int64, ctypes.c_void_p]
    lib.idx_store_keys_bf16.restype = ctypes.c_int
    lib.idx_status_string.argtypes = [ctypes.c_int]
    lib.idx_status_string.restype = ctypes.c_char_p
    lib.idx_abi_version.argtypes = []
    lib.idx_abi_version.restype = ctypes.c_int
    return lib


_lib = _load()


def idx_status_string(status: int) -> str:
    return _lib.idx_status_string(int(status)).decode()


def idx_abi_version() -> int:
    return int(_lib.idx_abi_version())


def _addr(x) -> int | None:
    if x is None:
        return None
    if isinstance(x, torch.Tensor):
        if x.device.type != "cuda":
            raise ValueError("tensors passed to the indexer library must be device tensors")
        return x.data_ptr()
    return int(x)


def _check(name: str, x, dtype, dense_rows: bool = False) -> None:
    """A tensor argument must have the element type the kernels read and the
    dense layout they assume: contiguous, or (``dense_rows``: tables and logits,
    whose row stride is passed separately) unit stride along its last dim.
    Raw addresses are passed through unchecked."""
    if not isinstance(x, torch.Tensor):
        return
    if x.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {x.dtype}")
    ok = (x.dim() == 0 or x.stride(-1) == 1 or x.shape[-1] <= 1) if dense_rows else x.is_contiguous()
    if not ok:
        raise ValueError(f"{name} must be " + ("unit-stride along its last dim" if dense_rows
                                                 else "contiguous"))


def _check_logits_args(q, kv_pages, kscale, page_table, seqlens, weights, out):
    _check("q", q, torch.bfloat16)
    if isinstance(kv_pages, torch.Tensor) and not kv_pages.is_contiguous():
        raise ValueError("kv_pages must be contiguous")
    if isinstance(kscale, torch.Tensor):
        _check("kscale", kscale, torch.float32)
    _check("page_table", page_table, torch.int32, dense_rows=True)
    _check("seqlens", seqlens, torch.int32)
    _check("weights", weights, torch.float32)
    _check("out", out, torch.float32)


def _stream_handle(stream, device) -> int | None:
    if stream is None:
        return torch.cuda.current_stream(device).cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _call(name, q, kv_pages, kscale, page_table, seqlens, weights, out, *, rows, num_heads,
          head_dim, table_width, num_pages, kv_page_stride, kscale_page_stride,
          page_table_row_stride, stream, check):
    _check_logits_args(q, kv_pages, kscale, page_table, seqlens, weights, out)
    dev = q.device if isinstance(q, torch.Tensor) else None
    fn = getattr(_lib, name)
    status = fn(_addr(q), _addr(kv_pages), _addr(kscale), _addr(page_table), _addr(seqlens),
                _addr(weights), _addr(out), int(rows), int(num_heads), int(head_dim),
                int(table_width), int(num_pages), int(kv_page_stride), int(kscale_page_stride),
                int(page_table_row_stride), _stream_handle(stream, dev))
    if check and status != IDX_OK:
        raise IdxError(status, f"{name}: {idx_status_string(status)}")
    return status


def _dims(q, page_table, table_width, rows, num_heads, head_dim, page_table_row_stride):
    if isinstance(q, torch.Tensor):
        if rows is None:
            rows = q.shape[0]
        if num_heads is None:
            num_heads = q.shape[1] if q.dim() == 3 else NUM_HEADS
        if head_dim is None:
            head_dim = q.shape[2] if q.dim() == 3 else HEAD_DIM
    if table_width is None:
        if not (isinstance(page_table, torch.Tensor) and page_table.dim() == 2):
            raise ValueError("table_width is required unless page_table is a 2-D tensor")
        table_width = page_table.shape[1]
    if page_table_row_stride is None:
        if not (isinstance(page_table, torch.Tensor) and page_table.dim() == 2):
            raise ValueError("page_table_row_stride is required unless page_table is a 2-D tensor")
        page_table_row_stride = 0 if page_table.shape[0] == 1 and rows != 1 else page_table.stride(0)
    return rows, num_heads, head_dim, table_width, page_table_row_stride


def idx_paged_mqa_logits_fp8(q, kv_pages, kscale, page_table, seqlens, weights, out, *,
                             num_pages, kv_page_stride=FP8_FUSED_PAGE_BYTES,
                             kscale_page_stride=FP8_FUSED_PAGE_BYTES, table_width=None,
                             page_table_row_stride=None, rows=None, num_heads=None,
                             head_dim=None, stream=None, check=True) -> int:
    """out[b, p] = sum_h w[b,h] * ReLU(s_p * <q[b,h], k_p>) for p < seqlens[b], else -inf.

    fp8 (e4m3fn) keys with a per-position fp32 scale.  ``kscale`` is a tensor or
    a device address; for the fused 8448-byte block pass
    ``kv_pages.data_ptr() + 8192``.  Returns the library status (raises
    IdxError on failure when ``check``).
    """
    rows, num_heads, head_dim, table_width, pts = _dims(
        q, page_table, table_width, rows, num_heads, head_dim, page_table_row_stride)
    return _call("idx_paged_mqa_logits_fp8", q, kv_pages, kscale, page_table, seqlens, weights,
                 out, rows=rows, num_heads=num_heads, head_dim=head_dim, table_width=table_width,
                 num_pages=num_pages, kv_page_stride=kv_page_stride,
                 kscale_page_stride=kscale_page_stride, page_table_row_stride=pts, stream=stream,
                 check=check)


def idx_paged_mqa_logits_bf16(q, kv_pages, kscale, page_table, seqlens, weights, out, *,
                              num_pages, kv_page_stride=BF16_PAGE_BYTES, kscale_page_stride=0,
                              table_width=None, page_table_row_stride=None, rows=None,
                              num_heads=None, head_dim=None, stream=None, check=True) -> int:
    """Same as :func:`idx_paged_mqa_logits_fp8` with bf16 keys and s_p = 1 (kscale must be None)."""
    rows, num_heads, head_dim, table_width, pts = _dims(
        q, page_table, table_width, rows, num_heads, head_dim, page_table_row_stride)
    return _call("idx_paged_mqa_logits_bf16", q, kv_pages, kscale, page_table, seqlens, weights,
                 out, rows=rows, num_heads=num_heads, head_dim=head_dim, table_width=table_width,
                 num_pages=num_pages, kv_page_stride=kv_page_stride,
                 kscale_page_stride=kscale_page_stride, page_table_row_stride=pts, stream=stream,
                 check=check)


def _call_varlen(name, q, kv_pages, kscale, page_table, row_table, seqlens, weights, out, *,
                 num_tables, num_pages, table_width, page_table_row_stride, kv_page_stride,
                 kscale_page_stride, rows, num_heads, head_dim, stream, check):
    if isinstance(q, torch.Tensor):
        rows = q.shape[0] if rows is None else rows
    num_heads = NUM_HEADS if num_heads is None else num_heads
    head_dim = HEAD_DIM if head_dim is None else head_dim
    _check_logits_args(q, kv_pages, kscale, page_table, seqlens, weights, out)
    _check("row_table", row_table, torch.int32)
    dev = q.device if isinstance(q, torch.Tensor) else None
    status = getattr(_lib, name)(
        _addr(q), _addr(kv_pages), _addr(kscale), _addr(page_table), _addr(row_table),
        int(num_tables), _addr(seqlens), _addr(weights), _addr(out), int(rows), int(num_heads),
        int(head_dim), int(table_width), int(num_pages), int(kv_page_stride),
        int(kscale_page_stride), int(page_table_row_stride), _stream_handle(stream, dev))
    if check and status != IDX_OK:
        raise IdxError(status, f"{name}: {idx_status_string(status)}")
    return status


def idx_paged_mqa_logits_varlen_fp8(q, kv_pages, kscale, page_table, row_table, seqlens, weights,
                                    out, *, num_tables, num_pages, table_width,
                                    page_table_row_stride=None,
                                    kv_page_stride=FP8_FUSED_PAGE_BYTES,
                                    kscale_page_stride=FP8_FUSED_PAGE_BYTES, rows=None,
                                    num_heads=None, head_dim=None, stream=None,
                                    check=True) -> int:
    """Several requests' query rows in one call: row b uses table row_table[b]
    (at page_table + row_table[b]*page_table_row_stride) and its own seqlen."""
    pts = table_width if page_table_row_stride is None else page_table_row_stride
    return _call_varlen("idx_paged_mqa_logits_varlen_fp8", q, kv_pages, kscale, page_table,
                        row_table, seqlens, weights, out, num_tables=num_tables,
                        num_pages=num_pages, table_width=table_width, page_table_row_stride=pts,
                        kv_page_stride=kv_page_stride, kscale_page_stride=kscale_page_stride,
                        rows=rows, num_heads=num_heads, head_dim=head_dim, stream=stream,
                        check=check)


def idx_paged_mqa_logits_varlen_bf16(q, kv_pages, kscale, page_table, row_table, seqlens, weights,
                                     out, *, num_tables, num_pages, table_width,
                                     page_table_row_stride=None, kv_page_stride=BF16_PAGE_BYTES,
                                     kscale_page_stride=0, rows=None, num_heads=None,
                                     head_dim=None, stream=None, check=True) -> int:
    """bf16-key counterpart of :func:`idx_paged_mqa_logits_varlen_fp8`."""
    pts = table_width if page_table_row_stride is None else page_table_row_stride
    return _call_varlen("idx_paged_mqa_logits_varlen_bf16", q, kv_pages, kscale, page_table,
                        row_table, seqlens, weights, out, num_tables=num_tables,
                        num_pages=num_pages, table_width=table_width, page_table_row_stride=pts,
                        kv_page_stride=kv_page_stride, kscale_page_stride=kscale_page_stride,
                        rows=rows, num_heads=num_heads, head_dim=head_dim, stream=stream,
                        check=check)


def idx_topk_logits(logits, seqlens, topk_idx, topk_val=None, *, k=None, rows=None, ncols=None,
                    row_stride=None, stream=None, check=True) -> int:
    """Per row b, the k largest of logits[b, :clamp(seqlens[b], 0, ncols)] (equal
    values by lower position, NaN last), in ascending position order, -1 padded.

    ``topk_idx`` int32 [rows, k]; ``topk_val`` optional fp32 [rows, k].  Dims
    default to the tensors' shapes.
    """
    if isinstance(logits, torch.Tensor):
        rows = logits.shape[0] if rows is None else rows
        ncols = logits.shape[1] if ncols is None else ncols
        row_stride = logits.stride(0) if row_stride is None else row_stride
    if k is None:
        k = topk_idx.shape[1]
    _check("logits", logits, torch.float32, dense_rows=True)
    _check("seqlens", seqlens, torch.int32)
    _check("topk_idx", topk_idx, torch.int32)
    _check("topk_val", topk_val, torch.float32)
    dev = topk_idx.device if isinstance(topk_idx, torch.Tensor) else None
    status = _lib.idx_topk_logits(_addr(logits), int(row_stride), _addr(seqlens), int(rows),
                                  int(ncols), int(k), _addr(topk_idx), _addr(topk_val),
                                  _stream_handle(stream, dev))
    if check and status != IDX_OK:
        raise IdxError(status, f"idx_topk_logits: {idx_status_string(status)}")
    return status


def _call_topk(name, q, kv_pages, kscale, page_table, seqlens, weights, logits, topk_idx, topk_val,
               *, k, rows, num_heads, head_dim, table_width, num_pages, kv_page_stride,
               kscale_page_stride, page_table_row_stride, stream, check):
    rows, num_heads, head_dim, table_width, pts = _dims(
        q, page_table, table_width, rows, num_heads, head_dim, page_table_row_stride)
    if k is None:
        k = topk_idx.shape[1]
    _check_logits_args(q, kv_pages, kscale, page_table, seqlens, weights, logits)
    _check("topk_idx", topk_idx, torch.int32)
    _check("topk_val", topk_val, torch.float32)
    dev = q.device if isinstance(q, torch.Tensor) else None
    status = getattr(_lib, name)(
        _addr(q), _addr(kv_pages), _addr(kscale), _addr(page_table), _addr(seqlens),
        _addr(weights), _addr(logits), int(rows), int(num_heads), int(head_dim), int(table_width),
        int(num_pages), int(kv_page_stride), int(kscale_page_stride), int(pts), int(k),
        _addr(topk_idx), _addr(topk_val), _stream_handle(stream, dev))
    if check and status != IDX_OK:
        raise IdxError(status, f"{name}: {idx_status_string(status)}")
    return status


def idx_paged_mqa_topk_fp8(q, kv_pages, kscale, page_table, seqlens, weights, logits, topk_idx,
                           topk_val=None, *, num_pages, k=None,
                           kv_page_stride=FP8_FUSED_PAGE_BYTES,
                           kscale_page_stride=FP8_FUSED_PAGE_BYTES, table_width=None,
                           page_table_row_stride=None, rows=None, num_heads=None, head_dim=None,
                           stream=None, check=True) -> int:
    """Logits into ``logits`` (only positions p < seqlens[b] defined afterwards),
    then their top-k into ``topk_idx`` / ``topk_val``, in one call."""
    return _call_topk("idx_paged_mqa_topk_fp8", q, kv_pages, kscale, page_table, seqlens, weights,
                      logits, topk_idx, topk_val, k=k, rows=rows, num_heads=num_heads,
                      head_dim=head_dim, table_width=table_width, num_pages=num_pages,
                      kv_page_stride=kv_page_stride, kscale_page_stride=kscale_page_stride,
                      page_table_row_stride=page_table_row_stride, stream=stream, check=check)


def idx_paged_mqa_topk_bf16(q, kv_pages, kscale, page_table, seqlens, weights, logits, topk_idx,
                            topk_val=None, *, num_pages, k=None, kv_page_stride=BF16_PAGE_BYTES,
                            kscale_page_stride=0, table_width=None, page_table_row_stride=None,
                            rows=None, num_heads=None, head_dim=None, stream=None,
                            check=True) -> int:
    """bf16-key counterpart of :func:`idx_paged_mqa_topk_fp8` (kscale must be None)."""
    return _call_topk("idx_paged_mqa_topk_bf16", q, kv_pages, kscale, page_table, seqlens, weights,
                      logits, topk_idx, topk_val, k=k, rows=rows, num_heads=num_heads,
                      head_dim=head_dim, table_width=table_width, num_pages=num_pages,
                      kv_page_stride=kv_page_stride, kscale_page_stride=kscale_page_stride,
                      page_table_row_stride=page_table_row_stride, stream=stream, check=check)


def idx_store_keys_fp8(keys, slots, kv_pages, kscale, *, num_pages, n=None,
                       kv_page_stride=FP8_FUSED_PAGE_BYTES, kscale_page_stride=FP8_FUSED_PAGE_BYTES,
                       stream=None, check=True) -> int:
    """Quantise bf16 keys [n, 128] (scale = amax/448, e4m3fn codes) into pool slots.

    ``slots`` is int64 [n] (64*page + position; out of range skips the key).
    ``kscale`` is a tensor or a device address (fused block: kv_pages + 8192).
    """
    if n is None:
        n = keys.shape[0]
    _check("keys", keys, torch.bfloat16)
    _check("slots", slots, torch.int64)
    if isinstance(kscale, torch.Tensor):
        _check("kscale", kscale, torch.float32)
    if isinstance(kv_pages, torch.Tensor) and not kv_pages.is_contiguous():
        raise ValueError("kv_pages must be contiguous")
    dev = keys.device if isinstance(keys, torch.Tensor) else None
    status = _lib.idx_store_keys_fp8(_addr(keys), _addr(slots), int(n), _addr(kv_pages),
                                     _addr(kscale), int(num_pages), int(kv_page_stride),
                                     int(kscale_page_stride), _stream_handle(stream, dev))
    if check and status != IDX_OK:
        raise IdxError(status, f"idx_store_keys_fp8: {idx_status_string(status)}")
    return status


def idx_store_keys_bf16(keys, slots, kv_pages, *, num_pages, n=None, kv_page_stride=BF16_PAGE_BYTES,
                        stream=None, check=True) -> int:
    """Copy bf16 keys [n, 128] into 16384-byte bf16 pages at the given slots."""
    if n is None:
        n = keys.shape[0]
    _check("keys", keys, torch.bfloat16)
    _check("slots", slots, torch.int64)
    if isinstance(kv_pages, torch.Tensor) and not kv_pages.is_contiguous():
        raise ValueError("kv_pages must be contiguous")
    dev = keys.device if isinstance(keys, torch.Tensor) else None
    status = _lib.idx_store_keys_bf16(_addr(keys), _addr(slots), int(n), _addr(kv_pages),
                                      int(num_pages), int(kv_page_stride), _stream_handle(stream, dev))
    if check and status != IDX_OK:
        raise IdxError(status, f"idx_store_keys_bf16: {idx_status_string(status)}")
    return status


__all__ = [
    "idx_paged_mqa_logits_fp8", "idx_paged_mqa_logits_bf16", "idx_paged_mqa_logits_varlen_fp8",
    "idx_paged_mqa_logits_varlen_bf16", "idx_topk_logits",
    "idx_paged_mqa_topk_fp8", "idx_paged_mqa_topk_bf16", "idx_store_keys_fp8",
    "idx_store_keys_bf16", "idx_status_string",
    "idx_abi_version", "IdxError", "LIB_PATH", "NUM_HEADS", "HEAD_DIM", "PAGE_POSITIONS",
]
