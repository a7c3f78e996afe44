"""CPU oracle of the paged MQA-logits indexer -- TEST INFRASTRUCTURE ONLY.

Only the tests, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline leg
may use this package.  It shares no code with the HIP library: the C source
(oracle.c) is compiled here with gcc and called through ctypes on host copies
of the very bytes the library reads.  Arithmetic is float64 in a fixed order;
see oracle.c for the definition and the passages it follows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from pathlib import Path

import numpy as np

ORACLE_DIR = Path(__file__).resolve().parent
SOURCE = ORACLE_DIR / "oracle.c"
LIB_PATH = ORACLE_DIR / "liboracle.so"


def build_command(source: Path = SOURCE, out: Path = LIB_PATH) -> list[str]:
    return ["gcc", "-O2", "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared",
            str(source), "-o", str(out), "-lm"]


def build(source: Path = SOURCE, out: Path = LIB_PATH) -> Path:
    """Compile an oracle source (always recompiles, writes atomically)."""
    tmp = out.with_name(out.name + ".tmp")
    res = subprocess.run(build_command(source, tmp), capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"oracle build failed:\n{res.stdout}{res.stderr}")
    os.replace(tmp, out)
    return out


class Oracle:
    """ctypes view of one compiled oracle library."""

    def __init__(self, lib_path: Path):
        lib = ctypes.CDLL(str(lib_path))
        lib.oracle_e4m3fn_value.argtypes = [ctypes.c_uint32]
        lib.oracle_e4m3fn_value.restype = ctypes.c_double
        lib.oracle_bf16_value.argtypes = [ctypes.c_uint16]
        lib.oracle_bf16_value.restype = ctypes.c_double
        P = ctypes.c_void_p
        lib.oracle_paged_mqa_logits.argtypes = [
            ctypes.c_int, P, P, ctypes.c_int64, P, ctypes.c_int64, ctypes.c_int64, P,
            ctypes.c_int64, P, ctypes.c_int32, P, P, ctypes.c_int32, ctypes.c_int32, P,
            ctypes.c_int32, P]
        lib.oracle_paged_mqa_logits.restype = None
        lib.oracle_e4m3fn_encode.argtypes = [ctypes.c_float]
        lib.oracle_e4m3fn_encode.restype = ctypes.c_uint32
        lib.oracle_quantize_keys_fp8.argtypes = [P, ctypes.c_int64, P, P]
        lib.oracle_quantize_keys_fp8.restype = None
        lib.oracle_topk.argtypes = [P, ctypes.c_int64, P, ctypes.c_int32, ctypes.c_int32,
                                    ctypes.c_int32, P]
        lib.oracle_topk.restype = None
        lib.oracle_num_threads.argtypes = []
        lib.oracle_num_threads.restype = ctypes.c_int
        lib.oracle_set_num_threads.argtypes = [ctypes.c_int]
        lib.oracle_set_num_threads.restype = None
        self.lib = lib

    def e4m3fn_value(self, code: int) -> float:
        return self.lib.oracle_e4m3fn_value(int(code))

    def bf16_value(self, bits: int) -> float:
        return self.lib.oracle_bf16_value(int(bits))

    def num_threads(self) -> int:
        return int(self.lib.oracle_num_threads())

    def set_num_threads(self, n: int) -> None:
        self.lib.oracle_set_num_threads(int(n))

    def e4m3fn_encode(self, y: float) -> int:
        return int(self.lib.oracle_e4m3fn_encode(float(y)))

    def quantize_keys_fp8(self, keys_bits: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
        """e4m3fn codes [n, 128] and float32 scales [n] of bf16 keys (bits [n, 128])."""
        k = np.ascontiguousarray(keys_bits, dtype=np.uint16).reshape(-1, 128)
        n = k.shape[0]
        codes = np.empty((n, 128), dtype=np.uint8)
        scales = np.empty(n, dtype=np.float32)
        if n:
            self.lib.oracle_quantize_keys_fp8(k.ctypes.data, n, codes.ctypes.data, scales.ctypes.data)
        return codes, scales

    def topk(self, values: np.ndarray, seqlens, k: int) -> np.ndarray:
        """int32 [rows, k]: per row, the k largest of values[b, :L] (ties and NaN
        as oracle.c states), in ascending position order, then -1 padding."""
        v = np.ascontiguousarray(values, dtype=np.float64)
        if v.ndim != 2:
            raise ValueError("values must be [rows, ncols]")
        rows, ncols = v.shape
        sl = np.ascontiguousarray(np.asarray(seqlens, dtype=np.int32).reshape(-1))
        if sl.size != rows:
            raise ValueError("one seqlen per row")
        if k < 0:
            raise ValueError("k must be >= 0")
        idx = np.empty((rows, k), dtype=np.int32)
        if rows and k:
            self.lib.oracle_topk(v.ctypes.data, ncols, sl.ctypes.data, rows, ncols, int(k),
                                 idx.ctypes.data)
        return idx

    def paged_mqa_logits(self, wl, rows=None) -> np.ndarray:
        """float64 logits [len(rows) or wl.rows, table_width*64] of a workload.

        ``wl`` carries host arrays laid out as the library's arguments (see
        workloads.Workload; ``row_table`` / ``num_tables`` map rows to page
        tables in a multi-request batch).  ``rows``: optional row indices.
        """
        kind = {"fp8": 0, "bf16": 1}[wl.key_kind]
        q = np.ascontiguousarray(wl.q, dtype=np.uint16)
        kv = np.ascontiguousarray(wl.kv, dtype=np.uint8)
        ks_addr = None
        if kind == 0:
            ks = kv if wl.ks is wl.kv else np.ascontiguousarray(wl.ks, dtype=np.uint8)
            ks_addr = ks.ctypes.data + int(wl.ks_offset)
        pt = np.ascontiguousarray(wl.page_table, dtype=np.int32)
        rt = getattr(wl, "row_table", None)
        if rt is not None:
            rt = np.ascontiguousarray(rt, dtype=np.int32)
        sl = np.ascontiguousarray(wl.seqlens, dtype=np.int32)
        w = np.ascontiguousarray(wl.weights, dtype=np.float32)
        if rows is None:
            row_ids, n_out = None, wl.rows
        else:
            row_ids = np.ascontiguousarray(np.asarray(rows, dtype=np.int32))
            if row_ids.size and (row_ids.min() < 0 or row_ids.max() >= wl.rows):
                raise IndexError("row index out of range")
            n_out = int(row_ids.size)
        out = np.empty((n_out, wl.table_width * 64), dtype=np.float64)
        if n_out and wl.table_width:
            self.lib.oracle_paged_mqa_logits(
                kind, q.ctypes.data, kv.ctypes.data, int(wl.kv_stride), ks_addr,
                int(wl.ks_stride), int(wl.num_pages), pt.ctypes.data, int(wl.pt_stride),
                None if rt is None else rt.ctypes.data, int(getattr(wl, "num_tables", 0)),
                sl.ctypes.data, w.ctypes.data, int(wl.rows), int(wl.table_width),
                None if row_ids is None else row_ids.ctypes.data, n_out, out.ctypes.data)
        return out


_default: Oracle | None = None


def default() -> Oracle:
    global _default
    if _default is None:
        if not LIB_PATH.exists() or LIB_PATH.stat().st_mtime < SOURCE.stat().st_mtime:
            build()
        _default = Oracle(LIB_PATH)
    return _default


def e4m3fn_value(code: int) -> float:
    return default().e4m3fn_value(code)


def bf16_value(bits: int) -> float:
    return default().bf16_value(bits)


def num_threads() -> int:
    return default().num_threads()


def set_num_threads(n: int) -> None:
    default().set_num_threads(n)


def paged_mqa_logits(wl, rows=None) -> np.ndarray:
    return default().paged_mqa_logits(wl, rows)


def e4m3fn_encode(y: float) -> int:
    return default().e4m3fn_encode(y)


def quantize_keys_fp8(keys_bits: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    return default().quantize_keys_fp8(keys_bits)


def topk(values: np.ndarray, seqlens, k: int) -> np.ndarray:
    return default().topk(values, seqlens, k)
