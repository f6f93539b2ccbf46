"""CPU oracle for the mask-only logits path -- TEST INFRASTRUCTURE ONLY.

Only tests, the smoke check and the benchmark's CPU-baseline leg import this
package.  The product path (the HIP library and its Python binding) never does,
and nothing here is shared with it.  The arithmetic lives in ``oracle.c`` (plain C,
fp64, OpenMP over output elements); this module compiles it with gcc and marshals
numpy arrays into it.

Every function here is pinned by CPU tests to something other than itself
(library routines, brute force, closed forms and exact-integer results); the
pins are listed in the test modules ``tests/test_oracle_*.py``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from pathlib import Path

import numpy as np

_DIR = Path(__file__).resolve().parent
_SRC = _DIR / "oracle.c"
_LIB = _DIR / "liboracle.so"
_lib = None

_i64 = ctypes.c_int64
_i32 = ctypes.c_int32
_p = ctypes.c_void_p


def build(force: bool = True) -> Path:
    """Compile oracle.c into oracle/liboracle.so with gcc and OpenMP."""
    if force or not _LIB.exists() or _LIB.stat().st_mtime < _SRC.stat().st_mtime:
        tmp = _LIB.with_suffix(".so.tmp")
        cmd = ["gcc", "-std=c11", "-O2", "-fopenmp", "-ffp-contract=off", "-fPIC", "-shared",
               "-Wall", "-Wextra", "-o", str(tmp), str(_SRC), "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not _LIB.exists() or _LIB.stat().st_mtime < _SRC.stat().st_mtime:
            build(force=True)
        lib = ctypes.CDLL(str(_LIB))
        lib.oracle_mask_compact.restype = _i64
        lib.oracle_mask_compact.argtypes = [_p, _i64, _i32, _p]
        lib.oracle_mask_compact_flags.restype = _i64
        lib.oracle_mask_compact_flags.argtypes = [_p, _i64, _p]
        lib.oracle_mask_compact_batched.restype = _i64
        lib.oracle_mask_compact_batched.argtypes = [_p, _p, _i32, _i32, _p, _p]
        lib.oracle_num_chunks.restype = _i64
        lib.oracle_num_chunks.argtypes = [_i64, _i64]
        lib.oracle_chunk_range.restype = None
        lib.oracle_chunk_range.argtypes = [_i64, _i64, _i64, ctypes.POINTER(_i64), ctypes.POINTER(_i64)]
        for name in ("oracle_masked_logits_bf16", "oracle_masked_logits_f32"):
            f = getattr(lib, name)
            f.restype = ctypes.c_int
            f.argtypes = [_p, _i64, _i64, _p, _i64, _p, _i64, _p, _i64, _p]
        lib.oracle_masked_logits_chunked_bf16.restype = ctypes.c_int
        lib.oracle_masked_logits_chunked_bf16.argtypes = [_p, _i64, _i64, _p, _i64, _p, _i64, _i64, _p]
        lib.oracle_masked_logits_argmax_lse_bf16.restype = ctypes.c_int
        lib.oracle_masked_logits_argmax_lse_bf16.argtypes = [_p, _i64, _i64, _p, _i64, _p, _i64, _p, _i64,
                                                             _p, _p, _p]
        lib.oracle_lazy_chunk_rows.restype = ctypes.c_int
        lib.oracle_lazy_chunk_rows.argtypes = [_i64, _i64, _i64, _i64, ctypes.POINTER(_i64), ctypes.POINTER(_i64)]
        lib.oracle_e4m3_value.restype = ctypes.c_double
        lib.oracle_e4m3_value.argtypes = [ctypes.c_uint8]
        lib.oracle_e4m3_encode.restype = ctypes.c_uint8
        lib.oracle_e4m3_encode.argtypes = [ctypes.c_float]
        lib.oracle_quantize_rows_e4m3.restype = ctypes.c_int
        lib.oracle_quantize_rows_e4m3.argtypes = [_p, _i64, _i64, ctypes.c_int, _p, _i64, _p, _p]
        lib.oracle_logits_fp8.restype = ctypes.c_int
        lib.oracle_logits_fp8.argtypes = [_p, _p, _i64, _p, _p, _i64, _i64, _p, _i64, _p]
        lib.oracle_logits_bytes.restype = _i64
        lib.oracle_logits_bytes.argtypes = [_i64, _i64, _i64]
        lib.oracle_num_threads.restype = ctypes.c_int
        lib.oracle_num_threads.argtypes = []
        lib.oracle_set_num_threads.restype = None
        lib.oracle_set_num_threads.argtypes = [ctypes.c_int]
        _lib = lib
    return _lib


def _np(x, dtype=None):
    """numpy view of a CPU torch tensor or array (bf16 as its uint16 bit pattern)."""
    try:
        import torch
        if isinstance(x, torch.Tensor):
            x = x.detach().cpu().contiguous()
            if x.dtype == torch.bfloat16:
                x = x.view(torch.int16).numpy().view(np.uint16)
            else:
                x = x.numpy()
    except ImportError:  # pragma: no cover
        pass
    x = np.ascontiguousarray(x)
    if dtype is not None:
        x = np.ascontiguousarray(x, dtype=dtype)
    return x


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def set_num_threads(n: int) -> None:
    """Threads of the oracle's later parallel loops (OpenMP), n >= 1."""
    _load().oracle_set_num_threads(int(n))


def logits_bytes(rows: int, V: int, esize: int) -> int:
    """rows * V * esize, or -1 on int64 overflow."""
    return int(_load().oracle_logits_bytes(int(rows), int(V), int(esize)))


def mask_compact(tokens, mask_id: int) -> np.ndarray:
    """Ascending positions p with tokens[p] == mask_id (int32)."""
    t = _np(tokens, np.int32)
    idx = np.empty(max(1, t.size), np.int32)
    m = _load().oracle_mask_compact(_ptr(t), t.size, int(mask_id), _ptr(idx))
    return idx[:m].copy()


def mask_compact_flags(flags) -> np.ndarray:
    f = _np(flags, np.uint8)
    idx = np.empty(max(1, f.size), np.int32)
    m = _load().oracle_mask_compact_flags(_ptr(f), f.size, _ptr(idx))
    return idx[:m].copy()


def mask_compact_batched(tokens, seq_offsets, mask_id: int):
    """(idx, idx_offsets) for a ragged batch; idx holds global positions."""
    t = _np(tokens, np.int32)
    so = _np(seq_offsets, np.int32)
    nseq = so.size - 1
    idx = np.empty(max(1, t.size), np.int32)
    off = np.empty(nseq + 1, np.int32)
    m = _load().oracle_mask_compact_batched(_ptr(t), _ptr(so), nseq, int(mask_id), _ptr(idx), _ptr(off))
    return idx[:m].copy(), off


def num_chunks(M: int, C: int) -> int:
    return int(_load().oracle_num_chunks(int(M), int(C)))


def chunk_range(M: int, C: int, k: int):
    r0, r1 = _i64(), _i64()
    _load().oracle_chunk_range(int(M), int(C), int(k), ctypes.byref(r0), ctypes.byref(r1))
    return int(r0.value), int(r1.value)


def lazy_chunk_rows(M: int, V: int, esize: int, budget: int):
    """(chunk_rows, num_chunks) of the lazy chunk choice; chunk_rows 0 = no chunking.
    Raises ValueError when one row does not fit the budget."""
    c, k = _i64(), _i64()
    rc = _load().oracle_lazy_chunk_rows(int(M), int(V), int(esize), int(budget), ctypes.byref(c), ctypes.byref(k))
    if rc != 0:
        raise ValueError("one row of logits does not fit the budget")
    return int(c.value), int(k.value)


def masked_logits(H, idx, W, rows=None) -> np.ndarray:
    """fp64 logits [len(rows), V] of output rows `rows` (default: all M rows).

    H [L, d] and W [V, d] are bf16 or fp32 (CPU torch tensors or numpy arrays;
    numpy uint16 means bf16 bit patterns)."""
    import torch
    is_bf16 = (isinstance(H, torch.Tensor) and H.dtype == torch.bfloat16) or \
              (isinstance(H, np.ndarray) and H.dtype == np.uint16)
    if is_bf16:
        h = _np(H, np.uint16)
        w = _np(W, np.uint16)
        f = _load().oracle_masked_logits_bf16
    else:
        h = _np(H, np.float32)
        w = _np(W, np.float32)
        f = _load().oracle_masked_logits_f32
    L, d = h.shape
    V = w.shape[0]
    assert w.shape[1] == d
    ix = _np(idx, np.int32)
    M = ix.size
    r = np.arange(M, dtype=np.int64) if rows is None else _np(rows, np.int64)
    out = np.empty((r.size, V), np.float64)
    if r.size == 0 or V == 0:
        return out
    rc = f(_ptr(h), L, d, _ptr(ix), M, _ptr(w), V, _ptr(r), r.size, _ptr(out))
    if rc != 0:
        raise IndexError("row or index out of range")
    return out


def masked_logits_argmax_lse(H, idx, W, rows=None):
    """Per-row consumer of the bf16 masked logits: (row_max fp64, row_argmax int64,
    row_lse fp64) for output rows `rows` (default: all M rows)."""
    h = _np(H, np.uint16)
    w = _np(W, np.uint16)
    L, d = h.shape
    V = w.shape[0]
    assert w.shape[1] == d
    ix = _np(idx, np.int32)
    M = ix.size
    r = np.arange(M, dtype=np.int64) if rows is None else _np(rows, np.int64)
    mx = np.empty(r.size, np.float64)
    am = np.empty(r.size, np.int64)
    lse = np.empty(r.size, np.float64)
    if r.size == 0:
        return mx, am, lse
    rc = _load().oracle_masked_logits_argmax_lse_bf16(_ptr(h), L, d, _ptr(ix), M, _ptr(w), V, _ptr(r), r.size,
                                                      _ptr(mx), _ptr(am), _ptr(lse))
    if rc == -1:
        raise IndexError("row or index out of range")
    if rc != 0:
        raise ValueError("empty vocabulary or out of memory")
    return mx, am, lse


def e4m3_value(code: int) -> float:
    """Value of an OCP FP8 E4M3 code."""
    return float(_load().oracle_e4m3_value(int(code)))


def e4m3_encode(x: float) -> int:
    """Nearest E4M3 code of an fp32 value (ties to even, saturating at +-448)."""
    return int(_load().oracle_e4m3_encode(float(np.float32(x))))


def quantize_rows_e4m3(X, row_idx=None):
    """Per-row E4M3 quantization of X [n, d] (bf16 or fp32, CPU tensor or array):
    returns (codes uint8 [rows, d], scales float32 [rows]); rows = row_idx (gathered)
    or all n rows."""
    import torch
    is_bf16 = (isinstance(X, torch.Tensor) and X.dtype == torch.bfloat16) or \
              (isinstance(X, np.ndarray) and X.dtype == np.uint16)
    x = _np(X, np.uint16 if is_bf16 else np.float32)
    n, d = x.shape
    ri = None if row_idx is None else _np(row_idx, np.int32)
    rows = n if ri is None else ri.size
    q = np.empty((rows, d), np.uint8)
    sc = np.empty(rows, np.float32)
    if rows == 0:
        return q, sc
    rc = _load().oracle_quantize_rows_e4m3(_ptr(x), n, d, int(is_bf16), None if ri is None else _ptr(ri), rows,
                                           _ptr(q), _ptr(sc))
    if rc != 0:
        raise IndexError("row index out of range")
    return q, sc


def logits_fp8(qh, scale_h, qw, scale_w, rows=None) -> np.ndarray:
    """fp64 logits of quantized rows: (sum_k qh[r, k] qw[v, k]) * scale_h[r] * scale_w[v]."""
    qh = np.ascontiguousarray(qh, np.uint8)
    qw = np.ascontiguousarray(qw, np.uint8)
    sh = np.ascontiguousarray(scale_h, np.float32)
    sw = np.ascontiguousarray(scale_w, np.float32)
    M, d = qh.shape
    V = qw.shape[0]
    r = np.arange(M, dtype=np.int64) if rows is None else np.ascontiguousarray(rows, np.int64)
    out = np.empty((r.size, V), np.float64)
    if r.size == 0 or V == 0:
        return out
    rc = _load().oracle_logits_fp8(_ptr(qh), _ptr(sh), M, _ptr(qw), _ptr(sw), V, d, _ptr(r), r.size, _ptr(out))
    if rc != 0:
        raise IndexError("row out of range")
    return out


def masked_logits_fp8(H, idx, W, rows=None) -> np.ndarray:
    """The FP8 LM head on the masked rows: quantize H[idx] and W per row, then logits_fp8."""
    qh, sh = quantize_rows_e4m3(H, idx)
    qw, sw = quantize_rows_e4m3(W)
    return logits_fp8(qh, sh, qw, sw, rows)


def masked_logits_chunked(H, idx, W, chunk_rows: int) -> np.ndarray:
    """The micro-batched LM head (bf16 only): slices of chunk_rows rows, concatenated."""
    h = _np(H, np.uint16)
    w = _np(W, np.uint16)
    L, d = h.shape
    V = w.shape[0]
    ix = _np(idx, np.int32)
    M = ix.size
    out = np.empty((M, V), np.float64)
    if M == 0:
        return out
    rc = _load().oracle_masked_logits_chunked_bf16(_ptr(h), L, d, _ptr(ix), M, _ptr(w), V,
                                                   int(chunk_rows), _ptr(out))
    if rc != 0:
        raise IndexError("index out of range")
    return out
