"""Thin Python binding of libmosaic.so (include/mosaic.h).

Each function has the name of the C entry point it calls and only marshals
arguments: torch tensors become device pointers, the current torch stream becomes
the hipStream_t, and a non-OK status becomes an exception.  Every step of the
path runs in the HIP kernels; there is no fallback.  If the library is missing the
import fails with an error that says how to build it.

PyTorch is used for device memory and streams only.
"""
from __future__ import annotations

import ctypes
from pathlib import Path

import torch

_LIB_PATH = Path(__file__).resolve().parent / "libmosaic.so"

MOSAIC_OK = 0
MOSAIC_ERR_INVALID_ARG = 1
MOSAIC_ERR_UNSUPPORTED = 2
MOSAIC_ERR_DEVICE = 3
MOSAIC_F32 = 0
MOSAIC_BF16 = 1
MOSAIC_NOALLOC_SCRATCH_BYTES = 32 << 20

# Every symbol include/mosaic.h declares.
EXPORTS = (
    "mosaic_status_string",
    "mosaic_mask_compact_workspace_bytes",
    "mosaic_mask_compact",
    "mosaic_mask_compact_flags",
    "mosaic_mask_compact_batched",
    "mosaic_masked_logits",
    "mosaic_masked_logits_device_count",
    "mosaic_num_chunks",
    "mosaic_logits_bytes",
    "mosaic_logits_variant",
    "mosaic_masked_logits_argmax_lse",
    "mosaic_masked_logits_argmax_lse_noalloc",
    "mosaic_masked_logits_argmax_lse_device_count",
    "mosaic_logits_argmax_lse_workspace_bytes",
    "mosaic_lazy_chunk_rows",
    "mosaic_quantize_rows_fp8",
    "mosaic_logits_fp8_workspace_bytes",
    "mosaic_masked_logits_fp8",
    "mosaic_debug_reload_env",
)


class MosaicError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {mosaic_status_string(status)} ({status})")


def _load() -> ctypes.CDLL:
    if not _LIB_PATH.exists():
        raise ImportError(f"{_LIB_PATH} is not built; run `python -m mask_only_logits_amd.build` "
                          "(or __graft_entry__.build()) first")
    lib = ctypes.CDLL(str(_LIB_PATH))
    i64, i32, p, st = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p, ctypes.c_int
    lib.mosaic_status_string.restype = ctypes.c_char_p
    lib.mosaic_status_string.argtypes = [st]
    sz = ctypes.c_size_t
    lib.mosaic_mask_compact_workspace_bytes.restype = sz
    lib.mosaic_mask_compact_workspace_bytes.argtypes = [i64]
    lib.mosaic_mask_compact.restype = st
    lib.mosaic_mask_compact.argtypes = [p, i64, i32, p, p, p, sz, p]
    lib.mosaic_mask_compact_flags.restype = st
    lib.mosaic_mask_compact_flags.argtypes = [p, i64, p, p, p, sz, p]
    lib.mosaic_mask_compact_batched.restype = st
    lib.mosaic_mask_compact_batched.argtypes = [p, i64, p, i32, i32, p, p, p, sz, p]
    lib.mosaic_masked_logits.restype = st
    lib.mosaic_masked_logits.argtypes = [p, i64, i64, p, i64, p, i64, p, i64, st, st, p]
    lib.mosaic_masked_logits_device_count.restype = st
    lib.mosaic_masked_logits_device_count.argtypes = [p, i64, i64, p, p, i64, p, i64, p, st, st, p]
    lib.mosaic_num_chunks.restype = i64
    lib.mosaic_num_chunks.argtypes = [i64, i64]
    lib.mosaic_logits_bytes.restype = st
    lib.mosaic_logits_bytes.argtypes = [i64, i64, st, ctypes.POINTER(i64)]
    lib.mosaic_logits_variant.restype = ctypes.c_int
    lib.mosaic_logits_variant.argtypes = [i64, i64, i64, st, st]
    lib.mosaic_masked_logits_argmax_lse.restype = st
    lib.mosaic_masked_logits_argmax_lse.argtypes = [p, i64, i64, p, i64, p, i64, p, i64, st, st, p, p, p, p, i64, p]
    lib.mosaic_masked_logits_argmax_lse_device_count.restype = st
    lib.mosaic_masked_logits_argmax_lse_device_count.argtypes = [p, i64, i64, p, p, i64, p, i64, p, st, st, p, p, p,
                                                                 p, i64, p]
    lib.mosaic_masked_logits_argmax_lse_noalloc.restype = st
    lib.mosaic_masked_logits_argmax_lse_noalloc.argtypes = [p, i64, i64, p, i64, p, i64, p, i64, st, st, p, p, p, p]
    lib.mosaic_logits_argmax_lse_workspace_bytes.restype = i64
    lib.mosaic_logits_argmax_lse_workspace_bytes.argtypes = [i64, i64, i64]
    lib.mosaic_quantize_rows_fp8.restype = st
    lib.mosaic_quantize_rows_fp8.argtypes = [p, i64, i64, st, p, i64, p, p, p]
    lib.mosaic_logits_fp8_workspace_bytes.restype = i64
    lib.mosaic_logits_fp8_workspace_bytes.argtypes = [i64, i64, i64]
    lib.mosaic_masked_logits_fp8.restype = st
    lib.mosaic_masked_logits_fp8.argtypes = [p, i64, i64, p, i64, p, p, i64, p, i64, st, p, i64, p]
    lib.mosaic_debug_reload_env.restype = None
    lib.mosaic_debug_reload_env.argtypes = []
    lib.mosaic_lazy_chunk_rows.restype = st
    lib.mosaic_lazy_chunk_rows.argtypes = [i64, i64, st, i64, ctypes.POINTER(i64), ctypes.POINTER(i64)]
    return lib


lib = _load()


def _dtype_code(t: torch.dtype) -> int:
    if t == torch.float32:
        return MOSAIC_F32
    if t == torch.bfloat16:
        return MOSAIC_BF16
    raise TypeError(f"unsupported dtype {t}")


def _torch_dtype(code: int) -> torch.dtype:
    return {MOSAIC_F32: torch.float32, MOSAIC_BF16: torch.bfloat16}[code]


def _dev(t: torch.Tensor | None, name: str, dtype: torch.dtype | None = None):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    return t.data_ptr() if t.numel() else None


def _stream(stream) -> int | None:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _check(status: int, where: str):
    if status != MOSAIC_OK:
        raise MosaicError(status, where)


def mosaic_debug_reload_env() -> None:
    """Make the library read MOSAIC_TUNE and MOSAIC_CHECK_IDX from the environment again."""
    lib.mosaic_debug_reload_env()


def mosaic_status_string(status: int) -> str:
    return lib.mosaic_status_string(int(status)).decode()


def mosaic_num_chunks(M: int, chunk_rows: int) -> int:
    return int(lib.mosaic_num_chunks(int(M), int(chunk_rows)))


def mosaic_logits_bytes(rows: int, V: int, dtype: torch.dtype) -> int:
    out = ctypes.c_int64()
    _check(lib.mosaic_logits_bytes(int(rows), int(V), _dtype_code(dtype), ctypes.byref(out)),
           "mosaic_logits_bytes")
    return int(out.value)


def mosaic_logits_variant(M: int, V: int, d: int, in_dtype: torch.dtype, out_dtype: torch.dtype) -> int:
    return int(lib.mosaic_logits_variant(int(M), int(V), int(d), _dtype_code(in_dtype), _dtype_code(out_dtype)))


def mosaic_lazy_chunk_rows(M: int, V: int, dtype: torch.dtype, budget_bytes: int):
    """(chunk_rows, num_chunks) of the lazy chunk choice for an [M, V] logits buffer of
    `dtype` under `budget_bytes`; chunk_rows 0 means no chunking."""
    c, k = ctypes.c_int64(), ctypes.c_int64()
    _check(lib.mosaic_lazy_chunk_rows(int(M), int(V), _dtype_code(dtype), int(budget_bytes), ctypes.byref(c),
                                      ctypes.byref(k)), "mosaic_lazy_chunk_rows")
    return int(c.value), int(k.value)


def mosaic_mask_compact_workspace_bytes(L: int) -> int:
    """Workspace bytes the compaction calls need for L positions."""
    return int(lib.mosaic_mask_compact_workspace_bytes(int(L)))


def _compact_workspace(L: int, workspace: torch.Tensor | None, device):
    """(pointer, bytes) of the compaction workspace, allocated if absent and needed."""
    if workspace is None:
        need = mosaic_mask_compact_workspace_bytes(L)
        if need == 0:
            return None, 0
        workspace = torch.empty(need, dtype=torch.uint8, device=device)
    return _dev(workspace, "workspace", torch.uint8), workspace.numel()


def mosaic_mask_compact(tokens: torch.Tensor, mask_id: int, idx: torch.Tensor | None = None,
                        count: torch.Tensor | None = None, workspace: torch.Tensor | None = None, stream=None):
    """Masked positions of int32 `tokens` in ascending order -> (idx [L] int32, count [1] int32).

    Asynchronous: idx[:count] holds the list once the stream reaches this point."""
    L = tokens.numel()
    if idx is None:
        idx = torch.empty(max(L, 1), dtype=torch.int32, device=tokens.device)
    if count is None:
        count = torch.empty(1, dtype=torch.int32, device=tokens.device)
    ws, wsb = _compact_workspace(L, workspace, tokens.device)
    _check(lib.mosaic_mask_compact(_dev(tokens, "tokens", torch.int32), L, int(mask_id),
                                   _dev(idx, "idx", torch.int32), _dev(count, "count", torch.int32), ws, wsb,
                                   _stream(stream)), "mosaic_mask_compact")
    return idx, count


def mosaic_mask_compact_flags(flags: torch.Tensor, idx: torch.Tensor | None = None,
                              count: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                              stream=None):
    """Positions with flags != 0 (uint8 or bool flags) -> (idx, count)."""
    if flags.dtype == torch.bool:
        flags = flags.view(torch.uint8)
    L = flags.numel()
    if idx is None:
        idx = torch.empty(max(L, 1), dtype=torch.int32, device=flags.device)
    if count is None:
        count = torch.empty(1, dtype=torch.int32, device=flags.device)
    ws, wsb = _compact_workspace(L, workspace, flags.device)
    _check(lib.mosaic_mask_compact_flags(_dev(flags, "flags", torch.uint8), L, _dev(idx, "idx", torch.int32),
                                         _dev(count, "count", torch.int32), ws, wsb, _stream(stream)),
           "mosaic_mask_compact_flags")
    return idx, count


def mosaic_mask_compact_batched(tokens: torch.Tensor, seq_offsets: torch.Tensor, mask_id: int,
                                idx: torch.Tensor | None = None, idx_offsets: torch.Tensor | None = None,
                                workspace: torch.Tensor | None = None, stream=None):
    """Ragged batch -> (idx [L] global positions, idx_offsets [nseq+1] CSR)."""
    L = tokens.numel()
    nseq = seq_offsets.numel() - 1
    if idx is None:
        idx = torch.empty(max(L, 1), dtype=torch.int32, device=tokens.device)
    if idx_offsets is None:
        idx_offsets = torch.empty(max(nseq + 1, 1), dtype=torch.int32, device=tokens.device)
    ws, wsb = _compact_workspace(L, workspace, tokens.device)
    _check(lib.mosaic_mask_compact_batched(_dev(tokens, "tokens", torch.int32), L,
                                           _dev(seq_offsets, "seq_offsets", torch.int32), nseq, int(mask_id),
                                           _dev(idx, "idx", torch.int32),
                                           _dev(idx_offsets, "idx_offsets", torch.int32), ws, wsb,
                                           _stream(stream)),
           "mosaic_mask_compact_batched")
    return idx, idx_offsets


def mosaic_masked_logits(H: torch.Tensor, idx: torch.Tensor, W: torch.Tensor, M: int | None = None,
                         out: torch.Tensor | None = None, chunk_rows: int = 0,
                         out_dtype: torch.dtype | None = None, stream=None) -> torch.Tensor:
    """logits[M, V] = H[idx[:M], :] @ W.T in chunks of at most chunk_rows rows.

    H [L, d] and W [V, d] share a dtype (bf16 or fp32); idx is int32 with at least M
    entries (M defaults to idx.numel()).  `out` (allocated if absent) is [M, V]."""
    if H.dim() != 2 or W.dim() != 2 or H.shape[1] != W.shape[1]:
        raise ValueError("H must be [L, d] and W [V, d]")
    if H.dtype != W.dtype:
        raise TypeError("H and W must share a dtype")
    L, d = H.shape
    V = W.shape[0]
    M = idx.numel() if M is None else int(M)
    if M > idx.numel():
        raise ValueError("M exceeds the length of idx")
    if out is None:
        out = torch.empty((M, V), dtype=out_dtype or H.dtype, device=H.device)
    elif out.numel() < M * V:
        raise ValueError("out is smaller than M * V")
    _check(lib.mosaic_masked_logits(_dev(H, "H"), L, d, _dev(idx, "idx", torch.int32), M, _dev(W, "W"), V,
                                    _dev(out, "out"), int(chunk_rows), _dtype_code(H.dtype),
                                    _dtype_code(out.dtype), _stream(stream)), "mosaic_masked_logits")
    return out


def mosaic_masked_logits_device_count(H: torch.Tensor, idx: torch.Tensor, W: torch.Tensor, count: torch.Tensor,
                                      max_rows: int | None = None, out: torch.Tensor | None = None,
                                      stream=None) -> torch.Tensor:
    """logits = H[idx[:M], :] @ W.T with M = clamp(count[0], 0, max_rows) read on the device
    (count: an int32 device tensor, e.g. mosaic_mask_compact's count); nothing waits for
    it.  bf16 H [L, d] and W [V, d] with d % 64 == 0.  `out` (allocated if absent) is
    [max_rows, V] (max_rows defaults to idx.numel()); rows >= M are not written."""
    if H.dim() != 2 or W.dim() != 2 or H.shape[1] != W.shape[1]:
        raise ValueError("H must be [L, d] and W [V, d]")
    if H.dtype != W.dtype:
        raise TypeError("H and W must share a dtype")
    L, d = H.shape
    V = W.shape[0]
    max_rows = idx.numel() if max_rows is None else int(max_rows)
    if max_rows > idx.numel():
        raise ValueError("max_rows exceeds the length of idx")
    if out is None:
        out = torch.empty((max_rows, V), dtype=H.dtype, device=H.device)
    elif out.numel() < max_rows * V:
        raise ValueError("out is smaller than max_rows * V")
    _check(lib.mosaic_masked_logits_device_count(_dev(H, "H"), L, d, _dev(idx, "idx", torch.int32),
                                                 _dev(count, "count", torch.int32), max_rows, _dev(W, "W"), V,
                                                 _dev(out, "out"), _dtype_code(H.dtype), _dtype_code(out.dtype),
                                                 _stream(stream)), "mosaic_masked_logits_device_count")
    return out


def mosaic_logits_argmax_lse_workspace_bytes(M: int, chunk_rows: int, V: int) -> int:
    """Workspace bytes mosaic_masked_logits_argmax_lse needs for M rows in chunks of chunk_rows."""
    n = int(lib.mosaic_logits_argmax_lse_workspace_bytes(int(M), int(chunk_rows), int(V)))
    if n < 0:
        raise ValueError("workspace size overflows")
    return n


def mosaic_masked_logits_argmax_lse(H: torch.Tensor, idx: torch.Tensor, W: torch.Tensor, M: int | None = None,
                                    chunk_rows: int = 0, store_logits: bool = False,
                                    out: torch.Tensor | None = None, row_max: torch.Tensor | None = None,
                                    row_argmax: torch.Tensor | None = None, row_lse: torch.Tensor | None = None,
                                    workspace: torch.Tensor | None = None, stream=None):
    """Per masked row i: (row_max[i], row_argmax[i], row_lse[i]) of its fp32 logits
    H[idx[i]] . W^T -- the largest logit, the first vocabulary index attaining it and
    log(sum_v exp(logit_v)).  bf16 H [L, d] and W [V, d] with d % 64 == 0.

    The logits are stored only if `store_logits` (or `out` is given): then `out`
    ([M, V] bf16, allocated if absent) holds them and is returned as the fourth item,
    else the fourth item is None.  `workspace` (uint8, allocated if absent) must hold
    mosaic_logits_argmax_lse_workspace_bytes(M, chunk_rows, V) bytes."""
    if H.dim() != 2 or W.dim() != 2 or H.shape[1] != W.shape[1]:
        raise ValueError("H must be [L, d] and W [V, d]")
    L, d = H.shape
    V = W.shape[0]
    M = idx.numel() if M is None else int(M)
    if M > idx.numel():
        raise ValueError("M exceeds the length of idx")
    dev = H.device
    if store_logits and out is None:
        out = torch.empty((M, V), dtype=torch.bfloat16, device=dev)
    if out is not None and out.numel() < M * V:
        raise ValueError("out is smaller than M * V")
    row_max = torch.empty(M, dtype=torch.float32, device=dev) if row_max is None else row_max
    row_argmax = torch.empty(M, dtype=torch.int32, device=dev) if row_argmax is None else row_argmax
    row_lse = torch.empty(M, dtype=torch.float32, device=dev) if row_lse is None else row_lse
    for name, t in (("row_max", row_max), ("row_argmax", row_argmax), ("row_lse", row_lse)):
        if t.numel() < M:
            raise ValueError(f"{name} has fewer than M entries")
    need = mosaic_logits_argmax_lse_workspace_bytes(M, chunk_rows, V)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    _check(lib.mosaic_masked_logits_argmax_lse(
        _dev(H, "H"), L, d, _dev(idx, "idx", torch.int32), M, _dev(W, "W"), V,
        _dev(out, "out") if out is not None else None, int(chunk_rows), _dtype_code(H.dtype),
        _dtype_code(out.dtype) if out is not None else MOSAIC_BF16,
        _dev(row_max, "row_max", torch.float32), _dev(row_argmax, "row_argmax", torch.int32),
        _dev(row_lse, "row_lse", torch.float32), _dev(workspace, "workspace", torch.uint8), workspace.numel(),
        _stream(stream)), "mosaic_masked_logits_argmax_lse")
    return row_max, row_argmax, row_lse, out


def mosaic_masked_logits_argmax_lse_device_count(H: torch.Tensor, idx: torch.Tensor, W: torch.Tensor,
                                                 count: torch.Tensor, max_rows: int | None = None,
                                                 store_logits: bool = False, out: torch.Tensor | None = None,
                                                 row_max: torch.Tensor | None = None,
                                                 row_argmax: torch.Tensor | None = None,
                                                 row_lse: torch.Tensor | None = None,
                                                 workspace: torch.Tensor | None = None, stream=None):
    """mosaic_masked_logits_argmax_lse with M = clamp(count[0], 0, max_rows) read on the
    device (count: an int32 device tensor, e.g. the compaction's count); nothing waits for
    it.  Arrays are sized for max_rows (default idx.numel()); rows >= M are not written."""
    if H.dim() != 2 or W.dim() != 2 or H.shape[1] != W.shape[1]:
        raise ValueError("H must be [L, d] and W [V, d]")
    L, d = H.shape
    V = W.shape[0]
    R = idx.numel() if max_rows is None else int(max_rows)
    if R > idx.numel():
        raise ValueError("max_rows exceeds the length of idx")
    dev = H.device
    if store_logits and out is None:
        out = torch.empty((R, V), dtype=torch.bfloat16, device=dev)
    if out is not None and out.numel() < R * V:
        raise ValueError("out is smaller than max_rows * V")
    row_max = torch.empty(R, dtype=torch.float32, device=dev) if row_max is None else row_max
    row_argmax = torch.empty(R, dtype=torch.int32, device=dev) if row_argmax is None else row_argmax
    row_lse = torch.empty(R, dtype=torch.float32, device=dev) if row_lse is None else row_lse
    for name, t in (("row_max", row_max), ("row_argmax", row_argmax), ("row_lse", row_lse)):
        if t.numel() < R:
            raise ValueError(f"{name} has fewer than max_rows entries")
    need = mosaic_logits_argmax_lse_workspace_bytes(R, 0, V)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    _check(lib.mosaic_masked_logits_argmax_lse_device_count(
        _dev(H, "H"), L, d, _dev(idx, "idx", torch.int32), _dev(count, "count", torch.int32), R, _dev(W, "W"), V,
        _dev(out, "out") if out is not None else None, _dtype_code(H.dtype),
        _dtype_code(out.dtype) if out is not None else MOSAIC_BF16,
        _dev(row_max, "row_max", torch.float32), _dev(row_argmax, "row_argmax", torch.int32),
        _dev(row_lse, "row_lse", torch.float32), _dev(workspace, "workspace", torch.uint8), workspace.numel(),
        _stream(stream)), "mosaic_masked_logits_argmax_lse_device_count")
    return row_max, row_argmax, row_lse, out


def mosaic_masked_logits_argmax_lse_noalloc(H: torch.Tensor, idx: torch.Tensor, W: torch.Tensor,
                                            row_max: torch.Tensor, row_argmax: torch.Tensor,
                                            row_lse: torch.Tensor, M: int | None = None, chunk_rows: int = 0,
                                            out: torch.Tensor | None = None, stream=None):
    """mosaic_masked_logits_argmax_lse without a workspace: the library allocates nothing
    and the partials use its own per-device scratch array.  The caller passes every
    output (row_max float32 [M], row_argmax int32 [M], row_lse float32 [M], and `out`
    [M, V] bf16 when the logits are wanted); this wrapper allocates nothing either."""
    if H.dim() != 2 or W.dim() != 2 or H.shape[1] != W.shape[1]:
        raise ValueError("H must be [L, d] and W [V, d]")
    L, d = H.shape
    V = W.shape[0]
    M = idx.numel() if M is None else int(M)
    if M > idx.numel():
        raise ValueError("M exceeds the length of idx")
    if out is not None and out.numel() < M * V:
        raise ValueError("out is smaller than M * V")
    for name, t in (("row_max", row_max), ("row_argmax", row_argmax), ("row_lse", row_lse)):
        if t.numel() < M:
            raise ValueError(f"{name} has fewer than M entries")
    _check(lib.mosaic_masked_logits_argmax_lse_noalloc(
        _dev(H, "H"), L, d, _dev(idx, "idx", torch.int32), M, _dev(W, "W"), V,
        _dev(out, "out") if out is not None else None, int(chunk_rows), _dtype_code(H.dtype),
        _dtype_code(out.dtype) if out is not None else MOSAIC_BF16,
        _dev(row_max, "row_max", torch.float32), _dev(row_argmax, "row_argmax", torch.int32),
        _dev(row_lse, "row_lse", torch.float32), _stream(stream)), "mosaic_masked_logits_argmax_lse_noalloc")
    return row_max, row_argmax, row_lse, out


def mosaic_quantize_rows_fp8(X: torch.Tensor, row_idx: torch.Tensor | None = None, rows: int | None = None,
                             q: torch.Tensor | None = None, scale: torch.Tensor | None = None, stream=None):
    """Per-row OCP E4M3 quantization of X [n, d] (bf16 or fp32): returns (codes uint8
    [rows, d], scales float32 [rows]); rows = len(row_idx) (gathered rows) or n."""
    if X.dim() != 2:
        raise ValueError("X must be [n, d]")
    n, d = X.shape
    if rows is None:
        rows = n if row_idx is None else row_idx.numel()
    if q is None:
        q = torch.empty((rows, d), dtype=torch.uint8, device=X.device)
    if scale is None:
        scale = torch.empty(rows, dtype=torch.float32, device=X.device)
    _check(lib.mosaic_quantize_rows_fp8(_dev(X, "X"), n, d, _dtype_code(X.dtype),
                                        _dev(row_idx, "row_idx", torch.int32) if row_idx is not None else None,
                                        int(rows), _dev(q, "q", torch.uint8), _dev(scale, "scale", torch.float32),
                                        _stream(stream)), "mosaic_quantize_rows_fp8")
    return q, scale


def mosaic_logits_fp8_workspace_bytes(M: int, chunk_rows: int, d: int) -> int:
    """Workspace bytes mosaic_masked_logits_fp8 needs for M rows in chunks of chunk_rows."""
    n = int(lib.mosaic_logits_fp8_workspace_bytes(int(M), int(chunk_rows), int(d)))
    if n < 0:
        raise ValueError("workspace size overflows")
    return n


def mosaic_masked_logits_fp8(H: torch.Tensor, idx: torch.Tensor, Wq: torch.Tensor, w_scale: torch.Tensor,
                             M: int | None = None, out: torch.Tensor | None = None, chunk_rows: int = 0,
                             workspace: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """bf16 logits [M, V] of the FP8 LM head: H[idx[:M]] quantized per row on the fly,
    times the pre-quantized W (Wq uint8 [V, d], w_scale float32 [V])."""
    if H.dim() != 2 or Wq.dim() != 2 or H.shape[1] != Wq.shape[1]:
        raise ValueError("H must be [L, d] and Wq [V, d]")
    L, d = H.shape
    V = Wq.shape[0]
    M = idx.numel() if M is None else int(M)
    if M > idx.numel():
        raise ValueError("M exceeds the length of idx")
    if out is None:
        out = torch.empty((M, V), dtype=torch.bfloat16, device=H.device)
    elif out.numel() < M * V:
        raise ValueError("out is smaller than M * V")
    if workspace is None:
        workspace = torch.empty(max(16, mosaic_logits_fp8_workspace_bytes(M, chunk_rows, d)), dtype=torch.uint8,
                                device=H.device)
    _check(lib.mosaic_masked_logits_fp8(_dev(H, "H", torch.bfloat16), L, d, _dev(idx, "idx", torch.int32), M,
                                        _dev(Wq, "Wq", torch.uint8), _dev(w_scale, "w_scale", torch.float32), V,
                                        _dev(out, "out"), int(chunk_rows), _dtype_code(out.dtype),
                                        _dev(workspace, "workspace", torch.uint8), workspace.numel(),
                                        _stream(stream)), "mosaic_masked_logits_fp8")
    return out
