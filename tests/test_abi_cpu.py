"""The C-ABI library without a GPU: it loads, exports every declared symbol, and its
host-side logic (status strings, chunk arithmetic, size helper, argument validation)
behaves as declared.  No call here enqueues device work: every call is rejected by
validation before any HIP call, or returns early for empty problems."""
import ctypes
import os
import re

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def m():
    from mask_only_logits_amd import mosaic
    return mosaic


def test_exports_every_declared_symbol(m):
    hdr = open(os.path.join(ROOT, "include", "mosaic.h"), encoding="utf-8").read()
    declared = set(re.findall(r"\b(mosaic_[a-z0-9_]+)\s*\(", hdr))
    assert declared == set(m.EXPORTS)
    for name in declared:
        assert hasattr(m.lib, name), name


def test_status_strings(m):
    assert m.mosaic_status_string(0) == "MOSAIC_OK"
    assert m.mosaic_status_string(1) == "MOSAIC_ERR_INVALID_ARG"
    assert m.mosaic_status_string(2) == "MOSAIC_ERR_UNSUPPORTED"
    assert m.mosaic_status_string(3) == "MOSAIC_ERR_DEVICE"
    assert m.mosaic_status_string(99) == "MOSAIC_ERR_UNKNOWN"


def test_num_chunks_matches_oracle(m):
    for M in list(range(0, 70)) + [1229, 29491, 39322]:
        for C in (-2, 0, 1, 2, 7, 63, 64, 65, 4096, 8192):
            assert m.mosaic_num_chunks(M, C) == oracle.num_chunks(M, C), (M, C)


def test_logits_bytes(m):
    import torch
    assert m.mosaic_logits_bytes(16 * 2048, 126464, torch.bfloat16) == 8_287_944_704
    assert m.mosaic_logits_bytes(29491, 126464, torch.bfloat16) == 7_459_099_648
    assert m.mosaic_logits_bytes(128, 1024, torch.float32) == 524_288
    out = ctypes.c_int64(-7)
    assert m.lib.mosaic_logits_bytes(2**62, 4, 1, ctypes.byref(out)) == m.MOSAIC_ERR_INVALID_ARG
    assert m.lib.mosaic_logits_bytes(-1, 4, 1, ctypes.byref(out)) == m.MOSAIC_ERR_INVALID_ARG
    assert m.lib.mosaic_logits_bytes(1, 4, 7, ctypes.byref(out)) == m.MOSAIC_ERR_INVALID_ARG
    assert m.lib.mosaic_logits_bytes(1, 4, 1, None) == m.MOSAIC_ERR_INVALID_ARG
    assert out.value == -7


def test_variant_choice(m):
    import torch
    bf, f32 = torch.bfloat16, torch.float32
    assert m.mosaic_logits_variant(4096, 126464, 4096, bf, bf) == 22     # persistent, 16 x 16 x 32 MFMA
    assert m.mosaic_logits_variant(65, 152064, 3584, bf, bf) == 22
    assert m.mosaic_logits_variant(21399, 152064, 3584, bf, bf) == 22
    assert m.mosaic_logits_variant(4096, 126464, 4096, bf, f32) == 12    # 8-wave tiled kernel
    assert m.mosaic_logits_variant(20, 152064, 3584, bf, bf) == 20       # low-M streaming kernel, shared H
    assert m.mosaic_logits_variant(64, 152064, 3584, bf, f32) == 20
    assert m.mosaic_logits_variant(20, 1000, 96, bf, bf) == 11           # d % 32 == 0 only
    assert m.mosaic_logits_variant(5000, 1000, 96, bf, f32) == 11
    assert m.mosaic_logits_variant(128, 1024, 256, f32, f32) == 0
    assert m.mosaic_logits_variant(10, 10, 72, bf, f32) == 2          # d % 64 != 0
    assert m.mosaic_logits_variant(10, 10, 12, bf, bf) == -1          # d % 8 != 0
    assert m.mosaic_logits_variant(10, 10, 64, f32, bf) == -1         # fp32 -> bf16 not offered


# Fake, never-dereferenced addresses: validation rejects these calls before any HIP call.
A16 = 1 << 20            # 16-byte aligned
A8 = (1 << 20) + 8       # misaligned for 16 bytes


def _logits(m, H=A16, L=100, d=64, idx=A16, M=10, W=A16, V=50, out=A16, C=0, i=1, o=1):
    return m.lib.mosaic_masked_logits(H, L, d, idx, M, W, V, out, C, i, o, None)


@pytest.mark.parametrize("kw,status", [
    (dict(M=-1), 1), (dict(V=-1), 1), (dict(L=-1), 1), (dict(d=-1), 1),
    (dict(H=None), 1), (dict(W=None), 1), (dict(idx=None), 1), (dict(out=None), 1),
    (dict(L=0), 1), (dict(d=0), 1),
    (dict(H=A8), 1), (dict(W=A8), 1), (dict(out=A8), 1), (dict(idx=A16 + 2), 1),
    (dict(i=5), 1), (dict(o=9), 1),
    (dict(d=12), 2), (dict(i=0, o=1), 2), (dict(i=0, o=0, d=6), 2),
    (dict(M=2**40, V=2**30), 1),
    (dict(L=2**31), 2),
])
def test_logits_validation(m, kw, status):
    assert _logits(m, **kw) == status


def test_empty_problems_are_ok_without_pointers(m):
    assert _logits(m, M=0, H=None, W=None, idx=None, out=None) == 0
    assert _logits(m, V=0, H=None, W=None, idx=None, out=None) == 0


def _logits_dc(m, H=A16, L=100, d=64, idx=A16, count=A16, R=10, W=A16, V=50, out=A16, i=1, o=1):
    return m.lib.mosaic_masked_logits_device_count(H, L, d, idx, count, R, W, V, out, i, o, None)


@pytest.mark.parametrize("kw,status", [
    (dict(R=-1), 1), (dict(V=-1), 1), (dict(L=-1), 1), (dict(d=-1), 1),
    (dict(H=None), 1), (dict(W=None), 1), (dict(idx=None), 1), (dict(out=None), 1), (dict(count=None), 1),
    (dict(L=0), 1),
    (dict(H=A8), 1), (dict(W=A8), 1), (dict(out=A8), 1), (dict(idx=A16 + 2), 1), (dict(count=A16 + 2), 1),
    (dict(i=5), 1), (dict(o=9), 1),
    # one form only: bf16 -> bf16, d % 64 == 0
    (dict(d=96), 2), (dict(i=0, o=0), 2), (dict(i=1, o=0), 2), (dict(i=0, o=1), 2),
    (dict(R=2**40, V=2**30), 1),
    (dict(L=2**31), 2), (dict(R=2**31), 2),
])
def test_logits_device_count_validation(m, kw, status):
    assert _logits_dc(m, **kw) == status


def test_device_count_empty_problems_are_ok_without_pointers(m):
    assert _logits_dc(m, R=0, H=None, W=None, idx=None, count=None, out=None) == 0
    assert _logits_dc(m, V=0, H=None, W=None, idx=None, count=None, out=None) == 0


def _lse_dc(m, H=A16, L=100, d=64, idx=A16, count=A16, R=10, W=A16, V=50, out=None, i=1, o=1, rm=A16, ra=A16,
            rl=A16, ws=A16, wsb=1 << 20):
    return m.lib.mosaic_masked_logits_argmax_lse_device_count(H, L, d, idx, count, R, W, V, out, i, o, rm, ra, rl,
                                                              ws, wsb, None)


@pytest.mark.parametrize("kw,status", [
    (dict(R=-1), 1), (dict(V=0), 1), (dict(count=None), 1), (dict(count=A16 + 2), 1), (dict(ws=None), 1),
    (dict(wsb=16), 1), (dict(rm=None), 1), (dict(rl=A16 + 2), 1), (dict(out=A8), 1),
    (dict(d=96), 2), (dict(i=0), 2), (dict(out=A16, o=0), 2), (dict(R=2**31), 2),
])
def test_argmax_lse_device_count_validation(m, kw, status):
    assert _lse_dc(m, **kw) == status


def test_argmax_lse_device_count_workspace_exact(m):
    need = m.mosaic_logits_argmax_lse_workspace_bytes(10, 0, 50)
    assert _lse_dc(m, wsb=need - 1) == 1
    assert _lse_dc(m, R=0, H=None, W=None, idx=None, count=None, rm=None, ra=None, rl=None, ws=None) == 0


def test_compact_workspace_bytes(m):
    f = m.lib.mosaic_mask_compact_workspace_bytes
    for L in (0, 1, 8192, 131072, 2**31 - 1):
        assert f(L) == 0
    assert m.mosaic_mask_compact_workspace_bytes(65536) == 0


def test_compact_validation(m):
    L = m.lib
    assert L.mosaic_mask_compact(A16, -1, 0, A16, A16, None, 0, None) == 1
    assert L.mosaic_mask_compact(None, 10, 0, A16, A16, None, 0, None) == 1
    assert L.mosaic_mask_compact(A16, 10, 0, None, A16, None, 0, None) == 1
    assert L.mosaic_mask_compact(A16, 10, 0, A16, None, None, 0, None) == 1
    assert L.mosaic_mask_compact(A16, 2**31, 0, A16, A16, None, 0, None) == 2
    assert L.mosaic_mask_compact_flags(None, 10, A16, A16, None, 0, None) == 1
    assert L.mosaic_mask_compact_flags(A16, 10, A16, None, None, 0, None) == 1
    assert L.mosaic_mask_compact_batched(A16, 10, A16, 0, 0, A16, A16, None, 0, None) == 1
    assert L.mosaic_mask_compact_batched(A16, 10, None, 2, 0, A16, A16, None, 0, None) == 1
    assert L.mosaic_mask_compact_batched(A16, 10, A16, 2, 0, A16, None, None, 0, None) == 1
    assert L.mosaic_mask_compact_batched(A16, 2**31, A16, 2, 0, A16, A16, None, 0, None) == 2


def test_compact_rejects_claimed_bytes_without_a_workspace(m):
    # bytes claimed for a NULL workspace are an inconsistent argument pair
    L = m.lib
    assert L.mosaic_mask_compact(A16, 10, 0, A16, A16, None, 64, None) == 1
    assert L.mosaic_mask_compact_flags(A16, 10, A16, A16, None, 64, None) == 1
    assert L.mosaic_mask_compact_batched(A16, 10, A16, 2, 0, A16, A16, None, 64, None) == 1
    # an empty sequence with a consistent (empty) workspace still validates its pointers
    assert L.mosaic_mask_compact(None, 0, 0, None, None, None, 0, None) == 1


def test_binding_rejects_host_tensors(m):
    import torch
    with pytest.raises(ValueError):
        m.mosaic_mask_compact(torch.zeros(4, dtype=torch.int32), 1,
                              idx=torch.zeros(4, dtype=torch.int32), count=torch.zeros(1, dtype=torch.int32))


def test_product_path_does_not_touch_the_oracle():
    # the package's sources never import or load the CPU oracle
    pkg = os.path.join(ROOT, "mask_only_logits_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".cpp", ".h")):
                text = open(os.path.join(dirpath, f), encoding="utf-8").read()
                assert "import oracle" not in text and "liboracle" not in text, f


def _argmax_lse(m, H=A16, L=100, d=64, idx=A16, M=10, W=A16, V=50, out=None, C=0, i=1, o=1,
                rmax=A16, rarg=A16, rlse=A16, ws=A16, wsb=1 << 20):
    return m.lib.mosaic_masked_logits_argmax_lse(H, L, d, idx, M, W, V, out, C, i, o, rmax, rarg, rlse, ws, wsb,
                                                 None)


def test_argmax_lse_workspace_bytes(m):
    f = m.lib.mosaic_logits_argmax_lse_workspace_bytes
    # (M, chunk_rows, V): sized by the largest chunk
    assert f(29491, 4096, 126464) == 12 * 494 * 4096
    assert f(4096, 0, 126464) == 12 * 494 * 4096
    assert f(10, 0, 1) == 120 and f(10, 0, 256) == 120 and f(10, 0, 257) == 240
    assert f(10, 100, 256) == 120                       # chunk_rows >= M: one chunk of M rows
    assert f(1000, 100, 256) == 1200 and f(1001, 100, 256) == 1200
    assert f(0, 0, 100) == 0 and f(0, 7, 100) == 0
    assert f(-1, 0, 10) == -1 and f(10, 0, -1) == -1
    assert f(2**62, 0, 2**20) == -1
    assert m.mosaic_logits_argmax_lse_workspace_bytes(1000, 100, 256) == 1200


def test_argmax_lse_rejects_a_workspace_one_byte_short(m):
    for M, C, V in ((10, 0, 50), (1000, 100, 300), (1001, 100, 300), (37, 5, 513)):
        need = m.mosaic_logits_argmax_lse_workspace_bytes(M, C, V)
        assert _argmax_lse(m, M=M, C=C, V=V, wsb=need - 1) == 1


@pytest.mark.parametrize("kw,status", [
    (dict(M=-1), 1), (dict(V=-1), 1), (dict(L=-1), 1), (dict(d=-1), 1),
    (dict(V=0), 1),                                     # the max of an empty row does not exist
    (dict(i=0), 2), (dict(i=0, d=4), 2),                # fp32 inputs are not offered
    (dict(d=72), 2), (dict(d=96), 2),                   # needs d % 64 == 0
    (dict(out=A16, o=0), 2),                            # stored logits are bf16 only
    (dict(i=7), 1), (dict(out=A16, o=7), 1),
    (dict(H=None), 1), (dict(W=None), 1), (dict(idx=None), 1),
    (dict(rmax=None), 1), (dict(rarg=None), 1), (dict(rlse=None), 1), (dict(ws=None), 1),
    (dict(H=A8), 1), (dict(ws=A8), 1), (dict(out=A8), 1), (dict(rmax=A16 + 2), 1), (dict(idx=A16 + 1), 1),
    (dict(wsb=12 * 1 * 10 - 1), 1),                     # one 256-entry tile x 10 rows needs 120 bytes
    (dict(V=300, wsb=12 * 1 * 10), 1),                  # two tiles need 240
    (dict(M=1000, C=100, wsb=12 * 1 * 100 - 4), 1),     # sized by the chunk, not by M
    (dict(L=2**31), 2),
])
def test_argmax_lse_validation(m, kw, status):
    assert _argmax_lse(m, **kw) == status


def test_argmax_lse_empty_is_ok_without_pointers(m):
    assert _argmax_lse(m, M=0, H=None, W=None, idx=None, rmax=None, rarg=None, rlse=None, ws=None, wsb=0) == 0


def test_lazy_chunk_rows_matches_oracle(m):
    import itertools

    import torch

    import oracle
    for M, V in itertools.product((1, 2, 7, 33, 100, 257), (1, 5, 64)):
        for dt, es in ((torch.bfloat16, 2), (torch.float32, 4)):
            for budget in sorted({V * es, V * es + 1, 3 * V * es - 1, M * V * es - 1, M * V * es, 10 * M * V * es}):
                if budget < V * es:
                    continue
                assert m.mosaic_lazy_chunk_rows(M, V, dt, budget) == oracle.lazy_chunk_rows(M, V, es, budget)
    assert m.mosaic_lazy_chunk_rows(29491, 126464, torch.bfloat16, 4096 * 126464 * 2) == (3687, 8)
    assert m.mosaic_lazy_chunk_rows(0, 10, torch.bfloat16, 0) == (0, 0)


def test_lazy_chunk_rows_errors(m):
    import ctypes
    c, k = ctypes.c_int64(), ctypes.c_int64()
    f = m.lib.mosaic_lazy_chunk_rows
    assert f(10, 500, 1, 999, ctypes.byref(c), ctypes.byref(k)) == 2        # one row does not fit
    assert f(-1, 500, 1, 999, ctypes.byref(c), ctypes.byref(k)) == 1
    assert f(10, 500, 7, 10**9, ctypes.byref(c), ctypes.byref(k)) == 1      # unknown dtype
    assert f(10, 500, 1, 10**9, None, ctypes.byref(k)) == 1
    assert f(2**40, 2**30, 1, 2**62, ctypes.byref(c), ctypes.byref(k)) == 0  # M * V * esize overflows int64
    assert c.value == 2**31 and k.value == 2**9


def test_fp8_workspace_bytes(m):
    f = m.lib.mosaic_logits_fp8_workspace_bytes
    # (M, chunk_rows, d): sized by the largest chunk
    assert f(4096, 0, 4096) == 4096 * 4096 + 4 * 4096
    assert f(29491, 4096, 4096) == 4096 * 4096 + 4 * 4096
    assert f(3, 0, 10) == 32 + 12
    assert f(30, 3, 10) == 32 + 12 and f(31, 3, 10) == 32 + 12
    assert f(0, 0, 10) == 0
    assert f(-1, 0, 10) == -1 and f(10, 0, -1) == -1
    assert f(2**62, 0, 2**10) == -1


def test_fp8_rejects_a_workspace_one_byte_short(m):
    for M, C, d in ((10, 0, 128), (1000, 100, 256), (1001, 100, 128)):
        need = m.mosaic_logits_fp8_workspace_bytes(M, C, d)
        assert _lf8(m, M=M, C=C, d=d, wb=need - 1) == 1


def _quant(m, X=A16, n=100, d=64, i=1, ridx=None, rows=10, q=A16, sc=A16):
    return m.lib.mosaic_quantize_rows_fp8(X, n, d, i, ridx, rows, q, sc, None)


@pytest.mark.parametrize("kw,status", [
    (dict(n=-1), 1), (dict(d=-1), 1), (dict(rows=-1), 1), (dict(i=7), 1),
    (dict(d=12), 2),                                   # d % 8 != 0
    (dict(X=None), 1), (dict(q=None), 1), (dict(sc=None), 1),
    (dict(X=A8), 1), (dict(q=A8), 1), (dict(sc=A16 + 2), 1), (dict(ridx=A16 + 1), 1),
    (dict(rows=101), 1),                               # more rows than the source without an index list
    (dict(n=2**40, d=2**30), 1),
])
def test_quantize_fp8_validation(m, kw, status):
    assert _quant(m, **kw) == status


def test_quantize_fp8_empty_is_ok(m):
    assert _quant(m, rows=0, X=None, q=None, sc=None) == 0


def _lf8(m, H=A16, L=100, d=128, idx=A16, M=10, Wq=A16, ws=A16, V=50, out=A16, C=0, o=1, w=A16, wb=1 << 20):
    return m.lib.mosaic_masked_logits_fp8(H, L, d, idx, M, Wq, ws, V, out, C, o, w, wb, None)


@pytest.mark.parametrize("kw,status", [
    (dict(M=-1), 1), (dict(V=-1), 1), (dict(L=-1), 1), (dict(d=-1), 1), (dict(o=5), 1),
    (dict(d=64), 2), (dict(d=192), 2),                 # d % 128 != 0
    (dict(o=0), 2),                                    # fp32 logits not offered
    (dict(H=None), 1), (dict(idx=None), 1), (dict(Wq=None), 1), (dict(ws=None), 1), (dict(out=None), 1),
    (dict(w=None), 1),
    (dict(H=A8), 1), (dict(Wq=A8), 1), (dict(out=A8), 1), (dict(w=A8), 1), (dict(ws=A16 + 4), 1),
    (dict(wb=10 * 128 + 40 - 1), 1),                   # 10 rows x 128 codes + 10 scales
    (dict(M=1000, C=100, wb=100 * 128 + 400 - 1), 1),  # sized by the chunk
    (dict(L=2**31), 2),
])
def test_logits_fp8_validation(m, kw, status):
    assert _lf8(m, **kw) == status


def test_logits_fp8_empty_is_ok(m):
    assert _lf8(m, M=0, H=None, idx=None, Wq=None, ws=None, out=None, w=None, wb=0) == 0


def _noalloc(m, H=A16, L=100, d=64, idx=A16, M=10, W=A16, V=50, out=None, C=0, i=1, o=1,
             rmax=A16, rarg=A16, rlse=A16):
    return m.lib.mosaic_masked_logits_argmax_lse_noalloc(H, L, d, idx, M, W, V, out, C, i, o, rmax, rarg, rlse,
                                                         None)


def test_noalloc_rejects_chunks_beyond_its_scratch(m):
    # 12 * ceil(V / 256) * C bytes of partials per chunk must fit the 32 MiB array
    V = 126464
    fits = m.MOSAIC_NOALLOC_SCRATCH_BYTES // (12 * 494)
    assert m.mosaic_logits_argmax_lse_workspace_bytes(fits, 0, V) <= m.MOSAIC_NOALLOC_SCRATCH_BYTES
    assert m.mosaic_logits_argmax_lse_workspace_bytes(fits + 1, 0, V) > m.MOSAIC_NOALLOC_SCRATCH_BYTES
    assert _noalloc(m, L=40000, d=4096, M=fits + 1, V=V) == 2              # one chunk too large
    assert _noalloc(m, L=40000, d=4096, M=29491, C=fits + 1, V=V) == 2     # chunks too large
    assert _noalloc(m, L=40000, d=4096, M=30000, C=6000, V=V) == 2


@pytest.mark.parametrize("kw,status", [
    (dict(M=-1), 1), (dict(V=0), 1), (dict(i=0), 2), (dict(d=72), 2), (dict(out=A16, o=0), 2),
    (dict(H=None), 1), (dict(W=None), 1), (dict(idx=None), 1), (dict(rmax=None), 1),
    (dict(H=A8), 1), (dict(rlse=A16 + 2), 1), (dict(L=2**31), 2),
])
def test_noalloc_validation(m, kw, status):
    assert _noalloc(m, **kw) == status


def test_noalloc_empty_is_ok_without_pointers(m):
    assert _noalloc(m, M=0, H=None, W=None, idx=None, rmax=None, rarg=None, rlse=None) == 0
