"""GPU FP8 (OCP E4M3) LM head vs the CPU oracle.

Quantization decides integers (the codes) from fp32 arithmetic, and both sides take
those decisions in the same fp32 operations (amax, 448 / amax, x * inv, round to
nearest even), so codes and scales are compared bit for bit.  The logits are the fp8
MFMA's fp32 sum of code products times both row scales, rounded to bf16; the oracle
sums the same products exactly in fp64.  The fp8 MFMA adds its partial products with
an error of order 1e-5 of the largest partial sum (measured), far below the bf16
output rounding, so the bf16 bar |g - o| <= 1e-2 * max(1, |o|) applies.
"""
import numpy as np
import pytest
import torch

import oracle
from mask_only_logits_amd import inputs
from tests.helpers import assert_close, sample_rows

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module")
def m():
    from mask_only_logits_amd import mosaic
    return mosaic


@pytest.mark.parametrize("dtype,n,d", [("bf16", 1000, 512), ("f32", 300, 136), ("bf16", 7, 4096), ("bf16", 64, 8)])
def test_quantize_bit_exact(m, dtype, n, d):
    X = inputs.make_random(n + d, L=n, d=d, V=4, M=1, dtype=dtype).H.clone()
    X[min(3, n - 1)] = 0
    if n > 10:
        X[5, 7] = 1e-30 if dtype == "f32" else X[5, 7]       # tiny values next to large ones
    q, sc = m.mosaic_quantize_rows_fp8(X.to(DEV))
    torch.cuda.synchronize()
    oq, osc = oracle.quantize_rows_e4m3(X)
    assert np.array_equal(q.cpu().numpy(), oq)
    assert np.array_equal(sc.cpu().numpy().view(np.uint32), osc.view(np.uint32))
    # gathered rows
    ridx = np.random.default_rng(n).integers(0, n, size=min(n, 50)).astype(np.int32)
    q2, sc2 = m.mosaic_quantize_rows_fp8(X.to(DEV), row_idx=torch.from_numpy(ridx).to(DEV))
    torch.cuda.synchronize()
    assert np.array_equal(q2.cpu().numpy(), oq[ridx]) and np.array_equal(sc2.cpu().numpy(), osc[ridx])


CASES = [
    # (L, d, V, M, chunk_rows)
    (700, 512, 1000, 600, 0),
    (700, 512, 1000, 600, 256),
    (400, 128, 1001, 257, 0),     # one K tile, V % 4 != 0
    (400, 256, 257, 256, 0),
    (300, 384, 3, 1, 0),          # a single row, odd K-tile count
    (900, 3584, 700, 513, 200),
]


@pytest.mark.parametrize("L,d,V,M,C", CASES)
def test_parity_random(m, L, d, V, M, C):
    wl = inputs.make_random(L * 3 + d + V + M, L=L, d=d, V=V, M=M, dtype="bf16")
    idx = oracle.mask_compact(wl.tokens, wl.mask_id)
    Wq, ws = m.mosaic_quantize_rows_fp8(wl.W.to(DEV))
    out = m.mosaic_masked_logits_fp8(wl.H.to(DEV), torch.from_numpy(idx).to(DEV), Wq, ws, chunk_rows=C)
    torch.cuda.synchronize()
    ref = oracle.masked_logits_fp8(wl.H, idx, wl.W)
    assert_close(out, ref, f"fp8 {L},{d},{V},{M},{C}")


@pytest.mark.parametrize("d", [128, 256, 384, 1024])   # 1, 2, 3 and 8 K tiles
def test_chunked_waves_and_determinism(m, lib_env, d):
    wl = inputs.make_random(55 + d, L=1500, d=d, V=2000, M=1100, dtype="bf16")
    idx_d = torch.from_numpy(oracle.mask_compact(wl.tokens, wl.mask_id)).to(DEV)
    H = wl.H.to(DEV)
    Wq, ws = m.mosaic_quantize_rows_fp8(wl.W.to(DEV))
    ref = m.mosaic_masked_logits_fp8(H, idx_d, Wq, ws)
    for C in (1, 64, 255, 256, 300, 1099, -1):
        assert torch.equal(m.mosaic_masked_logits_fp8(H, idx_d, Wq, ws, chunk_rows=C), ref), C
    for tune in ("waves=4", "waves=8"):   # the comparison forms; the default is the three-stage one
        lib_env("MOSAIC_TUNE", tune)
        assert torch.equal(m.mosaic_masked_logits_fp8(H, idx_d, Wq, ws), ref), tune
        assert torch.equal(m.mosaic_masked_logits_fp8(H, idx_d, Wq, ws, chunk_rows=300), ref), tune
    lib_env("MOSAIC_TUNE", None)
    torch.cuda.synchronize()


def test_close_to_bf16_logits(m):
    wl = inputs.make_random(56, L=600, d=1024, V=3000, M=400, dtype="bf16")
    idx = oracle.mask_compact(wl.tokens, wl.mask_id)
    idx_d = torch.from_numpy(idx).to(DEV)
    H, W = wl.H.to(DEV), wl.W.to(DEV)
    Wq, ws = m.mosaic_quantize_rows_fp8(W)
    f8 = m.mosaic_masked_logits_fp8(H, idx_d, Wq, ws).float()
    b16 = m.mosaic_masked_logits(H, idx_d, W, out_dtype=torch.float32)
    torch.cuda.synchronize()
    rel = ((f8 - b16).abs().max() / b16.abs().max()).item()
    assert 1e-4 < rel < 0.05, rel


def test_headline_shape_sampled_rows(m):
    # LLaDA-shaped LM head (V = 126464, d = 4096) on the logits-dominant workload's
    # masked rows, in its 4096-row chunks
    wl = inputs.make_workload("long_logits")
    idx = oracle.mask_compact(wl.tokens, wl.mask_id)
    Wq, ws = m.mosaic_quantize_rows_fp8(wl.W.to(DEV))
    out = m.mosaic_masked_logits_fp8(wl.H.to(DEV), torch.from_numpy(idx).to(DEV), Wq, ws,
                                     chunk_rows=wl.chunk_rows)
    torch.cuda.synchronize()
    rows = sample_rows(idx.size, wl.chunk_rows, 4, seed=11)
    rows = rows[np.linspace(0, rows.size - 1, 10).astype(int)]
    qh, sh = oracle.quantize_rows_e4m3(wl.H, idx)
    qw, sw = oracle.quantize_rows_e4m3(wl.W)
    # the device-quantized W equals the oracle's on every code
    assert np.array_equal(Wq.cpu().numpy(), qw) and np.array_equal(ws.cpu().numpy(), sw)
    ref = oracle.logits_fp8(qh, sh, qw, sw, rows=rows)
    assert_close(out[torch.from_numpy(rows).to(DEV)], ref, "fp8 long_logits sampled rows")


@pytest.mark.parametrize("name", ["llada_step", "ragged"])
def test_other_workloads_sampled_rows(m, name):
    # the LLaDA step (one 1229-row chunk) and the Dream-shaped ragged batch (d = 3584,
    # V = 152064, one 21399-row launch in CSR order) through the FP8 LM head
    wl = inputs.make_workload(name)
    if wl.seq_offsets is not None:
        idx = oracle.mask_compact_batched(wl.tokens, wl.seq_offsets, wl.mask_id)[0]
    else:
        idx = oracle.mask_compact(wl.tokens, wl.mask_id)
    Wq, ws = m.mosaic_quantize_rows_fp8(wl.W.to(DEV))
    out = m.mosaic_masked_logits_fp8(wl.H.to(DEV), torch.from_numpy(idx).to(DEV), Wq, ws,
                                     chunk_rows=wl.chunk_rows)
    torch.cuda.synchronize()
    rows = sample_rows(idx.size, wl.chunk_rows, 4, seed=13)
    rows = rows[np.linspace(0, rows.size - 1, min(rows.size, 10)).astype(int)]
    qh, sh = oracle.quantize_rows_e4m3(wl.H, idx)
    qw, sw = oracle.quantize_rows_e4m3(wl.W)
    ref = oracle.logits_fp8(qh, sh, qw, sw, rows=rows)
    assert_close(out[torch.from_numpy(rows).to(DEV)], ref, f"fp8 {name} sampled rows")


@pytest.mark.parametrize("name", ["long_logits", "ragged", "llada_step"])
def test_one_hot_w_full_shape_bit_exact(m, name):
    # W[v] = 448 e_(v mod d): each W row quantizes to the single code of 448 with row scale
    # exactly 1, so each logit is one exact product, value(Hq[i, v mod d]) * 448, times the
    # H row's scale in fp32 and rounded to bf16.  Every element of the full-size output is
    # then fixed by the oracle's quantization of the gathered H rows.
    wl = inputs.make_workload(name)
    d, V = wl.d, wl.V
    if wl.seq_offsets is not None:
        idx = oracle.mask_compact_batched(wl.tokens, wl.seq_offsets, wl.mask_id)[0]
    else:
        idx = oracle.mask_compact(wl.tokens, wl.mask_id)
    M = idx.size
    W1 = (inputs.one_hot_rows(V, d, dtype="f32") * 448.0).to(torch.bfloat16)
    Wq, ws = m.mosaic_quantize_rows_fp8(W1.to(DEV))
    code448 = oracle.e4m3_encode(448.0)
    cols = torch.arange(V, device=DEV) % d
    want_q = torch.zeros((V, d), dtype=torch.uint8, device=DEV)
    want_q[torch.arange(V, device=DEV), cols] = code448
    assert torch.equal(Wq, want_q) and torch.all(ws == 1.0)
    del want_q, W1
    out = m.mosaic_masked_logits_fp8(wl.H.to(DEV), torch.from_numpy(idx).to(DEV), Wq, ws,
                                     chunk_rows=wl.chunk_rows)
    torch.cuda.synchronize()
    qh, sh = oracle.quantize_rows_e4m3(wl.H, idx)
    lut = torch.tensor([oracle.e4m3_value(c) for c in range(256)], dtype=torch.float32)
    T = ((lut[torch.from_numpy(qh).long()] * 448.0) * torch.from_numpy(sh)[:, None]).to(torch.bfloat16).to(DEV)
    for r0 in range(0, M, 2048):
        r1 = min(M, r0 + 2048)
        assert torch.equal(out[r0:r1], T[r0:r1][:, cols]), (name, r0)


@pytest.mark.parametrize("name", ["long_logits", "ragged"])
def test_one_hot_h_full_shape_bit_exact(m, name):
    # H[p] = e_(p mod d): each gathered H row quantizes to the code of 448 at column
    # idx[i] mod d with the oracle's row scale s_h, so logit (i, v) is one exact product,
    # value(Wq[v, idx[i] mod d]) * 448, times (s_h * s_w[v]) in fp32 (the kernel's order),
    # rounded to bf16.  Every element of the full-size output is then fixed by the oracle's
    # quantization of W.
    wl = inputs.make_workload(name)
    d, V = wl.d, wl.V
    if wl.seq_offsets is not None:
        idx = oracle.mask_compact_batched(wl.tokens, wl.seq_offsets, wl.mask_id)[0]
    else:
        idx = oracle.mask_compact(wl.tokens, wl.mask_id)
    M = idx.size
    H1 = inputs.one_hot_rows(wl.L, d)
    qh, sh = oracle.quantize_rows_e4m3(H1, idx)
    code448 = oracle.e4m3_encode(448.0)
    assert np.all(qh[np.arange(M), idx % d] == code448) and np.count_nonzero(qh) == M
    assert np.all(sh == sh[0])
    Wq, ws = m.mosaic_quantize_rows_fp8(wl.W.to(DEV))
    qw, sw = oracle.quantize_rows_e4m3(wl.W)
    assert np.array_equal(Wq.cpu().numpy(), qw) and np.array_equal(ws.cpu().numpy(), sw)
    out = m.mosaic_masked_logits_fp8(H1.to(DEV), torch.from_numpy(idx).to(DEV), Wq, ws,
                                     chunk_rows=wl.chunk_rows)
    torch.cuda.synchronize()
    lut = torch.tensor([oracle.e4m3_value(c) for c in range(256)], dtype=torch.float32, device=DEV)
    Wt = (lut[Wq.long()] * 448.0).T.contiguous()                      # [d, V], exact
    hw = (torch.from_numpy(sh[:1]) * torch.from_numpy(sw)).to(DEV)    # s_h * s_w[v] in fp32
    kcol = torch.from_numpy(idx % d).to(DEV).long()
    for r0 in range(0, M, 2048):
        r1 = min(M, r0 + 2048)
        want = (Wt[kcol[r0:r1]] * hw[None, :]).to(torch.bfloat16)
        assert torch.equal(out[r0:r1], want), (name, r0)


def test_dream_shape_low_m_all_rows(m):
    # the low-M workload (Dream-shaped LM head: d = 3584, V = 152064; M = 20), every row
    wl = inputs.make_workload("lowm")
    idx = oracle.mask_compact(wl.tokens, wl.mask_id)
    Wq, ws = m.mosaic_quantize_rows_fp8(wl.W.to(DEV))
    out = m.mosaic_masked_logits_fp8(wl.H.to(DEV), torch.from_numpy(idx).to(DEV), Wq, ws)
    torch.cuda.synchronize()
    assert_close(out, oracle.masked_logits_fp8(wl.H, idx, wl.W), "fp8 lowm")


LOWM_CASES = [
    # (L, d, V, M): chunks of at most 64 rows take the W-streaming FP8 kernel
    (300, 128, 1001, 20), (300, 256, 3, 1), (300, 384, 4097, 33), (300, 3584, 5000, 64),
    # several blocks per wave: padding blocks (1024 waves own 128 or 129 rows), two store bursts
    (300, 256, 131584, 40), (300, 128, 300000, 20),
]


@pytest.mark.parametrize("L,d,V,M", LOWM_CASES)
def test_lowm_kernel_parity_and_bit_identity(m, lib_env, L, d, V, M):
    wl = inputs.make_random(L + 7 * d + V + M, L=L, d=d, V=V, M=M, dtype="bf16")
    idx = oracle.mask_compact(wl.tokens, wl.mask_id)
    H, idx_d = wl.H.to(DEV), torch.from_numpy(idx).to(DEV)
    Wq, ws = m.mosaic_quantize_rows_fp8(wl.W.to(DEV))
    out = m.mosaic_masked_logits_fp8(H, idx_d, Wq, ws)
    lib_env("MOSAIC_TUNE", "fp8lowm=0")          # the tiled FP8 kernel
    tiled = m.mosaic_masked_logits_fp8(H, idx_d, Wq, ws)
    torch.cuda.synchronize()
    assert torch.equal(out, tiled)
    assert_close(out, oracle.masked_logits_fp8(wl.H, idx, wl.W), f"fp8 lowm {d},{V},{M}")
