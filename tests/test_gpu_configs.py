"""GPU path on the named workloads at full size.

Compaction is compared with the oracle bit for bit.  Logits are compared with the
fp64 oracle on every element for the small workloads and on sampled rows (chunk and
tile boundaries plus seeded random rows) for the large ones, in the same launch
configuration the benchmark times (the workload's own chunk_rows).  Properties that
hold at any size are checked on every element: chunked == unchunked bit for bit, and
one-hot weights reproduce the gathered hidden-state columns exactly.
"""
import numpy as np
import pytest
import torch

import oracle
from mask_only_logits_amd import inputs
from tests.helpers import assert_close, bf16_rne, sample_rows

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module")
def m():
    from mask_only_logits_amd import mosaic
    return mosaic


def _step(m, wl, chunk_rows=None):
    """Compaction + count read-back + chunked logits, as the benchmark runs them."""
    tok = wl.tokens.to(DEV)
    H, W = wl.H.to(DEV), wl.W.to(DEV)
    if wl.seq_offsets is not None:
        idx, off = m.mosaic_mask_compact_batched(tok, wl.seq_offsets.to(DEV), wl.mask_id)
        M = int(off[-1].item())
    else:
        idx, cnt = m.mosaic_mask_compact(tok, wl.mask_id)
        M = int(cnt.item())
    C = wl.chunk_rows if chunk_rows is None else chunk_rows
    out = m.mosaic_masked_logits(H, idx, W, M=M, chunk_rows=C,
                                 out_dtype=torch.float32 if wl.out_dtype == "f32" else torch.bfloat16)
    torch.cuda.synchronize()
    return H, W, idx, M, out


def test_tiny_full(m):
    wl = inputs.make_workload("tiny")
    _, _, idx, M, out = _step(m, wl)
    want = oracle.mask_compact(wl.tokens, wl.mask_id)
    assert M == 128 and np.array_equal(idx[:M].cpu().numpy(), want)
    assert out.dtype == torch.float32
    assert_close(out, oracle.masked_logits(wl.H, want, wl.W), "tiny")


def test_lowm_full(m):
    wl = inputs.make_workload("lowm")
    _, _, idx, M, out = _step(m, wl)
    want = oracle.mask_compact(wl.tokens, wl.mask_id)
    assert M == 20 and np.array_equal(idx[:M].cpu().numpy(), want)
    assert_close(out, oracle.masked_logits(wl.H, want, wl.W), "lowm")


@pytest.mark.parametrize("name,n_random", [("llada_step", 16), ("long_logits", 8), ("long_ffn", 8)])
def test_large_sampled_and_chunk_bit_exact(m, name, n_random):
    wl = inputs.make_workload(name)
    H, W, idx, M, out = _step(m, wl)
    want = oracle.mask_compact(wl.tokens, wl.mask_id)
    assert M == want.size and np.array_equal(idx[:M].cpu().numpy(), want)
    rows = sample_rows(M, wl.chunk_rows, n_random, seed=M)
    ref = oracle.masked_logits(wl.H, want, wl.W, rows=rows)
    assert_close(out[torch.from_numpy(rows).to(DEV)], ref, f"{name} sampled rows")
    # chunked (the workload's max_num_logits, or a forced 1000-row chunking) == unchunked
    other = m.mosaic_masked_logits(H, idx, W, M=M, chunk_rows=0 if wl.chunk_rows else 1000)
    torch.cuda.synchronize()
    assert torch.equal(other, out)


def test_ragged_full_batch(m):
    wl = inputs.make_workload("ragged")
    H, W, idx, M, out = _step(m, wl)
    want_idx, want_off = oracle.mask_compact_batched(wl.tokens, wl.seq_offsets, wl.mask_id)
    assert M == want_off[-1] and np.array_equal(idx[:M].cpu().numpy(), want_idx)
    # each sequence's first and last masked row, rows around 256-row tile boundaries and
    # seeded random rows inside the sequences (CSR output order)
    rows = np.unique(np.concatenate([want_off[:-1], want_off[1:] - 1,
                                     sample_rows(M, 0, 24, seed=M)]).astype(np.int64))
    ref = oracle.masked_logits(wl.H, want_idx, wl.W, rows=rows)
    assert_close(out[torch.from_numpy(rows).to(DEV)], ref, "ragged sampled rows")
    other = m.mosaic_masked_logits(H, idx, W, M=M, chunk_rows=4096)
    torch.cuda.synchronize()
    assert torch.equal(other, out)


def _masked_rows(m, wl):
    tok = wl.tokens.to(DEV)
    if wl.seq_offsets is not None:
        idx, off = m.mosaic_mask_compact_batched(tok, wl.seq_offsets.to(DEV), wl.mask_id)
        return idx, int(off[-1].item())
    idx, cnt = m.mosaic_mask_compact(tok, wl.mask_id)
    return idx, int(cnt.item())


@pytest.mark.parametrize("name", ["long_logits", "long_ffn", "ragged", "llada_step"])
def test_one_hot_w_full_shape_bit_exact(m, name):
    # W[v, k] = [k == v mod d]: every logit is an exact copy of a gathered H element, so
    # every element of the full-size output pins the gather addressing bit for bit
    wl = inputs.make_workload(name)
    d, V = wl.d, wl.V
    W1 = inputs.one_hot_rows(V, d).to(DEV)
    idx, M = _masked_rows(m, wl)
    H = wl.H.to(DEV)
    out = m.mosaic_masked_logits(H, idx, W1, M=M, chunk_rows=wl.chunk_rows)
    cols = torch.arange(V, device=DEV) % d
    for r0 in range(0, M, 2048):
        r1 = min(M, r0 + 2048)
        want = H[idx[r0:r1].long()][:, cols]
        assert torch.equal(out[r0:r1], want), (name, r0)


@pytest.mark.parametrize("name", ["long_logits", "long_ffn", "ragged", "llada_step"])
def test_one_hot_h_full_shape_bit_exact(m, name):
    # H[p, k] = [k == p mod d]: row i of the output is column idx[i] mod d of W, exactly
    wl = inputs.make_workload(name)
    d, V = wl.d, wl.V
    idx, M = _masked_rows(m, wl)
    H1 = inputs.one_hot_rows(wl.L, d).to(DEV)
    W = wl.W.to(DEV)
    out = m.mosaic_masked_logits(H1, idx, W, M=M, chunk_rows=wl.chunk_rows)
    Wt = W.T.contiguous()                              # [d, V]: row k is column k of W
    for r0 in range(0, M, 2048):
        r1 = min(M, r0 + 2048)
        want = Wt[(idx[r0:r1].long() % d)]
        assert torch.equal(out[r0:r1], want), (name, r0)
    del Wt


def test_integer_inputs_full_shape_bit_exact(m):
    # integer-valued H, W in [-2, 2]: fp32 accumulation is exact, so bf16 outputs are the
    # unique RNE of the exact oracle value
    wl = inputs.make_workload("llada_step", with_weights=False)
    L, d, V = wl.L, wl.d, wl.V
    H = inputs.integer_valued(31, (L, d))
    W = inputs.integer_valued(32, (V, d))
    want = oracle.mask_compact(wl.tokens, wl.mask_id)
    idx = torch.from_numpy(want).to(DEV)
    out = m.mosaic_masked_logits(H.to(DEV), idx, W.to(DEV))
    torch.cuda.synchronize()
    rows = sample_rows(want.size, 0, 6, seed=5)
    ref = oracle.masked_logits(H, want, W, rows=rows)
    assert torch.equal(out[torch.from_numpy(rows).to(DEV)].cpu(), bf16_rne(ref))


@pytest.mark.parametrize("M", [33, 64])
def test_lowm_shape_two_row_blocks_every_element(m, M):
    # the low-M workload's H and W (d = 3584, V = 152064) with 33 and 64 masked rows: the
    # low-M kernel's two-row-block form across the full grid, bf16 and fp32 logits, every
    # element against the oracle
    wl = inputs.make_workload("lowm")
    idx = np.sort(np.random.default_rng(M).choice(wl.L, M, replace=False)).astype(np.int32)
    H, W, idx_d = wl.H.to(DEV), wl.W.to(DEV), torch.from_numpy(idx).to(DEV)
    assert m.mosaic_logits_variant(M, wl.V, wl.d, torch.bfloat16, torch.bfloat16) == 20
    out16 = m.mosaic_masked_logits(H, idx_d, W)
    out32 = m.mosaic_masked_logits(H, idx_d, W, out_dtype=torch.float32)
    torch.cuda.synchronize()
    ref = oracle.masked_logits(wl.H, idx, wl.W)
    assert_close(out16, ref, f"lowm shape M={M} bf16")
    assert_close(out32, ref, f"lowm shape M={M} fp32")


def test_chunk_tail_on_lowm_kernel_bit_exact(m):
    # 1200-row chunks of the LLaDA-shaped step leave a 29-row tail, which runs on the low-M
    # kernel while the first chunk runs on the tiled kernel: still bit-identical to the
    # unchunked call
    wl = inputs.make_workload("llada_step")
    H, W, idx, M, out = _step(m, wl)
    assert M == 1229 and m.mosaic_num_chunks(M, 1200) == 2
    assert m.mosaic_logits_variant(M - 1200, wl.V, wl.d, torch.bfloat16, torch.bfloat16) == 20
    chunked = m.mosaic_masked_logits(H, idx, W, M=M, chunk_rows=1200)
    torch.cuda.synchronize()
    assert torch.equal(chunked, out)
