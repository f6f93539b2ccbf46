"""GPU checks of the two workloads built on top of the path.

Dense vs mask-only: the mask-only logits are the masked rows of the dense logits (the
Mosaic review, 核心观察 #2, and the abstract's "exact model outputs").  At the
LLaDA-shaped step (L = 2048, d = 4096, V = 126464) with every position masked (mask
ratio 1.0) the path computes the dense product itself: it is compared with the oracle on
sampled rows, with a float32 library GEMM on every element, and with one-hot weights bit
for bit.  The dense-then-select baseline (all L rows, then the masked rows picked) gives
the same bits as the mask-only call, row by row.

Lazy chunk choice (the Mosaic paper page, §2.3: the minimal sufficient chunk count under a
memory limit): the chunk_rows that mosaic_lazy_chunk_rows picks for the headline workload
drives the kernel, and the result is bit-identical to the unchunked call and within the
bf16 bar of the oracle at the chunk boundaries.
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


@pytest.fixture(scope="module")
def llada():
    return inputs.make_workload("llada_step")


def test_mask_ratio_one_is_the_dense_product(m, llada):
    wl = llada
    L, V = wl.L, wl.V
    H, W = wl.H.to(DEV), wl.W.to(DEV)
    all_rows = np.arange(L, dtype=np.int32)
    out = m.mosaic_masked_logits(H, torch.from_numpy(all_rows).to(DEV), W)
    torch.cuda.synchronize()
    assert out.shape == (L, V)
    rows = sample_rows(L, 0, 16, seed=11)
    assert_close(out[torch.from_numpy(rows).to(DEV)], oracle.masked_logits(wl.H, all_rows, wl.W, rows=rows),
                 "ratio 1.0 sampled rows")
    # every element against a float32 library GEMM of the same bf16 inputs (a second,
    # independent product; its own fp32 rounding is far inside the bf16 bar)
    Wf = W.float()
    for r0 in range(0, L, 512):
        ref = (H[r0:r0 + 512].float() @ Wf.T).double()
        err = (out[r0:r0 + 512].double() - ref).abs() / ref.abs().clamp(min=1.0)
        assert float(err.max()) <= 1e-2, (r0, float(err.max()))
    del Wf


def test_mask_ratio_one_one_hot_every_element(m, llada):
    wl = llada
    L, d, V = wl.L, wl.d, wl.V
    H = wl.H.to(DEV)
    W1 = inputs.one_hot_rows(V, d).to(DEV)
    out = m.mosaic_masked_logits(H, torch.arange(L, dtype=torch.int32, device=DEV), W1)
    torch.cuda.synchronize()
    assert torch.equal(out, H[:, torch.arange(V, device=DEV) % d])


def test_dense_select_rows_equal_mask_only_rows(m, llada):
    # what bench.py's dense_select path does, against the mask-only call: same bits per row
    wl = llada
    H, W = wl.H.to(DEV), wl.W.to(DEV)
    want = oracle.mask_compact(wl.tokens, wl.mask_id)
    idx = torch.from_numpy(want).to(DEV)
    mask_only = m.mosaic_masked_logits(H, idx, W)
    dense = m.mosaic_masked_logits(H, torch.arange(wl.L, dtype=torch.int32, device=DEV), W)
    selected = torch.index_select(dense, 0, idx.long())
    torch.cuda.synchronize()
    assert torch.equal(selected, mask_only)
    # and the same with the dense product chunked the way the workloads chunk it
    dense_c = m.mosaic_masked_logits(H, torch.arange(wl.L, dtype=torch.int32, device=DEV), W, chunk_rows=700)
    torch.cuda.synchronize()
    assert torch.equal(dense_c, dense)


def test_mask_ratio_zero_is_no_work(m, llada):
    wl = llada
    H, W = wl.H.to(DEV), wl.W.to(DEV)
    poison = torch.full((4, wl.V), 7.0, dtype=torch.bfloat16, device=DEV)
    m.mosaic_masked_logits(H, torch.zeros(0, dtype=torch.int32, device=DEV), W, M=0, out=poison)
    torch.cuda.synchronize()
    assert bool((poison == 7.0).all())


@pytest.fixture(scope="module")
def headline(m):
    wl = inputs.make_workload("long_logits")
    tok = wl.tokens.to(DEV)
    idx, cnt = m.mosaic_mask_compact(tok, wl.mask_id)
    M = int(cnt.item())
    H, W = wl.H.to(DEV), wl.W.to(DEV)
    base = m.mosaic_masked_logits(H, idx, W, M=M)      # unchunked
    torch.cuda.synchronize()
    yield wl, H, W, idx, M, base
    del base


@pytest.mark.parametrize("budget_rows,want", [(4096, (3687, 8)), (7373, (7373, 4)), (29491, (0, 1))])
def test_lazy_chunk_rows_drive_the_kernel(m, headline, budget_rows, want):
    wl, H, W, idx, M, base = headline
    budget = budget_rows * wl.V * 2               # bytes of budget_rows bf16 logits rows
    C, k = m.mosaic_lazy_chunk_rows(M, wl.V, torch.bfloat16, budget)
    assert (C, k) == want
    assert m.mosaic_num_chunks(M, C) == k
    out = m.mosaic_masked_logits(H, idx, W, M=M, chunk_rows=C)
    torch.cuda.synchronize()
    assert torch.equal(out, base)
    # every chunk fits the budget, and the rows at the chunk boundaries match the oracle
    assert (C if C else M) * wl.V * 2 <= budget
    want_idx = idx[:M].cpu().numpy()
    edges = [b + o for b in range(C, M, C) for o in (-1, 0)] if C else []
    rows = np.unique(np.array([0, M - 1] + edges + [int(r) for r in np.random.default_rng(C).choice(M, 4)],
                              dtype=np.int64))
    assert_close(out[torch.from_numpy(rows).to(DEV)], oracle.masked_logits(wl.H, want_idx, wl.W, rows=rows),
                 f"lazy chunks C={C}")
