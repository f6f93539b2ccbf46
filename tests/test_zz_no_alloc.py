"""The allocation-free consumer entry point against the workspace one, on the GPU.

mosaic_masked_logits_argmax_lse_noalloc keeps the per-row partials in the library's own
per-device array instead of a caller workspace; it runs the same kernels, so its row
maxima, first argmax, log-sum-exp and stored logits must equal those of
mosaic_masked_logits_argmax_lse bit for bit.  Two calls in a row, the second on a smaller
problem, so the second reuses the array the first left behind.
"""
import numpy as np
import pytest
import torch

from mask_only_logits_amd import inputs

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module")
def m():
    from mask_only_logits_amd import mosaic
    return mosaic


def _both(m, wl, M, chunk_rows, store):
    H, W = wl.H.to(DEV), wl.W.to(DEV)
    rng = np.random.default_rng(M)
    idx = torch.from_numpy(np.sort(rng.choice(wl.L, M, replace=False)).astype(np.int32)).to(DEV)
    V = wl.V
    ref = m.mosaic_masked_logits_argmax_lse(H, idx, W, M=M, chunk_rows=chunk_rows, store_logits=store)
    outs = [torch.full((M,), float("nan"), device=DEV), torch.full((M,), -7, dtype=torch.int32, device=DEV),
            torch.full((M,), float("nan"), device=DEV)]
    out = torch.zeros((M, V), dtype=torch.bfloat16, device=DEV) if store else None
    got = m.mosaic_masked_logits_argmax_lse_noalloc(H, idx, W, *outs, M=M, chunk_rows=chunk_rows, out=out)
    torch.cuda.synchronize()
    for name, a, b in zip(("row_max", "row_argmax", "row_lse"), got[:3], ref[:3]):
        assert torch.equal(a, b), name
    if store:
        assert torch.equal(got[3], ref[3])


def test_noalloc_matches_workspace_entry_point_two_calls(m):
    big = inputs.make_workload("llada_step")                      # d = 4096, V = 126464
    small = inputs.make_random(77, L=900, d=256, V=1000, M=300, dtype="bf16")
    _both(m, big, 1229, 500, store=True)                         # three chunks, logits stored too
    _both(m, small, 300, 0, store=False)                         # smaller, reuses the array


def test_noalloc_rejects_too_large_chunks(m):
    # 12 bytes per row and 256-entry vocabulary tile: at V = 126464 the array holds the
    # partials of 5660 rows per chunk; one more is refused before anything is enqueued
    V, d = 126464, 64
    fits = m.MOSAIC_NOALLOC_SCRATCH_BYTES // (12 * ((V + 255) // 256))
    M = fits + 1
    H = torch.zeros((M, d), dtype=torch.bfloat16, device=DEV)
    W = torch.zeros((V, d), dtype=torch.bfloat16, device=DEV)
    idx = torch.arange(M, dtype=torch.int32, device=DEV)
    o = [torch.empty(M, device=DEV), torch.empty(M, dtype=torch.int32, device=DEV), torch.empty(M, device=DEV)]
    with pytest.raises(m.MosaicError) as e:
        m.mosaic_masked_logits_argmax_lse_noalloc(H, idx, W, *o, M=M)
    assert e.value.status == m.MOSAIC_ERR_UNSUPPORTED
    # the same rows in chunks that fit run
    m.mosaic_masked_logits_argmax_lse_noalloc(H, idx, W, *o, M=M, chunk_rows=fits)
    torch.cuda.synchronize()
    assert bool((o[0] == 0).all()) and bool((o[1] == 0).all())
