"""MOSAIC_CHECK_IDX=1: the logits entry points check idx on the device first.

The out-of-range indices used here (-1 and L) address the rows just outside the H
view, which this test allocates as real rows of a larger buffer: even a check that
missed them would read valid memory, so the test can only fail an assertion.
"""
import numpy as np
import pytest
import torch

import oracle
from mask_only_logits_amd import inputs

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module")
def m():
    from mask_only_logits_amd import mosaic
    return mosaic


def _setup(seed, L=300, d=256, V=700, M=100):
    wl = inputs.make_random(seed, L=L, d=d, V=V, M=M, dtype="bf16")
    big = torch.zeros((L + 2, d), dtype=torch.bfloat16, device=DEV)
    big[1:L + 1] = wl.H.to(DEV)
    H = big[1:L + 1]                       # rows -1 and L of H are real memory
    idx = torch.from_numpy(oracle.mask_compact(wl.tokens, wl.mask_id)).to(DEV)
    return wl, H, idx, wl.W.to(DEV)


@pytest.mark.parametrize("bad", [-1, "L"])
def test_check_rejects_out_of_range(m, lib_env, bad):
    wl, H, idx, W = _setup(41)
    L, V, M = H.shape[0], W.shape[0], idx.numel()
    bad_idx = idx.clone()
    bad_idx[M // 2] = L if bad == "L" else -1
    lib_env("MOSAIC_CHECK_IDX", "1")
    out = torch.full((M, V), 3.0, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(m.MosaicError) as e:
        m.mosaic_masked_logits(H, bad_idx, W, out=out)
    assert e.value.status == m.MOSAIC_ERR_INVALID_ARG
    rmax = torch.full((M,), 7.0, device=DEV)
    with pytest.raises(m.MosaicError):
        m.mosaic_masked_logits_argmax_lse(H, bad_idx, W, row_max=rmax)
    Wq, ws = m.mosaic_quantize_rows_fp8(W)
    with pytest.raises(m.MosaicError):
        m.mosaic_masked_logits_fp8(H, bad_idx, Wq, ws, out=out)
    torch.cuda.synchronize()
    assert torch.all(out == 3.0) and torch.all(rmax == 7.0)


def test_check_passes_valid_indices(m, lib_env):
    wl, H, idx, W = _setup(42)
    ref = m.mosaic_masked_logits(H, idx, W)
    ref_c = m.mosaic_masked_logits_argmax_lse(H, idx, W)
    lib_env("MOSAIC_CHECK_IDX", "1")
    got = m.mosaic_masked_logits(H, idx, W, chunk_rows=33)
    got_c = m.mosaic_masked_logits_argmax_lse(H, idx, W)
    torch.cuda.synchronize()
    assert torch.equal(got, ref)
    for x, y in zip(got_c[:3], ref_c[:3]):
        assert torch.equal(x, y)
