"""GPU per-row consumer (row max, first argmax, log-sum-exp) vs the CPU oracle.

Tolerances.  The kernel reduces the fp32 accumulators, which differ from the fp64
oracle logits by the fp32 accumulation error; the fp32 logits bound is
|z_gpu - z| <= 1e-4 * max(1, |z|).  The max of a row moves by at most the largest
element error and log-sum-exp is 1-Lipschitz in the max norm, so both are held to the
same bound (the exp2/log2 hardware approximations add ~1e-6 relative).  The argmax is
an integer decided in fp32: several indices are correct when logits lie within the
error bound of the maximum, so the test checks that the oracle's logit at the GPU's
index is within twice the bound of the oracle's maximum.  Exact pins (integer inputs,
zero and one-hot weights) are compared bit for bit.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from mask_only_logits_amd import inputs
from tests.helpers import sample_rows

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
TOL = 1e-4


@pytest.fixture(scope="module")
def m():
    from mask_only_logits_amd import mosaic
    return mosaic


def _idx(wl):
    idx = oracle.mask_compact(wl.tokens, wl.mask_id)
    return idx, torch.from_numpy(idx).to(DEV)


def _check(got, H, idx, W, rows=None, what=""):
    gmax, garg, glse = (t.cpu().numpy() for t in got[:3])
    r = np.arange(idx.size) if rows is None else rows
    omax, oarg, olse = oracle.masked_logits_argmax_lse(H, idx, W, rows=r)
    gmax, garg, glse = gmax[r].astype(np.float64), garg[r].astype(np.int64), glse[r].astype(np.float64)
    tol_max = TOL * np.maximum(1.0, np.abs(omax))
    assert np.all(np.abs(gmax - omax) <= tol_max), f"{what}: row max {np.abs(gmax - omax).max():.3e}"
    tol_lse = TOL * np.maximum(1.0, np.abs(olse))
    assert np.all(np.abs(glse - olse) <= tol_lse), f"{what}: lse {np.abs(glse - olse).max():.3e}"
    V = W.shape[0]
    assert np.all((garg >= 0) & (garg < V)), what
    z = oracle.masked_logits(H, idx, W, rows=r)
    zat = z[np.arange(r.size), garg]
    assert np.all(zat >= omax - 2 * tol_max), f"{what}: argmax not within the error bound of the max"
    return int((garg != oarg).sum())


CASES = [
    # (L, d, V, M, chunk_rows)
    (700, 512, 1000, 600, 0),
    (700, 512, 1000, 600, 256),
    (900, 3584, 700, 513, 200),
    (400, 64, 1001, 257, 0),     # one K tile
    (400, 128, 257, 256, 0),     # the last vocabulary tile holds one entry
    (300, 192, 3, 1, 0),         # a single row, tiny vocabulary
    (300, 256, 4097, 70, 33),
    (2000, 4096, 1500, 300, 0),
]


@pytest.mark.parametrize("L,d,V,M,C", CASES)
def test_parity_random(m, L, d, V, M, C):
    wl = inputs.make_random(L * 13 + d + V + M, L=L, d=d, V=V, M=M, dtype="bf16")
    idx, idx_d = _idx(wl)
    H, W = wl.H.to(DEV), wl.W.to(DEV)
    got = m.mosaic_masked_logits_argmax_lse(H, idx_d, W, chunk_rows=C)
    torch.cuda.synchronize()
    assert got[3] is None
    _check(got, wl.H, idx, wl.W, what=f"{L},{d},{V},{M},{C}")


@pytest.mark.parametrize("d,V,M", [(4096, 1000, 300), (512, 1001, 600), (64, 100, 50)])
def test_exact_integers(m, d, V, M):
    L = M + 50
    H = inputs.integer_valued(d + 5, (L, d))
    W = inputs.integer_valued(d + 6, (V, d))
    idx = np.sort(np.random.default_rng(d).choice(L, M, replace=False)).astype(np.int32)
    got = m.mosaic_masked_logits_argmax_lse(H.to(DEV), torch.from_numpy(idx).to(DEV), W.to(DEV))
    torch.cuda.synchronize()
    omax, oarg, olse = oracle.masked_logits_argmax_lse(H, idx, W)
    assert np.array_equal(got[0].cpu().numpy().astype(np.float64), omax)
    assert np.array_equal(got[1].cpu().numpy().astype(np.int64), oarg)
    np.testing.assert_allclose(got[2].cpu().numpy(), olse, rtol=1e-5, atol=1e-5)


def test_zero_weights(m):
    L, d, V, M = 300, 128, 5000, 100
    wl = inputs.make_random(77, L=L, d=d, V=V, M=M, dtype="bf16")
    _, idx_d = _idx(wl)
    W0 = torch.zeros((V, d), dtype=torch.bfloat16, device=DEV)
    mx, am, lse, _ = m.mosaic_masked_logits_argmax_lse(wl.H.to(DEV), idx_d, W0)
    torch.cuda.synchronize()
    assert torch.all(mx == 0) and torch.all(am == 0)
    np.testing.assert_allclose(lse.cpu().numpy(), math.log(V), rtol=0, atol=1e-5)


@pytest.mark.parametrize("d,V", [(64, 700), (256, 300), (128, 128)])
def test_one_hot_weights(m, d, V):
    L, M = 400, 150
    wl = inputs.make_random(d + V, L=L, d=d, V=V, M=M, dtype="bf16")
    idx, idx_d = _idx(wl)
    W1 = inputs.one_hot_rows(V, d)
    mx, am, _, _ = m.mosaic_masked_logits_argmax_lse(wl.H.to(DEV), idx_d, W1.to(DEV))
    torch.cuda.synchronize()
    h = wl.H.float().numpy()[idx][:, :min(d, V)]
    assert np.array_equal(mx.cpu().numpy(), h.max(axis=1))
    assert np.array_equal(am.cpu().numpy(), h.argmax(axis=1))     # first occurrence


def test_stored_logits_and_store_free_agree(m):
    wl = inputs.make_random(31, L=1200, d=512, V=3000, M=900, dtype="bf16")
    _, idx_d = _idx(wl)
    H, W = wl.H.to(DEV), wl.W.to(DEV)
    ref_logits = m.mosaic_masked_logits(H, idx_d, W, out_dtype=torch.bfloat16)
    a = m.mosaic_masked_logits_argmax_lse(H, idx_d, W)
    b = m.mosaic_masked_logits_argmax_lse(H, idx_d, W, store_logits=True)
    torch.cuda.synchronize()
    assert torch.equal(b[3], ref_logits)
    for x, y in zip(a[:3], b[:3]):
        assert torch.equal(x, y)


def test_chunked_equals_unchunked_and_deterministic(m):
    wl = inputs.make_random(32, L=1500, d=256, V=2000, M=1100, dtype="bf16")
    _, idx_d = _idx(wl)
    H, W = wl.H.to(DEV), wl.W.to(DEV)
    ref = m.mosaic_masked_logits_argmax_lse(H, idx_d, W)
    for C in (1, 64, 255, 256, 300, 1099, 1100, -1, 0):
        got = m.mosaic_masked_logits_argmax_lse(H, idx_d, W, chunk_rows=C)
        for x, y in zip(got[:3], ref[:3]):
            assert torch.equal(x, y), C
    torch.cuda.synchronize()


def test_rejected_call_leaves_outputs_untouched(m):
    wl = inputs.make_random(33, L=300, d=128, V=500, M=100, dtype="bf16")
    _, idx_d = _idx(wl)
    H, W = wl.H.to(DEV), wl.W.to(DEV)
    rmax = torch.full((100,), 7.0, device=DEV)
    small = torch.empty(16, dtype=torch.uint8, device=DEV)
    with pytest.raises(m.MosaicError):
        m.mosaic_masked_logits_argmax_lse(H, idx_d, W, row_max=rmax, workspace=small)
    torch.cuda.synchronize()
    assert torch.all(rmax == 7.0)


def test_headline_shape_sampled_rows(m):
    # the logits-dominant workload (L = 32768, d = 4096, V = 126464, 90% masked) in its
    # own 4096-row chunks, without storing the logits
    wl = inputs.make_workload("long_logits")
    idx, idx_d = _idx(wl)
    H, W = wl.H.to(DEV), wl.W.to(DEV)
    got = m.mosaic_masked_logits_argmax_lse(H, idx_d, W, chunk_rows=wl.chunk_rows)
    torch.cuda.synchronize()
    rows = sample_rows(idx.size, wl.chunk_rows, 4, seed=7)
    rows = rows[np.linspace(0, rows.size - 1, 12).astype(int)]
    _check(got, wl.H, idx, wl.W, rows=rows, what="long_logits")
    # the same rows through the unchunked call: identical bits
    again = m.mosaic_masked_logits_argmax_lse(H, idx_d, W)
    torch.cuda.synchronize()
    for x, y in zip(got[:3], again[:3]):
        assert torch.equal(x, y)


@pytest.mark.parametrize("name", ["ragged", "lowm", "llada_step", "long_ffn"])
def test_other_workloads_sampled_rows(m, name):
    # Dream-shaped (d = 3584, V = 152064) ragged batch and low-M case, the LLaDA step, and
    # the FFN-dominant workload in its 8192-row chunks
    wl = inputs.make_workload(name)
    if wl.seq_offsets is not None:
        idx = oracle.mask_compact_batched(wl.tokens, wl.seq_offsets, wl.mask_id)[0]
    else:
        idx = oracle.mask_compact(wl.tokens, wl.mask_id)
    idx_d = torch.from_numpy(idx).to(DEV)
    got = m.mosaic_masked_logits_argmax_lse(wl.H.to(DEV), idx_d, wl.W.to(DEV), chunk_rows=wl.chunk_rows)
    torch.cuda.synchronize()
    rows = sample_rows(idx.size, wl.chunk_rows, 4, seed=3)
    rows = rows[np.linspace(0, rows.size - 1, min(rows.size, 10)).astype(int)]
    _check(got, wl.H, idx, wl.W, rows=rows, what=name)


@pytest.mark.parametrize("name", ["long_logits", "ragged"])
def test_one_hot_w_full_shape(m, name):
    # W[v] = e_(v mod d) at full size, logits not stored: row i's logits are the gathered
    # H[idx[i], v mod d], exact in fp32, so its max is the gathered row's largest element
    # and its argmax the first column k attaining it (column k first appears at v = k), both
    # bit for bit on every row; its lse is log(sum_k c_k exp(H[idx[i], k])) with c_k the
    # number of v < V with v mod d == k, held to the bound above
    wl = inputs.make_workload(name)
    d, V = wl.d, wl.V
    if wl.seq_offsets is not None:
        idx = oracle.mask_compact_batched(wl.tokens, wl.seq_offsets, wl.mask_id)[0]
    else:
        idx = oracle.mask_compact(wl.tokens, wl.mask_id)
    W1 = inputs.one_hot_rows(V, d).to(DEV)
    mx, am, lse, _ = m.mosaic_masked_logits_argmax_lse(wl.H.to(DEV), torch.from_numpy(idx).to(DEV), W1,
                                                        chunk_rows=wl.chunk_rows)
    torch.cuda.synchronize()
    h = wl.H[torch.from_numpy(idx).long()].float().numpy()             # [M, d], exact
    assert np.array_equal(mx.cpu().numpy(), h.max(axis=1))
    assert np.array_equal(am.cpu().numpy(), h.argmax(axis=1))         # first occurrence
    c = np.full(d, V // d, dtype=np.float64) + (np.arange(d) < V % d)
    hd = h.astype(np.float64)
    top = hd.max(axis=1)
    want = top + np.log((np.exp(hd - top[:, None]) * c).sum(axis=1))
    got = lse.cpu().numpy().astype(np.float64)
    assert np.all(np.abs(got - want) <= TOL * np.maximum(1.0, np.abs(want))), np.abs(got - want).max()


@pytest.mark.parametrize("L,d,V,M,C", [CASES[0], CASES[2], CASES[4], CASES[6]])
def test_mfma_forms_match(m, lib_env, L, d, V, M, C):
    # the 32 x 32 x 16 MFMA form of the fused kernel (variant=16) against the default
    # 16 x 16 x 32 form: same fp32 logits, so the row max, argmax and stored logits are
    # identical; the exp sums are added in another order (oracle bound only)
    wl = inputs.make_random(L * 7 + d + V + M, L=L, d=d, V=V, M=M, dtype="bf16")
    idx, idx_d = _idx(wl)
    H, W = wl.H.to(DEV), wl.W.to(DEV)
    got = m.mosaic_masked_logits_argmax_lse(H, idx_d, W, chunk_rows=C, store_logits=True)
    only = m.mosaic_masked_logits_argmax_lse(H, idx_d, W, chunk_rows=C)
    lib_env("MOSAIC_TUNE", "variant=16")
    ref = m.mosaic_masked_logits_argmax_lse(H, idx_d, W, chunk_rows=C, store_logits=True)
    torch.cuda.synchronize()
    lib_env("MOSAIC_TUNE", None)
    assert torch.equal(got[0], ref[0]) and torch.equal(got[1], ref[1])
    assert torch.equal(got[3], ref[3])
    for x, y in zip(only[:3], got[:3]):
        assert torch.equal(x, y)
    _check(got, wl.H, idx, wl.W, what=f"{L},{d},{V},{M},{C}")
    _check(ref, wl.H, idx, wl.W, what=f"32x32 form {L},{d},{V},{M},{C}")
