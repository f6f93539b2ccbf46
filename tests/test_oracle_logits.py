"""Pins of the oracle's mask-only logits (row i = H[idx[i], :] . W^T, fp64).

Each pin is independent of the oracle's own loop:
- dense-then-select: numpy's fp64 BLAS product H @ W^T over all rows, then the
  masked rows picked out (the mask-only rows equal the dense logits' rows --
  "Mosaic: Unlocking Long-Context Inference for Diffusion LLMs via Global Memory"
  review, 核心观察 #2, and the Mosaic abstract's exact-outputs statement);
- mask ratio 1.0 is the dense GEMM itself;
- exact integers: H, W with small integer entries give exact integer logits, which
  numpy's int64 product reproduces bit for bit (catches dropped or extra terms and
  sign errors);
- one-hot weights: W[v, k] = [k == v mod d] gives out[i, v] = H[idx[i], v mod d]
  exactly (catches transposed operands and wrong gather indices); one-hot H rows
  give columns of W;
- math.fsum (an exactly rounded sum) bounds the accumulation error of each element
  by d * 2^-53 * sum |terms| (catches accumulating in a narrower type);
- permutation and power-of-two scaling invariants.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from mask_only_logits_amd import inputs


def _dense_select(H, idx, W):
    h = H.to(torch.float64).numpy()
    w = W.to(torch.float64).numpy()
    return (h @ w.T)[idx]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("L,d,V,M", [(64, 32, 48, 30), (300, 136, 257, 129), (17, 8, 5, 17), (1, 16, 3, 1)])
def test_dense_then_select(dtype, L, d, V, M):
    wl = inputs.make_random(L * 7 + d, L=L, d=d, V=V, M=M, dtype=dtype, std_w=0.5)
    idx = oracle.mask_compact(wl.tokens, wl.mask_id)
    assert idx.size == M
    got = oracle.masked_logits(wl.H, idx, wl.W)
    want = _dense_select(wl.H, idx, wl.W)
    assert got.shape == (M, V)
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)


def test_ratio_one_is_dense():
    wl = inputs.make_random(5, L=96, d=64, V=80, M=96, dtype="bf16")
    idx = oracle.mask_compact(wl.tokens, wl.mask_id)
    assert np.array_equal(idx, np.arange(96))
    dense = wl.H.double().numpy() @ wl.W.double().numpy().T
    np.testing.assert_allclose(oracle.masked_logits(wl.H, idx, wl.W), dense, rtol=1e-12, atol=1e-12)


def test_ratio_zero_is_no_work():
    wl = inputs.make_random(6, L=50, d=16, V=10, M=0, dtype="bf16")
    idx = oracle.mask_compact(wl.tokens, wl.mask_id)
    assert idx.size == 0
    assert oracle.masked_logits(wl.H, idx, wl.W).shape == (0, 10)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("d", [8, 256, 4096])
def test_exact_integers(dtype, d):
    L, V, M = 40, 70, 23
    H = inputs.integer_valued(1 + d, (L, d), dtype=dtype)
    W = inputs.integer_valued(2 + d, (V, d), dtype=dtype)
    rng = np.random.default_rng(d)
    idx = np.sort(rng.choice(L, M, replace=False)).astype(np.int32)
    got = oracle.masked_logits(H, idx, W)
    want = (H.to(torch.int64).numpy() @ W.to(torch.int64).numpy().T)[idx]
    assert np.array_equal(got, want.astype(np.float64))


@pytest.mark.parametrize("V,d", [(300, 64), (5, 64), (130, 128)])
def test_one_hot_weights(V, d):
    wl = inputs.make_random(3, L=77, d=d, V=V, M=31, dtype="bf16")
    idx = oracle.mask_compact(wl.tokens, wl.mask_id)
    W = inputs.one_hot_rows(V, d)
    got = oracle.masked_logits(wl.H, idx, W)
    h = wl.H.double().numpy()
    want = h[idx][:, np.arange(V) % d]
    assert np.array_equal(got, want)


def test_one_hot_hidden_rows():
    L, d, V = 40, 32, 50
    H = torch.zeros(L, d)
    H[torch.arange(L), torch.arange(L) % d] = 1.0
    H = H.to(torch.bfloat16)
    W = inputs.make_random(4, L=2, d=d, V=V, M=1, dtype="bf16").W
    idx = np.array([39, 0, 7, 7, 33], np.int32)     # unsorted and repeated rows are allowed
    got = oracle.masked_logits(H, idx, W)
    want = W.double().numpy()[:, idx % d].T
    assert np.array_equal(got, want)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_accumulation_error_bound_vs_fsum(dtype):
    wl = inputs.make_random(9, L=20, d=2048, V=6, M=5, dtype=dtype, std_w=1.0)
    idx = oracle.mask_compact(wl.tokens, wl.mask_id)
    got = oracle.masked_logits(wl.H, idx, wl.W)
    h = wl.H.double().numpy()
    w = wl.W.double().numpy()
    for i in range(idx.size):
        for v in range(6):
            terms = h[idx[i]] * w[v]          # exact in fp64 for bf16 and fp32 inputs
            exact = math.fsum(terms)
            bound = wl.d * 2.0**-53 * np.abs(terms).sum()
            assert abs(got[i, v] - exact) <= bound


def test_row_subset_permutation_and_scaling():
    wl = inputs.make_random(12, L=120, d=48, V=37, M=70, dtype="bf16")
    idx = oracle.mask_compact(wl.tokens, wl.mask_id)
    full = oracle.masked_logits(wl.H, idx, wl.W)
    rows = np.array([69, 0, 5, 5, 33], np.int64)
    assert np.array_equal(oracle.masked_logits(wl.H, idx, wl.W, rows=rows), full[rows])
    perm = np.random.default_rng(0).permutation(idx.size)
    assert np.array_equal(oracle.masked_logits(wl.H, idx[perm], wl.W), full[perm])
    W2 = (wl.W.float() * 2).to(torch.bfloat16)        # exact doubling
    assert np.array_equal(oracle.masked_logits(wl.H, idx, W2), 2 * full)


def test_out_of_range_index_is_an_error():
    wl = inputs.make_random(13, L=10, d=8, V=4, M=3, dtype="bf16")
    with pytest.raises(IndexError):
        oracle.masked_logits(wl.H, np.array([0, 10], np.int32), wl.W)
    with pytest.raises(IndexError):
        oracle.masked_logits(wl.H, np.array([0, 1], np.int32), wl.W, rows=np.array([2]))


def test_thread_count_does_not_change_results():
    # each logit is one ascending-k sum on one thread, so the thread count cannot matter
    wl = inputs.make_random(77, L=300, d=128, V=500, M=150, dtype="bf16")
    idx = oracle.mask_compact(wl.tokens, wl.mask_id)
    n = oracle.num_threads()
    ref = oracle.masked_logits(wl.H, idx, wl.W)
    oracle.set_num_threads(1)
    try:
        assert oracle.num_threads() == 1
        one = oracle.masked_logits(wl.H, idx, wl.W)
    finally:
        oracle.set_num_threads(n)
    assert oracle.num_threads() == n
    assert np.array_equal(one, ref)
