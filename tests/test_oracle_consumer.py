"""Pins of the oracle's per-row consumer (row max, first argmax, log-sum-exp of a
masked row's fp64 logits).

Each pin reaches the answer another way than the oracle's own loop:
- library routines: numpy's fp64 BLAS product (dense-then-select), numpy's max and
  argmax (first occurrence) and scipy's logsumexp;
- zero weights: every logit is 0, so max = 0, argmax = 0 (the first index, which pins
  the tie rule) and lse = log(V) exactly;
- one-hot weights W[v, k] = [k == v mod d]: z[v] = h[v mod d], so the argmax is the
  first k attaining max(h) and sum_v exp(z[v]) = sum_k c_k exp(h[k]) with c_k the
  number of v congruent to k (a grouped sum);
- exact integers: logits are integers computed exactly by numpy's int64 product;
- large logits (|z| ~ 2000): exp overflows without the max shift; scipy's stable
  logsumexp and the bounds max <= lse <= max + log(V) pin the shifted form.
"""
import math

import numpy as np
import pytest
import torch
from scipy.special import logsumexp

import oracle
from mask_only_logits_amd import inputs


def _dense_select(H, idx, W):
    h = H.to(torch.float64).numpy()
    w = W.to(torch.float64).numpy()
    return (h @ w.T)[idx]


@pytest.mark.parametrize("L,d,V,M", [(64, 32, 48, 30), (300, 136, 257, 129), (17, 8, 5, 17), (40, 16, 1, 7)])
def test_matches_library_routines(L, d, V, M):
    wl = inputs.make_random(L * 5 + d + V, L=L, d=d, V=V, M=M, dtype="bf16", std_w=0.5)
    idx = oracle.mask_compact(wl.tokens, wl.mask_id)
    mx, am, lse = oracle.masked_logits_argmax_lse(wl.H, idx, wl.W)
    z = _dense_select(wl.H, idx, wl.W)
    np.testing.assert_allclose(mx, z.max(axis=1), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse, logsumexp(z, axis=1), rtol=1e-12, atol=1e-12)
    ref_am = z.argmax(axis=1)
    for i in range(M):
        if am[i] != ref_am[i]:
            # only a near-tie within fp64 summation-order noise may differ
            assert abs(z[i, am[i]] - z[i, ref_am[i]]) <= 1e-12 * max(1.0, abs(z[i, ref_am[i]])), i


def test_zero_weights_closed_form():
    L, d, V, M = 50, 24, 1000, 20
    wl = inputs.make_random(7, L=L, d=d, V=V, M=M, dtype="bf16")
    W0 = torch.zeros((V, d), dtype=torch.bfloat16)
    idx = oracle.mask_compact(wl.tokens, wl.mask_id)
    mx, am, lse = oracle.masked_logits_argmax_lse(wl.H, idx, W0)
    assert np.all(mx == 0.0)
    assert np.all(am == 0)
    np.testing.assert_allclose(lse, math.log(V), rtol=0, atol=1e-13)


@pytest.mark.parametrize("d,V", [(16, 100), (32, 32), (8, 1001)])
def test_one_hot_weights_grouped_sum(d, V):
    L, M = 40, 25
    wl = inputs.make_random(d * 3 + V, L=L, d=d, V=V, M=M, dtype="bf16")
    idx = oracle.mask_compact(wl.tokens, wl.mask_id)
    W1 = inputs.one_hot_rows(V, d)
    mx, am, lse = oracle.masked_logits_argmax_lse(wl.H, idx, W1)
    h = wl.H.to(torch.float64).numpy()[idx]
    cols = min(d, V)                               # entries of h reachable as some v mod d
    counts = np.array([len(range(k, V, d)) for k in range(cols)], np.float64)
    for i in range(M):
        hr = h[i, :cols]
        assert mx[i] == hr.max()
        assert am[i] == int(np.flatnonzero(hr == hr.max())[0])
        grouped = math.fsum(c * math.exp(x - hr.max()) for c, x in zip(counts, hr))
        np.testing.assert_allclose(lse[i], hr.max() + math.log(grouped), rtol=1e-13, atol=1e-13)


def test_exact_integers():
    L, d, V, M = 60, 48, 300, 35
    H = inputs.integer_valued(11, (L, d))
    W = inputs.integer_valued(12, (V, d))
    idx = np.sort(np.random.default_rng(3).choice(L, M, replace=False)).astype(np.int32)
    mx, am, lse = oracle.masked_logits_argmax_lse(H, idx, W)
    z = (H.to(torch.int64).numpy() @ W.to(torch.int64).numpy().T)[idx]
    assert np.array_equal(mx, z.max(axis=1).astype(np.float64))
    assert np.array_equal(am, z.argmax(axis=1))
    # integer gaps: sum_v exp(z - max) grouped by gap value
    for i in range(M):
        gaps, cnt = np.unique(z[i].max() - z[i], return_counts=True)
        grouped = math.fsum(float(c) * math.exp(-float(g)) for g, c in zip(gaps, cnt))
        np.testing.assert_allclose(lse[i], z[i].max() + math.log(grouped), rtol=1e-14, atol=1e-13)


def test_large_logits_stable():
    L, d, V, M = 30, 64, 400, 12
    wl = inputs.make_random(99, L=L, d=d, V=V, M=M, dtype="bf16", std_w=1.0)
    H = (wl.H.float() * 64.0).to(torch.bfloat16)     # logits of magnitude ~ 10^3
    W = (wl.W.float() * 4.0).to(torch.bfloat16)
    idx = oracle.mask_compact(wl.tokens, wl.mask_id)
    mx, am, lse = oracle.masked_logits_argmax_lse(H, idx, W)
    z = _dense_select(H, idx, W)
    assert np.abs(z).max() > 800.0
    assert np.all(np.isfinite(lse))
    assert np.all(lse >= mx) and np.all(lse <= mx + math.log(V) + 1e-9)
    np.testing.assert_allclose(lse, logsumexp(z, axis=1), rtol=1e-12, atol=1e-9)


def test_rows_subset_and_errors():
    wl = inputs.make_random(5, L=80, d=16, V=50, M=40, dtype="bf16")
    idx = oracle.mask_compact(wl.tokens, wl.mask_id)
    full = oracle.masked_logits_argmax_lse(wl.H, idx, wl.W)
    rows = np.array([39, 0, 17], np.int64)
    sub = oracle.masked_logits_argmax_lse(wl.H, idx, wl.W, rows=rows)
    for a, b in zip(full, sub):
        assert np.array_equal(a[rows], b)
    with pytest.raises(IndexError):
        oracle.masked_logits_argmax_lse(wl.H, idx, wl.W, rows=np.array([40], np.int64))
