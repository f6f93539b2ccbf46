"""Pins of the oracle's FP8 (OCP E4M3) LM head.

- E4M3 decode of all 256 codes and encode of every midpoint between neighbouring
  codes plus random values: torch's float8_e4m3fn conversion (a library routine);
- encode(decode(c)) == c for every finite code; saturation at +-448;
- per-row quantization: the largest element of a nonzero row maps to +-448, a zero row
  gives zero codes and scale 0, the scale is fp32(amax / 448), and every element is
  within half a code spacing of its scaled value;
- logits of quantized rows: numpy's fp64 product of the dequantized matrices;
- exact case: integers in [-7, 7] with a +-7 in every row have scale 1/64 and exact
  codes, so the FP8 logits equal numpy's int64 product;
- the FP8 logits stay close to the exact bf16 logits (quantization error ~2^-4 per
  element, so a few percent of the logit scale).
"""
import math

import numpy as np
import pytest
import torch

import oracle
from mask_only_logits_amd import inputs

F8 = torch.float8_e4m3fn


def test_decode_all_codes():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(F8).to(torch.float64).numpy()
    got = np.array([oracle.e4m3_value(c) for c in range(256)])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan) and nan.sum() == 2
    assert np.array_equal(got[~nan], ref[~nan])


def test_encode_midpoints_and_random():
    vals = np.array(sorted({oracle.e4m3_value(c) for c in range(0x7F)}))     # finite non-negative
    mids = (vals[:-1] + vals[1:]) / 2
    rng = np.random.default_rng(0)
    xs = np.concatenate([vals, mids, -mids, rng.uniform(-448, 448, 4000), rng.normal(0, 1, 4000),
                         rng.normal(0, 0.01, 2000)]).astype(np.float32)
    ref = torch.from_numpy(xs).to(F8).view(torch.uint8).numpy()
    got = np.array([oracle.e4m3_encode(x) for x in xs], np.uint8)
    assert np.array_equal(got, ref)


def test_round_trip_and_saturation():
    for c in range(256):
        if c in (0x7F, 0xFF):
            continue
        assert oracle.e4m3_encode(np.float32(oracle.e4m3_value(c))) == c, hex(c)
    assert oracle.e4m3_encode(1000.0) == 0x7E and oracle.e4m3_encode(-1e9) == 0xFE
    assert oracle.e4m3_encode(464.0) == 0x7E      # the midpoint to the (non-finite) next code


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_quantize_rows_invariants(dtype):
    n, d = 50, 96
    X = inputs.make_random(5, L=n, d=d, V=4, M=1, dtype=dtype).H.clone()
    X[3] = 0                                            # a zero row
    q, sc = oracle.quantize_rows_e4m3(X)
    x = X.to(torch.float64).numpy()
    val = np.vectorize(oracle.e4m3_value)(q)
    assert np.all(q[3] == 0) and sc[3] == 0.0
    for r in range(n):
        if r == 3:
            continue
        amax = np.float32(np.abs(x[r]).max())
        assert sc[r] == np.float32(amax / np.float32(448.0))
        assert np.abs(val[r]).max() == 448.0
        inv = np.float32(np.float32(448.0) / amax)
        y = (x[r].astype(np.float32) * inv).astype(np.float64)
        # within half a code spacing: 2^-4 relative for normal codes, 2^-10 absolute for subnormals
        assert np.all(np.abs(val[r] - y) <= np.maximum(np.abs(y) * 2.0 ** -4, 2.0 ** -10) + 1e-12)
    # gathered rows are the same as quantizing the rows themselves
    ridx = np.array([7, 0, 7, 49], np.int32)
    q2, sc2 = oracle.quantize_rows_e4m3(X, ridx)
    assert np.array_equal(q2, q[ridx]) and np.array_equal(sc2, sc[ridx])
    with pytest.raises(IndexError):
        oracle.quantize_rows_e4m3(X, np.array([50], np.int32))


def test_logits_match_numpy_on_dequantized():
    wl = inputs.make_random(9, L=60, d=64, V=90, M=25, dtype="bf16")
    idx = oracle.mask_compact(wl.tokens, wl.mask_id)
    qh, sh = oracle.quantize_rows_e4m3(wl.H, idx)
    qw, sw = oracle.quantize_rows_e4m3(wl.W)
    out = oracle.logits_fp8(qh, sh, qw, sw)
    deq = lambda q, s: torch.from_numpy(q).view(F8).to(torch.float64).numpy() * s.astype(np.float64)[:, None]
    ref = deq(qh, sh) @ deq(qw, sw).T
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-15)
    assert np.array_equal(oracle.masked_logits_fp8(wl.H, idx, wl.W), out)


def test_exact_integers():
    rng = np.random.default_rng(4)
    L, d, V, M = 40, 64, 50, 20
    H = rng.integers(-7, 8, (L, d)).astype(np.float32)
    W = rng.integers(-7, 8, (V, d)).astype(np.float32)
    H[:, 0] = 7                                         # amax 7 in every row -> scale 1/64
    W[:, 1] = -7
    idx = np.sort(rng.choice(L, M, replace=False)).astype(np.int32)
    Hb, Wb = torch.from_numpy(H).to(torch.bfloat16), torch.from_numpy(W).to(torch.bfloat16)
    out = oracle.masked_logits_fp8(Hb, idx, Wb)
    exact = (H.astype(np.int64)[idx] @ W.astype(np.int64).T).astype(np.float64)
    assert np.array_equal(out, exact)


def test_close_to_exact_logits():
    wl = inputs.make_random(21, L=200, d=512, V=300, M=60, dtype="bf16")
    idx = oracle.mask_compact(wl.tokens, wl.mask_id)
    f8 = oracle.masked_logits_fp8(wl.H, idx, wl.W)
    ex = oracle.masked_logits(wl.H, idx, wl.W)
    rel = np.abs(f8 - ex).max() / np.abs(ex).max()
    assert rel < 0.05, rel
    assert math.isfinite(rel) and rel > 1e-4      # the quantization does change the values
