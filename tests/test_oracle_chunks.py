"""Pins of the oracle's row-chunk partition (dLLM-Serve's max_num_logits micro-batching).

"扩散大语言模型内存优化：从理论到系统设计", §3.2.2: rows that need logits are
processed whole when there are at most max_num_logits of them, otherwise in
consecutive slices of max_num_logits rows whose results are concatenated in order.
Checked against math.ceil, a direct enumeration of range(0, M, C) slices, the
closed forms of the long-context workloads, and the concatenation law on logits.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from mask_only_logits_amd import inputs


@pytest.mark.parametrize("M,C,K,last", [
    (29491, 4096, 8, 819),     # logits-dominant long context
    (39322, 8192, 5, 6554),    # FFN-dominant long context
    (1229, 0, 1, 1229),        # unchunked
    (1229, -5, 1, 1229),       # negative = unchunked
    (1229, 1229, 1, 1229),
    (1229, 4096, 1, 1229),
    (1229, 1228, 2, 1),
    (1, 1, 1, 1),
    (20, 1, 20, 1),
])
def test_closed_forms(M, C, K, last):
    assert oracle.num_chunks(M, C) == K
    r0, r1 = oracle.chunk_range(M, C, K - 1)
    assert r1 == M and r1 - r0 == last


def test_zero_rows_is_no_work():
    for C in (-1, 0, 1, 4096):
        assert oracle.num_chunks(0, C) == 0


def test_partition_matches_slices():
    rng = np.random.default_rng(0)
    cases = [(int(m), int(c)) for m, c in zip(rng.integers(1, 5000, 200), rng.integers(-3, 700, 200))]
    cases += [(M, C) for M in range(1, 40) for C in range(-1, 42)]
    for M, C in cases:
        K = oracle.num_chunks(M, C)
        if C <= 0 or C >= M:
            want = [(0, M)]
        else:
            assert K == math.ceil(M / C)
            want = [(i, min(i + C, M)) for i in range(0, M, C)]
        got = [oracle.chunk_range(M, C, k) for k in range(K)]
        assert got == want
        # consecutive, disjoint, covering [0, M), none longer than C
        assert got[0][0] == 0 and got[-1][1] == M
        assert all(a[1] == b[0] for a, b in zip(got, got[1:]))
        if C > 0:
            assert all(r1 - r0 <= C for r0, r1 in got)


def test_chunked_logits_concatenate_to_unchunked():
    wl = inputs.make_random(11, L=97, d=40, V=33, M=61, dtype="bf16")
    idx = oracle.mask_compact(wl.tokens, wl.mask_id)
    full = oracle.masked_logits(wl.H, idx, wl.W)
    for C in (0, 1, 7, 60, 61, 62, 1000):
        ch = oracle.masked_logits_chunked(wl.H, idx, wl.W, C)
        assert np.array_equal(ch, full)


def test_logits_size_printed_example():
    # tests/golden/dense_logits_size.txt: the page's dense-logits example
    path = __file__.replace("test_oracle_chunks.py", "golden/dense_logits_size.txt")
    rows = [ln.split() for ln in open(path, encoding="utf-8") if ln.strip() and not ln.startswith("#")]
    for B, Lq, V, es, gb in rows:
        n = oracle.logits_bytes(int(B) * int(Lq), int(V), int(es))
        assert n == 8_287_944_704
        assert round(n / 1e9, 1) == float(gb)
    assert oracle.logits_bytes(2**62, 4, 2) == -1
    assert oracle.logits_bytes(0, 126464, 2) == 0
