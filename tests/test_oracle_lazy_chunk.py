"""Pins of the oracle's lazy chunk choice for the logits operator.

Chunking stays off while the whole [M, V] logits buffer fits the budget; otherwise
the smallest number of chunks whose largest chunk fits is taken ("扩散大语言模型内存
优化：Mosaic系统突破与实践", §2.3: off by default, the minimal sufficient chunk count).

Pins:
- special cases: everything fits -> no chunking; one row does not fit -> error;
  M = 0 -> no chunks;
- worked settings from the pages: the recommended max_num_logits of 4096 rows at
  LLaDA's vocabulary of 126,464 bf16 entries ("扩散大语言模型内存优化：从理论到系统设计",
  §3.2.2 and §2.2) as the budget gives, for the 29,491 masked rows of a 32k
  sequence at ratio 0.9, the same 8 micro-batches as static 4096-row chunking but
  balanced to 3,687 rows; a budget of a quarter of the full buffer gives 4-way
  chunking (the Mosaic page's 4-way example at 32k, §2.3);
- invariants on an exhaustive sweep of small sizes: the chosen chunking fits, one
  chunk fewer does not, the chunks are balanced, and the chunk driver's own count
  (ceil(M / chunk_rows)) reproduces the chosen number of chunks.
"""
import itertools
import math

import pytest

import oracle


def test_no_chunking_when_everything_fits():
    assert oracle.lazy_chunk_rows(1000, 500, 2, 1000 * 500 * 2) == (0, 1)
    assert oracle.lazy_chunk_rows(1000, 500, 2, 10**12) == (0, 1)
    assert oracle.lazy_chunk_rows(0, 500, 2, 0) == (0, 0)
    assert oracle.lazy_chunk_rows(7, 0, 4, 0) == (0, 1)


def test_one_row_must_fit():
    with pytest.raises(ValueError):
        oracle.lazy_chunk_rows(10, 500, 2, 999)
    assert oracle.lazy_chunk_rows(10, 500, 2, 1000) == (1, 10)


def test_pages_settings():
    V, es = 126464, 2
    budget = 4096 * V * es                       # max_num_logits = 4096 rows of bf16 logits
    assert oracle.lazy_chunk_rows(29491, V, es, budget) == (3687, 8)
    assert oracle.lazy_chunk_rows(8192, V, es, budget) == (4096, 2)
    assert oracle.lazy_chunk_rows(4096, V, es, budget) == (0, 1)
    M = 29491
    quarter = math.ceil(M / 4) * V * es
    assert oracle.lazy_chunk_rows(M, V, es, quarter) == (math.ceil(M / 4), 4)


def test_invariants_exhaustive_small():
    for M, V, es in itertools.product(range(1, 40), (1, 3, 8), (1, 2, 4)):
        for budget in range(V * es, M * V * es + 2):
            C, k = oracle.lazy_chunk_rows(M, V, es, budget)
            rows = M if C == 0 else C
            assert rows * V * es <= budget                         # fits
            assert rows == math.ceil(M / k)                        # balanced
            if k > 1:
                assert math.ceil(M / (k - 1)) * V * es > budget    # one chunk fewer does not fit
                assert oracle.num_chunks(M, C) == k                # the driver makes k chunks
            else:
                assert C == 0


def test_monotone_in_budget():
    M, V, es = 1000, 77, 2
    prev = None
    for budget in range(V * es, M * V * es + 1, 97):
        _, k = oracle.lazy_chunk_rows(M, V, es, budget)
        assert prev is None or k <= prev
        prev = k
