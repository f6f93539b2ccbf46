"""Pins of the oracle's compaction (masked positions -> ascending index list).

The oracle is checked against things other than itself:
- numpy's flatnonzero (a library routine computing exactly the ascending list of
  set positions) on every mask of length <= 12 and on random masks;
- invariants (strictly increasing, in range, same set as the flagged positions,
  count = number of flags);
- closed forms (nothing masked, everything masked, alternating, trailing block);
- for ragged batches, numpy's searchsorted on the global list gives the CSR
  offsets, and each sequence's slice equals the single-sequence result shifted.
"""
import itertools

import numpy as np
import pytest

import oracle

MASK = 7


def tokens_from_flags(flags, rng=None):
    flags = np.asarray(flags, dtype=bool)
    rng = rng or np.random.default_rng(0)
    tok = rng.integers(0, MASK, size=flags.size).astype(np.int32)
    tok[flags] = MASK
    return tok


@pytest.mark.parametrize("L", range(0, 13))
def test_exhaustive_small(L):
    # every one of the 2^L masks of length L
    for bits in itertools.product([0, 1], repeat=L):
        f = np.array(bits, dtype=np.uint8)
        want = np.flatnonzero(f).astype(np.int32)
        got = oracle.mask_compact_flags(f)
        assert np.array_equal(got, want)
        got_t = oracle.mask_compact(tokens_from_flags(f), MASK)
        assert np.array_equal(got_t, want)


@pytest.mark.parametrize("L", [1, 63, 64, 65, 127, 128, 129, 255, 256, 257, 4095, 4096, 4097, 131072])
@pytest.mark.parametrize("ratio", [0.0, 0.005, 0.3, 0.5, 0.9, 1.0])
def test_random_masks_and_invariants(L, ratio):
    rng = np.random.default_rng(L * 1000 + int(ratio * 100))
    f = rng.random(L) < ratio
    tok = tokens_from_flags(f, rng)
    got = oracle.mask_compact(tok, MASK)
    assert got.dtype == np.int32
    assert np.array_equal(got, np.flatnonzero(f))
    # invariants
    assert got.size == int(f.sum())
    assert np.all(np.diff(got.astype(np.int64)) > 0)
    if got.size:
        assert got[0] >= 0 and got[-1] < L
    assert set(got.tolist()) == set(np.nonzero(tok == MASK)[0].tolist())


def test_closed_forms():
    L = 1000
    assert oracle.mask_compact(np.zeros(L, np.int32), MASK).size == 0
    assert np.array_equal(oracle.mask_compact(np.full(L, MASK, np.int32), MASK), np.arange(L))
    alt = np.where(np.arange(L) % 2 == 1, MASK, 0).astype(np.int32)
    assert np.array_equal(oracle.mask_compact(alt, MASK), 2 * np.arange(L // 2) + 1)
    # a trailing block of M positions: idx[i] = L - M + i
    L, M = 131072, 39322
    tail = np.zeros(L, np.int32)
    tail[L - M:] = MASK
    got = oracle.mask_compact(tail, MASK)
    assert got.size == M and got[0] == 91750
    assert np.array_equal(got, (L - M) + np.arange(M))


def test_mask_id_is_compared_not_thresholded():
    tok = np.array([MASK - 1, MASK, MASK + 1, -MASK, MASK], np.int32)
    assert oracle.mask_compact(tok, MASK).tolist() == [1, 4]
    assert oracle.mask_compact(tok, -MASK).tolist() == [3]


def _ragged(seed, nseq, Ls_max, ratio, allow_empty=True):
    rng = np.random.default_rng(seed)
    lens = rng.integers(0 if allow_empty else 1, Ls_max + 1, size=nseq)
    so = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    f = rng.random(int(so[-1])) < ratio
    return so, f, tokens_from_flags(f, rng)


@pytest.mark.parametrize("seed,nseq,Ls,ratio", [(1, 1, 50, 0.5), (2, 16, 300, 0.4), (3, 40, 20, 0.9),
                                                (4, 7, 0, 0.5), (5, 33, 129, 0.0), (6, 12, 65, 1.0)])
def test_batched(seed, nseq, Ls, ratio):
    so, f, tok = _ragged(seed, nseq, Ls, ratio)
    idx, off = oracle.mask_compact_batched(tok, so, MASK)
    # the global list is the flat compaction, and the CSR offsets come from searchsorted
    assert np.array_equal(idx, np.flatnonzero(f))
    assert np.array_equal(off, np.searchsorted(idx, so, side="left"))
    assert off[0] == 0 and off[-1] == idx.size and np.all(np.diff(off) >= 0)
    # each sequence's slice: global ids inside its own range, equal to a single-sequence
    # compaction shifted by the sequence start
    for s in range(nseq):
        sl = idx[off[s]:off[s + 1]]
        assert np.all(sl >= so[s]) and np.all(sl < so[s + 1])
        loc = oracle.mask_compact(tok[so[s]:so[s + 1]], MASK)
        assert np.array_equal(sl, loc + so[s])
