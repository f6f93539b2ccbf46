"""The seeded workload generator: exact masked counts, reproducibility, recipe."""
import math
import os

import numpy as np
import pytest
import torch

import oracle
from mask_only_logits_amd import inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "config_mask_counts.txt")


def _golden():
    out = {}
    for ln in open(GOLDEN, encoding="utf-8"):
        if ln.strip() and not ln.startswith("#"):
            name, L, r, M = ln.split()
            out[name] = (int(L), float(r), int(M))
    return out


@pytest.mark.parametrize("name", ["tiny", "llada_step", "long_logits", "long_ffn", "lowm"])
def test_mask_counts(name):
    L, r, M = _golden()[name]
    assert inputs.masked_count(r, L) == M
    wl = inputs.make_workload(name, with_weights=False)
    assert wl.L == L
    idx = oracle.mask_compact(wl.tokens, wl.mask_id)
    assert idx.size == M
    assert wl.mask_id == wl.V - 1
    # unmasked ids stay below the mask id
    t = wl.tokens.numpy()
    assert t.min() >= 0 and t.max() == wl.mask_id
    if name == "long_ffn":
        assert np.array_equal(idx, np.arange(L - M, L))


def test_ragged_recipe():
    wl = inputs.make_workload("ragged", with_weights=False)
    so = wl.seq_offsets.numpy()
    assert wl.nseq == 16 and so[-1] == 65536 and np.all(np.diff(so) == 4096)
    idx, off = oracle.mask_compact_batched(wl.tokens, so, wl.mask_id)
    ratios = wl.info["ratios"]
    assert all(0.01 <= r < 0.98 for r in ratios)
    for s in range(16):
        assert off[s + 1] - off[s] == math.floor(ratios[s] * 4096 + 0.5)


def test_reproducible_and_thread_independent(monkeypatch):
    a = inputs.gaussian((3, 5_000_000), 0.02, np.random.SeedSequence(77))
    monkeypatch.setattr(inputs, "_threads", lambda: 1)
    b = inputs.gaussian((3, 5_000_000), 0.02, np.random.SeedSequence(77))
    assert np.array_equal(a, b)
    assert abs(float(a.std()) - 0.02) < 1e-4


def test_bf16_rounding_is_rne():
    # values exactly halfway between two bf16 neighbours round to the even one
    x = np.array([1.0 + 2**-8, 1.0 + 3 * 2**-8, -(1.0 + 2**-8), 1.0 + 2**-8 + 2**-20], np.float32)
    b = inputs.to_dtype(x, "bf16").float().numpy()
    assert b.tolist() == [1.0, 1.0 + 4 * 2**-8, -1.0, 1.0 + 2 * 2**-8]


def test_tiny_is_fp32():
    wl = inputs.make_workload("tiny")
    assert wl.H.dtype == torch.float32 and wl.W.dtype == torch.float32
    assert wl.H.shape == (256, 256) and wl.W.shape == (1024, 256)
