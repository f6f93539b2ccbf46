"""Seeded synthetic workloads for the mask-only logits path.

This module only draws inputs: token ids with a mask pattern, hidden states H and
an LM-head weight W.  It holds none of the method's arithmetic (no compaction, no
chunking, no logits) so that the CPU oracle and the HIP path can both be fed from
it without sharing any computation.

Shapes and mask regimes follow the pages:
- the vocabulary size 126,464 of the LLaDA-8B LM head is the one used in the
  dense-logits size example of "扩散大语言模型内存优化：从理论到系统设计", §2.2;
- high mask ratios make logits the memory peak and low ones make the FFN the peak
  ("Mosaic: Unlocking Long-Context Inference for Diffusion LLMs via Global Memory"
  review, 核心观察 #3; "扩散大语言模型内存优化：Mosaic系统突破与实践", §1.2);
- a mask ratio of 0.6 appears in the usage example of the latter page, §5.1;
- the row-chunk sizes 4096 and 8192 are the recommended max_num_logits values of
  "扩散大语言模型内存优化：从理论到系统设计", §3.2.2 and §4.1.
The models' trained weights are not available; Gaussian H and W of the same shapes
stand in for them (H ~ N(0,1), W ~ N(0, 0.02) with 0.02 the standard deviation).

Generation recipe (fixed, so every consumer sees identical bits):
- numpy PCG64 streams derived from SeedSequence(seed); large Gaussian arrays are
  filled in fixed 16M-element blocks, block b drawing from the b-th spawned child
  sequence, so the bits do not depend on the number of worker threads;
- values are drawn as float32; bf16 workloads round them to bfloat16 with
  round-to-nearest-even (torch's CPU conversion);
- masked positions are drawn uniformly without replacement, so M is exact:
  M = floor(ratio * L + 1/2);
- unmasked token ids are uniform in [0, MASK_ID) with MASK_ID = V - 1, so no
  unmasked position carries the mask id by accident.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np
import torch

_BLOCK = 1 << 24

# Seeds of the shared LM-head weights, one per shape family, so W can be reused.
W_SEED = {(4096, 126464): 100, (3584, 152064): 200}


@dataclass
class Workload:
    """One synthetic problem.  Arrays are CPU tensors (torch) holding the exact bits."""

    name: str
    L: int
    d: int
    V: int
    dtype: str                      # "f32" or "bf16": dtype of H and W
    out_dtype: str                  # "f32" or "bf16": dtype of the logits
    mask_id: int
    tokens: torch.Tensor            # int32 [L]
    H: torch.Tensor                 # [L, d]
    W: torch.Tensor                 # [V, d]
    chunk_rows: int                 # max_num_logits; 0 = unchunked
    seq_offsets: torch.Tensor | None = None   # int32 [nseq+1] for ragged batches
    info: dict = field(default_factory=dict)

    @property
    def nseq(self) -> int:
        return 0 if self.seq_offsets is None else int(self.seq_offsets.numel() - 1)


# name: (seed, L or (nseq, Ls), d, V, in dtype, out dtype, mask rule, chunk rows)
CONFIGS = {
    # Tiny fp32 case: 50% of positions masked, MASK_ID = 1023.
    "tiny": dict(seed=1, L=256, d=256, V=1024, dtype="f32", out="f32",
                 mask=("scatter", 0.5), chunk=0),
    # LLaDA-shaped denoising step: ratio 0.6 scattered, single chunk.
    "llada_step": dict(seed=2, L=2048, d=4096, V=126464, dtype="bf16", out="bf16",
                       mask=("scatter", 0.6), chunk=0),
    # Logits-dominant long context: ratio 0.9 scattered, 4096-row chunks.
    "long_logits": dict(seed=3, L=32768, d=4096, V=126464, dtype="bf16", out="bf16",
                        mask=("scatter", 0.9), chunk=4096),
    # FFN-dominant long context: ratio 0.3 as the trailing positions, 8192-row chunks.
    "long_ffn": dict(seed=4, L=131072, d=4096, V=126464, dtype="bf16", out="bf16",
                     mask=("tail", 0.3), chunk=8192),
    # Ragged batch: 16 sequences of 4096, per-sequence ratio ~ U[0.01, 0.98).
    "ragged": dict(seed=5, L=(16, 4096), d=3584, V=152064, dtype="bf16", out="bf16",
                   mask=("ragged", 0.01, 0.98), chunk=0),
    # Low-M: one sequence, ratio 0.005 -> M = 20; streaming W dominates.
    "lowm": dict(seed=6, L=4096, d=3584, V=152064, dtype="bf16", out="bf16",
                 mask=("scatter", 0.005), chunk=0),
}


def masked_count(ratio: float, L: int) -> int:
    """Number of masked positions for a ratio: floor(ratio*L + 1/2)."""
    return int(math.floor(ratio * L + 0.5))


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def gaussian(shape, std: float, seed_seq: np.random.SeedSequence) -> np.ndarray:
    """float32 N(0, std^2) array filled block-wise from spawned PCG64 streams."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.float32)
    nb = max(1, (n + _BLOCK - 1) // _BLOCK)
    kids = seed_seq.spawn(nb)

    def fill(b):
        g = np.random.Generator(np.random.PCG64(kids[b]))
        s, e = b * _BLOCK, min(n, (b + 1) * _BLOCK)
        g.standard_normal(e - s, dtype=np.float32, out=out[s:e])
        if std != 1.0:
            out[s:e] *= np.float32(std)

    if nb == 1:
        fill(0)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(fill, range(nb)))
    return out.reshape(shape)


def to_dtype(x: np.ndarray, dtype: str) -> torch.Tensor:
    t = torch.from_numpy(x)
    if dtype == "bf16":
        return t.to(torch.bfloat16)
    if dtype == "f32":
        return t.clone()
    raise ValueError(dtype)


def mask_tokens(rng: np.random.Generator, L: int, positions: np.ndarray, mask_id: int) -> np.ndarray:
    """Token ids: uniform in [0, mask_id) everywhere, mask_id at `positions`."""
    tok = rng.integers(0, mask_id, size=L, dtype=np.int64).astype(np.int32)
    tok[positions] = mask_id
    return tok


def scattered_positions(rng: np.random.Generator, L: int, M: int) -> np.ndarray:
    return rng.choice(L, size=M, replace=False)


_W_CACHE: dict = {}


def lm_head(d: int, V: int, dtype: str, seed: int | None = None, cache: bool = True) -> torch.Tensor:
    """LM-head weight W[V, d] ~ N(0, 0.02), seeded per shape family."""
    if seed is None:
        seed = W_SEED.get((d, V), 1000 + d + V)
    key = (d, V, dtype, seed)
    if cache and key in _W_CACHE:
        return _W_CACHE[key]
    W = to_dtype(gaussian((V, d), 0.02, np.random.SeedSequence(seed)), dtype)
    if cache:
        _W_CACHE[key] = W
    return W


def make_workload(name: str, *, with_weights: bool = True) -> Workload:
    """Build one of the named configurations (see CONFIGS)."""
    c = CONFIGS[name]
    ss = np.random.SeedSequence(c["seed"])
    s_mask, s_tok, s_h = ss.spawn(3)
    rm = np.random.Generator(np.random.PCG64(s_mask))
    rt = np.random.Generator(np.random.PCG64(s_tok))
    d, V = c["d"], c["V"]
    mask_id = V - 1
    kind = c["mask"][0]
    seq_offsets = None
    info = {}
    if kind == "ragged":
        nseq, Ls = c["L"]
        L = nseq * Ls
        lo, hi = c["mask"][1], c["mask"][2]
        ratios = rm.uniform(lo, hi, size=nseq)
        pos = []
        for s in range(nseq):
            Ms = masked_count(float(ratios[s]), Ls)
            pos.append(s * Ls + scattered_positions(rm, Ls, Ms))
        positions = np.concatenate(pos)
        seq_offsets = torch.arange(0, L + 1, Ls, dtype=torch.int32)
        info["ratios"] = ratios.tolist()
    else:
        L = c["L"]
        ratio = c["mask"][1]
        M = masked_count(ratio, L)
        if kind == "scatter":
            positions = scattered_positions(rm, L, M)
        elif kind == "tail":
            positions = np.arange(L - M, L)
        else:  # pragma: no cover
            raise ValueError(kind)
    tokens = torch.from_numpy(mask_tokens(rt, L, positions, mask_id))
    if with_weights:
        H = to_dtype(gaussian((L, d), 1.0, s_h), c["dtype"])
        W = lm_head(d, V, c["dtype"])
    else:
        H = W = None
    return Workload(name=name, L=L, d=d, V=V, dtype=c["dtype"], out_dtype=c["out"],
                    mask_id=mask_id, tokens=tokens, H=H, W=W, chunk_rows=c["chunk"],
                    seq_offsets=seq_offsets, info=info)


def make_random(seed: int, L: int, d: int, V: int, M: int, *, dtype: str = "bf16",
                out_dtype: str | None = None, chunk_rows: int = 0, std_w: float = 0.02,
                nseq: int = 0) -> Workload:
    """A free-size problem for parity tests: M scattered masked rows of L."""
    ss = np.random.SeedSequence(seed)
    s_mask, s_tok, s_h, s_w = ss.spawn(4)
    rm = np.random.Generator(np.random.PCG64(s_mask))
    rt = np.random.Generator(np.random.PCG64(s_tok))
    mask_id = max(V - 1, 1)
    positions = scattered_positions(rm, L, M)
    tokens = torch.from_numpy(mask_tokens(rt, L, positions, mask_id))
    H = to_dtype(gaussian((L, d), 1.0, s_h), dtype)
    W = to_dtype(gaussian((V, d), std_w, s_w), dtype)
    seq_offsets = None
    if nseq:
        cuts = np.sort(rm.choice(np.arange(1, L), size=nseq - 1, replace=False)) if nseq > 1 else np.array([], np.int64)
        seq_offsets = torch.from_numpy(np.concatenate([[0], cuts, [L]]).astype(np.int32))
    return Workload(name=f"random{seed}", L=L, d=d, V=V, dtype=dtype,
                    out_dtype=out_dtype or dtype, mask_id=mask_id, tokens=tokens, H=H, W=W,
                    chunk_rows=chunk_rows, seq_offsets=seq_offsets)


def integer_valued(seed: int, shape, lo: int = -2, hi: int = 2, dtype: str = "bf16") -> torch.Tensor:
    """Uniform integers in [lo, hi], exactly representable in bf16 and fp32."""
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed)))
    x = g.integers(lo, hi + 1, size=shape).astype(np.float32)
    return to_dtype(x, dtype)


def one_hot_rows(V: int, d: int, dtype: str = "bf16") -> torch.Tensor:
    """W[v, k] = 1 if k == v mod d else 0."""
    W = torch.zeros((V, d), dtype=torch.float32)
    v = torch.arange(V)
    W[v, v % d] = 1.0
    return W.to(torch.bfloat16) if dtype == "bf16" else W
