"""Shared test helpers: tolerance checks against the fp64 oracle."""
import numpy as np
import torch

# |gpu - oracle| <= tol * max(1, |oracle|): 1e-2 for bf16 logits, 1e-4 for fp32 logits.
TOL = {torch.bfloat16: 1e-2, torch.float32: 1e-4}


def scaled_error(got: torch.Tensor, ref: np.ndarray) -> np.ndarray:
    g = got.detach().float().cpu().numpy().astype(np.float64)
    assert g.shape == ref.shape, (g.shape, ref.shape)
    return np.abs(g - ref) / np.maximum(1.0, np.abs(ref))


def assert_close(got: torch.Tensor, ref: np.ndarray, what: str = ""):
    err = scaled_error(got, ref)
    tol = TOL[got.dtype]
    bad = int((err > tol).sum())
    assert np.isfinite(err).all(), f"{what}: non-finite values"
    assert bad == 0, f"{what}: {bad} of {err.size} elements beyond {tol} (max {err.max():.3e})"
    return float(err.max())


def bf16_rne(x: np.ndarray) -> torch.Tensor:
    """Round fp64 values that are exact in fp32 to bf16 (torch CPU conversion, RNE)."""
    return torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16)


def sample_rows(M: int, chunk: int, n_random: int, seed: int = 0) -> np.ndarray:
    """First/last rows, rows around every chunk and 256-row tile boundary, plus random rows."""
    rows = {0, M - 1}
    for step in ([chunk] if chunk > 0 else []) + [256]:
        for b in range(step, M, step):
            rows.update({b - 1, b})
    rows = sorted(r for r in rows if 0 <= r < M)
    rng = np.random.default_rng(seed)
    if len(rows) > 48:
        rows = sorted(rng.choice(rows, 48, replace=False).tolist() + [0, M - 1])
    extra = rng.choice(M, size=min(M, n_random), replace=False)
    return np.unique(np.concatenate([np.array(rows, np.int64), extra.astype(np.int64)]))
