"""GPU compaction vs the CPU oracle: bit-exact idx, count and CSR offsets."""
import numpy as np
import pytest
import torch

import oracle
from mask_only_logits_amd import inputs

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
MASK = 1023


@pytest.fixture(scope="module")
def m():
    from mask_only_logits_amd import mosaic
    return mosaic


def _tokens(flags, seed):
    rng = np.random.default_rng(seed)
    t = rng.integers(0, MASK, size=flags.size).astype(np.int32)
    t[flags] = MASK
    return t


def _run(m, tok):
    t = torch.from_numpy(tok).to(DEV)
    idx = torch.full((max(tok.size, 1) + 5,), -7, dtype=torch.int32, device=DEV)
    cnt = torch.full((1,), -1, dtype=torch.int32, device=DEV)
    m.mosaic_mask_compact(t, MASK, idx=idx, count=cnt)
    torch.cuda.synchronize()
    c = int(cnt.item())
    return idx.cpu().numpy(), c


EDGE_L = [0, 1, 2, 63, 64, 65, 127, 128, 129, 255, 256, 257, 511, 512, 513, 1023, 1024, 1025,
          4095, 4096, 4097, 8191, 8192, 8193, 16383, 16384, 16385, 100_000, 131072]


@pytest.mark.parametrize("L", EDGE_L)
@pytest.mark.parametrize("pattern", ["none", "all", "alternate", "first", "last", "random30", "random97"])
def test_compact_patterns(m, L, pattern):
    p = np.arange(L)
    flags = {"none": p < 0, "all": p >= 0, "alternate": p % 2 == 1, "first": p == 0, "last": p == L - 1,
             "random30": np.random.default_rng(L).random(L) < 0.3,
             "random97": np.random.default_rng(L + 1).random(L) < 0.97}[pattern]
    tok = _tokens(flags, L)
    want = oracle.mask_compact(tok, MASK)
    got, c = _run(m, tok)
    assert c == want.size
    assert np.array_equal(got[:c], want)
    assert np.all(got[c:] == -7), "wrote past the masked count"


@pytest.mark.parametrize("L", [1, 64, 65, 4097, 131072])
def test_compact_flags(m, L):
    rng = np.random.default_rng(L)
    f = (rng.random(L) < 0.4).astype(np.uint8) * rng.integers(1, 255, size=L).astype(np.uint8)
    want = oracle.mask_compact_flags(f)
    idx, cnt = m.mosaic_mask_compact_flags(torch.from_numpy(f).to(DEV))
    torch.cuda.synchronize()
    c = int(cnt.item())
    assert c == want.size and np.array_equal(idx[:c].cpu().numpy(), want)


@pytest.mark.parametrize("name", ["tiny", "llada_step", "long_logits", "long_ffn", "lowm"])
def test_compact_workloads(m, name):
    wl = inputs.make_workload(name, with_weights=False)
    want = oracle.mask_compact(wl.tokens, wl.mask_id)
    idx, cnt = m.mosaic_mask_compact(wl.tokens.to(DEV), wl.mask_id)
    torch.cuda.synchronize()
    c = int(cnt.item())
    assert c == want.size and np.array_equal(idx[:c].cpu().numpy(), want)


def _batched(m, tok, so):
    idx, off = m.mosaic_mask_compact_batched(torch.from_numpy(tok).to(DEV), torch.from_numpy(so).to(DEV), MASK)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), off.cpu().numpy()


@pytest.mark.parametrize("seed,nseq,Lmax,ratio", [(1, 1, 300, 0.5), (2, 16, 4096, 0.4), (3, 300, 40, 0.9),
                                                  (4, 9, 0, 0.5), (5, 50, 129, 0.0), (6, 7, 1000, 1.0)])
def test_compact_batched(m, seed, nseq, Lmax, ratio):
    rng = np.random.default_rng(seed)
    lens = rng.integers(0, Lmax + 1, size=nseq)
    so = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    flags = rng.random(int(so[-1])) < ratio
    tok = _tokens(flags, seed)
    want_idx, want_off = oracle.mask_compact_batched(tok, so, MASK)
    got_idx, got_off = _batched(m, tok, so)
    assert np.array_equal(got_off, want_off)
    assert np.array_equal(got_idx[:want_off[-1]], want_idx)


def test_compact_ragged_workload(m):
    wl = inputs.make_workload("ragged", with_weights=False)
    want_idx, want_off = oracle.mask_compact_batched(wl.tokens, wl.seq_offsets, wl.mask_id)
    idx, off = m.mosaic_mask_compact_batched(wl.tokens.to(DEV), wl.seq_offsets.to(DEV), wl.mask_id)
    torch.cuda.synchronize()
    assert np.array_equal(off.cpu().numpy(), want_off)
    assert np.array_equal(idx[:want_off[-1]].cpu().numpy(), want_idx)


def test_compact_with_a_caller_workspace(m):
    # a caller that passes the workspace the query asks for (here 0 bytes, any buffer)
    # gets the same lists as one that passes none
    wl = inputs.make_workload("llada_step", with_weights=False)
    assert m.mosaic_mask_compact_workspace_bytes(wl.L) == 0
    ws = torch.empty(64, dtype=torch.uint8, device=DEV)
    want = oracle.mask_compact(wl.tokens, wl.mask_id)
    idx, cnt = m.mosaic_mask_compact(wl.tokens.to(DEV), wl.mask_id, workspace=ws)
    flags = torch.from_numpy((wl.tokens.numpy() == wl.mask_id).astype(np.uint8)).to(DEV)
    idx_f, cnt_f = m.mosaic_mask_compact_flags(flags, workspace=ws)
    so = torch.tensor([0, wl.L // 2, wl.L], dtype=torch.int32, device=DEV)
    idx_b, off_b = m.mosaic_mask_compact_batched(wl.tokens.to(DEV), so, wl.mask_id, workspace=ws)
    torch.cuda.synchronize()
    c = int(cnt.item())
    assert c == want.size and np.array_equal(idx[:c].cpu().numpy(), want)
    assert int(cnt_f.item()) == c and np.array_equal(idx_f[:c].cpu().numpy(), want)
    assert int(off_b[-1].item()) == c and np.array_equal(idx_b[:c].cpu().numpy(), want)
