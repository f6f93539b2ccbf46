"""GPU checks of mosaic_masked_logits_device_count and
mosaic_masked_logits_argmax_lse_device_count: the row count read by the kernels from device
memory (the compaction's count, with no read-back) gives the same bits as the calls that
take M from the host (which the oracle parity tests cover), writes no row at or past the
count, and clamps the count to [0, max_rows]."""
import numpy as np
import pytest
import torch

import oracle
from mask_only_logits_amd import inputs
from tests.helpers import assert_close, sample_rows

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
POISON = -12352.0    # exact in bf16


@pytest.fixture(scope="module")
def m():
    from mask_only_logits_amd import mosaic
    return mosaic


def _poisoned(rows, V):
    return torch.full((rows, V), POISON, dtype=torch.bfloat16, device=DEV)


@pytest.mark.parametrize("L,d,V,M", [(700, 64, 1000, 600), (900, 256, 5000, 700), (3000, 192, 2100, 2600),
                                     (300, 4096, 300, 1), (17000, 128, 700, 16500)])
def test_count_from_compaction_equals_host_count(m, L, d, V, M):
    wl = inputs.make_random(L + d + V, L=L, d=d, V=V, M=M, dtype="bf16")
    tokens = wl.tokens.to(DEV)
    H, W = wl.H.to(DEV), wl.W.to(DEV)
    idx, cnt = m.mosaic_mask_compact(tokens, wl.mask_id)            # count stays on the device
    out = _poisoned(L, V)
    m.mosaic_masked_logits_device_count(H, idx, W, cnt, max_rows=L, out=out)
    Mh = int(cnt.item())
    ref = m.mosaic_masked_logits(H, idx, W, M=Mh)
    torch.cuda.synchronize()
    assert torch.equal(out[:Mh], ref)
    assert bool((out[Mh:].float() == POISON).all())                 # rows past the count untouched
    want = oracle.mask_compact(wl.tokens, wl.mask_id)
    rows = sample_rows(Mh, 0, 12)
    assert_close(out[torch.as_tensor(rows, device=DEV)], oracle.masked_logits(wl.H, want[rows], wl.W), "devcount")


def test_count_is_clamped(m):
    wl = inputs.make_random(5, L=800, d=128, V=900, M=600, dtype="bf16")
    H, W = wl.H.to(DEV), wl.W.to(DEV)
    idx = torch.from_numpy(oracle.mask_compact(wl.tokens, wl.mask_id)).to(DEV)
    full = m.mosaic_masked_logits(H, idx, W)
    for c, rows in ((0, 0), (-5, 0), (1, 1), (300, 300), (500, 500), (600, 500), (10**6, 500)):
        out = _poisoned(500, wl.V)
        cnt = torch.tensor([c], dtype=torch.int32, device=DEV)
        m.mosaic_masked_logits_device_count(H, idx[:500], W, cnt, max_rows=500, out=out)
        torch.cuda.synchronize()
        assert torch.equal(out[:rows], full[:rows]), c
        assert bool((out[rows:].float() == POISON).all()), c


def test_llada_step_back_to_back(m):
    # the LLaDA-shaped step with no host read of the count: compaction then logits
    wl = inputs.make_workload("llada_step")
    tokens = wl.tokens.to(DEV)
    H, W = wl.H.to(DEV), wl.W.to(DEV)
    idx, cnt = m.mosaic_mask_compact(tokens, wl.mask_id)
    M = int(cnt.item())
    out = _poisoned(M, wl.V)
    for _ in range(3):                                               # repeated steps, same buffers
        m.mosaic_mask_compact(tokens, wl.mask_id, idx=idx, count=cnt)
        m.mosaic_masked_logits_device_count(H, idx, W, cnt, max_rows=M, out=out)
    ref = m.mosaic_masked_logits(H, idx, W, M=M)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)


def test_rejects_other_dtypes(m):
    wl = inputs.make_random(6, L=100, d=64, V=50, M=10, dtype="f32")
    idx = torch.arange(10, dtype=torch.int32, device=DEV)
    cnt = torch.tensor([10], dtype=torch.int32, device=DEV)
    with pytest.raises(m.MosaicError):
        m.mosaic_masked_logits_device_count(wl.H.to(DEV), idx, wl.W.to(DEV), cnt)


def test_compaction_and_logits_in_one_graph(m):
    # With the count read on the device, a step (compaction, then logits) has no host sync
    # and can be captured once and replayed; the mask changes between replays (eager work
    # and synchronisation in between), and every replay matches the eager calls.
    L, d, V = 3000, 256, 2000
    wl = inputs.make_random(91, L=L, d=d, V=V, M=2000, dtype="bf16")
    H, W = wl.H.to(DEV), wl.W.to(DEV)
    tokens = wl.tokens.to(DEV).clone()
    idx = torch.empty(L, dtype=torch.int32, device=DEV)
    cnt = torch.empty(1, dtype=torch.int32, device=DEV)
    out = _poisoned(L, V)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):                                     # eager run on the capture stream
        m.mosaic_mask_compact(tokens, wl.mask_id, idx=idx, count=cnt)
        m.mosaic_masked_logits_device_count(H, idx, W, cnt, max_rows=L, out=out)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        m.mosaic_mask_compact(tokens, wl.mask_id, idx=idx, count=cnt)
        m.mosaic_masked_logits_device_count(H, idx, W, cnt, max_rows=L, out=out)
    rng = np.random.default_rng(7)
    for ratio in (0.9, 0.3, 0.0, 0.65):
        t = rng.integers(0, wl.mask_id, size=L).astype(np.int32)
        t[rng.random(L) < ratio] = wl.mask_id
        tokens.copy_(torch.from_numpy(t).to(DEV))
        out.fill_(POISON)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        want = oracle.mask_compact(torch.from_numpy(t), wl.mask_id)
        M = int(cnt.item())
        assert M == want.size
        ref = m.mosaic_masked_logits(H, torch.from_numpy(want).to(DEV), W, M=M) if M else out[:0]
        torch.cuda.synchronize()
        assert torch.equal(out[:M], ref), ratio
        assert bool((out[M:].float() == POISON).all()), ratio


@pytest.mark.parametrize("L,d,V,store", [(900, 256, 5000, False), (3000, 192, 2100, True), (700, 64, 300, False),
                                         (17000, 128, 700, False)])
def test_consumer_count_from_compaction_equals_host_count(m, L, d, V, store):
    wl = inputs.make_random(L + d + V + 3, L=L, d=d, V=V, M=int(L * 0.7), dtype="bf16")
    tokens = wl.tokens.to(DEV)
    H, W = wl.H.to(DEV), wl.W.to(DEV)
    idx, cnt = m.mosaic_mask_compact(tokens, wl.mask_id)
    sent = (torch.full((L,), -3.0, device=DEV), torch.full((L,), -7, dtype=torch.int32, device=DEV),
            torch.full((L,), -5.0, device=DEV))
    out = _poisoned(L, V) if store else None
    rm, ra, rl, _ = m.mosaic_masked_logits_argmax_lse_device_count(H, idx, W, cnt, max_rows=L, out=out,
                                                                   row_max=sent[0], row_argmax=sent[1],
                                                                   row_lse=sent[2])
    M = int(cnt.item())
    hm, ha, hl, hout = m.mosaic_masked_logits_argmax_lse(H, idx, W, M=M, store_logits=store)
    torch.cuda.synchronize()
    assert torch.equal(rm[:M], hm) and torch.equal(ra[:M], ha) and torch.equal(rl[:M], hl)
    assert bool((rm[M:] == -3.0).all()) and bool((ra[M:] == -7).all()) and bool((rl[M:] == -5.0).all())
    if store:
        assert torch.equal(out[:M], hout) and bool((out[M:].float() == POISON).all())
    assert M == oracle.mask_compact(wl.tokens, wl.mask_id).size


def test_consumer_count_is_clamped(m):
    wl = inputs.make_random(17, L=800, d=128, V=900, M=600, dtype="bf16")
    H, W = wl.H.to(DEV), wl.W.to(DEV)
    idx = torch.from_numpy(oracle.mask_compact(wl.tokens, wl.mask_id)).to(DEV)
    fm, fa, fl, _ = m.mosaic_masked_logits_argmax_lse(H, idx[:500], W)
    for c, rows in ((0, 0), (-1, 0), (1, 1), (499, 499), (777, 500)):
        cnt = torch.tensor([c], dtype=torch.int32, device=DEV)
        ra = torch.full((500,), -7, dtype=torch.int32, device=DEV)
        _, ra, _, _ = m.mosaic_masked_logits_argmax_lse_device_count(H, idx[:500], W, cnt, max_rows=500, row_argmax=ra)
        torch.cuda.synchronize()
        assert torch.equal(ra[:rows], fa[:rows]), c
        assert bool((ra[rows:] == -7).all()), c


def test_compaction_and_consumer_in_one_graph(m):
    # The per-row consumer with the count read on the device, captured with the compaction in
    # one graph and replayed as the mask changes (eager work and synchronisation in between);
    # every replay equals the eager call that takes M from the host, bit for bit, and leaves
    # the rows at or past the count untouched.
    L, d, V = 2500, 192, 1700
    wl = inputs.make_random(93, L=L, d=d, V=V, M=1500, dtype="bf16")
    H, W = wl.H.to(DEV), wl.W.to(DEV)
    tokens = wl.tokens.to(DEV).clone()
    idx = torch.empty(L, dtype=torch.int32, device=DEV)
    cnt = torch.empty(1, dtype=torch.int32, device=DEV)
    rm = torch.empty(L, dtype=torch.float32, device=DEV)
    ra = torch.empty(L, dtype=torch.int32, device=DEV)
    rl = torch.empty(L, dtype=torch.float32, device=DEV)
    ws = torch.empty(max(16, m.mosaic_logits_argmax_lse_workspace_bytes(L, 0, V)), dtype=torch.uint8, device=DEV)

    def run():
        m.mosaic_mask_compact(tokens, wl.mask_id, idx=idx, count=cnt)
        m.mosaic_masked_logits_argmax_lse_device_count(H, idx, W, cnt, max_rows=L, row_max=rm, row_argmax=ra,
                                                       row_lse=rl, workspace=ws)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):                                     # eager run on the capture stream
        run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    rng = np.random.default_rng(11)
    for ratio in (0.8, 0.2, 0.0, 0.55):
        t = rng.integers(0, wl.mask_id, size=L).astype(np.int32)
        t[rng.random(L) < ratio] = wl.mask_id
        tokens.copy_(torch.from_numpy(t).to(DEV))
        for buf, val in ((rm, -3.0), (ra, -7), (rl, -5.0)):
            buf.fill_(val)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        want = oracle.mask_compact(torch.from_numpy(t), wl.mask_id)
        M = int(cnt.item())
        assert M == want.size
        if M:
            hm, ha, hl, _ = m.mosaic_masked_logits_argmax_lse(H, torch.from_numpy(want).to(DEV), W, M=M)
            torch.cuda.synchronize()
            assert torch.equal(rm[:M], hm) and torch.equal(ra[:M], ha) and torch.equal(rl[:M], hl), ratio
        assert bool((rm[M:] == -3.0).all()) and bool((ra[M:] == -7).all()) and bool((rl[M:] == -5.0).all()), ratio


def test_ragged_batch_count_from_csr(m):
    # A ragged batch, as the bench's ragged step runs it: the CSR compaction's last offset
    # (the batch's masked total) is the count the logits kernel and the consumer read.
    L, d, V = 6000, 256, 3000
    wl = inputs.make_random(97, L=L, d=d, V=V, M=3900, dtype="bf16", nseq=7)
    tokens, offs = wl.tokens.to(DEV), wl.seq_offsets.to(DEV)
    H, W = wl.H.to(DEV), wl.W.to(DEV)
    idx, idx_offsets = m.mosaic_mask_compact_batched(tokens, offs, wl.mask_id)
    cnt = idx_offsets[-1:]
    out = _poisoned(L, V)
    m.mosaic_masked_logits_device_count(H, idx, W, cnt, max_rows=L, out=out)
    rm, ra, rl, _ = m.mosaic_masked_logits_argmax_lse_device_count(H, idx, W, cnt, max_rows=L)
    M = int(cnt.item())
    want_idx, want_offs = oracle.mask_compact_batched(wl.tokens, wl.seq_offsets, wl.mask_id)
    assert M == want_idx.size and np.array_equal(idx_offsets.cpu().numpy(), want_offs)
    ref = m.mosaic_masked_logits(H, idx, W, M=M)
    hm, ha, hl, _ = m.mosaic_masked_logits_argmax_lse(H, idx, W, M=M)
    torch.cuda.synchronize()
    assert torch.equal(out[:M], ref) and bool((out[M:].float() == POISON).all())
    assert torch.equal(rm[:M], hm) and torch.equal(ra[:M], ha) and torch.equal(rl[:M], hl)
    rows = sample_rows(M, 0, 12)
    assert_close(out[torch.as_tensor(rows, device=DEV)], oracle.masked_logits(wl.H, want_idx[rows], wl.W), "ragged devcount")
