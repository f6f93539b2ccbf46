"""GPU gather-GEMM vs the CPU oracle at sizes the oracle finishes in seconds.

Shapes span several 256 x 256 tiles with ragged tails in M and V, odd and even
K-tile counts, vocabulary sizes that are not multiples of 4 (scalar stores), the
d % 64 != 0 kernel, all three dtype pairs, and row chunking.  Exact pins (integer
inputs, one-hot weights) are compared bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle
from mask_only_logits_amd import inputs
from tests.helpers import assert_close, bf16_rne

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
TD = {"bf16": torch.bfloat16, "f32": torch.float32}


@pytest.fixture(scope="module")
def m():
    from mask_only_logits_amd import mosaic
    return mosaic


def _gpu_idx(wl):
    idx = oracle.mask_compact(wl.tokens, wl.mask_id)
    return idx, torch.from_numpy(idx).to(DEV)


CASES = [
    # (in, out, L, d, V, M, chunk_rows)
    ("bf16", "bf16", 700, 512, 1000, 600, 0),
    ("bf16", "bf16", 700, 512, 1000, 600, 256),
    ("bf16", "bf16", 700, 512, 1000, 600, 77),
    ("bf16", "bf16", 2000, 4096, 1500, 300, 0),
    ("bf16", "bf16", 900, 3584, 700, 513, 200),
    ("bf16", "bf16", 400, 64, 1001, 257, 0),        # one K tile; V % 4 != 0
    ("bf16", "bf16", 400, 128, 257, 256, 0),        # two K tiles
    ("bf16", "bf16", 400, 192, 255, 255, 0),        # three K tiles (odd)
    ("bf16", "bf16", 300, 64, 3, 1, 0),             # a single row, tiny vocabulary
    ("bf16", "bf16", 300, 320, 513, 2, 0),
    ("bf16", "bf16", 300, 72, 300, 100, 0),         # d % 32 != 0 kernel
    ("bf16", "bf16", 400, 96, 1000, 300, 0),        # d % 64 != 0, d % 32 == 0: persistent BK-32 kernel
    ("bf16", "f32", 300, 160, 513, 70, 33),
    ("bf16", "bf16", 300, 8, 65, 33, 10),
    ("bf16", "f32", 700, 512, 1000, 600, 0),
    ("bf16", "f32", 300, 136, 129, 70, 0),
    ("bf16", "f32", 300, 256, 130, 70, 0),
    ("f32", "f32", 256, 256, 1024, 128, 0),
    ("f32", "f32", 300, 100, 131, 77, 30),
    ("f32", "f32", 70, 4, 1, 1, 0),
]


@pytest.mark.parametrize("dt_in,dt_out,L,d,V,M,C", CASES)
def test_parity_random(m, dt_in, dt_out, L, d, V, M, C):
    wl = inputs.make_random(L * 31 + d * 7 + V + M, L=L, d=d, V=V, M=M, dtype=dt_in, std_w=0.02)
    idx, idx_d = _gpu_idx(wl)
    out = m.mosaic_masked_logits(wl.H.to(DEV), idx_d, wl.W.to(DEV), chunk_rows=C, out_dtype=TD[dt_out])
    torch.cuda.synchronize()
    assert out.shape == (M, V) and out.dtype == TD[dt_out]
    assert_close(out, oracle.masked_logits(wl.H, idx, wl.W), f"{dt_in}->{dt_out} {L},{d},{V},{M},{C}")


LOWM_CASES = [
    # (out, L, d, V, M): the low-M streaming kernel (M <= 64, d % 64 == 0)
    ("bf16", 500, 3584, 5000, 20), ("bf16", 300, 64, 3, 1), ("bf16", 300, 128, 129, 2),
    ("bf16", 300, 192, 1001, 31), ("bf16", 300, 256, 777, 32), ("bf16", 300, 256, 4097, 33),
    ("bf16", 300, 512, 300, 63), ("bf16", 300, 512, 2000, 64), ("f32", 300, 256, 1031, 17),
    ("f32", 300, 320, 515, 50),
    # several 32-row blocks per wave; at V = 131584 the 1024 waves own 128 or 129 rows, so
    # the shorter ones run a padding block
    ("bf16", 300, 64, 131584, 20), ("bf16", 300, 128, 131584, 40), ("f32", 300, 64, 40000, 64),
    # more than 8 blocks per wave: the held results go out in two bursts
    ("bf16", 300, 64, 300000, 20), ("f32", 300, 64, 300000, 40),
]


@pytest.mark.parametrize("variant", [20])
@pytest.mark.parametrize("dt_out,L,d,V,M", LOWM_CASES)
def test_parity_lowm(m, lib_env, variant, dt_out, L, d, V, M):
    # the low-M streaming kernel (W streamed once, a workgroup-shared H tile)
    lib_env("MOSAIC_TUNE", f"variant={variant}")
    assert m.mosaic_logits_variant(M, V, d, torch.bfloat16, TD[dt_out]) == variant
    wl = inputs.make_random(L + d + V + M, L=L, d=d, V=V, M=M, dtype="bf16")
    idx, idx_d = _gpu_idx(wl)
    out = m.mosaic_masked_logits(wl.H.to(DEV), idx_d, wl.W.to(DEV), out_dtype=TD[dt_out])
    torch.cuda.synchronize()
    assert_close(out, oracle.masked_logits(wl.H, idx, wl.W), f"lowm {d},{V},{M}")


# every bf16 MFMA kernel form the library can select: persistent BK-32 (11), 8-wave tiled
# (12), persistent 32 x 32 x 16 (16), persistent 16 x 16 x 32 with every wave requesting K
# tiles (19) or one wave per SIMD (21; 22 with a third W stage), low-M streaming (20)
BF16_MFMA_VARIANTS = (11, 12, 16, 19, 20, 21, 22)


@pytest.mark.parametrize("M,d,V,out", [(20, 3584, 5000, "bf16"), (64, 256, 1001, "f32"), (700, 512, 1000, "bf16"),
                                       (1, 64, 300, "bf16"), (1000, 192, 40001, "bf16"), (777, 128, 30000, "f32"),
                                       (600, 64, 70000, "bf16"), (600, 1280, 70000, "bf16"),
                                       # whole tiles (rows and V multiples of 256), several per workgroup
                                       (1024, 512, 65536, "bf16"), (1024, 64, 65536, "bf16"),
                                       (2048, 128, 32768, "bf16"),
                                       # low-M shapes with several blocks per wave
                                       (20, 64, 131584, "bf16"), (64, 128, 40000, "f32"), (20, 64, 300000, "bf16"),
                                       # 65 row tiles: a full super-group of 64 (XCDs side by side) + 1
                                       (16500, 128, 2100, "bf16")])
def test_bf16_variants_bit_identical(m, lib_env, M, d, V, out):
    # every bf16 MFMA variant accumulates each output in the same MFMA k order
    wl = inputs.make_random(M + d + V, L=max(M, 300), d=d, V=V, M=M, dtype="bf16")
    _, idx_d = _gpu_idx(wl)
    H, W = wl.H.to(DEV), wl.W.to(DEV)
    ref = m.mosaic_masked_logits(H, idx_d, W, out_dtype=TD[out])
    for v in BF16_MFMA_VARIANTS:
        if v == 20 and M > 64:
            continue
        lib_env("MOSAIC_TUNE", f"variant={v}")
        if out == "bf16" or v not in (16, 19, 21, 22):  # the persistent deferred-store kernels write bf16 only
            assert m.mosaic_logits_variant(M, V, d, torch.bfloat16, TD[out]) == v
        got = m.mosaic_masked_logits(H, idx_d, W, out_dtype=TD[out])
        torch.cuda.synchronize()
        assert torch.equal(got, ref), v
    lib_env("MOSAIC_TUNE", None)


@pytest.mark.parametrize("group_m", [1, 2, 3, 8, 16])
def test_tile_order_group_sizes(m, lib_env, group_m):
    # The persistent kernels' tile lists (full super-groups of 8 * group_m row tiles with
    # the XCDs side by side, then contiguous runs) must cover every tile once whatever the
    # group size; the logits do not depend on it.
    wl = inputs.make_random(31 + group_m, L=16600, d=128, V=1300, M=16500, dtype="bf16")
    idx, idx_d = _gpu_idx(wl)
    H, W = wl.H.to(DEV), wl.W.to(DEV)
    ref = m.mosaic_masked_logits(H, idx_d, W)
    lib_env("MOSAIC_TUNE", f"group_m={group_m}")
    got = m.mosaic_masked_logits(H, idx_d, W)
    torch.cuda.synchronize()
    lib_env("MOSAIC_TUNE", None)
    assert torch.equal(got, ref)
    rows = np.random.default_rng(group_m).choice(16500, 40, replace=False)
    assert_close(got[torch.from_numpy(rows).to(DEV)], oracle.masked_logits(wl.H, idx[rows], wl.W), "group")


@pytest.mark.parametrize("d,V,M", [(4096, 1000, 300), (512, 1001, 600), (72, 100, 50)])
def test_exact_integers_bit_exact(m, d, V, M):
    L = M + 50
    H = inputs.integer_valued(d + 1, (L, d))
    W = inputs.integer_valued(d + 2, (V, d))
    idx = np.sort(np.random.default_rng(d).choice(L, M, replace=False)).astype(np.int32)
    out = m.mosaic_masked_logits(H.to(DEV), torch.from_numpy(idx).to(DEV), W.to(DEV))
    out32 = m.mosaic_masked_logits(H.to(DEV), torch.from_numpy(idx).to(DEV), W.to(DEV), out_dtype=torch.float32)
    torch.cuda.synchronize()
    ref = oracle.masked_logits(H, idx, W)           # exact integers (|x| <= 4d < 2^24)
    assert np.array_equal(out32.cpu().numpy().astype(np.float64), ref)
    assert torch.equal(out.cpu(), bf16_rne(ref))


@pytest.mark.parametrize("d,V", [(256, 1000), (4096, 700), (64, 5)])
def test_one_hot_weights_bit_exact(m, d, V):
    wl = inputs.make_random(5 + d, L=500, d=d, V=V, M=333, dtype="bf16")
    idx, idx_d = _gpu_idx(wl)
    W = inputs.one_hot_rows(V, d)
    out = m.mosaic_masked_logits(wl.H.to(DEV), idx_d, W.to(DEV))
    torch.cuda.synchronize()
    want = wl.H[torch.from_numpy(idx).long()][:, torch.arange(V) % d]
    assert torch.equal(out.cpu(), want)


def test_unsorted_and_repeated_rows(m):
    wl = inputs.make_random(77, L=300, d=256, V=600, M=10, dtype="bf16")
    idx = np.array([299, 0, 5, 5, 5, 17, 299, 3] * 40, np.int32)
    out = m.mosaic_masked_logits(wl.H.to(DEV), torch.from_numpy(idx).to(DEV), wl.W.to(DEV))
    torch.cuda.synchronize()
    assert_close(out, oracle.masked_logits(wl.H, idx, wl.W), "unsorted")
    o = out.cpu()
    assert torch.equal(o[2], o[3]) and torch.equal(o[0], o[6])


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_chunked_equals_unchunked_bit_exact(m, dt):
    wl = inputs.make_random(99, L=1500, d=256, V=900, M=1100, dtype=dt)
    _, idx_d = _gpu_idx(wl)
    H, W = wl.H.to(DEV), wl.W.to(DEV)
    ref = m.mosaic_masked_logits(H, idx_d, W)
    for C in (1, 63, 64, 255, 256, 257, 259, 1000, 1040, 1099, 1100, 5000, -1):   # 259, 1040: low-M last chunk
        got = m.mosaic_masked_logits(H, idx_d, W, chunk_rows=C)
        assert torch.equal(got, ref), C
    # streaming use: one call per chunk into a reused buffer
    C = 300
    buf = torch.empty((C, wl.V), dtype=ref.dtype, device=DEV)
    for k in range(m.mosaic_num_chunks(1100, C)):
        r0, r1 = k * C, min(1100, (k + 1) * C)
        m.mosaic_masked_logits(H, idx_d[r0:r1], W, out=buf[: r1 - r0])
        assert torch.equal(buf[: r1 - r0], ref[r0:r1]), k


def test_permutation_and_scaling_invariants(m):
    wl = inputs.make_random(7, L=800, d=512, V=700, M=600, dtype="bf16")
    idx, idx_d = _gpu_idx(wl)
    H, W = wl.H.to(DEV), wl.W.to(DEV)
    ref = m.mosaic_masked_logits(H, idx_d, W)
    perm = torch.randperm(600, generator=torch.Generator().manual_seed(0))
    got = m.mosaic_masked_logits(H, idx_d[perm.to(DEV)].contiguous(), W)
    assert torch.equal(got, ref[perm.to(DEV)])
    got2 = m.mosaic_masked_logits(H, idx_d, (W.float() * 2).to(torch.bfloat16))
    assert torch.equal(got2, (ref.float() * 2).to(torch.bfloat16))


def test_deterministic(m):
    wl = inputs.make_random(8, L=1000, d=1024, V=1300, M=700, dtype="bf16")
    _, idx_d = _gpu_idx(wl)
    H, W = wl.H.to(DEV), wl.W.to(DEV)
    a = m.mosaic_masked_logits(H, idx_d, W)
    b = m.mosaic_masked_logits(H, idx_d, W)
    assert torch.equal(a, b)


def test_zero_rows_leave_out_untouched(m):
    wl = inputs.make_random(9, L=100, d=64, V=50, M=10, dtype="bf16")
    _, idx_d = _gpu_idx(wl)
    poison = torch.full((10, 50), 7.0, dtype=torch.bfloat16, device=DEV)
    m.mosaic_masked_logits(wl.H.to(DEV), idx_d, wl.W.to(DEV), M=0, out=poison)
    torch.cuda.synchronize()
    assert bool((poison == 7.0).all())


def test_rejected_call_leaves_out_untouched(m):
    wl = inputs.make_random(10, L=100, d=64, V=50, M=10, dtype="bf16")
    _, idx_d = _gpu_idx(wl)
    poison = torch.full((10, 50), 7.0, dtype=torch.bfloat16, device=DEV)
    H = wl.H.to(DEV)
    with pytest.raises(m.MosaicError):
        m.mosaic_masked_logits(H[:, :60].contiguous(), idx_d, wl.W.to(DEV)[:, :60].contiguous().view(-1)[: 50 * 60]
                               .view(50, 60), out=poison)   # d = 60 is not a multiple of 8
    torch.cuda.synchronize()
    assert bool((poison == 7.0).all())
