"""GPU parity of the encoder-chunk Q4_0 dequant-GEMM (matrix cores) against the CPU oracle."""
import numpy as np
import pytest
import torch

from streaming_speech_text_amd import synth
from tests.gpu_util import assert_close, dev, host, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def vx():
    from streaming_speech_text_amd import vox
    vox.lib()
    return vox


def _gemm(vx, w, xb, m, n, k, split=True):
    """split: pass the workspace the call asks for (K may be split over workgroups)."""
    y = torch.full((m, n), float("nan"), dtype=torch.float32, device="cuda")
    need = vx.q4_gemm_workspace(m, n, k) if split else 0
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device="cuda") if need else None
    vx.q4_gemm(dev(w), dev(xb), y, m=m, n=n, k=k, workspace=ws)
    return host(y)


@pytest.mark.parametrize("m", synth.ENCODER_M)
def test_gemm_encoder_chunk(vx, orc, m):
    for name, n, k in synth.ENCODER_LINEARS:
        say(f"gemm {name}: m={m} n={n} k={k}")
        w, xb = synth.gemm_inputs(synth.SEED_GEMM, m, n, k)
        ref = orc.q4_gemm(w, xb)
        assert_close(_gemm(vx, w, xb, m, n, k), ref, f"gemm {name} m={m}")
        if vx.q4_gemm_workspace(m, n, k):
            assert_close(_gemm(vx, w, xb, m, n, k, split=False), ref, f"gemm {name} m={m} unsplit")


def test_gemm_split_repeatable(vx):
    # the sliced path adds the partial tiles in a fixed order: two calls agree bit for bit, and a
    # call with a dirty, larger workspace agrees too
    m, n, k = 64, 1280, 5120
    assert vx.q4_gemm_workspace(m, n, k) > 0
    w, xb = synth.gemm_inputs(612, m, n, k)
    a = _gemm(vx, w, xb, m, n, k)
    b = _gemm(vx, w, xb, m, n, k)
    assert np.array_equal(a, b)
    y = torch.empty((m, n), dtype=torch.float32, device="cuda")
    big = torch.full((vx.q4_gemm_workspace(m, n, k) + 4096,), 0x7F, dtype=torch.uint8, device="cuda")
    vx.q4_gemm(dev(w), dev(xb), y, m=m, n=n, k=k, workspace=big)
    assert np.array_equal(host(y), a)


@pytest.mark.parametrize("m,n,k", [(200, 5120, 1280), (750, 5120, 1280), (16, 1280, 1280)])
def test_gemm_workspace_on_unsplit_shape(vx, orc, m, n, k):
    # a workspace handed to a call that does not split K must leave y as the result (regression:
    # the single-slice tiled launch once wrote its tile into the workspace)
    assert vx.q4_gemm_workspace(m, n, k) == 0
    w, xb = synth.gemm_inputs(614, m, n, k)
    y = torch.full((m, n), float("nan"), dtype=torch.float32, device="cuda")
    ws = torch.zeros((4 * m * n + 4096,), dtype=torch.uint8, device="cuda")
    vx.q4_gemm(dev(w), dev(xb), y, m=m, n=n, k=k, workspace=ws)
    assert_close(host(y), orc.q4_gemm(w, xb), f"gemm {m}x{n}x{k} with an unused workspace")


def test_gemm_small_workspace(vx):
    m, n, k = 64, 1280, 5120
    need = vx.q4_gemm_workspace(m, n, k)
    w, xb = synth.gemm_inputs(613, m, n, k)
    y = torch.empty((m, n), dtype=torch.float32, device="cuda")
    ws = torch.empty((need - 16,), dtype=torch.uint8, device="cuda")
    with pytest.raises(vx.VoxError) as e:
        vx.q4_gemm(dev(w), dev(xb), y, m=m, n=n, k=k, workspace=ws)
    assert e.value.status == vx.VOX_E_WORKSPACE


@pytest.mark.parametrize("m,n,k", [(1, 1280, 1280), (17, 100, 96), (63, 65, 32), (65, 1000, 5120), (130, 64, 2080),
                                   (3, 5, 64), (97, 77, 1280), (751, 130, 5120), (40, 1280, 5120), (49, 1283, 5120),
                                   (129, 1283, 1280), (200, 3072, 3072), (64, 1280, 3072), (100, 3072, 3072),
                                   (70, 1100, 3072)])
def test_gemm_ragged(vx, orc, m, n, k):
    w, xb = synth.gemm_inputs(600 + m, m, n, k)
    say(f"gemm ragged m={m} n={n} k={k}")
    assert_close(_gemm(vx, w, xb, m, n, k), orc.q4_gemm(w, xb), f"gemm ragged {m}x{n}x{k}")


@pytest.mark.parametrize("m,n,k", [(70, 96, 1280), (64, 1280, 5120), (300, 200, 1280), (257, 130, 5120),
                                   (750, 1280, 1280), (256, 3072, 3072), (260, 10300, 1280), (16, 1280, 5120),
                                   (750, 1280, 5120), (600, 2000, 3072), (200, 1283, 1280)])
def test_gemm_exact_dyadic(vx, orc, m, n, k):
    # small-integer activations and power-of-two scales: every product and partial sum is exact,
    # so the matrix-core result must equal the oracle bit for bit (also when K is split)
    g = synth.generator(610)
    w = synth.q4_matrix(g, n, k).reshape(n, k // 32, 18)
    e = g.integers(-3, 1, size=(n, k // 32)).astype(np.float64)
    w[:, :, 0:2] = (2.0 ** e).astype("<f2").view(np.uint8).reshape(n, k // 32, 2)
    w = w.reshape(n, -1)
    xi = g.integers(-4, 5, size=(m, k)).astype(np.float32)
    xb = synth.bf16_bits(xi)
    ref = orc.q4_gemm(w, xb)
    say(f"gemm exact dyadic m={m} n={n} k={k}")
    assert np.array_equal(_gemm(vx, w, xb, m, n, k).astype(np.float64), ref)
    if vx.q4_gemm_workspace(m, n, k):
        assert np.array_equal(_gemm(vx, w, xb, m, n, k, split=False).astype(np.float64), ref)


@pytest.mark.parametrize("m,n,k", [(200, 1280, 1280), (200, 1283, 1280), (129, 2600, 1280)])
def test_gemm_narrow_tiles(vx, orc, m, n, k):
    # 64 x 32 tiles at K = 1280 where 64 x 64 tiles would need K slices: one launch, no workspace
    assert vx.q4_gemm_workspace(m, n, k) == 0
    w, xb = synth.gemm_inputs(640 + m, m, n, k)
    say(f"gemm narrow tiles m={m} n={n} k={k}")
    assert_close(_gemm(vx, w, xb, m, n, k), orc.q4_gemm(w, xb), f"gemm narrow {m}x{n}x{k}")


@pytest.mark.parametrize("m,n,k", [(750, 5120, 1280), (770, 5120, 3072), (1023, 3850, 5120), (260, 10300, 1280),
                                   (750, 3840, 1280)])
def test_gemm_wide_ragged(vx, orc, m, n, k):
    # long chunks with many 128 x 128 tiles run the wide product unsplit: edges in both
    # dimensions, every K
    w, xb = synth.gemm_inputs(620 + m, m, n, k)
    say(f"gemm wide m={m} n={n} k={k}")
    assert vx.q4_gemm_workspace(m, n, k) == 0
    assert_close(_gemm(vx, w, xb, m, n, k), orc.q4_gemm(w, xb), f"gemm wide {m}x{n}x{k}")


@pytest.mark.parametrize("m,n,k,slices", [(750, 1280, 5120, 4), (1000, 1100, 5120, 4), (400, 3000, 5120, 2),
                                          (600, 2000, 3072, 2)])
def test_gemm_wide_k_slices(vx, orc, m, n, k, slices):
    # the wide product with K split over the grid (10, 20 and 12 stages per slice) and the slice
    # sum; without a workspace the same call runs unsplit on the tiled kernel
    assert vx.q4_gemm_workspace(m, n, k) == slices * m * n * 4
    w, xb = synth.gemm_inputs(630 + m, m, n, k)
    say(f"gemm wide sliced m={m} n={n} k={k}")
    ref = orc.q4_gemm(w, xb)
    assert_close(_gemm(vx, w, xb, m, n, k), ref, f"gemm wide sliced {m}x{n}x{k}")
    assert_close(_gemm(vx, w, xb, m, n, k, split=False), ref, f"gemm {m}x{n}x{k} without workspace")


def test_gemm_fused_qkv_equals_separate(vx, orc):
    # q, k and v as one product over the stacked weights (rows of a Q4_0 matrix are independent):
    # the same values as three calls, within the bound of the oracle for each
    for m in (16, 64, 750):
        ws_ = [synth.gemm_inputs(640 + i, m, 1280, 1280) for i in range(3)]
        xb = ws_[0][1]
        wqkv = np.concatenate([w for w, _ in ws_], axis=0)
        say(f"gemm fused qkv m={m}")
        got = _gemm(vx, wqkv, xb, m, 3840, 1280)
        for i, (w, _) in enumerate(ws_):
            assert_close(got[:, 1280 * i:1280 * (i + 1)], orc.q4_gemm(w, xb), f"fused qkv part {i} m={m}")


def test_gemm_wide_repeatable(vx):
    m, n, k = 750, 5120, 1280
    w, xb = synth.gemm_inputs(616, m, n, k)
    assert np.array_equal(_gemm(vx, w, xb, m, n, k), _gemm(vx, w, xb, m, n, k))
    # sliced: fixed slice order, also with a dirty, larger workspace
    m, n, k = 750, 1280, 5120
    w, xb = synth.gemm_inputs(617, m, n, k)
    a = _gemm(vx, w, xb, m, n, k)
    assert np.array_equal(a, _gemm(vx, w, xb, m, n, k))
    y = torch.empty((m, n), dtype=torch.float32, device="cuda")
    big = torch.full((vx.q4_gemm_workspace(m, n, k) + 4096,), 0x7F, dtype=torch.uint8, device="cuda")
    vx.q4_gemm(dev(w), dev(xb), y, m=m, n=n, k=k, workspace=big)
    assert np.array_equal(host(y), a)


def test_gemm_row_matches_gemv(vx):
    # one GEMM row equals the GEMV of that row's (bf16-valued) activations
    m, n, k = 5, 3072, 3072
    w, xb = synth.gemm_inputs(611, m, n, k)
    y = _gemm(vx, w, xb, m, n, k)
    xf = (xb.astype(np.uint32) << 16).view(np.float32)
    yv = torch.empty(n, dtype=torch.float32, device="cuda")
    vx.q4_gemv(dev(w), dev(np.ascontiguousarray(xf[2])), yv)
    assert_close(y[2], host(yv), "gemm row vs gemv", rtol=1e-5, atol=1e-5)


def test_gemm_errors(vx):
    w = torch.zeros(18 * 64, dtype=torch.uint8, device="cuda")
    x = torch.zeros(4, 64, dtype=torch.uint16, device="cuda")
    y = torch.zeros(4, 32, dtype=torch.float32, device="cuda")
    with pytest.raises(vx.VoxError) as e:
        vx.q4_gemm(w, x, y, m=4, n=32, k=48)
    assert e.value.status == vx.VOX_E_INVAL
    vx.q4_gemm(w, x, y, m=0, n=32, k=64)


@pytest.mark.parametrize("m,n,k", [(5, 1283, 1280), (11, 77, 3072), (16, 3840, 1280), (2, 1280, 3072), (16, 1, 3072),
                                   (1, 5120, 1280), (13, 2000, 3072), (16, 1280, 5120), (3, 77, 5120), (40, 1283, 1280),
                                   (17, 77, 1280), (64, 3840, 1280), (40, 1000, 3072)])
def test_gemm_skinny(vx, orc, m, n, k):
    # at most 64 rows at K = 1280 / 3072 and 16 at K = 5120 (16-row tiles): the whole K of a
    # 16-column tile staged in LDS;
    # ragged column counts (the last tile repeats the last weight row) and rows below 16
    w, xb = synth.gemm_inputs(620 + m, m, n, k)
    assert vx.q4_gemm_workspace(m, n, k) == 0
    say(f"gemm skinny m={m} n={n} k={k}")
    assert_close(_gemm(vx, w, xb, m, n, k), orc.q4_gemm(w, xb), f"gemm skinny {m}x{n}x{k}")


@pytest.mark.parametrize("m,n,k", [(7, 130, 3072), (16, 1283, 1280), (3, 64, 1280), (9, 200, 5120), (33, 200, 1280)])
def test_gemm_skinny_exact_dyadic(vx, orc, m, n, k):
    # exact inputs: the skinny kernel's sum (eight waves' partial tiles added in order) is exact
    g = synth.generator(621)
    w = synth.q4_matrix(g, n, k).reshape(n, k // 32, 18)
    e = g.integers(-3, 1, size=(n, k // 32)).astype(np.float64)
    w[:, :, 0:2] = (2.0 ** e).astype("<f2").view(np.uint8).reshape(n, k // 32, 2)
    w = w.reshape(n, -1)
    xb = synth.bf16_bits(g.integers(-4, 5, size=(m, k)).astype(np.float32))
    assert np.array_equal(_gemm(vx, w, xb, m, n, k).astype(np.float64), orc.q4_gemm(w, xb))


@pytest.mark.parametrize("k", [1024, 1056, 1280, 1312])
def test_gemm_small_kernel_block_ranges(vx, orc, k):
    # the split-K-over-waves kernel keeps all five blocks of a wave in flight when a wave has
    # exactly five (K = 1280, and 1056 where some waves have four); others run four at a time
    m, n = 16, 200
    w, xb = synth.gemm_inputs(615, m, n, k)
    assert vx.q4_gemm_workspace(m, n, k) == 0
    assert_close(_gemm(vx, w, xb, m, n, k, split=False), orc.q4_gemm(w, xb), f"gemm {m}x{n}x{k} small kernel")
