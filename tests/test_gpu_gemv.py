"""GPU parity of Q4_0 dequantisation and the Q4_0 GEMV against the CPU oracle."""
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


def _all_finite_scale_blocks():
    dbits = np.array([h for h in range(65536) if ((h >> 10) & 31) != 31], dtype=np.uint16)
    blocks = np.zeros((dbits.size, 18), np.uint8)
    blocks[:, 0] = dbits & 0xFF
    blocks[:, 1] = dbits >> 8
    codes = np.arange(16, dtype=np.uint8)
    blocks[:, 2:] = codes | ((15 - codes) << 4)
    return blocks


def test_dequant_bit_exact(vx, orc):
    for name, blocks in [("all finite scales x all codes", _all_finite_scale_blocks()),
                         ("random blocks", synth.q4_matrix(synth.generator(51), 1000, 3072).reshape(-1, 18))]:
        say(f"dequant: {name} ({blocks.shape[0]} blocks)")
        w = dev(blocks.reshape(-1))
        out = torch.empty(blocks.shape[0] * 32, dtype=torch.float32, device="cuda")
        vx.q4_dequant(w, out)
        got = host(out)
        ref = orc.q4_dequant(blocks)
        assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), name
    # odd count and an unaligned source
    blocks = synth.q4_matrix(synth.generator(52), 1, 32 * 77).reshape(-1, 18)
    raw = torch.zeros(blocks.size + 3, dtype=torch.uint8, device="cuda")
    raw[3:] = dev(blocks.reshape(-1))
    out = torch.empty(77 * 32, dtype=torch.float32, device="cuda")
    vx.q4_dequant(raw[3:], out)
    assert np.array_equal(host(out).view(np.uint32), orc.q4_dequant(blocks).view(np.uint32))
    vx.q4_dequant(raw[3:], out, n_blocks=0)   # no-op


def _gemv_case(vx, orc, n, k, seed, what):
    say(f"gemv {what}: n={n} k={k} seed={seed}")
    w, x = synth.gemv_inputs(seed, n, k)
    y = torch.full((n,), float("nan"), dtype=torch.float32, device="cuda")
    vx.q4_gemv(dev(w), dev(x), y)
    got = host(y)
    ref = orc.q4_gemv(w, x)
    assert_close(got, ref, f"gemv {what} n={n} k={k}")
    return got


def test_gemv_single_3072(vx, orc):
    _gemv_case(vx, orc, 3072, 3072, synth.SEED_GEMV, "3072x3072")


def test_gemv_layer_linears(vx, orc):
    for i, (name, (n, k)) in enumerate(synth.LAYER_LINEARS.items()):
        _gemv_case(vx, orc, n, k, 100 * synth.SEED_LAYER + i, name)


def test_gemv_lm_head_shape(vx, orc):
    _gemv_case(vx, orc, 131072, 3072, 61, "lm-head")


@pytest.mark.parametrize("k", [3072, 4096, 9216, 1280, 5120])
@pytest.mark.parametrize("n", [1, 3, 17, 65, 1000, 4097])
def test_gemv_ragged_rows(vx, orc, n, k):
    _gemv_case(vx, orc, n, k, 7000 + n + k, "ragged")


def test_gemv_encoder_linears(vx, orc):
    # the encoder's linears (width 1280, feed-forward 5120) at one activation vector: the tiled
    # path at K = 1280 (16-row tiles, quad reductions) and K = 5120
    for i, (name, n, k) in enumerate(synth.ENCODER_LINEARS):
        _gemv_case(vx, orc, n, k, 8100 + i, f"encoder {name}")


@pytest.mark.parametrize("k", [32, 96, 1312, 2080])
def test_gemv_generic_widths(vx, orc, k):
    _gemv_case(vx, orc, 77, k, 8000 + k, "generic-k")


def test_gemv_unaligned_pointers(vx, orc):
    n, k = 300, 3072
    w, x = synth.gemv_inputs(91, n, k)
    raw = torch.zeros(w.size + 2, dtype=torch.uint8, device="cuda")
    raw[2:] = dev(w.reshape(-1))
    xr = torch.zeros(k + 1, dtype=torch.float32, device="cuda")
    xr[1:] = dev(x)
    y = torch.empty(n, dtype=torch.float32, device="cuda")
    vx.q4_gemv(raw[2:], xr[1:], y, n=n, k=k)
    assert_close(host(y), orc.q4_gemv(w, x), "gemv unaligned")


def test_gemv_exact_dyadic(vx, orc):
    # power-of-two scales and small integer activations: every partial sum is exact in fp32,
    # so the GPU must agree with the oracle bit for bit whatever the summation order
    for n, k in [(64, 3072), (40, 4096), (12, 9216), (9, 1280), (33, 1280), (21, 5120), (9, 1312)]:
        g = synth.generator(92, n, k)
        w = synth.q4_matrix(g, n, k).reshape(n, k // 32, 18)
        e = g.integers(-3, 1, size=(n, k // 32)).astype(np.float64)
        w[:, :, 0:2] = (2.0 ** e).astype("<f2").view(np.uint8).reshape(n, k // 32, 2)
        w = w.reshape(n, -1)
        x = g.integers(-3, 4, size=k).astype(np.float32)
        y = torch.empty(n, dtype=torch.float32, device="cuda")
        say(f"gemv exact dyadic n={n} k={k}")
        vx.q4_gemv(dev(w), dev(x), y)
        assert np.array_equal(host(y).astype(np.float64), orc.q4_gemv(w, x))


def test_gemv_deterministic(vx):
    w, x = synth.gemv_inputs(93, 18432, 3072)
    wd, xd = dev(w), dev(x)
    a = torch.empty(18432, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    vx.q4_gemv(wd, xd, a)
    vx.q4_gemv(wd, xd, b)
    assert torch.equal(a, b)


def test_gemv_empty_and_errors(vx):
    w = torch.zeros(18 * 4, dtype=torch.uint8, device="cuda")
    x = torch.zeros(128, dtype=torch.float32, device="cuda")
    y = torch.zeros(1, dtype=torch.float32, device="cuda")
    vx.q4_gemv(w, x, y, n=0, k=128)
    with pytest.raises(vx.VoxError) as e:
        vx.q4_gemv(w, x, y, n=1, k=100)
    assert e.value.status == vx.VOX_E_INVAL
