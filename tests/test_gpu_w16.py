"""GPU parity of the GEMV over 16-bit weights (bf16 and fp16) against the CPU oracle."""
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


def _gemv(vx, w, x, fmt):
    n = w.shape[0]
    y = torch.full((n,), float("nan"), dtype=torch.float32, device="cuda")
    vx.w16_gemv(dev(w), dev(x), y, fmt)
    return host(y)


@pytest.mark.parametrize("fmt", ["bf16", "f16"])
@pytest.mark.parametrize("n,k", [(3072, 3072), (4096, 3072), (9216, 3072), (3072, 9216), (131072, 3072)])
def test_w16_gemv_decoder_shapes(vx, orc, fmt, n, k):
    say(f"w16 gemv {fmt} {n}x{k}")
    w, x = synth.w16_gemv_inputs(synth.SEED_W16, n, k, fmt)
    assert_close(_gemv(vx, w, x, fmt), orc.w16_gemv(w, x, fmt), f"w16 {fmt} {n}x{k}")


@pytest.mark.parametrize("fmt", ["bf16", "f16"])
@pytest.mark.parametrize("n,k", [(1, 8), (7, 8), (1001, 1000), (5, 4104), (130, 520), (33, 4096), (3, 8200)])
def test_w16_gemv_ragged(vx, orc, fmt, n, k):
    w, x = synth.w16_gemv_inputs(900 + n, n, k, fmt)
    assert_close(_gemv(vx, w, x, fmt), orc.w16_gemv(w, x, fmt), f"w16 {fmt} ragged {n}x{k}")


@pytest.mark.parametrize("fmt", ["bf16", "f16"])
def test_w16_gemv_exact_dyadic(vx, orc, fmt):
    # small integers times powers of two, small-integer activations: every product and partial sum
    # is exact in fp32, so the result must equal the oracle bit for bit
    g = synth.generator(910)
    n, k = 257, 3072
    wi = g.integers(-8, 9, size=(n, k)).astype(np.float32) * np.float32(2.0) ** g.integers(-6, 1, size=(n, k))
    bits = synth.bf16_bits(wi) if fmt == "bf16" else wi.astype(np.float16).view(np.uint16)
    x = g.integers(-5, 6, size=k).astype(np.float32)
    assert np.array_equal(_gemv(vx, bits, x, fmt).astype(np.float64), orc.w16_gemv(bits, x, fmt))


def test_w16_gemv_errors(vx):
    w = torch.zeros(4, 12, dtype=torch.uint16, device="cuda")
    x = torch.zeros(12, dtype=torch.float32, device="cuda")
    y = torch.zeros(4, dtype=torch.float32, device="cuda")
    with pytest.raises(vx.VoxError) as e:
        vx.w16_gemv(w, x, y, "bf16")
    assert e.value.status == vx.VOX_E_INVAL
