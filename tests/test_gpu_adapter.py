"""GPU parity of the encoder-to-decoder adapter (a Q4_0 linear, GELU, a Q4_0 linear, on the matrix
cores) against the CPU oracle."""
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


def _adapter(vx, w1, w2, xb, n_out, extra=0, fill=0xFF):
    m, k = xb.shape
    n_mid = w1.shape[0]
    y = torch.full((m, n_out), float("nan"), dtype=torch.float32, device="cuda")
    need = vx.adapter_workspace(m, k, n_mid, n_out)
    assert need > 0
    ws = torch.full((need + extra,), fill, dtype=torch.uint8, device="cuda")
    vx.adapter(dev(w1), dev(w2), dev(xb), y, ws, m=m, k=k, n_mid=n_mid, n_out=n_out)
    return host(y)


@pytest.mark.parametrize("m", synth.ADAPTER_M)
def test_adapter_chunk_rows(vx, orc, m):
    # the adapter at the model's shape for the rows of one encoder chunk (M / 4)
    k, n_mid, n_out = synth.ADAPTER
    say(f"adapter m={m} {k}->{n_mid}->{n_out}")
    w1, w2, xb = synth.adapter_inputs(synth.SEED_ADAPTER, m, k, n_mid, n_out)
    assert_close(_adapter(vx, w1, w2, xb, n_out), orc.adapter(w1, w2, xb), f"adapter m={m}")


@pytest.mark.parametrize("m,k,n_mid,n_out", [(1, 1280, 1280, 64), (17, 1280, 3072, 100), (65, 3072, 1280, 33),
                                             (130, 5120, 1280, 1283), (3, 5120, 3072, 7), (200, 1280, 1280, 1280),
                                             (16, 3072, 3072, 1283), (11, 5120, 1280, 100), (64, 5120, 3072, 1283)])
def test_adapter_ragged(vx, orc, m, k, n_mid, n_out):
    say(f"adapter ragged m={m} {k}->{n_mid}->{n_out}")
    w1, w2, xb = synth.adapter_inputs(700 + m, m, k, n_mid, n_out)
    assert_close(_adapter(vx, w1, w2, xb, n_out), orc.adapter(w1, w2, xb), f"adapter {m} {k}->{n_mid}->{n_out}")


@pytest.mark.parametrize("m,k,n_mid,n_out", [(190, 5120, 3072, 3000), (520, 5120, 1280, 2000),
                                             (800, 1280, 3072, 3072), (190, 5120, 3072, 3456),
                                             (400, 1280, 3072, 2560), (800, 5120, 1280, 3000),
                                             (400, 3072, 3072, 640)])
def test_adapter_wide(vx, orc, m, k, n_mid, n_out):
    # longer chunks through the 128 x 128 tile product: GELU output with K split over the grid
    # (through the slice sum) and unsplit (stored by the product), pair input split and unsplit;
    # stages per workgroup: GELU output 10 (4 slices, unsplit) and 12 (2 slices), pair input 12, 16,
    # 24 (4, 3, 2 slices), 20 and 48 (unsplit)
    say(f"adapter wide m={m} {k}->{n_mid}->{n_out}")
    w1, w2, xb = synth.adapter_inputs(710 + m, m, k, n_mid, n_out)
    assert_close(_adapter(vx, w1, w2, xb, n_out), orc.adapter(w1, w2, xb), f"adapter {m} {k}->{n_mid}->{n_out}")


@pytest.mark.parametrize("m,n_mid", [(40, 1280), (9, 1280), (187, 3072)])
def test_adapter_gelu_between_the_linears(vx, orc, m, n_mid):
    # W2 = identity (code 9 on the diagonal, 8 elsewhere, scale 1): Y = GELU(X W1^T).  The GELU
    # value travels as a bf16 pair within 2^-18 of its fp32 value, so this holds well inside the
    # usual bound (m = 9: both products through the kernel for at most 16 rows; m = 187: through
    # the 128 x 128 tile product).
    k = 5120
    g = synth.generator(720)
    w1 = synth.q4_matrix(g, n_mid, k)
    xb = synth.bf16_normal(g, (m, k))
    eye = np.zeros((n_mid, n_mid // 32, 18), np.uint8)
    eye[:, :, 0:2] = np.frombuffer(np.float16(1.0).tobytes(), np.uint8)
    codes = np.full((n_mid, n_mid), 8, np.uint8)
    codes[np.arange(n_mid), np.arange(n_mid)] = 9
    for b in range(n_mid // 32):
        c = codes[:, 32 * b:32 * b + 32]
        eye[:, b, 2:] = c[:, :16] | (c[:, 16:] << 4)
    got = _adapter(vx, w1, eye.reshape(n_mid, -1), xb, n_mid)
    h = orc.q4_gemm(w1, xb)
    ref = orc.gelu(h)
    assert_close(got, ref, "adapter with identity W2", rtol=1e-4, atol=1e-5)
    assert (h < -2).any() and np.all(np.abs(got[h < -2]) < 0.1)


@pytest.mark.parametrize("m", [16, 187])
def test_adapter_repeatable(vx, m):
    # fixed summation order: two calls agree bit for bit, also with a larger, differently dirty workspace
    k, n_mid, n_out = synth.ADAPTER
    w1, w2, xb = synth.adapter_inputs(721, m, k, n_mid, n_out)
    a = _adapter(vx, w1, w2, xb, n_out)
    b = _adapter(vx, w1, w2, xb, n_out, extra=4096, fill=0x3C)
    assert np.array_equal(a, b)


def test_adapter_errors(vx):
    m, k, n_mid, n_out = 4, 1280, 1280, 64
    w1, w2, xb = synth.adapter_inputs(722, m, k, n_mid, n_out)
    y = torch.empty((m, n_out), dtype=torch.float32, device="cuda")
    need = vx.adapter_workspace(m, k, n_mid, n_out)
    ws = torch.empty((need - 16,), dtype=torch.uint8, device="cuda")
    with pytest.raises(vx.VoxError) as e:
        vx.adapter(dev(w1), dev(w2), dev(xb), y, ws, m=m, k=k, n_mid=n_mid, n_out=n_out)
    assert e.value.status == vx.VOX_E_WORKSPACE
    ws = torch.empty((need,), dtype=torch.uint8, device="cuda")
    with pytest.raises(vx.VoxError) as e:   # n_mid without a compiled stage sequence
        vx.adapter(dev(w1), dev(w2), dev(xb), y, ws, m=m, k=k, n_mid=2048, n_out=n_out)
    assert e.value.status == vx.VOX_E_UNSUPPORTED
