"""GPU parity of the encoder's chunk self-attention (causal, sliding window, fp32 matrix cores)
against the CPU oracle."""
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


def _run(vx, q, k, v, n_heads, window, extra=0):
    m, width = q.shape
    n_ctx = k.shape[0] - m
    out = torch.full((m, width), float("nan"), dtype=torch.float32, device="cuda")
    need = vx.enc_attn_workspace(m, n_ctx, n_heads, width // n_heads, window)
    ws = torch.full((need + extra,), 0xFF, dtype=torch.uint8, device="cuda") if need + extra else None
    vx.enc_attn(dev(q), dev(k), dev(v), out, n_heads, window, workspace=ws)
    return host(out)


@pytest.mark.parametrize("m", synth.ENCODER_M)
def test_enc_attn_chunk(vx, orc, m):
    # steady state: a full window of earlier rows (749) before the chunk
    n_ctx = synth.ENC_WINDOW - 1
    say(f"enc_attn m={m} n_ctx={n_ctx}")
    q, k, v = synth.enc_attention_inputs(synth.SEED_ENC_ATTN, m, n_ctx)
    got = _run(vx, q, k, v, synth.ENC_HEADS, synth.ENC_WINDOW)
    assert_close(got, orc.enc_attn(q, k, v, synth.ENC_HEADS, synth.ENC_WINDOW), f"enc_attn m={m}")


@pytest.mark.parametrize("m,n_ctx,heads,hd,window", [
    (1, 0, 32, 40, 750),        # the first frame of a stream: one key
    (37, 0, 32, 40, 750),       # stream start: no earlier rows, window not yet full
    (200, 300, 32, 40, 750),    # earlier rows fewer than the window
    (100, 20, 4, 40, 50),       # window shorter than the chunk
    (5, 3, 2, 40, 4),
    (17, 749, 3, 44, 750),      # head size 44, ragged query block
    (33, 10, 5, 8, 16),         # head size 8 (one partial 16-wide block)
    (64, 900, 2, 48, 750),      # more earlier rows than the window needs
    (40, 927, 1, 40, 907),      # 8 key splits: the merge's one-pass path at its limit
    (16, 1075, 1, 40, 1055),    # 9 key splits: the merge's two-pass path
    (5, 2000, 1, 40, 2000),     # 16 key splits
])
def test_enc_attn_shapes(vx, orc, m, n_ctx, heads, hd, window):
    say(f"enc_attn m={m} n_ctx={n_ctx} heads={heads} hd={hd} window={window}")
    q, k, v = synth.enc_attention_inputs(800 + m, m, n_ctx, heads * hd)
    got = _run(vx, q, k, v, heads, window)
    assert_close(got, orc.enc_attn(q, k, v, heads, window), f"enc_attn {m} {n_ctx} {heads}x{hd} w{window}")


def test_enc_attn_window_one_returns_own_values(vx):
    m, n_ctx, heads = 40, 9, 32
    q, k, v = synth.enc_attention_inputs(810, m, n_ctx)
    got = _run(vx, q, k, v, heads, 1)
    assert np.array_equal(got, v[n_ctx:])


def test_enc_attn_repeatable(vx):
    m, n_ctx = 16, 749
    q, k, v = synth.enc_attention_inputs(811, m, n_ctx)
    a = _run(vx, q, k, v, 32, 750)
    b = _run(vx, q, k, v, 32, 750, extra=4096)
    assert np.array_equal(a, b)


def test_enc_attn_errors(vx):
    m, n_ctx = 16, 749
    q, k, v = synth.enc_attention_inputs(812, m, n_ctx)
    out = torch.empty((m, 1280), dtype=torch.float32, device="cuda")
    need = vx.enc_attn_workspace(m, n_ctx, 32, 40, 750)
    assert need > 0
    ws = torch.empty((need - 16,), dtype=torch.uint8, device="cuda")
    with pytest.raises(vx.VoxError) as e:
        vx.enc_attn(dev(q), dev(k), dev(v), out, 32, 750, workspace=ws)
    assert e.value.status == vx.VOX_E_WORKSPACE
