"""GPU parity of grouped-query decode attention over a KV ring against the CPU oracle."""
import math

import numpy as np
import pytest
import torch

from streaming_speech_text_amd import synth
from tests.gpu_util import assert_close, dev, host, say

pytestmark = pytest.mark.gpu

HD = 128


@pytest.fixture(scope="module")
def vx():
    from streaming_speech_text_amd import vox
    vox.lib()
    return vox


def _run(vx, q, kc, vc, n_valid, scale=None):
    nq, hd = q.shape
    nkv, n_slots, _ = kc.shape
    scale = 1 / math.sqrt(hd) if scale is None else scale
    ws = torch.empty(vx.gqa_decode_attn_workspace(nq, nkv, hd, n_slots) // 4 + 4, dtype=torch.float32, device="cuda")
    out = torch.full((nq, hd), float("nan"), dtype=torch.float32, device="cuda")
    vx.gqa_decode_attn(dev(q), dev(kc), dev(vc), out, nq, nkv, hd, n_slots, n_valid, scale, ws)
    return host(out)


def _oracle(orc, q, kc, vc, slots, scale=None):
    scale = 1 / math.sqrt(q.shape[1]) if scale is None else scale
    return orc.gqa_attn(q.astype(np.float64), kc[:, slots].astype(np.float64), vc[:, slots].astype(np.float64),
                        scale)


@pytest.mark.parametrize("n_valid", [1024, 4096])
def test_attention_ring_lengths(vx, orc, n_valid):
    q, kc, vc = synth.attention_inputs(synth.SEED_ATTN, 32, 8, HD, 8192)
    say(f"attention n_valid={n_valid} of 8192 slots")
    got = _run(vx, q, kc, vc, n_valid)
    assert_close(got, _oracle(orc, q, kc, vc, np.arange(n_valid)), f"attn L={n_valid}")


def test_attention_full_ring_wrapped(vx, orc):
    # 8192 + 3000 writes: the ring is full and its oldest entry sits at slot 3000
    q, kc, vc = synth.attention_inputs(synth.SEED_ATTN, 32, 8, HD, 8192)
    w = 3000
    chrono = np.concatenate([np.arange(w, 8192), np.arange(0, w)])
    say("attention full ring, write index 3000")
    got = _run(vx, q, kc, vc, 8192)
    assert_close(got, _oracle(orc, q, kc, vc, chrono), "attn full wrapped ring")


@pytest.mark.parametrize("n_valid", [1, 2, 31, 32, 33, 63, 64, 65, 100, 1000, 8191])
def test_attention_edge_lengths(vx, orc, n_valid):
    q, kc, vc = synth.attention_inputs(900 + n_valid, 32, 8, HD, 8192)
    say(f"attention edge n_valid={n_valid}")
    got = _run(vx, q, kc, vc, n_valid)
    assert_close(got, _oracle(orc, q, kc, vc, np.arange(n_valid)), f"attn L={n_valid}")


@pytest.mark.parametrize("nq,nkv,n_slots,n_valid", [
    (32, 8, 20000, 20000),   # 32 chunks of 625: four full sub-chunks and a partial one each
    (32, 8, 16384, 16384),   # 32 chunks of 512: four full sub-chunks each
    (32, 8, 20000, 9000),    # chunks of 282: two full sub-chunks and a partial one (the last: 258)
    (16, 8, 20000, 20000),   # groups of two query heads
    (64, 8, 16384, 16000),   # groups of eight query heads
])
def test_attention_long_chunks(vx, orc, nq, nkv, n_slots, n_valid):
    # rings longer than 8192 slots: every chunk walks three to five 128-position sub-chunks, so each
    # full sub-chunk's K loads are issued during the one before, and a partial one follows them
    q, kc, vc = synth.attention_inputs(970 + nq, nq, nkv, HD, n_slots)
    say(f"attention long chunks nq={nq} nkv={nkv} n_slots={n_slots} n_valid={n_valid}")
    got = _run(vx, q, kc, vc, n_valid)
    assert_close(got, _oracle(orc, q, kc, vc, np.arange(n_valid)), f"attn {nq}/{nkv} L={n_valid} of {n_slots}")


@pytest.mark.parametrize("nq,nkv", [(8, 8), (16, 8), (64, 8), (4, 1), (8, 2)])
def test_attention_group_sizes(vx, orc, nq, nkv):
    q, kc, vc = synth.attention_inputs(950 + nq + nkv, nq, nkv, HD, 300)
    say(f"attention group nq={nq} nkv={nkv}")
    for n_valid in (1, 77, 300):
        got = _run(vx, q, kc, vc, n_valid, scale=0.05)
        assert_close(got, _oracle(orc, q, kc, vc, np.arange(n_valid), scale=0.05), f"attn {nq}/{nkv} L={n_valid}")


def test_attention_single_key_and_ones(vx):
    q, kc, vc = synth.attention_inputs(960, 32, 8, HD, 64)
    got = _run(vx, q, kc, vc, 1)
    assert np.array_equal(got, np.repeat(vc[:, 0], 4, axis=0))   # one key: its value, exactly
    got = _run(vx, q, kc, np.ones_like(vc), 64)
    assert np.allclose(got, 1.0, rtol=0, atol=1e-6)                # weights sum to one


def test_attention_deterministic(vx):
    q, kc, vc = synth.attention_inputs(961, 32, 8, HD, 8192)
    a = _run(vx, q, kc, vc, 8192)
    b = _run(vx, q, kc, vc, 8192)
    assert np.array_equal(a, b)


def test_attention_errors(vx):
    q = torch.zeros(32, HD, device="cuda")
    kc = torch.zeros(8, 64, HD, device="cuda")
    out = torch.zeros(32, HD, device="cuda")
    ws = torch.zeros(vx.gqa_decode_attn_workspace(32, 8, HD, 64), dtype=torch.uint8, device="cuda")
    for args, code in [((32, 8, HD, 64, 0), vx.VOX_E_INVAL), ((32, 8, HD, 64, 65), vx.VOX_E_INVAL),
                       ((32, 7, HD, 64, 10), vx.VOX_E_INVAL), ((32, 8, 64, 64, 10), vx.VOX_E_UNSUPPORTED),
                       ((48, 8, HD, 64, 10), vx.VOX_E_UNSUPPORTED)]:
        with pytest.raises(vx.VoxError) as e:
            vx.gqa_decode_attn(q, kc, kc, out, *args, 0.1, ws)
        assert e.value.status == code
    with pytest.raises(vx.VoxError) as e:
        vx.gqa_decode_attn(q, kc, kc, out, 32, 8, HD, 64, 10, 0.1, ws, workspace_bytes=16)
    assert e.value.status == vx.VOX_E_WORKSPACE
