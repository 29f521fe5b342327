"""The attention entry point that allocates nothing (its split partials in the library's fixed
per-GPU scratch array) against the workspace entry point and the oracle, through the C ABI."""
import ctypes as C
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


def _both(vx, q, kc, vc, n_valid):
    """Runs the workspace entry point, then the one without; returns both outputs."""
    nq, hd = q.shape
    nkv, n_slots, _ = kc.shape
    scale = 1 / math.sqrt(hd)
    qd, kd, vd = dev(q), dev(kc), dev(vc)
    ws = torch.empty(vx.gqa_decode_attn_workspace(nq, nkv, hd, n_slots), dtype=torch.uint8, device="cuda")
    ref = torch.full((nq, hd), float("nan"), dtype=torch.float32, device="cuda")
    out = torch.full((nq, hd), float("nan"), dtype=torch.float32, device="cuda")
    vx.gqa_decode_attn(qd, kd, vd, ref, nq, nkv, hd, n_slots, n_valid, scale, ws)
    st = vx.lib().vox_gqa_decode_attn_noalloc(vx._ptr(qd), vx._ptr(kd), vx._ptr(vd), vx._ptr(out), nq, nkv, hd,
                                              n_slots, n_valid, C.c_float(scale), vx._stream(None))
    assert st == vx.VOX_OK, vx.last_error()
    return host(ref), host(out)


def _oracle(orc, q, kc, vc, slots):
    return orc.gqa_attn(q.astype(np.float64), kc[:, slots].astype(np.float64), vc[:, slots].astype(np.float64),
                        1 / math.sqrt(q.shape[1]))


def test_noalloc_matches_workspace_entry_two_calls(vx, orc):
    # first call: the full 8192-slot ring written 8192 + 3000 times (32 chunks, grouped path,
    # 540,672 bytes of partials); second call, smaller: 1000 live slots of a 2048-slot ring
    # (8 chunks, per-head path), which reuses the array the first call filled
    q, kc, vc = synth.attention_inputs(synth.SEED_ATTN, 32, 8, HD, 8192)
    say("noalloc attention: 8192 slots full, write index 3000")
    ref, got = _both(vx, q, kc, vc, 8192)
    assert np.array_equal(ref, got)
    chrono = np.concatenate([np.arange(3000, 8192), np.arange(0, 3000)])
    assert_close(got, _oracle(orc, q, kc, vc, chrono), "noalloc attn full wrapped ring")

    q2, kc2, vc2 = synth.attention_inputs(977, 32, 8, HD, 2048)
    say("noalloc attention: 1000 of 2048 slots")
    ref2, got2 = _both(vx, q2, kc2, vc2, 1000)
    assert np.array_equal(ref2, got2)
    assert_close(got2, _oracle(orc, q2, kc2, vc2, np.arange(1000)), "noalloc attn 1000 of 2048")


def test_noalloc_small_and_grouped(vx, orc):
    # unsplit (one chunk), then group 8 with 12 chunks
    for seed, nq, nkv, slots, nv in ((978, 32, 8, 8192, 100), (979, 64, 8, 1536, 1536)):
        q, kc, vc = synth.attention_inputs(seed, nq, nkv, HD, slots)
        say(f"noalloc attention: {nq}/{nkv} heads, {nv} of {slots} slots")
        ref, got = _both(vx, q, kc, vc, nv)
        assert np.array_equal(ref, got)
        assert_close(got, _oracle(orc, q, kc, vc, np.arange(nv)), f"noalloc attn {nq}/{nkv} L={nv}")


def test_noalloc_rejects_beyond_scratch(vx):
    # 64 query heads over 8192 slots need 64 * 32 * 528 = 1,081,344 bytes of partials, past the
    # fixed 1 MiB array: refused before any device work
    q = torch.zeros(64, HD, device="cuda")
    kc = torch.zeros(8, 8192, HD, device="cuda")
    out = torch.zeros(64, HD, device="cuda")
    st = vx.lib().vox_gqa_decode_attn_noalloc(vx._ptr(q), vx._ptr(kc), vx._ptr(kc), vx._ptr(out), 64, 8, HD, 8192,
                                              100, C.c_float(0.1), vx._stream(None))
    assert st == vx.VOX_E_UNSUPPORTED
    assert "scratch" in vx.last_error()
