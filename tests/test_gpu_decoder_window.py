"""GPU parity of the decoder step over the rolling 8192-position window against the CPU oracle.

The voxtral.c page ("Mistral Voxtral Realtime 4B 음성 인식 모델의 순수 C 기반 CPU 전용 추론 구현",
GeekNews 26608, section 주요 기능) keeps a rolling KV cache over an 8192-position window so a
stream can run without bound.  These tests run the decoder (small width, 2 layers, GQA group 4) on
an 8192-slot ring through every split of the attention window: each graph bucket (1 to 32 chunks),
the per-head and the grouped attention kernels with their merges, the full ring, the wrapped ring,
and rotary angles at positions far past the window.
"""
import numpy as np
import pytest
import torch

from streaming_speech_text_amd import synth
from tests.gpu_util import assert_close, dev, host, say
from tests.test_gpu_decoder import cfg_of, device_weights, token_ok

pytestmark = pytest.mark.gpu

LONG = synth.DecoderShape(n_layers=2, dim=1024, n_heads=8, n_kv_heads=2, head_dim=128, hidden=2048,
                          vocab=4096, n_slots=8192, norm_eps=1e-5, rope_theta=1e6)
SEED = 76


@pytest.fixture(scope="module")
def vx():
    from streaming_speech_text_amd import vox
    vox.lib()
    return vox


@pytest.fixture(scope="module")
def weights():
    return synth.decoder_weights(SEED, LONG)


def window_values(pos: int):
    """Keys and values of positions max(0, pos - n_slots) .. pos - 1, oldest first: fp32 N(0, 1),
    [n_layers, len, n_kv*head_dim] each."""
    n = min(pos, LONG.n_slots)
    shape = (LONG.n_layers, n, LONG.n_kv_heads * LONG.head_dim)
    return (synth.normal_f32(synth.generator(SEED, 20, pos), shape),
            synth.normal_f32(synth.generator(SEED, 21, pos), shape))


def fill_ring(dec, pos: int, kw, vw):
    """Writes the window into the decoder's KV ring ([n_layers][2][n_kv][n_slots][head_dim] fp32),
    position p at slot p % n_slots; other slots get NaN, so reading one would show."""
    s = LONG
    ring = np.full((s.n_layers, 2, s.n_kv_heads, s.n_slots, s.head_dim), np.nan, dtype=np.float32)
    n = kw.shape[1]
    slots = np.arange(pos - n, pos) % s.n_slots
    for li in range(s.n_layers):
        ring[li, 0][:, slots, :] = kw[li].reshape(n, s.n_kv_heads, s.head_dim).transpose(1, 0, 2)
        ring[li, 1][:, slots, :] = vw[li].reshape(n, s.n_kv_heads, s.head_dim).transpose(1, 0, 2)
    dec.kv.view(torch.float32).copy_(torch.from_numpy(ring.reshape(-1)))


def resume_and_compare(vx, orc, wd, w, pos: int, n_steps: int = 3, graph: bool = True):
    """Resumes both sides at `pos` with the same window, then teacher-forces n_steps tokens and
    compares the logits of every step; returns the GPU logits."""
    dec = vx.Decoder(cfg_of(vx, LONG), wd)
    dec.set_graph(graph)
    o = orc.Decoder(LONG, w)
    kw, vw = window_values(pos)
    fill_ring(dec, pos, kw, vw)
    dec.seek(pos)
    o.load_window(pos, kw, vw)
    tokens = synth.generator(SEED, 22, pos).integers(0, LONG.vocab, size=n_steps).tolist()
    tok_in = torch.zeros(1, dtype=torch.int32, device="cuda")
    tok_out = torch.zeros(1, dtype=torch.int32, device="cuda")
    logits = torch.empty(LONG.vocab, dtype=torch.float32, device="cuda")
    out = []
    for i, t in enumerate(tokens):
        tok_in.fill_(int(t))
        dec.step(tok_in, tok_out, logits)
        _, lg_o = o.step(int(t))
        lg = host(logits)
        assert_close(lg, lg_o, f"resumed at {pos}, step {pos + i} (live slots {min(pos + i + 1, LONG.n_slots)})")
        assert token_ok(int(host(tok_out)[0]), lg_o), f"step {pos + i}: greedy token"
        out.append(lg.copy())
    assert dec.position == pos + n_steps == o.position
    dec.close()
    o.close()
    return out


# Resume positions: each pair of steps crosses a split boundary of the 8192-slot window (128
# positions per chunk, at most 32 chunks): 1 -> 2 chunks, 2 -> 3 (grid of 4), 4 -> 5 (grid of 8),
# 8 -> 9 (grouped kernel, grid of 16), 16 -> 17 (grid of 32), chunks of 128 -> 129 positions at 32
# chunks, the ring becoming full, the ring full with its write index at 3000, and a stream about 22
# hours long at 12.5 tokens per second.
RESUME_AT = [127, 255, 511, 1023, 2047, 4095, 8190, 8192 + 3000, 1_000_003]


@pytest.mark.parametrize("pos", RESUME_AT)
def test_decoder_resumed_window(vx, orc, weights, pos):
    say(f"decoder 8192-slot ring resumed at position {pos}")
    resume_and_compare(vx, orc, device_weights(weights), weights, pos)


def test_decoder_resumed_graph_matches_eager(vx, orc, weights):
    # the grouped split kernel and its merge inside the captured graph give the same bits as
    # direct launches
    wd = device_weights(weights)
    a = resume_and_compare(vx, orc, wd, weights, 5000, graph=True)
    b = resume_and_compare(vx, orc, wd, weights, 5000, graph=False)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def test_decoder_seek_errors(vx, weights):
    dec = vx.Decoder(cfg_of(vx, LONG), device_weights(weights))
    for bad in (-1, (1 << 40) + 1):
        with pytest.raises(vx.VoxError) as e:
            dec.seek(bad)
        assert e.value.status == vx.VOX_E_INVAL
    dec.seek(1 << 40)
    assert dec.position == 1 << 40
    dec.reset()
    assert dec.position == 0
    dec.close()


def run_stream(vx, orc, w, n_steps: int, checks: set, every: int):
    """Teacher-forced stream from position 0 over the 8192-slot ring, logits compared at the
    positions in `checks` and every `every` steps."""
    dec = vx.Decoder(cfg_of(vx, LONG), device_weights(w))
    o = orc.Decoder(LONG, w)
    tokens = synth.generator(SEED, 3).integers(0, LONG.vocab, size=n_steps).tolist()
    tok_in = torch.zeros(1, dtype=torch.int32, device="cuda")
    tok_out = torch.zeros(1, dtype=torch.int32, device="cuda")
    logits = torch.empty(LONG.vocab, dtype=torch.float32, device="cuda")
    worst, n_checked = 0.0, 0
    for i, t in enumerate(tokens):
        check = i in checks or i % every == 0 or i == n_steps - 1
        tok_in.fill_(int(t))
        dec.step(tok_in, tok_out, logits if check else None)
        nxt_o, lg_o = o.step(int(t), want_logits=check)
        if check:
            worst = max(worst, assert_close(host(logits), lg_o, f"stream step {i} (live slots "
                                                                f"{min(i + 1, LONG.n_slots)})"))
            assert token_ok(int(host(tok_out)[0]), lg_o), f"stream step {i}: greedy token"
            n_checked += 1
        if i % 500 == 499:
            say(f"  stream step {i + 1}/{n_steps}, worst err/limit {worst:.3f}")
    assert dec.position == n_steps
    dec.close()
    o.close()
    return worst, n_checked


# positions whose live window (position + 1) crosses a split boundary
TRANSITIONS = {p - 1 for p in (128, 129, 256, 257, 512, 513, 1024, 1025, 2048, 2049, 4096, 4097,
                               8192, 8193)}


def test_decoder_stream_through_splits(vx, orc, weights):
    # 2100 steps: every graph bucket and both attention kernels, in one stream whose ring the
    # decoder filled itself
    say("decoder stream over an 8192-slot ring, 2100 teacher-forced steps")
    worst, n = run_stream(vx, orc, weights, 2100, TRANSITIONS, 100)
    say(f"checked {n} steps, worst err/limit {worst:.3f}")


@pytest.mark.slow
@pytest.mark.timeout(900)
def test_decoder_stream_past_the_window(vx, orc, weights):
    # 8300 steps: the window fills (8192 positions) and rolls, the ring wraps inside the stream
    say("decoder stream over an 8192-slot ring, 8300 teacher-forced steps")
    worst, n = run_stream(vx, orc, weights, 8300, TRANSITIONS | {8200, 8250}, 250)
    say(f"checked {n} steps, worst err/limit {worst:.3f}")
