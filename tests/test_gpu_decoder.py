"""GPU parity of the whole decoder step against the CPU oracle (teacher-forced)."""
import numpy as np
import pytest
import torch

from streaming_speech_text_amd import synth
from tests.gpu_util import ATOL, RTOL, assert_close, dev, host, say

pytestmark = pytest.mark.gpu

SMALL = synth.DecoderShape(n_layers=2, dim=1024, n_heads=8, n_kv_heads=2, head_dim=128, hidden=2048,
                           vocab=4096, n_slots=64, norm_eps=1e-5, rope_theta=1e6)


@pytest.fixture(scope="module")
def vx():
    from streaming_speech_text_amd import vox
    vox.lib()
    return vox


def cfg_of(vx, s):
    return vx.DecoderConfig(s.n_layers, s.dim, s.n_heads, s.n_kv_heads, s.head_dim, s.hidden, s.vocab, s.n_slots,
                            s.norm_eps, s.rope_theta)


def device_weights(w):
    return {"tok_embd": dev(w["tok_embd"]), "out_norm": dev(w["out_norm"]),
            "layers": [{k: dev(v) for k, v in L.items()} for L in w["layers"]]}


def token_ok(tok_gpu, logits_oracle):
    """The GPU's greedy token must be the oracle's, or tie with it within the tolerance."""
    ref = logits_oracle.astype(np.float32).astype(np.float64)
    best = ref.max()
    return ref[tok_gpu] >= best - (ATOL + RTOL * abs(best))


def run_teacher_forced(vx, orc, shape, seed, tokens, graph=True, check_every=1):
    w = synth.decoder_weights(seed, shape)
    wd = device_weights(w)
    dec = vx.Decoder(cfg_of(vx, shape), wd)
    dec.set_graph(graph)
    o = orc.Decoder(shape, w)
    tok_in = torch.zeros(1, dtype=torch.int32, device="cuda")
    tok_out = torch.zeros(1, dtype=torch.int32, device="cuda")
    logits = torch.empty(shape.vocab, dtype=torch.float32, device="cuda")
    worst = 0.0
    near_ties = 0
    all_logits = []
    for i, t in enumerate(tokens):
        tok_in.fill_(int(t))
        dec.step(tok_in, tok_out, logits)
        nxt_o, lg_o = o.step(int(t), want_logits=(i % check_every == 0))
        if i % check_every == 0:
            lg = host(logits)
            all_logits.append(lg.copy())
            worst = max(worst, assert_close(lg, lg_o, f"decoder step {i} logits"))
            tg = int(host(tok_out)[0])
            assert token_ok(tg, lg_o), f"step {i}: gpu token {tg} vs oracle {nxt_o}"
            near_ties += int(tg != nxt_o)
    assert dec.position == len(tokens)
    dec.close()
    o.close()
    return worst, near_ties, all_logits


def test_decoder_small_window_wraps(vx, orc):
    tokens = synth.generator(71, 3).integers(0, SMALL.vocab, size=150).tolist()
    say("decoder small config, 150 teacher-forced steps over a 64-slot window")
    worst, ties, _ = run_teacher_forced(vx, orc, SMALL, 71, tokens)
    say(f"worst err/limit {worst:.3f}, near-tie token differences {ties}")


def test_decoder_split_window_wraps(vx, orc):
    # a 320-slot window: past 128 live positions the attention splits over the window and a
    # merge kernel combines the splits; 340 steps also wrap the ring
    shape = synth.DecoderShape(**{**SMALL.__dict__, "n_slots": 320})
    tokens = synth.generator(75, 3).integers(0, shape.vocab, size=340).tolist()
    say("decoder small config, 340 teacher-forced steps over a 320-slot window (split attention)")
    worst, ties, _ = run_teacher_forced(vx, orc, shape, 75, tokens, check_every=7)
    say(f"worst err/limit {worst:.3f}, near-tie token differences {ties}")


def test_decoder_graph_matches_eager(vx, orc):
    tokens = synth.generator(72, 3).integers(0, SMALL.vocab, size=70).tolist()
    _, _, a = run_teacher_forced(vx, orc, SMALL, 72, tokens, graph=True)
    _, _, b = run_teacher_forced(vx, orc, SMALL, 72, tokens, graph=False)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def test_decoder_greedy_feedback_and_reset(vx, orc):
    # greedy loop on the device (token_out feeds the next token_in) against the oracle's own
    # greedy sequence; then reset and replay
    shape = SMALL
    w = synth.decoder_weights(73, shape)
    dec = vx.Decoder(cfg_of(vx, shape), device_weights(w))
    o = orc.Decoder(shape, w)
    tok = torch.tensor([5], dtype=torch.int32, device="cuda")
    logits = torch.empty(shape.vocab, dtype=torch.float32, device="cuda")
    seq_gpu, cur = [], 5
    for i in range(40):
        dec.step(tok, tok, logits)
        seq_gpu.append(int(host(tok)[0]))
        nxt, lg = o.step(cur)
        assert token_ok(seq_gpu[-1], lg), f"greedy step {i}"
        if seq_gpu[-1] != nxt:
            break   # a legitimate near-tie: the sequences may diverge from here
        cur = nxt
    dec.reset()
    assert dec.position == 0
    tok.fill_(5)
    for i in range(5):
        dec.step(tok, tok, logits)
        assert int(host(tok)[0]) == seq_gpu[i]
    dec.close()


@pytest.mark.slow
@pytest.mark.timeout(900)
def test_decoder_full_voxtral_shape(vx, orc):
    """26 layers, width 3072, vocab 131072: the 38-position prefix then 64 more steps, logits every step."""
    s = synth.VOXTRAL_DECODER
    prefix, start = synth.decoder_tokens(synth.SEED_DECODER, s.vocab)
    tokens = list(prefix) + [start] + synth.generator(74, 1).integers(0, s.vocab, size=63).tolist()
    say(f"decoder full shape, {len(tokens)} teacher-forced steps")
    worst, ties, _ = run_teacher_forced(vx, orc, s, synth.SEED_DECODER, tokens)
    say(f"worst err/limit {worst:.3f}, near-tie token differences {ties}")


def test_decoder_config_errors(vx):
    import ctypes
    bad = cfg_of(vx, SMALL)
    bad.head_dim = 64
    kv, sc = ctypes.c_size_t(), ctypes.c_size_t()
    st = vx.lib().vox_decoder_workspace(ctypes.byref(bad), ctypes.byref(kv), ctypes.byref(sc))
    assert st == vx.VOX_E_UNSUPPORTED
    bad = cfg_of(vx, SMALL)
    bad.n_kv_heads = 3
    st = vx.lib().vox_decoder_workspace(ctypes.byref(bad), ctypes.byref(kv), ctypes.byref(sc))
    assert st == vx.VOX_E_INVAL
