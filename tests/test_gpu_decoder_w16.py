"""GPU parity of the decoder step over 16-bit weights against the CPU oracle (teacher-forced).

voxtral.c keeps the model's weights in BF16 and runs its GPU path in F16 ("Mistral Voxtral Realtime
4B 음성 인식 모델의 순수 C 기반 CPU 전용 추론 구현", GeekNews 26608, sections 모델 다운로드 및 구성 and
메모리 요구사항).  vox_decoder_create_w16 runs the same step as the Q4_0 decoder over bf16 or f16
matrices (every linear and the tied table); the oracle's 16-bit decoder is the reference.
"""
import ctypes

import numpy as np
import pytest
import torch

from streaming_speech_text_amd import synth
from tests.gpu_util import assert_close, host, say
from tests.test_gpu_decoder import SMALL, cfg_of, token_ok

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def vx():
    from streaming_speech_text_amd import vox
    vox.lib()
    return vox


def device_weights_w16(w):
    def d(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            a = a.view(np.int16)   # the bit patterns, as a dtype every torch build moves to the GPU
        return torch.from_numpy(a).to("cuda")
    return {"tok_embd": d(w["tok_embd"]), "out_norm": d(w["out_norm"]),
            "layers": [{k: d(v) for k, v in L.items()} for L in w["layers"]]}


def run_w16(vx, orc, shape, seed, fmt, tokens, graph=True, check_every=1):
    w = synth.decoder_weights_w16(seed, shape, fmt)
    dec = vx.Decoder(cfg_of(vx, shape), device_weights_w16(w), fmt=fmt)
    dec.set_graph(graph)
    o = orc.Decoder(shape, w, fmt=fmt)
    tok_in = torch.zeros(1, dtype=torch.int32, device="cuda")
    tok_out = torch.zeros(1, dtype=torch.int32, device="cuda")
    logits = torch.empty(shape.vocab, dtype=torch.float32, device="cuda")
    worst, near_ties, all_logits = 0.0, 0, []
    for i, t in enumerate(tokens):
        tok_in.fill_(int(t))
        dec.step(tok_in, tok_out, logits)
        nxt_o, lg_o = o.step(int(t), want_logits=(i % check_every == 0))
        if i % check_every == 0:
            lg = host(logits)
            all_logits.append(lg.copy())
            worst = max(worst, assert_close(lg, lg_o, f"{fmt} decoder step {i} logits"))
            tg = int(host(tok_out)[0])
            assert token_ok(tg, lg_o), f"{fmt} step {i}: gpu token {tg} vs oracle {nxt_o}"
            near_ties += int(tg != nxt_o)
    assert dec.position == len(tokens)
    dec.close()
    o.close()
    return worst, near_ties, all_logits


@pytest.mark.parametrize("fmt", ["bf16", "f16"])
def test_decoder_w16_small_window_wraps(vx, orc, fmt):
    tokens = synth.generator(81, 3).integers(0, SMALL.vocab, size=150).tolist()
    say(f"{fmt} decoder small config, 150 teacher-forced steps over a 64-slot window")
    worst, ties, _ = run_w16(vx, orc, SMALL, 81, fmt, tokens)
    say(f"worst err/limit {worst:.3f}, near-tie token differences {ties}")


def test_decoder_w16_split_window_wraps(vx, orc):
    # a 320-slot window: the split attention and its merge behind 16-bit linears, ring wrapped
    shape = synth.DecoderShape(**{**SMALL.__dict__, "n_slots": 320})
    tokens = synth.generator(82, 3).integers(0, shape.vocab, size=340).tolist()
    say("f16 decoder small config, 340 teacher-forced steps over a 320-slot window")
    worst, ties, _ = run_w16(vx, orc, shape, 82, "f16", tokens, check_every=7)
    say(f"worst err/limit {worst:.3f}, near-tie token differences {ties}")


def test_decoder_w16_graph_matches_eager(vx, orc):
    tokens = synth.generator(83, 3).integers(0, SMALL.vocab, size=40).tolist()
    _, _, a = run_w16(vx, orc, SMALL, 83, "bf16", tokens, graph=True)
    _, _, b = run_w16(vx, orc, SMALL, 83, "bf16", tokens, graph=False)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def test_decoder_w16_rejects_other_formats(vx):
    w = synth.decoder_weights_w16(84, SMALL, "bf16")
    wd = device_weights_w16(w)
    cfg = cfg_of(vx, SMALL)
    kv_bytes, sc_bytes = vx.decoder_workspace(cfg)
    kv = torch.empty(kv_bytes, dtype=torch.uint8, device="cuda")
    sc = torch.empty(sc_bytes, dtype=torch.uint8, device="cuda")
    layers = (vx.LayerWeights * SMALL.n_layers)()
    for i, L in enumerate(wd["layers"]):
        layers[i] = vx.LayerWeights(*[L[f].data_ptr() for f in ("attn_norm", "ffn_norm", "wq", "wk", "wv", "wo",
                                                                "w_gate", "w_up", "w_down")])
    dw = vx.DecoderWeights(wd["tok_embd"].data_ptr(), wd["out_norm"].data_ptr(), layers)
    h = ctypes.c_void_p()
    for bad in (2, -1):
        st = vx.lib().vox_decoder_create_w16(ctypes.byref(cfg), ctypes.byref(dw), bad, kv.data_ptr(), kv_bytes,
                                             sc.data_ptr(), sc_bytes, None, ctypes.byref(h))
        assert st == vx.VOX_E_INVAL and not h.value


@pytest.mark.slow
@pytest.mark.timeout(900)
def test_decoder_w16_full_voxtral_shape(vx, orc):
    """26 layers, width 3072, vocab 131072, f16 weights (6.86 GB): the first prefix tokens, logits
    every step."""
    s = synth.VOXTRAL_DECODER
    prefix, _ = synth.decoder_tokens(synth.SEED_DECODER, s.vocab)
    tokens = [int(t) for t in prefix[:4]]
    say(f"f16 decoder full shape, {len(tokens)} teacher-forced steps")
    worst, ties, _ = run_w16(vx, orc, s, synth.SEED_DECODER, "f16", tokens)
    say(f"worst err/limit {worst:.3f}, near-tie token differences {ties}")
