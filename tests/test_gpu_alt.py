"""GPU parity of the greedy token and its alternatives against the CPU oracle: the listed ids and
their count bit-exact, the probabilities within the usual bound."""
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


def _alt(vx, logits, cutoff, max_out):
    vocab = logits.size
    ids = torch.full((max_out,), -7, dtype=torch.int32, device="cuda")
    probs = torch.full((max_out,), float("nan"), dtype=torch.float32, device="cuda")
    count = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    ws = torch.full((vx.alt_tokens_workspace(vocab, max_out),), 0xFF, dtype=torch.uint8, device="cuda")
    vx.alt_tokens(dev(logits), cutoff, max_out, ids, probs, count, ws)
    n = int(host(count)[0])
    return host(ids)[:n], host(probs)[:n], host(ids)[n:], host(probs)[n:]


def _check(vx, orc, logits, cutoff, max_out, what):
    c32 = float(np.float32(cutoff))            # the cutoff as the device sees it
    ids, probs, rest_ids, rest_probs = _alt(vx, logits, c32, max_out)
    rid, rprobs = orc.alt_tokens(logits, c32, max_out)
    assert np.array_equal(ids.astype(np.int64), rid), f"{what}: ids {ids[:8]} vs {rid[:8]}"
    assert_close(probs, rprobs, f"{what}: probs")
    assert np.all(rest_ids == -7) and np.all(np.isnan(rest_probs)), f"{what}: wrote past the count"


@pytest.mark.parametrize("cutoff", [0.0, 0.5, 0.9, 0.99, 0.999, 1.0])
@pytest.mark.parametrize("max_out", [1, 8, 32])
def test_alt_tokens_vocab(vx, orc, cutoff, max_out):
    logits = (synth.normal_f32(synth.generator(950), (131072,)) * np.float32(3.0)).astype(np.float32)
    _check(vx, orc, logits, cutoff, max_out, f"alt vocab cutoff={cutoff} max_out={max_out}")


def test_alt_tokens_ties_and_masked(vx, orc):
    g = synth.generator(951)
    # coarse logits: many exact ties, listed by index; a block of -inf (masked) tokens
    logits = np.round(g.standard_normal(131072) * 2).astype(np.float32)
    logits[1000:5000] = -np.inf
    for cutoff, max_out in [(0.0, 32), (0.7, 32), (1.0, 32), (0.0, 3)]:
        _check(vx, orc, logits, cutoff, max_out, f"alt ties cutoff={cutoff}")
    # everything masked but a few tokens: cutoff 1 lists the masked ones with probability 0
    logits = np.full(3000, -np.inf, np.float32)
    logits[[5, 700, 2999]] = [1.0, 2.0, 2.0]
    _check(vx, orc, logits, 1.0, 6, "alt mostly masked")


@pytest.mark.parametrize("vocab", [1, 7, 511, 512, 513, 262144])
def test_alt_tokens_sizes(vx, orc, vocab):
    logits = synth.normal_f32(synth.generator(952, vocab), (vocab,))
    say(f"alt vocab={vocab}")
    _check(vx, orc, logits, 0.95, 16, f"alt vocab={vocab}")


def test_alt_tokens_on_decoder_logits(vx, orc):
    # logits from the decoder step itself (small shape), the greedy token first in the list
    from tests.test_gpu_decoder import SMALL, cfg_of, device_weights
    w = synth.decoder_weights(953, SMALL)
    dec = vx.Decoder(cfg_of(vx, SMALL), device_weights(w))
    tok_in = torch.full((1,), 17, dtype=torch.int32, device="cuda")
    tok_out = torch.zeros(1, dtype=torch.int32, device="cuda")
    logits = torch.empty(SMALL.vocab, dtype=torch.float32, device="cuda")
    dec.step(tok_in, tok_out, logits)
    lg = host(logits)
    ids, probs, _, _ = _alt(vx, lg, 0.99, 8)
    assert ids[0] == int(host(tok_out)[0])
    _check(vx, orc, lg, 0.99, 8, "alt on decoder logits")
    dec.close()


@pytest.mark.parametrize("kept", [1, 40, 64, 65, 128, 129, 256, 257, 512, 513, 2000])
@pytest.mark.parametrize("ties", [False, True])
def test_alt_tokens_kept_counts(vx, orc, kept, ties):
    # exactly `kept` tokens pass the threshold: 40 of them (or all, when fewer) in one 512-logit
    # block, so that block keeps more than max_out, the others spread over the vocabulary.  The
    # counts step over the sizes at which the gathered keys change sort network or overflow it.
    g = synth.generator(954, kept)
    vocab = 131072
    logits = np.full(vocab, -5.0, np.float32) - g.random(vocab).astype(np.float32)
    dense = np.arange(3 * 512, 3 * 512 + min(kept, 40))
    rest = g.choice(np.setdiff1d(np.arange(vocab), dense), kept - dense.size, replace=False)
    sel = np.concatenate([dense, rest])
    logits[sel] = 5.0 if ties else (4.0 + g.random(sel.size)).astype(np.float32)
    for max_out in (1, 8, 32):
        _check(vx, orc, logits, 0.9999, max_out, f"alt kept={kept} ties={ties} max_out={max_out}")
