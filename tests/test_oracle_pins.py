"""Pins of the CPU oracle against things other than itself (closed forms, exhaustive
checks against numpy/torch number handling, exact rational brute force, invariants and
library routines on small inputs).  CPU only."""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from streaming_speech_text_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def make_block(d_bits: int, qs) -> np.ndarray:
    b = np.zeros(18, np.uint8)
    b[0] = d_bits & 0xFF
    b[1] = d_bits >> 8
    b[2:] = np.asarray(qs, dtype=np.uint8)
    return b


def f32_bits(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float32).view(np.uint32)


# ---------------------------------------------------------------------------------------
# number formats
# ---------------------------------------------------------------------------------------

def test_fp16_decode_exhaustive(orc):
    allh = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = orc.fp16_to_double(allh)
    ref = allh.view(np.float16).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    # signs of zeros too
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def test_fp16_decode_closed_forms(orc):
    assert orc.lib().orc_fp16_to_double(0x3C00) == 1.0
    assert orc.lib().orc_fp16_to_double(0x0001) == 2.0 ** -24
    assert orc.lib().orc_fp16_to_double(0x0400) == 2.0 ** -14
    assert orc.lib().orc_fp16_to_double(0x7BFF) == 65504.0
    assert orc.lib().orc_fp16_to_double(0xC000) == -2.0
    assert math.copysign(1.0, orc.lib().orc_fp16_to_double(0x8000)) == -1.0
    assert math.isinf(orc.lib().orc_fp16_to_double(0x7C00))


def test_bf16_decode_exhaustive(orc):
    allb = np.arange(65536, dtype=np.uint32)
    got = orc.bf16_to_double(allb.astype(np.uint16))
    ref = (allb << 16).astype(np.uint32).view(np.float32)
    with np.errstate(invalid="ignore"):
        ref = ref.astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


def test_bf16_generator_rounding_matches_torch():
    # the generator's bf16 rounding (input preparation) is round-to-nearest-even, as torch's
    x = synth.normal_f32(synth.generator(99), (4096,))
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(synth.bf16_bits(x), ref)


# ---------------------------------------------------------------------------------------
# Q4_0 dequantisation
# ---------------------------------------------------------------------------------------

def test_dequant_handbuilt_unit_scale(orc):
    # d = 1.0; byte j: low nibble j, high nibble 15 - j
    qs = [j | ((15 - j) << 4) for j in range(16)]
    v = orc.q4_dequant(make_block(0x3C00, qs))
    expect = [j - 8 for j in range(16)] + [7 - j for j in range(16)]
    assert v.tolist() == [float(e) for e in expect]


def test_dequant_handbuilt_extremes(orc):
    # smallest subnormal scale: low nibbles 0 -> -8 * 2^-24, high nibbles 15 -> 7 * 2^-24
    v = orc.q4_dequant(make_block(0x0001, [0xF0] * 16))
    assert v[:16].tolist() == [-8 * 2.0 ** -24] * 16
    assert v[16:].tolist() == [7 * 2.0 ** -24] * 16
    # largest finite scale 65504: low 15 -> 7*65504, high 0 -> -8*65504
    v = orc.q4_dequant(make_block(0x7BFF, [0x0F] * 16))
    assert v[:16].tolist() == [458528.0] * 16
    assert v[16:].tolist() == [-524032.0] * 16
    # negative scale -0.5, code 8 everywhere -> (8-8) * -0.5 = -0.0 (sign kept)
    v = orc.q4_dequant(make_block(0xB800, [0x88] * 16))
    assert np.all(f32_bits(v) == 0x80000000)
    # scale -0.0: (q-8) * -0 is -0 for q >= 8 and +0 for q < 8
    qs = [j | (j << 4) for j in range(16)]
    v = orc.q4_dequant(make_block(0x8000, qs))
    sign = np.signbit(v[:16])
    assert sign.tolist() == [j >= 8 for j in range(16)]
    assert np.all(v == 0)


def test_dequant_exhaustive_codes_and_finite_scales(orc):
    # every finite fp16 scale with every code, in both nibble positions
    dbits = np.array([h for h in range(65536) if ((h >> 10) & 31) != 31], dtype=np.uint16)
    nb = dbits.size
    blocks = np.zeros((nb, 18), np.uint8)
    blocks[:, 0] = dbits & 0xFF
    blocks[:, 1] = dbits >> 8
    codes = np.arange(16, dtype=np.uint8)
    blocks[:, 2:] = codes | ((15 - codes) << 4)
    got = orc.q4_dequant(blocks).reshape(nb, 32)
    d = dbits.view(np.float16).astype(np.float64)
    lo = (codes.astype(np.float64) - 8)
    hi = (15 - codes.astype(np.float64) - 8)
    ref = np.concatenate([d[:, None] * lo[None, :], d[:, None] * hi[None, :]], axis=1)
    # the exact products fit fp32 (at most 15 significant bits)
    assert np.array_equal(ref.astype(np.float32).astype(np.float64), ref)
    assert np.array_equal(f32_bits(got), f32_bits(ref.astype(np.float32)))


def test_dequant_round_trip(orc):
    # bytes -> values -> re-encode with the block's own scale -> identical bytes
    g = synth.generator(11)
    blocks = synth.q4_matrix(g, 64, 32 * 8).reshape(-1, 18)
    vals = orc.q4_dequant(blocks).reshape(-1, 32).astype(np.float64)
    d = blocks[:, 0:2].copy().view("<f2").astype(np.float64).reshape(-1)
    codes = np.rint(vals / d[:, None] + 8).astype(np.int64)
    assert codes.min() >= 0 and codes.max() <= 15
    re = np.zeros_like(blocks)
    re[:, 0:2] = blocks[:, 0:2]
    re[:, 2:] = (codes[:, :16] | (codes[:, 16:] << 4)).astype(np.uint8)
    assert np.array_equal(re, blocks)
    # grid values -> encode -> dequant -> identical values
    codes2 = synth.generator(12).integers(0, 16, size=(64, 32))
    d2 = np.full(64, 0.0078125)  # 2^-7, exact in fp16
    enc = np.zeros((64, 18), np.uint8)
    enc[:, 0:2] = d2.astype("<f2").view(np.uint8).reshape(64, 2)
    enc[:, 2:] = (codes2[:, :16] | (codes2[:, 16:] << 4)).astype(np.uint8)
    back = orc.q4_dequant(enc).reshape(64, 32)
    assert np.array_equal(back.astype(np.float64), (codes2 - 8) * d2[:, None])


# ---------------------------------------------------------------------------------------
# GEMV / GEMM
# ---------------------------------------------------------------------------------------

def _np_dequant(w, n, k):
    """Independent numpy dequantisation used only as a cross-check."""
    b = np.ascontiguousarray(w).reshape(n, k // 32, 18)
    d = b[:, :, 0:2].copy().view("<f2").astype(np.float64)[..., 0]
    lo = (b[:, :, 2:] & 15).astype(np.float64) - 8
    hi = (b[:, :, 2:] >> 4).astype(np.float64) - 8
    return (np.concatenate([lo, hi], axis=2) * d[..., None]).reshape(n, k)


def _dyadic_q4(g, n, k):
    """Q4_0 matrix whose scales are powers of two (exact in fp16 and every partial sum)."""
    w = synth.q4_matrix(g, n, k).reshape(n, k // 32, 18)
    e = g.integers(-6, 2, size=(n, k // 32)).astype(np.float64)
    w[:, :, 0:2] = (2.0 ** e).astype("<f2").view(np.uint8).reshape(n, k // 32, 2)
    return w.reshape(n, -1)


def test_gemv_exact_bruteforce_fractions(orc):
    g = synth.generator(21)
    for n, k in [(1, 32), (3, 64), (5, 96), (7, 160)]:
        w = _dyadic_q4(g, n, k)
        x = g.integers(-7, 8, size=k).astype(np.float32)
        y = orc.q4_gemv(w, x)
        b = w.reshape(n, k // 32, 18)
        for r in range(n):
            acc = Fraction(0)
            for blk in range(k // 32):
                d = Fraction(float(b[r, blk, 0:2].copy().view("<f2")[0]))
                for j in range(16):
                    lo = int(b[r, blk, 2 + j]) & 15
                    hi = int(b[r, blk, 2 + j]) >> 4
                    acc += (lo - 8) * d * Fraction(float(x[blk * 32 + j]))
                    acc += (hi - 8) * d * Fraction(float(x[blk * 32 + j + 16]))
            assert Fraction(y[r]) == acc


def test_gemv_random_vs_numpy(orc):
    g = synth.generator(22)
    for n, k in [(37, 256), (64, 3072), (5, 9216), (300, 1280)]:
        w = synth.q4_matrix(g, n, k)
        x = synth.normal_f32(g, (k,))
        y = orc.q4_gemv(w, x)
        ref = _np_dequant(w, n, k) @ x.astype(np.float64)
        assert np.allclose(y, ref, rtol=1e-12, atol=1e-12)
        rows = np.array([0, n - 1, n // 2], np.int64)
        assert np.array_equal(orc.q4_gemv_rows(w, x, rows), y[rows])


def test_gemv_nonsquare_orientation(orc):
    # W is [n][k]; a transposed reading would not even have the right length
    g = synth.generator(23)
    w = synth.q4_matrix(g, 3, 64)
    x = np.zeros(64, np.float32)
    x[40] = 1.0  # picks column 40: block 1, element 8 -> low nibble of byte 8
    y = orc.q4_gemv(w, x)
    b = w.reshape(3, 2, 18)
    d = b[:, 1, 0:2].copy().view("<f2").astype(np.float64)[:, 0]
    assert np.array_equal(y, ((b[:, 1, 2 + 8] & 15).astype(np.float64) - 8) * d)
    x[:] = 0
    x[63] = 1.0  # block 1, element 31 -> high nibble of byte 15
    y = orc.q4_gemv(w, x)
    assert np.array_equal(y, ((b[:, 1, 2 + 15] >> 4).astype(np.float64) - 8) * d)


def test_gemm_exact_and_random(orc):
    g = synth.generator(24)
    # exact: dyadic scales, small-integer bf16 activations
    m, n, k = 5, 7, 96
    w = _dyadic_q4(g, n, k)
    xi = g.integers(-9, 10, size=(m, k)).astype(np.float32)
    y = orc.q4_gemm(w, synth.bf16_bits(xi))
    wd = _np_dequant(w, n, k)
    ref = np.array([[sum(Fraction(float(xi[r, i])) * Fraction(wd[c, i]) for i in range(k))
                     for c in range(n)] for r in range(m)])
    assert all(Fraction(y[r, c]) == ref[r, c] for r in range(m) for c in range(n))
    # random bf16 activations vs numpy
    m, n, k = 33, 40, 1280
    w = synth.q4_matrix(g, n, k)
    xb = synth.bf16_normal(g, (m, k))
    y = orc.q4_gemm(w, xb)
    xf = (xb.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    assert np.allclose(y, xf @ _np_dequant(w, n, k).T, rtol=1e-12, atol=1e-12)
    # a single row equals the GEMV of that row
    assert np.allclose(y[3], orc.q4_gemv(w, xf[3].astype(np.float32)), rtol=0, atol=0)


# ---------------------------------------------------------------------------------------
# RMSNorm, RoPE, attention, SwiGLU, argmax
# ---------------------------------------------------------------------------------------

def test_rmsnorm_closed_form_and_torch(orc):
    dim, eps = 3072, 1e-5
    c = 0.37
    out = orc.rmsnorm(np.full(dim, c), np.ones(dim, np.float32), eps)
    assert np.allclose(out, c / math.sqrt(c * c + eps), rtol=1e-12, atol=0)
    x = synth.normal_f32(synth.generator(31), (dim,)).astype(np.float64) * 3
    gain = synth.uniform_f32(synth.generator(32), (dim,), 0.5, 1.5)
    out = orc.rmsnorm(x, gain, eps)
    ref = F.rms_norm(torch.from_numpy(x), (dim,), torch.from_numpy(gain.astype(np.float64)), eps).numpy()
    assert np.allclose(out, ref, rtol=1e-13, atol=1e-14)
    # unit gain: output RMS = sqrt(ms / (ms + eps))
    o1 = orc.rmsnorm(x, np.ones(dim, np.float32), eps)
    ms = np.mean(x * x)
    assert abs(math.sqrt(np.mean(o1 * o1)) - math.sqrt(ms / (ms + eps))) < 1e-14


def test_rope_identity_norms_and_complex(orc):
    g = synth.generator(33)
    nh, hd, theta = 4, 128, 1e6
    x = g.standard_normal(nh * hd)
    assert np.array_equal(orc.rope(x, nh, hd, 0, theta), x)
    for pos in (1, 37, 8191, 123456):
        y = orc.rope(x, nh, hd, pos, theta)
        pn = (x.reshape(-1, 2) ** 2).sum(1)
        assert np.allclose((y.reshape(-1, 2) ** 2).sum(1), pn, rtol=1e-13)
        i = np.arange(hd // 2)
        ang = pos * theta ** (-2.0 * i / hd)
        z = (x[0::2] + 1j * x[1::2]).reshape(nh, hd // 2) * np.exp(1j * ang)[None, :]
        ref = np.stack([z.real, z.imag], axis=-1).reshape(-1)
        # angle = pos * freq: one ulp of freq moves the angle by about pos * 1e-16 rad
        assert np.allclose(y, ref, rtol=0, atol=1e-13 * (1 + pos))


def test_rope_relative_position(orc):
    g = synth.generator(34)
    hd = 128
    q = g.standard_normal(hd)
    k = g.standard_normal(hd)
    for a, b, t in [(5, 2, 11), (100, 0, 900), (7, 7, 3)]:
        lhs = orc.rope(q, 1, hd, a, 1e6) @ orc.rope(k, 1, hd, b, 1e6)
        rhs = orc.rope(q, 1, hd, a + t, 1e6) @ orc.rope(k, 1, hd, b + t, 1e6)
        assert abs(lhs - rhs) < 1e-9 * (1 + abs(lhs))


def test_attention_probability_sums_and_special_cases(orc):
    g = synth.generator(35)
    hd, L = 128, 300
    q = g.standard_normal(hd)
    k = g.standard_normal((L, hd)) * 2
    p = orc.attn_probs(q, k, 1 / math.sqrt(hd))
    assert abs(p.sum() - 1.0) < 1e-12 and p.min() >= 0
    # all-ones values -> every output is 1 (probabilities sum to one)
    nq, nkv = 32, 8
    qq = g.standard_normal((nq, hd))
    kk = g.standard_normal((nkv, L, hd))
    out = orc.gqa_attn(qq, kk, np.ones((nkv, L, hd)), 1 / math.sqrt(hd))
    assert np.allclose(out, 1.0, rtol=0, atol=1e-12)
    # one key -> its value exactly
    v1 = g.standard_normal((nkv, 1, hd))
    out = orc.gqa_attn(qq, kk[:, :1], v1, 0.1)
    assert np.array_equal(out, np.repeat(v1[:, 0], nq // nkv, axis=0))
    # all keys equal -> mean of the values
    keq = np.repeat(kk[:, :1], L, axis=1)
    vv = g.standard_normal((nkv, L, hd))
    out = orc.gqa_attn(qq, keq, vv, 0.3)
    assert np.allclose(out, np.repeat(vv.mean(1), nq // nkv, axis=0), rtol=1e-12, atol=1e-12)


def test_attention_vs_torch_sdpa_gqa(orc):
    g = synth.generator(36)
    for nq, nkv, hd, L in [(32, 8, 128, 77), (4, 4, 16, 5), (8, 2, 64, 513)]:
        q = g.standard_normal((nq, hd))
        k = g.standard_normal((nkv, L, hd))
        v = g.standard_normal((nkv, L, hd))
        sc = 1 / math.sqrt(hd)
        out = orc.gqa_attn(q, k, v, sc)
        ref = F.scaled_dot_product_attention(torch.from_numpy(q)[None, :, None, :], torch.from_numpy(k)[None],
                                             torch.from_numpy(v)[None], scale=sc, enable_gqa=True)
        assert np.allclose(out, ref[0, :, 0].numpy(), rtol=1e-12, atol=1e-12)


def test_attention_ring_order_invariance(orc):
    # a ring with write index w holds the same set as the chronological list; any slot
    # permutation gives the same attention output
    g = synth.generator(37)
    nq, nkv, hd, S, w = 8, 2, 32, 64, 23
    q = g.standard_normal((nq, hd))
    ring_k = g.standard_normal((nkv, S, hd))
    ring_v = g.standard_normal((nkv, S, hd))
    chrono = np.concatenate([np.arange(w, S), np.arange(0, w)])
    a = orc.gqa_attn(q, ring_k[:, chrono], ring_v[:, chrono], 0.2)
    b = orc.gqa_attn(q, ring_k, ring_v, 0.2)
    perm = g.permutation(S)
    c = orc.gqa_attn(q, ring_k[:, perm], ring_v[:, perm], 0.2)
    assert np.allclose(a, b, rtol=1e-12, atol=1e-13) and np.allclose(a, c, rtol=1e-12, atol=1e-13)


def test_attention_group_mapping(orc):
    # query head h must read KV head h // 4: put a distinct constant value in each KV head
    nq, nkv, hd, L = 32, 8, 16, 9
    g = synth.generator(38)
    q = g.standard_normal((nq, hd))
    k = g.standard_normal((nkv, L, hd))
    v = np.repeat(np.arange(nkv, dtype=np.float64)[:, None, None], L, axis=1).repeat(hd, axis=2)
    out = orc.gqa_attn(q, k, v, 0.25)
    assert np.allclose(out[:, 0], np.arange(nq) // 4, atol=1e-12)


def test_swiglu(orc):
    z = np.array([0.0, 1.0, -1.0, 30.0, -30.0, 2.5])
    u = np.array([3.0, 2.0, 2.0, 1.0, 1.0, -1.0])
    out = orc.swiglu(z, u)
    assert out[0] == 0.0
    assert abs(out[3] - 30.0) < 1e-9 and abs(out[4]) < 1e-9
    ref = (F.silu(torch.from_numpy(z)) * torch.from_numpy(u)).numpy()
    assert np.allclose(out, ref, rtol=1e-15, atol=0)


def test_argmax_ties_lowest_index(orc):
    v = np.array([1.0, 3.0, -2.0, 3.0, 3.0], np.float32)
    assert orc.argmax_f32(v) == 1 == int(np.argmax(v))
    assert orc.argmax_f64(v.astype(np.float64)) == 1
    v = synth.normal_f32(synth.generator(39), (131072,))
    assert orc.argmax_f32(v) == int(np.argmax(v))
    # the fp32 decision: two doubles that round to the same float tie at the lower index
    d = np.array([1.0, 1.0 + 2.0 ** -40, 0.5])
    assert orc.argmax_f64(d) == 1
    assert orc.argmax_f32(d.astype(np.float32)) == 0


# ---------------------------------------------------------------------------------------
# whole decoder step: tiny configuration against an independent torch float64 composition
# ---------------------------------------------------------------------------------------

TINY = synth.DecoderShape(n_layers=2, dim=64, n_heads=4, n_kv_heads=2, head_dim=16, hidden=192,
                          vocab=512, n_slots=16, norm_eps=1e-5, rope_theta=1e6)


def _np_w16(w, n, k, fmt):
    """Independent numpy decode of 16-bit weight patterns (bf16: the upper half of an fp32;
    f16: numpy's IEEE half), used only as a cross-check."""
    b = np.ascontiguousarray(w, dtype=np.uint16).reshape(n, k)
    if fmt == "bf16":
        return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return b.view(np.float16).astype(np.float64)


def _torch_decoder_reference(shape, weights, tokens, start_pos=0, window=None, fmt=None):
    """Second, independent composition from library routines (torch float64).  window: None, or
    (k, v) fp32 [n_layers, len, n_kv*head_dim] holding positions start_pos - len .. start_pos - 1.
    fmt: None for Q4_0 weights, "bf16" / "f16" for 16-bit ones."""
    s = shape
    t = torch.float64

    def deq(w, n, k):
        return torch.from_numpy(_np_dequant(w, n, k) if fmt is None else _np_w16(w, n, k, fmt))

    E = deq(weights["tok_embd"], s.vocab, s.dim)
    layers = []
    for L in weights["layers"]:
        layers.append({
            "an": torch.from_numpy(L["attn_norm"].astype(np.float64)),
            "fn": torch.from_numpy(L["ffn_norm"].astype(np.float64)),
            "wq": deq(L["wq"], s.n_heads * s.head_dim, s.dim),
            "wk": deq(L["wk"], s.n_kv_heads * s.head_dim, s.dim),
            "wv": deq(L["wv"], s.n_kv_heads * s.head_dim, s.dim),
            "wo": deq(L["wo"], s.dim, s.n_heads * s.head_dim),
            "wg": deq(L["w_gate"], s.hidden, s.dim),
            "wu": deq(L["w_up"], s.hidden, s.dim),
            "wd": deq(L["w_down"], s.dim, s.hidden),
        })
    on = torch.from_numpy(weights["out_norm"].astype(np.float64))
    inv = 1.0 / (s.rope_theta ** (torch.arange(0, s.head_dim, 2, dtype=t) / s.head_dim))

    def rope(x, nh, pos):
        z = torch.view_as_complex(x.reshape(nh, s.head_dim // 2, 2).contiguous())
        z = z * torch.polar(torch.ones_like(inv), pos * inv)[None, :]
        return torch.view_as_real(z).reshape(-1)

    cache = [([], []) for _ in layers]
    if window is not None:
        for li in range(len(layers)):
            for row_k, row_v in zip(window[0][li], window[1][li]):
                cache[li][0].append(torch.from_numpy(row_k.astype(np.float64)).reshape(s.n_kv_heads, s.head_dim))
                cache[li][1].append(torch.from_numpy(row_v.astype(np.float64)).reshape(s.n_kv_heads, s.head_dim))
    outs = []
    for pos, tok in enumerate(tokens, start=start_pos):
        h = E[tok].clone()
        for li, L in enumerate(layers):
            x = F.rms_norm(h, (s.dim,), L["an"], s.norm_eps)
            q = rope(L["wq"] @ x, s.n_heads, pos)
            k = rope(L["wk"] @ x, s.n_kv_heads, pos)
            v = L["wv"] @ x
            ks, vs = cache[li]
            ks.append(k.reshape(s.n_kv_heads, s.head_dim))
            vs.append(v.reshape(s.n_kv_heads, s.head_dim))
            K = torch.stack(ks[-s.n_slots:], dim=1)[None]
            V = torch.stack(vs[-s.n_slots:], dim=1)[None]
            o = F.scaled_dot_product_attention(q.reshape(1, s.n_heads, 1, s.head_dim), K, V,
                                               scale=1 / math.sqrt(s.head_dim), enable_gqa=True)
            h = h + L["wo"] @ o.reshape(-1)
            x = F.rms_norm(h, (s.dim,), L["fn"], s.norm_eps)
            h = h + L["wd"] @ (F.silu(L["wg"] @ x) * (L["wu"] @ x))
        logits = E @ F.rms_norm(h, (s.dim,), on, s.norm_eps)
        outs.append(logits.numpy())
    return outs


def test_decoder_tiny_vs_torch_composition(orc):
    w = synth.decoder_weights(41, TINY)
    n_steps = 40  # window of 16 wraps twice
    tokens = synth.generator(41, 9).integers(0, TINY.vocab, size=n_steps).tolist()
    dec = orc.Decoder(TINY, w)
    got = []
    for tok in tokens:
        nxt, lg = dec.step(tok)
        got.append(lg)
        assert nxt == int(np.argmax(lg.astype(np.float32)))
    assert dec.position == n_steps
    ref = _torch_decoder_reference(TINY, w, tokens)
    for a, b in zip(got, ref):
        assert np.allclose(a, b, rtol=1e-10, atol=1e-10)
    # reset restarts the sequence from position 0 with an empty window
    dec.reset()
    nxt, lg = dec.step(tokens[0])
    assert dec.position == 1 and np.allclose(lg, ref[0], rtol=1e-10, atol=1e-10)
    dec.close()


@pytest.mark.parametrize("fmt", ["bf16", "f16"])
def test_decoder_w16_tiny_vs_torch_composition(orc, fmt):
    # the step over 16-bit weights (voxtral.c page, sections 모델 다운로드 및 구성 / 메모리 요구사항:
    # BF16 weights, F16 on the GPU) against the torch composition on its own decode of the bits
    w = synth.decoder_weights_w16(41, TINY, fmt)
    n_steps = 40  # window of 16 wraps twice
    tokens = synth.generator(41, 9).integers(0, TINY.vocab, size=n_steps).tolist()
    dec = orc.Decoder(TINY, w, fmt=fmt)
    got = []
    for tok in tokens:
        nxt, lg = dec.step(tok)
        got.append(lg)
        assert nxt == int(np.argmax(lg.astype(np.float32)))
    ref = _torch_decoder_reference(TINY, w, tokens, fmt=fmt)
    for a, b in zip(got, ref):
        assert np.allclose(a, b, rtol=1e-10, atol=1e-10)
    dec.close()
    # the format flag is read: the same bits taken as the other format give other logits
    other = "f16" if fmt == "bf16" else "bf16"
    dec = orc.Decoder(TINY, w, fmt=other)
    assert not np.allclose(dec.step(tokens[0])[1], ref[0])
    dec.close()


def test_decoder_w16_resume_from_window(orc):
    w = synth.decoder_weights_w16(44, TINY, "f16")
    pos = 1_000_003
    kw = synth.normal_f32(synth.generator(44, 10), (TINY.n_layers, TINY.n_slots, TINY.n_kv_heads * TINY.head_dim))
    vw = synth.normal_f32(synth.generator(44, 11), (TINY.n_layers, TINY.n_slots, TINY.n_kv_heads * TINY.head_dim))
    tokens = synth.generator(44, 9).integers(0, TINY.vocab, size=12).tolist()
    dec = orc.Decoder(TINY, w, fmt="f16")
    dec.load_window(pos, kw, vw)
    got = [dec.step(t)[1] for t in tokens]
    ref = _torch_decoder_reference(TINY, w, tokens, start_pos=pos, window=(kw, vw), fmt="f16")
    for a, b in zip(got, ref):
        assert np.allclose(a, b, rtol=1e-9, atol=1e-9)
    dec.close()


@pytest.mark.parametrize("pos", [5, 16, 1_000_003])
def test_decoder_resume_from_window_vs_torch_composition(orc, pos):
    # a stream resumed at position pos with a given window (fewer entries than the ring holds, a
    # full ring, and a position far past any test's step count, where the rotary angles are large)
    w = synth.decoder_weights(43, TINY)
    n = min(pos, TINY.n_slots)
    kw = synth.normal_f32(synth.generator(43, 10), (TINY.n_layers, n, TINY.n_kv_heads * TINY.head_dim))
    vw = synth.normal_f32(synth.generator(43, 11), (TINY.n_layers, n, TINY.n_kv_heads * TINY.head_dim))
    tokens = synth.generator(43, 9).integers(0, TINY.vocab, size=20).tolist()
    dec = orc.Decoder(TINY, w)
    dec.step(tokens[-1])                      # a state that loading the window must replace
    dec.load_window(pos, kw, vw)
    assert dec.position == pos
    got = [dec.step(t)[1] for t in tokens]
    ref = _torch_decoder_reference(TINY, w, tokens, start_pos=pos, window=(kw, vw))
    for a, b in zip(got, ref):
        assert np.allclose(a, b, rtol=1e-9, atol=1e-9)
    # the loaded window matters: a different window changes the first step's logits
    dec.load_window(pos, kw, vw * np.float32(0.5))
    assert not np.allclose(dec.step(tokens[0])[1], ref[0])
    dec.close()


def test_decoder_window_drop_matters(orc):
    # with the window of 16, step 17 must differ from an unbounded-history reference
    w = synth.decoder_weights(42, TINY)
    tokens = synth.generator(42, 9).integers(0, TINY.vocab, size=20).tolist()
    wide = synth.DecoderShape(**{**TINY.__dict__, "n_slots": 64})
    a = orc.Decoder(TINY, w)
    b = orc.Decoder(wide, w)
    la = [a.step(t)[1] for t in tokens]
    lb = [b.step(t)[1] for t in tokens]
    for i in range(16):
        assert np.array_equal(la[i], lb[i])
    assert not np.allclose(la[17], lb[17])


# ---------------------------------------------------------------------------------------
# shapes against the figures the pages print
# ---------------------------------------------------------------------------------------

def test_page_figures_pin_shapes():
    fig = json.load(open(os.path.join(GOLDEN, "page_figures.json")))
    s = synth.VOXTRAL_DECODER
    assert s.vocab * s.dim * 4 == fig["embedding_table_f32_bytes"]["bytes"] == int(1.5 * 2 ** 30)
    kv = s.n_layers * s.n_slots * 2 * s.n_kv_heads * s.head_dim * 4
    assert 0.95 * fig["kv_cache_max_bytes"]["upper_bytes"] < kv <= fig["kv_cache_max_bytes"]["upper_bytes"]
    assert s.n_slots == fig["kv_window_positions"]["value"]
    d = fig["decoder"]
    assert (s.n_layers, s.dim, s.n_heads, s.n_kv_heads) == (d["n_layers"], d["dim"], d["n_heads"], d["n_kv_heads"])
    assert synth.DECODER_PREFIX == fig["decoder_prefix_positions"]["value"]
    # the quantised decoder (all linears + tied table) stays under the whole Q4 model size
    per_layer = sum(o * synth.q4_row_bytes(i) for o, i in synth.LAYER_LINEARS.values())
    total = s.n_layers * per_layer + s.vocab * synth.q4_row_bytes(s.dim)
    assert total < fig["q4_model_bytes"]["approx_bytes"]
    assert synth.ENCODER_LINEARS[0][1] == fig["encoder"]["dim"]


# ---------------------------------------------------------------------------------------
# adapter: linear, GELU, linear
# ---------------------------------------------------------------------------------------

def test_gelu_library_and_closed_forms(orc):
    from scipy.special import ndtr
    x = np.concatenate([np.linspace(-12, 12, 4801), synth.generator(30).standard_normal(2000) * 3])
    got = orc.gelu(x)
    # x * Phi(x) with the library's normal distribution function
    assert np.allclose(got, x * ndtr(x), rtol=1e-13, atol=1e-300)   # a few ulps in the far tail
    # torch's exact GELU in double (its 1 + erf form flushes the far negative tail to zero, so an
    # absolute floor of 1e-15 covers that tail)
    assert np.allclose(got, F.gelu(torch.from_numpy(x), approximate="none").numpy(), rtol=1e-14, atol=1e-15)
    # GELU(x) - GELU(-x) = x, since Phi(x) + Phi(-x) = 1
    assert np.allclose(got - orc.gelu(-x), x, rtol=0, atol=1e-13)
    assert orc.gelu([0.0])[0] == 0.0
    # Phi(1) = 0.841344746068543 (standard normal table); GELU(1) = Phi(1), GELU(-1) = -(1 - Phi(1))
    assert abs(orc.gelu([1.0])[0] - 0.841344746068543) < 1e-15
    assert abs(orc.gelu([-1.0])[0] + 0.158655253931457) < 1e-15
    # the tanh approximation is a different function: they differ by more than rounding here
    tanh_form = 0.5 * x * (1 + np.tanh(math.sqrt(2 / math.pi) * (x + 0.044715 * x ** 3)))
    assert np.abs(got - tanh_form).max() > 1e-4


def test_adapter_identity_second_linear(orc):
    # W2 = identity (code 9 on the diagonal, 8 elsewhere, scale 1): Y = GELU(X W1^T)
    g = synth.generator(32)
    m, k, n_mid = 6, 128, 64
    w1 = synth.q4_matrix(g, n_mid, k)
    xb = synth.bf16_normal(g, (m, k))
    eye = np.zeros((n_mid, n_mid // 32, 18), np.uint8)
    eye[:, :, 0:2] = np.frombuffer(np.float16(1.0).tobytes(), np.uint8)
    codes = np.full((n_mid, n_mid), 8, np.uint8)
    codes[np.arange(n_mid), np.arange(n_mid)] = 9
    for b in range(n_mid // 32):
        c = codes[:, 32 * b:32 * b + 32]
        eye[:, b, 2:] = c[:, :16] | (c[:, 16:] << 4)
    y = orc.adapter(w1, eye.reshape(n_mid, -1), xb)
    h = orc.q4_gemm(w1, xb)
    from scipy.special import ndtr
    assert np.allclose(y, h * ndtr(h), rtol=1e-13, atol=1e-300)
    # GELU really sits between the linears: negative pre-activations shrink toward zero
    assert (h < -1).any() and np.all(y[h < -1] > h[h < -1])


def test_adapter_bruteforce_tiny(orc):
    # pure-Python loops over the definition; non-square shapes catch a transposed operand
    g = synth.generator(33)
    m, k, n_mid, n_out = 3, 64, 96, 5
    w1 = synth.q4_matrix(g, n_mid, k)
    w2 = synth.q4_matrix(g, n_out, n_mid)
    xb = synth.bf16_normal(g, (m, k))

    def deq(w, n, kk):
        out = []
        for r in range(n):
            row = []
            for b in range(kk // 32):
                blk = w[r, 18 * b:18 * b + 18]
                d = float(blk[0:2].view(np.float16)[0])
                lo = [(int(q) & 15) - 8 for q in blk[2:]]
                hi = [(int(q) >> 4) - 8 for q in blk[2:]]
                row += [c * d for c in lo + hi]
            out.append(row)
        return out

    W1, W2 = deq(w1, n_mid, k), deq(w2, n_out, n_mid)
    X = [[float((np.uint32(v) << np.uint32(16)).view(np.float32)) for v in row] for row in xb]
    ref = []
    for r in range(m):
        hrow = []
        for c in range(n_mid):
            s = sum(X[r][i] * W1[c][i] for i in range(k))
            hrow.append(0.5 * s * (1 + math.erf(s / math.sqrt(2))))
        ref.append([sum(hrow[i] * W2[c][i] for i in range(n_mid)) for c in range(n_out)])
    got = orc.adapter(w1, w2, xb)
    assert got.shape == (m, n_out)
    assert np.allclose(got, np.array(ref), rtol=1e-12, atol=1e-12)


def test_page_figures_pin_adapter_shape():
    fig = json.load(open(os.path.join(GOLDEN, "page_figures.json")))["adapter"]
    assert synth.ADAPTER == (fig["in"], fig["mid"], fig["out"])
    # four encoder frames of width 1280 make one adapter row
    assert fig["in"] == 4 * json.load(open(os.path.join(GOLDEN, "page_figures.json")))["encoder"]["dim"]


# ---------------------------------------------------------------------------------------
# encoder self-attention over a chunk: causal, sliding window
# ---------------------------------------------------------------------------------------

def _sdpa_masked(q, k, v, n_heads, n_ctx, window):
    """torch float64 SDPA with an explicit boolean mask built from positions."""
    m, width = q.shape
    hd = width // n_heads
    T = k.shape[0]
    qh = torch.from_numpy(q).reshape(m, n_heads, hd).transpose(0, 1)
    kh = torch.from_numpy(k).reshape(T, n_heads, hd).transpose(0, 1)
    vh = torch.from_numpy(v).reshape(T, n_heads, hd).transpose(0, 1)
    qpos = n_ctx + np.arange(m)[:, None]
    kpos = np.arange(T)[None, :]
    mask = torch.from_numpy((kpos <= qpos) & (kpos > qpos - window))
    o = F.scaled_dot_product_attention(qh, kh, vh, attn_mask=mask)
    return o.transpose(0, 1).reshape(m, width).numpy()


def test_enc_attn_causal_matches_sdpa(orc):
    # no earlier rows and a window past the chunk: plain causal attention
    g = synth.generator(40)
    m, H, hd = 37, 4, 40
    q, k, v = (g.standard_normal((m, H * hd)) for _ in range(3))
    got = orc.enc_attn(q, k, v, H, window=1000)
    qh = torch.from_numpy(q).reshape(m, H, hd).transpose(0, 1)
    kh = torch.from_numpy(k).reshape(m, H, hd).transpose(0, 1)
    vh = torch.from_numpy(v).reshape(m, H, hd).transpose(0, 1)
    ref = F.scaled_dot_product_attention(qh, kh, vh, is_causal=True).transpose(0, 1).reshape(m, H * hd).numpy()
    assert np.allclose(got, ref, rtol=1e-12, atol=1e-12)


def test_enc_attn_sliding_window_matches_masked_sdpa(orc):
    g = synth.generator(41)
    for m, n_ctx, window in [(20, 9, 10), (5, 30, 7), (16, 0, 4), (33, 12, 13)]:
        H, hd = 3, 40
        q = g.standard_normal((m, H * hd))
        k, v = (g.standard_normal((n_ctx + m, H * hd)) for _ in range(2))
        got = orc.enc_attn(q, k, v, H, window)
        assert np.allclose(got, _sdpa_masked(q, k, v, H, n_ctx, window), rtol=1e-12, atol=1e-12)


def test_enc_attn_special_cases(orc):
    g = synth.generator(42)
    m, n_ctx, H, hd = 9, 6, 2, 40
    q = g.standard_normal((m, H * hd))
    k, v = (g.standard_normal((n_ctx + m, H * hd)) for _ in range(2))
    # a window of one position: each query returns its own value row
    assert np.allclose(orc.enc_attn(q, k, v, H, 1), v[n_ctx:], rtol=0, atol=1e-15)
    # equal keys: the mean of the values in the window (first = max(0, n_ctx + i - window + 1))
    w = 4
    kc = np.tile(k[:1], (n_ctx + m, 1))
    got = orc.enc_attn(q, kc, v, H, w)
    ref = np.stack([v[max(0, n_ctx + i - w + 1):n_ctx + i + 1].mean(axis=0) for i in range(m)])
    assert np.allclose(got, ref, rtol=1e-13, atol=1e-13)
    # values of ones give ones (weights sum to one)
    assert np.allclose(orc.enc_attn(q, k, np.ones_like(v), H, 5), 1.0, rtol=0, atol=1e-14)
    # the window edge matters: widening it by one changes every query that had a full window
    a, b = orc.enc_attn(q, k, v, H, 5), orc.enc_attn(q, k, v, H, 6)
    full = [i for i in range(m) if n_ctx + i >= 5]
    assert all(not np.allclose(a[i], b[i]) for i in full)
    # heads are independent: changing head 1's keys leaves head 0's output alone
    k2 = k.copy()
    k2[:, hd:] += g.standard_normal((n_ctx + m, hd))
    c = orc.enc_attn(q, k2, v, H, 5)
    assert np.array_equal(c[:, :hd], a[:, :hd]) and not np.allclose(c[:, hd:], a[:, hd:])
    # adding the same vector to every key of a head shifts each query's scores by a constant: no change
    k3 = k.copy()
    k3[:, hd:] += g.standard_normal(hd)
    assert np.allclose(orc.enc_attn(q, k3, v, H, 5), a, rtol=1e-12, atol=1e-12)


def test_enc_attn_bruteforce_tiny(orc):
    g = synth.generator(43)
    m, n_ctx, H, hd, w = 4, 3, 2, 40, 5
    q = g.standard_normal((m, H * hd))
    k, v = (g.standard_normal((n_ctx + m, H * hd)) for _ in range(2))
    ref = np.zeros((m, H * hd))
    for i in range(m):
        for h in range(H):
            rows = [j for j in range(n_ctx + m) if n_ctx + i - w < j <= n_ctx + i]
            s = [sum(q[i, h * hd + d] * k[j, h * hd + d] for d in range(hd)) / math.sqrt(hd) for j in rows]
            mx = max(s)
            e = [math.exp(x - mx) for x in s]
            z = sum(e)
            for d in range(hd):
                ref[i, h * hd + d] = sum(e[t] / z * v[j, h * hd + d] for t, j in enumerate(rows))
    assert np.allclose(orc.enc_attn(q, k, v, H, w), ref, rtol=1e-12, atol=1e-12)


def test_page_figures_pin_encoder_attention():
    enc = json.load(open(os.path.join(GOLDEN, "page_figures.json")))["encoder"]
    assert (synth.ENC_HEADS, synth.ENC_WINDOW) == (enc["n_heads"], enc["window"])
    assert synth.ENC_HEADS * synth.ENC_HEAD_DIM == enc["dim"]


# ---------------------------------------------------------------------------------------
# 16-bit weights (bf16 and fp16)
# ---------------------------------------------------------------------------------------

def test_w16_gemv_exact_bruteforce(orc):
    # dyadic weights (small integers times powers of two, exact in both formats) and small-integer
    # activations: every product and sum is exact, so the result must equal the rational sum
    g = synth.generator(50)
    n, k = 7, 96
    wi = g.integers(-8, 9, size=(n, k)).astype(np.float32) * np.float32(2.0) ** g.integers(-6, 2, size=(n, k))
    x = g.integers(-5, 6, size=k).astype(np.float32)
    for fmt, bits in (("bf16", synth.bf16_bits(wi)), ("f16", wi.astype(np.float16).view(np.uint16))):
        y = orc.w16_gemv(bits, x, fmt)
        ref = [sum(Fraction(float(wi[r, i])) * Fraction(float(x[i])) for i in range(k)) for r in range(n)]
        assert all(Fraction(y[r]) == ref[r] for r in range(n)), fmt


def test_w16_gemv_random_vs_numpy(orc):
    g = synth.generator(51)
    n, k = 300, 1000
    for fmt in ("bf16", "f16"):
        w, x = synth.w16_matrix(g, n, k, fmt), synth.normal_f32(g, (k,))
        wd = (w.astype(np.uint32) << 16).view(np.float32).astype(np.float64) if fmt == "bf16" \
            else w.view(np.float16).astype(np.float64)
        assert np.allclose(orc.w16_gemv(w, x, fmt), wd @ x.astype(np.float64), rtol=1e-12, atol=1e-12)
    # the two decodings differ: the same bits read as the other format give another result
    w, x = synth.w16_matrix(g, 4, 64, "bf16"), synth.normal_f32(g, (64,))
    assert not np.allclose(orc.w16_gemv(w, x, "bf16"), orc.w16_gemv(w, x, "f16"))


# ---------------------------------------------------------------------------------------
# alternative tokens
# ---------------------------------------------------------------------------------------

def _alt_numpy(l, cutoff, max_out):
    """The same definition through numpy: fp32 threshold, lexicographic sort, scipy softmax."""
    from scipy.special import softmax
    t = int(np.argmax(l))
    d = np.float32(-np.inf) if cutoff >= 1 else np.float32(np.log(1.0 - cutoff))
    tau = np.float32(l[t]) + d
    sel = np.nonzero(l >= tau)[0]
    order = np.lexsort((sel, -l[sel].astype(np.float64)))
    ids = sel[order][:max_out]
    return ids, softmax(l.astype(np.float64))[ids]


def test_alt_tokens_vs_numpy(orc):
    g = synth.generator(60)
    for vocab, cutoff, max_out in [(131072, 0.9, 8), (131072, 0.99, 32), (5000, 0.5, 5), (1000, 1.0, 7),
                                   (64, 0.0, 4), (300, 0.999, 300)]:
        l = (g.standard_normal(vocab) * 3).astype(np.float32)
        ids, probs = orc.alt_tokens(l, cutoff, max_out)
        rid, rprobs = _alt_numpy(l, cutoff, max_out)
        assert np.array_equal(ids, rid), (vocab, cutoff)
        assert np.allclose(probs, rprobs, rtol=1e-12, atol=1e-300)


def test_alt_tokens_closed_forms(orc):
    l = np.float32([1.0, 3.0, 3.0, 2.0, 0.5, 2.9, -np.inf])
    # cutoff 0: only the maximum (its tie too), the lower index first
    ids, probs = orc.alt_tokens(l, 0.0, 5)
    assert list(ids) == [1, 2] and probs[0] == probs[1]
    # p_i >= (1 - c) p_t  <=>  l_i >= l_t + ln(1 - c): c = 1 - e^-0.15 admits 2.9, not 2.0
    ids, _ = orc.alt_tokens(l, 1 - math.exp(-0.15), 5)
    assert list(ids) == [1, 2, 5]
    # cutoff 1: every token by logit, the count capped by max_out
    ids, probs = orc.alt_tokens(l, 1.0, 10)
    assert list(ids) == [1, 2, 5, 3, 0, 4, 6] and probs[-1] == 0.0
    assert list(orc.alt_tokens(l, 1.0, 3)[0]) == [1, 2, 5]
    # probabilities are the softmax over the whole vocabulary
    e = np.exp(l.astype(np.float64) - 3.0)
    assert np.allclose(probs, e[[1, 2, 5, 3, 0, 4, 6]] / e.sum(), rtol=1e-14, atol=0)


def test_alt_tokens_monotone_and_ratio(orc):
    g = synth.generator(61)
    l = (g.standard_normal(20000) * 2).astype(np.float32)
    prev = set()
    for c in (0.0, 0.3, 0.6, 0.9, 0.99, 0.999):
        ids, probs = orc.alt_tokens(l, c, 20000)
        assert prev <= set(ids.tolist())          # a higher cutoff keeps every earlier candidate
        prev = set(ids.tolist())
        assert np.all(probs / probs[0] >= (1 - c) * (1 - 1e-6))
        assert np.all(np.diff(probs) <= 0)
