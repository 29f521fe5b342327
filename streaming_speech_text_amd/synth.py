"""Seeded synthetic inputs for the streaming Voxtral decoder-step hot path.

This module only draws random numbers and lays them out in the storage formats the
path consumes (GGUF Q4_0 blocks, fp32 vectors, bf16 matrices, KV rings).  It holds
none of the method's arithmetic: no dequantisation, no products, no normalisation.
Both the HIP path and the CPU oracle are fed from here, so the two see the same bytes.

Model shapes come from the voxtral.c summary page ("Mistral Voxtral Realtime 4B 음성 인식
모델의 순수 C 기반 CPU 전용 추론 구현", GeekNews 26608, section 모델 아키텍처): decoder of 26
layers, width 3072, GQA with 32 query and 8 KV heads, Tekken vocabulary of 131,072; and
section 주요 기능: a rolling KV window of 8192 positions.  The Rust/Burn port page
("Mistral의 Voxtral Mini 4B Realtime 모델을 Rust로 구현해 브라우저에서 실행", GeekNews 26595,
section 아키텍처) names GGUF Q4_0 for every linear of the quantised path.  Head size 128,
SwiGLU width 9216, RMSNorm eps 1e-5 and RoPE base 1e6 are not on the pages; they are the
readings this build adopts (the 1.8 GB KV figure in section 메모리 요구사항 of the voxtral.c
page is consistent with fp32 K/V at head size 128 over 8192 positions).

Value distributions: Q4_0 scales d ~ U[0.001, 0.02] rounded to fp16 (round to nearest
even), nibbles ~ U{0..15}; activations, queries, keys and values ~ N(0, 1) in fp32;
GEMM activations ~ N(0, 1) rounded to bf16 (round to nearest even); RMSNorm gains
~ U[0.5, 1.5] (a random-init model has no trained gains; non-unit gains keep a dropped
multiply visible).
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

Q4_BLOCK = 32          # weights per GGUF Q4_0 block
Q4_BLOCK_BYTES = 18    # 2-byte fp16 scale followed by 16 bytes of packed nibbles


def generator(seed: int, *stream: int) -> np.random.Generator:
    """PCG64 generator for workload `seed`, child stream `stream` (a tuple of ints)."""
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=tuple(stream))))


def q4_row_bytes(k: int) -> int:
    if k % Q4_BLOCK:
        raise ValueError(f"k={k} is not a multiple of {Q4_BLOCK}")
    return (k // Q4_BLOCK) * Q4_BLOCK_BYTES


def q4_matrix(g: np.random.Generator, n: int, k: int, d_lo: float = 0.001, d_hi: float = 0.02) -> np.ndarray:
    """Random GGUF Q4_0 matrix of n rows by k inputs, as uint8 [n, k/32*18].

    Each block: bytes 0..1 hold the fp16 scale (little-endian), bytes 2..17 are uniform
    random bytes.  A uniform byte has independent uniform low and high nibbles, so the
    nibbles are U{0..15} without this module having to know which nibble is which element.
    """
    nb = k // Q4_BLOCK
    if nb * Q4_BLOCK != k:
        raise ValueError(f"k={k} is not a multiple of {Q4_BLOCK}")
    out = np.empty((n, nb, Q4_BLOCK_BYTES), dtype=np.uint8)
    d = g.uniform(d_lo, d_hi, size=(n, nb)).astype("<f2")
    out[:, :, 0:2] = d.view(np.uint8).reshape(n, nb, 2)
    out[:, :, 2:] = g.integers(0, 256, size=(n, nb, 16), dtype=np.uint8)
    return out.reshape(n, nb * Q4_BLOCK_BYTES)


def normal_f32(g: np.random.Generator, shape) -> np.ndarray:
    return g.standard_normal(shape, dtype=np.float32)


def uniform_f32(g: np.random.Generator, shape, lo: float, hi: float) -> np.ndarray:
    return g.uniform(lo, hi, size=shape).astype(np.float32)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round finite fp32 values to bf16 (nearest, ties to even); returns the uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def bf16_normal(g: np.random.Generator, shape) -> np.ndarray:
    return bf16_bits(normal_f32(g, shape))


# ---------------------------------------------------------------------------------------
# Workload shapes
# ---------------------------------------------------------------------------------------

@dataclass(frozen=True)
class DecoderShape:
    n_layers: int = 26
    dim: int = 3072
    n_heads: int = 32
    n_kv_heads: int = 8
    head_dim: int = 128
    hidden: int = 9216
    vocab: int = 131072
    n_slots: int = 8192
    norm_eps: float = 1e-5
    rope_theta: float = 1e6


VOXTRAL_DECODER = DecoderShape()
DECODER_PREFIX = 38       # KV prefix length of the decoder (Rust port page, section Q4 패딩 보정)
DECODER_STEPS = 64        # greedy steps timed after the prefix

# One decoder layer's linears (out, in) at the Voxtral decoder shape.
LAYER_LINEARS = {
    "q": (4096, 3072), "k": (1024, 3072), "v": (1024, 3072), "o": (3072, 4096),
    "gate": (9216, 3072), "up": (9216, 3072), "down": (3072, 9216),
}
# Encoder-chunk linears (out, in): width 1280 (voxtral.c page, section 모델 아키텍처), FFN 5120.
ENCODER_LINEARS = [("q", 1280, 1280), ("k", 1280, 1280), ("v", 1280, 1280), ("o", 1280, 1280),
                   ("ffn_up", 5120, 1280), ("ffn_down", 1280, 5120)]
ENCODER_M = (16, 64, 200, 750)
# Encoder self-attention: 32 heads over the 1280 width (head size 40), causal with a window of 750
# positions (voxtral.c page, section 모델 아키텍처).  A chunk of M frames attends over its own rows
# and the window's worth of earlier rows, 749 of them once the stream is past its start.
ENC_HEADS, ENC_WINDOW = 32, 750
ENC_HEAD_DIM = ENCODER_LINEARS[0][1] // ENC_HEADS
# Adapter (in, mid, out): a linear 5120 -> 3072, GELU, a linear 3072 -> 3072 (voxtral.c page,
# section 모델 아키텍처).  It reads the encoder output four frames to a row (4 x 1280 = 5120), so an
# encoder chunk of M frames gives M / 4 adapter rows.
ADAPTER = (5120, 3072, 3072)
ADAPTER_M = tuple(m // 4 for m in ENCODER_M)

# Seeds: one per workload.
SEED_GEMV, SEED_LAYER, SEED_ATTN, SEED_DECODER, SEED_GEMM, SEED_ADAPTER, SEED_ENC_ATTN, SEED_W16 = 1, 2, 3, 4, 5, 6, 7, 8


def gemv_inputs(seed: int, n: int, k: int):
    """(W q4 [n, k/32*18], x fp32 [k])."""
    return q4_matrix(generator(seed, 0), n, k), normal_f32(generator(seed, 1), (k,))


def gemm_inputs(seed: int, m: int, n: int, k: int):
    """(W q4 [n, k/32*18], X bf16 bits [m, k])."""
    return q4_matrix(generator(seed, 0, n, k), n, k), bf16_normal(generator(seed, 1, m, k), (m, k))


def w16_matrix(g: np.random.Generator, n: int, k: int, fmt: str) -> np.ndarray:
    """Random 16-bit weight matrix, uint16 [n, k]: values ~ N(0, 0.02^2) (the spread of a
    trained linear's weights at this width) rounded to bf16 or fp16 (nearest even)."""
    v = g.standard_normal((n, k), dtype=np.float32) * np.float32(0.02)
    if fmt == "bf16":
        return bf16_bits(v)
    if fmt == "f16":
        return v.astype(np.float16).view(np.uint16)
    raise ValueError(fmt)


def w16_gemv_inputs(seed: int, n: int, k: int, fmt: str):
    """(W uint16 [n, k], x fp32 [k])."""
    return w16_matrix(generator(seed, 0, n, k), n, k, fmt), normal_f32(generator(seed, 1, k), (k,))


def adapter_inputs(seed: int, m: int, k: int, n_mid: int, n_out: int):
    """(W1 q4 [n_mid, k/32*18], W2 q4 [n_out, n_mid/32*18], X bf16 bits [m, k])."""
    return (q4_matrix(generator(seed, 0, n_mid, k), n_mid, k), q4_matrix(generator(seed, 1, n_out, n_mid), n_out, n_mid),
            bf16_normal(generator(seed, 2, m, k), (m, k)))


def enc_attention_inputs(seed: int, m: int, n_ctx: int, width: int = 1280):
    """(q [m, width], k [n_ctx + m, width], v [n_ctx + m, width]) fp32 N(0, 1); row n_ctx + i of k
    and v belongs to query i."""
    return (normal_f32(generator(seed, 0, m, n_ctx), (m, width)), normal_f32(generator(seed, 1, m, n_ctx), (n_ctx + m, width)),
            normal_f32(generator(seed, 2, m, n_ctx), (n_ctx + m, width)))


def attention_inputs(seed: int, n_q_heads: int, n_kv_heads: int, head_dim: int, n_slots: int):
    """(q [n_q, hd], K ring [n_kv, n_slots, hd], V ring [n_kv, n_slots, hd]) all fp32 N(0,1)."""
    q = normal_f32(generator(seed, 0), (n_q_heads, head_dim))
    kc = normal_f32(generator(seed, 1), (n_kv_heads, n_slots, head_dim))
    vc = normal_f32(generator(seed, 2), (n_kv_heads, n_slots, head_dim))
    return q, kc, vc


def decoder_weights(seed: int, s: DecoderShape):
    """Random-init decoder weights: a dict with 'tok_embd' (tied Q4_0 embedding / LM head),
    'out_norm', and 'layers' (list of dicts with attn_norm, ffn_norm, wq, wk, wv, wo,
    w_gate, w_up, w_down)."""
    qd = s.n_heads * s.head_dim
    kvd = s.n_kv_heads * s.head_dim
    layers = []
    for li in range(s.n_layers):
        def g(t):
            return generator(seed, 1, li, t)
        layers.append({
            "attn_norm": uniform_f32(g(0), (s.dim,), 0.5, 1.5),
            "ffn_norm": uniform_f32(g(1), (s.dim,), 0.5, 1.5),
            "wq": q4_matrix(g(2), qd, s.dim),
            "wk": q4_matrix(g(3), kvd, s.dim),
            "wv": q4_matrix(g(4), kvd, s.dim),
            "wo": q4_matrix(g(5), s.dim, qd),
            "w_gate": q4_matrix(g(6), s.hidden, s.dim),
            "w_up": q4_matrix(g(7), s.hidden, s.dim),
            "w_down": q4_matrix(g(8), s.dim, s.hidden),
        })
    return {
        "tok_embd": q4_matrix(generator(seed, 0, 0), s.vocab, s.dim),
        "out_norm": uniform_f32(generator(seed, 0, 1), (s.dim,), 0.5, 1.5),
        "layers": layers,
    }


def decoder_weights_w16(seed: int, s: DecoderShape, fmt: str):
    """The same structure over 16-bit weights ("bf16" or "f16"): every linear and the tied table
    uint16 [n, k] (w16_matrix: N(0, 0.02^2) rounded to the format); norms as decoder_weights."""
    qd = s.n_heads * s.head_dim
    kvd = s.n_kv_heads * s.head_dim
    layers = []
    for li in range(s.n_layers):
        def g(t):
            return generator(seed, 3, li, t)
        layers.append({
            "attn_norm": uniform_f32(g(0), (s.dim,), 0.5, 1.5),
            "ffn_norm": uniform_f32(g(1), (s.dim,), 0.5, 1.5),
            "wq": w16_matrix(g(2), qd, s.dim, fmt),
            "wk": w16_matrix(g(3), kvd, s.dim, fmt),
            "wv": w16_matrix(g(4), kvd, s.dim, fmt),
            "wo": w16_matrix(g(5), s.dim, qd, fmt),
            "w_gate": w16_matrix(g(6), s.hidden, s.dim, fmt),
            "w_up": w16_matrix(g(7), s.hidden, s.dim, fmt),
            "w_down": w16_matrix(g(8), s.dim, s.hidden, fmt),
        })
    return {
        "tok_embd": w16_matrix(generator(seed, 3, 0), s.vocab, s.dim, fmt),
        "out_norm": uniform_f32(generator(seed, 3, 1), (s.dim,), 0.5, 1.5),
        "layers": layers,
    }


def decoder_tokens(seed: int, vocab: int, prefix: int = DECODER_PREFIX):
    """(prefix token ids [prefix] int32, start id int) for a decoder run."""
    g = generator(seed, 2)
    ids = g.integers(0, vocab, size=prefix + 1, dtype=np.int64).astype(np.int32)
    return ids[:prefix], int(ids[prefix])
