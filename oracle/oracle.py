"""ctypes front end of the CPU oracle (liboracle.so, built from oracle.c).

TEST INFRASTRUCTURE ONLY (tests, smoke check, benchmark CPU baseline).  Marshals numpy
arrays into the C functions; every number is computed in oracle.c.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# VOX_ORACLE_LIB selects another build of the same source (the sanitizer build, oracle/build.py)
_LIB_PATH = os.environ.get("VOX_ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")
_lib = None

_i64 = C.c_int64
_dbl = C.c_double
_vp = C.c_void_p


class DecoderConfig(C.Structure):
    _fields_ = [("n_layers", _i64), ("dim", _i64), ("n_heads", _i64), ("n_kv_heads", _i64),
                ("head_dim", _i64), ("hidden", _i64), ("vocab", _i64), ("n_slots", _i64),
                ("norm_eps", _dbl), ("rope_theta", _dbl)]


class LayerWeights(C.Structure):
    _fields_ = [("attn_norm", _vp), ("ffn_norm", _vp), ("wq", _vp), ("wk", _vp), ("wv", _vp),
                ("wo", _vp), ("w_gate", _vp), ("w_up", _vp), ("w_down", _vp)]


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            from . import build as _b
            _b.build()
        L = C.CDLL(_LIB_PATH)
        L.orc_fp16_to_double.restype = _dbl
        L.orc_fp16_to_double.argtypes = [C.c_uint16]
        L.orc_bf16_to_double.restype = _dbl
        L.orc_bf16_to_double.argtypes = [C.c_uint16]
        for name, args in {
            "orc_fp16_to_double_array": [_vp, _i64, _vp],
            "orc_bf16_to_double_array": [_vp, _i64, _vp],
            "orc_q4_dequant": [_vp, _i64, _vp],
            "orc_q4_gemv": [_vp, _vp, _vp, _i64, _i64],
            "orc_q4_gemv_f64": [_vp, _vp, _vp, _i64, _i64],
            "orc_q4_gemv_rows": [_vp, _vp, _vp, _i64, _vp, _i64],
            "orc_q4_gemm": [_vp, _vp, _vp, _i64, _i64, _i64],
            "orc_rmsnorm": [_vp, _vp, _i64, _dbl, _vp],
            "orc_rope": [_vp, _i64, _i64, _i64, _dbl],
            "orc_attn_probs": [_vp, _vp, _i64, _i64, _i64, _dbl, _vp],
            "orc_gqa_attn": [_vp, _vp, _vp, _i64, _i64, _i64, _i64, _dbl, _vp],
            "orc_swiglu": [_vp, _vp, _i64, _vp],
            "orc_w16_gemv": [_vp, _i64, _vp, _vp, _i64, _i64],
            "orc_gelu_array": [_vp, _i64, _vp],
            "orc_adapter": [_vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64],
            "orc_enc_attn": [_vp, _vp, _vp, _i64, _i64, _i64, _i64, _i64, _dbl, _vp],
            "orc_decoder_destroy": [_vp],
            "orc_decoder_reset": [_vp],
            "orc_decoder_load_window": [_vp, _i64, _vp, _vp],
        }.items():
            f = getattr(L, name)
            f.restype = None
            f.argtypes = args
        L.orc_alt_tokens.restype = _i64
        L.orc_alt_tokens.argtypes = [_vp, _i64, _dbl, _i64, _vp, _vp]
        L.orc_argmax_f32.restype = _i64
        L.orc_argmax_f32.argtypes = [_vp, _i64]
        L.orc_argmax_f64.restype = _i64
        L.orc_argmax_f64.argtypes = [_vp, _i64]
        L.orc_set_num_threads.restype = None
        L.orc_set_num_threads.argtypes = [_i64]
        L.orc_max_threads.restype = _i64
        L.orc_max_threads.argtypes = []
        L.orc_decoder_create.restype = _vp
        L.orc_decoder_create.argtypes = [C.POINTER(DecoderConfig), _vp, _vp, C.POINTER(LayerWeights)]
        L.orc_decoder_create_w16.restype = _vp
        L.orc_decoder_create_w16.argtypes = [C.POINTER(DecoderConfig), _i64, _vp, _vp, C.POINTER(LayerWeights)]
        L.orc_decoder_position.restype = _i64
        L.orc_decoder_position.argtypes = [_vp]
        L.orc_decoder_step.restype = _i64
        L.orc_decoder_step.argtypes = [_vp, _i64, _vp]
        L.orc_decoder_hidden.restype = C.POINTER(C.c_double)
        L.orc_decoder_hidden.argtypes = [_vp]
        _lib = L
    return _lib


def _p(a: np.ndarray):
    return a.ctypes.data_as(_vp)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def fp16_to_double(h) -> np.ndarray:
    h = _c(h, np.uint16)
    out = np.empty(h.shape, np.float64)
    lib().orc_fp16_to_double_array(_p(h), h.size, _p(out))
    return out


def bf16_to_double(b) -> np.ndarray:
    b = _c(b, np.uint16)
    out = np.empty(b.shape, np.float64)
    lib().orc_bf16_to_double_array(_p(b), b.size, _p(out))
    return out


def q4_dequant(blocks) -> np.ndarray:
    """blocks: uint8 [..., 18*nb] -> float32 [nb*32] (flattened in block order)."""
    b = _c(blocks, np.uint8)
    nb = b.size // 18
    out = np.empty(nb * 32, np.float32)
    lib().orc_q4_dequant(_p(b), nb, _p(out))
    return out


def q4_gemv(w, x) -> np.ndarray:
    """w: uint8 [n, k/32*18]; x: float32 [k] -> float64 [n]."""
    w = _c(w, np.uint8)
    x = _c(x, np.float32)
    k = x.size
    n = w.size // ((k // 32) * 18)
    y = np.empty(n, np.float64)
    lib().orc_q4_gemv(_p(w), _p(x), _p(y), n, k)
    return y


def q4_gemv_f64(w, x) -> np.ndarray:
    w = _c(w, np.uint8)
    x = _c(x, np.float64)
    k = x.size
    n = w.size // ((k // 32) * 18)
    y = np.empty(n, np.float64)
    lib().orc_q4_gemv_f64(_p(w), _p(x), _p(y), n, k)
    return y


def q4_gemv_rows(w, x, rows) -> np.ndarray:
    w = _c(w, np.uint8)
    x = _c(x, np.float32)
    rows = _c(rows, np.int64)
    y = np.empty(rows.size, np.float64)
    lib().orc_q4_gemv_rows(_p(w), _p(x), _p(rows), rows.size, _p(y), x.size)
    return y


def q4_gemm(w, x_bf16) -> np.ndarray:
    """w: uint8 [n, k/32*18]; x_bf16: uint16 [m, k] -> float64 [m, n]."""
    w = _c(w, np.uint8)
    x = _c(x_bf16, np.uint16)
    m, k = x.shape
    n = w.size // ((k // 32) * 18)
    y = np.empty((m, n), np.float64)
    lib().orc_q4_gemm(_p(w), _p(x), _p(y), m, n, k)
    return y


def rmsnorm(x, g, eps) -> np.ndarray:
    x = _c(x, np.float64)
    g = _c(g, np.float32)
    out = np.empty_like(x)
    lib().orc_rmsnorm(_p(x), _p(g), x.size, float(eps), _p(out))
    return out


def rope(x, n_heads, head_dim, pos, theta) -> np.ndarray:
    x = np.array(x, dtype=np.float64, copy=True)
    lib().orc_rope(_p(x), n_heads, head_dim, pos, float(theta))
    return x


def attn_probs(q, k, scale) -> np.ndarray:
    """q: [hd]; k: [len, hd] -> p [len]."""
    q = _c(q, np.float64)
    k = _c(k, np.float64)
    length, hd = k.shape
    p = np.empty(length, np.float64)
    lib().orc_attn_probs(_p(q), _p(k), length, hd, hd, float(scale), _p(p))
    return p


def gqa_attn(q, k, v, scale) -> np.ndarray:
    """q: [n_q, hd]; k, v: [n_kv, len, hd] in chronological order -> out [n_q, hd]."""
    q = _c(q, np.float64)
    k = _c(k, np.float64)
    v = _c(v, np.float64)
    n_q, hd = q.shape
    n_kv, length, _ = k.shape
    out = np.empty((n_q, hd), np.float64)
    lib().orc_gqa_attn(_p(q), _p(k), _p(v), n_q, n_kv, hd, length, float(scale), _p(out))
    return out


def swiglu(gate, up) -> np.ndarray:
    gate = _c(gate, np.float64)
    up = _c(up, np.float64)
    out = np.empty_like(gate)
    lib().orc_swiglu(_p(gate), _p(up), gate.size, _p(out))
    return out


def w16_gemv(w, x, fmt: str) -> np.ndarray:
    """w: uint16 [n, k] bit patterns of bf16 (fmt 'bf16') or fp16 (fmt 'f16'); x: float32 [k] -> float64 [n]."""
    w = _c(w, np.uint16)
    x = _c(x, np.float32)
    n, k = w.shape
    y = np.empty(n, np.float64)
    lib().orc_w16_gemv(_p(w), {"bf16": 0, "f16": 1}[fmt], _p(x), _p(y), n, k)
    return y


def gelu(x) -> np.ndarray:
    x = _c(x, np.float64)
    out = np.empty_like(x)
    lib().orc_gelu_array(_p(x), x.size, _p(out))
    return out


def adapter(w1, w2, x_bf16) -> np.ndarray:
    """w1: uint8 [n_mid, k/32*18]; w2: uint8 [n_out, n_mid/32*18]; x_bf16: uint16 [m, k]
    -> float64 [m, n_out] = GELU(X W1^T) W2^T."""
    w1 = _c(w1, np.uint8)
    w2 = _c(w2, np.uint8)
    x = _c(x_bf16, np.uint16)
    m, k = x.shape
    n_mid = w1.size // ((k // 32) * 18)
    n_out = w2.size // ((n_mid // 32) * 18)
    y = np.empty((m, n_out), np.float64)
    lib().orc_adapter(_p(w1), _p(w2), _p(x), _p(y), m, k, n_mid, n_out)
    return y


def enc_attn(q, k, v, n_heads, window, scale=None) -> np.ndarray:
    """q: [m, n_heads*hd]; k, v: [n_ctx + m, n_heads*hd] (query i at row n_ctx + i)
    -> out [m, n_heads*hd] (float64).  scale defaults to 1/sqrt(hd)."""
    q = _c(q, np.float64)
    k = _c(k, np.float64)
    v = _c(v, np.float64)
    m, width = q.shape
    n_ctx = k.shape[0] - m
    hd = width // n_heads
    if scale is None:
        scale = 1.0 / np.sqrt(hd)
    out = np.empty((m, width), np.float64)
    lib().orc_enc_attn(_p(q), _p(k), _p(v), m, n_ctx, n_heads, hd, window, float(scale), _p(out))
    return out


def alt_tokens(logits, cutoff, max_out):
    """-> (ids int64 [count], probs float64 [count]): the greedy token and its alternatives."""
    lg = _c(logits, np.float32)
    ids = np.empty(max_out, np.int64)
    probs = np.empty(max_out, np.float64)
    n = int(lib().orc_alt_tokens(_p(lg), lg.size, float(cutoff), int(max_out), _p(ids), _p(probs)))
    return ids[:n].copy(), probs[:n].copy()


def argmax_f32(v) -> int:
    v = _c(v, np.float32)
    return int(lib().orc_argmax_f32(_p(v), v.size))


def argmax_f64(v) -> int:
    v = _c(v, np.float64)
    return int(lib().orc_argmax_f64(_p(v), v.size))


def set_num_threads(n: int):
    """OpenMP threads of the oracle's loops (timing only; results do not depend on it)."""
    lib().orc_set_num_threads(int(n))


def max_threads() -> int:
    return int(lib().orc_max_threads())


class Decoder:
    """Oracle decoder over host weights (as produced by the synthetic generator): Q4_0 matrices,
    or with fmt "bf16" / "f16" 16-bit matrices (uint16 [n, k]) for every linear and the table."""

    def __init__(self, shape, weights, fmt=None):
        s = shape
        self.shape = s
        self._keep = []

        def keep(a, dtype):
            a = _c(a, dtype)
            self._keep.append(a)
            return _p(a)

        self.cfg = DecoderConfig(s.n_layers, s.dim, s.n_heads, s.n_kv_heads, s.head_dim, s.hidden,
                                 s.vocab, s.n_slots, s.norm_eps, s.rope_theta)
        arr = (LayerWeights * s.n_layers)()
        for i, L in enumerate(weights["layers"]):
            wt = np.uint8 if fmt is None else np.uint16
            arr[i] = LayerWeights(keep(L["attn_norm"], np.float32), keep(L["ffn_norm"], np.float32),
                                  keep(L["wq"], wt), keep(L["wk"], wt), keep(L["wv"], wt),
                                  keep(L["wo"], wt), keep(L["w_gate"], wt),
                                  keep(L["w_up"], wt), keep(L["w_down"], wt))
        self._layers = arr
        if fmt is None:
            self._h = lib().orc_decoder_create(C.byref(self.cfg), keep(weights["tok_embd"], np.uint8),
                                               keep(weights["out_norm"], np.float32), arr)
        else:
            code = {"bf16": 0, "f16": 1}[fmt]
            self._h = lib().orc_decoder_create_w16(C.byref(self.cfg), code, keep(weights["tok_embd"], np.uint16),
                                                   keep(weights["out_norm"], np.float32), arr)

    def step(self, token: int, want_logits: bool = True):
        logits = np.empty(self.shape.vocab, np.float64) if want_logits else None
        nxt = lib().orc_decoder_step(self._h, int(token), _p(logits) if want_logits else None)
        return int(nxt), logits

    def reset(self):
        lib().orc_decoder_reset(self._h)

    def load_window(self, pos: int, k, v):
        """Resume at position `pos`; k, v fp32 [n_layers, len, n_kv*head_dim], oldest first,
        len = min(pos, n_slots)."""
        s = self.shape
        n = min(pos, s.n_slots)
        k = _c(k, np.float32)
        v = _c(v, np.float32)
        assert k.shape == v.shape == (s.n_layers, n, s.n_kv_heads * s.head_dim)
        lib().orc_decoder_load_window(self._h, int(pos), _p(k), _p(v))

    @property
    def position(self) -> int:
        return int(lib().orc_decoder_position(self._h))

    def hidden(self) -> np.ndarray:
        p = lib().orc_decoder_hidden(self._h)
        return np.ctypeslib.as_array(p, shape=(self.shape.dim,)).copy()

    def close(self):
        if self._h:
            lib().orc_decoder_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
