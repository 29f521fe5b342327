"""Thin Python binding of libvox (the C ABI in include/vox.h).

Argument marshalling only: torch tensors supply device memory and the current HIP stream;
every step of the computation runs in the library's HIP kernels.  The library must be
built (streaming_speech_text_amd/build.py); importing this module without it raises.
"""
from __future__ import annotations

import ctypes as C
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libvox.so")

VOX_OK, VOX_E_INVAL, VOX_E_UNSUPPORTED, VOX_E_WORKSPACE, VOX_E_HIP = 0, -1, -2, -3, -4

_vp = C.c_void_p
_i64 = C.c_int64
_int = C.c_int
_sz = C.c_size_t
_f32 = C.c_float


class VoxError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"[{status}] {msg}")
        self.status = status


class DecoderConfig(C.Structure):
    _fields_ = [("n_layers", _int), ("dim", _int), ("n_heads", _int), ("n_kv_heads", _int),
                ("head_dim", _int), ("hidden", _int), ("vocab", _int), ("n_slots", _int),
                ("norm_eps", _f32), ("rope_theta", _f32)]


class LayerWeights(C.Structure):
    _fields_ = [("attn_norm", _vp), ("ffn_norm", _vp), ("wq", _vp), ("wk", _vp), ("wv", _vp),
                ("wo", _vp), ("w_gate", _vp), ("w_up", _vp), ("w_down", _vp)]


class DecoderWeights(C.Structure):
    _fields_ = [("tok_embd", _vp), ("out_norm", _vp), ("layers", C.POINTER(LayerWeights))]


_lib = None

_SIGS = {
    "vox_strerror": (C.c_char_p, [_int]),
    "vox_last_error": (C.c_char_p, []),
    "vox_q4_dequant": (_int, [_vp, _i64, _vp, _vp]),
    "vox_q4_gemv": (_int, [_vp, _vp, _vp, _i64, _i64, _vp]),
    "vox_w16_gemv": (_int, [_vp, _int, _vp, _vp, _i64, _i64, _vp]),
    "vox_q4_gemm_workspace": (_sz, [_i64, _i64, _i64]),
    "vox_q4_gemm": (_int, [_vp, _vp, _vp, _i64, _i64, _i64, _vp, _sz, _vp]),
    "vox_adapter_workspace": (_sz, [_i64, _i64, _i64, _i64]),
    "vox_adapter": (_int, [_vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _vp, _sz, _vp]),
    "vox_enc_attn_workspace": (_sz, [_i64, _i64, _int, _int, _int]),
    "vox_enc_attn": (_int, [_vp, _vp, _vp, _vp, _i64, _i64, _int, _int, _int, _f32, _vp, _sz, _vp]),
    "vox_gqa_decode_attn_workspace": (_sz, [_int, _int, _int, _int]),
    "vox_gqa_decode_attn": (_int, [_vp, _vp, _vp, _vp, _int, _int, _int, _int, _int, _f32, _vp, _sz, _vp]),
    "vox_gqa_decode_attn_noalloc": (_int, [_vp, _vp, _vp, _vp, _int, _int, _int, _int, _int, _f32, _vp]),
    "vox_alt_tokens_workspace": (_sz, [_i64, _int]),
    "vox_alt_tokens": (_int, [_vp, _i64, _f32, _int, _vp, _vp, _vp, _vp, _sz, _vp]),
    "vox_decoder_workspace": (_int, [C.POINTER(DecoderConfig), C.POINTER(_sz), C.POINTER(_sz)]),
    "vox_decoder_create": (_int, [C.POINTER(DecoderConfig), C.POINTER(DecoderWeights), _vp, _sz, _vp, _sz, _vp,
                                  C.POINTER(_vp)]),
    "vox_decoder_create_w16": (_int, [C.POINTER(DecoderConfig), C.POINTER(DecoderWeights), _int, _vp, _sz, _vp, _sz, _vp,
                                  C.POINTER(_vp)]),
    "vox_decoder_reset": (_int, [_vp, _vp]),
    "vox_decoder_seek": (_int, [_vp, _i64, _vp]),
    "vox_decoder_step": (_int, [_vp, _vp, _vp, _vp, _vp]),
    "vox_decoder_position": (_int, [_vp, C.POINTER(_i64)]),
    "vox_decoder_set_graph": (_int, [_vp, _int]),
    "vox_decoder_destroy": (None, [_vp]),
}


def lib():
    """Loads libvox.so (raises ImportError if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "python -m streaming_speech_text_amd.build")
        L = C.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            if not hasattr(L, name):
                continue   # calling it raises AttributeError; the ABI test checks exports
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def strerror(status: int) -> str:
    return lib().vox_strerror(status).decode()


def last_error() -> str:
    return lib().vox_last_error().decode()


def _check(status: int):
    if status != VOX_OK:
        raise VoxError(status, f"{strerror(status)}: {last_error()}")


def _stream(stream):
    if stream is None:
        return _vp(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, torch.cuda.Stream):
        return _vp(stream.cuda_stream)
    return _vp(stream)


def _ptr(t, dtype=None, name="tensor"):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        return _vp(int(t))
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return _vp(t.data_ptr())


def q4_dequant(w_q4, out, n_blocks=None, stream=None):
    n_blocks = w_q4.numel() // 18 if n_blocks is None else n_blocks
    _check(lib().vox_q4_dequant(_ptr(w_q4, torch.uint8, "w_q4"), n_blocks, _ptr(out, torch.float32, "out"),
                                _stream(stream)))


def q4_gemv(w_q4, x, y, n=None, k=None, stream=None):
    k = x.numel() if k is None else k
    n = y.numel() if n is None else n
    _check(lib().vox_q4_gemv(_ptr(w_q4, torch.uint8, "w_q4"), _ptr(x, torch.float32, "x"),
                             _ptr(y, torch.float32, "y"), n, k, _stream(stream)))


VOX_W16_BF16, VOX_W16_F16 = 0, 1


def w16_gemv(w, x, y, fmt="bf16", n=None, k=None, stream=None):
    """y = W x over 16-bit weights: w uint16 (or bfloat16 / float16) [n, k], x fp32 [k], y fp32 [n]."""
    if n is None or k is None:
        n, k = w.shape
    code = {"bf16": VOX_W16_BF16, "f16": VOX_W16_F16}[fmt]
    _check(lib().vox_w16_gemv(_ptr(w, None, "w"), code, _ptr(x, torch.float32, "x"), _ptr(y, torch.float32, "y"),
                              n, k, _stream(stream)))


def q4_gemm_workspace(m, n, k) -> int:
    return int(lib().vox_q4_gemm_workspace(m, n, k))


def q4_gemm(w_q4, x_bf16, y, m=None, n=None, k=None, workspace=None, stream=None):
    """workspace: None (K is never split) or a device buffer of at least q4_gemm_workspace(m, n, k)
    bytes (a zero-size request needs none)."""
    if m is None or k is None:
        m, k = x_bf16.shape
    n = y.shape[-1] if n is None else n
    xdt = torch.uint16 if x_bf16.dtype == torch.uint16 else torch.bfloat16
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().vox_q4_gemm(_ptr(w_q4, torch.uint8, "w_q4"), _ptr(x_bf16, xdt, "x_bf16"),
                             _ptr(y, torch.float32, "y"), m, n, k,
                             _ptr(workspace, None, "workspace") if wsb else None, wsb, _stream(stream)))


def adapter_workspace(m, k, n_mid, n_out) -> int:
    return int(lib().vox_adapter_workspace(m, k, n_mid, n_out))


def adapter(w1_q4, w2_q4, x_bf16, y, workspace, m=None, k=None, n_mid=None, n_out=None, stream=None):
    """Y = GELU(X W1^T) W2^T; workspace: a device buffer of at least adapter_workspace(m, k, n_mid, n_out)
    bytes."""
    if m is None or k is None:
        m, k = x_bf16.shape
    n_out = y.shape[-1] if n_out is None else n_out
    if n_mid is None:
        n_mid = w1_q4.numel() // ((k // 32) * 18)
    xdt = torch.uint16 if x_bf16.dtype == torch.uint16 else torch.bfloat16
    wsb = workspace.numel() * workspace.element_size()
    _check(lib().vox_adapter(_ptr(w1_q4, torch.uint8, "w1_q4"), _ptr(w2_q4, torch.uint8, "w2_q4"),
                             _ptr(x_bf16, xdt, "x_bf16"), _ptr(y, torch.float32, "y"), m, k, n_mid, n_out,
                             _ptr(workspace, None, "workspace"), wsb, _stream(stream)))


def enc_attn_workspace(m, n_ctx, n_heads, head_dim, window) -> int:
    return int(lib().vox_enc_attn_workspace(m, n_ctx, n_heads, head_dim, window))


def enc_attn(q, k, v, out, n_heads, window, scale=None, workspace=None, stream=None):
    """Encoder self-attention over a chunk: q [m, width], k/v [n_ctx + m, width], out [m, width] (fp32);
    workspace: None or a device buffer of at least enc_attn_workspace(...) bytes."""
    m, width = q.shape
    n_ctx = k.shape[0] - m
    hd = width // n_heads
    if scale is None:
        scale = hd ** -0.5
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().vox_enc_attn(_ptr(q, torch.float32, "q"), _ptr(k, torch.float32, "k"), _ptr(v, torch.float32, "v"),
                              _ptr(out, torch.float32, "out"), m, n_ctx, n_heads, hd, window, scale,
                              _ptr(workspace, None, "workspace") if wsb else None, wsb, _stream(stream)))


def alt_tokens_workspace(vocab, max_out) -> int:
    return int(lib().vox_alt_tokens_workspace(vocab, max_out))


def alt_tokens(logits, cutoff, max_out, ids, probs, count, workspace, stream=None):
    """Greedy token and alternatives: logits fp32 [vocab]; ids int32 [max_out], probs fp32 [max_out],
    count int32 [1] (device); workspace >= alt_tokens_workspace(vocab, max_out) bytes."""
    wsb = workspace.numel() * workspace.element_size()
    _check(lib().vox_alt_tokens(_ptr(logits, torch.float32, "logits"), logits.numel(), float(cutoff), int(max_out),
                                _ptr(ids, torch.int32, "ids"), _ptr(probs, torch.float32, "probs"),
                                _ptr(count, torch.int32, "count"), _ptr(workspace, None, "workspace"), wsb,
                                _stream(stream)))


def gqa_decode_attn_workspace(n_q_heads, n_kv_heads, head_dim, n_slots) -> int:
    return int(lib().vox_gqa_decode_attn_workspace(n_q_heads, n_kv_heads, head_dim, n_slots))


def gqa_decode_attn(q, k_cache, v_cache, out, n_q_heads, n_kv_heads, head_dim, n_slots, n_valid, scale,
                    workspace, workspace_bytes=None, stream=None):
    wsb = workspace.numel() * workspace.element_size() if workspace_bytes is None else workspace_bytes
    _check(lib().vox_gqa_decode_attn(_ptr(q, torch.float32, "q"), _ptr(k_cache, torch.float32, "k_cache"),
                                     _ptr(v_cache, torch.float32, "v_cache"), _ptr(out, torch.float32, "out"),
                                     n_q_heads, n_kv_heads, head_dim, n_slots, n_valid, float(scale),
                                     _ptr(workspace, None, "workspace"), wsb, _stream(stream)))


def gqa_decode_attn_noalloc(q, k_cache, v_cache, out, n_q_heads, n_kv_heads, head_dim, n_slots, n_valid, scale,
                            stream=None):
    """gqa_decode_attn without a workspace: the library's fixed per-GPU scratch holds the split partials."""
    _check(lib().vox_gqa_decode_attn_noalloc(_ptr(q, torch.float32, "q"), _ptr(k_cache, torch.float32, "k_cache"),
                                             _ptr(v_cache, torch.float32, "v_cache"), _ptr(out, torch.float32, "out"),
                                             n_q_heads, n_kv_heads, head_dim, n_slots, n_valid, float(scale),
                                             _stream(stream)))


def decoder_workspace(cfg: DecoderConfig):
    kv = _sz()
    sc = _sz()
    _check(lib().vox_decoder_workspace(C.byref(cfg), C.byref(kv), C.byref(sc)))
    return int(kv.value), int(sc.value)


class Decoder:
    """Owns a vox_decoder_t over device weights and caller-allocated buffers.

    `weights` holds device tensors: tok_embd (uint8), out_norm (fp32), and a list of layer
    dicts with attn_norm, ffn_norm, wq, wk, wv, wo, w_gate, w_up, w_down.  fmt None: Q4_0
    matrices (uint8 bytes); "bf16" / "f16": 16-bit matrices (uint16 / int16 [n, k])."""

    def __init__(self, cfg: DecoderConfig, weights, kv=None, scratch=None, stream=None, fmt=None):
        self.cfg = cfg
        kv_bytes, sc_bytes = decoder_workspace(cfg)
        dev = weights["tok_embd"].device
        self.kv = torch.empty(kv_bytes, dtype=torch.uint8, device=dev) if kv is None else kv
        self.scratch = torch.empty(sc_bytes, dtype=torch.uint8, device=dev) if scratch is None else scratch
        self._weights = weights   # keep device memory alive
        n = cfg.n_layers
        self._layers = (LayerWeights * n)()
        for i, L in enumerate(weights["layers"]):
            self._layers[i] = LayerWeights(*[_ptr(L[f], None, f) for f in
                                             ("attn_norm", "ffn_norm", "wq", "wk", "wv", "wo",
                                              "w_gate", "w_up", "w_down")])
        self._w = DecoderWeights(_ptr(weights["tok_embd"], torch.uint8 if fmt is None else None, "tok_embd"),
                                 _ptr(weights["out_norm"], torch.float32, "out_norm"), self._layers)
        h = _vp()
        if fmt is None:
            _check(lib().vox_decoder_create(C.byref(cfg), C.byref(self._w), _ptr(self.kv), kv_bytes,
                                            _ptr(self.scratch), sc_bytes, _stream(stream), C.byref(h)))
        else:
            code = {"bf16": VOX_W16_BF16, "f16": VOX_W16_F16}[fmt]
            _check(lib().vox_decoder_create_w16(C.byref(cfg), C.byref(self._w), code, _ptr(self.kv), kv_bytes,
                                                _ptr(self.scratch), sc_bytes, _stream(stream), C.byref(h)))
        self._h = h

    def step(self, token_in, token_out, logits=None, stream=None):
        _check(lib().vox_decoder_step(self._h, _ptr(token_in, torch.int32, "token_in"),
                                      _ptr(token_out, torch.int32, "token_out"),
                                      _ptr(logits, torch.float32, "logits"), _stream(stream)))

    def reset(self, stream=None):
        _check(lib().vox_decoder_reset(self._h, _stream(stream)))

    def seek(self, pos: int, stream=None):
        """Resume at absolute position `pos`; the KV ring must hold positions max(0, pos - n_slots) ..
        pos - 1 at slots p % n_slots."""
        _check(lib().vox_decoder_seek(self._h, int(pos), _stream(stream)))

    def set_graph(self, enable: bool):
        _check(lib().vox_decoder_set_graph(self._h, 1 if enable else 0))

    @property
    def position(self) -> int:
        p = _i64()
        _check(lib().vox_decoder_position(self._h, C.byref(p)))
        return int(p.value)

    def close(self):
        if getattr(self, "_h", None):
            lib().vox_decoder_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
