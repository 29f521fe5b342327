"""The C ABI: the library loads without a GPU, exports every function include/vox.h declares,
and rejects bad arguments before touching the device.  CPU only (no kernel is launched)."""
import ctypes as C
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "vox.h")


PROBE_HEADER = os.path.join(ROOT, "include", "vox_probe.h")


def header_functions(path=HEADER):
    text = open(path).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(vox_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    from streaming_speech_text_amd import vox
    return vox.lib()


def test_header_declares_the_boundary():
    fns = header_functions()
    for name in ("vox_q4_dequant", "vox_q4_gemv", "vox_q4_gemm", "vox_q4_gemm_workspace", "vox_gqa_decode_attn",
                 "vox_gqa_decode_attn_workspace", "vox_adapter", "vox_adapter_workspace", "vox_enc_attn",
                 "vox_enc_attn_workspace", "vox_w16_gemv", "vox_alt_tokens", "vox_alt_tokens_workspace",
                 "vox_decoder_step",
                 "vox_decoder_create", "vox_decoder_workspace", "vox_strerror", "vox_last_error"):
        assert name in fns


def test_library_exports_every_declared_function(lib):
    missing = [f for f in header_functions() if not hasattr(lib, f)]
    assert not missing, f"declared in vox.h but not exported: {missing}"
    assert "vox_gqa_decode_attn_noalloc" in header_functions() and "vox_decoder_seek" in header_functions()


def test_probe_library_exports_its_header():
    # the streaming-read probe (measurement aid) is a library of its own
    path = os.path.join(ROOT, "streaming_speech_text_amd", "libvox_probe.so")
    plib = C.CDLL(path)
    fns = header_functions(PROBE_HEADER)
    assert fns == ["vox_probe_handoff_persistent", "vox_probe_handoff_phase", "vox_probe_handoff_reset",
                   "vox_probe_handoff_work_bytes", "vox_probe_mfma_rate", "vox_probe_mfma_rate_entries",
                   "vox_probe_sink_entries", "vox_probe_stream_read", "vox_probe_stream_read_lds",
                   "vox_probe_stream_read_lds_nt", "vox_probe_stream_read_nt"]
    assert all(hasattr(plib, f) for f in fns)
    for fn in (plib.vox_probe_stream_read, plib.vox_probe_stream_read_nt, plib.vox_probe_stream_read_lds,
               plib.vox_probe_stream_read_lds_nt):
        fn.argtypes = [C.c_void_p, C.c_size_t, C.c_void_p, C.c_int, C.c_void_p]
        # bad arguments are refused before any HIP call
        assert fn(None, 16, C.c_void_p(0x1000), 1, None) == -1
        assert fn(C.c_void_p(0x1000), 24, C.c_void_p(0x1000), 1, None) == -1
        assert fn(C.c_void_p(0x1008), 32, C.c_void_p(0x1000), 1, None) == -1
    plib.vox_probe_mfma_rate.argtypes = [C.c_int, C.c_int, C.c_int, C.c_int, C.c_void_p, C.c_void_p]
    out = C.c_void_p(0x1000)
    assert plib.vox_probe_mfma_rate(2, 0, 1, 16, out, None) == -1     # no such product
    assert plib.vox_probe_mfma_rate(0, 8, 1, 16, out, None) == -1     # fp32 work not in 0/16/32/64
    assert plib.vox_probe_mfma_rate(0, 0, 5, 16, out, None) == -1     # waves per SIMD past 4
    assert plib.vox_probe_mfma_rate(0, 0, 1, 0, out, None) == -1      # no rounds
    assert plib.vox_probe_mfma_rate(1, 0, 1, 16, None, None) == -1    # no output


def test_header_compiles_as_c(tmp_path):
    src = tmp_path / "t.c"
    src.write_text('#include "vox.h"\n#include "vox_probe.h"\nint main(void) { return vox_strerror(0) == 0; }\n')
    import subprocess
    r = subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-fsyntax-only", "-I", os.path.join(ROOT, "include"),
                        str(src)], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


def test_status_strings(lib):
    from streaming_speech_text_amd import vox
    for code in (vox.VOX_OK, vox.VOX_E_INVAL, vox.VOX_E_UNSUPPORTED, vox.VOX_E_WORKSPACE, vox.VOX_E_HIP):
        assert vox.strerror(code)
    assert vox.strerror(12345) == "unknown status"


def test_validation_before_device_work(lib):
    # every call below must fail its host-side checks and return without any HIP call
    from streaming_speech_text_amd import vox
    p = C.c_void_p(0x1000)   # never dereferenced
    assert lib.vox_q4_gemv(p, p, p, 10, 100, None) == vox.VOX_E_INVAL          # k % 32
    assert lib.vox_q4_gemv(p, p, p, -1, 64, None) == vox.VOX_E_INVAL           # n < 0
    assert lib.vox_q4_gemv(None, p, p, 10, 64, None) == vox.VOX_E_INVAL        # null
    assert lib.vox_q4_gemv(p, p, p, 0, 64, None) == vox.VOX_OK                 # empty: no-op
    assert "multiple of 32" in vox.last_error() or vox.last_error() == ""
    assert lib.vox_q4_dequant(p, -1, p, None) == vox.VOX_E_INVAL
    assert lib.vox_q4_dequant(p, 0, p, None) == vox.VOX_OK
    assert lib.vox_q4_gemm(p, p, p, 4, 4, 48, None, 0, None) == vox.VOX_E_INVAL
    assert lib.vox_q4_gemm(p, p, p, 0, 4, 64, None, 0, None) == vox.VOX_OK
    assert lib.vox_q4_gemm(p, p, C.c_void_p(0x800000), 4, 4, 64, p, 0, None) == vox.VOX_E_INVAL   # ws without size
    # the workspace is sized only where K is split: long K on few output tiles
    assert lib.vox_q4_gemm_workspace(64, 1280, 5120) > 0
    assert lib.vox_q4_gemm_workspace(750, 5120, 1280) == 0
    assert lib.vox_q4_gemm_workspace(4, 4, 48) == 0
    # 128 x 128 tiles: K in 4 slices of 10 stages for 60 tiles, in 2 of 12 for 80; one slice from
    # 160 tiles on
    assert lib.vox_q4_gemm_workspace(750, 1280, 5120) == 4 * 750 * 1280 * 4
    assert lib.vox_q4_gemm_workspace(600, 2000, 3072) == 2 * 600 * 2000 * 4
    assert lib.vox_q4_gemm_workspace(750, 3840, 1280) == 0
    # 16-row tiles with the whole K in LDS: up to 64 rows at K = 1280 / 3072, 16 at K = 5120
    assert lib.vox_q4_gemm_workspace(16, 1280, 5120) == 0
    assert lib.vox_q4_gemm_workspace(64, 3840, 1280) == 0
    assert lib.vox_q4_gemm_workspace(64, 3072, 3072) == 0
    # 64 x 32 tiles at K = 1280 instead of K slices of 64 x 64 tiles; not at K = 5120
    assert lib.vox_q4_gemm_workspace(200, 1280, 1280) == 0
    assert lib.vox_q4_gemm_workspace(200, 1280, 5120) == 2 * 200 * 1280 * 4
    assert lib.vox_w16_gemv(p, 0, p, C.c_void_p(0x800000), 10, 12, None) == vox.VOX_E_INVAL    # k % 8
    assert lib.vox_w16_gemv(p, 2, p, C.c_void_p(0x800000), 10, 16, None) == vox.VOX_E_INVAL    # fmt
    assert lib.vox_w16_gemv(p, 1, p, C.c_void_p(0x800000), 0, 16, None) == vox.VOX_OK          # empty
    assert lib.vox_w16_gemv(C.c_void_p(0x1008), 0, p, C.c_void_p(0x800000), 10, 16, None) == vox.VOX_E_UNSUPPORTED
    assert lib.vox_alt_tokens_workspace(131072, 8) == 256 * 8 * 8 + 256 * 20
    assert lib.vox_alt_tokens_workspace(131072, 33) == 0 and lib.vox_alt_tokens_workspace(262145, 8) == 0
    q4 = (p, C.c_void_p(0x200000), C.c_void_p(0x300000), C.c_void_p(0x400000))
    assert lib.vox_alt_tokens(p, 1000, C.c_float(-0.5), 4, *q4[1:], C.c_void_p(0x500000), 4096, None) == vox.VOX_E_INVAL
    assert lib.vox_alt_tokens(p, 1000, C.c_float(0.5), 40, *q4[1:], C.c_void_p(0x500000), 4096, None) == \
        vox.VOX_E_UNSUPPORTED
    assert lib.vox_alt_tokens(p, 1000, C.c_float(0.5), 4, *q4[1:], C.c_void_p(0x500000), 8, None) == vox.VOX_E_WORKSPACE
    # adapter: workspace holds the GELU pairs (2 x bf16 per value) plus the larger product's partials
    assert lib.vox_adapter_workspace(16, 5120, 3072, 3072) >= 16 * 3072 * 4
    assert lib.vox_adapter_workspace(16, 5120, 3072, 3072) % 16 == 0
    assert lib.vox_adapter_workspace(16, 4096, 3072, 3072) == 0       # k without compiled stages
    assert lib.vox_adapter_workspace(16, 5120, 5120, 3072) == 0       # n_mid without compiled stages
    assert lib.vox_adapter_workspace(0, 5120, 3072, 3072) == 0
    # 187 rows: both products on 128 x 128 tiles with K in 4 slices (the GELU pairs, then the
    # larger product's partial tiles); at most 16 rows: the pairs only
    assert lib.vox_adapter_workspace(187, 5120, 3072, 3072) == 187 * 3072 * 4 + 4 * 187 * 3072 * 4
    assert lib.vox_adapter_workspace(16, 5120, 3072, 3072) == 16 * 3072 * 4
    big = C.c_void_p(0x10000000)
    aw = lib.vox_adapter_workspace(4, 1280, 1280, 64)
    assert lib.vox_adapter(p, p, p, p, 4, 48, 1280, 64, big, aw, None) == vox.VOX_E_INVAL          # k % 32
    assert lib.vox_adapter(p, p, p, p, 4, 1280, 1280, 0, big, aw, None) == vox.VOX_OK              # empty
    assert lib.vox_adapter(p, p, p, p, 4, 1024, 1280, 64, big, aw, None) == vox.VOX_E_UNSUPPORTED  # k
    assert lib.vox_adapter(p, p, p, p, 4, 1280, 1280, 64, None, 0, None) == vox.VOX_E_INVAL        # no workspace
    assert lib.vox_adapter(C.c_void_p(0x1008), p, p, big, 4, 1280, 1280, 64, big, aw, None) == \
        vox.VOX_E_UNSUPPORTED                                                                       # alignment
    assert lib.vox_adapter(p, C.c_void_p(0x200000), C.c_void_p(0x400000), C.c_void_p(0x800000), 4, 1280, 1280, 64,
                           big, aw - 16, None) == vox.VOX_E_WORKSPACE
    # encoder attention: short chunks split the key range (a workspace), long ones do not
    assert lib.vox_enc_attn_workspace(16, 749, 32, 40, 750) > 0
    assert lib.vox_enc_attn_workspace(16, 749, 32, 44, 750) > 0
    assert lib.vox_enc_attn_workspace(16, 749, 32, 42, 750) == 0       # head size not a multiple of 4
    assert lib.vox_enc_attn(p, p, p, C.c_void_p(0x800000), 0, 5, 32, 40, 750, 0.1, None, 0, None) == vox.VOX_OK
    assert lib.vox_enc_attn(p, p, p, C.c_void_p(0x800000), 4, 5, 32, 64, 750, 0.1, None, 0, None) == \
        vox.VOX_E_UNSUPPORTED
    assert lib.vox_enc_attn(p, p, p, C.c_void_p(0x800000), 4, -1, 32, 40, 750, 0.1, None, 0, None) == vox.VOX_E_INVAL
    assert lib.vox_enc_attn(p, C.c_void_p(0x200000), C.c_void_p(0x400000), C.c_void_p(0x800000), 16, 749, 32, 40,
                            750, 0.1, None, 0, None) == vox.VOX_E_WORKSPACE
    # v is read with 16-byte loads like q and k: a v offset by 4 bytes is refused before any launch
    assert lib.vox_enc_attn(p, C.c_void_p(0x200000), C.c_void_p(0x400004), C.c_void_p(0x800000), 4, 5, 32, 40,
                            750, 0.1, None, 0, None) == vox.VOX_E_UNSUPPORTED
    ws = lib.vox_gqa_decode_attn_workspace(32, 8, 128, 8192)
    assert ws > 0 and lib.vox_gqa_decode_attn_workspace(32, 8, 64, 8192) == 0
    args = (p, C.c_void_p(0x200000), C.c_void_p(0x400000), C.c_void_p(0x800000))
    assert lib.vox_gqa_decode_attn(*args, 32, 8, 128, 64, 0, 0.1, C.c_void_p(0x900000), ws, None) == vox.VOX_E_INVAL
    assert lib.vox_gqa_decode_attn(*args, 32, 7, 128, 64, 5, 0.1, C.c_void_p(0x900000), ws, None) == vox.VOX_E_INVAL
    assert lib.vox_gqa_decode_attn(*args, 48, 8, 128, 64, 5, 0.1, C.c_void_p(0x900000), ws, None) == \
        vox.VOX_E_UNSUPPORTED
    assert lib.vox_gqa_decode_attn(*args, 32, 8, 128, 64, 5, 0.1, C.c_void_p(0x900000), 8, None) == vox.VOX_E_WORKSPACE
    # output aliasing an input
    assert lib.vox_gqa_decode_attn(p, C.c_void_p(0x200000), C.c_void_p(0x400000), p, 32, 8, 128, 64, 5, 0.1,
                                   C.c_void_p(0x900000), ws, None) == vox.VOX_E_INVAL


def test_decoder_workspace_matches_page_kv_figure(lib):
    # KV ring at the Voxtral decoder shape: 26 x 2 x 8 x 8192 x 128 fp32 = 1,744,830,464 bytes,
    # within the "at most 1.8 GB" KV figure of the voxtral.c page (section 메모리 요구사항)
    from streaming_speech_text_amd import vox
    cfg = vox.DecoderConfig(26, 3072, 32, 8, 128, 9216, 131072, 8192, 1e-5, 1e6)
    kv, sc = vox.decoder_workspace(cfg)
    assert kv == 26 * 2 * 8 * 8192 * 128 * 4 == 1_744_830_464
    assert 0 < sc < 64 << 20
    bad = vox.DecoderConfig(26, 3072, 32, 8, 64, 9216, 131072, 8192, 1e-5, 1e6)
    k2, s2 = C.c_size_t(), C.c_size_t()
    assert lib.vox_decoder_workspace(C.byref(bad), C.byref(k2), C.byref(s2)) == vox.VOX_E_UNSUPPORTED
    bad = vox.DecoderConfig(26, 3072, 32, 7, 128, 9216, 131072, 8192, 1e-5, 1e6)
    assert lib.vox_decoder_workspace(C.byref(bad), C.byref(k2), C.byref(s2)) == vox.VOX_E_INVAL
    assert lib.vox_decoder_step(None, None, None, None, None) == vox.VOX_E_INVAL
    pos = C.c_int64()
    assert lib.vox_decoder_position(None, C.byref(pos)) == vox.VOX_E_INVAL
    # the 16-bit decoder refuses a format other than bf16 / f16 before looking at anything else
    h = C.c_void_p(0x1234)
    assert lib.vox_decoder_create_w16(C.byref(cfg), None, 2, None, 0, None, 0, None, C.byref(h)) == vox.VOX_E_INVAL
    assert not h.value
