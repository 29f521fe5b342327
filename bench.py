"""Benchmark of the streaming Voxtral decoder-step hot path on one MI355X.

Workload (one "step" = one decoder token): the full decoder shape - 26 layers, width 3072,
GQA 32 query / 8 KV heads of 128, SwiGLU 9216, tied Q4_0 embedding / LM head of 131072 rows,
8192-slot KV ring - with random-init Q4_0 weights from the seeded generator.  A 38-position
prefix is teacher-forced (untimed), then K greedy steps run back to back with the token fed
back on the device; each step replays the captured HIP graph of the step.

Printed: one JSON line with decoder ms/token, the roofline of the dominant kernel (the Q4_0
GEMV, timed with HIP events at the LM-head shape over rotating weight copies so that every
launch streams from HBM), and the CPU oracle timed on a bounded sample on the host.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0   # MI355X HBM3E, published


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=64)
    ap.add_argument("--warmup", type=int, default=8)
    ap.add_argument("--gemv-launches", type=int, default=200)
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="budget of the oracle CPU sample")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--leg", choices=["all", "gemv", "kernels", "probe"], default="all",
                    help="gemv: only the GEMV roofline leg and a copy of known size (for counter runs); "
                         "kernels: per-kernel timings of the other workloads, one JSON line each")
    return ap.parse_args()


def kernel_source_digest() -> str:
    h = hashlib.sha256()
    for name in ("gemv_core.h", "q4_gemv.hip", "vox_common.h"):
        with open(os.path.join(ROOT, "streaming_speech_text_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(digest: str, launch_bytes: int):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it was taken
    on the current kernel source; otherwise None."""
    p = os.path.join(ROOT, "profiles", "q4_gemv_lmhead_counters.json")
    try:
        with open(p) as f:
            d = json.load(f)
    except (OSError, ValueError):
        return None
    if d.get("kernel_source_digest") != digest:
        return None
    return d.get("hbm_bytes_per_launch")


def gemv_leg(args, torch, synth, vox, dev, stream):
    """The Q4_0 GEMV at the LM-head shape (131072 x 3072), rotating over weight copies (more
    than 1 GiB in total, so no launch is served from the 256 MB Infinity Cache).  The launches
    are captured in a HIP graph whose replays are timed with HIP events on the stream it runs on
    (median of five), so the per-launch time is the kernel's own duration plus the graph's launch
    gap."""
    n, k = synth.VOXTRAL_DECODER.vocab, synth.VOXTRAL_DECODER.dim
    gw, gx = synth.gemv_inputs(synth.SEED_GEMV, n, k)
    copies = max(1, int(np.ceil(1.1 * 2 ** 30 / gw.nbytes)))
    ws = [torch.from_numpy(gw).to(dev) for _ in range(copies)]
    xd = torch.from_numpy(gx).to(dev)
    y = torch.empty(n, dtype=torch.float32, device=dev)
    gemv_us = timed(torch, stream, lambda i: vox.q4_gemv(ws[i], xd, y), copies, args.gemv_launches)
    launch_bytes = n * synth.q4_row_bytes(k) + 4 * (n + k)
    achieved = launch_bytes / (gemv_us * 1e-6) / 1e9
    print(f"[bench] q4 gemv {n}x{k}: {gemv_us:.2f} us/launch, {achieved:.0f} GB/s", file=sys.stderr, flush=True)
    del ws
    torch.cuda.empty_cache()
    return {"n": n, "k": k, "us": gemv_us, "bytes": launch_bytes, "gbs": achieved}


def probe_lib():
    """The streaming-read probe (include/vox_probe.h), a library of its own beside libvox."""
    import ctypes as C
    path = os.path.join(ROOT, "streaming_speech_text_amd", "libvox_probe.so")
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with python -m streaming_speech_text_amd.build")
    L = C.CDLL(path)
    L.vox_probe_sink_entries.restype = C.c_int
    L.vox_probe_sink_entries.argtypes = [C.c_int]
    L.vox_probe_stream_read.restype = C.c_int
    L.vox_probe_stream_read.argtypes = [C.c_void_p, C.c_size_t, C.c_void_p, C.c_int, C.c_void_p]
    return L


def probe_ceiling(torch, dev, stream, sizes, reps=100):
    """Streaming-read rate (GB/s) of a plain 16-byte-load kernel for each byte count in `sizes`:
    launches read consecutive windows of a buffer of more than 1 GiB (so no window is served from
    the 256 MB Infinity Cache), captured in a graph and timed like the kernels; the best over
    1, 2, 4 and 8 workgroups per compute unit.  Returns {bytes: (us, GB/s, wg_per_cu)}."""
    L = probe_lib()
    GiB = 2 ** 30
    out = {}
    sink = torch.empty(8 * 1024, dtype=torch.int32, device=dev)
    for size in sizes:
        size = (size + 255) // 256 * 256
        n_win = max(2, int(np.ceil(1.1 * GiB / size)))
        buf = torch.empty(n_win * size, dtype=torch.uint8, device=dev)
        buf.fill_(1)
        best = None
        for wg in (1, 2, 4, 8):
            def launch(i, wg=wg):
                st = L.vox_probe_stream_read(buf.data_ptr() + i * size, size, sink.data_ptr(), wg,
                                             torch.cuda.current_stream().cuda_stream)
                if st:
                    raise RuntimeError(f"probe launch failed ({st})")
            us = timed(torch, stream, launch, n_win, reps)
            if best is None or us < best[0]:
                best = (us, size / us / 1e3, wg)
        out[size] = best
        del buf
        torch.cuda.empty_cache()
    return out


def copy_calibration(torch, dev):
    """A plain device copy of known size (256 MiB read + 256 MiB written), the reference the
    HBM byte counters are scaled by."""
    a = torch.ones(64 * 2 ** 20, dtype=torch.float32, device=dev)
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()


def timed(torch, stream, launch, copies, reps, replays=5):
    """Device time (us) of `launch(i)` (which enqueues on the current stream), averaged over `reps`
    launches rotating over `copies`.  The launches are captured once in a HIP graph, so host
    launch cost is not measured; after two warm replays, `replays` replays are timed one by one
    with HIP events on the stream the graph runs on, and the median is returned."""
    for i in range(min(copies, 4)):
        launch(i % copies)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            for i in range(reps):
                launch(i % copies)
    torch.cuda.synchronize()
    for _ in range(2):
        g.replay()
    torch.cuda.synchronize()
    per = []
    for _ in range(replays):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        per.append(e0.elapsed_time(e1) * 1e3 / reps)
    return float(np.median(per))


def kernels_leg(torch, synth, vox, dev, stream):
    """Per-kernel device times of the workloads beside the decoder step: the single 3072x3072
    GEMV, one decoder layer's linears, GQA attention at three ring fills, the encoder-chunk
    GEMM set, the encoder's chunk attention, the GEMV over 16-bit weights, the alternative tokens,
    the adapter.  The weight-streaming measurements rotate over more than 1 GiB of distinct copies."""
    GiB = 2 ** 30
    out = []

    def emit(d):
        print(json.dumps(d), flush=True)
        out.append(d)

    def gemv_case(name, n, k, seed):
        w, x = synth.gemv_inputs(seed, n, k)
        copies = max(2, int(np.ceil(1.1 * GiB / w.nbytes)))
        ws = [torch.from_numpy(w).to(dev) for _ in range(copies)]
        xd = torch.from_numpy(x).to(dev)
        y = torch.empty(n, dtype=torch.float32, device=dev)
        us = timed(torch, stream, lambda i: vox.q4_gemv(ws[i], xd, y), copies, 200)
        b = n * synth.q4_row_bytes(k) + 4 * (n + k)
        emit({"kernel": "q4_gemv", "case": name, "n": n, "k": k, "us": round(us, 3), "bytes": b,
              "gbs": round(b / us / 1e3, 1), "frac_hbm": round(b / us / 1e3 / HBM_PEAK_GBS, 4)})
        del ws

    gemv_case("single 3072x3072", 3072, 3072, synth.SEED_GEMV)
    for i, (name, (n, k)) in enumerate(synth.LAYER_LINEARS.items()):
        gemv_case(f"layer {name}", n, k, 100 * synth.SEED_LAYER + i)
    torch.cuda.empty_cache()

    # attention over an 8192-slot ring
    nq, nkv, hd, slots = 32, 8, 128, 8192
    q, kc, vc = synth.attention_inputs(synth.SEED_ATTN, nq, nkv, hd, slots)
    copies = max(2, int(np.ceil(1.1 * GiB / (kc.nbytes + vc.nbytes))))
    ks = [torch.from_numpy(kc).to(dev) for _ in range(copies)]
    vs = [torch.from_numpy(vc).to(dev) for _ in range(copies)]
    qd = torch.from_numpy(q).to(dev)
    o = torch.empty(nq, hd, dtype=torch.float32, device=dev)
    wsb = vox.gqa_decode_attn_workspace(nq, nkv, hd, slots)
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
    for L in (1024, 4096, 8192):
        us = timed(torch, stream, lambda i: vox.gqa_decode_attn(qd, ks[i], vs[i], o, nq, nkv, hd, slots, L,
                                                                 1 / np.sqrt(hd), ws), copies, 100)
        b = 8192 * L + 2 * nq * hd * 4
        emit({"kernel": "gqa_decode_attn", "case": f"n_valid {L}", "us": round(us, 3), "bytes": b,
              "gbs": round(b / us / 1e3, 1), "frac_hbm": round(b / us / 1e3 / HBM_PEAK_GBS, 4)})
    del ks, vs
    torch.cuda.empty_cache()

    # encoder-chunk GEMM set: the six linears of one layer, each M
    for m in synth.ENCODER_M:
        sets = []
        for name, n, k in synth.ENCODER_LINEARS:
            w, xb = synth.gemm_inputs(synth.SEED_GEMM, m, n, k)
            sets.append((name, n, k, w, torch.from_numpy(xb.view(np.int16)).to(dev)))
        wbytes = sum(s_[3].nbytes for s_ in sets)
        copies = max(2, int(np.ceil(1.1 * GiB / wbytes)))
        wdev = [[torch.from_numpy(s_[3]).to(dev) for s_ in sets] for _ in range(copies)]
        ys = [torch.empty(m, s_[1], dtype=torch.float32, device=dev) for s_ in sets]
        # one workspace serves the set (the launches run one after another on the stream)
        wsb = max(vox.q4_gemm_workspace(m, n, k) for _, n, k in synth.ENCODER_LINEARS)
        gws = torch.empty(max(wsb, 1), dtype=torch.uint8, device=dev)

        def launch(i):
            for j, (name, n, k, _, xd) in enumerate(sets):
                vox._check(vox.lib().vox_q4_gemm(vox._ptr(wdev[i][j]), vox._ptr(xd), vox._ptr(ys[j]), m, n, k,
                                                 vox._ptr(gws) if wsb else None, wsb, vox._stream(None)))
        us = timed(torch, stream, launch, copies, 50)
        flops = 2 * m * sum(n * k for _, n, k in synth.ENCODER_LINEARS)
        b = wbytes + sum(m * k * 2 + m * n * 4 for _, n, k in synth.ENCODER_LINEARS)
        emit({"kernel": "q4_gemm", "case": f"encoder linears set, M={m}", "us": round(us, 3), "flops": flops,
              "tflops": round(flops / us / 1e6, 2), "frac_mfma_bf16": round(flops / us / 1e6 / 2500.0, 4),
              "bytes": b, "gbs": round(b / us / 1e3, 1), "frac_hbm": round(b / us / 1e3 / HBM_PEAK_GBS, 4)})
        del wdev
        torch.cuda.empty_cache()

    # encoder self-attention over a chunk (32 heads x 40, window 750, a full window of earlier rows)
    H, W = synth.ENC_HEADS, synth.ENC_WINDOW
    hd, n_ctx = synth.ENC_HEAD_DIM, synth.ENC_WINDOW - 1
    for m in synth.ENCODER_M:
        q, k, v = synth.enc_attention_inputs(synth.SEED_ENC_ATTN, m, n_ctx)
        per = q.nbytes + k.nbytes + v.nbytes
        copies = max(2, int(np.ceil(1.1 * GiB / per)))
        qs = [torch.from_numpy(q).to(dev) for _ in range(copies)]
        kvs = [(torch.from_numpy(k).to(dev), torch.from_numpy(v).to(dev)) for _ in range(copies)]
        o = torch.empty(m, H * hd, dtype=torch.float32, device=dev)
        wsb = vox.enc_attn_workspace(m, n_ctx, H, hd, W)
        ews = torch.empty(max(wsb, 1), dtype=torch.uint8, device=dev)

        def launch(i):
            vox._check(vox.lib().vox_enc_attn(vox._ptr(qs[i]), vox._ptr(kvs[i][0]), vox._ptr(kvs[i][1]), vox._ptr(o), m,
                                              n_ctx, H, hd, W, hd ** -0.5, vox._ptr(ews) if wsb else None, wsb,
                                              vox._stream(None)))
        us = timed(torch, stream, launch, copies, 50)
        keys = sum(min(n_ctx + i + 1, W) for i in range(m))
        flops = 4 * keys * hd * H          # scores and weighted sums, as defined
        b = per + o.numel() * 4
        emit({"kernel": "enc_attn", "case": f"M={m}, {n_ctx} earlier rows", "us": round(us, 3), "flops": flops,
              "tflops": round(flops / us / 1e6, 2), "frac_mfma_fp32": round(flops / us / 1e6 / 157.3, 4),
              "bytes": b, "gbs": round(b / us / 1e3, 1)})
        del qs, kvs
        torch.cuda.empty_cache()

    # GEMV over 16-bit weights: the LM-head shape, then every GEMV of a decoder step (26 layers of
    # q, k, v, o, gate, up, down and the LM head, 4.2 GB of distinct weights) as one chain
    s_ = synth.VOXTRAL_DECODER
    for fmt in ("bf16", "f16"):
        n, k = s_.vocab, s_.dim
        w, x = synth.w16_gemv_inputs(synth.SEED_W16, n, k, fmt)
        head = [torch.from_numpy(w).to(dev) for _ in range(2)]
        del w
        xd = torch.from_numpy(x).to(dev)
        y = torch.empty(n, dtype=torch.float32, device=dev)
        us = timed(torch, stream, lambda i: vox.w16_gemv(head[i], xd, y, fmt), 2, 50)
        b = n * k * 2 + 4 * (n + k)
        emit({"kernel": "w16_gemv", "case": f"{fmt} {n}x{k} (LM-head shape)", "us": round(us, 3), "bytes": b,
              "gbs": round(b / us / 1e3, 1), "frac_hbm": round(b / us / 1e3 / HBM_PEAK_GBS, 4)})
        layer = []
        for j, (name, (ln, lk)) in enumerate(synth.LAYER_LINEARS.items()):
            lw, lx = synth.w16_gemv_inputs(synth.SEED_W16 + 1 + j, ln, lk, fmt)
            layer.append((ln, lk, torch.from_numpy(lw).to(dev), torch.from_numpy(lx).to(dev),
                          torch.empty(ln, dtype=torch.float32, device=dev)))
        chain = [[(ln, lk, wt.clone(), xt, yt) for ln, lk, wt, xt, yt in layer] for _ in range(s_.n_layers)]
        del layer

        def step(i):
            for lay in chain:
                for ln, lk, wt, xt, yt in lay:
                    vox.w16_gemv(wt, xt, yt, fmt)
            vox.w16_gemv(head[0], xd, y, fmt)
        us = timed(torch, stream, step, 1, 3)
        b = s_.n_layers * sum(o * i * 2 for o, i in synth.LAYER_LINEARS.values()) + n * k * 2
        emit({"kernel": "w16_gemv", "case": f"{fmt} decoder-step GEMV chain (26 layers + LM head)", "us": round(us, 3),
              "bytes": b, "gbs": round(b / us / 1e3, 1), "frac_hbm": round(b / us / 1e3 / HBM_PEAK_GBS, 4)})
        del chain, head
        torch.cuda.empty_cache()

    # the greedy token and its alternatives from one step's logits (vocabulary 131072)
    V = synth.VOXTRAL_DECODER.vocab
    lg = (synth.normal_f32(synth.generator(synth.SEED_DECODER, 9), (V,)) * np.float32(3.0))
    lgs = [torch.from_numpy(lg).to(dev) for _ in range(4)]
    for max_out in (8, 32):
        ids = torch.empty(max_out, dtype=torch.int32, device=dev)
        probs = torch.empty(max_out, dtype=torch.float32, device=dev)
        cnt = torch.empty(1, dtype=torch.int32, device=dev)
        aws = torch.empty(vox.alt_tokens_workspace(V, max_out), dtype=torch.uint8, device=dev)
        us = timed(torch, stream, lambda i: vox.alt_tokens(lgs[i], 0.9, max_out, ids, probs, cnt, aws), 4, 50)
        emit({"kernel": "alt_tokens", "case": f"vocab {V}, cutoff 0.9, max_out {max_out}", "us": round(us, 3),
              "bytes": V * 4, "gbs": round(V * 4 / us / 1e3, 1)})
    del lgs

    # adapter (linear 5120 -> 3072, GELU, linear 3072 -> 3072) over the rows of one encoder chunk
    k, n_mid, n_out = synth.ADAPTER
    for m in synth.ADAPTER_M:
        w1, w2, xb = synth.adapter_inputs(synth.SEED_ADAPTER, m, k, n_mid, n_out)
        wbytes = w1.nbytes + w2.nbytes
        copies = max(2, int(np.ceil(1.1 * GiB / wbytes)))
        w1s = [torch.from_numpy(w1).to(dev) for _ in range(copies)]
        w2s = [torch.from_numpy(w2).to(dev) for _ in range(copies)]
        xd = torch.from_numpy(xb.view(np.int16)).to(dev)
        y = torch.empty(m, n_out, dtype=torch.float32, device=dev)
        wsb = vox.adapter_workspace(m, k, n_mid, n_out)
        aws = torch.empty(wsb, dtype=torch.uint8, device=dev)

        def launch(i):
            vox._check(vox.lib().vox_adapter(vox._ptr(w1s[i]), vox._ptr(w2s[i]), vox._ptr(xd), vox._ptr(y), m, k, n_mid,
                                             n_out, vox._ptr(aws), wsb, vox._stream(None)))
        us = timed(torch, stream, launch, copies, 50)
        flops = 2 * m * (n_mid * k + n_out * n_mid)   # the two products as defined
        b = wbytes + m * k * 2 + m * n_out * 4
        emit({"kernel": "adapter", "case": f"{k}->{n_mid}->{n_out}, M={m} rows", "us": round(us, 3), "flops": flops,
              "tflops": round(flops / us / 1e6, 2), "bytes": b, "gbs": round(b / us / 1e3, 1),
              "frac_hbm": round(b / us / 1e3 / HBM_PEAK_GBS, 4)})
        del w1s, w2s
        torch.cuda.empty_cache()
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the layout over several GPUs "
              "is designed but not built.", file=sys.stderr)
        sys.exit(2)

    import torch
    from streaming_speech_text_amd import synth, vox

    vox.lib()   # raises if the HIP library is missing
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    if args.leg == "gemv":
        copy_calibration(torch, dev)
        g = gemv_leg(args, torch, synth, vox, dev, stream)
        print(json.dumps({"leg": "gemv", **g}), flush=True)
        return
    if args.leg == "kernels":
        kernels_leg(torch, synth, vox, dev, stream)
        return
    if args.leg == "probe":
        # the decoder kernels' byte counts (O, QKV, down, gate/up, LM head), config 1, and a sweep
        sizes = [7077888, 10616832, 15925248, 31850496, 226492416, 5308416, 1 << 20, 4 << 20, 16 << 20,
                 64 << 20, 256 << 20]
        for b, (us, gbs, wg) in probe_ceiling(torch, dev, stream, sizes).items():
            print(json.dumps({"leg": "probe", "bytes": b, "us": round(us, 3), "gbs": round(gbs, 1),
                              "frac_hbm": round(gbs / HBM_PEAK_GBS, 4), "wg_per_cu": wg}), flush=True)
        return
    s = synth.VOXTRAL_DECODER
    print(f"[bench] generating weights ({s.n_layers} layers, vocab {s.vocab})", file=sys.stderr, flush=True)
    w = synth.decoder_weights(synth.SEED_DECODER, s)
    wd = {"tok_embd": torch.from_numpy(w["tok_embd"]).to(dev), "out_norm": torch.from_numpy(w["out_norm"]).to(dev),
          "layers": [{k: torch.from_numpy(v).to(dev) for k, v in L.items()} for L in w["layers"]]}
    cfg = vox.DecoderConfig(s.n_layers, s.dim, s.n_heads, s.n_kv_heads, s.head_dim, s.hidden, s.vocab, s.n_slots,
                            s.norm_eps, s.rope_theta)
    dec = vox.Decoder(cfg, wd)
    prefix, start = synth.decoder_tokens(synth.SEED_DECODER, s.vocab)
    tok = torch.zeros(1, dtype=torch.int32, device=dev)

    def run_prefix():
        dec.reset()
        for t in prefix:
            tok.fill_(int(t))
            dec.step(tok, tok)
        tok.fill_(start)

    # warmup: captures the graphs of every attention bucket the timed positions use
    print("[bench] warmup", file=sys.stderr, flush=True)
    run_prefix()
    for _ in range(max(args.warmup, args.steps)):
        dec.step(tok, tok)
    torch.cuda.synchronize()

    run_prefix()
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        dec.step(tok, tok)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_token = wall * 1e3 / args.steps
    dev_ms = ev0.elapsed_time(ev1) / args.steps
    last_token = int(tok.item())
    step_weight_bytes = (s.n_layers * sum(o * synth.q4_row_bytes(i) for o, i in synth.LAYER_LINEARS.values())
                         + s.vocab * synth.q4_row_bytes(s.dim) + synth.q4_row_bytes(s.dim))
    kv_bytes = sum(s.n_layers * 2 * s.n_kv_heads * s.head_dim * 4 * min(p + 1, s.n_slots)
                   for p in range(len(prefix), len(prefix) + args.steps)) / args.steps
    step_bytes = step_weight_bytes + kv_bytes
    print(f"[bench] decoder {ms_per_token:.4f} ms/token (device {dev_ms:.4f}), "
          f"{step_bytes / (ms_per_token * 1e-3) / 1e9:.0f} GB/s", file=sys.stderr, flush=True)
    dec.close()
    del wd
    torch.cuda.empty_cache()

    gemv = gemv_leg(args, torch, synth, vox, dev, stream)
    traffic = measured_traffic(kernel_source_digest(), gemv["bytes"])

    # CPU baseline: the oracle on the host cores, bounded sample of the same decoder workload
    cpu = None
    if not args.no_cpu:
        import oracle
        threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
        od = oracle.Decoder(s, w)
        times = []
        t_start = time.perf_counter()
        for t in list(prefix):
            a = time.perf_counter()
            od.step(int(t), want_logits=False)
            times.append(time.perf_counter() - a)
            if time.perf_counter() - t_start > args.cpu_seconds and len(times) >= 3:
                break
        od.close()
        cpu = {"value": round(1e3 * float(np.mean(times)), 3), "unit": "ms/token", "cores": threads,
               "kind": "oracle",
               "sample": f"first {len(times)} teacher-forced steps of the 38-token prefix at the full decoder "
                         f"shape (fp64 oracle, OpenMP over output rows)"}

    out = {
        "metric": "decoder ms/token + Q4_0 GEMV achieved HBM GB/s (% of peak), 1 MI355X",
        "value": round(ms_per_token, 4),
        "unit": "ms/token",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_token, 4),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "q4_0 weights x fp32 activations, fp32 accumulate",
        "data": "synthetic (seeded random-init Q4_0 weights, seeded token ids)",
        "config": {"workload": "Voxtral decoder step: 26 layers, dim 3072, GQA 32/8 x 128, SwiGLU 9216, "
                               "tied Q4_0 head 131072, 8192-slot KV ring, 38-token prefix then greedy steps",
                   "tokens_timed": args.steps, "kv_positions": [len(prefix), len(prefix) + args.steps]},
        "roofline": {"bound": "hbm", "achieved": round(gemv["gbs"], 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gemv["gbs"] / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "kernel": f"q4_gemv {gemv['n']}x{gemv['k']} (LM-head shape)", "bytes_per_launch": gemv["bytes"],
                     "us_per_launch": round(gemv["us"], 3)},
        "decoder_device_ms_per_token": round(dev_ms, 4),
        "decoder_hbm_gbs": round(step_bytes / (ms_per_token * 1e-3) / 1e9, 1),
        "decoder_bytes_per_token": int(step_bytes),
        "last_token": last_token,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
