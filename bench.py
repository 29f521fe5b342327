"""Benchmark of the streaming Voxtral decoder-step hot path on one MI355X.

Workload (one "step" = one decoder token): the full decoder shape - 26 layers, width 3072,
GQA 32 query / 8 KV heads of 128, SwiGLU 9216, tied Q4_0 embedding / LM head of 131072 rows,
8192-slot KV ring - with random-init Q4_0 weights from the seeded generator.  A 38-position
prefix is teacher-forced (untimed), then K greedy steps run back to back with the token fed
back on the device; each step replays the captured HIP graph of the step.

Printed: one JSON line with decoder ms/token (median of five sequences of K steps, each timed
with HIP events on the stream the steps run on), the decoder at a full, wrapped 8192-position
window, the roofline of the dominant kernel (the Q4_0 GEMV, timed with HIP events at the LM-head
shape over rotating weight copies so that every launch streams from HBM) next to the read ceiling
of the streaming probe at the same byte count, a GEMV sweep over row counts at K = 3072, the
decoder's own dominant kernel from the committed kernel trace, the encoder-chunk GEMM set at 16
and 750 frames, and the CPU oracle timed on bounded samples on the host (at all its threads and
at one).

Other modes: --leg kernels (per-kernel timings of the other workloads), --leg gemv (the GEMV leg
alone, for counter runs), --leg probe (read ceilings and the grid-handoff probe), and
--summarize-trace CSV (per-kernel statistics of a rocprofv3 kernel trace).
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
    ap.add_argument("--sequences", type=int, default=5, help="decoder sequences timed (median reported)")
    ap.add_argument("--leg", choices=["all", "decoder", "decoder_full", "decoder_w16", "gemv", "kernels", "probe"],
                    default="all",
                    help="gemv: only the GEMV roofline leg and a copy of known size (for counter runs); "
                         "kernels: per-kernel timings of the other workloads, one JSON line each; "
                         "probe: read ceilings and the grid-handoff probe; decoder: only the decoder at the "
                         "bench configuration (for kernel traces); decoder_full: the decoder at the bench "
                         "configuration, then at a full, wrapped 8192-position window; decoder_w16: only the "
                         "decoder over f16 weights")
    ap.add_argument("--summarize-trace", metavar="CSV", help="print per-kernel statistics of a rocprofv3 "
                    "kernel_trace.csv (calls, mean, p10/p50/p90, min, max in us) and exit")
    ap.add_argument("--trace-json", metavar="OUT", help="with --summarize-trace: also write the statistics with "
                    "the digest of the decoder sources (the decoder_roofline input) to OUT")
    ap.add_argument("--decoder-steps", type=int, default=0, help="with --trace-json: decoder steps in the trace")
    ap.add_argument("--summarize-counters", metavar="CSV", help="print per-dispatch counter means of a rocprofv3 "
                    "--pmc counter_collection.csv per kernel and launch shape and exit")
    ap.add_argument("--counter-summary", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="HBM bytes per launch of the LM-head-shape GEMV from two rocprofv3 --pmc runs of "
                         "--leg gemv (FETCH_SIZE, then WRITE_SIZE), scaled by what the same counters read for "
                         "the leg's 256 MiB copies; prints the JSON that bench.py reads as `traffic`")
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
    per = timed_all(torch, stream, lambda i: vox.q4_gemv(ws[i], xd, y), copies, args.gemv_launches, replays=10)
    gemv_us = float(np.median(per))
    launch_bytes = n * synth.q4_row_bytes(k) + 4 * (n + k)
    achieved = launch_bytes / (gemv_us * 1e-6) / 1e9
    print(f"[bench] q4 gemv {n}x{k}: {gemv_us:.2f} us/launch, {achieved:.0f} GB/s", file=sys.stderr, flush=True)
    del ws
    torch.cuda.empty_cache()
    return {"n": n, "k": k, "us": gemv_us, "bytes": launch_bytes, "gbs": achieved,
            "spread": {"p10": round(float(np.percentile(per, 10)), 3), "p90": round(float(np.percentile(per, 90)), 3),
                       "replays": len(per), "launches_per_replay": args.gemv_launches}}


def probe_lib():
    """The streaming-read probe (include/vox_probe.h), a library of its own beside libvox."""
    import ctypes as C
    path = os.path.join(ROOT, "streaming_speech_text_amd", "libvox_probe.so")
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with python -m streaming_speech_text_amd.build")
    L = C.CDLL(path)
    L.vox_probe_sink_entries.restype = C.c_int
    L.vox_probe_sink_entries.argtypes = [C.c_int]
    for fn in (L.vox_probe_stream_read, L.vox_probe_stream_read_nt, L.vox_probe_stream_read_lds,
               L.vox_probe_stream_read_lds_nt):
        fn.restype = C.c_int
        fn.argtypes = [C.c_void_p, C.c_size_t, C.c_void_p, C.c_int, C.c_void_p]
    return L


def probe_ceiling(torch, dev, stream, sizes, reps=100, lds=False):
    """Streaming-read rate (GB/s) of a 16-byte-load kernel for each byte count in `sizes`:
    launches read consecutive windows of a buffer of more than 1 GiB (so no window is served from
    the 256 MB Infinity Cache), captured in a graph and timed like the kernels; the best over
    plain and non-temporal loads and 1, 2, 4 and 8 workgroups per compute unit (lds: instead the
    direct-to-LDS forms of the same loads at 1, 2 and 4 workgroups, whose 32 KB of LDS each allow
    no more).  Returns {bytes: (us, GB/s, wg_per_cu, loads)}."""
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
        forms = (((L.vox_probe_stream_read_lds, "direct-to-LDS"), (L.vox_probe_stream_read_lds_nt,
                  "direct-to-LDS non-temporal")) if lds else
                 ((L.vox_probe_stream_read, "plain"), (L.vox_probe_stream_read_nt, "non-temporal")))
        for fn, loads in forms:
            for wg in ((1, 2, 4) if lds else (1, 2, 4, 8)):
                def launch(i, wg=wg, fn=fn):
                    st = fn(buf.data_ptr() + i * size, size, sink.data_ptr(), wg, torch.cuda.current_stream().cuda_stream)
                    if st:
                        raise RuntimeError(f"probe launch failed ({st})")
                us = timed(torch, stream, launch, n_win, reps)
                if best is None or us < best[0]:
                    best = (us, size / us / 1e3, wg, loads)
        out[size] = best
        del buf
        torch.cuda.empty_cache()
    return out


def probe_leg(torch, dev, stream):
    """Read ceilings at the decoder kernels' byte counts (O, QKV, down, gate/up, LM head), config 1
    and a size sweep; then the grid-handoff probe: a persistent kernel with a grid barrier per
    phase (two barrier forms) against one launch per phase, with 0, 8, 16 and 32 MB of weights
    streamed per phase."""
    sizes = [7077888, 10616832, 15925248, 31850496, 226492416, 5308416, 1 << 20, 4 << 20, 16 << 20,
             64 << 20, 256 << 20]
    for b, (us, gbs, wg, loads) in probe_ceiling(torch, dev, stream, sizes).items():
        print(json.dumps({"leg": "probe", "bytes": b, "us": round(us, 3), "gbs": round(gbs, 1),
                          "frac_hbm": round(gbs / HBM_PEAK_GBS, 4), "wg_per_cu": wg, "loads": loads}), flush=True)
    # the same reads with direct-to-LDS loads (the data bypasses the registers) at the decoder
    # kernels' byte counts
    for b, (us, gbs, wg, loads) in probe_ceiling(torch, dev, stream, sizes[:6], lds=True).items():
        print(json.dumps({"leg": "probe", "bytes": b, "us": round(us, 3), "gbs": round(gbs, 1),
                          "frac_hbm": round(gbs / HBM_PEAK_GBS, 4), "wg_per_cu": wg, "loads": loads}), flush=True)
    import ctypes as C
    L = probe_lib()
    L.vox_probe_handoff_work_bytes.restype = C.c_size_t
    L.vox_probe_handoff_work_bytes.argtypes = []
    L.vox_probe_handoff_reset.argtypes = [C.c_void_p, C.c_void_p]
    L.vox_probe_handoff_persistent.argtypes = [C.c_int, C.c_int, C.c_int, C.c_void_p, C.c_size_t, C.c_void_p,
                                               C.c_void_p]
    L.vox_probe_handoff_phase.argtypes = [C.c_int, C.c_int, C.c_void_p, C.c_size_t, C.c_void_p, C.c_void_p]
    work = torch.empty(L.vox_probe_handoff_work_bytes(), dtype=torch.uint8, device=dev)
    wbytes = 1200 << 20
    wts = torch.empty(wbytes, dtype=torch.uint8, device=dev)
    wts.fill_(1)
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    nphase = 300

    def cur():
        return torch.cuda.current_stream().cuda_stream

    def status():
        torch.cuda.synchronize()
        c = work[:16].view(torch.int32).cpu().tolist()
        return {"expired_waits": c[1], "values_wrong": c[2]}

    for nch in (0, 4, 8, 16):
        phase_bytes = 8192 * nch * cus
        for mode, name in ((0, "persistent, gathered flags"), (1, "persistent, eight counters"),
                           (2, "persistent, poller wave")):
            per = []
            for _ in range(5):
                L.vox_probe_handoff_reset(work.data_ptr(), cur())
                torch.cuda.synchronize()
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                st = L.vox_probe_handoff_persistent(mode, nch, nphase, wts.data_ptr(), wbytes, work.data_ptr(), cur())
                e1.record(stream)
                if st:
                    raise RuntimeError(f"handoff probe failed ({st})")
                torch.cuda.synchronize()
                per.append(e0.elapsed_time(e1) * 1e3 / nphase)
            print(json.dumps({"leg": "handoff", "mode": name, "phase_bytes": phase_bytes,
                              "us_per_phase": round(float(np.median(per)), 3), **status()}), flush=True)
        L.vox_probe_handoff_reset(work.data_ptr(), cur())

        def launch(i, nch=nch):
            if L.vox_probe_handoff_phase(nch, i + 1, wts.data_ptr(), wbytes, work.data_ptr(), cur()):
                raise RuntimeError("handoff phase launch failed")
        us = timed(torch, stream, launch, nphase, nphase)
        print(json.dumps({"leg": "handoff", "mode": "one launch per phase (graph)", "phase_bytes": phase_bytes,
                          "us_per_phase": round(us, 3), **status()}), flush=True)

    # matrix-core rate: four independent bf16 products per round, alone and with 16/32/64
    # independent fp32 multiply-adds per round, at one and two waves per SIMD
    L.vox_probe_mfma_rate_entries.restype = C.c_int
    L.vox_probe_mfma_rate_entries.argtypes = [C.c_int]
    L.vox_probe_mfma_rate.restype = C.c_int
    L.vox_probe_mfma_rate.argtypes = [C.c_int, C.c_int, C.c_int, C.c_int, C.c_void_p, C.c_void_p]
    iters = 2048
    for wps in (1, 2):
        out = torch.empty(L.vox_probe_mfma_rate_entries(wps), dtype=torch.float32, device=dev)
        for kind, name, flop in ((0, "v_mfma_f32_32x32x16_bf16", 32768), (1, "v_mfma_f32_16x16x32_bf16", 16384)):
            for nv in (0, 16, 32, 64):
                per = []
                for rep in range(4):
                    e0 = torch.cuda.Event(enable_timing=True)
                    e1 = torch.cuda.Event(enable_timing=True)
                    e0.record(stream)
                    if L.vox_probe_mfma_rate(kind, nv, wps, iters, out.data_ptr(), cur()):
                        raise RuntimeError("matrix-core rate probe launch failed")
                    e1.record(stream)
                    torch.cuda.synchronize()
                    if rep:   # the first launch warms up
                        per.append(e0.elapsed_time(e1) * 1e3)
                us = float(np.median(per))
                products = cus * 4 * wps * iters * 4   # waves x rounds x 4
                print(json.dumps({"leg": "mfma_rate", "product": name, "waves_per_simd": wps, "fma_per_round": nv,
                                  "us": round(us, 2), "tflops": round(products * flop / us / 1e6, 1),
                                  "frac_bf16_peak": round(products * flop / us / 1e6 / 2500.0, 4),
                                  "cycles_per_round_per_wave_at_2.4GHz": round(us * 2400.0 / (iters * wps), 1)}),
                      flush=True)
        del out


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
    launches rotating over `copies`: the median over `replays` timed graph replays (timed_all)."""
    return float(np.median(timed_all(torch, stream, launch, copies, reps, replays)))


def timed_all(torch, stream, launch, copies, reps, replays=5):
    """Per-launch device times (us) of `launch(i)` (which enqueues on the current stream), one per
    timed replay, each averaged over `reps` launches rotating over `copies`.  The launches are
    captured once in a HIP graph, so host launch cost is not measured; after two warm replays,
    `replays` replays are timed one by one with HIP events on the stream the graph runs on."""
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
    return per


def gemm_set(torch, synth, vox, dev, stream, m: int, fused: bool) -> dict:
    """The encoder-chunk GEMM set at M = m: the six linears of one layer back to back (q, k, v, o,
    ffn_up, ffn_down); fused: q, k and v as one 3840-row product over their concatenated weights
    (the rows of a Q4_0 matrix are independent, so stacking Wq, Wk, Wv gives q, k, v side by side
    in one output).  Rotated weight copies (more than 1 GiB), graph replay, HIP events."""
    GiB = 1 << 30
    sets = []
    for name, n, k in synth.ENCODER_LINEARS:
        w, xb = synth.gemm_inputs(synth.SEED_GEMM, m, n, k)
        sets.append((name, n, k, w, torch.from_numpy(xb.view(np.int16)).to(dev)))
    if fused:
        qkv_w = np.concatenate([sets[0][3], sets[1][3], sets[2][3]], axis=0)
        sets = [("qkv", 3 * sets[0][1], sets[0][2], qkv_w, sets[0][4])] + sets[3:]
    wbytes = sum(s_[3].nbytes for s_ in sets)
    copies = max(2, int(np.ceil(1.1 * GiB / wbytes)))
    wdev = [[torch.from_numpy(s_[3]).to(dev) for s_ in sets] for _ in range(copies)]
    ys = [torch.empty(m, s_[1], dtype=torch.float32, device=dev) for s_ in sets]
    # one workspace serves the set (the launches run one after another on the stream)
    wsb = max(vox.q4_gemm_workspace(m, n_, k_) for _, n_, k_, _, _ in sets)
    gws = torch.empty(max(wsb, 1), dtype=torch.uint8, device=dev)

    def launch(i):
        for j, (name, n, k, _, xd) in enumerate(sets):
            vox._check(vox.lib().vox_q4_gemm(vox._ptr(wdev[i][j]), vox._ptr(xd), vox._ptr(ys[j]), m, n, k,
                                             vox._ptr(gws) if wsb else None, wsb, vox._stream(None)))
    us = timed(torch, stream, launch, copies, 50)
    flops = 2 * m * sum(n * k for _, n, k in synth.ENCODER_LINEARS)
    b = wbytes + sum(m * k_ * 2 + m * n_ * 4 for _, n_, k_, _, _ in sets)
    del wdev
    torch.cuda.empty_cache()
    return {"case": f"encoder linears set, M={m}" + (", q/k/v as one 3840-row call" if fused else ""),
            "us": round(us, 3), "flops": flops, "tflops": round(flops / us / 1e6, 2),
            "frac_mfma_bf16": round(flops / us / 1e6 / 2500.0, 4), "bytes": b, "gbs": round(b / us / 1e3, 1),
            "frac_hbm": round(b / us / 1e3 / HBM_PEAK_GBS, 4)}


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
    for name, n, k in synth.ENCODER_LINEARS[3:]:
        gemv_case(f"encoder width {name}", n, k, 8100 + n + k)
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

    # encoder-chunk GEMM set: the six linears of one layer, each M; then the same set with q, k and v
    # as one 3840-row product over their concatenated weights
    for m, fused in [(m_, f_) for m_ in synth.ENCODER_M for f_ in (False, True)]:
        emit({"kernel": "q4_gemm", **gemm_set(torch, synth, vox, dev, stream, m, fused)})

    # one product per launch at 750 frames (each linear of the set, q/k/v stacked), then the wide
    # product over K at 750 x 5120 (the cost of a stage and of a launch)
    def gemm_case(case, m, n, k):
        w, xb = synth.gemm_inputs(synth.SEED_GEMM, m, n, k)
        copies = max(2, int(np.ceil(1.1 * GiB / w.nbytes)))
        ws_ = [torch.from_numpy(w).to(dev) for _ in range(copies)]
        xd = torch.from_numpy(xb.view(np.int16)).to(dev)
        y = torch.empty(m, n, dtype=torch.float32, device=dev)
        wsb_ = vox.q4_gemm_workspace(m, n, k)
        gws_ = torch.empty(max(wsb_, 1), dtype=torch.uint8, device=dev)

        def launch(i):
            vox._check(vox.lib().vox_q4_gemm(vox._ptr(ws_[i]), vox._ptr(xd), vox._ptr(y), m, n, k,
                                             vox._ptr(gws_) if wsb_ else None, wsb_, vox._stream(None)))
        us = timed(torch, stream, launch, copies, 50)
        fl = 2 * m * n * k
        emit({"kernel": "q4_gemm", "case": case, "m": m, "n": n, "k": k, "us": round(us, 3),
              "tflops": round(fl / us / 1e6, 2), "frac_mfma_bf16": round(fl / us / 1e6 / 2500.0, 4)})
        del ws_
        torch.cuda.empty_cache()

    for name, n, k in synth.ENCODER_LINEARS[3:] + [("q/k/v stacked", 3840, 1280)]:
        gemm_case(f"encoder {name}, M=750", 750, n, k)
    for k in (1280, 3072, 5120):
        gemm_case("wide product over K at 750 x 5120", 750, 5120, k)

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


DECODER_SOURCES = ("decoder.hip", "gemv_core.h", "gqa_attn.h", "vox_common.h")


def source_digest(names) -> str:
    h = hashlib.sha256()
    for name in names:
        with open(os.path.join(ROOT, "streaming_speech_text_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def summarize_trace(path: str):
    """Per-kernel statistics of a rocprofv3 kernel_trace.csv: one JSON line per kernel name, in
    order of total time (calls, mean, p10, p50, p90, min, max; microseconds)."""
    import csv
    durs = {}
    with open(path, newline="") as f:
        for r in csv.DictReader(f):
            name = r.get("Kernel_Name") or r.get("KernelName") or r.get("Name")
            t0 = int(r.get("Start_Timestamp") or r.get("BeginNs") or r["Start"])
            t1 = int(r.get("End_Timestamp") or r.get("EndNs") or r["End"])
            durs.setdefault(name, []).append((t1 - t0) / 1e3)
    rows = []
    for name, d in durs.items():
        a = np.asarray(d)
        rows.append({"kernel": name, "calls": int(a.size), "total_us": round(float(a.sum()), 2),
                     "mean_us": round(float(a.mean()), 3), "p10_us": round(float(np.percentile(a, 10)), 3),
                     "p50_us": round(float(np.percentile(a, 50)), 3), "p90_us": round(float(np.percentile(a, 90)), 3),
                     "min_us": round(float(a.min()), 3), "max_us": round(float(a.max()), 3)})
    rows.sort(key=lambda r: -r["total_us"])
    for r in rows:
        print(json.dumps(r), flush=True)
    return rows


def summarize_counters(path: str):
    """Per-dispatch means of every counter in a rocprofv3 --pmc counter_collection.csv, grouped by
    kernel name and launch shape (grid and workgroup size): one JSON line per group, in order of
    dispatch count.  Where the counters allow: MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (SIMDs x
    GRBM_GUI_ACTIVE / XCDs) with 1024 SIMDs and 8 XCDs, and vector instructions per matrix-core
    instruction."""
    import csv
    per = {}
    with open(path, newline="") as f:
        for r in csv.DictReader(f):
            key = (r["Kernel_Name"], int(r["Grid_Size"]), int(r["Workgroup_Size"]))
            d = per.setdefault(key, {}).setdefault(r.get("Dispatch_Id") or r["Correlation_Id"], {})
            d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    rows = []
    for (name, grid, wg), disp in per.items():
        names = sorted({c for d in disp.values() for c in d})
        mean = {c: float(np.mean([d[c] for d in disp.values() if c in d])) for c in names}
        row = {"kernel": name, "grid_threads": grid, "workgroup": wg, "dispatches": len(disp),
               "mean": {c: round(v, 1) for c, v in mean.items()}}
        if "SQ_VALU_MFMA_BUSY_CYCLES" in mean and mean.get("GRBM_GUI_ACTIVE"):
            row["mfma_busy"] = round(mean["SQ_VALU_MFMA_BUSY_CYCLES"] / (1024 * mean["GRBM_GUI_ACTIVE"] / 8), 4)
        if mean.get("SQ_INSTS_MFMA") and "SQ_INSTS_VALU" in mean:
            row["valu_per_mfma"] = round(mean["SQ_INSTS_VALU"] / mean["SQ_INSTS_MFMA"], 2)
        rows.append(row)
    rows.sort(key=lambda r: -r["dispatches"])
    for r in rows:
        print(json.dumps(r), flush=True)
    return rows


def counter_summary(fetch_csv: str, write_csv: str):
    """FETCH_SIZE / WRITE_SIZE (KiB per dispatch) of the GEMV of --leg gemv, scaled by the values the
    same counters read for the leg's calibration copies (256 MiB read and written each)."""
    import csv

    def per_kernel(path, counter):
        vals = {}
        with open(path, newline="") as f:
            for r in csv.DictReader(f):
                if r.get("Counter_Name") != counter:
                    continue
                key = r.get("Dispatch_Id") or r.get("Correlation_Id")
                vals.setdefault(r["Kernel_Name"], {})
                vals[r["Kernel_Name"]][key] = vals[r["Kernel_Name"]].get(key, 0.0) + float(r["Counter_Value"])
        return {k: list(v.values()) for k, v in vals.items()}

    fetch = per_kernel(fetch_csv, "FETCH_SIZE")
    write = per_kernel(write_csv, "WRITE_SIZE")

    def pick(d, needle, big_only=False):
        for k, v in d.items():
            if needle in k:
                if big_only:
                    v = [x for x in v if x > 0.5 * max(v)]
                return float(np.mean(v)), len(v)
        raise KeyError(needle)

    cf, _ = pick(fetch, "copyBuffer", big_only=True)
    cw, _ = pick(write, "copyBuffer", big_only=True)
    gf, nd = pick(fetch, "q4_gemv_tiled_kernel")
    gw, _ = pick(write, "q4_gemv_tiled_kernel")
    copy_kib = 256 * 1024
    ffac, wfac = copy_kib / cf, copy_kib / cw
    n, k = 131072, 3072
    alg = n * (k // 32) * 18 + 4 * (n + k)
    hbm = int(round((gf * ffac + gw * wfac) * 1024))
    return {"kernel": "q4_gemv_tiled_kernel (vox_q4_gemv, 131072 x 3072, LM-head shape)",
            "kernel_source_digest": kernel_source_digest(),
            "digest_of": "sha256 of csrc/gemv_core.h + csrc/q4_gemv.hip + csrc/vox_common.h, first 16 hex digits",
            "calibration": {"reference": "torch copy of 256 MiB (__amd_rocclr_copyBuffer) in --leg gemv",
                            "fetch_size_kib_read_by_copy": round(cf, 2), "write_size_kib_written_by_copy": round(cw, 2),
                            "fetch_factor": round(ffac, 5), "write_factor": round(wfac, 5)},
            "per_dispatch_kib": {"FETCH_SIZE": round(gf, 2), "WRITE_SIZE": round(gw, 2), "dispatches": nd},
            "hbm_bytes_per_launch": hbm, "algorithmic_bytes_per_launch": alg,
            "traffic_over_algorithmic": round(hbm / alg, 4)}


def decoder_kernel_bytes(name: str, s, q4_row_bytes):
    """Algorithmic bytes of one launch of a decoder kernel at shape s, from the kernel's policy name:
    its Q4_0 weights once plus the fp32 vectors it must read and write."""
    qd, kvd = s.n_heads * s.head_dim, s.n_kv_heads * s.head_dim
    name = name.replace("vox::", "")
    if "GateUpPolicy" in name:
        return 2 * s.hidden * q4_row_bytes(s.dim) + 4 * (2 * s.dim + s.hidden)
    if "QkvPolicy" in name:
        return (qd + 2 * kvd) * q4_row_bytes(s.dim) + 4 * (2 * s.dim + qd + 2 * kvd)
    if "ResidualPolicy<GemvGeom<9216" in name:
        return s.dim * q4_row_bytes(s.hidden) + 4 * (s.hidden + 2 * s.dim)
    if "ResidualPolicy<GemvGeom<4096" in name:
        return s.dim * q4_row_bytes(qd) + 4 * (qd + 2 * s.dim)
    if "LmHeadPolicy" in name:
        return s.vocab * q4_row_bytes(s.dim) + 4 * 2 * s.dim
    return None


def decoder_trace_roofline(synth):
    """The decoder's dominant kernel (largest share of a token's time) from the committed kernel
    trace of the default bench workload, if that trace was taken on the current decoder sources:
    its algorithmic bytes per launch, mean duration in the trace and fraction of HBM peak."""
    p = os.path.join(ROOT, "profiles", "decoder_step_kernels.json")
    try:
        with open(p) as f:
            d = json.load(f)
    except (OSError, ValueError):
        return None
    if d.get("source_digest") != source_digest(DECODER_SOURCES):
        return {"stale": True, "note": "kernel trace taken on other decoder sources"}
    s = synth.VOXTRAL_DECODER
    steps = d["decoder_steps"]
    cands = [k for k in d["kernels"] if k["kernel"].replace("vox::", "").startswith(("void dec_", "dec_"))]
    top = max(cands, key=lambda k: k["total_us"])
    b = decoder_kernel_bytes(top["kernel"], s, synth.q4_row_bytes)
    out = {"kernel": top["kernel"], "us_per_launch": top["mean_us"], "p10_us": top["p10_us"], "p90_us": top["p90_us"],
           "launches_per_token": round(top["calls"] / steps, 2),
           "share_of_token": round(top["total_us"] / sum(k["total_us"] for k in cands), 4),
           "source": "profiles/decoder_step_kernels.json (rocprofv3 kernel trace)"}
    if b:
        gbs = b / top["mean_us"] / 1e3
        out.update({"bound": "hbm", "bytes_per_launch": b, "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                    "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4)})
    return out


def decoder_device_weights(torch, synth, w, dev):
    return {"tok_embd": torch.from_numpy(w["tok_embd"]).to(dev), "out_norm": torch.from_numpy(w["out_norm"]).to(dev),
            "layers": [{k: torch.from_numpy(v).to(dev) for k, v in L.items()} for L in w["layers"]]}


def time_sequences(torch, stream, dec, tok, n_seq, steps, before):
    """n_seq sequences of `steps` greedy steps (token fed back on the device); before(q) prepares
    sequence q untimed.  Each sequence is bracketed by synchronisations and timed with HIP events
    on the stream the steps run on (and by the host clock).  Returns (device ms/token, wall
    ms/token) lists."""
    dev_ms, wall_ms = [], []
    for q in range(n_seq):
        before(q)
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        e0.record(stream)
        for _ in range(steps):
            dec.step(tok, tok)
        e1.record(stream)
        torch.cuda.synchronize()
        wall_ms.append((time.perf_counter() - t0) * 1e3 / steps)
        dev_ms.append(e0.elapsed_time(e1) / steps)
    return dev_ms, wall_ms


def spread(v):
    a = np.asarray(v, dtype=np.float64)
    return {"median": round(float(np.median(a)), 4), "p10": round(float(np.percentile(a, 10)), 4),
            "p90": round(float(np.percentile(a, 90)), 4), "min": round(float(a.min()), 4),
            "max": round(float(a.max()), 4), "n": int(a.size)}


def decoder_legs(args, torch, synth, vox, dev, stream, w, full_window=True):
    """The decoder at the bench configuration (38-position prefix, then K greedy steps) and at a
    full, wrapped 8192-position window (ring filled with N(0, 1) keys and values, stream resumed
    at position 8192 + 3000)."""
    s = synth.VOXTRAL_DECODER
    wd = decoder_device_weights(torch, synth, w, dev)
    cfg = vox.DecoderConfig(s.n_layers, s.dim, s.n_heads, s.n_kv_heads, s.head_dim, s.hidden, s.vocab, s.n_slots,
                            s.norm_eps, s.rope_theta)
    dec = vox.Decoder(cfg, wd)
    prefix, start = synth.decoder_tokens(synth.SEED_DECODER, s.vocab)
    tok = torch.zeros(1, dtype=torch.int32, device=dev)

    def run_prefix(_q=0):
        dec.reset()
        for t in prefix:
            tok.fill_(int(t))
            dec.step(tok, tok)
        tok.fill_(start)

    # warmup: captures the graph of every attention bucket the timed positions use
    print("[bench] warmup", file=sys.stderr, flush=True)
    run_prefix()
    for _ in range(max(args.warmup, args.steps)):
        dec.step(tok, tok)
    torch.cuda.synchronize()
    dev_ms, wall_ms = time_sequences(torch, stream, dec, tok, args.sequences, args.steps, run_prefix)
    last_token = int(tok.item())
    weight_bytes = (s.n_layers * sum(o * synth.q4_row_bytes(i) for o, i in synth.LAYER_LINEARS.values())
                    + s.vocab * synth.q4_row_bytes(s.dim) + synth.q4_row_bytes(s.dim))
    kv_row = s.n_layers * 2 * s.n_kv_heads * s.head_dim * 4
    kv_bytes = sum(kv_row * min(p + 1, s.n_slots) for p in range(len(prefix), len(prefix) + args.steps)) / args.steps
    main = {"dev_ms": dev_ms, "wall_ms": wall_ms, "bytes": weight_bytes + kv_bytes, "last_token": last_token,
            "positions": [len(prefix), len(prefix) + args.steps], "prefix": prefix}
    print(f"[bench] decoder {np.median(dev_ms):.4f} ms/token (median of {len(dev_ms)} sequences; host clock "
          f"{np.median(wall_ms):.4f})", file=sys.stderr, flush=True)
    if not full_window:
        dec.close()
        return main, None

    # full window: every step reads all 8192 positions of every layer's K and V
    dec.kv.view(torch.float32).normal_()
    pos0 = s.n_slots + 3000
    dec.seek(pos0)
    tok.fill_(start)
    for _ in range(max(args.warmup, 2)):
        dec.step(tok, tok)
    torch.cuda.synchronize()
    f_dev, f_wall = time_sequences(torch, stream, dec, tok, args.sequences, args.steps, lambda q: None)
    full_bytes = weight_bytes + kv_row * s.n_slots
    fm = float(np.median(f_dev))
    full = {"ms_per_token": spread(f_dev), "host_clock_ms_per_token": round(float(np.median(f_wall)), 4),
            "positions": [pos0, pos0 + (max(args.warmup, 2) + args.sequences * args.steps)],
            "live_positions": s.n_slots, "bytes_per_token": int(full_bytes),
            "kv_bytes_per_token": int(kv_row * s.n_slots), "achieved_gbs": round(full_bytes / fm / 1e6, 1),
            "frac_hbm": round(full_bytes / fm / 1e6 / HBM_PEAK_GBS, 4),
            "note": "ring filled with N(0,1) keys and values, stream resumed past a wrapped window"}
    print(f"[bench] decoder full window {fm:.4f} ms/token, {full['achieved_gbs']:.0f} GB/s", file=sys.stderr,
          flush=True)
    dec.close()
    del wd
    torch.cuda.empty_cache()
    return main, full


def decoder_w16_leg(args, torch, synth, vox, dev, stream, fmt="f16", n_seq=3):
    """The decoder over 16-bit weights (the format voxtral.c's GPU path runs, F16) at the bench
    configuration: 38-token prefix untimed, then args.steps greedy steps per sequence, median of
    n_seq sequences."""
    s = synth.VOXTRAL_DECODER
    print(f"[bench] generating {fmt} weights", file=sys.stderr, flush=True)
    w = synth.decoder_weights_w16(synth.SEED_DECODER, s, fmt)

    def d(a):
        a = np.ascontiguousarray(a)
        return torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a).to(dev)
    wd = {"tok_embd": d(w["tok_embd"]), "out_norm": d(w["out_norm"]),
          "layers": [{k: d(v) for k, v in L.items()} for L in w["layers"]]}
    wbytes = sum(int(v.nbytes) for L in w["layers"] for k, v in L.items() if k.startswith("w")) + w["tok_embd"].nbytes
    del w
    cfg = vox.DecoderConfig(s.n_layers, s.dim, s.n_heads, s.n_kv_heads, s.head_dim, s.hidden, s.vocab, s.n_slots,
                            s.norm_eps, s.rope_theta)
    dec = vox.Decoder(cfg, wd, fmt=fmt)
    prefix, start = synth.decoder_tokens(synth.SEED_DECODER, s.vocab)
    tok = torch.zeros(1, dtype=torch.int32, device=dev)

    def run_prefix(_q=0):
        dec.reset()
        for t in prefix:
            tok.fill_(int(t))
            dec.step(tok, tok)
        tok.fill_(start)

    run_prefix()
    for _ in range(max(args.warmup, args.steps)):
        dec.step(tok, tok)
    torch.cuda.synchronize()
    dev_ms, wall_ms = time_sequences(torch, stream, dec, tok, n_seq, args.steps, run_prefix)
    kv_row = s.n_layers * 2 * s.n_kv_heads * s.head_dim * 4
    kv_bytes = sum(kv_row * min(p + 1, s.n_slots) for p in range(len(prefix), len(prefix) + args.steps)) / args.steps
    m = float(np.median(dev_ms))
    out = {"format": fmt, "ms_per_token": spread(dev_ms), "host_clock_ms_per_token": round(float(np.median(wall_ms)), 4),
           "bytes_per_token": int(wbytes + kv_bytes), "achieved_gbs": round((wbytes + kv_bytes) / m / 1e6, 1),
           "frac_hbm": round((wbytes + kv_bytes) / m / 1e6 / HBM_PEAK_GBS, 4),
           "note": "16-bit weights ~ N(0, 0.02^2); the pages' F16 step on Metal (M3 Max) is 23.5 ms"}
    print(f"[bench] decoder over {fmt} weights {m:.4f} ms/token, {out['achieved_gbs']:.0f} GB/s", file=sys.stderr,
          flush=True)
    dec.close()
    del wd
    torch.cuda.empty_cache()
    return out


def gemv_sweep(torch, synth, vox, dev, stream, k=3072, rows=(1024, 2048, 4096, 8192, 16384, 32768, 65536, 131072)):
    """The Q4_0 GEMV over row counts at K = 3072 (the decoder width), rotating over more than
    1 GiB of weight copies per point."""
    out = []
    w_all, x = synth.gemv_inputs(synth.SEED_GEMV, max(rows), k)
    xd = torch.from_numpy(x).to(dev)
    for n in rows:
        w = w_all[:n]
        copies = max(2, int(np.ceil(1.1 * 2 ** 30 / w.nbytes)))
        base = torch.from_numpy(np.ascontiguousarray(w)).to(dev)
        ws = [base] + [base.clone() for _ in range(copies - 1)]
        y = torch.empty(n, dtype=torch.float32, device=dev)
        us = timed(torch, stream, lambda i: vox.q4_gemv(ws[i], xd, y), copies, 200 if n <= 16384 else 100)
        b = n * synth.q4_row_bytes(k) + 4 * (n + k)
        out.append({"n": n, "k": k, "us": round(us, 3), "gbs": round(b / us / 1e3, 1),
                    "frac_hbm": round(b / us / 1e3 / HBM_PEAK_GBS, 4)})
        del ws, base
        torch.cuda.empty_cache()
    return out


def lscpu_model() -> str:
    try:
        import subprocess
        r = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10)
        for line in r.stdout.splitlines():
            if line.startswith("Model name:"):
                return line.split(":", 1)[1].strip()
    except (OSError, ValueError):
        pass
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_leg(args, synth, w):
    """The oracle (fp64 C, OpenMP over output rows or heads) on the host: the decoder step at the
    full shape (first teacher-forced steps of the prefix) and the single workloads, at the
    oracle's default thread count and at one thread.  Bounded samples: a few seconds each."""
    import oracle
    s = synth.VOXTRAL_DECODER
    prefix, _ = synth.decoder_tokens(synth.SEED_DECODER, s.vocab)
    n_threads = oracle.max_threads()

    def clock(fn, reps):
        t = []
        for _ in range(reps):
            a = time.perf_counter()
            fn()
            t.append(time.perf_counter() - a)
        return 1e3 * float(np.median(t))

    gw, gx = synth.gemv_inputs(synth.SEED_GEMV, 3072, 3072)
    hw = w["tok_embd"]
    hx = synth.normal_f32(synth.generator(synth.SEED_GEMV, 2), (s.dim,))
    q, kc, vc = synth.attention_inputs(synth.SEED_ATTN, 32, 8, 128, 8192)
    qd, kd, vd = q.astype(np.float64), kc.astype(np.float64), vc.astype(np.float64)
    gemm = [synth.gemm_inputs(synth.SEED_GEMM, 16, n, k) for _, n, k in synth.ENCODER_LINEARS]
    work = {}
    dec = {}
    for threads, budget in ((n_threads, args.cpu_seconds), (1, args.cpu_seconds / 2)):
        oracle.set_num_threads(threads)
        od = oracle.Decoder(s, w)
        times = []
        t_start = time.perf_counter()
        for t in prefix:
            a = time.perf_counter()
            od.step(int(t), want_logits=False)
            times.append(time.perf_counter() - a)
            if time.perf_counter() - t_start > budget and len(times) >= (3 if threads > 1 else 1):
                break
        od.close()
        dec[threads] = (1e3 * float(np.mean(times)), len(times))
        reps = 3 if threads > 1 else 1
        work.setdefault("gemv 3072x3072", {})[threads] = clock(lambda: oracle.q4_gemv(gw, gx), reps)
        work.setdefault("gemv 131072x3072 (LM-head shape)", {})[threads] = clock(lambda: oracle.q4_gemv(hw, hx), 1)
        work.setdefault("gqa attention, 8192 positions", {})[threads] = clock(
            lambda: oracle.gqa_attn(qd, kd, vd, 1 / np.sqrt(128)), reps)
        work.setdefault("encoder linears set, M=16", {})[threads] = clock(
            lambda: [oracle.q4_gemm(gw_, xb_) for gw_, xb_ in gemm], 1)
    oracle.set_num_threads(n_threads)
    nbytes = {"gemv 3072x3072": 3072 * synth.q4_row_bytes(3072) + 8 * 3072,
              "gemv 131072x3072 (LM-head shape)": s.vocab * synth.q4_row_bytes(s.dim) + 4 * (s.vocab + s.dim),
              "gqa attention, 8192 positions": 8192 * 8192 + 2 * 32 * 128 * 4,
              "encoder linears set, M=16": sum(n * synth.q4_row_bytes(k) + 16 * (2 * k + 4 * n)
                                               for _, n, k in synth.ENCODER_LINEARS)}
    per = {name: {"ms": {str(t): round(v, 3) for t, v in d.items()},
                  "gbs": {str(t): round(nbytes[name] / (v * 1e-3) / 1e9, 2) for t, v in d.items()}}
           for name, d in work.items()}
    return {"value": round(dec[n_threads][0], 3), "unit": "ms/token", "cores": n_threads, "kind": "oracle",
            "sample": f"first {dec[n_threads][1]} teacher-forced steps of the 38-token prefix at the full decoder "
                      f"shape (fp64 oracle, OpenMP over output rows); at 1 thread the first {dec[1][1]}",
            "threads": n_threads, "cpu_model": lscpu_model(), "host_cpus": os.cpu_count(),
            "value_1_thread": round(dec[1][0], 3), "workloads": per}


def main():
    args = parse()
    if args.counter_summary:
        print(json.dumps(counter_summary(*args.counter_summary), indent=1), flush=True)
        return
    if args.summarize_counters:
        summarize_counters(args.summarize_counters)
        return
    if args.summarize_trace:
        rows = summarize_trace(args.summarize_trace)
        if args.trace_json:
            with open(args.trace_json, "w") as f:
                json.dump({"source_digest": source_digest(DECODER_SOURCES), "decoder_steps": args.decoder_steps,
                           "trace": os.path.basename(args.summarize_trace), "kernels": rows}, f, indent=1)
        return
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
        for r in gemv_sweep(torch, synth, vox, dev, stream):
            print(json.dumps({"kernel": "q4_gemv", "case": "row sweep at K=3072", **r}), flush=True)
        return
    if args.leg == "probe":
        probe_leg(torch, dev, stream)
        return
    if args.leg == "decoder_w16":
        print(json.dumps({"leg": "decoder_w16", **decoder_w16_leg(args, torch, synth, vox, dev, stream)}), flush=True)
        return
    s = synth.VOXTRAL_DECODER
    print(f"[bench] generating weights ({s.n_layers} layers, vocab {s.vocab})", file=sys.stderr, flush=True)
    w = synth.decoder_weights(synth.SEED_DECODER, s)
    dm, full = decoder_legs(args, torch, synth, vox, dev, stream, w, full_window=args.leg in ("all", "decoder_full"))
    if args.leg == "decoder_full":
        print(json.dumps({"leg": "decoder_full", "ms_per_token": spread(dm["dev_ms"]), "full_window": full}),
              flush=True)
        return
    if args.leg == "decoder":
        n_steps = (args.sequences + 1) * len(dm["prefix"]) + max(args.warmup, args.steps) + args.sequences * args.steps
        print(json.dumps({"leg": "decoder", "ms_per_token": spread(dm["dev_ms"]), "decoder_steps": n_steps}),
              flush=True)
        return
    ms_per_token = float(np.median(dm["dev_ms"]))
    w16 = decoder_w16_leg(args, torch, synth, vox, dev, stream)

    gemv = gemv_leg(args, torch, synth, vox, dev, stream)
    traffic = measured_traffic(kernel_source_digest(), gemv["bytes"])
    ceil = probe_ceiling(torch, dev, stream, [gemv["bytes"] // 256 * 256], reps=50)
    c_us, c_gbs, c_wg, c_loads = next(iter(ceil.values()))
    sweep = gemv_sweep(torch, synth, vox, dev, stream)
    print(f"[bench] gemv sweep: " + ", ".join(f"{r['n']}:{r['gbs']:.0f}" for r in sweep), file=sys.stderr, flush=True)

    # the encoder-chunk GEMM set (q, k, v stacked) at the shortest and the longest chunk
    egemm = {}
    for m in (synth.ENCODER_M[0], synth.ENCODER_M[-1]):
        r = gemm_set(torch, synth, vox, dev, stream, m, True)
        egemm[f"M={m}"] = {k_: r[k_] for k_ in ("us", "tflops", "frac_mfma_bf16", "gbs", "frac_hbm")}
    print(f"[bench] encoder GEMM sets: " + ", ".join(f"{k_} {v_['us']:.1f} us" for k_, v_ in egemm.items()),
          file=sys.stderr, flush=True)

    cpu = None if args.no_cpu else cpu_leg(args, synth, w)

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
                   "tokens_timed": args.steps, "sequences": args.sequences, "kv_positions": dm["positions"]},
        "roofline": {"bound": "hbm", "achieved": round(gemv["gbs"], 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gemv["gbs"] / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "kernel": f"q4_gemv {gemv['n']}x{gemv['k']} (LM-head shape)", "bytes_per_launch": gemv["bytes"],
                     "us_per_launch": round(gemv["us"], 3), "us_per_launch_spread": gemv["spread"],
                     "ceiling": {"gbs": round(c_gbs, 1), "frac_hbm": round(c_gbs / HBM_PEAK_GBS, 4),
                                 "us": round(c_us, 3), "probe": "streaming read of the same byte count "
                                 "(libvox_probe.so)", "workgroups_per_cu": c_wg, "loads": c_loads},
                     "frac_of_ceiling": round(gemv["gbs"] / c_gbs, 4)},
        "decoder_ms_per_token": spread(dm["dev_ms"]),
        "decoder_host_clock_ms_per_token": spread(dm["wall_ms"]),
        "decoder_hbm_gbs": round(dm["bytes"] / (ms_per_token * 1e-3) / 1e9, 1),
        "decoder_bytes_per_token": int(dm["bytes"]),
        "decoder_full_window": full,
        "decoder_w16": w16,
        "decoder_roofline": decoder_trace_roofline(synth),
        "gemv_sweep_k3072": sweep,
        "encoder_gemm_set_qkv_stacked": egemm,
        "last_token": dm["last_token"],
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
