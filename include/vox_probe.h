/* vox_probe.h - measurement aids beside libvox (built as libvox_probe.so).
 *
 * Not operations of the decoder step: the streaming-read probe gives the HBM read rate a plain
 * kernel reaches on this GPU for a given number of bytes, the practical ceiling next to the
 * 8 TB/s nominal peak for kernels that stream their data once (the Q4_0 GEMVs of vox.h, whose
 * fused dequantisation follows the Rust port page, GeekNews 26595, section 아키텍처); the
 * matrix-core rate probe gives the same for the bf16 products of the Q4_0 GEMMs.
 */
#ifndef VOX_PROBE_H
#define VOX_PROBE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Number of sink entries (workgroups) of a launch with wg_per_cu workgroups per compute unit
 * (1..8) on the current device; -1 on a bad argument or a HIP failure. */
int vox_probe_sink_entries(int wg_per_cu);

/* Reads `bytes` bytes (a positive multiple of 16) at device address buf (16-byte aligned) once,
 * with 16-byte loads from vox_probe_sink_entries(wg_per_cu) workgroups of 256 threads, and
 * writes one checksum per workgroup to the device array sink.  Enqueued on `stream` (a
 * hipStream_t; NULL = the null stream).  Returns 0, -1 on a bad argument, -4 if the launch failed. */
int vox_probe_stream_read(const void *buf, size_t bytes, uint32_t *sink, int wg_per_cu, void *stream);
/* The same read with non-temporal loads (the form the GEMVs' weight streams use). */
int vox_probe_stream_read_nt(const void *buf, size_t bytes, uint32_t *sink, int wg_per_cu, void *stream);
/* The same read with direct-to-LDS 16-byte loads (the data lands in LDS without passing through
 * registers; 32 KB of LDS per workgroup), plain or non-temporal. */
int vox_probe_stream_read_lds(const void *buf, size_t bytes, uint32_t *sink, int wg_per_cu, void *stream);
int vox_probe_stream_read_lds_nt(const void *buf, size_t bytes, uint32_t *sink, int wg_per_cu, void *stream);

/* Grid-wide handoff probe: the cost of passing a 3072-float vector between phases inside one
 * persistent kernel (one 512-thread workgroup per compute unit, a grid barrier per phase, each
 * workgroup's next weight share of 8192 * nch bytes prefetched before the barrier) against one
 * launch per phase.  nch: 0, 4, 8 or 16 (0: the handoff alone).  Work buffer: device memory of
 * vox_probe_handoff_work_bytes() bytes, 256-byte aligned; its first 16 bytes are four uint32
 * (abort flag, expired waits, vector values read wrong, unused), cleared by vox_probe_handoff_reset.
 * weights: at least 8192 * nch * (number of compute units) bytes, 16-byte aligned (phases read
 * consecutive windows of it).  Every wait inside the persistent kernel is bounded (2^20 polls);
 * one expired wait ends all others.  Returns 0, -1 on a bad argument, -2 if a workgroup per
 * compute unit cannot be resident, -4 if the launch failed. */
size_t vox_probe_handoff_work_bytes(void);
int vox_probe_handoff_reset(void *work, void *stream);
/* mode 0: every workgroup stores a flag, one workgroup gathers them and releases the grid;
 * mode 1: eight counters, every workgroup polls their sum; mode 2: eight counters polled by a
 * ninth wave per workgroup that holds no weight loads, while the eight working waves keep the
 * next phase's loads in flight across the barrier.  Runs nphase phases (1..100000). */
int vox_probe_handoff_persistent(int mode, int nch, int nphase, const void *weights, size_t weight_bytes, void *work,
                                 void *stream);
/* Phase `phase` (1..100000) of the same work as its own launch, no prefetch, no barrier. */
int vox_probe_handoff_phase(int nch, int phase, const void *weights, size_t weight_bytes, void *work, void *stream);

/* Matrix-core rate probe.  Output entries (floats) of a launch with waves_per_simd (1..4) waves
 * per SIMD on the current device (workgroups of four waves, one per compute unit and wave per
 * SIMD); -1 on a bad argument or a HIP failure. */
int vox_probe_mfma_rate_entries(int waves_per_simd);
/* Every wave runs `iters` (1..2^24) rounds of four independent bf16 matrix-core products (kind 0:
 * v_mfma_f32_32x32x16_bf16, 32768 flop each; kind 1: v_mfma_f32_16x16x32_bf16, 16384 flop each)
 * plus nv (0, 16, 32 or 64) independent fp32 multiply-adds, then writes one value per lane to the
 * device array out (vox_probe_mfma_rate_entries(waves_per_simd) floats).  Enqueued on `stream`.
 * Returns 0, -1 on a bad argument, -4 if the launch failed. */
int vox_probe_mfma_rate(int kind, int nv, int waves_per_simd, int iters, float *out, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* VOX_PROBE_H */
