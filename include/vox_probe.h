/* vox_probe.h - measurement aid beside libvox (built as libvox_probe.so).
 *
 * Not an operation of the decoder step: the streaming-read probe gives the HBM read rate a
 * plain kernel reaches on this GPU for a given number of bytes, the practical ceiling next to
 * the 8 TB/s nominal peak for kernels that stream their data once (the Q4_0 GEMVs of vox.h,
 * whose fused dequantisation follows the Rust port page, GeekNews 26595, section 아키텍처).
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

#ifdef __cplusplus
}
#endif
#endif /* VOX_PROBE_H */
