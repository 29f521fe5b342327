// stream_read.hip - streaming-read probe: the HBM read rate a plain kernel reaches on this GPU.
//
// Not an operation of the decoder.  It reads a buffer once with 16-byte loads (plain or
// non-temporal) and keeps a checksum per workgroup, so the loads cannot be dropped.  The best rate
// it reaches at a given size is the practical ceiling for a kernel that must stream that many
// bytes once (the decoder's GEMVs stream their Q4_0 weights exactly once per token).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/vox_probe.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int PROBE_THREADS = 256;
constexpr int PROBE_UNROLL = 8;   // 16-byte loads in flight per thread per round

template <bool NT>
__device__ __forceinline__ u32x4 ld16(const u32x4 *p)
{
    if constexpr (NT)
        return __builtin_nontemporal_load(p);
    else
        return *p;
}

// Workgroup i reads 16-byte chunks i*T + t, then every gridDim*T further, PROBE_UNROLL rounds
// at a time (all loads of a round issued before their first use).  NT: non-temporal loads.
template <bool NT>
__global__ __launch_bounds__(PROBE_THREADS) void stream_read_kernel(const u32x4 *__restrict__ src, int64_t n16,
                                                                    uint32_t *__restrict__ sink)
{
    const int64_t stride = (int64_t)gridDim.x * PROBE_THREADS;
    int64_t i = (int64_t)blockIdx.x * PROBE_THREADS + threadIdx.x;
    u32x4 acc = {0u, 0u, 0u, 0u};
    for (; i + (PROBE_UNROLL - 1) * stride < n16; i += PROBE_UNROLL * stride) {
        u32x4 v[PROBE_UNROLL];
#pragma unroll
        for (int u = 0; u < PROBE_UNROLL; ++u)
            v[u] = ld16<NT>(src + i + u * stride);
#pragma unroll
        for (int u = 0; u < PROBE_UNROLL; ++u)
            acc ^= v[u];
    }
    for (; i < n16; i += stride)
        acc ^= ld16<NT>(src + i);
    __shared__ uint32_t red[PROBE_THREADS];
    red[threadIdx.x] = acc.x ^ acc.y ^ acc.z ^ acc.w;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t r = 0;
        for (int t = 0; t < PROBE_THREADS; ++t)
            r ^= red[t];
        sink[blockIdx.x] = r;
    }
}

// The same read with direct-to-LDS loads (global_load_lds_dwordx4): the 16 bytes of lane L land
// in LDS at the wave's slot base + 16 L without passing through registers.  Each round issues
// PROBE_UNROLL loads per thread into slots of their own, waits for all of them, then reads back the
// thread's first dword of each slot into the checksum.  NT: non-temporal loads.
template <bool NT>
__global__ __launch_bounds__(PROBE_THREADS) void stream_read_lds_kernel(const u32x4 *__restrict__ src, int64_t n16,
                                                                        uint32_t *__restrict__ sink)
{
    __shared__ uint32_t ring[PROBE_UNROLL][PROBE_THREADS * 4];   // slot u: 16 bytes per thread
    const int wave = threadIdx.x >> 6;
    const int64_t stride = (int64_t)gridDim.x * PROBE_THREADS;
    int64_t i = (int64_t)blockIdx.x * PROBE_THREADS + threadIdx.x;
    uint32_t acc = 0u;
    for (; i + (PROBE_UNROLL - 1) * stride < n16; i += PROBE_UNROLL * stride) {
#pragma unroll
        for (int u = 0; u < PROBE_UNROLL; ++u)
            __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void *)(src + i + u * stride),
                                             (__attribute__((address_space(3))) void *)&ring[u][wave * 256], 16, 0,
                                             NT ? 2 : 0);
        __builtin_amdgcn_s_waitcnt(0);   // every counter at zero: the round's data is in LDS
#pragma unroll
        for (int u = 0; u < PROBE_UNROLL; ++u)
            acc ^= ring[u][threadIdx.x * 4];
    }
    for (; i < n16; i += stride) {
        const u32x4 v = ld16<NT>(src + i);
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    __shared__ uint32_t red[PROBE_THREADS];
    red[threadIdx.x] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t r = 0;
        for (int t = 0; t < PROBE_THREADS; ++t)
            r ^= red[t];
        sink[blockIdx.x] = r;
    }
}

}  // namespace

extern "C" int vox_probe_sink_entries(int wg_per_cu)
{
    int dev = 0, cus = 0;
    if (wg_per_cu < 1 || wg_per_cu > 8 || hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
        return -1;
    return wg_per_cu * cus;
}

namespace {
template <bool NT, bool LDS = false>
int stream_read(const void *buf, size_t bytes, uint32_t *sink, int wg_per_cu, void *stream)
{
    if (!buf || !sink || bytes == 0 || bytes % 16 || ((uintptr_t)buf % 16))
        return -1;
    const int grid = vox_probe_sink_entries(wg_per_cu);
    if (grid < 1)
        return -1;
    if constexpr (LDS)
        hipLaunchKernelGGL(stream_read_lds_kernel<NT>, dim3(grid), dim3(PROBE_THREADS), 0, (hipStream_t)stream,
                           (const u32x4 *)buf, (int64_t)(bytes / 16), sink);
    else
        hipLaunchKernelGGL(stream_read_kernel<NT>, dim3(grid), dim3(PROBE_THREADS), 0, (hipStream_t)stream,
                           (const u32x4 *)buf, (int64_t)(bytes / 16), sink);
    return hipGetLastError() == hipSuccess ? 0 : -4;
}
}  // namespace

extern "C" int vox_probe_stream_read(const void *buf, size_t bytes, uint32_t *sink, int wg_per_cu, void *stream)
{
    return stream_read<false>(buf, bytes, sink, wg_per_cu, stream);
}

extern "C" int vox_probe_stream_read_nt(const void *buf, size_t bytes, uint32_t *sink, int wg_per_cu, void *stream)
{
    return stream_read<true>(buf, bytes, sink, wg_per_cu, stream);
}

extern "C" int vox_probe_stream_read_lds(const void *buf, size_t bytes, uint32_t *sink, int wg_per_cu, void *stream)
{
    return stream_read<false, true>(buf, bytes, sink, wg_per_cu, stream);
}

extern "C" int vox_probe_stream_read_lds_nt(const void *buf, size_t bytes, uint32_t *sink, int wg_per_cu,
                                            void *stream)
{
    return stream_read<true, true>(buf, bytes, sink, wg_per_cu, stream);
}
