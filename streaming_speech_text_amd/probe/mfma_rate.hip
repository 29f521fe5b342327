// mfma_rate.hip - matrix-core rate probe: what a loop of bf16 matrix-core products reaches on this
// GPU, alone and with independent vector work between the products.
//
// Not an operation of the encoder or the decoder.  The encoder-chunk Q4_0 products (fused
// dequantisation per the Rust port page, GeekNews 26595, section 아키텍처) run on
// v_mfma_f32_16x16x32_bf16 and v_mfma_f32_32x32x16_bf16 with vector unpacking and scaling beside
// them; this loop gives the rate those instructions reach on their own (the practical ceiling next
// to the nominal bf16 peak) and how much vector work hides under them.
//
// Each wave keeps four independent accumulators and runs `iters` rounds of four products plus
// NV independent fp32 multiply-adds (eight chains); every lane stores one folded value at the end.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "../../include/vox_probe.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int MR_THREADS = 256;

template <int KIND, int NV>
__global__ __launch_bounds__(MR_THREADS) void mfma_rate_kernel(float *__restrict__ out, int iters, float seed)
{
    bf16x8 a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        a[i] = (__bf16)(seed + 0.001f * (float)threadIdx.x + (float)i);
        b[i] = (__bf16)(seed - (float)i);
    }
    typedef typename std::conditional<KIND == 0, f32x16, f32x4>::type acc_t;
    acc_t acc[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
        acc[j] = 0.0f;
    float v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
        v[j] = seed * (float)(j + 1) + (float)threadIdx.x;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if constexpr (KIND == 0)
                acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[j], 0, 0, 0);
            else
                acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[j], 0, 0, 0);
        }
#pragma unroll
        for (int r = 0; r < NV / 8; ++r)
#pragma unroll
            for (int j = 0; j < 8; ++j)
                v[j] = fmaf(v[j], 1.0000001f, 1e-7f);
    }
    float s = 0.0f;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < (KIND == 0 ? 16 : 4); ++r)
            s += acc[j][r];
#pragma unroll
    for (int j = 0; j < 8; ++j)
        s += v[j];
    out[(size_t)blockIdx.x * MR_THREADS + threadIdx.x] = s;
}

template <int KIND>
int launch_kind(int nv, int grid, float *out, int iters, hipStream_t s)
{
    switch (nv) {
    case 0: hipLaunchKernelGGL((mfma_rate_kernel<KIND, 0>), dim3(grid), dim3(MR_THREADS), 0, s, out, iters, 1.0f); break;
    case 16: hipLaunchKernelGGL((mfma_rate_kernel<KIND, 16>), dim3(grid), dim3(MR_THREADS), 0, s, out, iters, 1.0f); break;
    case 32: hipLaunchKernelGGL((mfma_rate_kernel<KIND, 32>), dim3(grid), dim3(MR_THREADS), 0, s, out, iters, 1.0f); break;
    case 64: hipLaunchKernelGGL((mfma_rate_kernel<KIND, 64>), dim3(grid), dim3(MR_THREADS), 0, s, out, iters, 1.0f); break;
    default: return -1;
    }
    return hipGetLastError() == hipSuccess ? 0 : -4;
}

int cu_count()
{
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
        return -1;
    return cus;
}

}  // namespace

extern "C" int vox_probe_mfma_rate_entries(int waves_per_simd)
{
    const int cus = cu_count();
    if (waves_per_simd < 1 || waves_per_simd > 4 || cus < 1)
        return -1;
    return cus * waves_per_simd * MR_THREADS;
}

extern "C" int vox_probe_mfma_rate(int kind, int nv, int waves_per_simd, int iters, float *out, void *stream)
{
    if ((kind != 0 && kind != 1) || (nv != 0 && nv != 16 && nv != 32 && nv != 64) || waves_per_simd < 1 ||
        waves_per_simd > 4 || iters < 1 || iters > (1 << 24) || !out)
        return -1;   // refused before any HIP call
    const int entries = vox_probe_mfma_rate_entries(waves_per_simd);
    if (entries < 0)
        return -1;
    const int grid = entries / MR_THREADS;   // four waves per workgroup: one per SIMD and workgroup
    return kind == 0 ? launch_kind<0>(nv, grid, out, iters, (hipStream_t)stream)
                     : launch_kind<1>(nv, grid, out, iters, (hipStream_t)stream);
}
