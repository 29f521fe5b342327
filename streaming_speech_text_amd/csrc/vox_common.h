// vox_common.h - helpers shared by the HIP kernels and the host side of libvox.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace vox {

// ---------------------------------------------------------------------------------------
// device helpers
// ---------------------------------------------------------------------------------------

// fp16 bit pattern (low 16 bits) -> fp32, exact (gfx950 converts fp16 subnormals exactly).
__device__ __forceinline__ float half_bits_to_float(uint32_t bits)
{
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(bits & 0xFFFFu));
}

__device__ __forceinline__ float bf16_bits_to_float(uint32_t bits)
{
    return __builtin_bit_cast(float, bits << 16);
}

// Sum over the 64 lanes of a wavefront; every lane gets the total.
__device__ __forceinline__ float wave_sum(float v)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1)
        v += __shfl_xor(v, o, 64);
    return v;
}

__device__ __forceinline__ float wave_max(float v)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1)
        v = fmaxf(v, __shfl_xor(v, o, 64));
    return v;
}

// Order-preserving map of a non-NaN float to an unsigned key (larger float -> larger key).
__device__ __forceinline__ uint32_t float_order_key(float f)
{
    uint32_t u = __builtin_bit_cast(uint32_t, f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Packed (value, index) key for a device-wide argmax with atomicMax: the value decides,
// then the lower index wins a tie.
__device__ __forceinline__ unsigned long long argmax_key(float v, uint32_t idx)
{
    return ((unsigned long long)float_order_key(v) << 32) | (unsigned long long)(0xFFFFFFFFu - idx);
}

__device__ __forceinline__ uint32_t argmax_key_index(unsigned long long key)
{
    return 0xFFFFFFFFu - (uint32_t)(key & 0xFFFFFFFFull);
}

__device__ __forceinline__ float silu(float z)
{
    return z / (1.0f + __expf(-z));
}

}  // namespace vox
