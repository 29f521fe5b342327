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

// Cross-lane data movement with DPP (one VALU op each, no LDS round trip).
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}
constexpr int DPP_QUAD_XOR1 = 0xB1;   // quad_perm [1,0,3,2]
constexpr int DPP_QUAD_XOR2 = 0x4E;   // quad_perm [2,3,0,1]
constexpr int DPP_ROW_ROR4 = 0x124;   // rotate right by 4 within a row of 16 lanes
constexpr int DPP_ROW_ROR8 = 0x128;   // rotate right by 8 within a row of 16 lanes

// Sum over each row of 16 lanes; every lane of the row gets the row's total.  The order of the
// additions is fixed (deterministic).
__device__ __forceinline__ float row16_sum(float v)
{
    v += dpp_f<DPP_QUAD_XOR1>(v);
    v += dpp_f<DPP_QUAD_XOR2>(v);
    v += dpp_f<DPP_ROW_ROR4>(v);
    v += dpp_f<DPP_ROW_ROR8>(v);
    return v;
}

// Sum over each quad of lanes (fixed order); every lane of the quad gets the quad's total.
__device__ __forceinline__ float quad_sum(float v)
{
    v += dpp_f<DPP_QUAD_XOR1>(v);
    v += dpp_f<DPP_QUAD_XOR2>(v);
    return v;
}

__device__ __forceinline__ float row16_max(float v)
{
    v = fmaxf(v, dpp_f<DPP_QUAD_XOR1>(v));
    v = fmaxf(v, dpp_f<DPP_QUAD_XOR2>(v));
    v = fmaxf(v, dpp_f<DPP_ROW_ROR4>(v));
    v = fmaxf(v, dpp_f<DPP_ROW_ROR8>(v));
    return v;
}

__device__ __forceinline__ float lane_value(float v, int lane)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), lane));
}

// Sum over the 64 lanes of a wavefront, in a fixed order; every lane gets the total.
__device__ __forceinline__ float wave_sum(float v)
{
    v = row16_sum(v);
    return ((lane_value(v, 0) + lane_value(v, 16)) + lane_value(v, 32)) + lane_value(v, 48);
}

__device__ __forceinline__ float wave_max(float v)
{
    v = row16_max(v);
    return fmaxf(fmaxf(lane_value(v, 0), lane_value(v, 16)), fmaxf(lane_value(v, 32), lane_value(v, 48)));
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
