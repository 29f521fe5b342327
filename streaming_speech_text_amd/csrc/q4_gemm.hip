// q4_gemm.hip - encoder-chunk linear Y = X * W^T with GGUF Q4_0 weights on the matrix cores.
//
// Pages: the audio encoder is 1280 wide (voxtral.c page "Mistral Voxtral Realtime 4B 음성 인식
// 모델의 순수 C 기반 CPU 전용 추론 구현", GeekNews 26608, section 모델 아키텍처) and runs over chunks
// of frames (section 주요 기능); the quantised path keeps its linears as GGUF Q4_0 with
// dequantisation fused into the product (Rust port page, GeekNews 26595, section 아키텍처).
//
// Exactness: a dequantised weight (code - 8) * d needs up to 15 significant bits, more than
// bf16 holds, so the matrix cores never see it.  Each 32-input Q4_0 block is one
// v_mfma_f32_16x16x32_bf16 whose B operand holds the exact integers (code - 8) in bf16 and
// whose A operand holds the bf16 activations; the fp32 result is multiplied by the block's
// scale d and accumulated in fp32 on the vector units.
//
// Tiling: a workgroup of 4 waves owns a 64 x 64 tile of Y; each wave a 32 x 32 quarter (2 x 2
// MFMA blocks).  Per Q4_0 block column the workgroup stages X[64][32] (bf16) and the 64 weight
// blocks in LDS, expands the codes once into bf16 fragments in LDS, and every wave issues its
// four MFMAs.  The next block column is loaded into registers while the current one is used.
//
// Order of k inside a block: the MFMA sums over its 32 k slots; which hardware slot holds
// which input does not matter as long as A and B agree.  Lane group g (= lane / 16) takes
// code bytes 4g..4g+3, i.e. inputs {4g..4g+3} (low nibbles) then {16+4g..16+4g+3} (high
// nibbles), and reads the activations of the same inputs.
#include "vox_common.h"
#include "vox_host.h"

namespace vox {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4v __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2v __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));

constexpr int GM_TM = 64;          // tile rows (M)
constexpr int GM_TN = 64;          // tile columns (N)
constexpr int GM_THREADS = 256;
constexpr int XS_PITCH = 40;       // uint16 per staged X row: 32 inputs + 8 pad (bank spread)
constexpr int BS_PITCH = 40;       // uint16 per staged column: 4 fragments x 8 + 8 pad

// bf16 bits of the small integer v (exact): the upper half of its fp32 pattern.
__device__ __forceinline__ uint32_t pack_bf16_pair(float lo, float hi)
{
    return (__builtin_bit_cast(uint32_t, lo) >> 16) | (__builtin_bit_cast(uint32_t, hi) & 0xFFFF0000u);
}

__global__ __launch_bounds__(GM_THREADS) void q4_gemm_kernel(const uint8_t *__restrict__ w,
                                                            const uint16_t *__restrict__ x, float *__restrict__ y,
                                                            int m, int n, int k)
{
    __shared__ __attribute__((aligned(16))) uint16_t xs[GM_TM * XS_PITCH];   // X[64][32] of one block column
    __shared__ __attribute__((aligned(16))) uint16_t bs[GM_TN * BS_PITCH];   // (code-8) as bf16, fragment order
    __shared__ float ds[GM_TN];                                               // block scales

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int grp = lane >> 4;       // k group of the lane inside the MFMA
    const int l16 = lane & 15;
    const int m0 = blockIdx.y * GM_TM;
    const int n0 = blockIdx.x * GM_TN;
    const int wm = (wave >> 1) * 32;  // this wave's quarter of the tile
    const int wn = (wave & 1) * 32;
    const int nb = k / 32;
    const size_t row_bytes = (size_t)nb * 18;

    // staging roles: X: thread -> (row tid/4, 8 inputs (tid%4)*8 ..); W: thread -> (column tid/4,
    // code bytes 4*(tid%4) .. +3) plus, for tid%4 == 0, the scale
    const int xr = tid >> 2, xq = tid & 3;
    const int wc = tid >> 2, wq = tid & 3;
    const bool x_ok = m0 + xr < m;
    const bool w_ok = n0 + wc < n;
    const uint16_t *xrow = x + (size_t)(x_ok ? m0 + xr : 0) * k + xq * 8;
    const uint8_t *wrow = w + (size_t)(w_ok ? n0 + wc : 0) * row_bytes;

    f32x4v acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
            acc[i][j] = 0.0f;

    // prefetch registers for one block column
    u32x4v xv;
    uint32_t qv, dv;
    auto load = [&](int b) {
        xv = x_ok ? *reinterpret_cast<const u32x4v *>(xrow + (size_t)b * 32) : (u32x4v)0u;
        const uint8_t *blk = wrow + (size_t)b * 18;
        // the 4 code bytes 2+4q..5+4q sit at a 2-byte aligned address: two 16-bit loads
        const uint16_t *q16 = reinterpret_cast<const uint16_t *>(blk + 2 + 4 * wq);
        qv = w_ok ? ((uint32_t)q16[0] | ((uint32_t)q16[1] << 16)) : 0x88888888u;
        dv = w_ok ? (uint32_t)(*reinterpret_cast<const uint16_t *>(blk)) : 0u;
    };

    load(0);
    for (int b = 0; b < nb; ++b) {
        // stage this block column
        *reinterpret_cast<u32x4v *>(xs + xr * XS_PITCH + xq * 8) = xv;
        {
            // expand 8 codes into (code - 8) bf16 in fragment order: low nibbles then high
            const uint32_t lo = qv & 0x0F0F0F0Fu;
            const uint32_t hi = (qv >> 4) & 0x0F0F0F0Fu;
            float f[8];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                f[j] = (float)((lo >> (8 * j)) & 0xFFu) - 8.0f;
                f[4 + j] = (float)((hi >> (8 * j)) & 0xFFu) - 8.0f;
            }
            u32x4v packed;
            packed.x = pack_bf16_pair(f[0], f[1]);
            packed.y = pack_bf16_pair(f[2], f[3]);
            packed.z = pack_bf16_pair(f[4], f[5]);
            packed.w = pack_bf16_pair(f[6], f[7]);
            *reinterpret_cast<u32x4v *>(bs + wc * BS_PITCH + wq * 8) = packed;
            if (wq == 0)
                ds[wc] = half_bits_to_float(dv);
        }
        __syncthreads();
        if (b + 1 < nb)
            load(b + 1);   // next block column in flight during the MFMAs

        // A fragments: rows wm + 16i + l16, inputs {4g..4g+3} and {16+4g..16+4g+3}
        bf16x8 afr[2], bfr[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const uint16_t *xp = xs + (wm + 16 * i + l16) * XS_PITCH;
            const u32x2v a0 = *reinterpret_cast<const u32x2v *>(xp + 4 * grp);
            const u32x2v a1 = *reinterpret_cast<const u32x2v *>(xp + 16 + 4 * grp);
            const u32x4v a = {a0.x, a0.y, a1.x, a1.y};
            afr[i] = __builtin_bit_cast(bf16x8, a);
        }
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const u32x4v bv = *reinterpret_cast<const u32x4v *>(bs + (wn + 16 * j + l16) * BS_PITCH + grp * 8);
            bfr[j] = __builtin_bit_cast(bf16x8, bv);
        }
        float dcol[2];
#pragma unroll
        for (int j = 0; j < 2; ++j)
            dcol[j] = ds[wn + 16 * j + l16];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const f32x4v t = __builtin_amdgcn_mfma_f32_16x16x32_bf16(afr[i], bfr[j], (f32x4v)0.0f, 0, 0, 0);
                acc[i][j] += dcol[j] * t;
            }
        }
        __syncthreads();
    }

    // D layout of a 16x16 MFMA block: lane holds rows 4*(lane/16) .. +3 of column lane%16
#pragma unroll
    for (int i = 0; i < 2; ++i) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int col = n0 + wn + 16 * j + l16;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = m0 + wm + 16 * i + 4 * grp + r;
                if (row < m && col < n)
                    y[(size_t)row * n + col] = acc[i][j][r];
            }
        }
    }
}

}  // namespace vox

using namespace vox;

extern "C" int vox_q4_gemm(const void *w_q4, const uint16_t *x_bf16, float *y, int64_t m, int64_t n, int64_t k,
                           void *stream)
{
    if (m < 0 || n < 0 || k <= 0 || k % 32)
        return fail(VOX_E_INVAL, "vox_q4_gemm: need m, n >= 0 and k a positive multiple of 32 (m=%lld n=%lld k=%lld)",
                    (long long)m, (long long)n, (long long)k);
    if (m == 0 || n == 0)
        return ok();
    if (!w_q4 || !x_bf16 || !y)
        return fail(VOX_E_INVAL, "vox_q4_gemm: null pointer");
    if (m > (1 << 24) || n > (1 << 24) || k > (1 << 24))
        return fail(VOX_E_UNSUPPORTED, "vox_q4_gemm: dimension too large");
    if (!aligned(x_bf16, 16) || !aligned(w_q4, 2))
        return fail(VOX_E_UNSUPPORTED, "vox_q4_gemm: x must be 16-byte and w 2-byte aligned");
    const size_t wbytes = (size_t)n * (size_t)(k / 32) * 18, xbytes = (size_t)m * k * 2, ybytes = (size_t)m * n * 4;
    if (overlaps(y, ybytes, x_bf16, xbytes) || overlaps(y, ybytes, w_q4, wbytes))
        return fail(VOX_E_INVAL, "vox_q4_gemm: y overlaps an input");
    const dim3 grid((unsigned)((n + GM_TN - 1) / GM_TN), (unsigned)((m + GM_TM - 1) / GM_TM));
    hipLaunchKernelGGL(q4_gemm_kernel, grid, dim3(GM_THREADS), 0, (hipStream_t)stream, (const uint8_t *)w_q4, x_bf16,
                       y, (int)m, (int)n, (int)k);
    int st = check_launch("vox_q4_gemm");
    return st ? st : ok();
}
