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
// Work split: a workgroup of 8 waves owns a (16*MI) x (16*NJ) tile of Y.  The eight waves split
// the K blocks into eight contiguous ranges; each wave loads its MFMA operands straight from
// memory (no LDS staging, no barrier per block) with GEMV_PF blocks in flight in registers, and
// at the end the eight partial tiles are added in LDS in wave order (deterministic).  Chunks of
// a few frames (small M) are weight-streaming problems; splitting K over the waves is what
// puts enough requests in flight.
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

constexpr int GM_WAVES = 8;
constexpr int GM_THREADS = 64 * GM_WAVES;
constexpr int GM_PF = 4;           // K blocks in flight per wave

// bf16 bits of two small integers given as exact fp32 values: the upper halves.
__device__ __forceinline__ uint32_t pack_bf16_pair(float lo, float hi)
{
    return (__builtin_bit_cast(uint32_t, lo) >> 16) | (__builtin_bit_cast(uint32_t, hi) & 0xFFFF0000u);
}

// (code - 8) as bf16 for the 8 codes of one lane (4 code bytes): low nibbles then high nibbles.
__device__ __forceinline__ bf16x8 codes_to_bf16(uint32_t q)
{
    const uint32_t lo = q & 0x0F0F0F0Fu;
    const uint32_t hi = (q >> 4) & 0x0F0F0F0Fu;
    float f[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        f[e] = (float)((lo >> (8 * e)) & 0xFFu) - 8.0f;
        f[4 + e] = (float)((hi >> (8 * e)) & 0xFFu) - 8.0f;
    }
    u32x4v p;
    p.x = pack_bf16_pair(f[0], f[1]);
    p.y = pack_bf16_pair(f[2], f[3]);
    p.z = pack_bf16_pair(f[4], f[5]);
    p.w = pack_bf16_pair(f[6], f[7]);
    return __builtin_bit_cast(bf16x8, p);
}

template <int MI, int NJ>
__global__ __launch_bounds__(GM_THREADS) void q4_gemm_kernel(const uint8_t *__restrict__ w,
                                                            const uint16_t *__restrict__ x, float *__restrict__ y,
                                                            int m, int n, int k)
{
    __shared__ float red[GM_WAVES][MI * NJ][4][64];

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int grp = lane >> 4;
    const int l16 = lane & 15;
    const int n0 = blockIdx.x * 16 * NJ;
    const int m0 = blockIdx.y * 16 * MI;
    const int nb = k / 32;
    const size_t row_bytes = (size_t)nb * 18;
    const int kb0 = (int)((int64_t)wave * nb / GM_WAVES);
    const int kb1 = (int)((int64_t)(wave + 1) * nb / GM_WAVES);

    // operand rows of this lane (past the edge: the last valid row; masked at the store)
    const uint16_t *xrow[MI];
#pragma unroll
    for (int i = 0; i < MI; ++i) {
        const int r = min(m0 + 16 * i + l16, m - 1);
        xrow[i] = x + (size_t)r * k;
    }
    const uint8_t *wrow[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        const int c = min(n0 + 16 * j + l16, n - 1);
        wrow[j] = w + (size_t)c * row_bytes;
    }

    f32x4v acc[MI][NJ];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
            acc[i][j] = 0.0f;

    // ring of GM_PF prefetched blocks; loads are unconditional (indices clamped), the scale of
    // a block past the wave's range is zeroed instead
    u32x2v xa[GM_PF][MI][2];
    uint32_t qv[GM_PF][NJ], dv[GM_PF][NJ];
    auto load = [&](int slot, int b) {
        const int bb = b < kb1 ? b : (kb1 > kb0 ? kb1 - 1 : 0);
#pragma unroll
        for (int i = 0; i < MI; ++i) {
            const uint16_t *xp = xrow[i] + (size_t)bb * 32 + 4 * grp;
            xa[slot][i][0] = *reinterpret_cast<const u32x2v *>(xp);
            xa[slot][i][1] = *reinterpret_cast<const u32x2v *>(xp + 16);
        }
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            const uint8_t *blk = wrow[j] + (size_t)bb * 18;
            const uint16_t *q16 = reinterpret_cast<const uint16_t *>(blk + 2 + 4 * grp);   // 2-byte aligned
            qv[slot][j] = (uint32_t)q16[0] | ((uint32_t)q16[1] << 16);
            dv[slot][j] = (uint32_t)(*reinterpret_cast<const uint16_t *>(blk));
        }
    };
#pragma unroll
    for (int s = 0; s < GM_PF; ++s)
        load(s, kb0 + s);

    for (int b0 = kb0; b0 < kb1; b0 += GM_PF) {
#pragma unroll
        for (int s = 0; s < GM_PF; ++s) {
            const int b = b0 + s;
            bf16x8 afr[MI], bfr[NJ];
            float d[NJ];
#pragma unroll
            for (int i = 0; i < MI; ++i) {
                const u32x4v av = {xa[s][i][0].x, xa[s][i][0].y, xa[s][i][1].x, xa[s][i][1].y};
                afr[i] = __builtin_bit_cast(bf16x8, av);
            }
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                bfr[j] = codes_to_bf16(qv[s][j]);
                d[j] = b < kb1 ? half_bits_to_float(dv[s][j]) : 0.0f;
            }
            load(s, b + GM_PF);   // refill: the ring stays GM_PF blocks ahead
#pragma unroll
            for (int i = 0; i < MI; ++i)
#pragma unroll
                for (int j = 0; j < NJ; ++j) {
                    const f32x4v t = __builtin_amdgcn_mfma_f32_16x16x32_bf16(afr[i], bfr[j], (f32x4v)0.0f, 0, 0, 0);
                    acc[i][j] += d[j] * t;
                }
        }
    }

    // add the eight waves' partial tiles in wave order
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                red[wave][i * NJ + j][r][lane] = acc[i][j][r];
    __syncthreads();
    // D layout of a 16x16 MFMA block: lane holds rows 4*(lane/16) .. +3 of column lane%16
    for (int e = tid; e < MI * NJ * 4 * 64; e += GM_THREADS) {
        const int ln = e & 63, r = (e >> 6) & 3, blk = e >> 8;
        const int i = blk / NJ, j = blk % NJ;
        float v = red[0][blk][r][ln];
#pragma unroll
        for (int wv = 1; wv < GM_WAVES; ++wv)
            v += red[wv][blk][r][ln];
        const int row = m0 + 16 * i + 4 * (ln >> 4) + r;
        const int col = n0 + 16 * j + (ln & 15);
        if (row < m && col < n)
            y[(size_t)row * n + col] = v;
    }
}

template <int MI, int NJ>
static int launch_gemm(const void *w, const uint16_t *x, float *y, int m, int n, int k, hipStream_t s)
{
    const dim3 grid((unsigned)((n + 16 * NJ - 1) / (16 * NJ)), (unsigned)((m + 16 * MI - 1) / (16 * MI)));
    hipLaunchKernelGGL((q4_gemm_kernel<MI, NJ>), grid, dim3(GM_THREADS), 0, s, (const uint8_t *)w, x, y, m, n, k);
    return check_launch("vox_q4_gemm");
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
    if (!aligned(x_bf16, 8) || !aligned(w_q4, 2))
        return fail(VOX_E_UNSUPPORTED, "vox_q4_gemm: x must be 8-byte and w 2-byte aligned");
    const size_t wbytes = (size_t)n * (size_t)(k / 32) * 18, xbytes = (size_t)m * k * 2, ybytes = (size_t)m * n * 4;
    if (overlaps(y, ybytes, x_bf16, xbytes) || overlaps(y, ybytes, w_q4, wbytes))
        return fail(VOX_E_INVAL, "vox_q4_gemm: y overlaps an input");
    hipStream_t s = (hipStream_t)stream;
    int st;
    if (m <= 16)
        st = launch_gemm<1, 1>(w_q4, x_bf16, y, (int)m, (int)n, (int)k, s);
    else if (m <= 32)
        st = launch_gemm<2, 2>(w_q4, x_bf16, y, (int)m, (int)n, (int)k, s);
    else
        st = launch_gemm<4, 2>(w_q4, x_bf16, y, (int)m, (int)n, (int)k, s);
    return st ? st : ok();
}
