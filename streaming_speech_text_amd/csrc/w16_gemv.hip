// w16_gemv.hip - matrix-vector product over 16-bit weights (bf16 or fp16) with fp32 activations.
//
// Pages: voxtral.c keeps its weights as BF16 (voxtral.c page "Mistral Voxtral Realtime 4B 음성 인식
// 모델의 순수 C 기반 CPU 전용 추론 구현", GeekNews 26608, section 모델 다운로드 및 구성) and its Metal
// path runs from an F16 copy of them (section 메모리 요구사항); its decoder step time is quoted at
// that precision (section 성능 벤치마크).
//
// y[r] = sum_k W[r][k] x[k], fp32 accumulation.  One wave per R rows: lane L takes elements
// 8L + 512j of each row with 16-byte loads (one load instruction covers 1 KB of a row), and the
// loads of CH such chunks for all R rows are issued before any arithmetic.  x comes through the
// cache in the same chunks.  bf16 widens by a shift or a mask; fp16 goes through v_fma_mix_f32,
// which reads either half of a dword and rounds once.  Each row's 64 partial sums are added in a
// fixed order.
#include "gemv_core.h"   // fma_f16h, wave_sum
#include "vox_host.h"

namespace vox {

constexpr int W16_THREADS = 256;

typedef float f32x4w __attribute__((ext_vector_type(4)));

template <int FMT>   // 0: bf16, 1: fp16
__device__ __forceinline__ float dot8(const u32x4 &wq, const f32x4w &x0, const f32x4w &x1, float acc)
{
    const uint32_t q[4] = {wq.x, wq.y, wq.z, wq.w};
    const float xs[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        if constexpr (FMT == 0) {
            acc = fmaf(__builtin_bit_cast(float, q[i] << 16), xs[2 * i], acc);
            acc = fmaf(__builtin_bit_cast(float, q[i] & 0xFFFF0000u), xs[2 * i + 1], acc);
        } else {
            acc = fma_f16h<false>(q[i], xs[2 * i], acc);
            acc = fma_f16h<true>(q[i], xs[2 * i + 1], acc);
        }
    }
    return acc;
}

template <int FMT, int R, int CH>
__global__ __launch_bounds__(W16_THREADS) void w16_gemv_kernel(const uint16_t *__restrict__ w,
                                                               const float *__restrict__ x, float *__restrict__ y,
                                                               int n, int k)
{
    const int lane = threadIdx.x & 63;
    const int row0 = (blockIdx.x * (W16_THREADS / 64) + (threadIdx.x >> 6)) * R;
    if (row0 >= n)
        return;   // the whole wave (no barrier in this kernel)
    const uint16_t *wr[R];
#pragma unroll
    for (int r = 0; r < R; ++r)
        wr[r] = w + (size_t)min(row0 + r, n - 1) * (size_t)k;   // past the last row: reread it, not stored
    float acc[R];
#pragma unroll
    for (int r = 0; r < R; ++r)
        acc[r] = 0.0f;

    for (int c0 = 0; c0 < k; c0 += 512 * CH) {
        u32x4 wq[CH][R];
        f32x4w xa[CH][2];
#pragma unroll
        for (int j = 0; j < CH; ++j) {
            const int e = c0 + 512 * j + 8 * lane;
            const int ee = e < k ? e : 0;   // past the row end: read element 0, weigh it by 0
            // non-temporal: each weight is read once (measured on MI355X: the LM-head shape 126 ->
            // 113 us, the chain of a decoder step's GEMVs 6.5-7 % faster)
#pragma unroll
            for (int r = 0; r < R; ++r)
                wq[j][r] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(wr[r] + ee));
            xa[j][0] = *reinterpret_cast<const f32x4w *>(x + ee);
            xa[j][1] = *reinterpret_cast<const f32x4w *>(x + ee + 4);
            if (e >= k) {
                xa[j][0] = (f32x4w)0.0f;
                xa[j][1] = (f32x4w)0.0f;
            }
        }
#pragma unroll
        for (int j = 0; j < CH; ++j)
#pragma unroll
            for (int r = 0; r < R; ++r)
                acc[r] = dot8<FMT>(wq[j][r], xa[j][0], xa[j][1], acc[r]);
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const float s = wave_sum(acc[r]);
        if (lane == 0 && row0 + r < n)
            y[row0 + r] = s;
    }
}

template <int FMT, int R, int CH>
static void launch_w16(const void *w, const float *x, float *y, int64_t n, int64_t k, hipStream_t s)
{
    const int64_t waves = (n + R - 1) / R;
    const unsigned blocks = (unsigned)((waves + W16_THREADS / 64 - 1) / (W16_THREADS / 64));
    hipLaunchKernelGGL((w16_gemv_kernel<FMT, R, CH>), dim3(blocks), dim3(W16_THREADS), 0, s, (const uint16_t *)w, x,
                       y, (int)n, (int)k);
}

}  // namespace vox

using namespace vox;

extern "C" int vox_w16_gemv(const void *w, int fmt, const float *x, float *y, int64_t n, int64_t k, void *stream)
{
    if (n < 0 || k <= 0 || k % 8 || (fmt != VOX_W16_BF16 && fmt != VOX_W16_F16))
        return fail(VOX_E_INVAL, "vox_w16_gemv: need n >= 0, k a positive multiple of 8 and fmt bf16 or f16 "
                                 "(n=%lld k=%lld fmt=%d)",
                    (long long)n, (long long)k, fmt);
    if (n == 0)
        return ok();
    if (!w || !x || !y)
        return fail(VOX_E_INVAL, "vox_w16_gemv: null pointer");
    if (n > (1LL << 30) || k > (1LL << 30))
        return fail(VOX_E_UNSUPPORTED, "vox_w16_gemv: n and k up to 2^30");
    if (!aligned(w, 16) || !aligned(x, 16))
        return fail(VOX_E_UNSUPPORTED, "vox_w16_gemv: w and x must be 16-byte aligned");
    const size_t wbytes = (size_t)n * (size_t)k * 2;
    if (overlaps(y, (size_t)n * 4, w, wbytes) || overlaps(y, (size_t)n * 4, x, (size_t)k * 4))
        return fail(VOX_E_INVAL, "vox_w16_gemv: y overlaps an input");
    hipStream_t s = (hipStream_t)stream;
    // Chunks per batch, measured on MI355X: tall matrices (the LM head) stream best with a whole
    // row's loads in one batch (six chunks at 3072 inputs); the decoder layers' matrices (up to
    // 9216 rows) do better with batches of two chunks and more waves in flight.
    const bool tall = n >= 32768 && k <= 512 * 6;
    if (fmt == VOX_W16_BF16) {
        if (tall)
            launch_w16<0, 2, 6>(w, x, y, n, k, s);
        else
            launch_w16<0, 2, 2>(w, x, y, n, k, s);
    } else {
        if (tall)
            launch_w16<1, 2, 6>(w, x, y, n, k, s);
        else
            launch_w16<1, 2, 2>(w, x, y, n, k, s);
    }
    const int st = check_launch("vox_w16_gemv");
    return st ? st : ok();
}
