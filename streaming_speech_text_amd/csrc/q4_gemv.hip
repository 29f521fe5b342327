// q4_gemv.hip - Q4_0 dequantisation and the standalone Q4_0 GEMV entry points.
//
// Rust/Burn port page ("Mistral의 Voxtral Mini 4B Realtime 모델을 Rust로 구현해 브라우저에서
// 실행", GeekNews 26595), section 아키텍처: the Q4 GGUF path quantises the linears as GGUF Q4_0
// and fuses dequantisation with the matrix product in custom shaders.  This file is the
// MI355X form of that operation for one activation vector.
#include "gemv_core.h"
#include "vox_host.h"

namespace vox {

// ---------------------------------------------------------------------------------------
// Dequantisation: one thread per block.  (code - 8) * d in fp32 is exact.
// ---------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void q4_dequant_kernel(const uint8_t *__restrict__ w, float *__restrict__ out,
                                                         int64_t n_blocks)
{
    const int64_t b = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (b >= n_blocks)
        return;
    const uint8_t *blk = w + b * 18;
    const float d = half_bits_to_float((uint32_t)blk[0] | ((uint32_t)blk[1] << 8));
    float *o = out + b * 32;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        const uint32_t q = blk[2 + j];
        o[j] = (float)((int)(q & 15u) - 8) * d;
        o[j + 16] = (float)((int)(q >> 4) - 8) * d;
    }
}

// ---------------------------------------------------------------------------------------
// Generic GEMV for any k % 32 == 0 and any alignment: one wavefront per row, lanes stride
// over the blocks, byte loads.  Correct everywhere; the tiled kernel below is the fast path.
// ---------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void q4_gemv_generic_kernel(const uint8_t *__restrict__ w,
                                                              const float *__restrict__ x,
                                                              float *__restrict__ y, int64_t n, int64_t k)
{
    const int64_t row = (int64_t)blockIdx.x * 4 + threadIdx.x / 64;
    const int lane = threadIdx.x % 64;
    if (row >= n)
        return;
    const int64_t nb = k / 32;
    const uint8_t *rp = w + row * nb * 18;
    float acc = 0.0f;
    for (int64_t b = lane; b < nb; b += 64) {
        const uint8_t *blk = rp + b * 18;
        const float d = half_bits_to_float((uint32_t)blk[0] | ((uint32_t)blk[1] << 8));
        const float *xb = x + b * 32;
        float s = 0.0f;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const uint32_t q = blk[2 + j];
            s = fmaf((float)((int)(q & 15u) - 8), xb[j], s);
            s = fmaf((float)((int)(q >> 4) - 8), xb[j + 16], s);
        }
        acc = fmaf(d, s, acc);
    }
    acc = wave_sum(acc);
    if (lane == 0)
        y[row] = acc;
}

// ---------------------------------------------------------------------------------------
// Tiled fast path (K in {3072, 4096, 9216}: the decoder's linear widths; 1280, 5120: the
// encoder's).
// ---------------------------------------------------------------------------------------
template <class Gm>
struct PlainGemvPolicy {
    const uint8_t *w;
    const float *x;
    float *y;
    int64_t n;

    typedef PlainX<Gm::NT, Gm::K> XRegs;
    __device__ void x_issue(XRegs &r) { r.issue(x); }
    __device__ float x_stage(XRegs &r, float *xs, float *) { return r.stage(xs); }
    __device__ void pre(int) {}
    __device__ int num_tiles() const { return (int)((n + Gm::R - 1) / Gm::R); }
    __device__ const uint8_t *slice(int t, int, int &rows_valid) const
    {
        const int64_t r0 = (int64_t)t * Gm::R;
        const int64_t left = n - r0;
        rows_valid = left < Gm::R ? (int)left : Gm::R;
        return w + r0 * Gm::RB;
    }
    __device__ void epilogue(int t, const float *rowsum)
    {
        const int tid = threadIdx.x;
        const int64_t r = (int64_t)t * Gm::R + tid;
        if (tid < Gm::R && r < n)
            y[r] = rowsum[tid];
    }
    __device__ void finish(float *) {}
};

// Four waves per SIMD (at most 128 VGPRs): with 3-wave workgroups, five resident workgroups per
// compute unit.  Measured at the LM-head shape: 8-row tiles with four waves per SIMD beat
// 16-row tiles with three (16-row tiles do not fit 128 VGPRs).
template <class Gm>
__global__ __launch_bounds__(Gm::NT) __attribute__((amdgpu_waves_per_eu(4))) void q4_gemv_tiled_kernel(PlainGemvPolicy<Gm> P)
{
    gemv_tiles<Gm>(P);
}

template <class Gm>
static int launch_tiled(const void *w, const float *x, float *y, int64_t n, hipStream_t s)
{
    static std::atomic<int> occ_cache{0};
    const int occ = resident_per_cu(occ_cache, q4_gemv_tiled_kernel<Gm>, Gm::NT);
    const int64_t ntiles = (n + Gm::R - 1) / Gm::R;
    const int64_t cap = (int64_t)occ * cu_count();
    const int grid = (int)(ntiles < cap ? ntiles : cap);
    PlainGemvPolicy<Gm> P{(const uint8_t *)w, x, y, n};
    hipLaunchKernelGGL(q4_gemv_tiled_kernel<Gm>, dim3(grid), dim3(Gm::NT), 0, s, P);
    return check_launch("q4_gemv tiled launch");
}

// Picks the tile height: 8-row tiles for long matrices, 4-row ones so that a few thousand rows
// still spread over every compute unit.
static int pick_rows(int64_t n)
{
    return n >= 8 * 2 * (int64_t)cu_count() ? 8 : 4;
}

int q4_gemv_launch(const void *w, const float *x, float *y, int64_t n, int64_t k, hipStream_t s)
{
    const bool fast_layout = aligned(w, 16) && aligned(x, 16);
    const bool tall = pick_rows(n) == 8;
    if (fast_layout && k == 3072)
        return tall ? launch_tiled<GemvGeom<3072, 192, 8>>(w, x, y, n, s)
                    : launch_tiled<GemvGeom<3072, 192, 4>>(w, x, y, n, s);
    if (fast_layout && k == 4096)
        return tall ? launch_tiled<GemvGeom<4096, 256, 8>>(w, x, y, n, s)
                    : launch_tiled<GemvGeom<4096, 256, 4>>(w, x, y, n, s);
    if (fast_layout && k == 9216)
        return tall ? launch_tiled<GemvGeom<9216, 576, 8>>(w, x, y, n, s)
                    : launch_tiled<GemvGeom<9216, 576, 4>>(w, x, y, n, s);
    // the encoder widths ([VC] 모델 아키텍처: width 1280, feed-forward 5120): 20 or 80 threads per
    // row, five-wave workgroups; at K = 1280 a workgroup holds 16 row groups, so 16-row tiles
    if (fast_layout && k == 1280)
        return launch_tiled<GemvGeom<1280, 320, 16>>(w, x, y, n, s);
    if (fast_layout && k == 5120)
        return tall ? launch_tiled<GemvGeom<5120, 320, 8>>(w, x, y, n, s)
                    : launch_tiled<GemvGeom<5120, 320, 4>>(w, x, y, n, s);
    const int64_t grid = (n + 3) / 4;
    hipLaunchKernelGGL(q4_gemv_generic_kernel, dim3((unsigned)grid), dim3(256), 0, s, (const uint8_t *)w, x, y, n,
                       k);
    return check_launch("q4_gemv generic launch");
}

}  // namespace vox

using namespace vox;

extern "C" int vox_q4_dequant(const void *w_q4, int64_t n_blocks, float *out, void *stream)
{
    if (n_blocks < 0)
        return fail(VOX_E_INVAL, "vox_q4_dequant: n_blocks < 0");
    if (n_blocks == 0)
        return ok();
    if (!w_q4 || !out)
        return fail(VOX_E_INVAL, "vox_q4_dequant: null pointer");
    if (n_blocks > ((int64_t)1 << 40))
        return fail(VOX_E_INVAL, "vox_q4_dequant: n_blocks too large");
    if (overlaps(w_q4, (size_t)n_blocks * 18, out, (size_t)n_blocks * 128))
        return fail(VOX_E_INVAL, "vox_q4_dequant: out overlaps the weights");
    const int64_t grid = (n_blocks + 255) / 256;
    if (grid > 0x7FFFFFFF)
        return fail(VOX_E_UNSUPPORTED, "vox_q4_dequant: too many blocks for one launch");
    hipLaunchKernelGGL(q4_dequant_kernel, dim3((unsigned)grid), dim3(256), 0, (hipStream_t)stream,
                       (const uint8_t *)w_q4, out, n_blocks);
    int st = check_launch("vox_q4_dequant");
    return st ? st : ok();
}

extern "C" int vox_q4_gemv(const void *w_q4, const float *x, float *y, int64_t n, int64_t k, void *stream)
{
    if (n < 0 || k <= 0 || k % 32)
        return fail(VOX_E_INVAL, "vox_q4_gemv: need n >= 0 and k a positive multiple of 32 (n=%lld k=%lld)",
                    (long long)n, (long long)k);
    if (n == 0)
        return ok();
    if (!w_q4 || !x || !y)
        return fail(VOX_E_INVAL, "vox_q4_gemv: null pointer");
    if (n > 0x7FFFFFFFll || k > (1ll << 24))
        return fail(VOX_E_UNSUPPORTED, "vox_q4_gemv: n or k too large");
    const size_t wbytes = (size_t)n * (size_t)(k / 32) * 18;
    if (overlaps(y, (size_t)n * 4, x, (size_t)k * 4) || overlaps(y, (size_t)n * 4, w_q4, wbytes))
        return fail(VOX_E_INVAL, "vox_q4_gemv: y overlaps an input");
    int st = q4_gemv_launch(w_q4, x, y, n, k, (hipStream_t)stream);
    return st ? st : ok();
}
