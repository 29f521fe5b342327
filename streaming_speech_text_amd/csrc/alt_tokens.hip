// alt_tokens.hip - the greedy token and its alternatives from one step's logits.
//
// Pages: voxtral.c can show candidate tokens beside the chosen one, more of them for a higher
// cutoff (voxtral.c page "Mistral Voxtral Realtime 4B 음성 인식 모델의 순수 C 기반 CPU 전용 추론 구현",
// GeekNews 26608, section 사용 방법, --alt <cutoff>), the number of alternatives set on the stream
// (section C API 구조).
//
// Operation: with t the greedy token (largest logit, lowest index on a tie), token i is listed
// when l_i >= l_t + d in fp32, d = ln(1 - cutoff) rounded to fp32 (every token when cutoff >= 1),
// i.e. when its probability is at least (1 - cutoff) times the greedy token's.  The list runs by
// logit, higher first, ties to the lower index, at most max_out entries, each with its softmax
// probability over the whole vocabulary.
//
// Two kernels.  Each wave of the first takes 512 logits: their max and the sum of exp(l - max)
// (fixed order), and its max_out best (logit, index) keys from a bitonic sort held in registers
// (VALU lane exchanges, no LDS, no barriers).  One workgroup of the second folds all partial lists into the best
// max_out with the same in-wave sort, adds the partial sums rescaled to the global max (fixed
// order), and writes the list.  Keys pack an order-preserving image of the
// logit above the inverted index, so a larger key is a larger logit, then a lower index.
#include <cmath>

#include "vox_common.h"
#include "vox_host.h"

namespace vox {

constexpr int ALT_BLOCK = 512;         // logits per first-pass wave
constexpr int ALT_T2 = 1024;           // second-pass threads (16 waves)
constexpr int ALT_MAX_OUT = 32;
constexpr int64_t ALT_MAX_VOCAB = 262144;

typedef unsigned long long u64;

__device__ __forceinline__ float key_logit(u64 key)
{
    const uint32_t k = (uint32_t)(key >> 32);
    return __builtin_bit_cast(float, (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u(uint32_t v)
{
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, true);
}

// Larger and smaller of (own key, key of lane ^ m), m a power of two below 64, with VALU lane
// operations only.  m = 1, 2, 8: DPP quad permutes and a row rotation by 8; m = 4: DPP
// row_half_mirror (lane ^ 7) then quad_perm [3,2,1,0] (^ 3).  m = 16, 32: v_permlane16/32_swap,
// whose two results hold the own and the partner's value (in an order that depends on the row),
// so only their max and min are used.
__device__ __forceinline__ void pair_minmax(u64 v, int m, u64 &mx, u64 &mn)
{
    const uint32_t lo = (uint32_t)v, hi = (uint32_t)(v >> 32);
    u64 a = v, b;
    switch (m) {
    case 1: b = ((u64)dpp_u<0xB1>(hi) << 32) | dpp_u<0xB1>(lo); break;   // quad_perm [1,0,3,2]
    case 2: b = ((u64)dpp_u<0x4E>(hi) << 32) | dpp_u<0x4E>(lo); break;   // quad_perm [2,3,0,1]
    case 4: b = ((u64)dpp_u<0x1B>(dpp_u<0x141>(hi)) << 32) | dpp_u<0x1B>(dpp_u<0x141>(lo)); break;
    case 8: b = ((u64)dpp_u<0x128>(hi) << 32) | dpp_u<0x128>(lo); break;   // row_ror 8 = ^ 8 in a row
    case 16: {
        const auto l = __builtin_amdgcn_permlane16_swap(lo, lo, false, false);
        const auto h = __builtin_amdgcn_permlane16_swap(hi, hi, false, false);
        a = ((u64)h[0] << 32) | l[0];
        b = ((u64)h[1] << 32) | l[1];
        break;
    }
    default: {
        const auto l = __builtin_amdgcn_permlane32_swap(lo, lo, false, false);
        const auto h = __builtin_amdgcn_permlane32_swap(hi, hi, false, false);
        a = ((u64)h[0] << 32) | l[0];
        b = ((u64)h[1] << 32) | l[1];
        break;
    }
    }
    mx = a > b ? a : b;
    mn = a > b ? b : a;
}

// Descending bitonic sort of a wave's 512 keys, element r * 64 + lane in v[r], without barriers
// or LDS: pairs 64 or more apart are two registers of one lane, nearer pairs one register of two
// lanes exchanged with VALU lane operations.
__device__ __forceinline__ void wave_sort512_desc(u64 (&v)[8])
{
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int k = 2; k <= 512; k <<= 1) {
#pragma unroll
        for (int j = k >> 1; j > 0; j >>= 1) {
            if (j >= 64) {
                const int jr = j >> 6;
#pragma unroll
                for (int r = 0; r < 8; ++r) {
                    if (r & jr)
                        continue;
                    const bool desc = ((r * 64 + lane) & k) == 0;   // the pair's run goes downwards
                    const u64 a = v[r], b = v[r | jr];
                    const bool sw = desc ? a < b : a > b;
                    v[r] = sw ? b : a;
                    v[r | jr] = sw ? a : b;
                }
            } else {
#pragma unroll
                for (int r = 0; r < 8; ++r) {
                    u64 mx, mn;
                    pair_minmax(v[r], j, mx, mn);
                    const bool desc = ((r * 64 + lane) & k) == 0;
                    const bool lower = (lane & j) == 0;
                    const bool keep_max = lower == desc;   // the lower slot of a downward run keeps the larger
                    v[r] = keep_max ? mx : mn;
                }
            }
        }
    }
}

// One wave per 512 logits: their max, the sum of exp(l - max) (fixed order), and the kout best
// keys (the first kout of the sorted 512).
__global__ __launch_bounds__(64) void alt_partial_kernel(const float *__restrict__ logits, int vocab, int kout,
                                                         u64 *__restrict__ pkeys, float *__restrict__ pm,
                                                         float *__restrict__ ps)
{
    const int b = blockIdx.x;
    const int lane = threadIdx.x;
    float l[8];
    u64 v[8];
    float mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < 8; ++r) {
        const int i = b * ALT_BLOCK + r * 64 + lane;
        const bool in = i < vocab;
        l[r] = in ? logits[i] : -INFINITY;
        // -0 keys as +0 so that equal logits tie on the index; key 0 ranks below every logit
        v[r] = in ? argmax_key(l[r] == 0.0f ? 0.0f : l[r], (uint32_t)i) : 0ull;
        mx = fmaxf(mx, l[r]);
    }
    mx = wave_max(mx);
    float sum = 0.0f;
    if (mx != -INFINITY) {
#pragma unroll
        for (int r = 0; r < 8; ++r)
            sum += expf(l[r] - mx);
    }
    sum = wave_sum(sum);
    wave_sort512_desc(v);
    if (lane < kout)
        pkeys[(size_t)b * kout + lane] = v[0];
    if (lane == 0) {
        pm[b] = mx;
        ps[b] = sum;
    }
}

// One workgroup: each wave folds chunks of the partial keys into its running best kout (kept in
// the first kout slots, sorted with 512 - kout new keys at a time), wave 0 merges the 16 waves'
// lists, then the sum is rescaled to the global max (fixed order) and the list written.
__global__ __launch_bounds__(ALT_T2) void alt_final_kernel(const u64 *__restrict__ pkeys, const float *__restrict__ pm,
                                                           const float *__restrict__ ps, int nblk, int kout, float d,
                                                           int max_out, int32_t *__restrict__ ids,
                                                           float *__restrict__ probs, int32_t *__restrict__ count)
{
    constexpr int WAVES = ALT_T2 / 64;
    __shared__ u64 best[WAVES * ALT_MAX_OUT];
    __shared__ float red[WAVES];
    __shared__ float gmax;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int n = nblk * kout;
    const int fresh = ALT_BLOCK - kout;   // new keys per chunk
    u64 v[8];
#pragma unroll
    for (int r = 0; r < 8; ++r)
        v[r] = 0ull;
    for (int c0 = wave * fresh; c0 < n; c0 += WAVES * fresh) {
        // slots 0 .. kout-1 keep the running best; the others take keys c0 ...
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            const int e = r * 64 + lane;
            if (e >= kout) {
                const int i = c0 + e - kout;
                v[r] = i < n ? pkeys[i] : 0ull;
            }
        }
        wave_sort512_desc(v);
    }
    if (lane < kout)
        best[wave * kout + lane] = v[0];
    __syncthreads();
    if (wave == 0) {
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            const int e = r * 64 + lane;
            v[r] = e < WAVES * kout ? best[e] : 0ull;
        }
        wave_sort512_desc(v);   // the final list is v[0] of lanes 0 .. max_out-1
        if (lane == 0)
            gmax = key_logit(v[0]);
    }
    __syncthreads();
    const float M = gmax;   // the greedy token's logit, the global max
    float z = 0.0f;
    for (int b = threadIdx.x; b < nblk; b += ALT_T2)
        z += pm[b] == -INFINITY ? 0.0f : ps[b] * expf(pm[b] - M);
    z = wave_sum(z);
    if (lane == 0)
        red[wave] = z;
    __syncthreads();
    if (wave == 0) {
        float zt = 0.0f;
        for (int w = 0; w < WAVES; ++w)
            zt += red[w];
        const float tau = M + d;
        const u64 key = lane < max_out ? v[0] : 0ull;
        const float lj = key_logit(key);
        const bool take = lane < max_out && key != 0ull && lj >= tau;
        // the keys are sorted and the test is monotone in the logit: the taken ones are a prefix
        const u64 mask = __ballot(take);
        if (take) {
            ids[lane] = (int32_t)argmax_key_index(key);
            probs[lane] = expf(lj - M) / zt;
        }
        if (lane == 0)
            *count = (int32_t)__popcll(mask);
    }
}

}  // namespace vox

using namespace vox;

extern "C" size_t vox_alt_tokens_workspace(int64_t vocab, int max_out)
{
    if (vocab <= 0 || vocab > ALT_MAX_VOCAB || max_out < 1 || max_out > ALT_MAX_OUT)
        return 0;
    const int64_t nblk = (vocab + ALT_BLOCK - 1) / ALT_BLOCK;
    return (size_t)nblk * max_out * 8 + (size_t)nblk * 8;
}

extern "C" int vox_alt_tokens(const float *logits, int64_t vocab, float cutoff, int max_out, int32_t *ids,
                              float *probs, int32_t *count, void *workspace, size_t workspace_bytes, void *stream)
{
    if (vocab <= 0 || !(cutoff >= 0.0f) || max_out < 1)
        return fail(VOX_E_INVAL, "vox_alt_tokens: need vocab > 0, cutoff >= 0 and max_out >= 1");
    if (vocab > ALT_MAX_VOCAB || max_out > ALT_MAX_OUT)
        return fail(VOX_E_UNSUPPORTED, "vox_alt_tokens: vocab up to %lld and max_out up to %d",
                    (long long)ALT_MAX_VOCAB, ALT_MAX_OUT);
    if (!logits || !ids || !probs || !count || !workspace)
        return fail(VOX_E_INVAL, "vox_alt_tokens: null pointer");
    const size_t need = vox_alt_tokens_workspace(vocab, max_out);
    if (workspace_bytes < need)
        return fail(VOX_E_WORKSPACE, "vox_alt_tokens: workspace of %zu bytes, need %zu", workspace_bytes, need);
    if (!aligned(workspace, 8))
        return fail(VOX_E_INVAL, "vox_alt_tokens: workspace must be 8-byte aligned");
    const int nblk = (int)((vocab + ALT_BLOCK - 1) / ALT_BLOCK);
    unsigned long long *pkeys = (unsigned long long *)workspace;
    float *pm = (float *)(pkeys + (size_t)nblk * max_out);
    float *ps = pm + nblk;
    // d = ln(1 - cutoff) rounded to fp32 (computed here in double; every token when cutoff >= 1)
    const float d = cutoff >= 1.0f ? -INFINITY : (float)std::log(1.0 - (double)cutoff);
    hipStream_t s = (hipStream_t)stream;
    hipLaunchKernelGGL(alt_partial_kernel, dim3((unsigned)nblk), dim3(64), 0, s, logits, (int)vocab, max_out, pkeys,
                       pm, ps);
    int st = check_launch("vox_alt_tokens partial");
    if (st)
        return st;
    hipLaunchKernelGGL(alt_final_kernel, dim3(1), dim3(ALT_T2), 0, s, pkeys, pm, ps, nblk, max_out, d, max_out, ids,
                       probs, count);
    st = check_launch("vox_alt_tokens final");
    return st ? st : ok();
}
