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
// Three kernels, all selections on keys that pack an order-preserving image of the logit above
// the inverted index (a larger key is a larger logit, then a lower index):
//  * stats: each wave takes 512 logits: their max, the sum of exp(l - max) in a fixed order, and
//    their largest key;
//  * select: each wave finds the largest key of the whole vocabulary from the per-block ones
//    (this is the greedy token t), forms the threshold and keeps its logits that pass it.  Up to
//    max_out of them are written as they are; past that, a bitonic sort held in registers (VALU
//    lane exchanges, no LDS or barriers) picks the best max_out;
//  * final: one workgroup gathers the kept keys.  When at most 512 remain, one wave sorts them
//    with the smallest power-of-two network that holds them (64 keys in the usual case, where a
//    handful of tokens pass); otherwise the waves fold all per-block lists through 512-key sorts.
//    The partial sums are rescaled to the global max (fixed order) and the list written.
// The selected list is unique (the keys are distinct), so the gathering order does not matter.
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

// Descending bitonic sort of a wave's 64 R keys (R a power of two), element r * 64 + lane in v[r],
// without barriers or LDS: pairs 64 or more apart are two registers of one lane, nearer pairs one
// register of two lanes exchanged with VALU lane operations.
template <int R>
__device__ __forceinline__ void wave_sort_desc(u64 (&v)[R])
{
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int k = 2; k <= 64 * R; k <<= 1) {
#pragma unroll
        for (int j = k >> 1; j > 0; j >>= 1) {
            if (j >= 64) {
                const int jr = j >> 6;
#pragma unroll
                for (int r = 0; r < R; ++r) {
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
                for (int r = 0; r < R; ++r) {
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

// Largest of the wave's keys, in every lane.
__device__ __forceinline__ u64 wave_max_key(u64 v)
{
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) {
        u64 mx, mn;
        pair_minmax(v, m, mx, mn);
        v = mx;
    }
    return v;
}

// Largest key of the vocabulary from the per-block largest keys, in every lane of the wave.
__device__ __forceinline__ u64 global_max_key(const u64 *__restrict__ pk, int nblk)
{
    const int lane = threadIdx.x & 63;
    u64 m = 0ull;
    for (int b = lane; b < nblk; b += 64)
        m = pk[b] > m ? pk[b] : m;
    return wave_max_key(m);
}

// One wave per 512 logits: their max, the sum of exp(l - max) (fixed order), their largest key.
__global__ __launch_bounds__(64) void alt_stats_kernel(const float *__restrict__ logits, int vocab,
                                                       float *__restrict__ pm, float *__restrict__ ps,
                                                       u64 *__restrict__ pk)
{
    const int b = blockIdx.x;
    const int lane = threadIdx.x;
    float l[8];
    float mx = -INFINITY;
    u64 km = 0ull;
#pragma unroll
    for (int r = 0; r < 8; ++r) {
        const int i = b * ALT_BLOCK + r * 64 + lane;
        const bool in = i < vocab;
        l[r] = in ? logits[i] : -INFINITY;
        // -0 keys as +0 so that equal logits tie on the index; key 0 ranks below every logit
        const u64 key = in ? argmax_key(l[r] == 0.0f ? 0.0f : l[r], (uint32_t)i) : 0ull;
        km = key > km ? key : km;
        mx = fmaxf(mx, l[r]);
    }
    mx = wave_max(mx);
    km = wave_max_key(km);
    float sum = 0.0f;
    if (mx != -INFINITY) {
#pragma unroll
        for (int r = 0; r < 8; ++r)
            sum += expf(l[r] - mx);
    }
    sum = wave_sum(sum);
    if (lane == 0) {
        pm[b] = mx;
        ps[b] = sum;
        pk[b] = km;
    }
}

// One wave per 512 logits: the keys of those at or above the threshold M + d (M the largest logit
// of the vocabulary), at most kout of them (the best kout by a sort when more pass), into the
// block's kout slots, the rest of the slots 0; their number into pc[b].
__global__ __launch_bounds__(64) void alt_select_kernel(const float *__restrict__ logits, int vocab, int nblk,
                                                        int kout, float d, const u64 *__restrict__ pk,
                                                        u64 *__restrict__ pkeys, int32_t *__restrict__ pc)
{
    const int b = blockIdx.x;
    const int lane = threadIdx.x;
    float l[8];
#pragma unroll
    for (int r = 0; r < 8; ++r) {
        const int i = b * ALT_BLOCK + r * 64 + lane;
        l[r] = i < vocab ? logits[i] : -INFINITY;
    }
    const float tau = key_logit(global_max_key(pk, nblk)) + d;
    u64 v[8];
    bool pass[8];
    int c = 0;
#pragma unroll
    for (int r = 0; r < 8; ++r) {
        const int i = b * ALT_BLOCK + r * 64 + lane;
        pass[r] = i < vocab && l[r] >= tau;
        v[r] = pass[r] ? argmax_key(l[r] == 0.0f ? 0.0f : l[r], (uint32_t)i) : 0ull;
        c += __popcll(__ballot(pass[r]));
    }
    u64 *out = pkeys + (size_t)b * kout;
    if (c <= kout) {
        // in element order: a lane's slot is the count of passing elements before it
        int base = 0;
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            const u64 m = __ballot(pass[r]);
            const int before = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0));
            if (pass[r])
                out[base + before] = v[r];
            base += __popcll(m);
        }
        if (lane >= c && lane < kout)
            out[lane] = 0ull;
    } else {
        wave_sort_desc<8>(v);
        if (lane < kout)
            out[lane] = v[0];
        c = kout;
    }
    if (lane == 0)
        pc[b] = c;
}

// Sort of the first T <= 64 R keys of cand (the rest as key 0) by one wave; lane j of the result
// holds the j-th largest.
template <int R>
__device__ __forceinline__ u64 sort_gathered(const u64 *cand, int T)
{
    const int lane = threadIdx.x & 63;
    u64 v[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int e = r * 64 + lane;
        v[r] = e < T ? cand[e] : 0ull;
    }
    wave_sort_desc<R>(v);
    return v[0];
}

// One workgroup; thread b < nblk owns block b.  Every per-block value it needs (kept count, first
// kept key, largest key, max, sum) is loaded at the start, so the kernel waits for one memory
// round trip (two when a block keeps more than one key).  Each thread appends its block's kept keys
// to cand (the order does not matter).  At most 512 in all: wave 0 sorts them.  More: each wave
// folds chunks of all the blocks' slots into its running best kout (kept in the first kout slots,
// sorted with 512 - kout new keys at a time) and wave 0 merges the 16 waves' lists.  Then the sum
// is rescaled to the global max (fixed order) and the list written.
static_assert(ALT_MAX_VOCAB / ALT_BLOCK <= ALT_T2, "one final-pass thread per block");
__global__ __launch_bounds__(ALT_T2) void alt_final_kernel(const u64 *__restrict__ pkeys, const int32_t *__restrict__ pc,
                                                           const u64 *__restrict__ pk, const float *__restrict__ pm,
                                                           const float *__restrict__ ps, int nblk, int kout, float d,
                                                           int32_t *__restrict__ ids, float *__restrict__ probs,
                                                           int32_t *__restrict__ count)
{
    constexpr int WAVES = ALT_T2 / 64;
    static_assert(WAVES * ALT_MAX_OUT <= ALT_BLOCK, "the waves' lists share the gathering buffer");
    __shared__ u64 cand[ALT_BLOCK];
    __shared__ u64 wmax[WAVES];
    __shared__ float red[WAVES];
    __shared__ int total;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const bool own = tid < nblk;
    const int c = own ? pc[tid] : 0;
    const u64 k0 = own ? pkeys[(size_t)tid * kout] : 0ull;   // slot 0: the first kept key, or 0
    const u64 kb = own ? pk[tid] : 0ull;
    const float mb = own ? pm[tid] : -INFINITY;
    const float sb = own ? ps[tid] : 0.0f;
    if (tid == 0)
        total = 0;
    const u64 wk = wave_max_key(kb);
    if (lane == 0)
        wmax[wave] = wk;
    __syncthreads();
    if (c > 0) {
        const int at = atomicAdd(&total, c);
        if (at < ALT_BLOCK)
            cand[at] = k0;
        for (int j = 1; j < c && at + j < ALT_BLOCK; ++j)
            cand[at + j] = pkeys[(size_t)tid * kout + j];
    }
    u64 gk = wmax[0];
#pragma unroll
    for (int w = 1; w < WAVES; ++w)
        gk = wmax[w] > gk ? wmax[w] : gk;
    const float M = key_logit(gk);   // the greedy token's logit, the global max
    // this block's sum rescaled to M; the 16 waves' sums are added in order below
    const float z = wave_sum(mb == -INFINITY ? 0.0f : sb * expf(mb - M));
    if (lane == 0)
        red[wave] = z;
    __syncthreads();
    const int T = total;
    u64 top = 0ull;   // in wave 0: lane j holds the j-th best kept key
    if (T <= ALT_BLOCK) {
        if (wave == 0)
            top = T <= 64 ? sort_gathered<1>(cand, T)
                : T <= 128 ? sort_gathered<2>(cand, T)
                : T <= 256 ? sort_gathered<4>(cand, T)
                           : sort_gathered<8>(cand, T);
    } else {
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
            wave_sort_desc<8>(v);
        }
        if (lane < kout)
            cand[wave * kout + lane] = v[0];
        __syncthreads();
        if (wave == 0)
            top = sort_gathered<8>(cand, WAVES * kout);
    }
    if (wave == 0) {
        float zt = 0.0f;
        for (int w = 0; w < WAVES; ++w)
            zt += red[w];
        const float tau = M + d;
        const u64 key = lane < kout ? top : 0ull;
        const float lj = key_logit(key);
        const bool take = lane < kout && key != 0ull && lj >= tau;
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
    // kept keys, largest keys, maxima, sums, kept counts
    return (size_t)nblk * max_out * 8 + (size_t)nblk * (8 + 4 + 4 + 4);
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
    u64 *pkeys = (u64 *)workspace;
    u64 *pk = pkeys + (size_t)nblk * max_out;
    float *pm = (float *)(pk + nblk);
    float *ps = pm + nblk;
    int32_t *pc = (int32_t *)(ps + nblk);
    // d = ln(1 - cutoff) rounded to fp32 (computed here in double; every token when cutoff >= 1)
    const float d = cutoff >= 1.0f ? -INFINITY : (float)std::log(1.0 - (double)cutoff);
    hipStream_t s = (hipStream_t)stream;
    hipLaunchKernelGGL(alt_stats_kernel, dim3((unsigned)nblk), dim3(64), 0, s, logits, (int)vocab, pm, ps, pk);
    int st = check_launch("vox_alt_tokens stats");
    if (st)
        return st;
    hipLaunchKernelGGL(alt_select_kernel, dim3((unsigned)nblk), dim3(64), 0, s, logits, (int)vocab, nblk, max_out, d,
                       pk, pkeys, pc);
    st = check_launch("vox_alt_tokens select");
    if (st)
        return st;
    hipLaunchKernelGGL(alt_final_kernel, dim3(1), dim3(ALT_T2), 0, s, pkeys, pc, pk, pm, ps, nblk, max_out, d, ids,
                       probs, count);
    st = check_launch("vox_alt_tokens final");
    return st ? st : ok();
}
