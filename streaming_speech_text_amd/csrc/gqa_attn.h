// gqa_attn.h - grouped-query decode attention of one token over a KV ring (split-K).
//
// Pages: the decoder uses GQA with 32 query heads over 8 KV heads (voxtral.c page "Mistral
// Voxtral Realtime 4B 음성 인식 모델의 순수 C 기반 CPU 전용 추론 구현", GeekNews 26608, section
// 모델 아키텍처; Rust port page, GeekNews 26595, section 아키텍처) and keeps a rolling KV cache
// over an 8192-position sliding window (GeekNews 26608, section 주요 기능).
//
// For query head h of group g = h / GROUP:  s_t = scale * <q_h, K[g][t]>,
// p = softmax(s) over the live slots, out_h = sum_t p_t V[g][t].
//
// MI355X mapping: eight KV heads cannot fill 256 compute units, so a long live window is
// split into S chunks of at least 128 positions (grid = S x n_kv_heads).  A workgroup of 8
// waves streams its chunk of K and V for one KV head once and serves all GROUP query heads
// of that head from the same loads.  Inside the chunk it walks 128-position sub-chunks with
// an online softmax (running max and sum).  With one chunk the workgroup writes the output
// directly; otherwise it writes a partial (max, sum, unnormalised output) and a second kernel
// merges the partials in a fixed order.  A window of up to eight chunks is instead run with
// GROUP = 1 and one workgroup per (query head, chunk) (kv_shift maps it to its KV head): the same
// K and V are read once per query head, mostly from the cache, and the arithmetic spreads over
// GROUP times as many compute units.
#pragma once

#include <type_traits>

#include "vox_common.h"

namespace vox {

constexpr int ATTN_HD = 128;          // head size handled by the kernels
constexpr int ATTN_WAVES = 8;         // waves per workgroup
constexpr int ATTN_THREADS = 64 * ATTN_WAVES;
constexpr int ATTN_SUB = 128;         // positions per online-softmax sub-chunk
constexpr int ATTN_MIN_CHUNK = 128;   // do not split below this many positions
constexpr int ATTN_PART = 132;        // floats per partial: m, l, 2 pad, o[128]
constexpr int ATTN_MAX_SPLITS = 32;   // most chunks of one window (the merge is sized for it)

__host__ __device__ inline int ceil_div_i(int a, int b) { return (a + b - 1) / b; }

// Split plan for n_valid live slots with at most `s_max` chunks.  Every chunk is non-empty.
struct AttnPlan {
    int splits, chunk;
};

__host__ __device__ inline AttnPlan attn_plan(int n_valid, int s_max)
{
    int s = ceil_div_i(n_valid, ATTN_MIN_CHUNK);
    if (s > s_max)
        s = s_max;
    if (s < 1)
        s = 1;
    const int chunk = ceil_div_i(n_valid, s);
    return AttnPlan{ceil_div_i(n_valid, chunk), chunk};
}

// Most chunks a ring of n_slots may be split into.
__host__ __device__ inline int attn_split_cap(int n_slots)
{
    // ATTN_MAX_SPLITS = 32 chunks at most (a 8192-slot ring splits into 256-position chunks):
    // measured on MI355X, 64 chunks of 128 were 4 % slower at 8192 positions, 16 chunks 20 %
    int c = ceil_div_i(n_slots, ATTN_MIN_CHUNK);
    return c < 1 ? 1 : (c > ATTN_MAX_SPLITS ? ATTN_MAX_SPLITS : c);
}

struct AttnArgs {
    const float *q;          // [n_q][128]
    const float *kc, *vc;    // [n_kv][n_slots][128]
    float *out;              // [n_q][128]
    float *part;             // [n_kv][s_cap][GROUP][ATTN_PART]
    const int64_t *pos;      // when set: n_valid = min(*pos + 1, n_slots)
    int n_slots, n_valid;
    int s_cap;               // split cap (partials stride); the grid has >= plan.splits columns
    float scale;
    int kv_shift;            // with GROUP = 1 per workgroup: KV head = blockIdx.y >> kv_shift
};

// Merges the nsplit partials (m_s, l_s, o_s) of query head h of KV head g in a fixed order:
//   M = max_s m_s,  w_s = e^(m_s - M),  out = (sum_s w_s o_s) / (sum_s w_s l_s).
// One workgroup of ATTN_MERGE_THREADS per query head.  Every load is issued before the first
// use (the partials were written by another kernel, so each load is a full memory round trip;
// issuing them all at once keeps the merge at about one round trip).  Thread (j, d) sums the
// splits s = j, j + 4, ... of output dim d; the four part sums and the weight sums are added
// in a fixed order, so the result does not depend on timing.
constexpr int ATTN_MERGE_THREADS = 512;
constexpr int ATTN_MERGE_J = ATTN_MERGE_THREADS / ATTN_HD;          // 4 split phases
constexpr int ATTN_MERGE_PER = ATTN_MAX_SPLITS / ATTN_MERGE_J;      // 8 splits per thread
struct AttnMergeLds {
    float w[ATTN_MAX_SPLITS];                 // e^(m_s - M)
    float wred[ATTN_MERGE_THREADS / 64][2];   // per-wave max, then per-wave sum of w_s l_s
    float osum[ATTN_MERGE_J][ATTN_HD];
};
template <int GROUP>
__device__ __forceinline__ void attn_merge(const AttnArgs &a, int g, int h, int nsplit, AttnMergeLds &L)
{
    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const size_t sstride = (size_t)GROUP * ATTN_PART;
    const float *p0 = a.part + ((size_t)g * a.s_cap * GROUP + h) * ATTN_PART;
    // (m_s, l_s) for s = tid, then o_s[d] for this thread's splits; indices are clamped so that
    // every load is unconditional, and out-of-range splits get weight 0 below
    const int sm = tid < nsplit ? tid : 0;
    const float m_s = p0[(size_t)sm * sstride];
    const float l_s = p0[(size_t)sm * sstride + 1];
    const int j = tid / ATTN_HD, d = tid % ATTN_HD;
    float ov[ATTN_MERGE_PER];
#pragma unroll
    for (int i = 0; i < ATTN_MERGE_PER; ++i) {
        const int sp = j + ATTN_MERGE_J * i;
        ov[i] = p0[(size_t)(sp < nsplit ? sp : 0) * sstride + 4 + d];
    }
    // M over the splits (max is exact in any order)
    const float mv = tid < nsplit ? m_s : -INFINITY;
    const float wm = wave_max(mv);
    if ((tid & 63) == 0)
        L.wred[wave][0] = wm;
    __syncthreads();
    float M = L.wred[0][0];
#pragma unroll
    for (int w = 1; w < ATTN_MERGE_THREADS / 64; ++w)
        M = fmaxf(M, L.wred[w][0]);
    const float w_s = tid < nsplit ? __expf(m_s - M) : 0.0f;
    if (tid < ATTN_MAX_SPLITS)
        L.w[tid] = w_s;
    const float ws = wave_sum(w_s * l_s);
    if ((tid & 63) == 0)
        L.wred[wave][1] = ws;
    __syncthreads();
    float o = 0.0f;
#pragma unroll
    for (int i = 0; i < ATTN_MERGE_PER; ++i)
        o = fmaf(L.w[j + ATTN_MERGE_J * i], ov[i], o);
    L.osum[j][d] = o;
    __syncthreads();
    if (tid < ATTN_HD) {
        float tot = 0.0f;
#pragma unroll
        for (int w = 0; w < (ATTN_MAX_SPLITS + 63) / 64; ++w)   // the waves that hold splits
            tot += L.wred[w][1];
        float os = L.osum[0][tid];
#pragma unroll
        for (int jj = 1; jj < ATTN_MERGE_J; ++jj)
            os += L.osum[jj][tid];
        a.out[((size_t)g * GROUP + h) * ATTN_HD + tid] = os / tot;
    }
}

typedef float kvf2 __attribute__((ext_vector_type(2)));
typedef float kvf4 __attribute__((ext_vector_type(4)));
// K / V loads; NT: non-temporal (the row is read once per call)
template <bool NT>
__device__ __forceinline__ float2 ld_kv2(const float *p)
{
    if constexpr (NT) {
        const kvf2 v = __builtin_nontemporal_load(reinterpret_cast<const kvf2 *>(p));
        return make_float2(v.x, v.y);
    } else {
        return *reinterpret_cast<const float2 *>(p);
    }
}
template <bool NT>
__device__ __forceinline__ float4 ld_kv4(const float *p)
{
    if constexpr (NT) {
        const kvf4 v = __builtin_nontemporal_load(reinterpret_cast<const kvf4 *>(p));
        return make_float4(v.x, v.y, v.z, v.w);
    } else {
        return *reinterpret_cast<const float4 *>(p);
    }
}

// LATE_V: issue the V loads after the scores instead of with the K loads, so the V latency
// overlaps the scores and the softmax; used when the window is split.  With GROUP = 1, K and V
// never hold registers at the same time (two workgroups fit a compute unit).  With GROUP > 1
// each K and V row is read by one workgroup only, and the loads are non-temporal (measured on
// MI355X: the decoder at a full 8192-position window 1.220 -> 1.173 ms/token; with one workgroup
// per query head, where four workgroups read each row, they made the short-window step 2.8 %
// slower).
template <int GROUP, bool LATE_V>
__device__ __forceinline__ void attn_chunk(const AttnArgs &a)
{
    __shared__ float sc[GROUP][ATTN_SUB];                 // scores, then weights, of a sub-chunk
    __shared__ float alpha_s[GROUP];                      // rescale of the running sums
    __shared__ float ored[ATTN_WAVES][GROUP][ATTN_HD];    // per-wave partial outputs
    __shared__ float ml[GROUP][2];

    // With one workgroup per (query head, chunk), the query heads of a KV head read the same rows:
    // workgroups go to the eight XCDs round-robin in dispatch order (x fastest), so the mapping
    // below gives each XCD whole groups of them, and that XCD's L2 fetches the rows from HBM once
    // instead of once per query head (measured on MI355X: the decoder step 0.817 -> 0.808 ms/token
    // at 39-102 positions, one chunk; a 1024-position window in 8 chunks 7.6 -> 7.5 us).  Dispatch slot L = x + w y on XCD L % 8 takes group
    // (L % 8) (w n_kv / 8) + (L / 8) / G (KV head = group / w, chunk = group % w) and query head
    // L / 8 % G of it: a bijection whenever w n_kv is a multiple of 8.
    int g = blockIdx.y, s = blockIdx.x;
    if constexpr (GROUP == 1) {
        const int w = gridDim.x, sh = a.kv_shift, nkv = gridDim.y >> sh;
        if (sh > 0 && (w * nkv) % 8 == 0) {
            const int L = blockIdx.x + w * blockIdx.y;
            const int grp = (L & 7) * ((w * nkv) >> 3) + ((L >> 3) >> sh);
            const int j = (L >> 3) & ((1 << sh) - 1);
            if ((w & (w - 1)) == 0) {   // the decoder's widths: shifts only
                const int lw = __builtin_ctz(w);
                g = ((grp >> lw) << sh) + j;
                s = grp & (w - 1);
            } else {
                g = (grp / w << sh) + j;
                s = grp % w;
            }
        }
    }
    int nv = a.n_valid;
    if (a.pos) {
        const int64_t p = *a.pos + 1;
        nv = p < a.n_slots ? (int)p : a.n_slots;
    }
    const AttnPlan plan = attn_plan(nv, a.s_cap);   // the host derives the same plan
    if (s >= plan.splits)
        return;
    const int t0 = s * plan.chunk;
    const int t1 = min(nv, t0 + plan.chunk);

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int pslot = lane >> 4;     // score phase: 4 positions per wave, 16 lanes each
    const int seg = lane & 15;       // 8 dims per lane

    const int kvh = g >> a.kv_shift;   // one workgroup per query head when GROUP = 1 serves a group
    const float *kbase = a.kc + (size_t)kvh * a.n_slots * ATTN_HD;
    const float *vbase = a.vc + (size_t)kvh * a.n_slots * ATTN_HD;

    float m_run[GROUP], l_run[GROUP];
    float2 acc[GROUP];
#pragma unroll
    for (int h = 0; h < GROUP; ++h) {
        m_run[h] = -INFINITY;
        l_run[h] = 0.0f;
        acc[h] = make_float2(0.0f, 0.0f);
    }
    float qv[GROUP][8];
    bool q_loaded = false;

    // PF: with GROUP > 1 and late V loads, the next sub-chunk's K loads are issued right after
    // this sub-chunk's V loads (the K registers are free once the scores are taken), so a chunk of
    // two sub-chunks waits on three rounds of loads instead of four.  Each sub-chunk body is
    // compiled for a full or a partial sub-chunk and with or without that prefetch, so every body
    // is straight-line code and the waits before each use count exactly the loads issued after it
    // (measured on MI355X: the decoder step 0.830 -> 0.821 ms/token at 39-102 positions, where each
    // window is one partial sub-chunk; unchanged, 1.175, at a full window)
    constexpr bool PF = LATE_V && GROUP > 1 && GROUP <= 4;
    float4 kr[4][2];
    auto load_k = [&](int b0, auto full_c) {
        if constexpr (decltype(full_c)::value) {
#pragma unroll
            for (int it = 0; it < 4; ++it) {
                const int t = b0 + it * 32 + wave * 4 + pslot;
                const float *k4 = kbase + (size_t)t * ATTN_HD + 8 * seg;
                kr[it][0] = ld_kv4<(GROUP > 1)>(k4);
                kr[it][1] = ld_kv4<(GROUP > 1)>(k4 + 4);
            }
        } else {
#pragma unroll
            for (int it = 0; it < 4; ++it) {
                const int t = b0 + it * 32 + wave * 4 + pslot;
                if (t < t1) {
                    const float *k4 = kbase + (size_t)t * ATTN_HD + 8 * seg;
                    kr[it][0] = ld_kv4<(GROUP > 1)>(k4);
                    kr[it][1] = ld_kv4<(GROUP > 1)>(k4 + 4);
                } else {
                    kr[it][0] = make_float4(0.f, 0.f, 0.f, 0.f);
                    kr[it][1] = kr[it][0];
                }
            }
        }
    };
    bool k_ready = false;

    auto iter = [&](int base, auto full_c, auto pfn_c) {
        constexpr bool FULLC = decltype(full_c)::value;
        constexpr bool PFN = decltype(pfn_c)::value;
        // issue the K (unless prefetched) and V loads of the sub-chunk first (the first time, the
        // query loads follow them so the two latencies overlap).  A full sub-chunk loads
        // unconditionally; a partial one skips the positions past the chunk end, whose scores are
        // -inf below, so their weights are exactly 0.
        float2 vr[16];
        constexpr bool full = FULLC;
        auto load_v = [&]() {
            if constexpr (full) {
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int t = base + wave + ATTN_WAVES * i;
                    vr[i] = ld_kv2<(GROUP > 1)>(vbase + (size_t)t * ATTN_HD + 2 * lane);
                }
            } else {
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int t = base + wave + ATTN_WAVES * i;
                    vr[i] = t < t1 ? ld_kv2<(GROUP > 1)>(vbase + (size_t)t * ATTN_HD + 2 * lane)
                                   : make_float2(0.0f, 0.0f);
                }
            }
        };
        if (!PF || !k_ready)
            load_k(base, full_c);
        if constexpr (!LATE_V)
            load_v();
        if (!q_loaded) {
#pragma unroll
            for (int h = 0; h < GROUP; ++h) {
                const float4 *q4 =
                    reinterpret_cast<const float4 *>(a.q + ((size_t)g * GROUP + h) * ATTN_HD + 8 * seg);
                const float4 u = q4[0], v = q4[1];
                qv[h][0] = u.x; qv[h][1] = u.y; qv[h][2] = u.z; qv[h][3] = u.w;
                qv[h][4] = v.x; qv[h][5] = v.y; qv[h][6] = v.z; qv[h][7] = v.w;
            }
            q_loaded = true;
        }
        // scores
#pragma unroll
        for (int it = 0; it < 4; ++it) {
            const int p = it * 32 + wave * 4 + pslot;
            const float kk[8] = {kr[it][0].x, kr[it][0].y, kr[it][0].z, kr[it][0].w,
                                 kr[it][1].x, kr[it][1].y, kr[it][1].z, kr[it][1].w};
#pragma unroll
            for (int h = 0; h < GROUP; ++h) {
                float d = 0.0f;
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    d = fmaf(qv[h][i], kk[i], d);
                d = row16_sum(d);   // the 16 lanes of a row hold one position
                if (seg == 0)
                    sc[h][p] = (base + p < t1) ? d * a.scale : -INFINITY;
            }
        }
        if constexpr (LATE_V)
            load_v();
        if constexpr (PFN) {
            load_k(base + ATTN_SUB, std::true_type());   // the next sub-chunk, a full one
            k_ready = true;
        } else {
            k_ready = false;
        }
        __syncthreads();
        // online softmax update: wave (h % 8) handles query head h, two positions per lane
#pragma unroll
        for (int h = 0; h < GROUP; ++h) {
            if ((h % ATTN_WAVES) != wave)
                continue;
            const float v0 = sc[h][lane];
            const float v1 = sc[h][lane + 64];
            const float mx = wave_max(fmaxf(v0, v1));
            const float m_new = fmaxf(m_run[h], mx);
            const float e0 = (v0 == -INFINITY) ? 0.0f : __expf(v0 - m_new);
            const float e1 = (v1 == -INFINITY) ? 0.0f : __expf(v1 - m_new);
            const float sum = wave_sum(e0 + e1);
            sc[h][lane] = e0;
            sc[h][lane + 64] = e1;
            const float al = (m_run[h] == -INFINITY) ? 0.0f : __expf(m_run[h] - m_new);
            if (lane == 0)
                alpha_s[h] = al;
            l_run[h] = fmaf(l_run[h], al, sum);
            m_run[h] = m_new;
        }
        __syncthreads();
        // weighted values: wave w takes positions w, w+8, ...; lane owns dims 2*lane, 2*lane+1
#pragma unroll
        for (int h = 0; h < GROUP; ++h) {
            const float al = alpha_s[h];
            acc[h].x *= al;
            acc[h].y *= al;
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int p = wave + ATTN_WAVES * i;
#pragma unroll
            for (int h = 0; h < GROUP; ++h) {
                const float w = sc[h][p];
                acc[h].x = fmaf(w, vr[i].x, acc[h].x);
                acc[h].y = fmaf(w, vr[i].y, acc[h].y);
            }
        }
        __syncthreads();
    };
    typedef std::integral_constant<bool, true> T_;
    typedef std::integral_constant<bool, false> F_;
    for (int base = t0; base < t1; base += ATTN_SUB) {
        if (base + ATTN_SUB <= t1) {
            if (PF && base + 2 * ATTN_SUB <= t1)
                iter(base, T_(), std::integral_constant<bool, PF>());
            else
                iter(base, T_(), F_());
        } else {
            iter(base, F_(), F_());
        }
    }

    // combine the waves' partial outputs
#pragma unroll
    for (int h = 0; h < GROUP; ++h) {
        ored[wave][h][2 * lane] = acc[h].x;
        ored[wave][h][2 * lane + 1] = acc[h].y;
    }
#pragma unroll
    for (int h = 0; h < GROUP; ++h) {
        if ((h % ATTN_WAVES) == wave && lane == 0) {
            ml[h][0] = m_run[h];
            ml[h][1] = l_run[h];
        }
    }
    __syncthreads();

    auto wave_total = [&](int h, int d) {
        float o = ored[0][h][d];
#pragma unroll
        for (int w = 1; w < ATTN_WAVES; ++w)
            o += ored[w][h][d];
        return o;
    };
    if (plan.splits == 1) {
        for (int i = tid; i < GROUP * ATTN_HD; i += ATTN_THREADS) {
            const int h = i / ATTN_HD, d = i % ATTN_HD;
            a.out[((size_t)g * GROUP + h) * ATTN_HD + d] = wave_total(h, d) / ml[h][1];
        }
        return;
    }

    float *mypart = a.part + ((size_t)g * a.s_cap + s) * GROUP * ATTN_PART;
    for (int i = tid; i < GROUP * ATTN_HD; i += ATTN_THREADS) {
        const int h = i / ATTN_HD, d = i % ATTN_HD;
        mypart[h * ATTN_PART + 4 + d] = wave_total(h, d);
    }
    if (tid < GROUP) {
        mypart[tid * ATTN_PART + 0] = ml[tid][0];
        mypart[tid * ATTN_PART + 1] = ml[tid][1];
    }
}

}  // namespace vox
