// enc_attn.hip - self-attention of the audio encoder over one chunk of frames: causal, with a
// sliding window, on the fp32 matrix cores.
//
// Pages: the audio encoder is a causal transformer of width 1280 with 32 heads and a window of
// 750 (voxtral.c page "Mistral Voxtral Realtime 4B 음성 인식 모델의 순수 C 기반 CPU 전용 추론 구현",
// GeekNews 26608, section 모델 아키텍처), run over chunks of the audio (section 주요 기능).
//
// Operation (per head h, query i of the chunk at row n_ctx + i of K and V):
//   s_j = scale * <q_i, k_j> for j in [n_ctx + i - window + 1, n_ctx + i] (and j >= 0),
//   out_i = sum_j softmax(s)_j v_j.
//
// A workgroup of four waves takes 64 queries of one head; K and V reach LDS in blocks of 64 keys
// (one copy serves the four waves), and each wave owns 16 queries.  With 16 keys per step a wave computes
// S^T = K Q^T (16 keys x 16 queries) with v_mfma_f32_16x16x4_f32 over the head size (inputs in
// any order A and B agree on: lane group g supplies dims 16s + 4g + r in product 4s + r), so each
// lane ends up holding four keys (4g .. 4g+3) of one query (lane % 16).  That is exactly the
// layout of the B operand of O^T += V^T P^T, whose k slots are the same keys (product t takes key
// 4g + t from lane group g), so the probabilities never leave the registers.  Online softmax in
// base 2 (q pre-scaled by scale * log2 e); the row max is shared by the four lane groups of a
// query through two lane swaps, the row sums stay per lane until the end.  Per 64-key block a wave
// computes all four score blocks first, updates the running max once, and rescales the output
// only when some query's max grew.
//
// Short chunks split each wave's key range over the grid's third dimension; partial (max, sum,
// unnormalised output) go to the workspace and enc_attn_merge_kernel combines them in split order.
#include <cmath>

#include "vox_common.h"
#include "vox_host.h"

namespace vox {

typedef float f32x4e __attribute__((ext_vector_type(4)));

constexpr int EA_MAX_HD = 48;                 // head sizes up to 48 (three 16-wide blocks)

struct EncAttnArgs {
    const float *q, *k, *v;
    float *out;          // [m][width] when unsplit
    float *part;         // split: [splits][n_heads][m][hd] unnormalised outputs
    float *pm, *pl;      // split: [splits][n_heads][m] running max (base 2) and sum
    int m, n_ctx, n_heads, hd, width, window;
    int steps_per_split; // 16-key steps per split
    float qscale;        // scale * log2(e)
};

// Lane exchanges across rows of 16 lanes (v_permlane16_swap / v_permlane32_swap): each returns the
// pair {own value, value of lane ^ 16 (or ^ 32)} in some order, so max and sum need no select.
__device__ __forceinline__ float max_xor16(float v)
{
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_xor32(float v)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor16(float v)
{
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float sum_xor32(float v)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

constexpr int EA_WAVES = 4;    // waves per workgroup, 16 queries each
constexpr int EA_KB = 64;      // keys per LDS block

// Head size HD (a multiple of 4 up to 48) at compile time.  A workgroup of four waves takes 64
// consecutive queries of one head; per block of 64 keys the workgroup copies K and V rows to LDS
// (rows padded to HD + 4 floats), and each wave whose queries' windows meet the block runs its four
// 16-key steps with operands read from LDS.  The next block's rows wait in registers while the
// current block is computed.  Score products: the full 16-dim blocks take dims 16s + 4g + r in
// product (s, r) (a float4 per lane); the last block's HD % 16 dims take dims 16s + 4r + g in
// product r (one float per lane and product), so no product runs on padding.
template <int HD>
__global__ __launch_bounds__(64 * EA_WAVES) void enc_attn_kernel(EncAttnArgs a)
{
    constexpr int FULL = HD / 16;             // full 16-dim blocks
    constexpr int TAILP = (HD % 16) / 4;      // products of the last, partial block
    constexpr int NDB = (HD + 15) / 16;       // 16-dim output blocks
    constexpr int LD = HD + 4;                // LDS row stride (floats)
    constexpr int ROW4 = HD / 4;              // float4 per row
    constexpr int NCOPY = (2 * EA_KB * ROW4 + 64 * EA_WAVES - 1) / (64 * EA_WAVES);   // float4 per thread
    __shared__ __attribute__((aligned(16))) float lk[EA_KB * LD];
    __shared__ __attribute__((aligned(16))) float lv[EA_KB * LD];

    const int h = blockIdx.x;           // head in the fast grid dimension: a head's waves share an XCD
    const int z = blockIdx.z;           // key split
    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int qi = lane & 15, g = lane >> 4;
    const int width = a.width;
    const int q0 = blockIdx.y * (16 * EA_WAVES);     // first query of the workgroup
    const int i0 = q0 + 16 * wave;                   // first query of the wave
    const bool live = i0 < a.m;                      // wave has queries (uniform)
    const int iq = min(i0 + qi, a.m - 1);            // this lane's query (clamped; stores are masked)
    const float *qrow = a.q + (uint32_t)(iq * width + h * HD);

    // B operand of S^T
    f32x4e qv[FULL > 0 ? FULL : 1];
    float qt[TAILP > 0 ? TAILP : 1];
#pragma unroll
    for (int s = 0; s < FULL; ++s)
        qv[s] = *reinterpret_cast<const f32x4e *>(qrow + 16 * s + 4 * g) * a.qscale;
#pragma unroll
    for (int r = 0; r < TAILP; ++r)
        qt[r] = qrow[16 * FULL + 4 * r + g] * a.qscale;

    // key blocks of the workgroup (union over its queries), this split's share of them
    const int T = a.n_ctx + a.m;
    const int jlo = max(0, a.n_ctx + q0 - a.window + 1);
    const int jhi = a.n_ctx + min(q0 + 16 * EA_WAVES - 1, a.m - 1);   // inclusive
    const int nblk = (jhi - jlo + EA_KB) / EA_KB;
    const int b0 = z * a.steps_per_split;
    const int b1 = min(nblk, b0 + a.steps_per_split);
    // the wave's key range and this lane's own query bounds
    const int w_lo = max(0, a.n_ctx + i0 - a.window + 1);
    const int w_hi = a.n_ctx + min(i0 + 15, a.m - 1);
    const int my_hi = a.n_ctx + i0 + qi, my_lo = my_hi - a.window + 1;
    // V operand columns: dims 16 db + qi (past the head size: column 0, weight 0)
    bool vok[NDB];
    int vcol[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
        vok[db] = 16 * db + qi < HD;
        vcol[db] = vok[db] ? 16 * db + qi : 0;
    }

    f32x4e o[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db)
        o[db] = (f32x4e)0.0f;
    float mrun = -INFINITY, lpart = 0.0f;

    // cooperative copy of one block: element e < 2 * 64 * ROW4 is (K or V, row, float4)
    f32x4e stage[NCOPY];
    auto fetch = [&](int b) {
        const int kb = jlo + EA_KB * b;
#pragma unroll
        for (int c = 0; c < NCOPY; ++c) {
            const int e = min(tid + 64 * EA_WAVES * c, 2 * EA_KB * ROW4 - 1);
            const int which = e / (EA_KB * ROW4), rem = e % (EA_KB * ROW4);
            const int row = rem / ROW4, c4 = rem % ROW4;
            const float *src = (which ? a.v : a.k) + (uint32_t)(min(kb + row, T - 1) * width + h * HD + 4 * c4);
            stage[c] = *reinterpret_cast<const f32x4e *>(src);
        }
    };
    auto store = [&]() {
#pragma unroll
        for (int c = 0; c < NCOPY; ++c) {
            const int e = tid + 64 * EA_WAVES * c;
            if (e < 2 * EA_KB * ROW4) {
                const int which = e / (EA_KB * ROW4), rem = e % (EA_KB * ROW4);
                const int row = rem / ROW4, c4 = rem % ROW4;
                *reinterpret_cast<f32x4e *>((which ? lv : lk) + row * LD + 4 * c4) = stage[c];
            }
        }
    };

    if (b0 < b1)
        fetch(b0);
    for (int b = b0; b < b1; ++b) {
        __syncthreads();   // the previous block's LDS reads are done
        store();
        __syncthreads();
        if (b + 1 < b1)
            fetch(b + 1);
        const int kb0 = jlo + EA_KB * b;
        if (!live || kb0 > w_hi || kb0 + EA_KB - 1 < w_lo)
            continue;   // no key of this block is in the wave's windows (uniform)
        // scores of the whole block first (independent products the scheduler can overlap with
        // the softmax work), then one running-max update per block
        f32x4e sc[EA_KB / 16];
#pragma unroll
        for (int u = 0; u < EA_KB / 16; ++u) {
            // K operand: row 16u + qi
            const float *kr = lk + (16 * u + qi) * LD;
            sc[u] = (f32x4e)0.0f;
#pragma unroll
            for (int s = 0; s < FULL; ++s) {
                const f32x4e kc = *reinterpret_cast<const f32x4e *>(kr + 16 * s + 4 * g);
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    sc[u] = __builtin_amdgcn_mfma_f32_16x16x4f32(kc[r], qv[s][r], sc[u], 0, 0, 0);
            }
#pragma unroll
            for (int r = 0; r < TAILP; ++r)
                sc[u] = __builtin_amdgcn_mfma_f32_16x16x4f32(kr[16 * FULL + 4 * r + g], qt[r], sc[u], 0, 0, 0);
        }
        // masked scores (lane holds keys kb0 + 16u + 4g + r of query i0 + qi), block max over the
        // query's four lane groups
        float bmax = -INFINITY;
#pragma unroll
        for (int u = 0; u < EA_KB / 16; ++u) {
            const int j0 = kb0 + 16 * u + 4 * g;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                sc[u][r] = (j0 + r >= my_lo && j0 + r <= my_hi) ? sc[u][r] : -INFINITY;
                bmax = fmaxf(bmax, sc[u][r]);
            }
        }
        bmax = max_xor32(max_xor16(bmax));
        const float mnew = fmaxf(mrun, bmax);
        const float ms = mnew == -INFINITY ? 0.0f : mnew;   // nothing live yet: weights stay 0
        const float c = __builtin_amdgcn_exp2f(mrun - ms);
        const bool grew = mnew > mrun;                      // c < 1 only where the max grew
        mrun = mnew;
        float psum = 0.0f;
#pragma unroll
        for (int u = 0; u < EA_KB / 16; ++u)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                sc[u][r] = __builtin_amdgcn_exp2f(sc[u][r] - ms);
                psum += sc[u][r];
            }
        lpart = lpart * c + psum;
        if (__any(grew)) {   // rescale only when some query's max grew (c = 1 elsewhere)
#pragma unroll
            for (int db = 0; db < NDB; ++db)
                o[db] *= c;
        }
        // O^T += V^T P^T: product (u, t) takes key kb0 + 16u + 4g + t from lane group g
#pragma unroll
        for (int u = 0; u < EA_KB / 16; ++u) {
            float vc[NDB][4];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const float *vr = lv + (16 * u + 4 * g + t) * LD;
#pragma unroll
                for (int db = 0; db < NDB; ++db)
                    vc[db][t] = vok[db] ? vr[vcol[db]] : 0.0f;
            }
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int t = 0; t < 4; ++t)
                    o[db] = __builtin_amdgcn_mfma_f32_16x16x4f32(vc[db][t], sc[u][t], o[db], 0, 0, 0);
        }
    }

    // this query's sum over the four lane groups (all share mrun)
    const float l = sum_xor32(sum_xor16(lpart));
    const int i = i0 + qi;
    if (i >= a.m)
        return;
    // O^T layout: lane holds dims 16 db + 4g + r of query i0 + qi
    if (a.part == nullptr) {
        const float inv = 1.0f / l;
        float *orow = a.out + (size_t)i * width + (size_t)h * HD;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int d = 16 * db + 4 * g + r;
                if (d < HD)
                    orow[d] = o[db][r] * inv;
            }
    } else {
        const size_t row = ((size_t)z * a.n_heads + h) * a.m + i;
        float *prow = a.part + row * HD;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int d = 16 * db + 4 * g + r;
                if (d < HD)
                    prow[d] = o[db][r];
            }
        if (g == 0) {
            a.pm[row] = mrun;
            a.pl[row] = l;
        }
    }
}

// out[i][h*hd + d] = sum_z 2^(m_z - M) O_z[d] / sum_z 2^(m_z - M) l_z, splits in order z = 0, 1, ...
// One thread per output value.  With NF > 0 (at least as many as the splits) every load is issued
// before the first use (one memory round trip); NF = 0 takes two passes over the partials.
template <int NF>
__global__ __launch_bounds__(256) void enc_attn_merge_kernel(EncAttnArgs a, int splits)
{
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t total = (int64_t)a.m * a.n_heads * a.hd;
    if (t >= total)
        return;
    const int d = (int)(t % a.hd);
    const int64_t hi = t / a.hd;           // (i * n_heads + h)
    const int h = (int)(hi % a.n_heads);
    const int i = (int)(hi / a.n_heads);
    if constexpr (NF > 0) {
        float pmv[NF], plv[NF], ov[NF];
#pragma unroll
        for (int z = 0; z < NF; ++z) {
            const size_t row = ((size_t)(z < splits ? z : 0) * a.n_heads + h) * a.m + i;
            pmv[z] = a.pm[row];
            plv[z] = a.pl[row];
            ov[z] = a.part[row * a.hd + d];
        }
        float mx = -INFINITY;
#pragma unroll
        for (int z = 0; z < NF; ++z)
            if (z < splits)
                mx = fmaxf(mx, pmv[z]);
        float l = 0.0f, o = 0.0f;
#pragma unroll
        for (int z = 0; z < NF; ++z)
            if (z < splits) {
                const float w = __builtin_amdgcn_exp2f(pmv[z] - mx);   // an empty split (max -inf) weighs 0
                l += w * plv[z];
                o += w * ov[z];
            }
        a.out[(size_t)i * a.width + (size_t)h * a.hd + d] = o / l;
    } else {
        float mx = -INFINITY;
        for (int z = 0; z < splits; ++z)
            mx = fmaxf(mx, a.pm[((size_t)z * a.n_heads + h) * a.m + i]);
        float l = 0.0f, o = 0.0f;
        for (int z = 0; z < splits; ++z) {
            const size_t row = ((size_t)z * a.n_heads + h) * a.m + i;
            const float w = __builtin_amdgcn_exp2f(a.pm[row] - mx);   // an empty split (max -inf) weighs 0
            l += w * a.pl[row];
            o += w * a.part[row * a.hd + d];
        }
        a.out[(size_t)i * a.width + (size_t)h * a.hd + d] = o / l;
    }
}

struct EncAttnPlan {
    int qblocks, steps, splits, per;   // steps: 64-key blocks of the longest workgroup range
};

// Splits: enough waves for about two per SIMD, at least two 64-key blocks per split (measured on
// MI355X over the chunk sizes 16 .. 750: one block per split, or a target of one or four waves per
// SIMD, was slower somewhere and faster nowhere by more than a few percent).
static EncAttnPlan enc_attn_plan(int64_t m, int64_t n_ctx, int n_heads, int window)
{
    EncAttnPlan p;
    p.qblocks = (int)((m + 16 * EA_WAVES - 1) / (16 * EA_WAVES));
    // the longest key range of a workgroup: window - 1 earlier keys plus its 64 queries
    const int64_t span = std::min<int64_t>(n_ctx + m, (int64_t)window + 16 * EA_WAVES - 1);
    p.steps = (int)((span + EA_KB - 1) / EA_KB);
    const int64_t waves = (int64_t)p.qblocks * n_heads * EA_WAVES;
    int splits = (int)std::min<int64_t>((2048 + waves - 1) / waves, std::max(1, p.steps / 2));
    splits = std::max(splits, 1);
    p.per = (p.steps + splits - 1) / splits;
    p.splits = (p.steps + p.per - 1) / p.per;
    return p;
}

static size_t enc_attn_ws(const EncAttnPlan &p, int64_t m, int n_heads, int hd)
{
    if (p.splits <= 1)
        return 0;
    const size_t rows = (size_t)p.splits * n_heads * m;
    return (rows * hd + 2 * rows) * sizeof(float);
}

}  // namespace vox

using namespace vox;

extern "C" size_t vox_enc_attn_workspace(int64_t m, int64_t n_ctx, int n_heads, int head_dim, int window)
{
    if (m <= 0 || n_ctx < 0 || n_heads <= 0 || head_dim <= 0 || head_dim > EA_MAX_HD || head_dim % 4 || window <= 0)
        return 0;
    return enc_attn_ws(enc_attn_plan(m, n_ctx, n_heads, window), m, n_heads, head_dim);
}

extern "C" int vox_enc_attn(const float *q, const float *k, const float *v, float *out, int64_t m, int64_t n_ctx,
                            int n_heads, int head_dim, int window, float scale, void *workspace,
                            size_t workspace_bytes, void *stream)
{
    if (m < 0 || n_ctx < 0 || n_heads <= 0 || head_dim <= 0 || window <= 0)
        return fail(VOX_E_INVAL, "vox_enc_attn: need m, n_ctx >= 0 and n_heads, head_dim, window > 0");
    if (m == 0)
        return ok();
    if (head_dim > EA_MAX_HD || head_dim % 4)
        return fail(VOX_E_UNSUPPORTED, "vox_enc_attn: head_dim must be a multiple of 4 up to %d (got %d)", EA_MAX_HD,
                    head_dim);
    const int64_t width = (int64_t)n_heads * head_dim, T = n_ctx + m;
    if (m > 65535LL * 16 || n_heads > 65535 || T * width >= (1LL << 31))
        return fail(VOX_E_UNSUPPORTED, "vox_enc_attn: sizes beyond the grid or 32-bit element offsets");
    if (!q || !k || !v || !out)
        return fail(VOX_E_INVAL, "vox_enc_attn: null pointer");
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16))
        return fail(VOX_E_UNSUPPORTED, "vox_enc_attn: q, k and v must be 16-byte aligned");
    const size_t qbytes = (size_t)m * width * 4, kvbytes = (size_t)T * width * 4;
    if (overlaps(out, qbytes, q, qbytes) || overlaps(out, qbytes, k, kvbytes) || overlaps(out, qbytes, v, kvbytes))
        return fail(VOX_E_INVAL, "vox_enc_attn: out overlaps an input");
    const EncAttnPlan p = enc_attn_plan(m, n_ctx, n_heads, window);
    const size_t need = enc_attn_ws(p, m, n_heads, head_dim);
    if (need > workspace_bytes || (need && !workspace))
        return fail(VOX_E_WORKSPACE, "vox_enc_attn: workspace of %zu bytes, need %zu", workspace_bytes, need);
    if (need && (!aligned(workspace, 16) || overlaps(workspace, need, out, qbytes) ||
                 overlaps(workspace, need, q, qbytes) || overlaps(workspace, need, k, kvbytes) ||
                 overlaps(workspace, need, v, kvbytes)))
        return fail(VOX_E_INVAL, "vox_enc_attn: workspace must be 16-byte aligned and apart from the other buffers");

    EncAttnArgs a;
    a.q = q;
    a.k = k;
    a.v = v;
    a.out = out;
    const size_t rows = (size_t)p.splits * n_heads * m;
    a.part = p.splits > 1 ? (float *)workspace : nullptr;
    a.pm = p.splits > 1 ? a.part + rows * head_dim : nullptr;
    a.pl = p.splits > 1 ? a.pm + rows : nullptr;
    a.m = (int)m;
    a.n_ctx = (int)n_ctx;
    a.n_heads = n_heads;
    a.hd = head_dim;
    a.width = (int)width;
    a.window = window;
    a.steps_per_split = p.per;
    a.qscale = scale * 1.4426950408889634f;
    hipStream_t s = (hipStream_t)stream;
    const dim3 grid((unsigned)n_heads, (unsigned)p.qblocks, (unsigned)p.splits);
    switch (head_dim) {
    case 4: hipLaunchKernelGGL(enc_attn_kernel<4>, grid, dim3(64 * EA_WAVES), 0, s, a); break;
    case 8: hipLaunchKernelGGL(enc_attn_kernel<8>, grid, dim3(64 * EA_WAVES), 0, s, a); break;
    case 12: hipLaunchKernelGGL(enc_attn_kernel<12>, grid, dim3(64 * EA_WAVES), 0, s, a); break;
    case 16: hipLaunchKernelGGL(enc_attn_kernel<16>, grid, dim3(64 * EA_WAVES), 0, s, a); break;
    case 20: hipLaunchKernelGGL(enc_attn_kernel<20>, grid, dim3(64 * EA_WAVES), 0, s, a); break;
    case 24: hipLaunchKernelGGL(enc_attn_kernel<24>, grid, dim3(64 * EA_WAVES), 0, s, a); break;
    case 28: hipLaunchKernelGGL(enc_attn_kernel<28>, grid, dim3(64 * EA_WAVES), 0, s, a); break;
    case 32: hipLaunchKernelGGL(enc_attn_kernel<32>, grid, dim3(64 * EA_WAVES), 0, s, a); break;
    case 36: hipLaunchKernelGGL(enc_attn_kernel<36>, grid, dim3(64 * EA_WAVES), 0, s, a); break;
    case 40: hipLaunchKernelGGL(enc_attn_kernel<40>, grid, dim3(64 * EA_WAVES), 0, s, a); break;
    case 44: hipLaunchKernelGGL(enc_attn_kernel<44>, grid, dim3(64 * EA_WAVES), 0, s, a); break;
    default: hipLaunchKernelGGL(enc_attn_kernel<48>, grid, dim3(64 * EA_WAVES), 0, s, a); break;
    }
    int st = check_launch("vox_enc_attn");
    if (st || p.splits == 1)
        return st ? st : ok();
    const int64_t total = m * width;
    const dim3 mg((unsigned)((total + 255) / 256));
    if (p.splits <= 2)
        hipLaunchKernelGGL(enc_attn_merge_kernel<2>, mg, dim3(256), 0, s, a, p.splits);
    else if (p.splits <= 4)
        hipLaunchKernelGGL(enc_attn_merge_kernel<4>, mg, dim3(256), 0, s, a, p.splits);
    else if (p.splits <= 8)
        hipLaunchKernelGGL(enc_attn_merge_kernel<8>, mg, dim3(256), 0, s, a, p.splits);
    else
        hipLaunchKernelGGL(enc_attn_merge_kernel<0>, mg, dim3(256), 0, s, a, p.splits);
    st = check_launch("vox_enc_attn merge");
    return st ? st : ok();
}
