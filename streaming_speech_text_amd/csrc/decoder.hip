// decoder.hip - the per-token decoder step of streaming Voxtral Mini 4B Realtime.
//
// Pages: voxtral.c page ("Mistral Voxtral Realtime 4B 음성 인식 모델의 순수 C 기반 CPU 전용 추론
// 구현", GeekNews 26608): section 모델 아키텍처 - LLM decoder of 26 layers, width 3072, GQA 32 query
// heads / 8 KV heads, "Ministral-3 based" (read as a Llama-style pre-norm block with RMSNorm,
// rotary positions and a SwiGLU feed-forward); section 주요 기능 - rolling KV cache with an
// 8192-position window; section 성능 벤치마크 - the whole token is one GPU submission.  Rust port
// page ("Mistral의 Voxtral Mini 4B Realtime 모델을 Rust로 구현해 브라우저에서 실행", GeekNews 26595):
// section 아키텍처 - GGUF Q4_0 linears with dequantisation fused into the product; section 브라우저
// 실행을 위한 기술적 해결 - the embedding stays on the GPU as Q4 and one row is used per token.
//
// One step = 5 kernels per layer (6 with a split window) + 2:
//   qkv    RMSNorm prologue (layer 0: from the token's embedding row), Q/K/V Q4_0 GEMV over one
//          concatenated row space, RoPE on q and k, k and v written to ring slot pos % n_slots
//   attn   grouped attention over min(pos+1, n_slots) slots (split over the window when it is
//          long, with a merge kernel after it)
//   o      Q4_0 GEMV of the attention output, added into the residual stream
//   ffn    RMSNorm prologue, gate and up rows in the same tile, silu(gate) * up
//   down   Q4_0 GEMV, added into the residual stream
//   head   final RMSNorm, tied Q4_0 table as LM head, logits (optional) and each workgroup's
//          best (logit, index) key
//   final  one workgroup reduces the keys, writes the token, advances pos and fills the
//          (cos, sin) table of the new position for the next step's RoPE
// The sequence is captured once into a HIP graph and replayed per token.
#include <math.h>
#include <stdlib.h>

#include <new>
#include <type_traits>
#include <vector>

#include "gemv_core.h"
#include "gqa_attn.h"
#include "vox_host.h"

namespace vox {

struct DecCtl {
    int64_t pos;                  // absolute position of the next token
    float rope_cs[ATTN_HD];       // (cos, sin) of pos * theta^(-2i/128) for pair i, i < 64
};

// Rotation table of position p for the pair of thread i < 64: the angle is formed in fp64 in
// units of pi (freq_pi[i] = theta^(-2i/128) / pi), so that its range reduction is exact.
__device__ __forceinline__ void rope_fill(DecCtl *ctl, const double *freq_pi, int64_t p)
{
    const int i = threadIdx.x;
    if (i < ATTN_HD / 2) {
        double sn, cs;
        sincospi((double)p * freq_pi[i], &sn, &cs);
        ctl->rope_cs[2 * i] = (float)cs;
        ctl->rope_cs[2 * i + 1] = (float)sn;
    }
}

constexpr int MAX_HEAD_WGS = 4096;   // most LM-head workgroups (one argmax key each)

// ---------------------------------------------------------------------------------------
// policies for the shared Q4_0 tile pipeline (gemv_core.h)
// ---------------------------------------------------------------------------------------

struct QkvArgs {
    const uint8_t *wq;
    int64_t dk, dv;              // byte offsets from wq to the K and V weights
    int qrows, kvrows;
    const float *h;              // residual stream (layers >= 1)
    float *h_out;                // layer 0: receives the embedding row
    const uint8_t *emb;
    const int32_t *tok;
    int vocab;
    const float *gain;
    float eps;
    float *q_out, *kc, *vc;      // q [qrows]; this layer's K, V rings [n_kv][n_slots][128]
    const DecCtl *ctl;           // position and its rotation table
    int n_slots;
};

// xs = RMSNorm(row) * gain for the token's row of the embedding table (Q4_0 or 16-bit); the
// workgroup that passes h_out also stores the raw row there (it is the first residual stream).
template <int NT, int K, int FMT = FMT_Q4>
struct EmbedRmsNormX {
    static constexpr int PAIRS = K / 64;
    static constexpr int PER = (PAIRS + NT - 1) / NT;
    static constexpr int GPER = (K / 4) / NT;
    static constexpr int WORDS = FMT == FMT_Q4 ? 9 : 32;   // dwords of 64 values
    static_assert((K / 4) % NT == 0, "the workgroup must cover the vector evenly");
    uint32_t raw[PER][WORDS];
    f32x4 gv[GPER];

    __device__ __forceinline__ void issue(const uint8_t *__restrict__ row, const float *__restrict__ gain)
    {
#pragma unroll
        for (int j = 0; j < PER; ++j) {
            const int c = min((int)threadIdx.x + j * NT, PAIRS - 1);   // unconditional load
            const uint32_t *p = reinterpret_cast<const uint32_t *>(row + 4 * WORDS * c);
#pragma unroll
            for (int i = 0; i < WORDS; ++i)
                raw[j][i] = p[i];
        }
        const f32x4 *g4 = reinterpret_cast<const f32x4 *>(gain);
#pragma unroll
        for (int j = 0; j < GPER; ++j)
            gv[j] = g4[threadIdx.x + j * NT];
    }
    __device__ __forceinline__ float stage(float *xs, float eps, float *wsum, float *h_out)
    {
        float ss = 0.0f;
#pragma unroll
        for (int j = 0; j < PER; ++j) {
            const int c = threadIdx.x + j * NT;
            if (c < PAIRS) {
                float v[64];
                if constexpr (FMT == FMT_Q4) {
                    dequant_pair_words(raw[j], v);
                } else {
#pragma unroll
                    for (int i = 0; i < 32; ++i) {
                        const uint32_t u = raw[j][i];
                        if constexpr (FMT == FMT_BF16) {
                            v[2 * i] = __builtin_bit_cast(float, u << 16);
                            v[2 * i + 1] = __builtin_bit_cast(float, u & 0xFFFF0000u);
                        } else {
                            v[2 * i] = half_bits_to_float(u & 0xFFFFu);
                            v[2 * i + 1] = half_bits_to_float(u >> 16);
                        }
                    }
                }
                float4 *d4 = reinterpret_cast<float4 *>(xs + XS_ROW * c);
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const float4 q = make_float4(v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3]);
                    d4[i] = q;
                    if (h_out)
                        reinterpret_cast<float4 *>(h_out + 64 * c)[i] = q;
                }
#pragma unroll
                for (int i = 0; i < 64; ++i)
                    ss = fmaf(v[i], v[i], ss);
            }
        }
        const float tot = block_sum_fixed<NT>(ss, wsum);   // its barriers also publish xs
        const float inv = 1.0f / sqrtf(tot / (float)K + eps);
#pragma unroll
        for (int j = 0; j < GPER; ++j) {
            f32x4 *p = reinterpret_cast<f32x4 *>(xs + xs_index(4 * (threadIdx.x + j * NT)));
            *p = *p * inv * gv[j];
        }
        __syncthreads();
        return 1.0f;
    }
};

template <class Gm, bool EMBED>
struct QkvPolicy {
    QkvArgs a;
    int64_t pos;
    float rot_c, rot_s;   // cos and sin of this thread's row pair in the next tile

    __host__ __device__ static int tiles(const QkvArgs &a) { return (a.qrows + 2 * a.kvrows) / Gm::R; }

    typedef std::conditional_t<EMBED, EmbedRmsNormX<Gm::NT, Gm::K, Gm::FMT>, RmsNormX<Gm::NT, Gm::K>> XRegs;
    __device__ void x_issue(XRegs &x)
    {
        if constexpr (EMBED) {
            int t = *a.tok;
            t = t < 0 ? 0 : (t >= a.vocab ? a.vocab - 1 : t);
            x.issue(a.emb + (size_t)t * Gm::RB, a.gain);
        } else {
            x.issue(a.h, a.gain);
        }
    }
    __device__ float x_stage(XRegs &x, float *xs, float *wsum)
    {
        if constexpr (EMBED)
            return x.stage(xs, a.eps, wsum, blockIdx.x == 0 ? a.h_out : nullptr);
        else
            return x.stage(xs, a.eps, wsum);
    }
    __device__ void pre(int t)
    {
        pos = a.ctl->pos;
        const int r0 = t * Gm::R + 2 * min((int)threadIdx.x, Gm::R / 2 - 1);
        rot_c = a.ctl->rope_cs[r0 % ATTN_HD];       // unconditional loads (v rows ignore them)
        rot_s = a.ctl->rope_cs[r0 % ATTN_HD + 1];
    }
    __device__ int num_tiles() const { return tiles(a); }
    __device__ const uint8_t *slice(int t, int, int &rows_valid) const
    {
        // integer selects (a choice among pointer fields would be lowered to an indexed load
        // from a stack copy of the arguments)
        rows_valid = Gm::R;
        const int r0 = t * Gm::R;
        const bool is_q = r0 < a.qrows, is_k = !is_q && r0 < a.qrows + a.kvrows;
        const int64_t off = is_q ? (int64_t)r0 * Gm::RB
                                 : (is_k ? a.dk + (int64_t)(r0 - a.qrows) * Gm::RB
                                         : a.dv + (int64_t)(r0 - a.qrows - a.kvrows) * Gm::RB);
        return a.wq + off;
    }
    __device__ void epilogue(int t, const float *rs)
    {
        const int tid = threadIdx.x;
        if (tid >= Gm::R / 2)
            return;
        const int r0 = t * Gm::R + 2 * tid;
        float y0 = rs[2 * tid], y1 = rs[2 * tid + 1];
        const int region = r0 < a.qrows ? 0 : (r0 < a.qrows + a.kvrows ? 1 : 2);
        if (region < 2) {
            // rotary position: pair i of the head turns by pos * theta^(-2i/128) radians
            const float u = y0 * rot_c - y1 * rot_s;
            const float v = y0 * rot_s + y1 * rot_c;
            y0 = u;
            y1 = v;
        }
        if (region == 0) {
            a.q_out[r0] = y0;
            a.q_out[r0 + 1] = y1;
        } else {
            const int rr = r0 - a.qrows - (region == 2 ? a.kvrows : 0);
            const int slot = (int)(pos % a.n_slots);
            float *dst = (region == 1 ? a.kc : a.vc) + ((size_t)(rr / ATTN_HD) * a.n_slots + slot) * ATTN_HD +
                         rr % ATTN_HD;
            dst[0] = y0;
            dst[1] = y1;
        }
    }
    __device__ void finish(float *) {}
};

struct ResidualArgs {
    const uint8_t *w;
    const float *x;
    float *h;
    int n;
};

// y = W x added into the residual stream h (attention output projection, FFN down).
template <class Gm>
struct ResidualPolicy {
    ResidualArgs a;
    float hv;   // residual value of this thread's row, loaded with the tile

    __host__ __device__ static int tiles(const ResidualArgs &a) { return a.n / Gm::R; }
    typedef PlainX<Gm::NT, Gm::K> XRegs;
    __device__ void x_issue(XRegs &r) { r.issue(a.x); }
    __device__ float x_stage(XRegs &r, float *xs, float *) { return r.stage(xs); }
    __device__ void pre(int t)
    {
        hv = a.h[t * Gm::R + min((int)threadIdx.x, Gm::R - 1)];   // unconditional load
    }
    __device__ int num_tiles() const { return tiles(a); }
    __device__ const uint8_t *slice(int t, int, int &rows_valid) const
    {
        rows_valid = Gm::R;
        return a.w + (size_t)t * Gm::R * Gm::RB;
    }
    __device__ void epilogue(int t, const float *rs)
    {
        const int tid = threadIdx.x;
        if (tid < Gm::R)
            a.h[t * Gm::R + tid] = hv + rs[tid];
    }
    __device__ void finish(float *) {}
};

struct GateUpArgs {
    const uint8_t *wg, *wu;
    int n;                  // hidden width
    const float *h, *gain;
    float eps;
    float *act;
};

// act = silu(Wg x) * (Wu x) with x = RMSNorm(h) * gain; a tile holds R/2 gate rows then the
// matching R/2 up rows.
template <class Gm>
struct GateUpPolicy {
    GateUpArgs a;

    __host__ __device__ static int tiles(const GateUpArgs &a) { return a.n / (Gm::R / 2); }
    typedef RmsNormX<Gm::NT, Gm::K> XRegs;
    __device__ void x_issue(XRegs &r) { r.issue(a.h, a.gain); }
    __device__ float x_stage(XRegs &r, float *xs, float *wsum) { return r.stage(xs, a.eps, wsum); }
    __device__ void pre(int) {}
    __device__ int num_tiles() const { return tiles(a); }
    __device__ const uint8_t *slice(int t, int part, int &rows_valid) const
    {
        rows_valid = Gm::R / 2;
        return (part == 0 ? a.wg : a.wu) + (size_t)t * (Gm::R / 2) * Gm::RB;
    }
    __device__ void epilogue(int t, const float *rs)
    {
        const int tid = threadIdx.x;
        if (tid < Gm::R / 2)
            a.act[t * (Gm::R / 2) + tid] = silu(rs[tid]) * rs[Gm::R / 2 + tid];
    }
    __device__ void finish(float *) {}
};

struct LmHeadArgs {
    const uint8_t *emb;
    int vocab;
    const float *h, *gain;
    float eps;
    float *logits;                 // may be null
    unsigned long long *keys;      // [gridDim.x] best (logit, index) key of each workgroup
};

template <class Gm>
struct LmHeadPolicy {
    LmHeadArgs a;
    unsigned long long best;

    __host__ __device__ static int tiles(const LmHeadArgs &a) { return (a.vocab + Gm::R - 1) / Gm::R; }
    typedef RmsNormX<Gm::NT, Gm::K> XRegs;
    __device__ void x_issue(XRegs &r)
    {
        best = 0ull;
        r.issue(a.h, a.gain);
    }
    __device__ float x_stage(XRegs &r, float *xs, float *wsum) { return r.stage(xs, a.eps, wsum); }
    __device__ void pre(int) {}
    __device__ int num_tiles() const { return tiles(a); }
    __device__ const uint8_t *slice(int t, int, int &rows_valid) const
    {
        const int r0 = t * Gm::R;
        rows_valid = a.vocab - r0 < Gm::R ? a.vocab - r0 : Gm::R;
        return a.emb + (size_t)r0 * Gm::RB;
    }
    __device__ void epilogue(int t, const float *rs)
    {
        const int tid = threadIdx.x;
        const int r = t * Gm::R + tid;
        if (tid < Gm::R && r < a.vocab) {
            const float v = rs[tid];
            if (a.logits)
                a.logits[r] = v;
            const unsigned long long k = argmax_key(v, (uint32_t)r);
            best = k > best ? k : best;
        }
    }
    __device__ void finish(float *)
    {
        __shared__ unsigned long long keys[Gm::R];
        const int tid = threadIdx.x;
        if (tid < Gm::R)
            keys[tid] = best;
        __syncthreads();
        if (tid == 0) {
            unsigned long long m = 0ull;
            for (int i = 0; i < Gm::R; ++i)
                m = keys[i] > m ? keys[i] : m;
            a.keys[blockIdx.x] = m;
        }
    }
};

// Greedy choice: the largest of the LM-head workgroups' keys (value first, then the lowest
// index); writes the token and advances the position.  One workgroup of 256 threads.
__global__ __launch_bounds__(256) void dec_finalize_kernel(DecCtl *ctl, const unsigned long long *keys, int nkeys,
                                                           int32_t *tok_out, const double *freq_pi)
{
    __shared__ unsigned long long part[256];
    const int64_t next = ctl->pos + 1;
    rope_fill(ctl, freq_pi, next);   // the next step's rotation table
    unsigned long long m = 0ull;
    for (int i = threadIdx.x; i < nkeys; i += 256)
        m = keys[i] > m ? keys[i] : m;
    part[threadIdx.x] = m;
    __syncthreads();
    for (int w = 128; w > 0; w >>= 1) {
        if ((int)threadIdx.x < w) {
            const unsigned long long o = part[threadIdx.x + w];
            part[threadIdx.x] = o > part[threadIdx.x] ? o : part[threadIdx.x];
        }
        __syncthreads();
    }
    if (threadIdx.x == 0) {
        tok_out[0] = (int32_t)argmax_key_index(part[0]);
        ctl->pos = next;
    }
}

// At least three waves per SIMD: four resident 3-wave workgroups per compute unit.
template <class Gm, class Policy>
__global__ __launch_bounds__(Gm::NT) __attribute__((amdgpu_waves_per_eu(3))) void dec_gemv_kernel(Policy P)
{
    gemv_tiles<Gm>(P);
}

// LATE_V for the split-window buckets: two resident workgroups per compute unit.
template <int GROUP, bool LATE_V>
__global__ __launch_bounds__(ATTN_THREADS) __attribute__((amdgpu_waves_per_eu(LATE_V && GROUP == 1 ? 4 : LATE_V && GROUP <= 4 ? 2 : 1))) void dec_attn_kernel(AttnArgs a)
{
    attn_chunk<GROUP, LATE_V>(a);
}

// Merges the split partials of one query head (only launched when the window may be split).
template <int GROUP>
__global__ __launch_bounds__(ATTN_MERGE_THREADS) void dec_attn_merge_kernel(AttnArgs a)
{
    __shared__ AttnMergeLds lds;
    const int64_t p = *a.pos + 1;
    const int nv = p < a.n_slots ? (int)p : a.n_slots;
    const AttnPlan plan = attn_plan(nv, a.s_cap);
    if (plan.splits > 1)
        attn_merge<GROUP>(a, blockIdx.x / GROUP, blockIdx.x % GROUP, plan.splits, lds);
}

// RoPE frequencies theta^(-2i/head_dim) / pi, i < head_dim/2, in fp64 (once per decoder).
__global__ void dec_rope_table_kernel(double *freq, float theta)
{
    const int i = threadIdx.x;
    if (i < ATTN_HD / 2)
        freq[i] = pow((double)theta, -2.0 * (double)i / (double)ATTN_HD) / 3.14159265358979323846;
}

// Sets the position of the next token (0 for a reset) and its rotation table.
__global__ void dec_seek_kernel(DecCtl *ctl, const double *freq_pi, int64_t pos)
{
    rope_fill(ctl, freq_pi, pos);
    if (threadIdx.x == 0)
        ctl->pos = pos;
}

// ---------------------------------------------------------------------------------------
// host dispatch: widths are compile-time in the kernels
// ---------------------------------------------------------------------------------------

template <int K>
constexpr int nt_for()
{
    return K == 1024 ? 128 : K == 2048 ? 128 : K == 3072 ? 192 : K == 4096 ? 256 : 576;
}

template <int K, int R, int NPART = 1, int FMT = FMT_Q4>
using DGeom = GemvGeom<K, nt_for<K>(), R, NPART, FMT>;

template <class Gm, class Policy, class Args>
static int launch_gemv(const Args &args, hipStream_t s, const char *what, int *grid_out = nullptr)
{
    static std::atomic<int> occ_cache{0};
    const int occ = resident_per_cu(occ_cache, dec_gemv_kernel<Gm, Policy>, Gm::NT);
    const int ntiles = Policy::tiles(args);
    const int cap = occ * cu_count();
    int grid = ntiles < cap ? ntiles : cap;
    if (grid > MAX_HEAD_WGS)
        grid = MAX_HEAD_WGS;
    if (grid_out)
        *grid_out = grid;
    Policy P{args};
    hipLaunchKernelGGL((dec_gemv_kernel<Gm, Policy>), dim3(grid > 0 ? grid : 1), dim3(Gm::NT), 0, s, P);
    return check_launch(what);
}

// R choices: the group count G (= NT / (K/64)) must divide R.
template <int K>
constexpr int min_rows()
{
    return nt_for<K>() / (K / 64);
}

// 16-bit rows take the shortest tile the row groups allow (4 rows, 8 at width 1024): a row is
// 3.6 times the bytes of a Q4_0 row, so these tiles carry about as many bytes as the Q4_0 ones.
template <int K, int FMT>
constexpr int w16_rows()
{
    return min_rows<K>() > 4 ? min_rows<K>() : 4;
}

template <int K, bool EMBED, int FMT>
static int run_qkv(const QkvArgs &a, int, hipStream_t s)
{
    constexpr int R = FMT == FMT_Q4 ? 8 : w16_rows<K, FMT>();
    return launch_gemv<DGeom<K, R, 1, FMT>, QkvPolicy<DGeom<K, R, 1, FMT>, EMBED>>(a, s, "decoder qkv");
}

template <int K, int FMT>
static int run_residual(const ResidualArgs &a, int R, hipStream_t s)
{
    if constexpr (FMT != FMT_Q4) {
        constexpr int RW = w16_rows<K, FMT>();
        return launch_gemv<DGeom<K, RW, 1, FMT>, ResidualPolicy<DGeom<K, RW, 1, FMT>>>(a, s, "decoder residual gemv");
    } else {
        if (R == 16)
            return launch_gemv<DGeom<K, 16>, ResidualPolicy<DGeom<K, 16>>>(a, s, "decoder residual gemv");
        if constexpr (12 % min_rows<K>() == 0) {
            if (R == 12)
                return launch_gemv<DGeom<K, 12>, ResidualPolicy<DGeom<K, 12>>>(a, s, "decoder residual gemv");
        }
        if (R == 8 || min_rows<K>() > 4)
            return launch_gemv<DGeom<K, 8>, ResidualPolicy<DGeom<K, 8>>>(a, s, "decoder residual gemv");
        if constexpr (min_rows<K>() <= 4)
            return launch_gemv<DGeom<K, 4>, ResidualPolicy<DGeom<K, 4>>>(a, s, "decoder residual gemv");
        return VOX_E_UNSUPPORTED;
    }
}

template <int K, int FMT>
static int run_gateup(const GateUpArgs &a, int R, hipStream_t s)
{
    if constexpr (FMT != FMT_Q4) {
        constexpr int RW = w16_rows<K, FMT>();
        return launch_gemv<DGeom<K, RW, 2, FMT>, GateUpPolicy<DGeom<K, RW, 2, FMT>>>(a, s, "decoder gate/up");
    } else {
        if (R == 16)
            return launch_gemv<DGeom<K, 16, 2>, GateUpPolicy<DGeom<K, 16, 2>>>(a, s, "decoder gate/up");
        return launch_gemv<DGeom<K, 8, 2>, GateUpPolicy<DGeom<K, 8, 2>>>(a, s, "decoder gate/up");
    }
}

template <int K, int FMT>
static int run_lmhead(const LmHeadArgs &a, int R, hipStream_t s, int *grid)
{
    if constexpr (FMT != FMT_Q4) {
        constexpr int RW = w16_rows<K, FMT>();
        return launch_gemv<DGeom<K, RW, 1, FMT>, LmHeadPolicy<DGeom<K, RW, 1, FMT>>>(a, s, "decoder lm head", grid);
    } else {
        if (R == 16)
            return launch_gemv<DGeom<K, 16>, LmHeadPolicy<DGeom<K, 16>>>(a, s, "decoder lm head", grid);
        return launch_gemv<DGeom<K, 8>, LmHeadPolicy<DGeom<K, 8>>>(a, s, "decoder lm head", grid);
    }
}

static bool model_width(int k) { return k == 1024 || k == 3072; }
static bool attn_width(int k) { return k == 1024 || k == 4096; }
static bool ffn_width(int k) { return k == 2048 || k == 9216; }

// Tile height for n row-tiles-worth of work: tall tiles when there are plenty, otherwise short
// ones so that every compute unit gets work.
static int pick_r(int64_t rows, int min_r)
{
    const int64_t cu = cu_count();
    if (rows >= 16 * 4 * cu)
        return 16;
    if (rows >= 8 * 2 * cu || min_r > 4)
        return 8;
    return 4;
}

struct Layout {
    size_t ctl, keys, rope, h, q, o, act, part, total;
};

static size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

static Layout scratch_layout(const vox_decoder_config &c)
{
    Layout L{};
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t at = off;
        off = align_up(off + bytes, 256);
        return at;
    };
    const int group = c.n_heads / c.n_kv_heads;
    L.ctl = take(sizeof(DecCtl));
    L.keys = take(sizeof(unsigned long long) * MAX_HEAD_WGS);
    L.rope = take(sizeof(double) * ATTN_HD / 2);
    L.h = take((size_t)c.dim * 4);
    L.q = take((size_t)c.n_heads * c.head_dim * 4);
    L.o = take((size_t)c.n_heads * c.head_dim * 4);
    L.act = take((size_t)c.hidden * 4);
    L.part = take((size_t)c.n_kv_heads * attn_split_cap(c.n_slots) * group * ATTN_PART * 4);
    L.total = off;
    return L;
}

static size_t kv_bytes_for(const vox_decoder_config &c)
{
    return (size_t)c.n_layers * 2 * c.n_kv_heads * c.n_slots * c.head_dim * sizeof(float);
}

static int check_config(const vox_decoder_config *c)
{
    if (!c)
        return fail(VOX_E_INVAL, "decoder: null config");
    if (c->n_layers < 1 || c->dim < 1 || c->n_heads < 1 || c->n_kv_heads < 1 || c->head_dim < 1 || c->hidden < 1 ||
        c->vocab < 1 || c->n_slots < 1)
        return fail(VOX_E_INVAL, "decoder: every size must be positive");
    if (c->n_heads % c->n_kv_heads)
        return fail(VOX_E_INVAL, "decoder: n_heads must be a multiple of n_kv_heads");
    if (!(c->norm_eps >= 0.0f) || !(c->rope_theta > 0.0f))
        return fail(VOX_E_INVAL, "decoder: need norm_eps >= 0 and rope_theta > 0");
    const int group = c->n_heads / c->n_kv_heads;
    if (c->head_dim != ATTN_HD || (group != 1 && group != 2 && group != 4 && group != 8) || c->n_kv_heads > 64)
        return fail(VOX_E_UNSUPPORTED, "decoder: needs head_dim 128, n_heads/n_kv_heads in {1,2,4,8}, n_kv_heads <= 64");
    if (!model_width(c->dim) || !attn_width(c->n_heads * c->head_dim) || !ffn_width(c->hidden))
        return fail(VOX_E_UNSUPPORTED,
                    "decoder: widths (dim %d, heads*head_dim %d, hidden %d) must be (3072|1024, 4096|1024, 9216|2048)",
                    c->dim, c->n_heads * c->head_dim, c->hidden);
    if (c->n_slots > (1 << 24) || c->vocab > (1 << 28))
        return fail(VOX_E_UNSUPPORTED, "decoder: n_slots or vocab too large");
    return VOX_OK;
}

}  // namespace vox

using namespace vox;

struct vox_decoder {
    vox_decoder_config c;
    std::vector<vox_layer_weights> layers;
    const uint8_t *tok_embd;
    const float *out_norm;
    float *kv;
    uint8_t *scratch;
    Layout lay;
    DecCtl *ctl;
    unsigned long long *keys;
    double *rope;
    float *h, *q, *o, *act, *part;
    int fmt;   // FMT_Q4, FMT_BF16 or FMT_F16: the format of every matrix
    int group, s_cap;
    int r_qkv, r_o, r_ffn, r_down, r_head;
    int64_t host_pos;
    bool use_graph;
    hipStream_t cap_stream;
    hipGraphExec_t graphs[16];
    const int32_t *g_in;
    int32_t *g_out;
    float *g_logits;
};

namespace vox {

static int attn_bucket(const vox_decoder *d, int64_t pos)
{
    const int64_t nv64 = pos + 1 < d->c.n_slots ? pos + 1 : d->c.n_slots;
    const int splits = attn_plan((int)nv64, d->s_cap).splits;
    int b = 0;
    while ((1 << b) < splits)
        ++b;
    return b;   // grid width 1 << b, capped at s_cap at launch
}

// Up to eight chunks: one workgroup per (query head, chunk), each reading its KV head's chunk
// (the group's heads share it through the cache), so the scores and the weighted sums of the
// heads run on compute units of their own.  More chunks: one workgroup per (KV head, chunk)
// serving the group's query heads from one load of K and V (measured on MI355X: past eight
// chunks the extra reads of the shared chunks cost more than the spread).  A split window ends
// with the merge.
template <int GROUP>
static int launch_attn(const AttnArgs &a, int width, int n_kv, hipStream_t s)
{
    const bool per_head = width <= 8;
    AttnArgs b = a;
    if (per_head)
        b.kv_shift = GROUP == 8 ? 3 : GROUP == 4 ? 2 : GROUP == 2 ? 1 : 0;
    if (width == 1)
        hipLaunchKernelGGL((dec_attn_kernel<1, false>), dim3(1, n_kv * GROUP), dim3(ATTN_THREADS), 0, s, b);
    else if (per_head)
        hipLaunchKernelGGL((dec_attn_kernel<1, true>), dim3(width, n_kv * GROUP), dim3(ATTN_THREADS), 0, s, b);
    else
        hipLaunchKernelGGL((dec_attn_kernel<GROUP, true>), dim3(width, n_kv), dim3(ATTN_THREADS), 0, s, b);
    int st = check_launch("decoder attention");
    if (st || width == 1)
        return st;
    if (per_head)
        hipLaunchKernelGGL(dec_attn_merge_kernel<1>, dim3(n_kv * GROUP), dim3(ATTN_MERGE_THREADS), 0, s, b);
    else
        hipLaunchKernelGGL(dec_attn_merge_kernel<GROUP>, dim3(n_kv * GROUP), dim3(ATTN_MERGE_THREADS), 0, s, b);
    return check_launch("decoder attention merge");
}

template <int FMT>
static int enqueue_step_fmt(vox_decoder *d, const int32_t *tok_in, int32_t *tok_out, float *logits, int bucket,
                            hipStream_t s)
{
    const vox_decoder_config &c = d->c;
    const int qd = c.n_heads * c.head_dim, kvd = c.n_kv_heads * c.head_dim;
    const size_t ring = (size_t)c.n_kv_heads * c.n_slots * c.head_dim;
    int width = 1 << bucket;
    if (width > d->s_cap)
        width = d->s_cap;
    int st = VOX_OK;
    for (int l = 0; l < c.n_layers && !st; ++l) {
        const vox_layer_weights &L = d->layers[l];
        float *kc = d->kv + (size_t)(2 * l) * ring;
        float *vc = d->kv + (size_t)(2 * l + 1) * ring;

        QkvArgs qa{};
        qa.wq = (const uint8_t *)L.wq;
        qa.dk = (int64_t)((uintptr_t)L.wk - (uintptr_t)L.wq);
        qa.dv = (int64_t)((uintptr_t)L.wv - (uintptr_t)L.wq);
        qa.qrows = qd;
        qa.kvrows = kvd;
        qa.h = d->h;
        qa.h_out = d->h;
        qa.emb = d->tok_embd;
        qa.tok = tok_in;
        qa.vocab = c.vocab;
        qa.gain = L.attn_norm;
        qa.eps = c.norm_eps;
        qa.q_out = d->q;
        qa.kc = kc;
        qa.vc = vc;
        qa.ctl = d->ctl;
        qa.n_slots = c.n_slots;
        if (c.dim == 3072)
            st = l == 0 ? run_qkv<3072, true, FMT>(qa, d->r_qkv, s) : run_qkv<3072, false, FMT>(qa, d->r_qkv, s);
        else
            st = l == 0 ? run_qkv<1024, true, FMT>(qa, d->r_qkv, s) : run_qkv<1024, false, FMT>(qa, d->r_qkv, s);
        if (st)
            break;

        AttnArgs aa{};
        aa.q = d->q;
        aa.kc = kc;
        aa.vc = vc;
        aa.out = d->o;
        aa.part = d->part;
        aa.pos = &d->ctl->pos;
        aa.n_slots = c.n_slots;
        aa.n_valid = 0;
        aa.s_cap = d->s_cap;
        aa.scale = 1.0f / sqrtf((float)c.head_dim);
        switch (d->group) {
        case 1: st = launch_attn<1>(aa, width, c.n_kv_heads, s); break;
        case 2: st = launch_attn<2>(aa, width, c.n_kv_heads, s); break;
        case 4: st = launch_attn<4>(aa, width, c.n_kv_heads, s); break;
        default: st = launch_attn<8>(aa, width, c.n_kv_heads, s); break;
        }
        if (st)
            break;

        ResidualArgs oa{(const uint8_t *)L.wo, d->o, d->h, c.dim};
        st = qd == 4096 ? run_residual<4096, FMT>(oa, d->r_o, s) : run_residual<1024, FMT>(oa, d->r_o, s);
        if (st)
            break;

        GateUpArgs ga{(const uint8_t *)L.w_gate, (const uint8_t *)L.w_up, c.hidden, d->h, L.ffn_norm, c.norm_eps,
                      d->act};
        st = c.dim == 3072 ? run_gateup<3072, FMT>(ga, d->r_ffn, s) : run_gateup<1024, FMT>(ga, d->r_ffn, s);
        if (st)
            break;

        ResidualArgs da{(const uint8_t *)L.w_down, d->act, d->h, c.dim};
        st = c.hidden == 9216 ? run_residual<9216, FMT>(da, d->r_down, s) : run_residual<2048, FMT>(da, d->r_down, s);
    }
    if (st)
        return st;
    LmHeadArgs la{d->tok_embd, c.vocab, d->h, d->out_norm, c.norm_eps, logits, d->keys};
    int grid = 0;
    int st2 = c.dim == 3072 ? run_lmhead<3072, FMT>(la, d->r_head, s, &grid) : run_lmhead<1024, FMT>(la, d->r_head, s, &grid);
    if (st2)
        return st2;
    hipLaunchKernelGGL(dec_finalize_kernel, dim3(1), dim3(256), 0, s, d->ctl, (const unsigned long long *)d->keys, grid,
                       tok_out, (const double *)d->rope);
    return check_launch("decoder finalize");
}

static int enqueue_step(vox_decoder *d, const int32_t *tok_in, int32_t *tok_out, float *logits, int bucket,
                        hipStream_t s)
{
    switch (d->fmt) {
    case FMT_BF16: return enqueue_step_fmt<FMT_BF16>(d, tok_in, tok_out, logits, bucket, s);
    case FMT_F16: return enqueue_step_fmt<FMT_F16>(d, tok_in, tok_out, logits, bucket, s);
    default: return enqueue_step_fmt<FMT_Q4>(d, tok_in, tok_out, logits, bucket, s);
    }
}

static void drop_graphs(vox_decoder *d)
{
    for (auto &g : d->graphs) {
        if (g)
            (void)hipGraphExecDestroy(g);   // teardown: nothing to report
        g = nullptr;
    }
}

}  // namespace vox

extern "C" int vox_decoder_workspace(const vox_decoder_config *c, size_t *kv_bytes, size_t *scratch_bytes)
{
    int st = check_config(c);
    if (st)
        return st;
    if (!kv_bytes || !scratch_bytes)
        return fail(VOX_E_INVAL, "vox_decoder_workspace: null output pointer");
    *kv_bytes = kv_bytes_for(*c);
    *scratch_bytes = scratch_layout(*c).total;
    return ok();
}

namespace vox {

static int create_decoder(const vox_decoder_config *c, const vox_decoder_weights *w, int fmt, void *kv,
                          size_t kv_bytes, void *scratch, size_t scratch_bytes, void *stream, vox_decoder_t **out)
{
    if (!out)
        return fail(VOX_E_INVAL, "vox_decoder_create: null output handle");
    *out = nullptr;
    int st = check_config(c);
    if (st)
        return st;
    if (!w || !w->tok_embd || !w->out_norm || !w->layers || !kv || !scratch)
        return fail(VOX_E_INVAL, "vox_decoder_create: null weight or buffer pointer");
    for (int l = 0; l < c->n_layers; ++l) {
        const vox_layer_weights &L = w->layers[l];
        const void *ps[] = {L.attn_norm, L.ffn_norm, L.wq, L.wk, L.wv, L.wo, L.w_gate, L.w_up, L.w_down};
        for (const void *p : ps) {
            if (!p)
                return fail(VOX_E_INVAL, "vox_decoder_create: layer %d has a null weight", l);
            if (!aligned(p, 16))
                return fail(VOX_E_UNSUPPORTED, "vox_decoder_create: layer %d weight not 16-byte aligned", l);
        }
    }
    if (!aligned(w->tok_embd, 16) || !aligned(w->out_norm, 16) || !aligned(kv, 256) || !aligned(scratch, 256))
        return fail(VOX_E_UNSUPPORTED, "vox_decoder_create: embedding/norm need 16-byte, buffers 256-byte alignment");
    const Layout lay = scratch_layout(*c);
    if (kv_bytes < kv_bytes_for(*c) || scratch_bytes < lay.total)
        return fail(VOX_E_WORKSPACE, "vox_decoder_create: kv %zu (need %zu), scratch %zu (need %zu)", kv_bytes,
                    kv_bytes_for(*c), scratch_bytes, lay.total);
    if (overlaps(kv, kv_bytes_for(*c), scratch, lay.total))
        return fail(VOX_E_INVAL, "vox_decoder_create: kv and scratch overlap");

    vox_decoder *d = new (std::nothrow) vox_decoder();
    if (!d)
        return fail(VOX_E_INVAL, "vox_decoder_create: out of host memory");
    d->c = *c;
    d->fmt = fmt;
    d->layers.assign(w->layers, w->layers + c->n_layers);
    d->tok_embd = (const uint8_t *)w->tok_embd;
    d->out_norm = w->out_norm;
    d->kv = (float *)kv;
    d->scratch = (uint8_t *)scratch;
    d->lay = lay;
    d->ctl = (DecCtl *)(d->scratch + lay.ctl);
    d->keys = (unsigned long long *)(d->scratch + lay.keys);
    d->rope = (double *)(d->scratch + lay.rope);
    d->h = (float *)(d->scratch + lay.h);
    d->q = (float *)(d->scratch + lay.q);
    d->o = (float *)(d->scratch + lay.o);
    d->act = (float *)(d->scratch + lay.act);
    d->part = (float *)(d->scratch + lay.part);
    d->group = c->n_heads / c->n_kv_heads;
    d->s_cap = attn_split_cap(c->n_slots);
    const int qd = c->n_heads * c->head_dim;
    d->r_qkv = 8;   // 8-row tiles stay inside one of the q, k, v row ranges for every width
    d->r_o = pick_r(c->dim, qd == 4096 ? 4 : 8);
    d->r_ffn = pick_r(2 * c->hidden, 8);
    d->r_down = pick_r(c->dim, 4);
    d->r_head = pick_r(c->vocab, 8);
    if (c->dim == 3072 && qd == 4096 && c->hidden == 9216) {
        // measured on MI355X at this shape (decoder ms/token over tile heights per kernel, with
        // the rest of the step as it is): 4-row tiles for the O and down projections (768
        // workgroups of one tile), 8-row gate/up tiles (4 + 4) and LM-head tiles
        d->r_qkv = 8;
        d->r_o = 4;
        d->r_ffn = 8;
        d->r_down = 4;
        d->r_head = 8;
    }
    d->host_pos = 0;
    d->use_graph = true;
    d->cap_stream = nullptr;
    for (auto &g : d->graphs)
        g = nullptr;
    st = check_hip(hipStreamCreateWithFlags(&d->cap_stream, hipStreamNonBlocking), "vox_decoder_create: stream");
    if (!st) {
        hipLaunchKernelGGL(dec_rope_table_kernel, dim3(1), dim3(64), 0, (hipStream_t)stream, d->rope, c->rope_theta);
        hipLaunchKernelGGL(dec_seek_kernel, dim3(1), dim3(64), 0, (hipStream_t)stream, d->ctl, (const double *)d->rope,
                           (int64_t)0);
        st = check_launch("vox_decoder_create: init");
    }
    if (st) {
        if (d->cap_stream)
            (void)hipStreamDestroy(d->cap_stream);
        delete d;
        return st;
    }
    *out = d;
    return ok();
}

}  // namespace vox

extern "C" int vox_decoder_create(const vox_decoder_config *c, const vox_decoder_weights *w, void *kv, size_t kv_bytes,
                                  void *scratch, size_t scratch_bytes, void *stream, vox_decoder_t **out)
{
    return create_decoder(c, w, FMT_Q4, kv, kv_bytes, scratch, scratch_bytes, stream, out);
}

extern "C" int vox_decoder_create_w16(const vox_decoder_config *c, const vox_decoder_weights *w, int fmt, void *kv,
                                      size_t kv_bytes, void *scratch, size_t scratch_bytes, void *stream,
                                      vox_decoder_t **out)
{
    if (out)
        *out = nullptr;
    if (fmt != VOX_W16_BF16 && fmt != VOX_W16_F16)
        return fail(VOX_E_INVAL, "vox_decoder_create_w16: fmt %d is neither VOX_W16_BF16 nor VOX_W16_F16", fmt);
    return create_decoder(c, w, fmt == VOX_W16_BF16 ? FMT_BF16 : FMT_F16, kv, kv_bytes, scratch, scratch_bytes, stream,
                          out);
}

extern "C" int vox_decoder_reset(vox_decoder_t *d, void *stream)
{
    if (!d)
        return fail(VOX_E_INVAL, "vox_decoder_reset: null handle");
    return vox_decoder_seek(d, 0, stream);
}

extern "C" int vox_decoder_seek(vox_decoder_t *d, int64_t pos, void *stream)
{
    if (!d)
        return fail(VOX_E_INVAL, "vox_decoder_seek: null handle");
    if (pos < 0 || pos > VOX_DECODER_MAX_POS)
        return fail(VOX_E_INVAL, "vox_decoder_seek: position %lld outside [0, 2^40]", (long long)pos);
    hipLaunchKernelGGL(dec_seek_kernel, dim3(1), dim3(64), 0, (hipStream_t)stream, d->ctl, (const double *)d->rope, pos);
    int st = check_launch("vox_decoder_seek");
    if (st)
        return st;
    d->host_pos = pos;
    return ok();
}

extern "C" int vox_decoder_step(vox_decoder_t *d, const int32_t *token_in, int32_t *token_out, float *logits,
                                void *stream)
{
    if (!d || !token_in || !token_out)
        return fail(VOX_E_INVAL, "vox_decoder_step: null pointer");
    hipStream_t s = (hipStream_t)stream;
    const int bucket = attn_bucket(d, d->host_pos);
    int st;
    if (!d->use_graph) {
        st = enqueue_step(d, token_in, token_out, logits, bucket, s);
    } else {
        if (d->g_in != token_in || d->g_out != token_out || d->g_logits != logits) {
            drop_graphs(d);
            d->g_in = token_in;
            d->g_out = token_out;
            d->g_logits = logits;
        }
        if (!d->graphs[bucket]) {
            st = check_hip(hipStreamBeginCapture(d->cap_stream, hipStreamCaptureModeThreadLocal), "begin capture");
            if (st)
                return st;
            st = enqueue_step(d, token_in, token_out, logits, bucket, d->cap_stream);
            hipGraph_t graph = nullptr;
            const int st2 = check_hip(hipStreamEndCapture(d->cap_stream, &graph), "end capture");
            if (!st)
                st = st2;
            if (!st)
                st = check_hip(hipGraphInstantiate(&d->graphs[bucket], graph, nullptr, nullptr, 0), "instantiate");
            if (graph)
                (void)hipGraphDestroy(graph);
            if (st) {
                d->graphs[bucket] = nullptr;
                return st;
            }
        }
        st = check_hip(hipGraphLaunch(d->graphs[bucket], s), "graph launch");
    }
    if (st)
        return st;
    d->host_pos += 1;
    return ok();
}

extern "C" int vox_decoder_position(const vox_decoder_t *d, int64_t *pos)
{
    if (!d || !pos)
        return fail(VOX_E_INVAL, "vox_decoder_position: null pointer");
    *pos = d->host_pos;
    return ok();
}

extern "C" int vox_decoder_set_graph(vox_decoder_t *d, int enable)
{
    if (!d)
        return fail(VOX_E_INVAL, "vox_decoder_set_graph: null handle");
    d->use_graph = enable != 0;
    return ok();
}

extern "C" void vox_decoder_destroy(vox_decoder_t *d)
{
    if (!d)
        return;
    drop_graphs(d);
    if (d->cap_stream)
        (void)hipStreamDestroy(d->cap_stream);
    delete d;
}
