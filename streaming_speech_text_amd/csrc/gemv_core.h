// gemv_core.h - Q4_0 matrix-vector product with dequantisation fused into the product.
//
// The quantised path of the Rust/Burn port ("Mistral의 Voxtral Mini 4B Realtime 모델을 Rust로
// 구현해 브라우저에서 실행", GeekNews 26595, section 아키텍처) keeps every linear in GGUF Q4_0 and
// fuses dequantisation into the matrix product; on the voxtral.c page ("Mistral Voxtral Realtime
// 4B ... 순수 C 기반 CPU 전용 추론 구현", GeekNews 26608, section 성능 벤치마크) the decoder token
// is bandwidth-heavy GPU work.  Here the product streams the 18-byte blocks from HBM once.
//
// Layout of the work (gfx950, wave64):
//  * A workgroup owns tiles of R consecutive rows.  Rows are contiguous in memory, so a
//    tile is one contiguous byte range (R * 9K/16 bytes, 16-byte aligned when K % 256 == 0)
//    loaded with fully coalesced 16-byte loads into LDS.  The loads of the next tile are
//    issued into registers before the current tile is computed (software pipelining), and
//    workgroups loop over tiles (persistent grid sized to the occupancy of the chip).
//  * Two consecutive blocks (36 bytes = 9 dwords, dword aligned) form a "pair".  Thread c of
//    a row group owns pair column c for every row of the group: it holds the 64 activations
//    of that column in registers for the whole kernel, reads its 9 dwords per row from LDS,
//    unpacks the nibbles in registers and accumulates in fp32.
//  * Per block: sum_j (code_j - 8) x_j = sum_j code_j x_j - 8 sum_j x_j; the second term is
//    computed once per kernel.  Nibbles masked in place inside 16-bit halves are exact fp16
//    subnormals and feed mixed-precision FMAs directly, so a weight costs one FMA plus a
//    share of the masks (no separate integer-to-float conversion).
//  * The K/64 partial sums of a row are combined through LDS in a fixed order (the result is
//    deterministic run to run).
//  * The same pipeline streams rows of 16-bit weights (bf16 or IEEE binary16, the formats of
//    voxtral.c's weights and of its GPU path: page GeekNews 26608, sections 모델 다운로드 및 구성
//    and 메모리 요구사항): 2K bytes per row, thread c of a row group taking its 16-byte chunks c,
//    c + K/64, ... of every row with the activations of the same elements.
#pragma once

#include "vox_common.h"

namespace vox {

// Native 16-byte vector (HIP's uint4 is a union-based struct that keeps arrays of it out of
// registers).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Weight formats of a matrix row: GGUF Q4_0 blocks, or 16-bit values (bf16 or IEEE binary16).
enum { FMT_Q4 = 0, FMT_BF16 = 1, FMT_F16 = 2 };

template <int K_, int NT_, int R_, int NPART_ = 1, int FMT_ = FMT_Q4>
struct GemvGeom {
    static constexpr int K = K_;
    static constexpr int NT = NT_;
    static constexpr int R = R_;
    static constexpr int NPART = NPART_;        // tile = NPART slices of R/NPART rows
    static constexpr int FMT = FMT_;
    static constexpr int NB = K / 32;           // Q4_0 blocks per row
    static constexpr int RB = FMT == FMT_Q4 ? NB * 18 : K * 2;   // bytes per row
    static constexpr int TR = K / 64;           // threads per row (one block pair each)
    static constexpr int G = NT / TR;           // row groups per workgroup
    static constexpr int RPP = R / NPART;       // rows per slice
    static constexpr int TC = R * RB / 16;      // 16-byte chunks per tile
    static constexpr int PC = RPP * RB / 16;    // 16-byte chunks per slice
    static constexpr int CPT = (TC + NT - 1) / NT;
    static_assert(K % 256 == 0, "rows must be 16-byte aligned");
    static_assert(NT % 64 == 0 && NT % TR == 0, "workgroup must hold whole row groups");
    static_assert(R % G == 0 && R % NPART == 0, "tile rows must split over the row groups");
};

// The activation vector is staged in LDS as rows of 64 floats (one block pair each) padded to
// XS_ROW floats: thread c reads row c, and with a 256-byte row pitch every lane of a wave
// would start on the same bank; the 16-byte pad spreads consecutive rows over the banks.
constexpr int XS_ROW = 68;
__device__ __forceinline__ int xs_index(int i) { return (i >> 6) * XS_ROW + (i & 63); }

// acc + h * x with h the fp16 value in the low (HI = false) or high half of h2, x and acc fp32
// (one v_fma_mix_f32: the fp16 operand is widened exactly and the FMA rounds once, in fp32).
template <bool HI>
__device__ __forceinline__ float fma_f16h(uint32_t h2, float x, float acc)
{
    if constexpr (HI)
        asm("v_fma_mix_f32 %0, %1, %2, %0 op_sel:[1,0,0] op_sel_hi:[1,0,0]" : "+v"(acc) : "v"(h2), "v"(x));
    else
        asm("v_fma_mix_f32 %0, %1, %2, %0 op_sel_hi:[1,0,0]" : "+v"(acc) : "v"(h2), "v"(x));
    return acc;
}

// Sum over one block of (code - 8) * x, without the scale.  qs: the 16 code bytes;
// x: the block's 32 activations; neg8sum = -8 * sum(x).
// A nibble masked in place inside a 16-bit half is an fp16 subnormal: bits 0-3 read as
// code * 2^-24, bits 4-7 as code * 2^-20, both exact.  So each weight costs one v_fma_mix_f32
// plus a share of five masks per four code bytes, and every product carries the factor 2^-24
// (the high nibbles 16 * 2^-24, removed with the 1/16 below), undone exactly at the end.
__device__ __forceinline__ float q4_block_dot(const uint32_t (&qs)[4], const float *x, float neg8sum)
{
    float lo_acc = neg8sum * 0x1p-24f;
    float hi_acc = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        // code bytes 4i .. 4i+3: bytes 0 and 2 sit at the bottom of the two halves of q,
        // bytes 1 and 3 at the bottom of the halves of q >> 8
        const uint32_t q = qs[i], t = q >> 8;
        const uint32_t lo02 = q & 0x000F000Fu, hi02 = q & 0x00F000F0u;
        const uint32_t lo13 = t & 0x000F000Fu, hi13 = t & 0x00F000F0u;
        const float *xl = x + 4 * i, *xh = x + 16 + 4 * i;
        lo_acc = fma_f16h<false>(lo02, xl[0], lo_acc);
        hi_acc = fma_f16h<false>(hi02, xh[0], hi_acc);
        lo_acc = fma_f16h<false>(lo13, xl[1], lo_acc);
        hi_acc = fma_f16h<false>(hi13, xh[1], hi_acc);
        lo_acc = fma_f16h<true>(lo02, xl[2], lo_acc);
        hi_acc = fma_f16h<true>(hi02, xh[2], hi_acc);
        lo_acc = fma_f16h<true>(lo13, xl[3], lo_acc);
        hi_acc = fma_f16h<true>(hi13, xh[3], hi_acc);
    }
    return fmaf(hi_acc, 0.0625f, lo_acc) * 0x1p24f;
}

// Dot product of one block pair (9 dwords as stored) with its 64 activations.
// dword 0 = d0 | codes0[0..1]; dwords 1..3 = codes0[2..13]; dword 4 = codes0[14..15] | d1;
// dwords 5..8 = codes1[0..15].
__device__ __forceinline__ float q4_pair_dot(const uint32_t (&D)[9], const float (&x)[64], float n8a,
                                             float n8b)
{
    const uint32_t q0[4] = {(D[0] >> 16) | (D[1] << 16), (D[1] >> 16) | (D[2] << 16),
                            (D[2] >> 16) | (D[3] << 16), (D[3] >> 16) | (D[4] << 16)};
    const uint32_t q1[4] = {D[5], D[6], D[7], D[8]};
    const float d0 = half_bits_to_float(D[0]);
    const float d1 = half_bits_to_float(D[4] >> 16);
    const float s0 = q4_block_dot(q0, x, n8a);
    const float s1 = q4_block_dot(q1, x + 32, n8b);
    return fmaf(d0, s0, d1 * s1);
}

// Dot product of 64 16-bit weights (eight 16-byte chunks, eight values each, in order) with
// their activations x[64].  bf16: a value is the upper half of an fp32 (one shift or mask);
// fp16: widened exactly inside v_fma_mix_f32.  Four partial sums over the chunks j % 4, added in a
// fixed order.
template <int FMT>
__device__ __forceinline__ float w16_dot64(const u32x4 (&W)[8], const float (&x)[64])
{
    float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const uint32_t u[4] = {W[j].x, W[j].y, W[j].z, W[j].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float x0 = x[8 * j + 2 * i], x1 = x[8 * j + 2 * i + 1];
            if constexpr (FMT == FMT_BF16) {
                acc[j & 3] = fmaf(__builtin_bit_cast(float, u[i] << 16), x0, acc[j & 3]);
                acc[j & 3] = fmaf(__builtin_bit_cast(float, u[i] & 0xFFFF0000u), x1, acc[j & 3]);
            } else {
                acc[j & 3] = fma_f16h<false>(u[i], x0, acc[j & 3]);
                acc[j & 3] = fma_f16h<true>(u[i], x1, acc[j & 3]);
            }
        }
    }
    return (acc[0] + acc[1]) + (acc[2] + acc[3]);
}

// Per-kernel prologue result: the thread's 64 activations and the two -8*sum terms.
struct PairX {
    float x[64];
    float n8a, n8b;
    float scale;   // applied to every row sum (1 unless the prologue normalises afterwards)

    __device__ __forceinline__ void finish()
    {
        float a = 0.0f, b = 0.0f;
#pragma unroll
        for (int j = 0; j < 32; ++j) {
            a += x[j];
            b += x[32 + j];
        }
        n8a = -8.0f * a;
        n8b = -8.0f * b;
    }
};

// Workgroup-wide sum of one float per thread in a fixed order: a butterfly within each wave,
// then the wave totals in wave order.  `buf` holds at least NT/64 floats of LDS.  All threads
// return the same value.
template <int NT>
__device__ __forceinline__ float block_sum_fixed(float v, float *buf)
{
    v = wave_sum(v);
    if ((threadIdx.x & 63) == 0)
        buf[threadIdx.x >> 6] = v;
    __syncthreads();
    float s = 0.0f;
#pragma unroll
    for (int w = 0; w < NT / 64; ++w)
        s += buf[w];
    __syncthreads();
    return s;
}
// Issues the 16-byte loads of tile t into the thread's prefetch registers.  The loads are
// unconditional (chunks past the end of a short tile re-read the tile's first chunk), so no
// branch separates them and the compiler's wait counts stay exact.  They are non-temporal: each
// weight is read once per call (measured on MI355X: the decoder step 0.871 -> 0.828 ms/token, the
// 9216 x 3072 GEMV 6.06 -> 5.64 us, results identical).
template <class Gm, class Policy>
__device__ __forceinline__ void gemv_fetch(Policy &P, int t, u32x4 (&pf)[Gm::CPT])
{
    const uint8_t *base[Gm::NPART];
    int valid_chunks[Gm::NPART];
#pragma unroll
    for (int p = 0; p < Gm::NPART; ++p) {
        int rows_valid;
        base[p] = P.slice(t, p, rows_valid);
        valid_chunks[p] = rows_valid * (Gm::RB / 16);
    }
    // one base pointer plus integer offsets: a choice between pointers would turn the loads
    // into flat loads, which also count against the LDS wait counter
    const int64_t delta = Gm::NPART == 1 ? 0 : (int64_t)((uintptr_t)base[Gm::NPART - 1] - (uintptr_t)base[0]);
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < Gm::CPT; ++i) {
        const int ch = tid + i * Gm::NT;
        const int p = Gm::NPART == 1 ? 0 : (ch < Gm::PC ? 0 : 1);
        int off = ch - p * Gm::PC;
        off = (ch < Gm::TC && off < valid_chunks[p]) ? off : 0;
        pf[i] = __builtin_nontemporal_load(
            reinterpret_cast<const u32x4 *>(base[0] + (p ? delta : (int64_t)0) + (int64_t)off * 16));
    }
}

// Row sums of the tile in LDS: each thread takes the block pair `c` of rows g, g+G, ...; the
// partial dots go through `red` and are added per row in a fixed order into rowsum[R].
// Ends with a workgroup barrier, after which the tile buffer may be overwritten.
template <class Gm>
__device__ __forceinline__ void gemv_tile_rows(const u32x4 *tile, float *red, float *rowsum, const PairX &px)
{
    const int tid = threadIdx.x;
    const int c = tid % Gm::TR;
    const int g = tid / Gm::TR;
    if constexpr (Gm::FMT == FMT_Q4) {
        const uint32_t *lds32 = reinterpret_cast<const uint32_t *>(tile);
#pragma unroll
        for (int j = 0; j < Gm::R / Gm::G; ++j) {
            const int rr = g + j * Gm::G;
            const uint32_t *p = lds32 + rr * (Gm::RB / 4) + 9 * c;
            uint32_t D[9];
#pragma unroll
            for (int i = 0; i < 9; ++i)
                D[i] = p[i];
            red[rr * Gm::TR + c] = q4_pair_dot(D, px.x, px.n8a, px.n8b);
        }
    } else {
        // 16-bit rows: thread c takes the row's 16-byte chunks c, c + TR, ... (eight of them), so a
        // wave's LDS reads are consecutive; px.x holds the matching activations (w16_load_x)
#pragma unroll
        for (int j = 0; j < Gm::R / Gm::G; ++j) {
            const int rr = g + j * Gm::G;
            const u32x4 *p = tile + rr * (Gm::RB / 16) + c;
            u32x4 W[8];
#pragma unroll
            for (int i = 0; i < 8; ++i)
                W[i] = p[i * Gm::TR];
            red[rr * Gm::TR + c] = w16_dot64<Gm::FMT>(W, px.x);
        }
    }
    __syncthreads();
    // Each row's TR partials are added by RL lanes (TR/RL each, then a DPP tree): a row of 16
    // lanes when TR is a multiple of 16, else a quad; in a fixed order.  Rows beyond NT/RL take
    // another pass.
    constexpr int RL = Gm::TR % 16 == 0 ? 16 : 4;
    static_assert(Gm::TR % RL == 0, "row partials split over 16 or 4 lanes");
    constexpr int ROWS_PER_PASS = Gm::NT / RL;
#pragma unroll
    for (int r0 = 0; r0 < Gm::R; r0 += ROWS_PER_PASS) {
        const int row = r0 + tid / RL;
        if (row < Gm::R) {   // uniform over each group of RL lanes
            const int j = tid % RL;
            float s = 0.0f;
#pragma unroll
            for (int i = 0; i < Gm::TR / RL; ++i)
                s += red[row * Gm::TR + i * RL + j];
            s = RL == 16 ? row16_sum(s) : quad_sum(s);
            if (j == 0)
                rowsum[row] = s * px.scale;
        }
    }
    __syncthreads();
}

// The workgroup stages the activation vector once in LDS (normalisation applied there); each
// thread then keeps the 64 values of its pair column in registers.  Ends with a barrier, after
// which the LDS of xs may be reused.
template <class Gm, class Policy>
__device__ __forceinline__ void gemv_load_x(Policy &P, typename Policy::XRegs &xr, float *xs, float *wsum, PairX &px)
{
    px.scale = P.x_stage(xr, xs, wsum);
    if constexpr (Gm::FMT == FMT_Q4) {
        const float4 *x4 = reinterpret_cast<const float4 *>(xs + XS_ROW * (threadIdx.x % Gm::TR));
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const float4 v = x4[i];
            px.x[4 * i + 0] = v.x;
            px.x[4 * i + 1] = v.y;
            px.x[4 * i + 2] = v.z;
            px.x[4 * i + 3] = v.w;
        }
        px.finish();
    } else {
        // the activations of the thread's chunks c, c + TR, ...: elements 8 (c + j TR) .. + 7
        const int c = threadIdx.x % Gm::TR;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const float4 *x4 = reinterpret_cast<const float4 *>(xs + xs_index(8 * (c + j * Gm::TR)));
            const float4 a = x4[0], b = x4[1];
            px.x[8 * j + 0] = a.x;
            px.x[8 * j + 1] = a.y;
            px.x[8 * j + 2] = a.z;
            px.x[8 * j + 3] = a.w;
            px.x[8 * j + 4] = b.x;
            px.x[8 * j + 5] = b.y;
            px.x[8 * j + 6] = b.z;
            px.x[8 * j + 7] = b.w;
        }
    }
    __syncthreads();
}

// The tile pipeline shared by every GEMV flavour (Q4_0 or 16-bit rows).  Policy supplies:
//   XRegs, x_issue(XRegs&)                 issue the activation loads into registers
//   x_stage(XRegs&, float* xs, float* wsum) fill xs with the activations, element i at
//                                          xs[xs_index(i)] (all threads call it; it ends with a
//                                          workgroup barrier); returns a factor applied to the
//                                          row sums
//   num_tiles()                            tiles of R rows
//   pre(tile)                              early loads the epilogue of `tile` will need
//   slice(tile, part, &rows_valid)         base pointer of slice `part` of the tile
//   epilogue(tile, const float* rowsum)    consume the R row sums (all threads call it)
//   finish(float* lds_scratch)             after the last tile (all threads call it)
// A workgroup walks tiles blockIdx.x, +gridDim.x, ... with the next tile's loads in flight
// while it computes the current one.
template <class Gm, class Policy>
__device__ __forceinline__ void gemv_tiles(Policy &P)
{
    // The staged activation vector is dead once every thread holds its 64 values in registers,
    // so the weight tile reuses its LDS (a barrier separates the two uses).
    constexpr int TILE_VEC = Gm::CPT * Gm::NT;                 // padded: every thread stores all its chunks
    constexpr int XS_VEC = (Gm::K / 64 * XS_ROW + 3) / 4;      // the activation vector (padded rows)
    __shared__ u32x4 lds_main[TILE_VEC > XS_VEC ? TILE_VEC : XS_VEC];
    u32x4 *const tile = lds_main;
    float *const xs = reinterpret_cast<float *>(lds_main);
    __shared__ float red[Gm::R * Gm::TR];
    __shared__ float rowsum[Gm::R];
    __shared__ float wsum[Gm::NT / 64];

    const int tid = threadIdx.x;
    const int ntiles = P.num_tiles();
    u32x4 pf[Gm::CPT];

    // Memory requests in issue order: the activations (needed first), then the first tile of
    // weights, then whatever the epilogue needs.  Loads retire in order, so waiting for the
    // activations leaves the weight tile in flight while the prologue runs.
    typename Policy::XRegs xr;
    P.x_issue(xr);
    int t = blockIdx.x;
    {
        // unconditional (no branch around the loads); the grid never exceeds the tile count
        const int t0 = t < ntiles ? t : ntiles - 1;
        gemv_fetch<Gm>(P, t0, pf);
        P.pre(t0);
    }
    // keeps the compiler from sinking the weight loads below the prologue
    asm volatile("" ::: "memory");
    PairX px;
    gemv_load_x<Gm>(P, xr, xs, wsum, px);

    for (; t < ntiles; t += gridDim.x) {
#pragma unroll
        for (int i = 0; i < Gm::CPT; ++i)
            tile[tid + i * Gm::NT] = pf[i];
        __syncthreads();
        if (t + (int)gridDim.x < ntiles) {
            gemv_fetch<Gm>(P, t + gridDim.x, pf);   // next tile's loads stay in flight during the compute
        }
        asm volatile("" ::: "memory");
        gemv_tile_rows<Gm>(tile, red, rowsum, px);
        P.epilogue(t, rowsum);
        if (t + (int)gridDim.x < ntiles)
            P.pre(t + gridDim.x);
    }
    P.finish(red);
}

// ---------------------------------------------------------------------------------------
// Prologues: stage the activation vector in LDS
// ---------------------------------------------------------------------------------------

// Activation staging in two halves: *_issue loads this thread's share of the vector into
// registers (fully unrolled, so every load is in flight at once), *_stage finishes the
// arithmetic and writes xs[K] in LDS.

// xs = x (a global fp32 vector of K values).
template <int NT, int K>
struct PlainX {
    static constexpr int PER = (K / 4 + NT - 1) / NT;
    f32x4 v[PER];

    static_assert((K / 4) % NT == 0, "the workgroup must cover the vector evenly");

    __device__ __forceinline__ void issue(const float *__restrict__ xg)
    {
        const f32x4 *src = reinterpret_cast<const f32x4 *>(xg);
#pragma unroll
        for (int j = 0; j < PER; ++j)
            v[j] = src[threadIdx.x + j * NT];
    }
    __device__ __forceinline__ float stage(float *xs)
    {
#pragma unroll
        for (int j = 0; j < PER; ++j)
            *reinterpret_cast<f32x4 *>(xs + xs_index(4 * (threadIdx.x + j * NT))) = v[j];
        __syncthreads();
        return 1.0f;
    }
};

// xs = RMSNorm(h) * gain: h / sqrt(mean(h^2) + eps) * gain, eps inside the root; the sum of
// squares is taken in a fixed order.
template <int NT, int K>
struct RmsNormX {
    static constexpr int PER = (K / 4 + NT - 1) / NT;
    f32x4 hv[PER], gv[PER];

    static_assert((K / 4) % NT == 0, "the workgroup must cover the vector evenly");

    __device__ __forceinline__ void issue(const float *__restrict__ h, const float *__restrict__ gain)
    {
        const f32x4 *h4 = reinterpret_cast<const f32x4 *>(h);
        const f32x4 *g4 = reinterpret_cast<const f32x4 *>(gain);
#pragma unroll
        for (int j = 0; j < PER; ++j) {
            hv[j] = h4[threadIdx.x + j * NT];
            gv[j] = g4[threadIdx.x + j * NT];
        }
    }
    // Stages h * gain; the normalisation 1/rms(h) is returned and applied to the row sums (the
    // product is linear in x), so one barrier publishes both the vector and the wave sums.
    __device__ __forceinline__ float stage(float *xs, float eps, float *wsum)
    {
        float ss = 0.0f;
#pragma unroll
        for (int j = 0; j < PER; ++j) {
            ss = fmaf(hv[j].x, hv[j].x, ss);
            ss = fmaf(hv[j].y, hv[j].y, ss);
            ss = fmaf(hv[j].z, hv[j].z, ss);
            ss = fmaf(hv[j].w, hv[j].w, ss);
        }
#pragma unroll
        for (int j = 0; j < PER; ++j)
            *reinterpret_cast<f32x4 *>(xs + xs_index(4 * (threadIdx.x + j * NT))) = hv[j] * gv[j];
        ss = wave_sum(ss);
        if ((threadIdx.x & 63) == 0)
            wsum[threadIdx.x >> 6] = ss;
        __syncthreads();
        float tot = 0.0f;
#pragma unroll
        for (int w = 0; w < NT / 64; ++w)
            tot += wsum[w];
        return 1.0f / sqrtf(tot / (float)K + eps);
    }
};

// Dequantise one block pair given as its 9 dwords into 64 floats: (code - 8) * d (exact).
__device__ __forceinline__ void dequant_pair_words(const uint32_t (&D)[9], float (&out)[64])
{
    const uint32_t q0[4] = {(D[0] >> 16) | (D[1] << 16), (D[1] >> 16) | (D[2] << 16),
                            (D[2] >> 16) | (D[3] << 16), (D[3] >> 16) | (D[4] << 16)};
    const float d0 = half_bits_to_float(D[0]);
    const float d1 = half_bits_to_float(D[4] >> 16);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            out[4 * i + j] = (float)((int)((q0[i] >> (8 * j)) & 15u) - 8) * d0;
            out[16 + 4 * i + j] = (float)((int)((q0[i] >> (8 * j + 4)) & 15u) - 8) * d0;
            out[32 + 4 * i + j] = (float)((int)((D[5 + i] >> (8 * j)) & 15u) - 8) * d1;
            out[48 + 4 * i + j] = (float)((int)((D[5 + i] >> (8 * j + 4)) & 15u) - 8) * d1;
        }
    }
}

}  // namespace vox
