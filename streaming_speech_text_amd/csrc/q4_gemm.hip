// q4_gemm.hip - encoder-chunk linear Y = X * W^T with GGUF Q4_0 weights on the matrix cores.
//
// Pages: the audio encoder is 1280 wide (voxtral.c page "Mistral Voxtral Realtime 4B 음성 인식
// 모델의 순수 C 기반 CPU 전용 추론 구현", GeekNews 26608, section 모델 아키텍처) and runs over chunks
// of frames (section 주요 기능); the quantised path keeps its linears as GGUF Q4_0 with
// dequantisation fused into the product (Rust port page, GeekNews 26595, section 아키텍처).
//
// Exactness: a dequantised weight (code - 8) * d needs up to 15 significant bits, more than
// bf16 holds, so the matrix cores never see it.  Each 32-input Q4_0 block is one
// v_mfma_f32_16x16x32_bf16 per 16 x 16 output block whose B operand holds exact small integers
// in bf16 and whose A operand holds the bf16 activations; the fp32 result is multiplied by the
// block's scale d and accumulated in fp32 on the vector units.
//
// Two kernels:
//  * small outputs: a workgroup of 8 waves owns a (16*MI) x (16*NJ) tile; the waves
//    split the K blocks into eight contiguous ranges, load their operands straight from memory
//    with GM_PF blocks in flight, and the eight partial tiles are added in LDS in wave order.
//    These are weight-streaming problems; splitting K over the waves puts requests in flight.
//    B holds (code - 8).  Lane group g (= lane / 16) takes code bytes 4g..4g+3, i.e. inputs
//    {4g..4g+3} (low nibbles) then {16+4g..16+4g+3} (high nibbles), and the activations of
//    the same inputs (the MFMA's k slots may hold the inputs in any order A and B agree on).
//  * longer chunks: the tiled kernel further down (64 x 64 tiles, weights staged through LDS),
//    optionally with K split over workgroups (partial tiles in the caller's workspace, added in
//    a fixed order by a second kernel).
//
// The adapter between encoder and decoder (voxtral.c page, section 모델 아키텍처: a linear from
// 5120 to 3072 inputs, GELU, a linear from 3072 to 3072) is two tiled products.  The first one's
// epilogue applies GELU (the exact x * Phi(x) form) in fp32 and stores each value as a pair of
// bf16 values (hi + lo, within 2^-18 of it); the second product reads the pairs as activations
// over a doubled K, every weight stage serving the hi and then the lo half.
#include <type_traits>

#include "vox_common.h"
#include "vox_host.h"

namespace vox {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4v __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2v __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));

constexpr int GM_WAVES = 8;
constexpr int GM_THREADS = 64 * GM_WAVES;
constexpr int GM_PF = 4;           // K blocks in flight per wave (5 when a wave has exactly 5)

// bf16 bits of two small integers given as exact fp32 values: the upper halves.
__device__ __forceinline__ uint32_t pack_bf16_pair(float lo, float hi)
{
    // bytes 2, 3 of lo then bytes 2, 3 of hi (one v_perm_b32)
    return __builtin_amdgcn_perm(__builtin_bit_cast(uint32_t, hi), __builtin_bit_cast(uint32_t, lo), 0x07060302u);
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

// GELU(v) = v * Phi(v) = v * erfc(-v / sqrt 2) / 2 in fp32, stored as hi = GELU(v) rounded to
// bf16 and lo = the (exact fp32) remainder rounded to bf16, so hi + lo is within 2^-18 |GELU(v)|.
// Layout: row `row` of hl is 2n values; column c of 128-input stage s = c / 128 puts hi at
// 256 s + c % 128 and lo 128 further, i.e. the stages of K alternate hi and lo halves.
constexpr int GELU_STAGE = 128;
__device__ __forceinline__ void store_gelu_pair(uint16_t *hl, int n, int64_t row, int col, float v)
{
    const float g = 0.5f * v * erfcf(-0.70710678118654752f * v);
    const __bf16 hi = (__bf16)g;
    const __bf16 lo = (__bf16)(g - (float)hi);
    uint16_t *p = hl + row * 2 * n + 2 * (col & ~(GELU_STAGE - 1)) + (col & (GELU_STAGE - 1));
    p[0] = __builtin_bit_cast(uint16_t, hi);
    p[GELU_STAGE] = __builtin_bit_cast(uint16_t, lo);
}

template <int MI, int NJ, int PF>
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
    u32x2v xa[PF][MI][2];
    uint32_t qv[PF][NJ], dv[PF][NJ];
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
    for (int s = 0; s < PF; ++s)
        load(s, kb0 + s);

    for (int b0 = kb0; b0 < kb1; b0 += PF) {
#pragma unroll
        for (int s = 0; s < PF; ++s) {
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
            load(s, b + PF);   // refill: the ring stays PF blocks ahead
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

// ---------------------------------------------------------------------------------------
// Tiled kernel for longer chunks (K of 1280, 3072 or 5120).  A workgroup of 4 waves owns a
// 64 x 64 tile of Y and walks K in stages of 4 Q4_0 blocks; in every stage wave w takes block w,
// so each wave computes the whole tile over a quarter of K and no operand is shared:
//  * the wave loads its A operands straight from memory two stages ahead: lane L's 16 bytes
//    of a 16-row block are row L % 16, inputs 8(L/16) .. 8(L/16)+7 of the Q4_0 block;
//  * the workgroup copies the stage's weight bytes (4 blocks = 72 contiguous, 8-byte aligned
//    bytes per row) to LDS with 8-byte loads; each wave then reads the bytes of its block
//    with aligned dword reads and unpacks the codes in registers to exact bf16: lane group g
//    of a column takes inputs 8g .. 8g+7, i.e. the low (g < 2) or high (g >= 2) nibbles of
//    code bytes 8(g%2) .. 8(g%2)+7;
//  * per block the wave runs 4 x 4 matrix-core products of A with the exact values
//    16 (code - 8), each 16 times the block's sum of a * (code - 8) up to fp32 rounding (the
//    factor 16 is exact and commutes with every rounding while the sums stay below 2^124 in
//    magnitude, i.e. for every output short of the top 1/16 of the fp32 range); scale * product
//    goes into fp32, and the epilogue multiplies the tile by 1/16.
// The four waves' partial tiles are added through LDS in a fixed tree order at the end.  Two
// workgroups share a compute unit (at most 256 VGPRs per wave), so one's stage barrier overlaps
// the other's work (measured on MI355X against eight-wave workgroups with 8-block stages, one
// per compute unit: the encoder linear sets 6 % faster at 64-750 frames).
// ---------------------------------------------------------------------------------------
constexpr int GT_BM = 64, GT_BN = 64, GT_KC = 4, GT_THREADS = 256;
constexpr int GT_STAGE = GT_KC * 32;                        // inputs per stage
constexpr int GT_WAVES = GT_THREADS / 64;
constexpr int GT_RAW = GT_KC * 18;                          // weight bytes of one row per stage
constexpr int GT_WB = 8;                                    // bytes per weight piece (72 = 9 x 8)
constexpr int GT_W_CHUNKS = GT_BN * GT_RAW / GT_WB;         // weight pieces per stage
constexpr int GT_WR = (GT_W_CHUNKS + GT_THREADS - 1) / GT_THREADS;   // load rounds per stage
static_assert(GT_RAW % GT_WB == 0, "a row's stage bytes split into whole pieces");
static_assert(GT_KC == GT_THREADS / 64, "one block per wave per stage");
static_assert(GELU_STAGE == GT_STAGE, "a GELU pair stage is one weight stage of the second product");

// Byte j of v as a float (one v_cvt_f32_ubyte{j}).
__device__ __forceinline__ float ubyte_to_f(uint32_t v, int j)
{
    float r;
    switch (j) {
    case 0: asm("v_cvt_f32_ubyte0 %0, %1" : "=v"(r) : "v"(v)); break;
    case 1: asm("v_cvt_f32_ubyte1 %0, %1" : "=v"(r) : "v"(v)); break;
    case 2: asm("v_cvt_f32_ubyte2 %0, %1" : "=v"(r) : "v"(v)); break;
    default: asm("v_cvt_f32_ubyte3 %0, %1" : "=v"(r) : "v"(v)); break;
    }
    return r;
}

// 16 (code - 8) for 8 codes taken from one nibble of 8 bytes (lo: bytes 0-3, hi: 4-7), exact in
// bf16.  sh = 4 moves low nibbles to the top of their bytes (high nibbles: sh = 0); flipping the
// top bit then leaves a byte that, read as a signed integer, is 16 (code - 8), because code ^ 8 is
// code - 8 as a 4-bit two's complement number.  One sign-extending byte conversion per value.
// (Feeding the raw codes and adding -8 times the activations' block sum through the accumulator
// saves more but cancels two sums of size 8 sum|a|: measured on MI355X, no faster, and its
// rounding shows where the weights are sparse.)
__device__ __forceinline__ u32x4v nibbles_to_bf16_x16(uint32_t lo, uint32_t hi, uint32_t sh)
{
    const uint32_t a = ((lo << sh) & 0xF0F0F0F0u) ^ 0x80808080u;
    const uint32_t b = ((hi << sh) & 0xF0F0F0F0u) ^ 0x80808080u;
    u32x4v p;
    p.x = pack_bf16_pair((float)(int8_t)a, (float)(int8_t)(a >> 8));
    p.y = pack_bf16_pair((float)(int8_t)(a >> 16), (float)(int8_t)(a >> 24));
    p.z = pack_bf16_pair((float)(int8_t)b, (float)(int8_t)(b >> 8));
    p.w = pack_bf16_pair((float)(int8_t)(b >> 16), (float)(int8_t)(b >> 24));
    return p;
}

// Reads the bytes of block `blk` (0..GT_KC-1 of the stage) of the four 16-column blocks from the
// raw stage copy (GT_RAW bytes per row) with aligned dword reads and unpacks this lane's operand
// (column 16j + l16, inputs 8*grp .. 8*grp+7) and scale.  ODD: blk is odd, so the block starts
// at 2 mod 4 and its code bytes are 4-aligned; otherwise the block is 4-aligned and the code
// bytes are 2 mod 4.
template <bool ODD>
__device__ __forceinline__ void unpack_b(const uint32_t *raw, int blk, int l16, int grp, bf16x8 (&bf)[4],
                                         float (&d)[4])
{
    uint32_t dw[4][4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const uint32_t *p = raw + (((16 * j + l16) * GT_RAW + 18 * blk) >> 2);
        if constexpr (ODD) {
            const uint32_t *q = p + 1 + 2 * (grp & 1);
            dw[j][0] = p[0];
            dw[j][1] = q[0];
            dw[j][2] = q[1];
        } else {
            const uint32_t *q = p + 2 * (grp & 1);
            dw[j][0] = p[0];
            dw[j][1] = q[0];
            dw[j][2] = q[1];
            dw[j][3] = q[2];
        }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        uint32_t d16, lo, hi;
        if constexpr (ODD) {
            d16 = dw[j][0] >> 16;
            lo = dw[j][1];
            hi = dw[j][2];
        } else {
            d16 = dw[j][0] & 0xFFFFu;
            lo = __builtin_amdgcn_alignbyte(dw[j][2], dw[j][1], 2);
            hi = __builtin_amdgcn_alignbyte(dw[j][3], dw[j][2], 2);
        }
        bf[j] = __builtin_bit_cast(bf16x8, nibbles_to_bf16_x16(lo, hi, grp >= 2 ? 0u : 4u));
        float df = half_bits_to_float(d16);
        asm volatile("" : "+v"(df));   // an fp32 scale, so the multiply-adds are v_fmac_f32, not v_fma_mix_f32
        d[j] = df;
    }
}

// Modes of the tiled kernel (compile-time, so the plain product carries no code of the others):
//  T_PLAIN      fp32 output y;
//  T_GELU_OUT   the unsplit output goes through GELU into hl as store_gelu_pair lays it out;
//  T_PAIR_IN    the activations are GELU pairs (row length k = 2 x the weights' K): stage st
//               reads weight stage st / 2, so each weight stage serves its hi and lo halves.
enum { T_PLAIN = 0, T_GELU_OUT = 1, T_PAIR_IN = 2 };

// NS: stages (of GT_STAGE inputs) per workgroup, fixed at compile time.  Workgroup z of the grid's
// third dimension takes stages z*NS .. z*NS+NS-1; with one slice it writes the output itself,
// otherwise its fp32 partial tile goes to part[z][m][n] and q4_gemm_reduce_kernel adds the
// slices.  k is the activations' row length.
template <int NS, int MODE>
__global__ __launch_bounds__(GT_THREADS) __attribute__((amdgpu_waves_per_eu(2))) void q4_gemm_tiled_kernel(const uint8_t *__restrict__ w,
                                                                   const uint16_t *__restrict__ x,
                                                                   float *__restrict__ y, uint16_t *__restrict__ hl,
                                                                   float *__restrict__ part, int m, int n, int k)
{
    __shared__ __attribute__((aligned(16))) uint32_t braw[2][GT_BN * GT_RAW / 4];
    __shared__ f32x4v red[GT_WAVES / 2][16][64];   // tree reduction of the waves' tiles

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int l16 = lane & 15, grp = lane >> 4;
    const int m0 = blockIdx.y * GT_BM;
    const int n0 = blockIdx.x * GT_BN;
    const int st0 = blockIdx.z * NS, st_end = st0 + NS;
    constexpr int KWS = MODE == T_PAIR_IN ? 1 : 0;   // weight stage = activation stage >> KWS
    const uint32_t row_bytes = (uint32_t)((k >> KWS) / 32) * 18;

    // A operands of this lane: rows m0 + 16i + l16 (clamped), inputs 8*grp .. of block `wave`
    uint32_t aoff[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
        aoff[i] = (uint32_t)min(m0 + 16 * i + l16, m - 1) * (uint32_t)k + (uint32_t)(32 * wave + 8 * grp);
    // weight pieces: chunk c -> row c / (GT_RAW / GT_WB) of the tile, piece c % (GT_RAW / GT_WB);
    // rounds past the last chunk are clamped to it (a duplicate load and an identical LDS store)
    uint32_t woff[GT_WR];
    int wlds[GT_WR];
#pragma unroll
    for (int r = 0; r < GT_WR; ++r) {
        const int c = min(tid + GT_THREADS * r, GT_W_CHUNKS - 1);
        const int col = min(n0 + c / (GT_RAW / GT_WB), n - 1);
        woff[r] = (uint32_t)col * row_bytes + (uint32_t)(GT_WB * (c % (GT_RAW / GT_WB)));
        wlds[r] = (GT_WB / 4) * c;
    }

    // two stages of loads in flight: register slots 0 and 1 (compile-time indices)
    u32x4v ar[2][4];
    u32x2v wr[2][GT_WR];
    auto load_stage = [&](int st, auto slot) {
        constexpr int S = decltype(slot)::value;
        st = min(st, st_end - 1);   // past the slice: a harmless reload of its last stage
        const uint16_t *xs = x + (size_t)st * GT_STAGE;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            ar[S][i] = *reinterpret_cast<const u32x4v *>(xs + aoff[i]);
        const uint8_t *ws = w + (size_t)(st >> KWS) * GT_RAW;
#pragma unroll
        for (int r = 0; r < GT_WR; ++r)
            wr[S][r] = *reinterpret_cast<const u32x2v *>(ws + woff[r]);
    };

    f32x4v acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
            acc[i][j] = 0.0f;

    auto stage = [&](int st, auto slot) {
        constexpr int S = decltype(slot)::value;
        const int b = st & 1;
#pragma unroll
        for (int r = 0; r < GT_WR; ++r)
            *reinterpret_cast<u32x2v *>(&braw[b][wlds[r]]) = wr[S][r];
        bf16x8 af[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            af[i] = __builtin_bit_cast(bf16x8, ar[S][i]);
        __syncthreads();   // braw[b] complete; braw[b] is next written two stages later
        // B operands of block `wave` for the four 16-column blocks.  The block of column c
        // starts at byte o = c*GT_RAW + 18*wave: 4-aligned for even waves, 2 mod 4 for odd ones
        // (the parity is uniform over a wave, so each wave runs one straight-line path).
        bf16x8 bf[4];
        float d[4];
        if ((wave & 1) == 0)
            unpack_b<false>(&braw[b][0], wave, l16, grp, bf, d);
        else
            unpack_b<true>(&braw[b][0], wave, l16, grp, bf, d);
        // products in two rounds of 8 with independent result registers, then the scaled sums
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            f32x4v t[2][4];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    t[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[2 * h + i], bf[j], (f32x4v)0.0f, 0, 0, 0);
            }
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[2 * h + i][j] += d[j] * t[i][j];
        }
        load_stage(st + 2, slot);   // after the products, so the slot's registers are free
    };
    typedef std::integral_constant<int, 0> S0;
    typedef std::integral_constant<int, 1> S1;
    load_stage(st0, S0());
    load_stage(st0 + 1, S1());
    for (int r = 0; r + 1 < NS; r += 2) {
        stage(st0 + r, S0());
        stage(st0 + r + 1, S1());
    }
    if constexpr (NS % 2)
        stage(st_end - 1, S0());

    // tree: (w + half) -> w for half = waves/2 .. 1; fixed order
#pragma unroll
    for (int half = GT_WAVES / 2; half >= 1; half >>= 1) {
        if (wave >= half && wave < 2 * half) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    red[wave - half][i * 4 + j][lane] = acc[i][j];
        }
        __syncthreads();
        if (wave < half) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] += red[wave][i * 4 + j][lane];
        }
        __syncthreads();
    }
    if (wave == 0) {
        const bool gelu = MODE == T_GELU_OUT && !part;   // uniform over the workgroup
        float *const dst = part ? part + (size_t)blockIdx.z * m * n : y;
        // D layout of a 16x16 block: lane holds rows 4*(lane/16) .. +3 of column lane%16
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int col = n0 + 16 * j + l16;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int row = m0 + 16 * i + 4 * grp + r;
                    if (row < m && col < n) {
                        const float yv = acc[i][j][r] * 0.0625f;   // the B operands were 16 (code - 8)
                        if (gelu)
                            store_gelu_pair(hl, n, row, col, yv);
                        else
                            dst[(size_t)row * n + col] = yv;
                    }
                }
            }
    }
}

// y = sum over z of part[z] (count values per slice, rows of n), slices added in order z = 0, 1,
// ...; GELU: GELU pairs of the sums go to hl instead (store_gelu_pair).
template <bool GELU, int NB>
__global__ __launch_bounds__(256) void q4_gemm_reduce_kernel(const float *__restrict__ part, float *__restrict__ y,
                                                             uint16_t *__restrict__ hl, int64_t count, int n,
                                                             int slices, bool vec4)
{
    // NB > 0 (at least the slice count): every slice's load is issued before the first add, so
    // the kernel waits for one memory round trip; NB = 0: one load after another.
    auto sum = [&](auto ld) {
        auto a = ld(0);
        if constexpr (NB > 0) {
            decltype(a) v[NB];
#pragma unroll
            for (int z = 1; z < NB; ++z)
                v[z] = ld(z < slices ? z : 0);
#pragma unroll
            for (int z = 1; z < NB; ++z)
                if (z < slices)
                    a += v[z];
        } else {
            for (int z = 1; z < slices; ++z)
                a += ld(z);
        }
        return a;
    };
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (vec4) {
        const int64_t i = 4 * t;
        if (i >= count)
            return;
        const f32x4v a = sum([&](int z) { return *reinterpret_cast<const f32x4v *>(part + (size_t)z * count + i); });
        if constexpr (GELU) {
            const int64_t row = i / n;
            const int col = (int)(i - row * n);
#pragma unroll
            for (int e = 0; e < 4; ++e)
                store_gelu_pair(hl, n, row, col + e, a[e]);
        } else {
            *reinterpret_cast<f32x4v *>(y + i) = a;
        }
    } else {
        if (t >= count)
            return;
        const float a = sum([&](int z) { return part[(size_t)z * count + t]; });
        if constexpr (GELU)
            store_gelu_pair(hl, n, t / n, (int)(t % n), a);
        else
            y[t] = a;
    }
}

// K values with a compiled stage sequence (the encoder's widths and the decoder's)
static bool tiled_k(int64_t k) { return k == 1280 || k == 3072 || k == 5120; }

// Whether the tiled kernel runs (given 16-byte aligned operands): a compiled K, offsets that fit
// 32 bits, and either a long K or an output past 64 x 1280 values (K = 1280) or 48 x 1280 (K =
// 3072) - measured on MI355X at the encoder's shapes, the split-K-over-waves kernel is the faster
// one below that (at K = 1280 with all five blocks of a wave in flight: 16 x 5120 and 64 x 1280
// outputs 9.1 / 8.7 us against 10.0 / 9.5 tiled, 64 x 5120 19.1 against 12.4).
static bool tiled_shape(int64_t m, int64_t n, int64_t k)
{
    const size_t wbytes = (size_t)n * (size_t)(k / 32) * 18;
    return tiled_k(k) && (uint64_t)m * (uint64_t)k < (1ull << 31) && wbytes < (1ull << 31) &&
           (k >= 5120 || m * n > (k == 1280 ? 64 : 48) * 1280);
}

// K slices for the tiled kernel (measured on MI355X at the encoder's shapes): none once the
// output tiles alone give 160 workgroups, else the fewest slices (dividing the stages, at least
// two stages each) that reach 160 workgroups, else the most (320 or 512 workgroups was slower).
// The slices' partial tiles are added by q4_gemm_reduce_kernel.
constexpr int GT_TARGET_WGS = 160;
static int tiled_slices(int64_t m, int64_t n, int64_t k)
{
    const int64_t tiles = ((n + GT_BN - 1) / GT_BN) * ((m + GT_BM - 1) / GT_BM);
    const int nst = (int)(k / GT_STAGE);
    if (tiles >= GT_TARGET_WGS)
        return 1;
    int most = 1;
    for (int ks = 2; 2 * ks <= nst; ++ks)
        if (nst % ks == 0) {
            if (tiles * ks >= GT_TARGET_WGS)
                return ks;
            most = ks;
        }
    return most;
}

static size_t tiled_workspace(int64_t m, int64_t n, int slices)
{
    return slices > 1 ? (size_t)slices * (size_t)m * (size_t)n * sizeof(float) : 0;
}

template <int S, int MODE>
static void launch_tiled_slices(const void *w, const uint16_t *x, float *y, uint16_t *hl, float *part, int m, int n,
                                int k, int slices, hipStream_t s)
{
    const dim3 grid((unsigned)((n + GT_BN - 1) / GT_BN), (unsigned)((m + GT_BM - 1) / GT_BM), (unsigned)slices);
    hipLaunchKernelGGL((q4_gemm_tiled_kernel<S, MODE>), grid, dim3(GT_THREADS), 0, s, (const uint8_t *)w, x, y, hl,
                       part, m, n, k);
}

// Output: y (fp32), or for T_GELU_OUT GELU pairs in hl (n a multiple of 256).  part: slices x m x n
// floats when slices > 1, else null (the kernel then writes the output itself).  k: the
// activations' row length.
template <int MODE>
static int launch_gemm_tiled(const void *w, const uint16_t *x, float *y, uint16_t *hl, float *part, int m, int n,
                             int k, int slices, hipStream_t s)
{
    constexpr bool gelu = MODE == T_GELU_OUT;
    if ((slices > 1) != (part != nullptr) || (gelu ? (hl == nullptr || n % GELU_STAGE) : y == nullptr))
        return fail(VOX_E_INVAL, "q4 tiled product: one output, and a partial-tile buffer exactly when K is split");
    switch ((k / GT_STAGE) / slices) {   // stages per workgroup
    case 48: launch_tiled_slices<48, MODE>(w, x, y, hl, part, m, n, k, slices, s); break;
    case 40: launch_tiled_slices<40, MODE>(w, x, y, hl, part, m, n, k, slices, s); break;
    case 24: launch_tiled_slices<24, MODE>(w, x, y, hl, part, m, n, k, slices, s); break;
    case 16: launch_tiled_slices<16, MODE>(w, x, y, hl, part, m, n, k, slices, s); break;
    case 20: launch_tiled_slices<20, MODE>(w, x, y, hl, part, m, n, k, slices, s); break;
    case 12: launch_tiled_slices<12, MODE>(w, x, y, hl, part, m, n, k, slices, s); break;
    case 10: launch_tiled_slices<10, MODE>(w, x, y, hl, part, m, n, k, slices, s); break;
    case 8: launch_tiled_slices<8, MODE>(w, x, y, hl, part, m, n, k, slices, s); break;
    case 6: launch_tiled_slices<6, MODE>(w, x, y, hl, part, m, n, k, slices, s); break;
    case 5: launch_tiled_slices<5, MODE>(w, x, y, hl, part, m, n, k, slices, s); break;
    case 4: launch_tiled_slices<4, MODE>(w, x, y, hl, part, m, n, k, slices, s); break;
    case 3: launch_tiled_slices<3, MODE>(w, x, y, hl, part, m, n, k, slices, s); break;
    case 2: launch_tiled_slices<2, MODE>(w, x, y, hl, part, m, n, k, slices, s); break;
    case 1: launch_tiled_slices<1, MODE>(w, x, y, hl, part, m, n, k, slices, s); break;
    default: return fail(VOX_E_UNSUPPORTED, "q4 tiled product: no compiled stage count for k=%d in %d slices", k, slices);
    }
    int st = check_launch("q4 tiled product");
    if (st || slices == 1)
        return st;
    const int64_t count = (int64_t)m * n;
    const bool vec4 = count % 4 == 0 && (gelu ? n % 4 == 0 : aligned(y, 16));
    const int64_t threads = vec4 ? count / 4 : count;
    const dim3 rg((unsigned)((threads + 255) / 256));
    if (slices <= 2)
        hipLaunchKernelGGL((q4_gemm_reduce_kernel<gelu, 2>), rg, dim3(256), 0, s, part, y, hl, count, n, slices, vec4);
    else if (slices <= 4)
        hipLaunchKernelGGL((q4_gemm_reduce_kernel<gelu, 4>), rg, dim3(256), 0, s, part, y, hl, count, n, slices, vec4);
    else if (slices <= 8)
        hipLaunchKernelGGL((q4_gemm_reduce_kernel<gelu, 8>), rg, dim3(256), 0, s, part, y, hl, count, n, slices, vec4);
    else
        hipLaunchKernelGGL((q4_gemm_reduce_kernel<gelu, 0>), rg, dim3(256), 0, s, part, y, hl, count, n, slices, vec4);
    return check_launch("q4 tiled product: slice sum");
}

// Blocks in flight per wave: all of them when a wave has exactly five (K = 1280: the whole range
// in one memory round trip; measured on MI355X, 16 x 1280 x 1280 took 5.5 us against 7.4 with
// four), else four (five or eight for longer ranges was slower, e.g. 16 x 3072 x 3072: 15.6 us
// against 13.0).
template <int MI, int NJ>
static int launch_gemm(const void *w, const uint16_t *x, float *y, int m, int n, int k, hipStream_t s)
{
    const dim3 grid((unsigned)((n + 16 * NJ - 1) / (16 * NJ)), (unsigned)((m + 16 * MI - 1) / (16 * MI)));
    const int per_wave = (k / 32 + GM_WAVES - 1) / GM_WAVES;
    if (per_wave == 5)
        hipLaunchKernelGGL((q4_gemm_kernel<MI, NJ, 5>), grid, dim3(GM_THREADS), 0, s, (const uint8_t *)w, x, y, m, n, k);
    else
        hipLaunchKernelGGL((q4_gemm_kernel<MI, NJ, GM_PF>), grid, dim3(GM_THREADS), 0, s, (const uint8_t *)w, x, y, m, n,
                           k);
    return check_launch("vox_q4_gemm");
}

}  // namespace vox

using namespace vox;

extern "C" size_t vox_q4_gemm_workspace(int64_t m, int64_t n, int64_t k)
{
    if (m <= 0 || n <= 0 || k <= 0 || k % 32 || m > 65535 * 16 || n > (1 << 24) || k > (1 << 24) ||
        !tiled_shape(m, n, k))
        return 0;
    return tiled_workspace(m, n, tiled_slices(m, n, k));
}

extern "C" int vox_q4_gemm(const void *w_q4, const uint16_t *x_bf16, float *y, int64_t m, int64_t n, int64_t k,
                           void *workspace, size_t workspace_bytes, void *stream)
{
    if (m < 0 || n < 0 || k <= 0 || k % 32)
        return fail(VOX_E_INVAL, "vox_q4_gemm: need m, n >= 0 and k a positive multiple of 32 (m=%lld n=%lld k=%lld)",
                    (long long)m, (long long)n, (long long)k);
    if (m == 0 || n == 0)
        return ok();
    if (!w_q4 || !x_bf16 || !y)
        return fail(VOX_E_INVAL, "vox_q4_gemm: null pointer");
    if (m > 65535 * 16 || n > (1 << 24) || k > (1 << 24))   // grid rows: m / 16 <= 65535
        return fail(VOX_E_UNSUPPORTED, "vox_q4_gemm: dimension too large (m <= 1048560, n, k <= 2^24)");
    if (!aligned(x_bf16, 8) || !aligned(w_q4, 2))
        return fail(VOX_E_UNSUPPORTED, "vox_q4_gemm: x must be 8-byte and w 2-byte aligned");
    const size_t wbytes = (size_t)n * (size_t)(k / 32) * 18, xbytes = (size_t)m * k * 2, ybytes = (size_t)m * n * 4;
    if (overlaps(y, ybytes, x_bf16, xbytes) || overlaps(y, ybytes, w_q4, wbytes))
        return fail(VOX_E_INVAL, "vox_q4_gemm: y overlaps an input");
    if (!workspace != !workspace_bytes)
        return fail(VOX_E_INVAL, "vox_q4_gemm: workspace and workspace_bytes must be both set or both zero");
    hipStream_t s = (hipStream_t)stream;
    int st;
    if (aligned(x_bf16, 16) && aligned(w_q4, 16) && tiled_shape(m, n, k)) {
        int slices = workspace ? tiled_slices(m, n, k) : 1;
        const size_t need = tiled_workspace(m, n, slices);
        if (need > workspace_bytes)
            return fail(VOX_E_WORKSPACE, "vox_q4_gemm: workspace of %zu bytes, need %zu", workspace_bytes, need);
        if (need && (!aligned(workspace, 16) || overlaps(workspace, need, y, ybytes) ||
                     overlaps(workspace, need, x_bf16, xbytes) || overlaps(workspace, need, w_q4, wbytes)))
            return fail(VOX_E_INVAL, "vox_q4_gemm: workspace must be 16-byte aligned and apart from x, y and w");
        // the partial tiles go to the workspace only when K is split; one slice writes y
        st = launch_gemm_tiled<T_PLAIN>(w_q4, x_bf16, y, nullptr, slices > 1 ? (float *)workspace : nullptr, (int)m,
                                        (int)n, (int)k, slices, s);
    } else {
        st = launch_gemm<1, 1>(w_q4, x_bf16, y, (int)m, (int)n, (int)k, s);
    }
    return st ? st : ok();
}


// ---------------------------------------------------------------------------------------
// Adapter: Y = GELU(X W1^T) W2^T.  Workspace: the GELU pairs H [m][2 n_mid] bf16 (rounded up to
// 256 bytes), then the partial tiles of whichever product splits K (the two products run one
// after the other on the stream, so they share that region).
// ---------------------------------------------------------------------------------------
namespace vox {

static size_t adapter_h_bytes(int64_t m, int64_t n_mid)
{
    return ((size_t)m * (size_t)n_mid * 4 + 255) & ~(size_t)255;
}

static size_t adapter_part_bytes(int64_t m, int64_t k, int64_t n_mid, int64_t n_out)
{
    const size_t a = tiled_workspace(m, n_mid, tiled_slices(m, n_mid, k));
    const size_t b = tiled_workspace(m, n_out, tiled_slices(m, n_out, 2 * n_mid));
    return a > b ? a : b;
}

// shapes the adapter runs: compiled stage sequences for K = k and 2 n_mid, 32-bit operand
// offsets, grid rows
static bool adapter_shape(int64_t m, int64_t k, int64_t n_mid, int64_t n_out)
{
    return tiled_k(k) && (n_mid == 1280 || n_mid == 3072) && m <= 65535LL * GT_BM && n_out <= (1 << 24) &&
           (uint64_t)m * (uint64_t)k < (1ull << 31) && (uint64_t)m * (uint64_t)(2 * n_mid) < (1ull << 31) &&
           (uint64_t)n_out * (uint64_t)(n_mid / 32) * 18 < (1ull << 31);
}

}  // namespace vox

extern "C" size_t vox_adapter_workspace(int64_t m, int64_t k, int64_t n_mid, int64_t n_out)
{
    if (m <= 0 || n_out <= 0 || !adapter_shape(m, k, n_mid, n_out))
        return 0;
    return adapter_h_bytes(m, n_mid) + adapter_part_bytes(m, k, n_mid, n_out);
}

extern "C" int vox_adapter(const void *w1_q4, const void *w2_q4, const uint16_t *x_bf16, float *y, int64_t m,
                           int64_t k, int64_t n_mid, int64_t n_out, void *workspace, size_t workspace_bytes,
                           void *stream)
{
    if (m < 0 || n_out < 0 || k <= 0 || k % 32 || n_mid <= 0 || n_mid % 32)
        return fail(VOX_E_INVAL,
                    "vox_adapter: need m, n_out >= 0 and k, n_mid positive multiples of 32 (m=%lld k=%lld n_mid=%lld "
                    "n_out=%lld)",
                    (long long)m, (long long)k, (long long)n_mid, (long long)n_out);
    if (m == 0 || n_out == 0)
        return ok();
    if (!adapter_shape(m, k, n_mid, n_out))
        return fail(VOX_E_UNSUPPORTED,
                    "vox_adapter: k must be 1280, 3072 or 5120, n_mid 1280 or 3072, and the operands within 2^31 "
                    "elements (k=%lld n_mid=%lld m=%lld)",
                    (long long)k, (long long)n_mid, (long long)m);
    if (!w1_q4 || !w2_q4 || !x_bf16 || !y || !workspace)
        return fail(VOX_E_INVAL, "vox_adapter: null pointer");
    if (!aligned(x_bf16, 16) || !aligned(w1_q4, 16) || !aligned(w2_q4, 16))
        return fail(VOX_E_UNSUPPORTED, "vox_adapter: x, w1 and w2 must be 16-byte aligned");
    const size_t need = vox_adapter_workspace(m, k, n_mid, n_out);
    if (workspace_bytes < need)
        return fail(VOX_E_WORKSPACE, "vox_adapter: workspace of %zu bytes, need %zu", workspace_bytes, need);
    const size_t xbytes = (size_t)m * k * 2, ybytes = (size_t)m * n_out * 4;
    const size_t w1bytes = (size_t)n_mid * (k / 32) * 18, w2bytes = (size_t)n_out * (n_mid / 32) * 18;
    if (!aligned(workspace, 16) || overlaps(workspace, need, x_bf16, xbytes) || overlaps(workspace, need, y, ybytes) ||
        overlaps(workspace, need, w1_q4, w1bytes) || overlaps(workspace, need, w2_q4, w2bytes))
        return fail(VOX_E_INVAL, "vox_adapter: workspace must be 16-byte aligned and apart from x, y and the weights");
    if (overlaps(y, ybytes, x_bf16, xbytes) || overlaps(y, ybytes, w1_q4, w1bytes) || overlaps(y, ybytes, w2_q4, w2bytes))
        return fail(VOX_E_INVAL, "vox_adapter: y overlaps an input");
    hipStream_t s = (hipStream_t)stream;
    uint16_t *h = (uint16_t *)workspace;
    float *part = (float *)((char *)workspace + adapter_h_bytes(m, n_mid));
    const int s1 = tiled_slices(m, n_mid, k), s2 = tiled_slices(m, n_out, 2 * n_mid);
    int st = launch_gemm_tiled<T_GELU_OUT>(w1_q4, x_bf16, nullptr, h, s1 > 1 ? part : nullptr, (int)m, (int)n_mid,
                                           (int)k, s1, s);
    if (!st)
        st = launch_gemm_tiled<T_PAIR_IN>(w2_q4, h, y, nullptr, s2 > 1 ? part : nullptr, (int)m, (int)n_out,
                                          (int)(2 * n_mid), s2, s);
    return st ? st : ok();
}
