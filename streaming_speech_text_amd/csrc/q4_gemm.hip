// q4_gemm.hip - encoder-chunk linear Y = X * W^T with GGUF Q4_0 weights on the matrix cores.
//
// Pages: the audio encoder is 1280 wide (voxtral.c page "Mistral Voxtral Realtime 4B 음성 인식
// 모델의 순수 C 기반 CPU 전용 추론 구현", GeekNews 26608, section 모델 아키텍처) and runs over chunks
// of frames (section 주요 기능); the quantised path keeps its linears as GGUF Q4_0 with
// dequantisation fused into the product (Rust port page, GeekNews 26595, section 아키텍처).
//
// Exactness: a dequantised weight (code - 8) * d needs up to 15 significant bits, more than
// bf16 holds, so the matrix cores never see it.  Each 32-input Q4_0 block is one product per
// output block (v_mfma_f32_16x16x32_bf16, or two v_mfma_f32_32x32x16_bf16 in the wide product)
// whose B operand holds exact small integers in bf16 and whose A operand holds the bf16
// activations; the fp32 result is multiplied by the block's scale d and accumulated in fp32 on
// the vector units.
//
// Four products:
//  * small outputs: a workgroup of 8 waves owns a (16*MI) x (16*NJ) tile; the waves
//    split the K blocks into eight contiguous ranges, load their operands straight from memory
//    with GM_PF blocks in flight, and the eight partial tiles are added in LDS in wave order.
//    These are weight-streaming problems; splitting K over the waves puts requests in flight.
//    B holds (code - 8).  Lane group g (= lane / 16) takes code bytes 4g..4g+3, i.e. inputs
//    {4g..4g+3} (low nibbles) then {16+4g..16+4g+3} (high nibbles), and the activations of
//    the same inputs (the MFMA's k slots may hold the inputs in any order A and B agree on).
//  * at most 64 rows at K = 1280 or 3072, 16 at K = 5120: the skinny kernel (16 x 16 tiles whose
//    weights for the whole of K are staged through LDS in one round trip, the same per-block
//    products);
//  * longer chunks: the tiled kernel further down (64 x 64 tiles, weights staged through LDS),
//    optionally with K split over workgroups (partial tiles in the caller's workspace, added in
//    a fixed order by a second kernel).
//  * long chunks: the wide product (128 x 128 tiles on v_mfma_f32_32x32x16_bf16, the same
//    exact operands and per-block scale), K split over the grid where its tiles are too few.
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

// Modes of the tiled and skinny kernels (compile-time, so the plain product carries no code of the others):
//  T_PLAIN      fp32 output y;
//  T_GELU_OUT   the unsplit output goes through GELU into hl as store_gelu_pair lays it out;
//  T_PAIR_IN    the activations are GELU pairs (row length k = 2 x the weights' K): stage st
//               reads weight stage st / 2, so each weight stage serves its hi and lo halves.
enum { T_PLAIN = 0, T_GELU_OUT = 1, T_PAIR_IN = 2 };

// WAVES: waves splitting K.  (Sixteen waves with all ten blocks of each in flight for 16 x 1280 x
// 5120 were measured on MI355X at 19.3 us against 13 us for the tiled kernel and its slice sum:
// the lanes' 4-byte pieces of 16 weight rows make every load touch 16 cache lines.)
template <int MI, int NJ, int PF, int WAVES = GM_WAVES>
__global__ __launch_bounds__(64 * WAVES) void q4_gemm_kernel(const uint8_t *__restrict__ w,
                                                            const uint16_t *__restrict__ x, float *__restrict__ y,
                                                            int m, int n, int k)
{
    __shared__ float red[WAVES][MI * NJ][4][64];

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int grp = lane >> 4;
    const int l16 = lane & 15;
    const int n0 = blockIdx.x * 16 * NJ;
    const int m0 = blockIdx.y * 16 * MI;
    const int nb = k / 32;
    const size_t row_bytes = (size_t)nb * 18;
    const int kb0 = (int)((int64_t)wave * nb / WAVES);
    const int kb1 = (int)((int64_t)(wave + 1) * nb / WAVES);

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

    // one pass over the PF blocks of the ring starting at block b0; REFILL: load the blocks PF
    // further into the slots as they are consumed (the ring stays PF blocks ahead)
    auto ring_pass = [&](int b0, auto refill) {
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
            if constexpr (decltype(refill)::value)
                load(s, b + PF);
#pragma unroll
            for (int i = 0; i < MI; ++i)
#pragma unroll
                for (int j = 0; j < NJ; ++j) {
                    const f32x4v t = __builtin_amdgcn_mfma_f32_16x16x32_bf16(afr[i], bfr[j], (f32x4v)0.0f, 0, 0, 0);
                    acc[i][j] += d[j] * t;
                }
        }
    };
    // every pass but the last refills; the last one issues no loads (a wave whose range holds at
    // most PF blocks, e.g. K = 1280 with PF = 5, loads each block once)
    int b0 = kb0;
    for (; b0 + PF < kb1; b0 += PF)
        ring_pass(b0, std::true_type{});
    if (b0 < kb1)
        ring_pass(b0, std::false_type{});

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
    for (int e = tid; e < MI * NJ * 4 * 64; e += 64 * WAVES) {
        const int ln = e & 63, r = (e >> 6) & 3, blk = e >> 8;
        const int i = blk / NJ, j = blk % NJ;
        float v = red[0][blk][r][ln];
#pragma unroll
        for (int wv = 1; wv < WAVES; ++wv)
            v += red[wv][blk][r][ln];
        const int row = m0 + 16 * i + 4 * (ln >> 4) + r;
        const int col = n0 + 16 * j + (ln & 15);
        if (row < m && col < n)
            y[(size_t)row * n + col] = v;
    }
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

// ---------------------------------------------------------------------------------------
// Skinny products (16-row tiles of up to 64 rows of X, K of 1280, 3072 or 5120): one workgroup of 8
// waves per 16 columns and 16 rows of Y.  The workgroup copies its 16 weight rows for the whole of K into LDS with
// coalesced 16-byte loads (one memory round trip, at most 46 KB), while each wave loads the
// activations of its eighth of K straight into registers, one 16-byte load per block and lane
// (row L % 16, inputs 8(L/16) .. 8(L/16)+7: a wave's load covers 64 contiguous bytes of each of
// the 16 rows); then every wave unpacks its blocks from LDS to the exact values 16 (code - 8)
// (lane group g: the low (g < 2) or high (g >= 2) nibbles of code bytes 8(g%2) .. 8(g%2)+7, as in
// the tiled kernel) and runs one v_mfma_f32_16x16x32_bf16 per block with the scale d / 16, and the
// eight partial tiles are added in LDS in wave order.  (Two 8-byte activation loads per block,
// each covering 32 bytes of the 16 rows, took 10.1 / 5.0 / 9.5 us at 16 x 1280 x 5120 / 1280 x
// 1280 / 3072 x 3072 on MI355X against 8.4 / 4.2 / 6.2: a compute unit's load throughput, not
// the bytes, bounds these shapes.)
// ---------------------------------------------------------------------------------------
// MODE (T_PLAIN, T_GELU_OUT, T_PAIR_IN): as for the tiled kernel; with T_PAIR_IN a block's hi and
// lo activations (128 apart in the pair layout) go through two products into one result before its
// scale, and with T_GELU_OUT the outputs go to hl as GELU pairs.
template <int NB, int MODE = T_PLAIN>
__global__ __launch_bounds__(512) void q4_gemm_skinny_kernel(const uint8_t *__restrict__ w,
                                                             const uint16_t *__restrict__ x, float *__restrict__ y,
                                                             uint16_t *__restrict__ hl, int m, int n)
{
    constexpr int K = NB * 32 * (MODE == T_PAIR_IN ? 2 : 1);   // the activations' row length
    constexpr int NA = MODE == T_PAIR_IN ? 2 : 1;              // activation halves per block
    constexpr int RB = NB * 18;              // bytes per weight row
    constexpr int RW = RB / 4 + 1;           // LDS dwords per row: odd, so the 16 rows fall in 16 banks
    constexpr int CH = RB / 16;              // 16-byte chunks per row
    constexpr int PER = (16 * CH + 511) / 512;
    constexpr int BPW = NB / 8;              // blocks per wave
    static_assert(RB % 16 == 0 && NB % 8 == 0, "whole chunks per row, whole blocks per wave");
    __shared__ uint32_t wt[16 * RW];
    __shared__ float red[8][4][64];

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int grp = lane >> 4;
    const int l16 = lane & 15;
    const int n0 = blockIdx.x * 16;
    const int m0 = blockIdx.y * 16;   // the workgroup's 16-row tile
    const int kb0 = wave * BPW;

    // activations of this lane: row m0 + l16 (past m: the last row, not stored), inputs 8g..8g+7 of
    // each of the wave's blocks (one 16-byte load per block; pairs: the hi and lo halves)
    const uint16_t *xr = x + (size_t)min(m0 + l16, m - 1) * K;
    u32x4v xa[BPW][NA];
#pragma unroll
    for (int b = 0; b < BPW; ++b) {
        const int kb = kb0 + b;
        const uint16_t *xp = xr + (MODE == T_PAIR_IN ? (size_t)(256 * (kb >> 2) + 32 * (kb & 3)) : (size_t)kb * 32) +
                             8 * grp;
#pragma unroll
        for (int a = 0; a < NA; ++a)
            xa[b][a] = *reinterpret_cast<const u32x4v *>(xp + 128 * a);
    }
    // the 16 weight rows (rows past n repeat row n - 1): chunk q -> row q / CH, chunk q % CH;
    // threads past the last chunk reload it (an identical LDS store).  Non-temporal loads: at 16
    // rows each weight is read once (measured on MI355X: the M = 16 sets 3-4 % faster; the tiled
    // and wide products, whose row tiles share the weights, were 3-10 % slower with them)
    u32x4v wr[PER];
#pragma unroll
    for (int p = 0; p < PER; ++p) {
        const int q = min(tid + 512 * p, 16 * CH - 1);
        const int col = min(n0 + q / CH, n - 1);
        wr[p] = __builtin_nontemporal_load(
            reinterpret_cast<const u32x4v *>(w + (size_t)col * RB + (size_t)16 * (q % CH)));
    }
#pragma unroll
    for (int p = 0; p < PER; ++p) {
        const int q = min(tid + 512 * p, 16 * CH - 1);
        uint32_t *dst = wt + (q / CH) * RW + 4 * (q % CH);
        dst[0] = wr[p].x;
        dst[1] = wr[p].y;
        dst[2] = wr[p].z;
        dst[3] = wr[p].w;
    }
    __syncthreads();

    const uint32_t *row = wt + l16 * RW;
    f32x4v acc = 0.0f;
#pragma unroll
    for (int b = 0; b < BPW; ++b) {
        const int kb = kb0 + b;
        const int o = 18 * kb;   // byte offset of the block in its row: 4-aligned for even kb
        // lane group g: inputs 8g .. 8g+7 = the low (g < 2) or high (g >= 2) nibbles of code bytes
        // 8 (g % 2) .. 8 (g % 2) + 7, as 16 (code - 8)
        uint32_t lo, hi, d16;
        const int c = 8 * (grp & 1);
        const uint32_t *q = row + ((o + 2 + c) >> 2);
        if ((kb & 1) == 0) {     // uniform over the wave
            d16 = row[o >> 2] & 0xFFFFu;
            lo = __builtin_amdgcn_alignbyte(q[1], q[0], 2);
            hi = __builtin_amdgcn_alignbyte(q[2], q[1], 2);
        } else {
            d16 = row[(o - 2) >> 2] >> 16;
            lo = q[0];
            hi = q[1];
        }
        const bf16x8 bq = __builtin_bit_cast(bf16x8, nibbles_to_bf16_x16(lo, hi, grp >= 2 ? 0u : 4u));
        f32x4v t = 0.0f;
#pragma unroll
        for (int a = 0; a < NA; ++a)
            t = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, xa[b][a]), bq, t, 0, 0, 0);
        acc += (half_bits_to_float(d16) * 0.0625f) * t;
    }

    // add the eight waves' partial tiles in wave order
#pragma unroll
    for (int r = 0; r < 4; ++r)
        red[wave][r][lane] = acc[r];
    __syncthreads();
    // D layout of a 16x16 MFMA block: lane holds rows 4*(lane/16) .. +3 of column lane%16
    if (tid < 256) {
        const int ln = tid & 63, r = tid >> 6;
        float v = red[0][r][ln];
#pragma unroll
        for (int wv = 1; wv < 8; ++wv)
            v += red[wv][r][ln];
        const int rowi = m0 + 4 * (ln >> 4) + r;
        const int col = n0 + (ln & 15);
        if (rowi < m && col < n) {
            if constexpr (MODE == T_GELU_OUT)
                store_gelu_pair(hl, n, rowi, col, v);
            else
                y[(size_t)rowi * n + col] = v;
        }
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

// Reads the bytes of block `blk` (0..GT_KC-1 of the stage) of the NJ 16-column blocks from the
// raw stage copy (GT_RAW bytes per row) with aligned dword reads and unpacks this lane's operand
// (column 16j + l16, inputs 8*grp .. 8*grp+7) and scale.  ODD: blk is odd, so the block starts
// at 2 mod 4 and its code bytes are 4-aligned; otherwise the block is 4-aligned and the code
// bytes are 2 mod 4.
template <bool ODD, int NJ>
__device__ __forceinline__ void unpack_b(const uint32_t *raw, int blk, int l16, int grp, bf16x8 (&bf)[NJ],
                                         float (&d)[NJ])
{
    uint32_t dw[NJ][4];
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
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
    for (int j = 0; j < NJ; ++j) {
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


// NS: stages (of GT_STAGE inputs) per workgroup, fixed at compile time.  Workgroup z of the grid's
// third dimension takes stages z*NS .. z*NS+NS-1; with one slice it writes the output itself,
// otherwise its fp32 partial tile goes to part[z][m][n] and q4_gemm_reduce_kernel adds the
// slices.  k is the activations' row length.  NJ: 16-column blocks per tile (4: 64 x 64 tiles; 2:
// 64 x 32 tiles, for outputs that reach enough workgroups that way without splitting K).
template <int NS, int MODE, int NJ = 4>
__global__ __launch_bounds__(GT_THREADS) __attribute__((amdgpu_waves_per_eu(2))) void q4_gemm_tiled_kernel(const uint8_t *__restrict__ w,
                                                                   const uint16_t *__restrict__ x,
                                                                   float *__restrict__ y, uint16_t *__restrict__ hl,
                                                                   float *__restrict__ part, int m, int n, int k)
{
    constexpr int BN = 16 * NJ;                                   // tile columns
    constexpr int W_CHUNKS = BN * GT_RAW / GT_WB;                 // weight pieces per stage
    constexpr int WR = (W_CHUNKS + GT_THREADS - 1) / GT_THREADS;  // load rounds per stage
    __shared__ __attribute__((aligned(16))) uint32_t braw[2][BN * GT_RAW / 4];
    __shared__ f32x4v red[GT_WAVES / 2][4 * NJ][64];   // tree reduction of the waves' tiles

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int l16 = lane & 15, grp = lane >> 4;
    const int m0 = blockIdx.y * GT_BM;
    const int n0 = blockIdx.x * BN;
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
    uint32_t woff[WR];
    int wlds[WR];
#pragma unroll
    for (int r = 0; r < WR; ++r) {
        const int c = min(tid + GT_THREADS * r, W_CHUNKS - 1);
        const int col = min(n0 + c / (GT_RAW / GT_WB), n - 1);
        woff[r] = (uint32_t)col * row_bytes + (uint32_t)(GT_WB * (c % (GT_RAW / GT_WB)));
        wlds[r] = (GT_WB / 4) * c;
    }

    // two stages of loads in flight: register slots 0 and 1 (compile-time indices)
    u32x4v ar[2][4];
    u32x2v wr[2][WR];
    auto load_stage = [&](int st, auto slot) {
        constexpr int S = decltype(slot)::value;
        st = min(st, st_end - 1);   // past the slice: a harmless reload of its last stage
        const uint16_t *xs = x + (size_t)st * GT_STAGE;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            ar[S][i] = *reinterpret_cast<const u32x4v *>(xs + aoff[i]);
        const uint8_t *ws = w + (size_t)(st >> KWS) * GT_RAW;
#pragma unroll
        for (int r = 0; r < WR; ++r)
            wr[S][r] = *reinterpret_cast<const u32x2v *>(ws + woff[r]);
    };

    f32x4v acc[4][NJ];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
            acc[i][j] = 0.0f;

    auto stage = [&](int st, auto slot) {
        constexpr int S = decltype(slot)::value;
        const int b = st & 1;
#pragma unroll
        for (int r = 0; r < WR; ++r)
            *reinterpret_cast<u32x2v *>(&braw[b][wlds[r]]) = wr[S][r];
        bf16x8 af[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            af[i] = __builtin_bit_cast(bf16x8, ar[S][i]);
        __syncthreads();   // braw[b] complete; braw[b] is next written two stages later
        // B operands of block `wave` for the four 16-column blocks.  The block of column c
        // starts at byte o = c*GT_RAW + 18*wave: 4-aligned for even waves, 2 mod 4 for odd ones
        // (the parity is uniform over a wave, so each wave runs one straight-line path).
        bf16x8 bf[NJ];
        float d[NJ];
        if ((wave & 1) == 0)
            unpack_b<false, NJ>(&braw[b][0], wave, l16, grp, bf, d);
        else
            unpack_b<true, NJ>(&braw[b][0], wave, l16, grp, bf, d);
        // products in two rounds of 8 with independent result registers, then the scaled sums
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            f32x4v t[2][NJ];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
#pragma unroll
                for (int j = 0; j < NJ; ++j)
                    t[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[2 * h + i], bf[j], (f32x4v)0.0f, 0, 0, 0);
            }
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < NJ; ++j)
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
                for (int j = 0; j < NJ; ++j)
                    red[wave - half][i * NJ + j][lane] = acc[i][j];
        }
        __syncthreads();
        if (wave < half) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < NJ; ++j)
                    acc[i][j] += red[wave][i * NJ + j][lane];
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
            for (int j = 0; j < NJ; ++j) {
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

// ---------------------------------------------------------------------------------------
// Long chunks on 128 x 128 tiles (the wide product).  Each Q4_0 block of a 32 x 32 output block
// is two v_mfma_f32_32x32x16_bf16 products on the exact operands 16 (code - 8) into a zeroed
// temporary, which 16 fp32 multiply-adds per lane scale by the block's d / 16 into the
// accumulator.  The 32 x 32 x 16 product does twice the work of a 16 x 16 x 32 one in about the
// same issue time, and a wave's unpacked block serves 128 rows.
//
// Workgroup: 4 waves per K group, a 128 x 128 tile of Y.  Wave w of a group owns columns 32w ..
// 32w+31 for all 128 rows (four 32 x 32 output blocks) over the group's blocks of each stage, so
// each weight is unpacked once, in the registers of the wave that uses it.  K runs in stages of 4
// Q4_0 blocks (128 inputs): the stage's activations (128 rows x 128 bf16, rows padded by 16 bytes)
// and raw weight bytes (128 columns x 72 bytes) go through LDS, and the loads of a later stage are
// in flight in registers while the current one is computed.  Operand layouts of the 32 x 32 x 16
// product: lane L of A holds row L % 32, inputs 8(L/32) .. 8(L/32)+7 of a 16-input step; lane L of
// B holds column L % 32 and the same inputs; result register r of lane L is row 8(r/4) + 4(L/32) +
// r % 4, column L % 32, so a lane's 16 results share one column and one scale.  A Q4_0 block is
// two steps, its low nibbles (inputs 0-15) then its high nibbles (16-31); lane group g takes code
// bytes 8g .. 8g+7 in both.  Workgroup z of the grid's third dimension takes stages z*NS ..
// z*NS+NS-1 and, when part is set, writes its partial tile to part[z] instead of y.
// ---------------------------------------------------------------------------------------
typedef float f32x16v __attribute__((ext_vector_type(16)));

constexpr int GH_BM = 128, GH_BN = 128, GH_THREADS = 256;
constexpr int GH_KC = 4, GH_STAGE = GH_KC * 32;                   // Q4_0 blocks / inputs per stage
constexpr int GH_AROW = GH_STAGE + 8;                              // bf16 per LDS row of A (16-byte pad)
constexpr int GH_RAW = GH_KC * 18;                                 // weight bytes of a column per stage
constexpr int GH_A_PER = GH_BM * GH_STAGE * 2 / 16 / GH_THREADS;   // 16-byte pieces of A per thread: 8
constexpr int GH_W_PIECES = GH_BN * GH_RAW / 8;                    // 8-byte pieces of the weights: 1152
constexpr int GH_W_PER = (GH_W_PIECES + GH_THREADS - 1) / GH_THREADS;   // 5
static_assert(GH_A_PER * GH_THREADS * 8 == GH_BM * GH_STAGE, "the threads cover a stage of A");
static_assert(GH_RAW % 8 == 0, "a column's stage bytes are whole 8-byte pieces");

// Exact B operands 16 (code - 8) of block `blk` for this lane's column (both 16-input steps) and the
// block's scale d / 16, from the column's raw stage bytes in LDS.
__device__ __forceinline__ void unpack_codes(const uint32_t *col, int blk, int g, bf16x8 (&bq)[2], float &ds)
{
    const int base = 18 * blk;
    uint32_t d16, c0, c1;
    if ((blk & 1) == 0) {
        d16 = col[base >> 2] & 0xFFFFu;
        const uint32_t *q = col + ((base + 2 + 8 * g) >> 2);
        const uint32_t q0 = q[0], q1 = q[1], q2 = q[2];
        c0 = __builtin_amdgcn_alignbyte(q1, q0, 2);
        c1 = __builtin_amdgcn_alignbyte(q2, q1, 2);
    } else {
        d16 = col[(base - 2) >> 2] >> 16;
        const uint32_t *q = col + ((base + 2 + 8 * g) >> 2);
        c0 = q[0];
        c1 = q[1];
    }
    bq[0] = __builtin_bit_cast(bf16x8, nibbles_to_bf16_x16(c0, c1, 4u));   // low nibbles: first step
    bq[1] = __builtin_bit_cast(bf16x8, nibbles_to_bf16_x16(c0, c1, 0u));   // high nibbles: second step
    float d = half_bits_to_float(d16) * 0.0625f;   // exact: the operands were 16 (code - 8)
    asm volatile("" : "+v"(d));   // an fp32 scale, so the multiply-adds are v_fmac_f32
    ds = d;
}

// KW: wave groups splitting K inside the workgroup.  Group kg (waves 4 kg .. 4 kg + 3) takes
// blocks kg * GH_KC / KW .. of every stage, so each weight is still unpacked once, by the one wave
// that uses it; with KW = 2 every SIMD runs two waves, one's products covering the other's vector
// work and LDS reads.  The groups' partial tiles are added through LDS at the end, group 0's first.
// LDS holds two stages: the waves store stage s + 1 (loaded from memory during stage s - 1) into
// the other buffer after their first block of stage s, then issue the loads of stage s + 2, so one
// barrier per stage suffices.
// MODE: T_PLAIN, T_GELU_OUT or T_PAIR_IN as for the tiled kernel (a pair stage reads weight stage
// st / 2; with K split over the grid a GELU output goes through the slice sum).
template <int NS, int KW, int MODE>
__global__ __launch_bounds__(GH_THREADS * KW) __attribute__((amdgpu_waves_per_eu(2))) void q4_gemm_wide_kernel(
    const uint8_t *__restrict__ w, const uint16_t *__restrict__ x, float *__restrict__ y, uint16_t *__restrict__ hl,
    float *__restrict__ part, int m, int n, int k)
{
    constexpr int NT = GH_THREADS * KW;
    constexpr int A_PER = GH_A_PER / KW;                        // 16-byte pieces of A per thread
    constexpr int W_PER = (GH_W_PIECES + NT - 1) / NT;          // 8-byte weight pieces per thread
    constexpr int MI = 4;                                        // 32-row blocks per wave
    constexpr int BPW = GH_KC / KW;                              // blocks per wave and stage
    constexpr int A_BUF = GH_BM * GH_AROW;                       // bf16 per stage of A
    constexpr int W_BUF = GH_BN * GH_RAW / 4;                    // dwords per stage of weights
    static_assert(GH_A_PER % KW == 0 && GH_KC % KW == 0, "the wave groups share the stage evenly");
    static_assert(KW == 1 || (KW - 1) * 4 * MI * 16 * 64 * 4 <= 2 * A_BUF * 2, "the partial tiles fit in LDS");
    __shared__ __attribute__((aligned(16))) uint16_t as[2 * A_BUF];
    __shared__ __attribute__((aligned(16))) uint32_t wraw[2 * W_BUF];

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int wn = wave & 3, kg = wave >> 2;   // column quarter, K group
    const int lane = tid & 63;
    const int l32 = lane & 31, g = lane >> 5;
    const int m0 = blockIdx.y * GH_BM;
    const int n0 = blockIdx.x * GH_BN;
    const int st0 = blockIdx.z * NS;
    constexpr int KWS = MODE == T_PAIR_IN ? 1 : 0;   // weight stage = activation stage >> KWS
    const uint32_t row_bytes = (uint32_t)((k >> KWS) / 32) * 18;

    // activations: piece p = tid + NT j is row p / 16, inputs 8 (p % 16) .. of the stage (rows past
    // m repeat the last row; their outputs are not stored)
    // (32-bit byte offsets, the stage's added each time: below 2^32 since m k and the weight bytes
    // are below 2^31, so a load takes the uniform base and one offset register)
    uint32_t aoff[A_PER];
    int alds[A_PER];
#pragma unroll
    for (int j = 0; j < A_PER; ++j) {
        const int p = tid + NT * j, r = p >> 4, c = p & 15;
        aoff[j] = 2u * ((uint32_t)min(m0 + r, m - 1) * (uint32_t)k + (uint32_t)(8 * c));
        alds[j] = r * GH_AROW + 8 * c;
    }
    // weights: piece q is column q / 9, bytes 8 (q % 9) .. of its stage bytes; pieces past the last
    // repeat it (a duplicate load and an identical LDS store); columns past n repeat the last one
    uint32_t woff[W_PER];
    int wlds[W_PER];
#pragma unroll
    for (int j = 0; j < W_PER; ++j) {
        const int q = min(tid + NT * j, GH_W_PIECES - 1);
        const int col = min(n0 + q / (GH_RAW / 8), n - 1);
        woff[j] = (uint32_t)col * row_bytes + (uint32_t)(8 * (q % (GH_RAW / 8)));
        wlds[j] = (q / (GH_RAW / 8)) * (GH_RAW / 4) + 2 * (q % (GH_RAW / 8));
    }

    u32x4v ar[A_PER];
    u32x2v wr[W_PER];
    const uint8_t *xb = reinterpret_cast<const uint8_t *>(x);
    auto load_stage = [&](int st) {
        const uint32_t xo = (uint32_t)st * (GH_STAGE * 2), wo = (uint32_t)(st >> KWS) * GH_RAW;
#pragma unroll
        for (int j = 0; j < A_PER; ++j)
            ar[j] = *reinterpret_cast<const u32x4v *>(xb + (aoff[j] + xo));
#pragma unroll
        for (int j = 0; j < W_PER; ++j)
            wr[j] = *reinterpret_cast<const u32x2v *>(w + (woff[j] + wo));
    };
    auto store_stage = [&](int buf) {
#pragma unroll
        for (int j = 0; j < A_PER; ++j)
            *reinterpret_cast<u32x4v *>(&as[buf * A_BUF + alds[j]]) = ar[j];
#pragma unroll
        for (int j = 0; j < W_PER; ++j)
            *reinterpret_cast<u32x2v *>(&wraw[buf * W_BUF + wlds[j]]) = wr[j];
    };

    f32x16v acc[MI], t[MI];   // t: the last block's unscaled products
#pragma unroll
    for (int i = 0; i < MI; ++i) {
        acc[i] = 0.0f;
        t[i] = 0.0f;
    }
    float dprev = 0.0f;   // the last block's scale

    load_stage(st0);
    store_stage(0);
    if (NS > 1)
        load_stage(st0 + 1);
    __syncthreads();
    // block b of the stage in buffer cur.  The previous block's products are scaled into the
    // accumulators while this block's products of the tile before are in flight.
    auto block = [&](int cur, int b) {
        const uint32_t *colw = wraw + cur * W_BUF + (32 * wn + l32) * (GH_RAW / 4);
        const uint16_t *arow = as + cur * A_BUF + l32 * GH_AROW + 8 * g;
        bf16x8 bq[2];
        float ds;
        unpack_codes(colw, b, g, bq, ds);
        bf16x8 af[MI][2];
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int h = 0; h < 2; ++h)
                af[i][h] = *reinterpret_cast<const bf16x8 *>(arow + 32 * i * GH_AROW + 32 * b + 16 * h);
#pragma unroll
        for (int i = 0; i < MI; ++i) {
            acc[i] += dprev * t[i];
            t[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i][0], bq[0], (f32x16v)0.0f, 0, 0, 0);
            t[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i][1], bq[1], t[i], 0, 0, 0);
        }
        dprev = ds;
        // one product, then eight vector instructions
#pragma unroll
        for (int i = 0; i < 2 * MI; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);
        }
    };
    // one straight-line body per stage: after its first block the waves store the next stage
    // (loaded during the stage before) into the other buffer, last read in the stage before, and
    // load the one after (past the last stage: a harmless reload of it).  The loop takes two
    // stages per iteration, so each body's LDS buffer is a constant folded into the instruction
    // offsets (measured on MI355X: 201 instead of 217 vector instructions per stage and wave, the
    // products over 750 x 5120 x 1280 / 5120 1-6 % faster)
    auto stage = [&](int s, auto cur_c) {
        constexpr int cur = decltype(cur_c)::value;
        block(cur, kg * BPW);
        store_stage(cur ^ 1);
        load_stage(min(st0 + s + 2, st0 + NS - 1));
#pragma unroll
        for (int bb = 1; bb < BPW; ++bb)
            block(cur, kg * BPW + bb);
        __syncthreads();
    };
    static_assert(NS % 2 == 0, "stages are taken in pairs");
    for (int s = 0; s + 2 < NS; s += 2) {
        stage(s, std::integral_constant<int, 0>{});
        stage(s + 1, std::integral_constant<int, 1>{});
    }
    stage(NS - 2, std::integral_constant<int, 0>{});
#pragma unroll
    for (int bb = 0; bb < BPW; ++bb)
        block((NS - 1) & 1, kg * BPW + bb);
#pragma unroll
    for (int i = 0; i < MI; ++i)
        acc[i] += dprev * t[i];

    if constexpr (KW > 1) {
        // groups 1.. leave their partial tiles in LDS, over the stage buffers once every wave has
        // read the last stage; group 0 adds them in group order
        float *red = reinterpret_cast<float *>(as);
        __syncthreads();
        if (kg > 0) {
#pragma unroll
            for (int i = 0; i < MI; ++i)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    red[((((kg - 1) * 4 + wn) * MI + i) * 16 + r) * 64 + lane] = acc[i][r];
        }
        __syncthreads();
        if (kg > 0)
            return;
#pragma unroll
        for (int q = 1; q < KW; ++q)
#pragma unroll
            for (int i = 0; i < MI; ++i)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    acc[i][r] += red[((((q - 1) * 4 + wn) * MI + i) * 16 + r) * 64 + lane];
    }

    const bool gelu = MODE == T_GELU_OUT && !part;   // uniform over the grid
    float *const dst = part ? part + (size_t)blockIdx.z * m * n : y;
    const int col = n0 + 32 * wn + l32;
    if (col < n) {
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = m0 + 32 * i + 8 * (r >> 2) + 4 * g + (r & 3);
                if (row < m) {
                    if (gelu)
                        store_gelu_pair(hl, n, row, col, acc[i][r]);
                    else
                        dst[(size_t)row * n + col] = acc[i][r];
                }
            }
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

// 64 x 32 tiles at K = 1280 where they alone give GT_TARGET_WGS workgroups and 64 x 64 tiles would
// need K slices: measured on MI355X, 200 x 1280 x 1280 9.2 us against 11.4 with two slices and
// their sum; at K = 5120 and 3072 the unsplit chain of 64 x 32 tiles was slower (200 x 1280 x 5120
// 24.2 against 22.3 us, 100 x 3072 x 3072 17.5 against 17.2), and where 64 x 64 tiles need no
// slices 64 x 32 ones were 10-20 % slower (750 x 1280 x 1280 15.4 against 12.9 us).
static bool tiled_narrow(int64_t m, int64_t n, int64_t k)
{
    const int64_t rows = (m + GT_BM - 1) / GT_BM;
    return tiled_shape(m, n, k) && k == 1280 && ((n + GT_BN - 1) / GT_BN) * rows < GT_TARGET_WGS &&
           ((n + 31) / 32) * rows >= GT_TARGET_WGS;
}

static size_t tiled_workspace(int64_t m, int64_t n, int slices)
{
    return slices > 1 ? (size_t)slices * (size_t)m * (size_t)n * sizeof(float) : 0;
}

template <int S, int MODE, int NJ = 4>
static void launch_tiled_slices(const void *w, const uint16_t *x, float *y, uint16_t *hl, float *part, int m, int n,
                                int k, int slices, hipStream_t s)
{
    const dim3 grid((unsigned)((n + 16 * NJ - 1) / (16 * NJ)), (unsigned)((m + GT_BM - 1) / GT_BM), (unsigned)slices);
    hipLaunchKernelGGL((q4_gemm_tiled_kernel<S, MODE, NJ>), grid, dim3(GT_THREADS), 0, s, (const uint8_t *)w, x, y,
                       hl, part, m, n, k);
}

// Output: y (fp32), or for T_GELU_OUT GELU pairs in hl (n a multiple of 256).  part: slices x m x n
// floats when slices > 1, else null (the kernel then writes the output itself).  k: the
// activations' row length.
// y (or GELU pairs in hl) = the sum of `slices` partial tiles part[z][m][n], added in order z = 0, 1, ...
template <bool GELU>
static int launch_slice_sum(const float *part, float *y, uint16_t *hl, int m, int n, int slices, hipStream_t s)
{
    const int64_t count = (int64_t)m * n;
    const bool vec4 = count % 4 == 0 && (GELU ? n % 4 == 0 : aligned(y, 16));
    const int64_t threads = vec4 ? count / 4 : count;
    const dim3 rg((unsigned)((threads + 255) / 256));
    if (slices <= 2)
        hipLaunchKernelGGL((q4_gemm_reduce_kernel<GELU, 2>), rg, dim3(256), 0, s, part, y, hl, count, n, slices, vec4);
    else if (slices <= 4)
        hipLaunchKernelGGL((q4_gemm_reduce_kernel<GELU, 4>), rg, dim3(256), 0, s, part, y, hl, count, n, slices, vec4);
    else if (slices <= 8)
        hipLaunchKernelGGL((q4_gemm_reduce_kernel<GELU, 8>), rg, dim3(256), 0, s, part, y, hl, count, n, slices, vec4);
    else
        hipLaunchKernelGGL((q4_gemm_reduce_kernel<GELU, 0>), rg, dim3(256), 0, s, part, y, hl, count, n, slices, vec4);
    return check_launch("q4 product: slice sum");
}

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
    const int st = check_launch("q4 tiled product");
    return st || slices == 1 ? st : launch_slice_sum<gelu>(part, y, hl, m, n, slices, s);
}

// The wide product (q4_gemm_wide_kernel) takes chunks of at least WIDE_MIN_M rows whose 128 x 128
// tiles, with K split over the grid into slices of at least WIDE_MIN_STAGES stages where needed
// (the partial tiles in the caller's workspace, then the slice sum), give at least WIDE_MIN_WGS
// workgroups.  Measured on MI355X: 750 x 5120 x 1280 22.4 us, 750 x 5120 x 5120 64.1 us (a stage
// 1.39 us, a launch about 8.5 us besides); the same tiles with the exact hi and lo bf16 parts of
// every weight as B operands (twice the products, no per-block scale) took 27.4 and 83.7 us.
// Two wave groups splitting K inside the workgroup (two waves per SIMD) with one barrier per
// stage: 27.6 to 28.0 us against 29.3 for four waves with two barriers per stage (30.4 with one)
// in the hi/lo form; eight waves each 32 x 64 (every weight unpacked twice): 30.5 us; eight-block
// stages: no faster.
constexpr int64_t WIDE_MIN_M = 128;
constexpr int WIDE_MIN_WGS = 160;
constexpr int WIDE_MIN_STAGES = 10;
constexpr int WIDE_KW = 2;   // wave groups splitting K per workgroup

// Slices of K over the grid for the wide product: 1 (unsplit), more (a workspace of that many
// partial tiles), or 0 where the wide product does not take the shape.  k is the activations' row
// length; kws = 1 for GELU-pair activations (weights of k / 2 inputs).
static int wide_slices(int64_t m, int64_t n, int64_t k, int kws = 0)
{
    const size_t wbytes = (size_t)n * (size_t)((k >> kws) / 32) * 18;
    if (!tiled_k(k >> kws) || m < WIDE_MIN_M || (uint64_t)m * (uint64_t)k >= (1ull << 31) || wbytes >= (1ull << 31) ||
        (m + GH_BM - 1) / GH_BM > 65535)
        return 0;
    const int64_t tiles = ((n + GH_BN - 1) / GH_BN) * ((m + GH_BM - 1) / GH_BM);
    const int nst = (int)(k / GH_STAGE);
    for (int ks = 1; nst / ks >= WIDE_MIN_STAGES; ++ks)
        if (nst % ks == 0 && tiles * ks >= WIDE_MIN_WGS)
            return ks;
    return 0;
}

template <int NS, int MODE>
static void launch_wide_ns(const void *w, const uint16_t *x, float *y, uint16_t *hl, float *part, int m, int n, int k,
                           int slices, hipStream_t s)
{
    const dim3 grid((unsigned)((n + GH_BN - 1) / GH_BN), (unsigned)((m + GH_BM - 1) / GH_BM), (unsigned)slices);
    hipLaunchKernelGGL((q4_gemm_wide_kernel<NS, WIDE_KW, MODE>), grid, dim3(GH_THREADS * WIDE_KW), 0, s,
                       (const uint8_t *)w, x, y, hl, part, m, n, k);
}

// The wide product; part holds `slices` partial tiles when K is split, and a GELU output (into hl)
// then goes through the slice sum.
template <int MODE>
static int launch_gemm_wide(const void *w, const uint16_t *x, float *y, uint16_t *hl, float *part, int m, int n, int k,
                            int slices, hipStream_t s)
{
    constexpr bool gelu = MODE == T_GELU_OUT;
    if ((slices > 1) != (part != nullptr) || (gelu ? (hl == nullptr || n % GELU_STAGE) : y == nullptr))
        return fail(VOX_E_INVAL, "q4 wide product: one output, and a partial-tile buffer exactly when K is split");
    switch ((k / GH_STAGE) / slices) {   // stages per workgroup
    case 48: launch_wide_ns<48, MODE>(w, x, y, hl, part, m, n, k, slices, s); break;
    case 40: launch_wide_ns<40, MODE>(w, x, y, hl, part, m, n, k, slices, s); break;
    case 24: launch_wide_ns<24, MODE>(w, x, y, hl, part, m, n, k, slices, s); break;
    case 20: launch_wide_ns<20, MODE>(w, x, y, hl, part, m, n, k, slices, s); break;
    case 16: launch_wide_ns<16, MODE>(w, x, y, hl, part, m, n, k, slices, s); break;
    case 12: launch_wide_ns<12, MODE>(w, x, y, hl, part, m, n, k, slices, s); break;
    case 10: launch_wide_ns<10, MODE>(w, x, y, hl, part, m, n, k, slices, s); break;
    default: return fail(VOX_E_UNSUPPORTED, "q4 wide product: no compiled stage count for k=%d in %d slices", k, slices);
    }
    const int st = check_launch("q4 wide product");
    return st || slices == 1 ? st : launch_slice_sum<gelu>(part, y, hl, m, n, slices, s);
}

// The skinny kernel takes the products of at most 64 rows at K = 1280 or 3072 and of at most 16
// rows at K = 5120 (a workgroup per 16-row tile; the weights of a 16-column tile fit in LDS for
// the whole of K).  Measured on MI355X: 16 x 1280 x 1280 4.2 us, 16 x 5120 x 1280 5.4,
// q/k/v stacked 4.2, 16 x 3072 x 3072 6.2, 16 x 1280 x 5120 8.4 against 10.1 for the tiled kernel
// with K split over the grid and its slice sum (and 5.6 / 9.0 / 5.7 / 13.0 us for the first shapes
// on the split-K-over-waves or tiled kernels); 64 x 1280 x 1280 5.4 against 8.9 us (split-K over
// waves), 64 x 3840 x 1280 8.1 against 12.6, 64 x 5120 x 1280 9.4 against 11.8 and 24 / 64 x 3072 x
// 3072 8.2 / 12.5 against 11.5 / 13.5 (tiled and slice sum), but 64 x 1280 x 5120 13.2 against
// 12.0 and 64 x 3072 x 5120 19.3 against 17.5, where every 16-row tile reads all of K of its
// activations once per 16 columns.
static bool skinny_shape(int64_t m, int64_t n, int64_t k)
{
    return m >= 1 && (k == 1280 || k == 3072 || (k == 5120 && m <= 16)) && m <= 64 &&
           (uint64_t)n * (uint64_t)(k / 32) * 18 < (1ull << 31) && (n + 15) / 16 <= 0x7FFFFFFF;
}

static int launch_gemm_skinny(const void *w, const uint16_t *x, float *y, int m, int n, int k, hipStream_t s)
{
    const dim3 grid((unsigned)((n + 15) / 16), (unsigned)((m + 15) / 16));
    switch (k) {
    case 1280: hipLaunchKernelGGL((q4_gemm_skinny_kernel<40>), grid, dim3(512), 0, s, (const uint8_t *)w, x, y, nullptr, m, n); break;
    case 3072: hipLaunchKernelGGL((q4_gemm_skinny_kernel<96>), grid, dim3(512), 0, s, (const uint8_t *)w, x, y, nullptr, m, n); break;
    case 5120: hipLaunchKernelGGL((q4_gemm_skinny_kernel<160>), grid, dim3(512), 0, s, (const uint8_t *)w, x, y, nullptr, m, n); break;
    default: return fail(VOX_E_UNSUPPORTED, "q4 skinny product: no compiled K for k=%d", k);
    }
    return check_launch("q4 skinny product");
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
    if (m <= 0 || n <= 0 || k <= 0 || k % 32 || m > 65535 * 16 || n > (1 << 24) || k > (1 << 24))
        return 0;
    if (const int ws = wide_slices(m, n, k))
        return ws > 1 ? tiled_workspace(m, n, ws) : 0;
    if (skinny_shape(m, n, k))
        return 0;
    if (!tiled_shape(m, n, k) || tiled_narrow(m, n, k))
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
    const int wide = aligned(x_bf16, 16) && aligned(w_q4, 16) ? wide_slices(m, n, k) : 0;
    if (wide == 1 || (wide > 1 && workspace)) {
        const size_t need = wide > 1 ? tiled_workspace(m, n, wide) : 0;
        if (need > workspace_bytes)
            return fail(VOX_E_WORKSPACE, "vox_q4_gemm: workspace of %zu bytes, need %zu", workspace_bytes, need);
        if (need && (!aligned(workspace, 16) || overlaps(workspace, need, y, ybytes) ||
                     overlaps(workspace, need, x_bf16, xbytes) || overlaps(workspace, need, w_q4, wbytes)))
            return fail(VOX_E_INVAL, "vox_q4_gemm: workspace must be 16-byte aligned and apart from x, y and w");
        st = launch_gemm_wide<T_PLAIN>(w_q4, x_bf16, y, nullptr, wide > 1 ? (float *)workspace : nullptr, (int)m,
                                       (int)n, (int)k, wide, s);
    } else if (aligned(x_bf16, 16) && aligned(w_q4, 16) && skinny_shape(m, n, k)) {
        st = launch_gemm_skinny(w_q4, x_bf16, y, (int)m, (int)n, (int)k, s);
    } else if (aligned(x_bf16, 16) && aligned(w_q4, 16) && tiled_narrow(m, n, k)) {
        launch_tiled_slices<10, T_PLAIN, 2>(w_q4, x_bf16, y, nullptr, nullptr, (int)m, (int)n, (int)k, 1, s);
        st = check_launch("q4 tiled product");
    } else if (aligned(x_bf16, 16) && aligned(w_q4, 16) && tiled_shape(m, n, k)) {
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

// K slices of the adapter's two products: the wide product's where it takes the shape (wide set),
// else the tiled kernel's.
struct AdapterPlan {
    bool skinny1, skinny2, wide1, wide2;
    int s1, s2;   // K slices (1: unsplit)
};
static AdapterPlan adapter_plan(int64_t m, int64_t k, int64_t n_mid, int64_t n_out)
{
    AdapterPlan p;
    p.skinny1 = p.skinny2 = m <= 16;
    const int w1 = wide_slices(m, n_mid, k), w2 = wide_slices(m, n_out, 2 * n_mid, 1);
    p.wide1 = !p.skinny1 && w1 > 0;
    p.wide2 = !p.skinny2 && w2 > 0;
    p.s1 = p.skinny1 ? 1 : p.wide1 ? w1 : tiled_slices(m, n_mid, k);
    p.s2 = p.skinny2 ? 1 : p.wide2 ? w2 : tiled_slices(m, n_out, 2 * n_mid);
    return p;
}

static size_t adapter_part_bytes(int64_t m, int64_t k, int64_t n_mid, int64_t n_out)
{
    const AdapterPlan p = adapter_plan(m, k, n_mid, n_out);
    const size_t a = tiled_workspace(m, n_mid, p.s1);
    const size_t b = tiled_workspace(m, n_out, p.s2);
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

// The adapter's products through the skinny kernel at most 16 rows (no K slices), the first
// writing the GELU pairs, the second reading them.  Measured on MI355X: 4 rows 18.6 us against
// 28.7 with the tiled products and their slice sums, 16 rows 27.3 against 29.5 (before the skinny
// kernel's 16-byte activation loads; with them 14.0 and 18.8 us).  The second product through it
// at 50 rows as well: 37.8 against 36.4 us.
static int adapter_skinny_first(const void *w1, const uint16_t *x, uint16_t *h, int m, int k, int n_mid, hipStream_t s)
{
    const dim3 g1((unsigned)((n_mid + 15) / 16), (unsigned)((m + 15) / 16));
    switch (k) {
    case 1280: hipLaunchKernelGGL((q4_gemm_skinny_kernel<40, T_GELU_OUT>), g1, dim3(512), 0, s, (const uint8_t *)w1, x, nullptr, h, m, n_mid); break;
    case 3072: hipLaunchKernelGGL((q4_gemm_skinny_kernel<96, T_GELU_OUT>), g1, dim3(512), 0, s, (const uint8_t *)w1, x, nullptr, h, m, n_mid); break;
    default: hipLaunchKernelGGL((q4_gemm_skinny_kernel<160, T_GELU_OUT>), g1, dim3(512), 0, s, (const uint8_t *)w1, x, nullptr, h, m, n_mid); break;
    }
    return check_launch("adapter, first product");
}

static int adapter_skinny_second(const void *w2, const uint16_t *h, float *y, int m, int n_mid, int n_out, hipStream_t s)
{
    const dim3 g2((unsigned)((n_out + 15) / 16), (unsigned)((m + 15) / 16));
    if (n_mid == 1280)
        hipLaunchKernelGGL((q4_gemm_skinny_kernel<40, T_PAIR_IN>), g2, dim3(512), 0, s, (const uint8_t *)w2, h, y, nullptr, m, n_out);
    else
        hipLaunchKernelGGL((q4_gemm_skinny_kernel<96, T_PAIR_IN>), g2, dim3(512), 0, s, (const uint8_t *)w2, h, y, nullptr, m, n_out);
    return check_launch("adapter, second product");
}

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
    const AdapterPlan p = adapter_plan(m, k, n_mid, n_out);
    float *p1 = p.s1 > 1 ? part : nullptr, *p2 = p.s2 > 1 ? part : nullptr;
    int st = p.skinny1 ? adapter_skinny_first(w1_q4, x_bf16, h, (int)m, (int)k, (int)n_mid, s)
             : p.wide1 ? launch_gemm_wide<T_GELU_OUT>(w1_q4, x_bf16, nullptr, h, p1, (int)m, (int)n_mid, (int)k, p.s1, s)
                       : launch_gemm_tiled<T_GELU_OUT>(w1_q4, x_bf16, nullptr, h, p1, (int)m, (int)n_mid, (int)k, p.s1, s);
    if (!st)
        st = p.skinny2 ? adapter_skinny_second(w2_q4, h, y, (int)m, (int)n_mid, (int)n_out, s)
             : p.wide2 ? launch_gemm_wide<T_PAIR_IN>(w2_q4, h, y, nullptr, p2, (int)m, (int)n_out, (int)(2 * n_mid), p.s2, s)
                       : launch_gemm_tiled<T_PAIR_IN>(w2_q4, h, y, nullptr, p2, (int)m, (int)n_out, (int)(2 * n_mid),
                                                      p.s2, s);
    return st ? st : ok();
}
