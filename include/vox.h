/* vox.h - C ABI of the MI355X (gfx950) library for the per-token decoder step of the
 * streaming Voxtral Mini 4B Realtime speech-to-text model.
 *
 * Source pages this interface follows:
 *  [RS] "Mistral의 Voxtral Mini 4B Realtime 모델을 Rust로 구현해 브라우저에서 실행"
 *       (GeekNews 26595): section 아키텍처 - the Q4 path stores every linear as GGUF Q4_0 and
 *       fuses dequantisation into the matrix product in custom shaders; section 브라우저 실행을
 *       위한 기술적 해결 - the embedding stays on the GPU as Q4 and one row is looked up per token.
 *  [VC] "Mistral Voxtral Realtime 4B 음성 인식 모델의 순수 C 기반 CPU 전용 추론 구현"
 *       (GeekNews 26608): section 모델 아키텍처 - decoder of 26 layers, width 3072, GQA with 32
 *       query heads over 8 KV heads, encoder width 1280, vocabulary 131,072; section 주요 기능 -
 *       a rolling KV cache over an 8192-position sliding window; section C API 구조 - a `vox_`
 *       prefixed C API around an opaque stream handle; section 성능 벤치마크 - the whole decoder
 *       token is one GPU submission.
 *
 * Conventions for every entry point:
 *  - Buffer pointers are DEVICE pointers owned by the caller.  The library never allocates
 *    device memory; callers size workspaces with the *_workspace queries.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).  Calls only enqueue
 *    work; results are ready when the caller synchronises the stream.
 *  - Arguments are validated on the host before any device work; a failed check returns a
 *    negative status and enqueues nothing.  vox_last_error() then holds a message.
 *  - Launch failures return VOX_E_HIP.  Faults inside kernels surface at the caller's next
 *    synchronisation.  No C++ exception crosses this interface.
 *  - GGUF Q4_0 weights: a matrix of n rows by k inputs is n*k/32 blocks of 18 bytes, row
 *    major, k/32 consecutive blocks per row.  Block: bytes 0..1 = fp16 scale d
 *    (little-endian); byte 2+j (j=0..15) low nibble = code of weight j, high nibble = code of
 *    weight j+16; weight = (code - 8) * d.  k must be a positive multiple of 32.
 */
#ifndef VOX_H
#define VOX_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
    VOX_OK = 0,
    VOX_E_INVAL = -1,        /* bad argument: null pointer, size, aliasing, layout */
    VOX_E_UNSUPPORTED = -2,  /* valid request outside what the kernels implement */
    VOX_E_WORKSPACE = -3,    /* workspace or buffer too small */
    VOX_E_HIP = -4           /* HIP runtime error while enqueuing */
};

/* Static description of a status code. */
const char *vox_strerror(int status);
/* Detail of the most recent failure on the calling thread ("" if none). */
const char *vox_last_error(void);

/* Q4_0 dequantisation ([RS] 아키텍처).  out[32*b + j] = (code_j - 8) * d_b for n_blocks blocks,
 * fp32, bit-exact (every product is exactly representable).  w_q4: n_blocks*18 bytes, any
 * alignment.  out: n_blocks*32 floats, must not overlap w_q4.  n_blocks == 0 is a no-op. */
int vox_q4_dequant(const void *w_q4, int64_t n_blocks, float *out, void *stream);

/* Q4_0 matrix-vector product with dequantisation fused into the product ([RS] 아키텍처):
 * y[r] = sum_i W[r][i] * x[i], fp32 accumulation.  w_q4: n rows by k inputs (layout above);
 * x: k floats; y: n floats, must not overlap x or w_q4.  n == 0 is a no-op.
 * k % 32 != 0 or k <= 0 -> VOX_E_INVAL. */
int vox_q4_gemv(const void *w_q4, const float *x, float *y, int64_t n, int64_t k, void *stream);

/* Matrix-vector product over 16-bit weights ([VC] 모델 다운로드 및 구성: the weights ship as BF16;
 * [VC] 메모리 요구사항: the GPU copy is F16): y[r] = sum_i W[r][i] * x[i], fp32 accumulation.
 * w: n rows by k, row-major bit patterns of bf16 (fmt VOX_W16_BF16) or IEEE binary16
 * (VOX_W16_F16); x: k floats; y: n floats, must not overlap x or w.  n == 0 is a no-op.
 * k not a positive multiple of 8, or another fmt -> VOX_E_INVAL; w, x not 16-byte aligned ->
 * VOX_E_UNSUPPORTED. */
enum { VOX_W16_BF16 = 0, VOX_W16_F16 = 1 };
int vox_w16_gemv(const void *w, int fmt, const float *x, float *y, int64_t n, int64_t k, void *stream);

/* Encoder-chunk linear Y = X * W^T with Q4_0 weights ([VC] 모델 아키텍처: encoder width 1280;
 * [RS] 아키텍처: Q4_0 linears), on the matrix cores.  x_bf16: m rows by k, bf16 bit patterns,
 * row major; w_q4: n rows by k; y: m by n fp32, row major, must not overlap the inputs.
 * Products of the exact Q4 codes with bf16 activations, fp32 accumulation.
 * workspace: NULL with workspace_bytes 0, or device memory of at least
 * vox_q4_gemm_workspace(m, n, k) bytes, 16-byte aligned, apart from x, y and w, contents
 * irrelevant (the call may then split K over more workgroups and add the slices' partial
 * results in a fixed order; results do not depend on the split beyond fp32 rounding order, and
 * exact sums stay exact).  A non-null workspace below the size -> VOX_E_WORKSPACE.
 * m == 0 or n == 0 is a no-op.  k % 32 != 0 -> VOX_E_INVAL; m > 1048560 or n, k > 2^24 ->
 * VOX_E_UNSUPPORTED.  x_bf16 must be 8-byte and w_q4 2-byte aligned (VOX_E_UNSUPPORTED). */
size_t vox_q4_gemm_workspace(int64_t m, int64_t n, int64_t k);
int vox_q4_gemm(const void *w_q4, const uint16_t *x_bf16, float *y, int64_t m, int64_t n, int64_t k,
                void *workspace, size_t workspace_bytes, void *stream);

/* Adapter from the audio encoder to the decoder ([VC] 모델 아키텍처: a linear from 5120 to 3072
 * inputs, GELU, a linear from 3072 to 3072; [RS] 아키텍처: Q4_0 linears):
 *   Y = GELU(X * W1^T) * W2^T,
 * GELU(v) = v * Phi(v) with Phi the standard normal distribution function (the exact form), no
 * biases.  x_bf16: m rows by k, bf16 bit patterns, row major; w1_q4: n_mid rows by k; w2_q4:
 * n_out rows by n_mid; y: m by n_out fp32, row major, must not overlap the inputs.  Products of
 * the exact Q4 codes with bf16 activations on the matrix cores, fp32 accumulation; the GELU
 * output is computed in fp32 and enters the second product as a pair of bf16 values whose sum
 * is within 2^-18 of it (relative).  workspace: at least vox_adapter_workspace(m, k, n_mid, n_out)
 * bytes of device memory, 16-byte aligned, apart from the other buffers, contents irrelevant.
 * The call is deterministic: the order of every sum is fixed.
 * m == 0 or n_out == 0 is a no-op.  k or n_mid not a positive multiple of 32 -> VOX_E_INVAL;
 * k outside {1280, 3072, 5120}, n_mid outside {1280, 3072}, or m * k, 2 * m * n_mid >= 2^31 ->
 * VOX_E_UNSUPPORTED (the workspace query then returns 0); x_bf16, w1_q4, w2_q4 not 16-byte
 * aligned -> VOX_E_UNSUPPORTED; a null or smaller workspace -> VOX_E_INVAL / VOX_E_WORKSPACE. */
size_t vox_adapter_workspace(int64_t m, int64_t k, int64_t n_mid, int64_t n_out);
int vox_adapter(const void *w1_q4, const void *w2_q4, const uint16_t *x_bf16, float *y, int64_t m, int64_t k,
                int64_t n_mid, int64_t n_out, void *workspace, size_t workspace_bytes, void *stream);

/* Self-attention of the audio encoder over one chunk of frames ([VC] 모델 아키텍처: causal
 * transformer, 32 heads over width 1280, window 750; [VC] 주요 기능: the encoder runs over chunks).
 * q: m rows of n_heads * head_dim fp32 (the chunk's queries, heads side by side as a linear writes
 * them); k, v: n_ctx + m rows of the same width, the n_ctx positions before the chunk followed by
 * the chunk's own, so query i sits at row n_ctx + i; out: m rows like q.  Per head h and query i:
 *   s_j = scale * <q_i, k_j> for n_ctx + i - window + 1 <= j <= n_ctx + i (and j >= 0),
 *   out_i = sum_j softmax(s)_j v_j.
 * fp32 throughout (fp32 matrix cores).  workspace: vox_enc_attn_workspace(...) bytes of device
 * memory, 16-byte aligned, apart from the other buffers (0 bytes -> may be NULL), contents
 * irrelevant.  m == 0 is a no-op.  head_dim not a multiple of 4 or above 48 ->
 * VOX_E_UNSUPPORTED; q, k, v not 16-byte aligned -> VOX_E_UNSUPPORTED; out overlapping an input ->
 * VOX_E_INVAL; a smaller workspace -> VOX_E_WORKSPACE. */
size_t vox_enc_attn_workspace(int64_t m, int64_t n_ctx, int n_heads, int head_dim, int window);
int vox_enc_attn(const float *q, const float *k, const float *v, float *out, int64_t m, int64_t n_ctx, int n_heads,
                 int head_dim, int window, float scale, void *workspace, size_t workspace_bytes, void *stream);

/* Grouped-query decode attention of one token over a KV ring ([RS] 아키텍처 and [VC] 모델
 * 아키텍처: query head h reads KV head h / (n_q_heads / n_kv_heads); [VC] 주요 기능: rolling
 * window).  q: [n_q_heads][head_dim]; k_cache, v_cache: [n_kv_heads][n_slots][head_dim];
 * out: [n_q_heads][head_dim]; all fp32.  Attends over ring slots [0, n_valid) - the set of
 * cached positions, in any slot order:
 *   s_t = scale * <q_h, K[g][t]>,  out_h = sum_t softmax(s)_t * V[g][t].
 * workspace: at least vox_gqa_decode_attn_workspace(...) bytes of device memory, 16-byte
 * aligned, contents irrelevant.  head_dim must be 128 and n_q_heads / n_kv_heads in
 * {1, 2, 4, 8} (else VOX_E_UNSUPPORTED); 1 <= n_valid <= n_slots (else VOX_E_INVAL). */
size_t vox_gqa_decode_attn_workspace(int n_q_heads, int n_kv_heads, int head_dim, int n_slots);
int vox_gqa_decode_attn(const float *q, const float *k_cache, const float *v_cache, float *out,
                        int n_q_heads, int n_kv_heads, int head_dim, int n_slots, int n_valid,
                        float scale, void *workspace, size_t workspace_bytes, void *stream);

/* The same attention for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): no workspace argument and no
 * allocation of any kind.  The split partials live in a fixed device array of the library,
 * 1 MiB (1,048,576 bytes), one copy per GPU, held until the process ends; the partials need
 * n_q_heads * min(32, ceil(n_slots / 128)) * 528 bytes (540,672 at 32 heads over 8192 slots),
 * and a request beyond the array returns VOX_E_UNSUPPORTED before any device work.  Every call
 * on one GPU shares that array: calls that overlap in time on one GPU (different streams, or
 * other host threads) race and their results are undefined; calls on one stream are ordered.
 * Arguments, results and other errors as vox_gqa_decode_attn; the first call on a device also
 * looks up the array's device address (VOX_E_HIP if that fails). */
int vox_gqa_decode_attn_noalloc(const float *q, const float *k_cache, const float *v_cache, float *out,
                                int n_q_heads, int n_kv_heads, int head_dim, int n_slots, int n_valid,
                                float scale, void *stream);

/* The greedy token and its alternatives from one step's logits ([VC] 사용 방법: --alt <cutoff>
 * lists candidate tokens beside the chosen one, more for a higher cutoff; [VC] C API 구조: the
 * number of alternatives is set per stream).  With t the largest logit (lowest index on a tie),
 * token i is listed when logits[i] >= logits[t] + d, the sum taken in fp32 with d = ln(1 - cutoff)
 * rounded to fp32 (every token when cutoff >= 1): its probability is at least (1 - cutoff) times
 * t's.  The list (t first) runs by logit, higher first, ties to the lower index, at most max_out
 * entries: ids[j] and probs[j] (softmax over all vocab logits, fp32), *count = its length; entries
 * past the count are left untouched.  logits: vocab fp32 values, no NaN.  ids, probs: max_out
 * entries; count: one int32; all device memory.  workspace: vox_alt_tokens_workspace(vocab,
 * max_out) bytes, 8-byte aligned, contents irrelevant.  vocab < 1, cutoff < 0 or NaN, max_out < 1
 * -> VOX_E_INVAL; vocab > 262144 or max_out > 32 -> VOX_E_UNSUPPORTED. */
size_t vox_alt_tokens_workspace(int64_t vocab, int max_out);
int vox_alt_tokens(const float *logits, int64_t vocab, float cutoff, int max_out, int32_t *ids, float *probs,
                   int32_t *count, void *workspace, size_t workspace_bytes, void *stream);

/* ------------------------------------------------------------------------------------
 * Whole decoder step ([VC] 모델 아키텍처, 주요 기능, 성능 벤치마크).  Per token:
 *   h = dequant(tok_embd[token]);
 *   per layer: x = RMSNorm(h)*attn_norm; q,k,v = Wq x, Wk x, Wv x; RoPE(q, k) at the absolute
 *   position (interleaved pairs); K/V written to ring slot pos % n_slots; grouped attention
 *   over min(pos+1, n_slots) slots with scale 1/sqrt(head_dim); h += Wo o;
 *   x = RMSNorm(h)*ffn_norm; h += Wdown (silu(Wgate x) * (Wup x));
 *   logits = tok_embd * (RMSNorm(h)*out_norm)  (tied Q4_0 table as LM head);
 *   token_out = first index of the largest logit; pos += 1.
 * The whole step is captured once as a HIP graph and replayed, so a token costs one
 * submission; position and token ids stay on the device between steps.
 * ---------------------------------------------------------------------------------- */

typedef struct vox_decoder vox_decoder_t;   /* opaque */

typedef struct {
    int n_layers, dim, n_heads, n_kv_heads, head_dim, hidden, vocab, n_slots;
    float norm_eps, rope_theta;
} vox_decoder_config;

typedef struct {
    const float *attn_norm, *ffn_norm;                          /* [dim] fp32 */
    const void *wq, *wk, *wv, *wo, *w_gate, *w_up, *w_down;     /* Q4_0 */
} vox_layer_weights;

typedef struct {
    const void *tok_embd;                 /* Q4_0 [vocab][dim], embedding and LM head */
    const float *out_norm;                /* [dim] */
    const vox_layer_weights *layers;      /* host array of n_layers (copied at create) */
} vox_decoder_weights;

/* Sizes of the two caller-allocated device buffers: the KV ring
 * ([n_layers][2][n_kv_heads][n_slots][head_dim] fp32) and the step scratch. */
int vox_decoder_workspace(const vox_decoder_config *c, size_t *kv_bytes, size_t *scratch_bytes);

/* Creates a decoder over caller-owned weights and buffers (which must outlive it and stay
 * unchanged while work is in flight).  Supported shapes: head_dim 128, n_heads/n_kv_heads in
 * {1,2,4,8}, n_kv_heads <= 64, and the width triple (dim, n_heads*head_dim, hidden) drawn from
 * dim in {3072, 1024}, n_heads*head_dim in {4096, 1024}, hidden in {9216, 2048} (the Voxtral
 * decoder and a small test shape); anything else returns VOX_E_UNSUPPORTED.
 * Enqueues the initialisation of the scratch (position 0, RoPE tables) on `stream`. */
int vox_decoder_create(const vox_decoder_config *c, const vox_decoder_weights *w, void *kv,
                       size_t kv_bytes, void *scratch, size_t scratch_bytes, void *stream,
                       vox_decoder_t **out);
/* The same decoder over 16-bit weights (voxtral.c page, GeekNews 26608, section 모델 다운로드 및
 * 구성: BF16 weights; section 메모리 요구사항: converted to F16 for the GPU): every layer matrix and
 * the tied table tok_embd are n x k row-major 16-bit values, fmt VOX_W16_BF16 or VOX_W16_F16 (the
 * vox_layer_weights pointers then point at them; 16-byte aligned).  Everything else as
 * vox_decoder_create; another fmt -> VOX_E_INVAL. */
int vox_decoder_create_w16(const vox_decoder_config *c, const vox_decoder_weights *w, int fmt, void *kv,
                           size_t kv_bytes, void *scratch, size_t scratch_bytes, void *stream, vox_decoder_t **out);
/* Position back to 0 (the KV window is logically emptied); enqueued on `stream`. */
int vox_decoder_reset(vox_decoder_t *d, void *stream);
/* Resumes a stream at absolute position pos (0 <= pos <= VOX_DECODER_MAX_POS, else VOX_E_INVAL),
 * e.g. one whose KV ring the caller saved and copied back ([VC] 주요 기능: the window rolls over an
 * unbounded stream).  The ring must then hold the keys (after rotation) and values of positions
 * max(0, pos - n_slots) .. pos - 1, position p at slot p % n_slots; the next step is token pos.
 * vox_decoder_reset is vox_decoder_seek(d, 0).  Enqueued on `stream`. */
#define VOX_DECODER_MAX_POS ((int64_t)1 << 40)
int vox_decoder_seek(vox_decoder_t *d, int64_t pos, void *stream);
/* One token: reads token_in[0] (device int32 in [0, vocab); an id outside is clamped to the
 * range), writes token_out[0] (device int32) and, when logits is not NULL, logits[vocab] fp32.
 * token_out may equal token_in. */
int vox_decoder_step(vox_decoder_t *d, const int32_t *token_in, int32_t *token_out, float *logits,
                     void *stream);
/* Number of steps taken since create/reset (the absolute position of the next token). */
int vox_decoder_position(const vox_decoder_t *d, int64_t *pos);
/* 1 (default): replay a captured HIP graph per step; 0: launch the kernels directly. */
int vox_decoder_set_graph(vox_decoder_t *d, int enable);
void vox_decoder_destroy(vox_decoder_t *d);

#ifdef __cplusplus
}
#endif
#endif /* VOX_H */
