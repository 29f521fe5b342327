/* oracle.c - CPU oracle for the streaming Voxtral decoder-step hot path.
 *
 * TEST INFRASTRUCTURE ONLY: loaded by the test suite, the package smoke check and the
 * CPU-baseline leg of the benchmark; never by the product path.  Shares no code with
 * the HIP library.
 *
 * Everything is computed in double precision with plain loops in the order the
 * definitions state (sums run over the input index in ascending order).  OpenMP only
 * splits independent output rows or heads across threads; every output is still
 * produced by one thread in one fixed order.
 *
 * Source pages (web pages on the streaming Voxtral Mini 4B Realtime model):
 *  [RS] "Mistral의 Voxtral Mini 4B Realtime 모델을 Rust로 구현해 브라우저에서 실행"
 *       (GeekNews 26595) - Rust/Burn port with a GGUF Q4_0 path.
 *  [VC] "Mistral Voxtral Realtime 4B 음성 인식 모델의 순수 C 기반 CPU 전용 추론 구현"
 *       (GeekNews 26608) - voxtral.c.
 *  [RB] "Voxtral Mini 4B: Rust로 구현한 브라우저 실시간 음성 인식" (rebugui blog).
 * The pages name the pieces (GGUF Q4_0 linears, a Ministral-3 style decoder with GQA
 * 32Q/8KV, a rolling 8192-position KV cache, greedy decoding) but print no formulas;
 * where they are silent the plainest reading is taken and marked READING.
 */
#include "oracle.h"

#include <math.h>
#include <omp.h>
#include <stdlib.h>
#include <string.h>

/* Threads of the OpenMP loops below (for timing the oracle at a chosen thread count). */
void orc_set_num_threads(int64_t n) { omp_set_num_threads(n > 0 ? (int)n : 1); }
int64_t orc_max_threads(void) { return omp_get_max_threads(); }

/* ------------------------------------------------------------------------------------
 * Number formats
 * ---------------------------------------------------------------------------------- */

/* IEEE binary16: sign bit 15, exponent bits 14..10 (bias 15), fraction bits 9..0.
 * Used for the Q4_0 block scale ([RS] section 아키텍처 names GGUF Q4_0). */
double orc_fp16_to_double(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 31;
    int m = h & 1023;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24);                 /* zero or subnormal: m * 2^-24 */
    else if (e < 31)
        v = ldexp((double)(1024 + m), e - 25);     /* normal: (1 + m/1024) * 2^(e-15) */
    else
        v = m ? NAN : INFINITY;
    return sign ? -v : v;
}

/* bfloat16 is the upper half of an IEEE binary32. */
double orc_bf16_to_double(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

void orc_fp16_to_double_array(const uint16_t *h, int64_t n, double *out)
{
    for (int64_t i = 0; i < n; i++)
        out[i] = orc_fp16_to_double(h[i]);
}

void orc_bf16_to_double_array(const uint16_t *b, int64_t n, double *out)
{
    for (int64_t i = 0; i < n; i++)
        out[i] = orc_bf16_to_double(b[i]);
}

/* ------------------------------------------------------------------------------------
 * GGUF Q4_0 ([RS] section 아키텍처: the quantised path stores its linears as GGUF Q4_0;
 * the pages do not spell out the bytes, so this is the GGUF definition of the block):
 * 18 bytes per 32 weights.  Bytes 0..1: scale d, fp16, little-endian.  Byte 2+j
 * (j = 0..15): low nibble = code of weight j, high nibble = code of weight j+16.
 * Weight value = (code - 8) * d.
 * ---------------------------------------------------------------------------------- */

static void q4_block_values(const uint8_t *blk, double v[32])
{
    double d = orc_fp16_to_double((uint16_t)(blk[0] | (blk[1] << 8)));
    for (int j = 0; j < 16; j++) {
        int lo = blk[2 + j] & 15;
        int hi = blk[2 + j] >> 4;
        v[j] = (double)(lo - 8) * d;
        v[j + 16] = (double)(hi - 8) * d;
    }
}

/* The product of a 4-bit integer and an fp16 value has at most 15 significant bits,
 * so the double result converts to fp32 exactly. */
void orc_q4_dequant(const uint8_t *blocks, int64_t n_blocks, float *out)
{
    for (int64_t b = 0; b < n_blocks; b++) {
        double v[32];
        q4_block_values(blocks + b * 18, v);
        for (int j = 0; j < 32; j++)
            out[b * 32 + j] = (float)v[j];
    }
}

/* y[r] = sum over k ascending of W[r][k] * x[k]; row r is k/32 consecutive blocks. */
static double q4_row_dot(const uint8_t *row, const double *x, int64_t k)
{
    double acc = 0.0;
    for (int64_t b = 0; b < k / 32; b++) {
        double v[32];
        q4_block_values(row + b * 18, v);
        for (int j = 0; j < 32; j++)
            acc += v[j] * x[b * 32 + j];
    }
    return acc;
}

void orc_q4_gemv_f64(const uint8_t *w, const double *x, double *y, int64_t n, int64_t k)
{
    const int64_t row_bytes = (k / 32) * 18;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < n; r++)
        y[r] = q4_row_dot(w + r * row_bytes, x, k);
}

void orc_q4_gemv(const uint8_t *w, const float *x, double *y, int64_t n, int64_t k)
{
    double *xd = (double *)malloc(sizeof(double) * (size_t)k);
    for (int64_t i = 0; i < k; i++)
        xd[i] = x[i];
    orc_q4_gemv_f64(w, xd, y, n, k);
    free(xd);
}

/* The same dot products for a chosen subset of rows (for spot checks of huge matrices). */
void orc_q4_gemv_rows(const uint8_t *w, const float *x, const int64_t *rows, int64_t n_rows,
                      double *y, int64_t k)
{
    const int64_t row_bytes = (k / 32) * 18;
    double *xd = (double *)malloc(sizeof(double) * (size_t)k);
    for (int64_t i = 0; i < k; i++)
        xd[i] = x[i];
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n_rows; i++)
        y[i] = q4_row_dot(w + rows[i] * row_bytes, xd, k);
    free(xd);
}

/* Y[m][n] = sum over k ascending of X[m][k] * W[n][k], X in double. */
static void q4_gemm_f64(const uint8_t *w, const double *xd, double *y, int64_t m, int64_t n, int64_t k)
{
    const int64_t row_bytes = (k / 32) * 18;
#pragma omp parallel for schedule(static)
    for (int64_t c = 0; c < n; c++) {
        double *wrow = (double *)malloc(sizeof(double) * (size_t)k);
        for (int64_t b = 0; b < k / 32; b++)
            q4_block_values(w + c * row_bytes + b * 18, wrow + b * 32);
        for (int64_t r = 0; r < m; r++) {
            double acc = 0.0;
            for (int64_t i = 0; i < k; i++)
                acc += xd[r * k + i] * wrow[i];
            y[r * n + c] = acc;
        }
        free(wrow);
    }
}

/* Encoder-chunk linear: Y[m][n] = sum over k ascending of bf16(X[m][k]) * W[n][k]
 * ([VC] section 모델 아키텍처: encoder width 1280; [RS] section 아키텍처: Q4_0 linears). */
void orc_q4_gemm(const uint8_t *w, const uint16_t *x_bf16, double *y, int64_t m, int64_t n, int64_t k)
{
    double *xd = (double *)malloc(sizeof(double) * (size_t)(m * k));
    for (int64_t i = 0; i < m * k; i++)
        xd[i] = orc_bf16_to_double(x_bf16[i]);
    q4_gemm_f64(w, xd, y, m, n, k);
    free(xd);
}

/* ------------------------------------------------------------------------------------
 * 16-bit weights ([VC] section 모델 다운로드 및 구성: the weights ship as BF16; section 메모리
 * 요구사항: the GPU cache holds them converted from BF16 to F16).  y[r] = sum over k ascending of
 * W[r][k] * x[k], W row-major n x k of bf16 (fmt 0) or IEEE binary16 (fmt 1) bit patterns.
 * ---------------------------------------------------------------------------------- */
void orc_w16_gemv(const uint16_t *w, int64_t fmt, const float *x, double *y, int64_t n, int64_t k)
{
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < n; r++) {
        double acc = 0.0;
        for (int64_t i = 0; i < k; i++) {
            const uint16_t b = w[r * k + i];
            acc += (fmt ? orc_fp16_to_double(b) : orc_bf16_to_double(b)) * (double)x[i];
        }
        y[r] = acc;
    }
}

/* ------------------------------------------------------------------------------------
 * Adapter from the encoder to the decoder ([VC] section 모델 아키텍처: a linear from 5120 to
 * 3072 inputs, GELU, a linear from 3072 to 3072).  READINGS: no biases (the pages name none,
 * and the Q4_0 linears of the quantised path carry none); GELU is the exact form
 * x * Phi(x) with Phi the standard normal distribution function, not the tanh approximation;
 * the GELU output enters the second linear unrounded (here in double).
 * ---------------------------------------------------------------------------------- */

/* GELU(x) = x * Phi(x), Phi(x) = (1 + erf(x / sqrt 2)) / 2 = erfc(-x / sqrt 2) / 2 (the erfc form
 * keeps full relative precision where Phi is tiny, far below zero). */
double orc_gelu(double x)
{
    return 0.5 * x * erfc(-x / sqrt(2.0));
}

void orc_gelu_array(const double *x, int64_t n, double *out)
{
    for (int64_t i = 0; i < n; i++)
        out[i] = orc_gelu(x[i]);
}

/* Y[m][n_out] = GELU(X W1^T) W2^T: X bf16 [m][k], W1 Q4_0 [n_mid][k], W2 Q4_0 [n_out][n_mid];
 * both products, GELU and the intermediate in double. */
void orc_adapter(const uint8_t *w1, const uint8_t *w2, const uint16_t *x_bf16, double *y, int64_t m,
                 int64_t k, int64_t n_mid, int64_t n_out)
{
    double *h = (double *)malloc(sizeof(double) * (size_t)(m * n_mid));
    orc_q4_gemm(w1, x_bf16, h, m, n_mid, k);
    for (int64_t i = 0; i < m * n_mid; i++)
        h[i] = orc_gelu(h[i]);
    q4_gemm_f64(w2, h, y, m, n_out, n_mid);
    free(h);
}

/* ------------------------------------------------------------------------------------
 * Encoder self-attention over a chunk ([VC] section 모델 아키텍처: the audio encoder is a causal
 * transformer, 1280 wide, 32 heads, window 750; section 주요 기능: the encoder runs over chunks of
 * the audio).  READINGS: the window counts the query's own position (a query at position p sees
 * keys p - window + 1 .. p); scores are scaled by 1/sqrt(head_dim); positions are already in q and
 * k when they arrive (nothing positional inside the operation); keys before the chunk come from the
 * previous chunks' K/V.
 * Layout: q [m][n_heads*head_dim] holds the chunk's queries; k, v [n_ctx + m][n_heads*head_dim]
 * hold n_ctx earlier positions followed by the chunk's own, so query i is at row n_ctx + i of k.
 * out [m][n_heads*head_dim].
 * ---------------------------------------------------------------------------------- */
void orc_enc_attn(const double *q, const double *k, const double *v, int64_t m, int64_t n_ctx,
                  int64_t n_heads, int64_t head_dim, int64_t window, double scale, double *out)
{
    const int64_t width = n_heads * head_dim;
#pragma omp parallel for schedule(static) collapse(2)
    for (int64_t i = 0; i < m; i++)
        for (int64_t h = 0; h < n_heads; h++) {
            const int64_t last = n_ctx + i;                          /* the query's own row */
            const int64_t first = last - window + 1 > 0 ? last - window + 1 : 0;
            const int64_t len = last - first + 1;
            double *p = (double *)malloc(sizeof(double) * (size_t)len);
            orc_attn_probs(q + i * width + h * head_dim, k + first * width + h * head_dim, len, head_dim,
                           width, scale, p);
            for (int64_t d = 0; d < head_dim; d++) {
                double acc = 0.0;
                for (int64_t t = 0; t < len; t++)
                    acc += p[t] * v[(first + t) * width + h * head_dim + d];
                out[i * width + h * head_dim + d] = acc;
            }
            free(p);
        }
}

/* ------------------------------------------------------------------------------------
 * Decoder pieces.  [VC] section 모델 아키텍처: the LLM decoder is a 26-layer transformer
 * "based on Ministral-3" with GQA (32 heads / 8 KV heads).  READING: a Llama-style
 * pre-norm block - RMSNorm, attention with rotary positions, residual add, RMSNorm,
 * SwiGLU feed-forward, residual add; no biases.
 * ---------------------------------------------------------------------------------- */

/* RMSNorm: out_i = x_i / sqrt(mean(x^2) + eps) * g_i  (eps inside the root). */
void orc_rmsnorm(const double *x, const float *g, int64_t dim, double eps, double *out)
{
    double ss = 0.0;
    for (int64_t i = 0; i < dim; i++)
        ss += x[i] * x[i];
    double inv = 1.0 / sqrt(ss / (double)dim + eps);
    for (int64_t i = 0; i < dim; i++)
        out[i] = x[i] * inv * (double)g[i];
}

/* Rotary position embedding at absolute position `pos` (READING: interleaved pairs).
 * Head vector x[h*hd .. h*hd+hd); pair i = (x[2i], x[2i+1]) rotated by angle
 * pos * theta^(-2i/hd). */
void orc_rope(double *x, int64_t n_heads, int64_t head_dim, int64_t pos, double theta)
{
    for (int64_t h = 0; h < n_heads; h++) {
        double *v = x + h * head_dim;
        for (int64_t i = 0; i < head_dim / 2; i++) {
            double freq = pow(theta, -2.0 * (double)i / (double)head_dim);
            double a = (double)pos * freq;
            double c = cos(a), s = sin(a);
            double x0 = v[2 * i], x1 = v[2 * i + 1];
            v[2 * i] = x0 * c - x1 * s;
            v[2 * i + 1] = x0 * s + x1 * c;
        }
    }
}

/* Softmax weights of one query head over `len` keys: s_t = scale * <q, k_t>;
 * p_t = exp(s_t - max s) / sum_u exp(s_u - max s).  Key t starts at k + t*stride_t. */
void orc_attn_probs(const double *q, const double *k, int64_t len, int64_t head_dim,
                    int64_t stride_t, double scale, double *p)
{
    double mx = -INFINITY;
    for (int64_t t = 0; t < len; t++) {
        double s = 0.0;
        for (int64_t d = 0; d < head_dim; d++)
            s += q[d] * k[t * stride_t + d];
        p[t] = s * scale;
        if (p[t] > mx)
            mx = p[t];
    }
    double z = 0.0;
    for (int64_t t = 0; t < len; t++) {
        p[t] = exp(p[t] - mx);
        z += p[t];
    }
    for (int64_t t = 0; t < len; t++)
        p[t] /= z;
}

/* Grouped-query attention of one new token over a chronological list of `len` cached
 * keys/values ([RS] section 아키텍처 and [VC] section 모델 아키텍처: 32 query heads share
 * 8 KV heads).  Query head h reads KV head h / (n_q_heads / n_kv_heads).
 * Layouts: q [n_q][hd]; k, v [n_kv][len][hd]; out [n_q][hd]. */
static void gqa_attn_strided(const double *q, const double *k, const double *v, int64_t n_q_heads,
                             int64_t n_kv_heads, int64_t head_dim, int64_t len, int64_t stride_g,
                             int64_t stride_t, double scale, double *out)
{
    const int64_t group = n_q_heads / n_kv_heads;
#pragma omp parallel for schedule(static)
    for (int64_t h = 0; h < n_q_heads; h++) {
        const int64_t g = h / group;
        double *p = (double *)malloc(sizeof(double) * (size_t)len);
        orc_attn_probs(q + h * head_dim, k + g * stride_g, len, head_dim, stride_t, scale, p);
        for (int64_t d = 0; d < head_dim; d++) {
            double acc = 0.0;
            for (int64_t t = 0; t < len; t++)
                acc += p[t] * v[g * stride_g + t * stride_t + d];
            out[h * head_dim + d] = acc;
        }
        free(p);
    }
}

void orc_gqa_attn(const double *q, const double *k, const double *v, int64_t n_q_heads,
                  int64_t n_kv_heads, int64_t head_dim, int64_t len, double scale, double *out)
{
    gqa_attn_strided(q, k, v, n_q_heads, n_kv_heads, head_dim, len, len * head_dim, head_dim,
                     scale, out);
}

/* SwiGLU (READING: silu on the gate, times the up projection): a_i = g_i / (1 + e^-g_i) * u_i. */
void orc_swiglu(const double *gate, const double *up, int64_t n, double *out)
{
    for (int64_t i = 0; i < n; i++)
        out[i] = gate[i] / (1.0 + exp(-gate[i])) * up[i];
}

/* Greedy decoding takes the most likely token ([RB] section 구현 및 코드 예시 sketches a
 * decode step ending in an argmax over the last logits).  Ties go to the lowest index. */
int64_t orc_argmax_f32(const float *v, int64_t n)
{
    int64_t best = 0;
    for (int64_t i = 1; i < n; i++)
        if (v[i] > v[best])
            best = i;
    return best;
}

int64_t orc_argmax_f64(const double *v, int64_t n)
{
    int64_t best = 0;
    for (int64_t i = 1; i < n; i++)
        if (v[i] > v[best])
            best = i;
    return best;
}

/* ------------------------------------------------------------------------------------
 * Alternative tokens ([VC] section 사용 방법: --alt <cutoff> shows candidate tokens beside the
 * chosen one, more of them for a higher cutoff; section C API 구조: the number of alternatives is
 * set on the stream).  READING: with p = softmax(logits) and t the greedy token, a token i is a
 * candidate when p_i >= (1 - cutoff) p_t, i.e. l_i >= l_t + ln(1 - cutoff); the comparison is made
 * on the fp32 logits against tau = l_t + d in fp32 arithmetic, d = ln(1 - cutoff) rounded to fp32
 * (cutoff >= 1: every token).  The candidates (the greedy token first) are listed by logit, higher
 * first, ties to the lower index, at most max_out of them, each with its probability (double).
 * Returns the count.
 * ---------------------------------------------------------------------------------- */
static int alt_before(const float *l, int64_t a, int64_t b)   /* a listed before b */
{
    return l[a] > l[b] || (l[a] == l[b] && a < b);
}

int64_t orc_alt_tokens(const float *logits, int64_t vocab, double cutoff, int64_t max_out, int64_t *ids,
                       double *probs)
{
    const int64_t top = orc_argmax_f32(logits, vocab);
    const float lt = logits[top];
    const float d = cutoff >= 1.0 ? -INFINITY : (float)log(1.0 - cutoff);
    const float tau = lt + d;
    double z = 0.0;
    for (int64_t i = 0; i < vocab; i++)
        z += exp((double)logits[i] - (double)lt);
    /* selection by insertion into the sorted output list */
    int64_t count = 0;
    for (int64_t i = 0; i < vocab; i++) {
        if (!(logits[i] >= tau))
            continue;
        int64_t pos = count;
        while (pos > 0 && alt_before(logits, i, ids[pos - 1]))
            pos--;
        if (pos >= max_out)
            continue;
        int64_t end = count < max_out ? count : max_out - 1;
        for (int64_t j = end; j > pos; j--)
            ids[j] = ids[j - 1];
        ids[pos] = i;
        if (count < max_out)
            count++;
    }
    for (int64_t j = 0; j < count; j++)
        probs[j] = exp((double)logits[ids[j]] - (double)lt) / z;
    return count;
}

/* ------------------------------------------------------------------------------------
 * Whole decoder step.
 * ---------------------------------------------------------------------------------- */

struct orc_decoder {
    orc_decoder_config c;
    int64_t wfmt;      /* -1: Q4_0 weights; 0: bf16; 1: IEEE binary16 */
    const uint8_t *tok_embd;
    const float *out_norm;
    orc_layer_weights *layers;
    int64_t pos;       /* absolute position of the next token */
    int64_t len;       /* number of cached positions, <= n_slots */
    int64_t cap;       /* allocated positions per layer */
    double **kcache;   /* per layer: [cap][n_kv][hd], chronological, oldest first */
    double **vcache;
    double *h;         /* residual stream [dim] */
};

orc_decoder *orc_decoder_create(const orc_decoder_config *c, const uint8_t *tok_embd,
                                const float *out_norm, const orc_layer_weights *layers)
{
    orc_decoder *d = (orc_decoder *)calloc(1, sizeof *d);
    d->c = *c;
    d->wfmt = -1;
    d->tok_embd = tok_embd;
    d->out_norm = out_norm;
    d->layers = (orc_layer_weights *)malloc(sizeof(orc_layer_weights) * (size_t)c->n_layers);
    memcpy(d->layers, layers, sizeof(orc_layer_weights) * (size_t)c->n_layers);
    d->kcache = (double **)calloc((size_t)c->n_layers, sizeof(double *));
    d->vcache = (double **)calloc((size_t)c->n_layers, sizeof(double *));
    d->h = (double *)calloc((size_t)c->dim, sizeof(double));
    return d;
}

/* The same decoder over 16-bit weights (voxtral.c page, section 모델 다운로드 및 구성: BF16
 * weights; section 메모리 요구사항: converted to F16 for the GPU).  Every matrix (the layers'
 * linears and the tied embedding / LM head) holds n x k 16-bit patterns, row-major: fmt 0 bf16,
 * fmt 1 IEEE binary16; the layer pointers of orc_layer_weights point at those uint16 arrays. */
orc_decoder *orc_decoder_create_w16(const orc_decoder_config *c, int64_t fmt, const uint16_t *tok_embd,
                                    const float *out_norm, const orc_layer_weights *layers)
{
    orc_decoder *d = orc_decoder_create(c, (const uint8_t *)tok_embd, out_norm, layers);
    d->wfmt = fmt ? 1 : 0;
    return d;
}

void orc_decoder_destroy(orc_decoder *d)
{
    if (!d)
        return;
    for (int64_t l = 0; l < d->c.n_layers; l++) {
        free(d->kcache[l]);
        free(d->vcache[l]);
    }
    free(d->kcache);
    free(d->vcache);
    free(d->layers);
    free(d->h);
    free(d);
}

void orc_decoder_reset(orc_decoder *d)
{
    d->pos = 0;
    d->len = 0;
}

int64_t orc_decoder_position(const orc_decoder *d) { return d->pos; }

static void ensure_capacity(orc_decoder *d, int64_t need);

/* Resumes a stream at absolute position pos with a given window ([VC] section 주요 기능: the
 * window rolls over an unbounded stream, keeping the last 8192 positions).  k and v hold, per
 * layer, the keys (already rotated) and values of positions pos - len .. pos - 1, oldest first,
 * len = min(pos, n_slots), each row n_kv*head_dim floats: layout [n_layers][len][n_kv][hd]. */
void orc_decoder_load_window(orc_decoder *d, int64_t pos, const float *k, const float *v)
{
    const int64_t len = pos < d->c.n_slots ? pos : d->c.n_slots;
    const int64_t row = d->c.n_kv_heads * d->c.head_dim;
    ensure_capacity(d, len);
    for (int64_t l = 0; l < d->c.n_layers; l++)
        for (int64_t i = 0; i < len * row; i++) {
            d->kcache[l][i] = (double)k[(l * len) * row + i];
            d->vcache[l][i] = (double)v[(l * len) * row + i];
        }
    d->pos = pos;
    d->len = len;
}

const double *orc_decoder_hidden(const orc_decoder *d) { return d->h; }

/* Rolling KV window ([VC] section 주요 기능: an 8192-position sliding window whose cache
 * compacts itself, so audio length is unbounded).  The list is kept oldest-first; when it
 * is full the oldest entry is dropped before the new one is appended.  READING: the window
 * includes the current token (append first, then attend over min(pos+1, n_slots)). */
static void kv_append(orc_decoder *d, int64_t layer, const double *k, const double *v)
{
    const int64_t row = d->c.n_kv_heads * d->c.head_dim;
    double *kc = d->kcache[layer], *vc = d->vcache[layer];
    if (d->len == d->c.n_slots) {
        memmove(kc, kc + row, sizeof(double) * (size_t)((d->len - 1) * row));
        memmove(vc, vc + row, sizeof(double) * (size_t)((d->len - 1) * row));
        memcpy(kc + (d->len - 1) * row, k, sizeof(double) * (size_t)row);
        memcpy(vc + (d->len - 1) * row, v, sizeof(double) * (size_t)row);
    } else {
        memcpy(kc + d->len * row, k, sizeof(double) * (size_t)row);
        memcpy(vc + d->len * row, v, sizeof(double) * (size_t)row);
    }
}

static void ensure_capacity(orc_decoder *d, int64_t need)
{
    if (need <= d->cap)
        return;
    int64_t cap = d->cap ? d->cap : 64;
    while (cap < need)
        cap *= 2;
    if (cap > d->c.n_slots)
        cap = d->c.n_slots;
    const int64_t row = d->c.n_kv_heads * d->c.head_dim;
    for (int64_t l = 0; l < d->c.n_layers; l++) {
        d->kcache[l] = (double *)realloc(d->kcache[l], sizeof(double) * (size_t)(cap * row));
        d->vcache[l] = (double *)realloc(d->vcache[l], sizeof(double) * (size_t)(cap * row));
    }
    d->cap = cap;
}

/* y = W x in double for the decoder's weight format: Q4_0 rows, or 16-bit rows widened exactly. */
static void dec_linear(const orc_decoder *d, const uint8_t *w, const double *x, double *y, int64_t n, int64_t k)
{
    if (d->wfmt < 0) {
        orc_q4_gemv_f64(w, x, y, n, k);
        return;
    }
    const uint16_t *w16 = (const uint16_t *)w;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < n; r++) {
        double acc = 0.0;
        for (int64_t i = 0; i < k; i++) {
            const uint16_t b = w16[r * k + i];
            acc += (d->wfmt ? orc_fp16_to_double(b) : orc_bf16_to_double(b)) * x[i];
        }
        y[r] = acc;
    }
}

int64_t orc_decoder_step(orc_decoder *d, int64_t token, double *logits)
{
    const orc_decoder_config *c = &d->c;
    const int64_t dim = c->dim, hd = c->head_dim;
    const int64_t qd = c->n_heads * hd, kvd = c->n_kv_heads * hd;
    const int64_t row_bytes = (dim / 32) * 18;
    const int64_t new_len = d->len < c->n_slots ? d->len + 1 : c->n_slots;
    ensure_capacity(d, new_len);

    double *xn = (double *)malloc(sizeof(double) * (size_t)dim);
    double *q = (double *)malloc(sizeof(double) * (size_t)qd);
    double *k = (double *)malloc(sizeof(double) * (size_t)kvd);
    double *v = (double *)malloc(sizeof(double) * (size_t)kvd);
    double *o = (double *)malloc(sizeof(double) * (size_t)qd);
    double *y = (double *)malloc(sizeof(double) * (size_t)dim);
    double *gt = (double *)malloc(sizeof(double) * (size_t)c->hidden);
    double *up = (double *)malloc(sizeof(double) * (size_t)c->hidden);
    double *a = (double *)malloc(sizeof(double) * (size_t)c->hidden);
    double *lg = logits ? logits : (double *)malloc(sizeof(double) * (size_t)c->vocab);

    /* Input: the token's row of the tied embedding table ([RS] section 브라우저 실행을 위한 기술적
     * 해결: the embedding stays on the GPU as Q4 and a row is looked up per token), Q4_0 or 16-bit. */
    if (d->wfmt < 0) {
        for (int64_t b = 0; b < dim / 32; b++)
            q4_block_values(d->tok_embd + token * row_bytes + b * 18, d->h + b * 32);
    } else {
        const uint16_t *row = (const uint16_t *)d->tok_embd + token * dim;
        for (int64_t i = 0; i < dim; i++)
            d->h[i] = d->wfmt ? orc_fp16_to_double(row[i]) : orc_bf16_to_double(row[i]);
    }

    const double scale = 1.0 / sqrt((double)hd);
    for (int64_t l = 0; l < c->n_layers; l++) {
        const orc_layer_weights *L = &d->layers[l];
        /* attention block */
        orc_rmsnorm(d->h, L->attn_norm, dim, c->norm_eps, xn);
        dec_linear(d, L->wq, xn, q, qd, dim);
        dec_linear(d, L->wk, xn, k, kvd, dim);
        dec_linear(d, L->wv, xn, v, kvd, dim);
        orc_rope(q, c->n_heads, hd, d->pos, c->rope_theta);
        orc_rope(k, c->n_kv_heads, hd, d->pos, c->rope_theta);
        kv_append(d, l, k, v);
        /* cached rows are [t][n_kv][hd]: head stride hd, time stride n_kv*hd */
        gqa_attn_strided(q, d->kcache[l], d->vcache[l], c->n_heads, c->n_kv_heads, hd, new_len,
                         hd, kvd, scale, o);
        dec_linear(d, L->wo, o, y, dim, qd);
        for (int64_t i = 0; i < dim; i++)
            d->h[i] += y[i];
        /* feed-forward block */
        orc_rmsnorm(d->h, L->ffn_norm, dim, c->norm_eps, xn);
        dec_linear(d, L->w_gate, xn, gt, c->hidden, dim);
        dec_linear(d, L->w_up, xn, up, c->hidden, dim);
        orc_swiglu(gt, up, c->hidden, a);
        dec_linear(d, L->w_down, a, y, dim, c->hidden);
        for (int64_t i = 0; i < dim; i++)
            d->h[i] += y[i];
    }
    d->len = new_len;

    /* Output: final RMSNorm, then the tied table as LM head, then the greedy choice taken over
     * fp32 logits (the precision the GPU path decides in). */
    orc_rmsnorm(d->h, d->out_norm, dim, c->norm_eps, xn);
    dec_linear(d, d->tok_embd, xn, lg, c->vocab, dim);
    float *lf = (float *)malloc(sizeof(float) * (size_t)c->vocab);
    for (int64_t i = 0; i < c->vocab; i++)
        lf[i] = (float)lg[i];
    int64_t next = orc_argmax_f32(lf, c->vocab);
    free(lf);

    d->pos += 1;
    free(xn); free(q); free(k); free(v); free(o); free(y); free(gt); free(up); free(a);
    if (!logits)
        free(lg);
    return next;
}
