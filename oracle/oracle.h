/* oracle.h - CPU oracle for the streaming Voxtral decoder-step hot path.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the package smoke check and the
 * CPU-baseline leg of the benchmark may load this library.  The product path never
 * links, loads or calls it, and it shares no code with the HIP library.
 *
 * Plain scalar C in double precision, written from the definitions; see oracle.c for
 * the passage of the source pages each function follows.
 */
#ifndef VOX_ORACLE_H
#define VOX_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Number formats */
double orc_fp16_to_double(uint16_t h);
double orc_bf16_to_double(uint16_t b);
void orc_fp16_to_double_array(const uint16_t *h, int64_t n, double *out);
void orc_bf16_to_double_array(const uint16_t *b, int64_t n, double *out);

/* GGUF Q4_0 */
void orc_q4_dequant(const uint8_t *blocks, int64_t n_blocks, float *out);
void orc_q4_gemv(const uint8_t *w, const float *x, double *y, int64_t n, int64_t k);
void orc_q4_gemv_f64(const uint8_t *w, const double *x, double *y, int64_t n, int64_t k);
void orc_q4_gemv_rows(const uint8_t *w, const float *x, const int64_t *rows, int64_t n_rows,
                      double *y, int64_t k);
void orc_q4_gemm(const uint8_t *w, const uint16_t *x_bf16, double *y, int64_t m, int64_t n, int64_t k);

/* 16-bit weights (fmt 0: bf16, 1: fp16) */
void orc_w16_gemv(const uint16_t *w, int64_t fmt, const float *x, double *y, int64_t n, int64_t k);

/* Adapter: linear, GELU, linear */
double orc_gelu(double x);
void orc_gelu_array(const double *x, int64_t n, double *out);
void orc_adapter(const uint8_t *w1, const uint8_t *w2, const uint16_t *x_bf16, double *y, int64_t m,
                 int64_t k, int64_t n_mid, int64_t n_out);

/* Encoder self-attention over a chunk (causal, sliding window) */
void orc_enc_attn(const double *q, const double *k, const double *v, int64_t m, int64_t n_ctx,
                  int64_t n_heads, int64_t head_dim, int64_t window, double scale, double *out);

/* Decoder pieces */
void orc_rmsnorm(const double *x, const float *g, int64_t dim, double eps, double *out);
void orc_rope(double *x, int64_t n_heads, int64_t head_dim, int64_t pos, double theta);
void orc_attn_probs(const double *q, const double *k, int64_t len, int64_t head_dim,
                    int64_t stride_t, double scale, double *p);
void orc_gqa_attn(const double *q, const double *k, const double *v, int64_t n_q_heads,
                  int64_t n_kv_heads, int64_t head_dim, int64_t len, double scale, double *out);
void orc_swiglu(const double *gate, const double *up, int64_t n, double *out);
int64_t orc_argmax_f32(const float *v, int64_t n);
int64_t orc_argmax_f64(const double *v, int64_t n);

/* Alternative tokens: candidates within ln(1 - cutoff) of the top logit, listed by logit */
int64_t orc_alt_tokens(const float *logits, int64_t vocab, double cutoff, int64_t max_out, int64_t *ids,
                       double *probs);

/* OpenMP threads used by the loops (timing only; results do not depend on it). */
void orc_set_num_threads(int64_t n);
int64_t orc_max_threads(void);

/* Whole decoder step */
typedef struct {
    int64_t n_layers, dim, n_heads, n_kv_heads, head_dim, hidden, vocab, n_slots;
    double norm_eps, rope_theta;
} orc_decoder_config;

typedef struct {
    const float *attn_norm, *ffn_norm;
    const uint8_t *wq, *wk, *wv, *wo, *w_gate, *w_up, *w_down;
} orc_layer_weights;

typedef struct orc_decoder orc_decoder;

orc_decoder *orc_decoder_create(const orc_decoder_config *c, const uint8_t *tok_embd,
                                const float *out_norm, const orc_layer_weights *layers);
/* The same step over 16-bit weights: every matrix n x k uint16, row-major, fmt 0 bf16, fmt 1
 * IEEE binary16 (the orc_layer_weights pointers then point at uint16 arrays). */
orc_decoder *orc_decoder_create_w16(const orc_decoder_config *c, int64_t fmt, const uint16_t *tok_embd,
                                    const float *out_norm, const orc_layer_weights *layers);
void orc_decoder_destroy(orc_decoder *d);
void orc_decoder_reset(orc_decoder *d);
int64_t orc_decoder_position(const orc_decoder *d);
/* Resumes at position pos with the window given as k, v [n_layers][len][n_kv][hd] (fp32),
 * oldest first, len = min(pos, n_slots). */
void orc_decoder_load_window(orc_decoder *d, int64_t pos, const float *k, const float *v);
/* One step on `token`.  Writes logits[vocab] (double) when non-NULL and returns the
 * greedy next token: the first index of the largest logit, taken over fp32 logits. */
int64_t orc_decoder_step(orc_decoder *d, int64_t token, double *logits);
/* The residual stream after the last step (dim doubles); for diagnostics. */
const double *orc_decoder_hidden(const orc_decoder *d);

#ifdef __cplusplus
}
#endif
#endif
