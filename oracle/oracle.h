/*
 * oracle.h -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, double-precision CPU definition of one pre-LayerNorm GPT layer with a KV cache,
 * and of the group-wise symmetric int8 weight quantizer. It exists so that the GPU library can be
 * checked against something that is obviously correct. Only the tests, the smoke check and the
 * CPU-baseline leg of the benchmark may load it; the GPU library never does, and the two share no
 * source, header, table or helper.
 *
 * Sources (cited by page title and section; the pages are the text of public web pages):
 *   [KP]  "DeepSpeed Inference 内核优化深度解析：多 GPU 自适应并行、算子融合推理内核与 MoQ 量化支持"
 *         (blog.gitcode.com) -- section 三 (3.2: the four fusion regions of one transformer layer,
 *         3.3: the mechanisms), section 五 (5.2: int8 inference with quantize_groups), section 四
 *         (4.2: dtype fp32/fp16/int8, max_out_tokens).
 *   [MP]  "DeepSpeed MoE 大规模稀疏模型推理实战指南" (blog.gitcode.com) -- the inference-config table,
 *         row triangular_masking (default True: the attention score mask type); the MoE sections:
 *         a number of experts per MoE layer, MoE types 'standard' and 'residual' (PR-MoE).
 *
 * Where the pages are silent the oracle takes these readings:
 *   LayerNorm uses the biased variance and eps = 1e-5 unless the caller passes another eps;
 *   GeLU is the exact erf form u*Phi(u) unless gelu_tanh is set; the attention scale is 1/sqrt(d);
 *   Q, K, V are rows [0,H), [H,2H), [2H,3H) of the fused projection, head j owning [j*d,(j+1)*d);
 *   the order inside region 3 is Wo -> +bo -> +x -> LN2 -> W1 -> +b1 -> GeLU, then W2 -> +b2 -> +x2;
 *   keys past a row's own position are excluded from its softmax (not added as -inf);
 *   int8 groups are consecutive elements along the reduction dimension of one weight row (64 in
 *   the configs; the caller passes the size, finer for the MLP matrices with mlp_extra_grouping),
 *   scale = fp16_RNE(amax/127), code = clamp(round_half_even(w/scale), -127, 127), amax = 0 -> 0.
 *
 * Layouts: every matrix is [N][K] row-major (K contiguous); activations are [B][T][width];
 * the K and V caches are [B][heads][cap][head_dim]; lens[b] is the number of filled cache rows.
 */
#ifndef DS_ORACLE_H
#define DS_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
  int hidden, heads, head_dim, ffn;
  double ln_eps;
  int gelu_tanh;           /* 0: u*Phi(u) with erf; 1: the tanh approximation            */
  int triangular_masking;  /* 1: row at position p sees keys 0..p; 0: sees every key     */
  int kv_int8;             /* 1: the cache holds each appended K and V row of one head as  */
                           /*    int8 codes with one fp16 scale (ora_quantize_row_i8); the */
                           /*    cache arrays here receive the dequantized values q*s      */
} ora_desc;

typedef struct {
  const double *ln1_g, *ln1_b, *w_qkv, *b_qkv, *w_o, *b_o;
  const double *ln2_g, *ln2_b, *w_ff1, *b_ff1, *w_ff2, *b_ff2;
} ora_weights;

/* Optional per-stage outputs (NULL entries are skipped), each [B][T][width]. */
typedef struct {
  double *ln1;  /* width H  : LN1(x)                         */
  double *qkv;  /* width 3H : Wqkv LN1(x) + bqkv             */
  double *ctx;  /* width H  : attention output, heads concatenated */
  double *x2;   /* width H  : x + Wo ctx + bo                */
  double *ln2;  /* width H  : LN2(x2)                        */
  double *ff1;  /* width F  : W1 LN2(x2) + b1 (pre-activation) */
  double *act;  /* width F  : GeLU of ff1                    */
} ora_stages;

/* ---- single steps ---- */
void   ora_layernorm(const double* x, int n, const double* g, const double* b, double eps, double* out);
void   ora_linear(const double* w, const double* bias, const double* x, int n_out, int k, double* out);
double ora_gelu(double u, int tanh_form);
void   ora_softmax(const double* s, int n, double* p);
/* One query against keys/values 0..nkeys-1 of one head ([nkeys][d] each). */
void   ora_attend(const double* q, const double* keys, const double* vals, int nkeys, int d, double* out);

/* ---- the layer ----
 * Appends the T new rows of K and V at rows lens[b]..lens[b]+T-1, then attends, then advances
 * lens[b] by T. Returns 0, or -1 when a shape is inconsistent or the cache would overflow. */
int ora_layer_forward(const ora_desc* desc, const ora_weights* w, double* k_cache, double* v_cache,
                      int cap, int* lens, const double* x, double* y, int batch, int ntok,
                      ora_stages* stages);

/* ---- the ends of a generation step (the text-generation example of [KP] section 二) ----
 * After the last layer: a final LayerNorm and the LM head, logits = W_vocab LN(y; g, b) with
 * w_vocab [V][H] (no bias), then greedy decoding. */
void ora_lm_head(const double* y, int H, const double* g, const double* b, double eps,
                 const double* w_vocab, int V, double* logits);
/* Greedy choice: the index of the largest of n values; among equal largest values, the smallest
 * index. n >= 1; the values are finite. */
int  ora_argmax(const double* v, int n);

/* ---- the MoE expert FF ([MP]: num_experts per layer, type standard | residual) ----
 * The pages name the experts and the two types but not the gate. Readings:
 * h = LN(x2; ln_g, ln_b); gate logits = W_gate h (no bias); p = softmax over the E experts; the
 * top_k experts are the k largest p, taken one at a time, the smallest index first among equal
 * values; an expert is the dense FF, FF_e(h) = W2_e GeLU(W1_e h + b1_e) + b2_e; the combine
 * weights are the chosen p renormalized to sum 1 (combine 0) or the p themselves (combine 1);
 * 'residual' adds a dense MLP of the same form: y = x2 + sum_i w_i FF_{e_i}(h) [+ FF_r(h)]. */
typedef struct {
  int hidden, ffn, experts, top_k;
  double ln_eps;
  int gelu_tanh;
  int residual;  /* 1: PR-MoE, a dense MLP added to the experts' output */
  int combine;   /* 0: chosen probabilities renormalized; 1: the softmax probabilities */
} ora_moe_desc;

typedef struct {
  const double *ln_g, *ln_b;                /* [H]                                   */
  const double *w_gate;                     /* [E][H]                                */
  const double *w1, *b1;                    /* [E][F][H], [E][F]                     */
  const double *w2, *b2;                    /* [E][H][F], [E][H]                     */
  const double *r_w1, *r_b1, *r_w2, *r_b2;  /* the residual MLP, or NULL (standard) */
} ora_moe_weights;

/* x2, y: [T][H]. sel, wgt: [T][top_k] outputs (may be NULL). force_sel: [T][top_k] experts to use
 * in place of the top-k (their weights still come from p), or NULL. Returns 0, or -1 on a bad
 * shape or a forced expert out of range. */
int ora_moe_forward(const ora_moe_desc* d, const ora_moe_weights* w, const double* x2, int tokens,
                    const int* force_sel, double* y, int* sel, double* wgt);

/* The int8 KV cache reading (the pages do not quantize the cache; this follows their group-wise
 * weight quantizer with one group per cached row of one head): scale = fp16_RNE(amax/127),
 * code = clamp(round_half_even(x/scale), -127, 127); amax = 0 -> scale 0, codes 0. x: n doubles. */
void ora_quantize_row_i8(const double* x, int n, int8_t* q, uint16_t* s);

/* ---- IEEE binary16 ---- */
uint16_t ora_fp16_from_double(double v); /* round to nearest, ties to even; overflow -> inf */
double   ora_fp16_to_double(uint16_t h);

/* ---- group-wise symmetric int8 ([KP] section 五 5.2) ----
 * w: float32 [n][k]; q: int8 [n][k]; s: fp16 bits [n][k/group]. Returns 0, or -1 if k % group. */
int  ora_quantize_i8(const float* w, int n, int k, int group, int8_t* q, uint16_t* s);
/* w = q * s in double (exact). */
int  ora_dequantize_i8(const int8_t* q, const uint16_t* s, int n, int k, int group, double* w);

#ifdef __cplusplus
}
#endif
#endif
