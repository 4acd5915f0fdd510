/*
 * oracle.c -- TEST INFRASTRUCTURE ONLY: the double-precision CPU definition of the layer.
 * See oracle.h for the sources cited and the readings taken where the pages are silent.
 * Every loop is the textbook definition; nothing is blocked, fused or reordered.
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* [KP] section 三 3.2, region 1 and region 3: LayerNorm over one row of n values.
 * mean = sum(x)/n, var = sum((x-mean)^2)/n, out = (x-mean)/sqrt(var+eps)*g + b. */
void ora_layernorm(const double* x, int n, const double* g, const double* b, double eps, double* out) {
  double mean = 0.0;
  for (int i = 0; i < n; ++i) mean += x[i];
  mean /= n;
  double var = 0.0;
  for (int i = 0; i < n; ++i) var += (x[i] - mean) * (x[i] - mean);
  var /= n;
  double inv = 1.0 / sqrt(var + eps);
  for (int i = 0; i < n; ++i) out[i] = (x[i] - mean) * inv * g[i] + b[i];
}

/* [KP] section 三 3.2: every GeMM of the layer followed by its bias-add.
 * out[o] = bias[o] + sum_k w[o][k] * x[k]  (w is [n_out][k] row-major). bias may be NULL. */
void ora_linear(const double* w, const double* bias, const double* x, int n_out, int k, double* out) {
  for (int o = 0; o < n_out; ++o) {
    double acc = 0.0;
    for (int i = 0; i < k; ++i) acc += w[(size_t)o * k + i] * x[i];
    out[o] = (bias ? bias[o] : 0.0) + acc;
  }
}

/* [KP] section 三 3.2, region 3: GELU. Exact form u*Phi(u) = u/2 * (1 + erf(u/sqrt 2));
 * the tanh form is u/2 * (1 + tanh(sqrt(2/pi) * (u + 0.044715 u^3))). */
double ora_gelu(double u, int tanh_form) {
  if (tanh_form) {
    const double c = sqrt(2.0 / M_PI);
    return 0.5 * u * (1.0 + tanh(c * (u + 0.044715 * u * u * u)));
  }
  return 0.5 * u * (1.0 + erf(u / sqrt(2.0)));
}

/* Softmax over n scores: p_i = exp(s_i - max) / sum_j exp(s_j - max). */
void ora_softmax(const double* s, int n, double* p) {
  double m = s[0];
  for (int i = 1; i < n; ++i)
    if (s[i] > m) m = s[i];
  double z = 0.0;
  for (int i = 0; i < n; ++i) {
    p[i] = exp(s[i] - m);
    z += p[i];
  }
  for (int i = 0; i < n; ++i) p[i] /= z;
}

/* [KP] section 三 3.2, region 2: the attention of one query of one head.
 * s_i = q . k_i / sqrt(d) over the given keys, p = softmax(s), out = sum_i p_i v_i. */
void ora_attend(const double* q, const double* keys, const double* vals, int nkeys, int d, double* out) {
  double* s = (double*)malloc(sizeof(double) * (size_t)nkeys);
  double* p = (double*)malloc(sizeof(double) * (size_t)nkeys);
  const double scale = 1.0 / sqrt((double)d);
  for (int i = 0; i < nkeys; ++i) {
    double dot = 0.0;
    for (int e = 0; e < d; ++e) dot += q[e] * keys[(size_t)i * d + e];
    s[i] = dot * scale;
  }
  ora_softmax(s, nkeys, p);
  for (int e = 0; e < d; ++e) {
    double acc = 0.0;
    for (int i = 0; i < nkeys; ++i) acc += p[i] * vals[(size_t)i * d + e];
    out[e] = acc;
  }
  free(s);
  free(p);
}

static double* stage_row(double* base, int b, int t, int ntok, int width) {
  return base ? base + ((size_t)b * ntok + t) * width : NULL;
}

static void put(double* dst, const double* src, int n) {
  if (dst) memcpy(dst, src, sizeof(double) * (size_t)n);
}

/* The pre-LN GPT layer of [KP] section 三 3.2 (regions 1-4) with a KV cache, for T new rows of
 * each of B sequences. All rows' keys and values are appended before any row attends. */
int ora_layer_forward(const ora_desc* dsc, const ora_weights* w, double* k_cache, double* v_cache,
                      int cap, int* lens, const double* x, double* y, int batch, int ntok,
                      ora_stages* st) {
  const int H = dsc->hidden, nh = dsc->heads, d = dsc->head_dim, F = dsc->ffn;
  if (H != nh * d || H <= 0 || F <= 0 || batch < 0 || ntok < 0) return -1;
  for (int b = 0; b < batch; ++b)
    if (lens[b] < 0 || lens[b] + ntok > cap) return -1;

  double* h = (double*)malloc(sizeof(double) * (size_t)H);
  double* qkv = (double*)malloc(sizeof(double) * (size_t)batch * ntok * 3 * H);
  double* ctx = (double*)malloc(sizeof(double) * (size_t)H);
  double* x2 = (double*)malloc(sizeof(double) * (size_t)H);
  double* tmp = (double*)malloc(sizeof(double) * (size_t)H);
  double* u = (double*)malloc(sizeof(double) * (size_t)F);
  double* g = (double*)malloc(sizeof(double) * (size_t)F);

  /* Region 1: LN1, then the fused Q/K/V projection with bias, for every new row. */
  for (int b = 0; b < batch; ++b)
    for (int t = 0; t < ntok; ++t) {
      const double* xr = x + ((size_t)b * ntok + t) * H;
      ora_layernorm(xr, H, w->ln1_g, w->ln1_b, dsc->ln_eps, h);
      double* z = qkv + ((size_t)b * ntok + t) * 3 * H;
      ora_linear(w->w_qkv, w->b_qkv, h, 3 * H, H, z);
      put(stage_row(st ? st->ln1 : NULL, b, t, ntok, H), h, H);
      put(stage_row(st ? st->qkv : NULL, b, t, ntok, 3 * H), z, 3 * H);
    }

  /* Append: K[b][j][p] = k_j and V[b][j][p] = v_j at p = lens[b] + t; with an int8 cache each
   * head row is stored quantized, and attention below reads the dequantized row. */
  int8_t* codes = (int8_t*)malloc((size_t)d);
  for (int b = 0; b < batch; ++b)
    for (int t = 0; t < ntok; ++t) {
      const double* z = qkv + ((size_t)b * ntok + t) * 3 * H;
      const int p = lens[b] + t;
      for (int j = 0; j < nh; ++j) {
        double* kr = k_cache + (((size_t)b * nh + j) * cap + p) * d;
        double* vr = v_cache + (((size_t)b * nh + j) * cap + p) * d;
        for (int e = 0; e < d; ++e) {
          kr[e] = z[H + j * d + e];
          vr[e] = z[2 * H + j * d + e];
        }
        if (dsc->kv_int8) {
          double* rows[2] = {kr, vr};
          for (int m = 0; m < 2; ++m) {
            uint16_t sb;
            ora_quantize_row_i8(rows[m], d, codes, &sb);
            const double sv = ora_fp16_to_double(sb);
            for (int e = 0; e < d; ++e) rows[m][e] = (double)codes[e] * sv;
          }
        }
      }
    }
  free(codes);

  for (int b = 0; b < batch; ++b)
    for (int t = 0; t < ntok; ++t) {
      const double* xr = x + ((size_t)b * ntok + t) * H;
      const double* z = qkv + ((size_t)b * ntok + t) * 3 * H;
      const int p = lens[b] + t;
      /* triangular_masking ([MP] config table): row at position p sees keys 0..p. */
      const int nkeys = dsc->triangular_masking ? p + 1 : lens[b] + ntok;

      /* Region 2: per-head attention over the cache. */
      for (int j = 0; j < nh; ++j) {
        const size_t head = ((size_t)b * nh + j) * cap * d;
        ora_attend(z + j * d, k_cache + head, v_cache + head, nkeys, d, ctx + j * d);
      }
      /* Attention-output GeMM, bias and residual: x2 = x + Wo ctx + bo. */
      ora_linear(w->w_o, w->b_o, ctx, H, H, tmp);
      for (int i = 0; i < H; ++i) x2[i] = xr[i] + tmp[i];

      /* Region 3: LN2, intermediate FF with bias, GeLU. */
      ora_layernorm(x2, H, w->ln2_g, w->ln2_b, dsc->ln_eps, h);
      ora_linear(w->w_ff1, w->b_ff1, h, F, H, u);
      for (int i = 0; i < F; ++i) g[i] = ora_gelu(u[i], dsc->gelu_tanh);

      /* Region 4: output GeMM, bias and residual: y = x2 + W2 g + b2. */
      double* yr = y + ((size_t)b * ntok + t) * H;
      ora_linear(w->w_ff2, w->b_ff2, g, H, F, tmp);
      for (int i = 0; i < H; ++i) yr[i] = x2[i] + tmp[i];

      put(stage_row(st ? st->ctx : NULL, b, t, ntok, H), ctx, H);
      put(stage_row(st ? st->x2 : NULL, b, t, ntok, H), x2, H);
      put(stage_row(st ? st->ln2 : NULL, b, t, ntok, H), h, H);
      put(stage_row(st ? st->ff1 : NULL, b, t, ntok, F), u, F);
      put(stage_row(st ? st->act : NULL, b, t, ntok, F), g, F);
    }

  for (int b = 0; b < batch; ++b) lens[b] += ntok;
  free(h); free(qkv); free(ctx); free(x2); free(tmp); free(u); free(g);
  return 0;
}

/* The end of a generation step ([KP] section 二, the GPT-Neo-2.7B text-generation example): the
 * final LayerNorm of the last layer's output, then the LM head, logits[v] = sum_k w[v][k] h[k]. */
void ora_lm_head(const double* y, int H, const double* g, const double* b, double eps,
                 const double* w_vocab, int V, double* logits) {
  double* h = (double*)malloc(sizeof(double) * (size_t)H);
  ora_layernorm(y, H, g, b, eps, h);
  ora_linear(w_vocab, NULL, h, V, H, logits);
  free(h);
}

/* Greedy decoding: scan left to right and keep the first position holding the largest value. */
int ora_argmax(const double* v, int n) {
  int best = 0;
  for (int i = 1; i < n; ++i)
    if (v[i] > v[best]) best = i;
  return best;
}

/* One expert (or the residual MLP): out = W2 GeLU(W1 h + b1) + b2. */
static void moe_expert(const double* w1, const double* b1, const double* w2, const double* b2, const double* h,
                       int H, int F, int tanh_form, double* u, double* out) {
  ora_linear(w1, b1, h, F, H, u);
  for (int i = 0; i < F; ++i) u[i] = ora_gelu(u[i], tanh_form);
  ora_linear(w2, b2, u, H, F, out);
}

/* The MoE expert FF ([MP], MoE sections; readings in oracle.h). */
int ora_moe_forward(const ora_moe_desc* d, const ora_moe_weights* w, const double* x2, int tokens,
                    const int* force_sel, double* y, int* sel, double* wgt) {
  const int H = d->hidden, F = d->ffn, E = d->experts, K = d->top_k;
  if (H < 1 || F < 1 || E < 1 || K < 1 || K > E || tokens < 0) return -1;
  if (d->residual && !(w->r_w1 && w->r_b1 && w->r_w2 && w->r_b2)) return -1;
  double* h = (double*)malloc(sizeof(double) * (size_t)H);
  double* logit = (double*)malloc(sizeof(double) * (size_t)E);
  double* p = (double*)malloc(sizeof(double) * (size_t)E);
  double* q = (double*)malloc(sizeof(double) * (size_t)E);
  double* u = (double*)malloc(sizeof(double) * (size_t)F);
  double* o = (double*)malloc(sizeof(double) * (size_t)H);
  int* chosen = (int*)malloc(sizeof(int) * (size_t)K);
  int rc = 0;
  for (int t = 0; t < tokens && rc == 0; ++t) {
    const double* xt = x2 + (size_t)t * H;
    double* yt = y + (size_t)t * H;
    ora_layernorm(xt, H, w->ln_g, w->ln_b, d->ln_eps, h);
    ora_linear(w->w_gate, NULL, h, E, H, logit);
    ora_softmax(logit, E, p);
    /* the k largest probabilities, one at a time: argmax over the experts not yet taken */
    for (int e = 0; e < E; ++e) q[e] = p[e];
    for (int i = 0; i < K; ++i) {
      if (force_sel) {
        chosen[i] = force_sel[(size_t)t * K + i];
        if (chosen[i] < 0 || chosen[i] >= E) rc = -1;
      } else {
        chosen[i] = ora_argmax(q, E);
        q[chosen[i]] = -1.0; /* below every probability */
      }
    }
    if (rc) break;
    double psum = 0.0;
    for (int i = 0; i < K; ++i) psum += p[chosen[i]];
    for (int c = 0; c < H; ++c) yt[c] = xt[c];
    for (int i = 0; i < K; ++i) {
      const int e = chosen[i];
      const double wi = d->combine ? p[e] : p[e] / psum;
      moe_expert(w->w1 + (size_t)e * F * H, w->b1 + (size_t)e * F, w->w2 + (size_t)e * H * F, w->b2 + (size_t)e * H, h,
                 H, F, d->gelu_tanh, u, o);
      for (int c = 0; c < H; ++c) yt[c] += wi * o[c];
      if (sel) sel[(size_t)t * K + i] = e;
      if (wgt) wgt[(size_t)t * K + i] = wi;
    }
    if (d->residual) {
      moe_expert(w->r_w1, w->r_b1, w->r_w2, w->r_b2, h, H, F, d->gelu_tanh, u, o);
      for (int c = 0; c < H; ++c) yt[c] += o[c];
    }
  }
  free(h); free(logit); free(p); free(q); free(u); free(o); free(chosen);
  return rc;
}

/* IEEE 754 binary16 from a double, rounding to nearest with ties to even.
 * Normal numbers have an 11-bit significand and exponents -14..15; below 2^-14 the spacing is
 * the fixed 2^-24 (subnormals); a rounded magnitude of 2^16 or more becomes infinity. */
uint16_t ora_fp16_from_double(double v) {
  uint16_t sign = signbit(v) ? 0x8000u : 0u;
  double a = fabs(v);
  if (isnan(v)) return (uint16_t)(sign | 0x7e00u);
  if (isinf(a)) return (uint16_t)(sign | 0x7c00u);
  if (a == 0.0) return sign;
  int e2;
  frexp(a, &e2);            /* a = f * 2^e2, f in [0.5, 1): the leading bit has weight 2^(e2-1) */
  int ex = e2 - 1;          /* unbiased exponent of the leading bit                             */
  if (ex < -14) ex = -14;   /* subnormal range: quantum fixed at 2^-24                          */
  double quantum = ldexp(1.0, ex - 10);
  double m = nearbyint(a / quantum); /* exact scaling by a power of two, then ties-to-even    */
  if (m >= 2048.0) {        /* rounding carried into the next binade                            */
    m /= 2.0;
    ex += 1;
  }
  if (m < 1024.0) return (uint16_t)(sign | (uint16_t)m); /* subnormal (or rounded to zero) */
  if (ex > 15) return (uint16_t)(sign | 0x7c00u);
  return (uint16_t)(sign | (uint16_t)((ex + 15) << 10) | (uint16_t)((int)m - 1024));
}

double ora_fp16_to_double(uint16_t h) {
  int sign = (h >> 15) & 1, ex = (h >> 10) & 0x1f, man = h & 0x3ff;
  double v;
  if (ex == 0x1f) v = man ? NAN : INFINITY;
  else if (ex == 0) v = ldexp((double)man, -24);
  else v = ldexp((double)(man + 1024), ex - 25);
  return sign ? -v : v;
}

/* [KP] section 五 5.2: int8 weights with one scale per group of quantize_groups elements.
 * For every row and every group of `group` consecutive elements along k:
 *   amax = max |w|; s = fp16_RNE(amax / 127); q = clamp(round_half_even(w / s), -127, 127);
 *   a group whose scale is zero gets codes of zero. */
int ora_quantize_i8(const float* w, int n, int k, int group, int8_t* q, uint16_t* s) {
  if (group <= 0 || k % group) return -1;
  const int ng = k / group;
  for (int r = 0; r < n; ++r)
    for (int gi = 0; gi < ng; ++gi) {
      const float* src = w + (size_t)r * k + (size_t)gi * group;
      int8_t* dst = q + (size_t)r * k + (size_t)gi * group;
      double amax = 0.0;
      for (int i = 0; i < group; ++i)
        if (fabs((double)src[i]) > amax) amax = fabs((double)src[i]);
      uint16_t sb = ora_fp16_from_double(amax / 127.0);
      s[(size_t)r * ng + gi] = sb;
      double sv = ora_fp16_to_double(sb);
      for (int i = 0; i < group; ++i) {
        double c = (sv == 0.0) ? 0.0 : nearbyint((double)src[i] / sv);
        if (c > 127.0) c = 127.0;
        if (c < -127.0) c = -127.0;
        dst[i] = (int8_t)c;
      }
    }
  return 0;
}

void ora_quantize_row_i8(const double* x, int n, int8_t* q, uint16_t* s) {
  double amax = 0.0;
  for (int i = 0; i < n; ++i)
    if (fabs(x[i]) > amax) amax = fabs(x[i]);
  const uint16_t sb = ora_fp16_from_double(amax / 127.0);
  *s = sb;
  const double sv = ora_fp16_to_double(sb);
  for (int i = 0; i < n; ++i) {
    double c = (sv == 0.0) ? 0.0 : nearbyint(x[i] / sv);
    if (c > 127.0) c = 127.0;
    if (c < -127.0) c = -127.0;
    q[i] = (int8_t)c;
  }
}

int ora_dequantize_i8(const int8_t* q, const uint16_t* s, int n, int k, int group, double* w) {
  if (group <= 0 || k % group) return -1;
  const int ng = k / group;
  for (int r = 0; r < n; ++r)
    for (int i = 0; i < k; ++i)
      w[(size_t)r * k + i] = (double)q[(size_t)r * k + i] * ora_fp16_to_double(s[(size_t)r * ng + i / group]);
  return 0;
}
