// layer.cpp -- the C ABI of libdslayer.so (include/ds_layer.h): host-side validation, workspace
// layout and the launch sequence of one layer step. No device memory is allocated here.
//
// The step follows the four fusion regions of one transformer layer on the page "DeepSpeed
// Inference 内核优化深度解析" (blog.gitcode.com), section 三 3.2, with the kernel boundaries at the
// two all-reduce points of section 三 3.1 (after the attention-output GeMM, after the FF2 GeMM):
//   1 LN1 + QKV GEMV + bias, q to the workspace, k/v into the cache rows  (region 1 + transform)
//   2 attention over the cache, chunked over positions, merged in-kernel  (region 2)
//   3 output projection + bias + residual                                 (all-reduce point 1)
//   4 LN2 + FF1 + bias + GeLU                                             (region 3)
//   5 FF2 + bias + residual, then the cache length advances               (region 4, point 2)
// With fp16 (or bf16) weights and activations and at least kMfmaMinRows rows per step (prefill, or a
// large decode batch) the projections are dense GEMMs and run on the MFMA path instead
// (kernels_prefill.hip): LayerNorm
// rows, the QKV GEMM scattering k/v into the cache, flash attention, and the O, FF1, FF2 GEMMs with
// their bias, residual and GeLU epilogues.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>

#include "ds_internal.hpp"
#include "ds_launch.hpp"
#include "ds_prefill.hpp"

namespace {
thread_local std::string g_err;
}  // namespace

int ds::set_error(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

namespace {

template <typename... Args>
int fail(int code, const char* fmt, Args... args) {
  return ds::set_error(code, fmt, args...);
}

int hip_fail(hipError_t e, const char* where) {
  return fail(DS_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }


size_t up256(size_t v) { return (v + 255) / 256 * 256; }

// the layer's cache holds int8 rows with fp16 scales
bool kv_int8(const ds_layer_desc& d) { return d.kv_dtype == DS_I8; }

// ds_layer_time_kernels: events recorded after each kernel launch of one step (the calling thread's
// timer; null outside that call).
constexpr int kMaxMarks = 16;
struct KernelTimer {
  hipEvent_t ev[kMaxMarks + 1] = {};
  int kinds[kMaxMarks] = {};
  int n = 0;
  bool failed = false;
};
thread_local KernelTimer* g_timer = nullptr;

void mark(hipStream_t st, int kind) {
  KernelTimer* t = g_timer;
  if (!t || t->failed) return;
  if (t->n >= kMaxMarks || hipEventRecord(t->ev[t->n + 1], st) != hipSuccess) {
    t->failed = true;
    return;
  }
  t->kinds[t->n++] = kind;
}

struct WsLayout {
  size_t q, part, cnt, ctx, x2, f, h, sk_part, sk_cnt, kvn, wdq, total;
  int chunk, nchunk, n_sk_cnt;
};

WsLayout ws_layout(const ds_layer_desc& d, int rows, int cap) {
  WsLayout L{};
  L.chunk = ds::attn_chunk_for(rows, d.heads, cap);
  L.nchunk = (cap + L.chunk - 1) / L.chunk;
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t at = off; off += up256(bytes); return at; };
  L.q = take((size_t)rows * d.hidden * 4);
  L.part = take((size_t)rows * d.heads * L.nchunk * (d.head_dim + 2) * 4);
  L.cnt = take((size_t)rows * d.heads * 4);
  L.ctx = take((size_t)rows * d.hidden * 4);
  L.x2 = take((size_t)rows * d.hidden * 4);
  L.f = take((size_t)rows * d.ffn * 4);
  L.h = take((size_t)rows * d.hidden * 2);  // fp16 LayerNorm rows of the MFMA path
  // partial tiles and counters of the skinny products that split K over workgroups
  const int n_max = d.hidden > d.ffn ? d.hidden : d.ffn;
  L.sk_part = take(ds::skinny_part_bytes(n_max));
  L.sk_cnt = take(ds::skinny_cnt_bytes(n_max));
  L.n_sk_cnt = (n_max + 15) / 16;
  // an int8 cache: the new k and v rows (fp32) between the QKV product and their quantization
  L.kvn = kv_int8(d) ? take((size_t)rows * 2 * d.hidden * 4) : 0;
  // int8 weights at more rows than the skinny kernel takes: one matrix at a time dequantized into
  // fp16 for the many-row GEMM (the largest of Wqkv [3H][H], W1 [F][H], W2 [H][F])
  const size_t wmax = (size_t)d.hidden * (size_t)(3 * d.hidden > d.ffn ? 3 * d.hidden : d.ffn);
  L.wdq = d.weight_dtype == DS_I8 && rows > ds::kSkinnyMaxRows ? take(wmax * 2) : 0;
  L.total = off;
  return L;
}

int check_kv(const ds_layer* L, const ds_kv_cache* kv, int batch, int ntok) {
  if (!kv) return fail(DS_ERR_NULL, "kv cache is NULL");
  if (!kv->k || !kv->v || !kv->d_len) return fail(DS_ERR_NULL, "kv cache k, v or d_len is NULL");
  if (!aligned16(kv->k) || !aligned16(kv->v)) return fail(DS_ERR_ALIGN, "kv cache k or v is not 16-byte aligned");
  if (kv->batch < 1 || kv->capacity < 1) return fail(DS_ERR_SHAPE, "kv cache batch %d / capacity %d must be >= 1", kv->batch, kv->capacity);
  if (batch < 0 || batch > kv->batch) return fail(DS_ERR_SHAPE, "batch %d outside [0, %d]", batch, kv->batch);
  if (ntok < 0) return fail(DS_ERR_SHAPE, "token count %d < 0", ntok);
  if (L->desc.kv_dtype == DS_I8) {
    if (!kv->k_scale || !kv->v_scale) return fail(DS_ERR_NULL, "an int8 kv cache needs k_scale and v_scale");
    if (!aligned16(kv->k_scale) || !aligned16(kv->v_scale)) return fail(DS_ERR_ALIGN, "kv scales are not 16-byte aligned");
  } else if (kv->k_scale || kv->v_scale) {
    return fail(DS_ERR_DTYPE, "kv scales are set but the layer's cache is not int8");
  }
  if (kv->h_len)
    for (int b = 0; b < batch; ++b)
      if (kv->h_len[b] < 0 || (int64_t)kv->h_len[b] + ntok > kv->capacity)
        return fail(DS_ERR_KV_FULL, "sequence %d: %d rows + %d new > capacity %d", b, kv->h_len[b], ntok, kv->capacity);
  return DS_OK;
}

constexpr int kMfmaMinRows = 16;

// The MFMA path takes fp16 or bf16 weights with activations of the same type (and a cache of that
// type or int8), at least kMfmaMinRows rows, and operands whose byte sizes stay inside one buffer
// descriptor's 31-bit range. int8 weights with fp16 activations take it above the skinny kernel's
// row limit, each matrix dequantized into fp16 in the workspace just before its product.
bool use_mfma(const ds_layer_desc& d, int rows) {
  const bool f16 = d.weight_dtype == DS_F16 && d.act_dtype == DS_F16;
  const bool bf16 = d.weight_dtype == DS_BF16 && d.act_dtype == DS_BF16;
  const bool i8 = d.weight_dtype == DS_I8 && d.act_dtype == DS_F16 && rows > ds::kSkinnyMaxRows;
  if (!(f16 || bf16 || i8) || rows < kMfmaMinRows) return false;
  const int64_t kmax = d.hidden > d.ffn ? d.hidden : d.ffn;
  const int64_t lim = int64_t(1) << 31;
  return (int64_t)rows * kmax * 2 < lim && (int64_t)d.ffn * d.hidden * 2 < lim && 3 * (int64_t)d.hidden * d.hidden * 2 < lim;
}

// Steps of a few rows (fewer than the MFMA tile path takes) with fp16 activations and fp16 or int8
// weights, or bf16 weights and activations, run the same LayerNorm / attention kernels with the
// skinny GEMM, which streams every weight row once whatever the row count. With an int8 cache the
// new k and v rows leave the QKV product in fp32 and are quantized by the store kernel before the
// attention reads the cache.
bool use_skinny(const ds_layer_desc& d, int rows) {
  if (rows < 1 || rows > ds::kSkinnyMaxRows) return false;
  if (d.act_dtype == DS_BF16) return d.weight_dtype == DS_BF16 && rows < kMfmaMinRows;
  if (d.act_dtype != DS_F16) return false;
  if (d.weight_dtype == DS_F16) return rows < kMfmaMinRows;
  // the int8 skinny kernel applies one scale per 64-element block of K
  return d.weight_dtype == DS_I8 && d.quant_group == 64 && (d.quant_group_mlp == 0 || d.quant_group_mlp == 64);
}

int forward_mfma(const ds_layer* L, ds_kv_cache* kv, const void* x, void* y, int batch, int ntok, char* base,
                 const WsLayout& W, bool skinny, hipStream_t st) {
  const ds_layer_desc& d = L->desc;
  const int rows = batch * ntok, H = d.hidden, F = d.ffn;
  int dev = 0, cus = 0;
  if (hipError_t e = hipGetDevice(&dev)) return hip_fail(e, "hipGetDevice");
  if (hipError_t e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev)) return hip_fail(e, "CU count");
  auto* h = reinterpret_cast<ds::half_t*>(base + W.h);
  auto* q = reinterpret_cast<ds::half_t*>(base + W.q);
  auto* ctx = reinterpret_cast<ds::half_t*>(base + W.ctx);
  auto* x2 = reinterpret_cast<float*>(base + W.x2);
  auto* f = reinterpret_cast<ds::half_t*>(base + W.f);
  auto hp = [](const void* p) { return static_cast<const ds::half_t*>(p); };

  ds::GemmArgs g{};
  g.d_len = kv->d_len;
  g.tokens = ntok;
  g.heads = d.heads;
  g.head_dim = d.head_dim;
  g.cap = kv->capacity;
  g.hidden = H;
  g.gelu_tanh = d.gelu_tanh;
  g.k_cache = static_cast<ds::half_t*>(kv->k);
  g.v_cache = static_cast<ds::half_t*>(kv->v);
  g.M = rows;
  if (skinny) {
    g.sk_part = reinterpret_cast<float*>(base + W.sk_part);
    g.sk_cnt = reinterpret_cast<uint32_t*>(base + W.sk_cnt);
    g.n_sk_cnt = W.n_sk_cnt;
  }
  const bool i8 = d.weight_dtype == DS_I8;
  const bool bf16 = d.act_dtype == DS_BF16;  // the 16-bit type of this path's rows (bf16 or fp16)
  g.group = d.quant_group;
  // one weight matrix (fp16, or int8 codes with their scales) and its product
  auto gemm = [&](ds::GemmEpi epi, ds::GemmArgs& a, const void* w, const void* s) -> hipError_t {
    if (i8 && skinny) {
      a.wq = static_cast<const int8_t*>(w);
      a.wscale = static_cast<const ds::half_t*>(s);
    } else if (i8) {
      // the many-row GEMM takes fp16 operands: the codes times their group scales, rounded once
      const int grp = epi == ds::EPI_FF1 || epi == ds::EPI_FF2 ? (d.quant_group_mlp ? d.quant_group_mlp : d.quant_group)
                                                               : d.quant_group;
      auto* wdq = reinterpret_cast<ds::half_t*>(base + W.wdq);
      if (hipError_t e = ds::launch_dequantize_i8_f16(static_cast<const int8_t*>(w), static_cast<const uint16_t*>(s),
                                                      wdq, a.N, a.K, grp, st))
        return e;
      a.w = wdq;
    } else {
      a.w = static_cast<const ds::half_t*>(w);
    }
    if (skinny) return ds::launch_skinny(epi, i8, bf16, a, cus, st);
    return ds::launch_gemm(epi, bf16, a, L->gemm_cfg >= 0 ? L->gemm_cfg : ds::gemm_pick(a.M, a.N, a.K, cus), st);
  };

  // 1: h = LN1(x); [q | k | v] = h Wqkv^T + bqkv, k and v into the cache rows d_len[b] + t
  if (hipError_t e = ds::launch_ln_rows(bf16, false, x, L->w.ln1_g, L->w.ln1_b, h, rows, H, d.ln_eps, st))
    return hip_fail(e, "ln1 launch");
  mark(st, DS_PART_LN1);
  ds::GemmArgs a = g;
  a.a = h; a.bias = hp(L->w.b_qkv); a.out = q; a.N = 3 * H; a.K = H;
  const bool chunked_attn = skinny && ntok == 1;  // decode: chunked attention with an in-kernel merge
  if (chunked_attn) {
    a.attn_counters = reinterpret_cast<uint32_t*>(base + W.cnt);
    a.n_counters = rows * d.heads;
  }
  float* kvn = kv_int8(d) ? reinterpret_cast<float*>(base + W.kvn) : nullptr;
  a.kv_new = kvn;  // an int8 cache: k and v leave the product in fp32 and are quantized next
  if (hipError_t e = gemm(ds::EPI_QKV, a, L->w.w_qkv, L->w.s_qkv)) return hip_fail(e, "qkv gemm launch");
  if (kvn) {
    if (hipError_t e = ds::launch_kv_store_i8(ds::F32, kvn, kvn + H, 2 * H, kv->k, kv->v, kv->k_scale, kv->v_scale,
                                              kv->d_len, batch, ntok, d.heads, d.head_dim, kv->capacity, st))
      return hip_fail(e, "int8 kv store launch");
  }
  mark(st, DS_PART_QKV);

  // 2: attention of the new rows over the cache
  ds::AttnPrefillArgs at{};
  at.q = q; at.k_cache = g.k_cache; at.v_cache = g.v_cache; at.d_len = kv->d_len; at.ctx = ctx;
  at.batch = batch; at.tokens = ntok; at.heads = d.heads; at.head_dim = d.head_dim; at.cap = kv->capacity;
  at.causal = d.triangular_masking; at.scale = 1.f / std::sqrt((float)d.head_dim);
  at.k_scale = kvn ? kv->k_scale : nullptr;
  at.v_scale = kvn ? kv->v_scale : nullptr;
  if (chunked_attn) {
    ds::AttnArgs ad{};
    ad.q16 = q; ad.ctx16 = ctx;
    ad.k_cache = kv->k; ad.v_cache = kv->v; ad.d_len = kv->d_len;
    ad.part = reinterpret_cast<float*>(base + W.part);
    ad.counters = reinterpret_cast<uint32_t*>(base + W.cnt);
    ad.rows = rows; ad.tokens = ntok; ad.heads = d.heads; ad.head_dim = d.head_dim;
    ad.cap = kv->capacity; ad.chunk = W.chunk; ad.causal = d.triangular_masking;
    ad.nchunk = ds::attn_chunks_for(rows, d.heads, kv->capacity, W.chunk, W.nchunk, cus);
    ad.k_scale = kvn ? kv->k_scale : nullptr;
    ad.v_scale = kvn ? kv->v_scale : nullptr;
    if (hipError_t e = ds::launch_attn_decode_16(bf16, ad, st)) return hip_fail(e, "attention launch");
  } else if (hipError_t e = ds::launch_attn_prefill(bf16, at, st)) {
    return hip_fail(e, "attention launch");
  }
  mark(st, DS_PART_ATTN);

  // 3: x2 = x + ctx Wo^T + bo
  a = g;
  a.a = ctx; a.bias = hp(L->w.b_o); a.out = x2; a.resid = x; a.N = H; a.K = H;
  if (hipError_t e = gemm(ds::EPI_OPROJ, a, L->w.w_o, L->w.s_o)) return hip_fail(e, "o gemm launch");
  mark(st, DS_PART_O);

  // 4: f = GeLU(LN2(x2) W1^T + b1); the LN2 launch also advances d_len by ntok (the QKV epilogue
  // and attention, its only readers in this step, have run)
  if (hipError_t e = ds::launch_ln_rows(bf16, true, x2, L->w.ln2_g, L->w.ln2_b, h, rows, H, d.ln_eps, st, kv->d_len,
                                        batch, ntok, kv->capacity))
    return hip_fail(e, "ln2 launch");
  mark(st, DS_PART_LN2);
  a = g;
  a.a = h; a.bias = hp(L->w.b_ff1); a.out = f; a.N = F; a.K = H;
  if (hipError_t e = gemm(ds::EPI_FF1, a, L->w.w_ff1, L->w.s_ff1)) return hip_fail(e, "ff1 gemm launch");
  mark(st, DS_PART_FF1);

  // 5: y = x2 + f W2^T + b2
  a = g;
  a.a = f; a.bias = hp(L->w.b_ff2); a.out = y; a.resid = x2; a.N = H; a.K = F;
  if (hipError_t e = gemm(ds::EPI_FF2, a, L->w.w_ff2, L->w.s_ff2)) return hip_fail(e, "ff2 gemm launch");
  mark(st, DS_PART_FF2);
  if (kv->h_len)
    for (int b = 0; b < batch; ++b) kv->h_len[b] += ntok;
  return DS_OK;
}

int forward_rows(const ds_layer* L, ds_kv_cache* kv, const void* x, void* y, int batch, int ntok,
                 void* ws, size_t ws_bytes, void* stream) {
  if (!L) return fail(DS_ERR_NULL, "layer is NULL");
  if (int rc = check_kv(L, kv, batch, ntok)) return rc;
  if (batch == 0 || ntok == 0) return DS_OK;
  if (!x || !y || !ws) return fail(DS_ERR_NULL, "x, y or workspace is NULL");
  if (!aligned16(x) || !aligned16(y) || !aligned16(ws)) return fail(DS_ERR_ALIGN, "x, y or workspace is not 16-byte aligned");
  const ds_layer_desc& d = L->desc;
  const int rows = batch * ntok;
  const WsLayout W = ws_layout(d, rows, kv->capacity);
  if (ws_bytes < W.total) return fail(DS_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, W.total);

  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  char* base = static_cast<char*>(ws);
  if (use_mfma(L->desc, rows)) return forward_mfma(L, kv, x, y, batch, ntok, base, W, false, st);
  if (use_skinny(L->desc, rows)) return forward_mfma(L, kv, x, y, batch, ntok, base, W, true, st);
  const ds::Dt wdt = static_cast<ds::Dt>(d.weight_dtype), adt = static_cast<ds::Dt>(d.act_dtype);
  const int H = d.hidden, F = d.ffn;

  ds::GemvArgs g{};
  const int group_mlp = d.quant_group_mlp ? d.quant_group_mlp : d.quant_group;
  g.group = d.quant_group;
  g.rows = rows;
  g.tokens = ntok;
  g.cap = kv->capacity;
  g.heads = d.heads;
  g.head_dim = d.head_dim;
  g.hidden = H;
  g.eps = d.ln_eps;
  g.gelu_tanh = d.gelu_tanh;
  g.d_len = kv->d_len;

  // 1: LN1 + QKV + bias; q -> workspace, k/v -> cache rows d_len[b] + t
  ds::GemvArgs a = g;
  a.w = L->w.w_qkv; a.s = L->w.s_qkv; a.bias = L->w.b_qkv; a.in = x;
  a.ln_g = L->w.ln1_g; a.ln_b = L->w.ln1_b;
  a.n = 3 * H; a.k = H;
  a.q_out = reinterpret_cast<float*>(base + W.q);
  a.k_cache = kv->k; a.v_cache = kv->v;
  a.attn_counters = reinterpret_cast<uint32_t*>(base + W.cnt);
  if (kv_int8(d)) a.kv_new = reinterpret_cast<float*>(base + W.kvn);
  if (hipError_t e = ds::launch_gemv(wdt, adt, ds::KIND_QKV, a, st)) return hip_fail(e, "ln_qkv launch");
  if (kv_int8(d)) {
    const float* kvn = reinterpret_cast<const float*>(base + W.kvn);
    if (hipError_t e = ds::launch_kv_store_i8(ds::F32, kvn, kvn + H, 2 * H, kv->k, kv->v, kv->k_scale, kv->v_scale,
                                              kv->d_len, batch, ntok, d.heads, d.head_dim, kv->capacity, st))
      return hip_fail(e, "int8 kv store launch");
  }
  mark(st, DS_PART_QKV);

  // 2: attention over the cache
  ds::AttnArgs at{};
  at.q = reinterpret_cast<const float*>(base + W.q);
  at.k_cache = kv->k; at.v_cache = kv->v; at.d_len = kv->d_len;
  at.part = reinterpret_cast<float*>(base + W.part);
  at.counters = reinterpret_cast<uint32_t*>(base + W.cnt);
  at.ctx = reinterpret_cast<float*>(base + W.ctx);
  at.rows = rows; at.tokens = ntok; at.heads = d.heads; at.head_dim = d.head_dim;
  at.cap = kv->capacity; at.chunk = W.chunk; at.nchunk = W.nchunk; at.causal = d.triangular_masking;
  at.k_scale = kv_int8(d) ? kv->k_scale : nullptr;
  at.v_scale = kv_int8(d) ? kv->v_scale : nullptr;
  if (hipError_t e = ds::launch_attn_decode(adt, at, st)) return hip_fail(e, "attention launch");
  mark(st, DS_PART_ATTN);

  // 3: x2 = x + Wo ctx + bo
  a = g;
  a.w = L->w.w_o; a.s = L->w.s_o; a.bias = L->w.b_o;
  a.in = base + W.ctx; a.resid = x; a.out = base + W.x2;
  a.n = H; a.k = H;
  if (hipError_t e = ds::launch_gemv(wdt, adt, ds::KIND_OPROJ, a, st)) return hip_fail(e, "o_proj launch");
  mark(st, DS_PART_O);

  // 4: f = GeLU(W1 LN2(x2) + b1)
  a = g;
  a.w = L->w.w_ff1; a.s = L->w.s_ff1; a.bias = L->w.b_ff1;
  a.in = base + W.x2; a.ln_g = L->w.ln2_g; a.ln_b = L->w.ln2_b; a.out = base + W.f;
  a.n = F; a.k = H; a.group = group_mlp;
  if (hipError_t e = ds::launch_gemv(wdt, adt, ds::KIND_FF1, a, st)) return hip_fail(e, "ln_ff1 launch");
  mark(st, DS_PART_FF1);

  // 5: y = x2 + W2 f + b2, then d_len += ntok
  a = g;
  a.w = L->w.w_ff2; a.s = L->w.s_ff2; a.bias = L->w.b_ff2;
  a.in = base + W.f; a.resid = base + W.x2; a.out = y;
  a.n = H; a.k = F; a.group = group_mlp;
  if (hipError_t e = ds::launch_gemv(wdt, adt, ds::KIND_FF2, a, st)) return hip_fail(e, "ff2 launch");
  mark(st, DS_PART_FF2);
  if (hipError_t e = ds::launch_len_advance(kv->d_len, batch, ntok, kv->capacity, st)) return hip_fail(e, "len advance launch");
  mark(st, DS_PART_LEN);

  if (kv->h_len)
    for (int b = 0; b < batch; ++b) kv->h_len[b] += ntok;
  return DS_OK;
}

}  // namespace

extern "C" {

const char* ds_last_error(void) { return g_err.c_str(); }

int ds_layer_create(const ds_layer_desc* desc, const ds_layer_weights* w, ds_layer_t** out) {
  if (!desc || !w || !out) return fail(DS_ERR_NULL, "desc, weights or out is NULL");
  *out = nullptr;
  const ds_layer_desc& d = *desc;
  if (d.heads < 1 || (d.head_dim != 64 && d.head_dim != 128))
    return fail(DS_ERR_SHAPE, "heads %d must be >= 1 and head_dim %d must be 64 or 128", d.heads, d.head_dim);
  if ((int64_t)d.heads * d.head_dim != d.hidden)
    return fail(DS_ERR_SHAPE, "hidden %d != heads %d * head_dim %d", d.hidden, d.heads, d.head_dim);
  if (d.hidden % 64 || d.ffn < 64 || d.ffn % 64 || d.hidden > 65536 || d.ffn > 262144)
    return fail(DS_ERR_SHAPE, "hidden %d and ffn %d must be positive multiples of 64 (hidden <= 65536, ffn <= 262144)", d.hidden, d.ffn);
  const bool pair_ok = (d.weight_dtype == DS_F32 && d.act_dtype == DS_F32) ||
                       (d.weight_dtype == DS_F16 && d.act_dtype == DS_F16) ||
                       (d.weight_dtype == DS_I8 && d.act_dtype == DS_F16) ||
                       (d.weight_dtype == DS_BF16 && d.act_dtype == DS_BF16);
  if (!pair_ok) return fail(DS_ERR_DTYPE, "unsupported (weight, activation) dtype pair (%d, %d)", d.weight_dtype, d.act_dtype);
  if (d.weight_dtype == DS_I8) {
    // a lane's 16 consecutive codes share one scale: groups are multiples of 16 dividing the
    // reduction dimension of their matrices (hidden for W_qkv, W_o, W_ff1; ffn for W_ff2)
    const int gm = d.quant_group_mlp ? d.quant_group_mlp : d.quant_group;
    if (d.quant_group < 16 || d.quant_group % 16 || d.hidden % d.quant_group)
      return fail(DS_ERR_SHAPE, "int8 quant_group %d must be a multiple of 16 dividing hidden %d", d.quant_group, d.hidden);
    if (d.quant_group_mlp < 0 || gm < 16 || gm % 16 || d.hidden % gm || d.ffn % gm)
      return fail(DS_ERR_SHAPE, "int8 MLP group %d must be a multiple of 16 dividing hidden %d and ffn %d", gm, d.hidden,
                  d.ffn);
  } else if (d.quant_group != 0 || d.quant_group_mlp != 0) {
    return fail(DS_ERR_DTYPE, "quant_group %d and quant_group_mlp %d must be 0 for non-int8 weights", d.quant_group,
                d.quant_group_mlp);
  }
  if (!(d.ln_eps > 0.f) || !std::isfinite(d.ln_eps)) return fail(DS_ERR_SHAPE, "ln_eps must be finite and > 0");
  if (d.kv_dtype != 0 && d.kv_dtype != DS_I8) return fail(DS_ERR_DTYPE, "kv_dtype %d must be 0 or DS_I8", d.kv_dtype);
  if (d.kv_dtype == DS_I8 && d.act_dtype != DS_F16 && d.act_dtype != DS_BF16)
    return fail(DS_ERR_DTYPE, "an int8 kv cache needs fp16 or bf16 activations");
  if ((d.gelu_tanh != 0 && d.gelu_tanh != 1) || (d.triangular_masking != 0 && d.triangular_masking != 1))
    return fail(DS_ERR_SHAPE, "gelu_tanh and triangular_masking must be 0 or 1");

  const void* req[] = {w->ln1_g, w->ln1_b, w->w_qkv, w->b_qkv, w->w_o, w->b_o,
                       w->ln2_g, w->ln2_b, w->w_ff1, w->b_ff1, w->w_ff2, w->b_ff2};
  for (const void* p : req) {
    if (!p) return fail(DS_ERR_NULL, "a weight, bias or LayerNorm pointer is NULL");
    if (!aligned16(p)) return fail(DS_ERR_ALIGN, "a weight, bias or LayerNorm pointer is not 16-byte aligned");
  }
  const void* sc[] = {w->s_qkv, w->s_o, w->s_ff1, w->s_ff2};
  for (const void* p : sc) {
    if (d.weight_dtype == DS_I8) {
      if (!p) return fail(DS_ERR_NULL, "int8 weights need all four scale pointers");
      if (!aligned16(p)) return fail(DS_ERR_ALIGN, "a scale pointer is not 16-byte aligned");
    } else if (p) {
      return fail(DS_ERR_DTYPE, "scale pointers must be NULL for non-int8 weights");
    }
  }
  ds_layer* L = new (std::nothrow) ds_layer;
  if (!L) return fail(DS_ERR_NULL, "out of host memory");
  L->desc = d;
  L->w = *w;
  if (const char* env = std::getenv("DS_GEMM_CONFIG")) {
    char* end = nullptr;
    const long v = std::strtol(env, &end, 10);
    if (end != env && *end == '\0' && v >= 0 && v <= 2) L->gemm_cfg = (int)v;
  }
  *out = L;
  return DS_OK;
}

int ds_layer_destroy(ds_layer_t* layer) {
  delete layer;
  return DS_OK;
}

size_t ds_layer_workspace_bytes(const ds_layer_t* layer, int32_t max_batch, int32_t max_tokens, int32_t capacity) {
  if (!layer || max_batch < 1 || max_tokens < 1 || capacity < 1) return 0;
  return ws_layout(layer->desc, max_batch * max_tokens, capacity).total;
}

int ds_kv_append(const ds_layer_t* layer, ds_kv_cache* kv, const void* k_new, const void* v_new,
                 int32_t batch, int32_t ntok, void* stream) {
  if (!layer) return fail(DS_ERR_NULL, "layer is NULL");
  if (int rc = check_kv(layer, kv, batch, ntok)) return rc;
  if (batch == 0 || ntok == 0) return DS_OK;
  if (!k_new || !v_new) return fail(DS_ERR_NULL, "k_new or v_new is NULL");
  if (!aligned16(k_new) || !aligned16(v_new)) return fail(DS_ERR_ALIGN, "k_new or v_new is not 16-byte aligned");
  const ds_layer_desc& d = layer->desc;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  hipError_t e = kv_int8(d) ? ds::launch_kv_store_i8(static_cast<ds::Dt>(d.act_dtype), k_new, v_new, d.hidden, kv->k,
                                                     kv->v, kv->k_scale, kv->v_scale, kv->d_len, batch, ntok, d.heads,
                                                     d.head_dim, kv->capacity, st)
                            : ds::launch_kv_append(static_cast<ds::Dt>(d.act_dtype), k_new, v_new, kv->k, kv->v,
                                                   kv->d_len, batch, ntok, d.heads, d.head_dim, kv->capacity, st);
  if (e != hipSuccess) return hip_fail(e, "kv_append launch");
  if (hipError_t e = ds::launch_len_advance(kv->d_len, batch, ntok, kv->capacity, st)) return hip_fail(e, "len advance launch");
  if (kv->h_len)
    for (int b = 0; b < batch; ++b) kv->h_len[b] += ntok;
  return DS_OK;
}

int ds_layer_forward_decode(const ds_layer_t* layer, ds_kv_cache* kv, const void* x, void* y, int32_t batch,
                            void* workspace, size_t workspace_bytes, void* stream) {
  return forward_rows(layer, kv, x, y, batch, 1, workspace, workspace_bytes, stream);
}

int ds_layer_forward_prefill(const ds_layer_t* layer, ds_kv_cache* kv, const void* x, void* y, int32_t batch,
                             int32_t seq, void* workspace, size_t workspace_bytes, void* stream) {
  if (seq < 0) return fail(DS_ERR_SHAPE, "seq %d < 0", seq);
  return forward_rows(layer, kv, x, y, batch, seq, workspace, workspace_bytes, stream);
}

int ds_layer_time_kernels(const ds_layer_t* layer, ds_kv_cache* kv, const void* x, void* y, int32_t batch,
                          int32_t ntok, void* workspace, size_t workspace_bytes, void* stream, float* ms,
                          int32_t* kinds, int32_t max) {
  if (!ms || !kinds) return fail(DS_ERR_NULL, "ms or kinds is NULL");
  if (max < 1 || ntok < 1) return fail(DS_ERR_SHAPE, "max %d and ntok %d must be >= 1", max, ntok);
  KernelTimer t;
  int made = 0;
  hipError_t e = hipSuccess;
  for (; made <= kMaxMarks && e == hipSuccess; ++made) e = hipEventCreate(&t.ev[made]);
  if (e != hipSuccess) --made;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  int rc = DS_OK;
  if (e == hipSuccess) e = ds::launch_delay(200, st);
  if (e == hipSuccess) e = hipEventRecord(t.ev[0], st);
  if (e != hipSuccess) {
    rc = hip_fail(e, "timer set-up");
  } else {
    g_timer = &t;
    rc = forward_rows(layer, kv, x, y, batch, ntok, workspace, workspace_bytes, stream);
    g_timer = nullptr;
    if (rc == DS_OK && t.failed) rc = fail(DS_ERR_HIP, "recording the kernel events failed");
    if (rc == DS_OK) {
      if ((e = hipEventSynchronize(t.ev[t.n])) != hipSuccess) rc = hip_fail(e, "timer wait");
      for (int i = 0; i < t.n && i < max && rc == DS_OK; ++i) {
        if ((e = hipEventElapsedTime(&ms[i], t.ev[i], t.ev[i + 1])) != hipSuccess) rc = hip_fail(e, "event time");
        kinds[i] = t.kinds[i];
      }
    }
  }
  for (int i = 0; i < made; ++i) (void)hipEventDestroy(t.ev[i]);
  return rc == DS_OK ? (t.n < max ? t.n : max) : rc;
}

int ds_quantize_i8(const float* w, int8_t* q, void* s, int32_t n, int32_t k, int32_t group, void* stream) {
  if (!w || !q || !s) return fail(DS_ERR_NULL, "w, q or s is NULL");
  if (n < 0 || k < 0 || group < 16 || group % 16 || k % group) return fail(DS_ERR_SHAPE, "need n, k >= 0, group a multiple of 16 dividing k");
  if (!aligned16(w) || !aligned16(q)) return fail(DS_ERR_ALIGN, "w or q is not 16-byte aligned");
  if (hipError_t e = ds::launch_quantize_i8(w, q, static_cast<uint16_t*>(s), n, k, group, reinterpret_cast<hipStream_t>(stream)))
    return hip_fail(e, "quantize launch");
  return DS_OK;
}

int ds_read_probe(const void* buf, size_t bytes, uint32_t* out, void* stream) {
  if (!buf || !out) return fail(DS_ERR_NULL, "buf or out is NULL");
  if (!aligned16(buf) || bytes % 16) return fail(DS_ERR_ALIGN, "buf must be 16-byte aligned and bytes a multiple of 16");
  if (hipError_t e = ds::launch_read_probe(buf, bytes, out, reinterpret_cast<hipStream_t>(stream)))
    return hip_fail(e, "read probe launch");
  return DS_OK;
}

int ds_dequantize_i8(const int8_t* q, const void* s, float* w, int32_t n, int32_t k, int32_t group, void* stream) {
  if (!w || !q || !s) return fail(DS_ERR_NULL, "q, s or w is NULL");
  if (n < 0 || k < 0 || group < 16 || group % 16 || k % group) return fail(DS_ERR_SHAPE, "need n, k >= 0, group a multiple of 16 dividing k");
  if (!aligned16(q)) return fail(DS_ERR_ALIGN, "q is not 16-byte aligned");
  if (hipError_t e = ds::launch_dequantize_i8(q, static_cast<const uint16_t*>(s), w, n, k, group, reinterpret_cast<hipStream_t>(stream)))
    return hip_fail(e, "dequantize launch");
  return DS_OK;
}

}  // extern "C"
