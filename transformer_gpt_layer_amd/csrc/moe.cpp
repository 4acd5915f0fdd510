// moe.cpp -- the C ABI of the MoE expert FF (include/ds_layer.h, ds_moe_*): validation, the
// workspace layout and the launch sequence (kernels_moe.hip). No device memory is allocated here.
//
// Source: "DeepSpeed MoE 大规模稀疏模型推理实战指南" (blog.gitcode.com), the MoE sections (experts
// per MoE layer; types 'standard' and 'residual'); the gate is the reading stated in ds_layer.h.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <new>

#include "ds_internal.hpp"
#include "ds_launch.hpp"

struct ds_moe {
  ds_moe_desc d;
  ds_moe_weights w;
};

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
size_t up256(size_t v) { return (v + 255) / 256 * 256; }
// the staged type of the experts' activations: fp32 for fp32 weights, else 2 bytes
size_t staged_size(int wdt) { return wdt == DS_F32 ? 4 : 2; }

int slots(const ds_moe_desc& d) { return d.top_k + (d.residual ? 1 : 0); }

struct MoeWs {
  size_t h, logits, sel, wgt, route, f, z, total;
  int umax;
};

MoeWs moe_ws(const ds_moe_desc& d, int T) {
  MoeWs L{};
  const int KS = slots(d), P = T * KS;
  const int ne = d.experts + (d.residual ? 1 : 0);
  L.umax = P < ne ? P : ne;
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t at = off; off += up256(bytes); return at; };
  L.h = take((size_t)T * d.hidden * staged_size(d.weight_dtype));
  L.logits = take((size_t)T * d.experts * 4);
  L.sel = take((size_t)P * 4);
  L.wgt = take((size_t)P * 4);
  L.route = take((size_t)(1 + 3 * L.umax + P) * 4);
  L.f = take((size_t)P * d.ffn * staged_size(d.weight_dtype));
  L.z = take((size_t)P * d.hidden * 4);
  L.total = off;
  return L;
}

int enqueue(const ds_moe* M, const void* x2, void* y, int tokens, int32_t* sel_out, float* wgt_out, void* ws,
            size_t ws_bytes, void* stream, ds::MoeKernelHook hook, void* ctx) {
  if (!M || !x2 || !y || !ws) return ds::set_error(DS_ERR_NULL, "moe, x2, y or workspace is NULL");
  const ds_moe_desc& d = M->d;
  if (tokens < 1 || (int64_t)tokens * slots(d) > ds::kMoeMaxPairs)
    return ds::set_error(DS_ERR_SHAPE, "tokens %d: need 1..%d tokens x %d slots", tokens, ds::kMoeMaxPairs, slots(d));
  if (!aligned16(x2) || !aligned16(y) || !aligned16(ws)) return ds::set_error(DS_ERR_ALIGN, "x2, y or workspace is not 16-byte aligned");
  const MoeWs L = moe_ws(d, tokens);
  if (ws_bytes < L.total) return ds::set_error(DS_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, L.total);
  char* base = static_cast<char*>(ws);
  ds::MoeArgs a{};
  a.x2 = x2;
  a.y = y;
  a.ln_g = M->w.ln_g; a.ln_b = M->w.ln_b; a.w_gate = M->w.w_gate;
  a.w1 = M->w.w1; a.b1 = M->w.b1; a.s1 = M->w.s1;
  a.w2 = M->w.w2; a.b2 = M->w.b2; a.s2 = M->w.s2;
  a.r_w1 = M->w.r_w1; a.r_b1 = M->w.r_b1; a.r_s1 = M->w.r_s1;
  a.r_w2 = M->w.r_w2; a.r_b2 = M->w.r_b2; a.r_s2 = M->w.r_s2;
  a.h = base + L.h;
  a.logits = reinterpret_cast<float*>(base + L.logits);
  a.sel = reinterpret_cast<int32_t*>(base + L.sel);
  a.wgt = reinterpret_cast<float*>(base + L.wgt);
  a.route = reinterpret_cast<int32_t*>(base + L.route);
  a.f = base + L.f;
  a.z = reinterpret_cast<float*>(base + L.z);
  a.sel_out = sel_out;
  a.wgt_out = wgt_out;
  a.T = tokens;
  a.H = d.hidden;
  a.F = d.ffn;
  a.E = d.experts;
  a.k = d.top_k;
  a.KS = slots(d);
  a.umax = L.umax;
  a.group = d.quant_group > 0 ? d.quant_group : 1;
  a.residual = d.residual;
  a.combine = d.combine;
  a.gelu_tanh = d.gelu_tanh;
  a.eps = d.ln_eps;
  const hipError_t e = ds::launch_moe(static_cast<ds::Dt>(d.weight_dtype), static_cast<ds::Dt>(d.act_dtype), a,
                                      reinterpret_cast<hipStream_t>(stream), hook, ctx);
  if (e != hipSuccess) return ds::set_error(DS_ERR_HIP, "moe launch: %s", hipGetErrorString(e));
  return DS_OK;
}

struct MoeTimer {
  hipEvent_t ev[6] = {};
  int n = 0;
  bool failed = false;
};

void moe_mark(void* ctx, hipStream_t st, int) {
  MoeTimer* t = static_cast<MoeTimer*>(ctx);
  if (t->failed || t->n >= 5 || hipEventRecord(t->ev[t->n + 1], st) != hipSuccess) {
    t->failed = true;
    return;
  }
  ++t->n;
}

}  // namespace

extern "C" {

int ds_moe_create(const ds_moe_desc* desc, const ds_moe_weights* w, ds_moe_t** out) {
  if (!desc || !w || !out) return ds::set_error(DS_ERR_NULL, "desc, weights or out is NULL");
  *out = nullptr;
  const ds_moe_desc& d = *desc;
  if (d.hidden < 64 || d.hidden % 64 || d.ffn < 64 || d.ffn % 64 || d.hidden > 65536 || d.ffn > 262144)
    return ds::set_error(DS_ERR_SHAPE, "hidden %d and ffn %d must be positive multiples of 64", d.hidden, d.ffn);
  if (d.experts < 1 || d.experts > ds::kMoeMaxExperts || d.top_k < 1 || d.top_k > ds::kMoeMaxK || d.top_k > d.experts)
    return ds::set_error(DS_ERR_SHAPE, "experts %d must be 1..%d and top_k %d 1..min(%d, experts)", d.experts,
                         ds::kMoeMaxExperts, d.top_k, ds::kMoeMaxK);
  const bool pair_ok = (d.weight_dtype == DS_F32 && d.act_dtype == DS_F32) ||
                       (d.weight_dtype == DS_F16 && d.act_dtype == DS_F16) ||
                       (d.weight_dtype == DS_I8 && d.act_dtype == DS_F16) ||
                       (d.weight_dtype == DS_BF16 && d.act_dtype == DS_BF16);
  if (!pair_ok) return ds::set_error(DS_ERR_DTYPE, "unsupported (weight, activation) dtype pair (%d, %d)", d.weight_dtype, d.act_dtype);
  const bool i8 = d.weight_dtype == DS_I8;
  if (i8 && (d.quant_group < 16 || d.quant_group % 16 || d.hidden % d.quant_group || d.ffn % d.quant_group))
    return ds::set_error(DS_ERR_SHAPE, "int8 quant_group %d must be a multiple of 16 dividing hidden and ffn", d.quant_group);
  if (!i8 && d.quant_group != 0) return ds::set_error(DS_ERR_DTYPE, "quant_group must be 0 for non-int8 weights");
  if (!(d.ln_eps > 0.f) || !std::isfinite(d.ln_eps)) return ds::set_error(DS_ERR_SHAPE, "ln_eps must be finite and > 0");
  if ((d.gelu_tanh != 0 && d.gelu_tanh != 1) || (d.residual != 0 && d.residual != 1) || (d.combine != 0 && d.combine != 1))
    return ds::set_error(DS_ERR_SHAPE, "gelu_tanh, residual and combine must be 0 or 1");
  const void* req[] = {w->ln_g, w->ln_b, w->w_gate, w->w1, w->b1, w->w2, w->b2};
  for (const void* p : req) {
    if (!p) return ds::set_error(DS_ERR_NULL, "a gate, expert or LayerNorm pointer is NULL");
    if (!aligned16(p)) return ds::set_error(DS_ERR_ALIGN, "a gate, expert or LayerNorm pointer is not 16-byte aligned");
  }
  const void* res[] = {w->r_w1, w->r_b1, w->r_w2, w->r_b2};
  for (const void* p : res) {
    if (d.residual && !p) return ds::set_error(DS_ERR_NULL, "the residual type needs r_w1, r_b1, r_w2 and r_b2");
    if (!d.residual && p) return ds::set_error(DS_ERR_SHAPE, "residual MLP pointers are set on a standard MoE");
    if (p && !aligned16(p)) return ds::set_error(DS_ERR_ALIGN, "a residual MLP pointer is not 16-byte aligned");
  }
  const void* sc[] = {w->s1, w->s2, w->r_s1, w->r_s2};
  for (int i = 0; i < 4; ++i) {
    const void* p = sc[i];
    const bool needed = i8 && (i < 2 || d.residual);
    if (needed && !p) return ds::set_error(DS_ERR_NULL, "int8 weights need their scale pointers");
    if (!needed && p) return ds::set_error(DS_ERR_DTYPE, "scale pointers must be NULL here");
    if (p && !aligned16(p)) return ds::set_error(DS_ERR_ALIGN, "a scale pointer is not 16-byte aligned");
  }
  // every expert matrix and its scales fit one 32-bit offset range per expert
  if ((int64_t)d.hidden * d.ffn * (int64_t)(d.weight_dtype == DS_F32 ? 4 : (i8 ? 1 : 2)) >= (int64_t(1) << 31))
    return ds::set_error(DS_ERR_SHAPE, "one expert matrix must stay under 2 GiB");
  ds_moe* M = new (std::nothrow) ds_moe;
  if (!M) return ds::set_error(DS_ERR_NULL, "out of host memory");
  M->d = d;
  M->w = *w;
  *out = M;
  return DS_OK;
}

int ds_moe_destroy(ds_moe_t* moe) {
  delete moe;
  return DS_OK;
}

size_t ds_moe_workspace_bytes(const ds_moe_t* moe, int32_t max_tokens) {
  if (!moe || max_tokens < 1 || (int64_t)max_tokens * slots(moe->d) > ds::kMoeMaxPairs) return 0;
  return moe_ws(moe->d, max_tokens).total;
}

int ds_moe_forward(const ds_moe_t* moe, const void* x2, void* y, int32_t tokens, int32_t* sel_out, float* wgt_out,
                   void* workspace, size_t workspace_bytes, void* stream) {
  return enqueue(moe, x2, y, tokens, sel_out, wgt_out, workspace, workspace_bytes, stream, nullptr, nullptr);
}

int ds_moe_time_kernels(const ds_moe_t* moe, const void* x2, void* y, int32_t tokens, void* workspace,
                        size_t workspace_bytes, void* stream, float* ms, int32_t max) {
  if (!ms) return ds::set_error(DS_ERR_NULL, "ms is NULL");
  if (max < 1) return ds::set_error(DS_ERR_SHAPE, "max %d must be >= 1", max);
  MoeTimer t;
  int made = 0;
  hipError_t e = hipSuccess;
  for (; made < 6 && e == hipSuccess; ++made) e = hipEventCreate(&t.ev[made]);
  if (e != hipSuccess) --made;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  int rc = DS_OK;
  if (e == hipSuccess) e = ds::launch_delay(200, st);
  if (e == hipSuccess) e = hipEventRecord(t.ev[0], st);
  if (e != hipSuccess) {
    rc = ds::set_error(DS_ERR_HIP, "timer set-up: %s", hipGetErrorString(e));
  } else {
    rc = enqueue(moe, x2, y, tokens, nullptr, nullptr, workspace, workspace_bytes, stream, moe_mark, &t);
    if (rc == DS_OK && t.failed) rc = ds::set_error(DS_ERR_HIP, "recording the kernel events failed");
    if (rc == DS_OK) {
      if ((e = hipEventSynchronize(t.ev[t.n])) != hipSuccess) rc = ds::set_error(DS_ERR_HIP, "timer wait: %s", hipGetErrorString(e));
      for (int i = 0; i < t.n && i < max && rc == DS_OK; ++i)
        if ((e = hipEventElapsedTime(&ms[i], t.ev[i], t.ev[i + 1])) != hipSuccess)
          rc = ds::set_error(DS_ERR_HIP, "event time: %s", hipGetErrorString(e));
    }
  }
  for (int i = 0; i < made; ++i) (void)hipEventDestroy(t.ev[i]);
  return rc == DS_OK ? (t.n < max ? t.n : max) : rc;
}

}  // extern "C"
