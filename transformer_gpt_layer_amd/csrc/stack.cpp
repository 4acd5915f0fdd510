// stack.cpp -- C ABI of the persistent multi-layer decode (ds_stack_* in include/ds_layer.h).
//
// A stack binds L layers that share one description to their L KV caches and runs a whole decode
// step -- every fusion region of every layer ("DeepSpeed Inference 内核优化深度解析", section 三 3.2)
// -- in one cooperative launch. Its persistent device state (the sync block: launch counter, exit
// count, error flag; then the table of layer pointers) lives in a caller-owned buffer; the library
// allocates no device memory.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstring>
#include <mutex>
#include <new>
#include <random>
#include <unordered_map>
#include <vector>

#include "ds_internal.hpp"
#include "ds_stack.hpp"

struct ds_stack {
  ds_layer_desc desc;
  std::vector<ds_kv_cache> caches;
  int n_layers = 0, max_batch = 0, G = 0, nchunk = 0, device = 0;
  uint64_t uid = 0;  // never reused: names this stack in the workspace registry
  ds::StackHead head{};                 // V == 0: no LM head
  ds::StackLayer* d_layers = nullptr;  // inside the caller's state buffer
  uint32_t* d_sync = nullptr;          // the state buffer's first kSyncBytes
  size_t sync_words = 0;
  uint64_t timeout_ticks = 200000000ull;  // 2 s at the 100 MHz wall clock
};

namespace {

constexpr size_t kStateTable = 1024;  // byte offset of the layer table in the state buffer
static_assert(kStateTable >= ds::kSyncBytes, "sync block fits before the table");

// Launches of one stack on one workspace between two clears: the tags of 2^19 consecutive launches
// are distinct, and the margin covers the counter steps of failed launches that ds_stack_check
// skips.
constexpr uint32_t kClearEvery = (1u << ds::kLaunchBits) - 64u;

// Which stack last used each workspace (by device address), how many of its launches ran since the
// workspace was last cleared, and how many bytes that clear covered.
struct WsUse {
  uint64_t uid = 0;
  uint32_t launches = 0;
  size_t bytes = 0;
};
std::mutex& ws_mutex() {
  static std::mutex m;
  return m;
}
std::unordered_map<uintptr_t, WsUse>& ws_registry() {
  static std::unordered_map<uintptr_t, WsUse> r;
  return r;
}
std::atomic<uint64_t> g_next_uid{1};

// The workspace of ds_stack_forward_decode_static: a file-scope device array, one copy per GPU.
// Host code never passes the array's name to a kernel (on the host it is only a stand-in symbol);
// it passes the device address hipGetSymbolAddress returns for the current device, looked up once
// per device and kept.
constexpr size_t kStaticScratch = DS_STACK_STATIC_SCRATCH_BYTES;
__device__ __align__(256) unsigned char scratch[kStaticScratch];
constexpr int kMaxDevices = 64;
std::mutex& scratch_mutex() {
  static std::mutex m;
  return m;
}
void* g_scratch_ptr[kMaxDevices] = {};

int hip_err(hipError_t e, const char* where);

int static_scratch(void** out) {
  int dev = 0;
  if (hipError_t e = hipGetDevice(&dev)) return hip_err(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return ds::set_error(DS_ERR_UNSUPPORTED, "device %d beyond %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> g(scratch_mutex());
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch))) return hip_err(e, "static scratch address");
    if (!p) return ds::set_error(DS_ERR_HIP, "static scratch address is NULL");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return DS_OK;
}

int stack_forward(ds_stack_t* S, const void* x, void* y, float* logits, int32_t* tokens, bool head, int32_t batch,
                  void* ws, size_t ws_bytes, void* stream);

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
size_t up256(size_t v) { return (v + 255) / 256 * 256; }
int slice_elems(int wdt) { return wdt == DS_F32 ? 256 : (wdt == DS_I8 ? 1024 : 512); }
int weight_bytes(int wdt) { return wdt == DS_F32 ? 4 : (wdt == DS_I8 ? 1 : 2); }
size_t act_bytes(int adt) { return adt == DS_F32 ? 4 : 2; }

// fp16 group scales the workgroup stages for its largest phase (int8 weights; 0 otherwise)
uint32_t scale_halves(const ds_layer_desc& d, int V, int G) {
  if (d.weight_dtype != DS_I8) return 0u;
  const int gm = d.quant_group_mlp ? d.quant_group_mlp : d.quant_group;
  return ds::stack_scale_halves(d.hidden, d.ffn, V, G, d.quant_group, gm);
}

// The largest int8 scale group among the stack's matrices (1 for other weight dtypes).
int max_group(const ds_layer_desc& d) {
  if (d.weight_dtype != DS_I8) return 1;
  const int gm = d.quant_group_mlp ? d.quant_group_mlp : d.quant_group;
  return gm > d.quant_group ? gm : d.quant_group;
}

struct StackWs {
  size_t q, knew, vnew, part, ctx, x2, f, y, total;
};

// Every value that crosses workgroups is stored tagged: 8 bytes per element.
StackWs stack_ws(const ds_stack& S, int batch) {
  const ds_layer_desc& d = S.desc;
  StackWs W{};
  size_t off = 0;
  auto take = [&](size_t elems) { size_t at = off; off += up256(elems * 8); return at; };
  W.q = take((size_t)batch * d.hidden);
  W.knew = take((size_t)batch * d.hidden);
  W.vnew = take((size_t)batch * d.hidden);
  W.part = take((size_t)batch * d.heads * S.nchunk * (d.head_dim + 2));
  W.ctx = take((size_t)batch * d.hidden);
  W.x2 = take((size_t)batch * d.hidden);
  W.f = take((size_t)batch * d.ffn);
  W.y = take((size_t)batch * d.hidden);
  W.total = off;
  return W;
}

int hip_err(hipError_t e, const char* where) {
  return ds::set_error(DS_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

// Before a launch of stack S on the workspace ws (bytes used by this launch): clear it when another
// stack used it last, when this launch uses bytes the last clear did not cover, or when the launch
// counter could come round to a tag the workspace still holds.
int prepare_workspace(const ds_stack& S, void* ws, size_t bytes, hipStream_t st) {
  bool clear;
  {
    std::lock_guard<std::mutex> g(ws_mutex());
    WsUse& u = ws_registry()[reinterpret_cast<uintptr_t>(ws)];
    clear = u.uid != S.uid || u.launches >= kClearEvery || u.bytes < bytes;
    if (clear) u = WsUse{S.uid, 0u, bytes > u.bytes || u.uid != S.uid ? bytes : u.bytes};
    ++u.launches;
  }
  if (clear)
    if (hipError_t e = ds::launch_fill_zero(ws, bytes, st)) return hip_err(e, "workspace clear launch");
  return DS_OK;
}

}  // namespace

extern "C" {

size_t ds_stack_state_bytes(int32_t n_layers) {
  if (n_layers < 1) return 0;
  return up256(kStateTable + sizeof(ds::StackLayer) * (size_t)n_layers);
}

int ds_stack_create(const ds_layer_t* const* layers, const ds_kv_cache* caches, int32_t n_layers,
                    int32_t max_batch, const ds_lm_head* head, void* state, size_t state_bytes,
                    ds_stack_t** out) {
  if (!layers || !caches || !out) return ds::set_error(DS_ERR_NULL, "layers, caches or out is NULL");
  *out = nullptr;
  if (n_layers < 1) return ds::set_error(DS_ERR_SHAPE, "n_layers %d < 1", n_layers);
  if (n_layers > ds::kStackMaxLayers)
    return ds::set_error(DS_ERR_UNSUPPORTED, "persistent decode handles at most %d layers, got %d", ds::kStackMaxLayers, n_layers);
  if (!state) return ds::set_error(DS_ERR_NULL, "state buffer is NULL");
  if (!aligned16(state)) return ds::set_error(DS_ERR_ALIGN, "state buffer is not 16-byte aligned");
  if (state_bytes < ds_stack_state_bytes(n_layers))
    return ds::set_error(DS_ERR_WORKSPACE, "state buffer %zu bytes < %zu needed", state_bytes, ds_stack_state_bytes(n_layers));
  if (max_batch < 1 || max_batch > 4)
    return ds::set_error(DS_ERR_UNSUPPORTED, "persistent decode handles batch 1..4, got %d", max_batch);
  if (layers[0] && layers[0]->desc.weight_dtype == DS_F32 && max_batch > 1)
    return ds::set_error(DS_ERR_UNSUPPORTED, "persistent decode with fp32 weights handles batch 1 only");
  for (int l = 0; l < n_layers; ++l)
    if (!layers[l]) return ds::set_error(DS_ERR_NULL, "layer %d is NULL", l);
  const ds_layer_desc d = layers[0]->desc;
  const bool kv8 = d.kv_dtype == DS_I8;
  if (kv8 && d.act_dtype != DS_F16 && d.act_dtype != DS_BF16)
    return ds::set_error(DS_ERR_UNSUPPORTED, "persistent decode with an int8 kv cache needs fp16 or bf16 activations");
  for (int l = 1; l < n_layers; ++l)
    if (std::memcmp(&layers[l]->desc, &d, sizeof d) != 0)
      return ds::set_error(DS_ERR_SHAPE, "layer %d has a different description from layer 0", l);
  const int sl = slice_elems(d.weight_dtype);
  const size_t wsz = (size_t)weight_bytes(d.weight_dtype);
  if ((size_t)d.hidden * d.ffn * wsz >= (1ull << 31) || (size_t)3 * d.hidden * d.hidden * wsz >= (1ull << 31))
    return ds::set_error(DS_ERR_UNSUPPORTED, "persistent decode needs every weight matrix under 2 GiB");
  if (d.hidden % sl || d.ffn % sl || d.hidden > 8192)
    return ds::set_error(DS_ERR_UNSUPPORTED, "persistent decode needs hidden and ffn multiples of %d and hidden <= 8192", sl);
  if (d.weight_dtype == DS_I8 && (size_t)(d.hidden > d.ffn ? d.hidden : d.ffn) * (size_t)max_group(d) >= (1ull << 32))
    return ds::set_error(DS_ERR_UNSUPPORTED, "persistent decode needs row length x int8 group below 2^32");
  for (int l = 0; l < n_layers; ++l) {
    const ds_kv_cache& c = caches[l];
    if (!c.k || !c.v || !c.d_len) return ds::set_error(DS_ERR_NULL, "cache %d: k, v or d_len is NULL", l);
    if (!aligned16(c.k) || !aligned16(c.v)) return ds::set_error(DS_ERR_ALIGN, "cache %d is not 16-byte aligned", l);
    if (kv8 && (!c.k_scale || !c.v_scale))
      return ds::set_error(DS_ERR_NULL, "cache %d: an int8 kv cache needs k_scale and v_scale", l);
    if (kv8 && (!aligned16(c.k_scale) || !aligned16(c.v_scale)))
      return ds::set_error(DS_ERR_ALIGN, "cache %d: kv scales are not 16-byte aligned", l);
    if (!kv8 && (c.k_scale || c.v_scale))
      return ds::set_error(DS_ERR_DTYPE, "cache %d has scales but the layers' kv cache is not int8", l);
    if (c.batch < max_batch || c.capacity < 1 || c.capacity != caches[0].capacity)
      return ds::set_error(DS_ERR_SHAPE, "cache %d: batch %d < %d or capacity differs from cache 0", l, c.batch, max_batch);
    if ((size_t)c.batch * d.heads * c.capacity * d.head_dim * (kv8 ? 1 : act_bytes(d.act_dtype)) >= (1ull << 31))
      return ds::set_error(DS_ERR_UNSUPPORTED, "cache %d is 2 GiB or larger", l);
  }

  if (head) {
    if (!head->ln_g || !head->ln_b || !head->w) return ds::set_error(DS_ERR_NULL, "LM head ln_g, ln_b or w is NULL");
    if (!aligned16(head->ln_g) || !aligned16(head->ln_b) || !aligned16(head->w))
      return ds::set_error(DS_ERR_ALIGN, "an LM head pointer is not 16-byte aligned");
    if ((d.weight_dtype == DS_I8) != (head->s != nullptr) || (head->s && !aligned16(head->s)))
      return ds::set_error(DS_ERR_DTYPE, "LM head scales: required (16-byte aligned) for int8 weights, NULL otherwise");
    if (head->vocab < 1 || (size_t)head->vocab * d.hidden * wsz >= (1ull << 31))
      return ds::set_error(DS_ERR_SHAPE, "LM head vocab %d must be >= 1 with its weights under 2 GiB", head->vocab);
  }
  ds_stack* S = new (std::nothrow) ds_stack;
  if (!S) return ds::set_error(DS_ERR_NULL, "out of host memory");
  S->desc = d;
  S->caches.assign(caches, caches + n_layers);
  S->n_layers = n_layers;
  S->max_batch = max_batch;
  S->nchunk = (caches[0].capacity + ds::kStackChunk - 1) / ds::kStackChunk;
  if (head) S->head = ds::StackHead{head->ln_g, head->ln_b, head->w, head->s, head->vocab};
  const ds::Dt wdt = static_cast<ds::Dt>(d.weight_dtype), adt = static_cast<ds::Dt>(d.act_dtype);
  hipError_t e = hipGetDevice(&S->device);
  int cus = 0;
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, S->device);
  const int wsz_i = weight_bytes(d.weight_dtype);
  const int bm = max_batch <= 1 ? 1 : 4;
  int G = cus;  // one workgroup of kStackThreads per CU
  for (int iter = 0; e == hipSuccess && iter < 3; ++iter) {
    const ds::StackLds lay = ds::stack_lds_layout(wsz_i, bm, d.hidden, d.ffn, ds::stack_rows_per_wg(d.hidden, d.ffn, S->head.V, G),
                                                  S->nchunk, d.head_dim, scale_halves(d, S->head.V, G), n_layers);
    if (lay.total > (uint32_t)ds::kStackLdsMax - 4096u) {  // the static control block takes the rest
      delete S;
      return ds::set_error(DS_ERR_UNSUPPORTED, "persistent decode: %u bytes of LDS per workgroup needed", lay.total);
    }
    int fit = 0;
    e = ds::stack_max_groups(wdt, adt, kv8, max_batch, ds::stack_group_slices(wdt, d.hidden, d.ffn), lay.total, &fit);
    if (e == hipSuccess) G = G < fit ? G : fit;
  }
  if (e != hipSuccess || G < 1) {
    delete S;
    return e != hipSuccess ? hip_err(e, "stack occupancy query") : ds::set_error(DS_ERR_UNSUPPORTED, "no co-resident workgroup fits");
  }
  S->G = G;

  std::vector<ds::StackLayer> table(n_layers);
  for (int l = 0; l < n_layers; ++l) {
    const ds_layer_weights& w = layers[l]->w;
    table[l] = ds::StackLayer{w.ln1_g, w.ln1_b, w.w_qkv, w.b_qkv, w.s_qkv, w.w_o, w.b_o, w.s_o,
                              w.ln2_g, w.ln2_b, w.w_ff1, w.b_ff1, w.s_ff1, w.w_ff2, w.b_ff2, w.s_ff2,
                              caches[l].k, caches[l].v, caches[l].d_len, caches[l].k_scale, caches[l].v_scale};
  }
  S->sync_words = ds::kSyncWords;
  S->uid = g_next_uid.fetch_add(1);
  S->d_sync = static_cast<uint32_t*>(state);
  S->d_layers = reinterpret_cast<ds::StackLayer*>(static_cast<char*>(state) + kStateTable);
  e = hipMemcpy(S->d_layers, table.data(), sizeof(ds::StackLayer) * n_layers, hipMemcpyHostToDevice);
  if (e == hipSuccess) {
    // the launch counter starts at a random value: a second line of defence, besides the clear on
    // a change of owner, against values some other stack left in a shared workspace
    std::vector<uint32_t> init(S->sync_words, 0u);
    init[ds::kSyncLaunch] = std::random_device{}() & ds::kLaunchMask;
    e = hipMemcpy(S->d_sync, init.data(), S->sync_words * 4, hipMemcpyHostToDevice);
  }
  if (e == hipSuccess) e = hipDeviceSynchronize();
  if (e != hipSuccess) {
    delete S;
    return hip_err(e, "stack device state");
  }
  *out = S;
  return DS_OK;
}

int ds_stack_destroy(ds_stack_t* S) {
  if (!S) return DS_OK;
  {
    std::lock_guard<std::mutex> g(ws_mutex());
    auto& reg = ws_registry();
    for (auto it = reg.begin(); it != reg.end();)
      it = it->second.uid == S->uid ? reg.erase(it) : std::next(it);
  }
  delete S;
  return DS_OK;
}

size_t ds_stack_workspace_bytes(const ds_stack_t* S, int32_t batch) {
  if (!S || batch < 1 || batch > S->max_batch) return 0;
  return stack_ws(*S, batch).total;
}

int32_t ds_stack_groups(const ds_stack_t* S) { return S ? S->G : 0; }

int ds_stack_forward_decode(ds_stack_t* S, const void* x, void* y, int32_t batch, void* ws, size_t ws_bytes,
                            void* stream) {
  return stack_forward(S, x, y, nullptr, nullptr, false, batch, ws, ws_bytes, stream);
}

int ds_stack_forward_generate(ds_stack_t* S, const void* x, void* y, float* logits, int32_t* tokens, int32_t batch,
                              void* ws, size_t ws_bytes, void* stream) {
  if (!S) return ds::set_error(DS_ERR_NULL, "stack is NULL");
  if (S->head.V < 1) return ds::set_error(DS_ERR_UNSUPPORTED, "this stack was created without an LM head");
  if (!tokens) return ds::set_error(DS_ERR_NULL, "tokens is NULL");
  if (!aligned16(tokens) || (logits && !aligned16(logits)))
    return ds::set_error(DS_ERR_ALIGN, "tokens or logits is not 16-byte aligned");
  return stack_forward(S, x, y, logits, tokens, true, batch, ws, ws_bytes, stream);
}

int ds_stack_forward_decode_static(ds_stack_t* S, const void* x, void* y, int32_t batch, void* stream) {
  if (!S) return ds::set_error(DS_ERR_NULL, "stack is NULL");
  if (batch < 1 || batch > S->max_batch) return ds::set_error(DS_ERR_SHAPE, "batch %d outside [1, %d]", batch, S->max_batch);
  const size_t need = stack_ws(*S, batch).total;
  if (need > kStaticScratch)
    return ds::set_error(DS_ERR_WORKSPACE, "step needs %zu bytes of workspace; the static scratch holds %zu", need,
                         kStaticScratch);
  void* ws = nullptr;
  if (int rc = static_scratch(&ws)) return rc;
  return stack_forward(S, x, y, nullptr, nullptr, false, batch, ws, kStaticScratch, stream);
}

}  // extern "C"

namespace {

int stack_forward(ds_stack_t* S, const void* x, void* y, float* logits, int32_t* tokens, bool head, int32_t batch,
                  void* ws, size_t ws_bytes, void* stream) {
  if (!S) return ds::set_error(DS_ERR_NULL, "stack is NULL");
  if (batch < 1 || batch > S->max_batch) return ds::set_error(DS_ERR_SHAPE, "batch %d outside [1, %d]", batch, S->max_batch);
  if (!x || !y || !ws) return ds::set_error(DS_ERR_NULL, "x, y or workspace is NULL");
  if (!aligned16(x) || !aligned16(y) || !aligned16(ws)) return ds::set_error(DS_ERR_ALIGN, "x, y or workspace is not 16-byte aligned");
  const StackWs W = stack_ws(*S, batch);
  if (ws_bytes < W.total) return ds::set_error(DS_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, W.total);
  const int cap = S->caches[0].capacity;
  for (int l = 0; l < S->n_layers; ++l) {
    const int32_t* hl = S->caches[l].h_len;
    if (!hl) continue;
    for (int b = 0; b < batch; ++b)
      if (hl[b] < 0 || hl[b] + 1 > cap)
        return ds::set_error(DS_ERR_KV_FULL, "layer %d sequence %d: %d rows + 1 > capacity %d", l, b, hl[b], cap);
  }
  const ds_layer_desc& d = S->desc;
  char* base = static_cast<char*>(ws);
  ds::StackArgs a{};
  a.layers = S->d_layers;
  a.n_layers = S->n_layers;
  a.x = x;
  a.y = y;
  a.B = batch;
  a.H = d.hidden;
  a.nh = d.heads;
  a.d = d.head_dim;
  a.F = d.ffn;
  a.cap = cap;
  a.group = d.quant_group;
  a.group_mlp = d.quant_group_mlp ? d.quant_group_mlp : d.quant_group;
  a.kv8 = d.kv_dtype == DS_I8 ? 1 : 0;
  a.eps = d.ln_eps;
  a.gelu_tanh = d.gelu_tanh;
  a.q = reinterpret_cast<uint2*>(base + W.q);
  a.knew = reinterpret_cast<uint2*>(base + W.knew);
  a.vnew = reinterpret_cast<uint2*>(base + W.vnew);
  a.part = reinterpret_cast<uint2*>(base + W.part);
  a.ctx = reinterpret_cast<uint2*>(base + W.ctx);
  a.x2 = reinterpret_cast<uint2*>(base + W.x2);
  a.f = reinterpret_cast<uint2*>(base + W.f);
  a.ybuf = reinterpret_cast<uint2*>(base + W.y);
  a.sync = S->d_sync;
  a.G = S->G;
  a.nchunk = S->nchunk;
  a.timeout_ticks = S->timeout_ticks;
  a.head = head ? 1 : 0;
  a.V = S->head.V;
  a.head_g = S->head.ln_g;
  a.head_b = S->head.ln_b;
  a.head_w = S->head.w;
  a.head_s = S->head.s;
  a.logits = logits;
  a.tokens = tokens;
  const ds::Dt wdt = static_cast<ds::Dt>(d.weight_dtype), adt = static_cast<ds::Dt>(d.act_dtype);
  const int wsz_i = weight_bytes(d.weight_dtype);
  a.lds = ds::stack_lds_layout(wsz_i, batch <= 1 ? 1 : 4, d.hidden, d.ffn, ds::stack_rows_per_wg(d.hidden, d.ffn, S->head.V, S->G),
                               S->nchunk, d.head_dim, scale_halves(d, S->head.V, S->G), S->n_layers);
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (int rc = prepare_workspace(*S, ws, W.total, st)) return rc;
  if (hipError_t e = ds::launch_stack_decode(wdt, adt, a, st))
    return hip_err(e, "persistent decode launch");
  for (int l = 0; l < S->n_layers; ++l)
    if (int32_t* hl = S->caches[l].h_len)
      for (int b = 0; b < batch; ++b) hl[b] += 1;
  return DS_OK;
}

}  // namespace

extern "C" {

int ds_stack_check(ds_stack_t* S) {
  if (!S) return ds::set_error(DS_ERR_NULL, "stack is NULL");
  std::vector<uint32_t> words(S->sync_words);
  hipError_t e = hipDeviceSynchronize();
  if (e == hipSuccess) e = hipMemcpy(words.data(), S->d_sync, S->sync_words * 4, hipMemcpyDeviceToHost);
  if (e != hipSuccess) return hip_err(e, "stack check");
  const uint32_t err = words[ds::kSyncError], exits = words[ds::kSyncExit];
  if (err != 0u || exits != 0u) {
    // a failed launch: clear the error and the exit count, and move the launch counter on so that
    // no value that launch stored carries a tag the next one waits for
    words[ds::kSyncError] = 0u;
    words[ds::kSyncExit] = 0u;
    words[ds::kSyncLaunch] = (words[ds::kSyncLaunch] + 1u) & ds::kLaunchMask;
    for (int i = 0; i < 4 * ds::kStackMaxBatch; ++i) words[ds::kSyncArgmax + i] = 0u;  // both key slots
    (void)hipMemcpy(S->d_sync, words.data(), S->sync_words * 4, hipMemcpyHostToDevice);
    // the host mirrors were advanced when the failed steps were enqueued; the device lengths were
    // not (only a completed launch advances them): take the device's
    for (const ds_kv_cache& c : S->caches)
      if (c.h_len) (void)hipMemcpy(c.h_len, c.d_len, sizeof(int32_t) * (size_t)S->max_batch, hipMemcpyDeviceToHost);
    (void)hipDeviceSynchronize();
    return ds::set_error(DS_ERR_HIP, "persistent decode: a wait timed out (error flag %u, %u of %d workgroups "
                         "finished); state reset, outputs of the failed step are invalid", err, exits, S->G);
  }
  return DS_OK;
}

int ds_stack_set_timeout_us(ds_stack_t* S, int64_t us) {
  if (!S) return ds::set_error(DS_ERR_NULL, "stack is NULL");
  if (us < 1) return ds::set_error(DS_ERR_SHAPE, "timeout must be >= 1 us");
  S->timeout_ticks = (uint64_t)us * 100u;
  return DS_OK;
}

}  // extern "C"
