// ds_launch.hpp -- internal interface between the C ABI (layer.cpp) and the kernel launchers.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace ds {

enum Dt { F32 = 0, F16 = 1, I8 = 2, BF16 = 3 };
enum GemvKind { KIND_QKV = 0, KIND_OPROJ = 1, KIND_FF1 = 2, KIND_FF2 = 3 };

// Arguments of one fused GEMV launch over `rows` activation rows (rows = batch * tokens).
struct GemvArgs {
  const void* w;       // [n][k] weights (f32, f16 or int8)
  const void* s;       // fp16 [n][k/group] scales (int8 only)
  const void* bias;    // [n] in the activation type
  const void* in;      // [rows][k] input: activation type for KIND_QKV, else fp32 workspace
  const void* ln_g;    // LayerNorm parameters (KIND_QKV, KIND_FF1), activation type
  const void* ln_b;
  const void* resid;   // [rows][n] residual: activation type (KIND_OPROJ) or fp32 (KIND_FF2)
  void* out;           // fp32 [rows][n] (KIND_OPROJ, KIND_FF1), activation type (KIND_FF2)
  // KIND_QKV scatter: q to fp32 [rows][H], k and v into the caches at row d_len[seq] + t
  float* q_out;
  void* k_cache;
  void* v_cache;
  const int32_t* d_len;
  uint32_t* attn_counters;  // zeroed by the KIND_QKV launch: rows * heads counters
  float* kv_new;            // KIND_QKV with an int8 cache: k and v as fp32 [rows][2H] instead of the cache
  int n, k, group, rows, tokens, cap, heads, head_dim, hidden;
  float eps;
  int gelu_tanh;
};

struct AttnArgs {
  const float* q;      // [rows][H] fp32 (unscaled)
  const void* k_cache; // [batch][heads][cap][d]
  const void* v_cache;
  const int32_t* d_len;
  float* part;         // [rows][heads][nchunk][d + 2] partial (max, sum, acc[d])
  uint32_t* counters;  // [rows][heads]
  float* ctx;          // [rows][H] fp32 output
  int rows, tokens, heads, head_dim, cap, chunk, nchunk, causal;
  // 16-bit q and ctx in place of q and ctx (launch_attn_decode_16: fp16, or bf16 values)
  const _Float16* q16;
  _Float16* ctx16;
  // an int8 cache: fp16 row scales [batch][heads][cap] (null for a cache in the activation type)
  const void* k_scale;
  const void* v_scale;
};

// The MoE expert FF of one step (kernels_moe.hip). T tokens, each with k chosen experts plus, for
// the residual type, the residual MLP as slot k: KS = k + residual slots per token.
constexpr int kMoeMaxK = 8;          // experts per token at most
constexpr int kMoeMaxExperts = 1023; // experts per layer at most (the residual MLP is one more)
constexpr int kMoeMaxPairs = 4096;   // tokens x slots at most per step
struct MoeArgs {
  const void* x2;      // [T][H] activation type
  void* y;             // [T][H] activation type
  const void *ln_g, *ln_b, *w_gate;                     // [H], [H], [E][H] activation type
  const void *w1, *b1, *s1, *w2, *b2, *s2;              // experts [E][F][H], [E][F], ..., [E][H][F], [E][H]
  const void *r_w1, *r_b1, *r_s1, *r_w2, *r_b2, *r_s2;  // the residual MLP, or null
  void* h;             // [T][H] LayerNorm output in the staged type
  float* logits;       // [T][E] gate logits
  int32_t* sel;        // [T][KS] expert of each slot (E: the residual MLP)
  float* wgt;          // [T][KS] combine weight of each slot
  int32_t* route;      // 1 + 3 umax + T KS ints (kernels_moe.hip, Route)
  void* f;             // [T KS][F] GeLU(W1 h + b1) per slot, in the staged type
  float* z;            // [T KS][H] W2 f + b2 per slot
  int32_t* sel_out;    // optional [T][k]
  float* wgt_out;      // optional [T][k]
  int T, H, F, E, k, KS, umax, group, residual, combine, gelu_tanh;
  int lds_act;         // activation staging bytes of an expert workgroup (set by the launcher)
  float eps;
};
// Called after each of the five launches (part 0 gate, 1 route, 2 FF1, 3 FF2, 4 combine) when set.
typedef void (*MoeKernelHook)(void* ctx, hipStream_t st, int part);
hipError_t launch_moe(Dt wdt, Dt adt, const MoeArgs& a, hipStream_t st, MoeKernelHook hook, void* hook_ctx);

hipError_t launch_gemv(Dt wdt, Dt adt, GemvKind kind, const GemvArgs& a, hipStream_t st);
hipError_t launch_attn_decode(Dt adt, const AttnArgs& a, hipStream_t st);
// The same attention with 16-bit q and ctx (q16, ctx16: fp16, or bf16 with bf16 set, the pointers
// then holding bf16 values) over a cache of that type, or an int8 cache when k_scale is set.
hipError_t launch_attn_decode_16(bool bf16, const AttnArgs& a, hipStream_t st);
int attn_chunk_for(int rows, int heads, int cap);
// Chunks per (row, head) for one launch, at most nmax (see the definition).
int attn_chunks_for(int rows, int heads, int cap, int chunk, int nmax, int cus);

hipError_t launch_kv_append(Dt adt, const void* k_new, const void* v_new, void* kc, void* vc,
                            const int32_t* d_len, int batch, int ntok, int heads, int head_dim,
                            int cap, hipStream_t st);
// An int8 cache (fp16 row scales ks, vs): the rows [batch][ntok] of k and v, each `stride` elements
// apart (type IT: F32 for fp32 rows from a projection, or the activation type), quantized per
// (row, head) into the cache rows d_len[b] + t and their scales.
hipError_t launch_kv_store_i8(Dt it, const void* ksrc, const void* vsrc, int stride, void* kc, void* vc, void* ks,
                              void* vs, const int32_t* d_len, int batch, int ntok, int heads, int head_dim, int cap,
                              hipStream_t st);
// A GPU-side wait of about `microseconds` (the wall clock of the device, one thread).
hipError_t launch_delay(uint32_t microseconds, hipStream_t st);
// Zeroes `bytes` bytes at p (16-byte aligned; the size is rounded down to whole 16-byte pieces).
hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t st);
// d_len[b] += ntok for b < batch, unless that would pass cap
hipError_t launch_len_advance(int32_t* d_len, int batch, int ntok, int cap, hipStream_t st);
// Reads bytes (a multiple of 16) from buf with streaming loads; *out ^= a digest of the data.
hipError_t launch_read_probe(const void* buf, size_t bytes, uint32_t* out, hipStream_t st);
hipError_t launch_quantize_i8(const float* w, int8_t* q, uint16_t* s, int n, int k, int group,
                              hipStream_t st);
hipError_t launch_dequantize_i8(const int8_t* q, const uint16_t* s, float* w, int n, int k,
                                int group, hipStream_t st);
// The same into fp16 (each weight rounded once): the operand of the many-row GEMM for int8 layers.
hipError_t launch_dequantize_i8_f16(const int8_t* q, const uint16_t* s, _Float16* w, int n, int k, int group,
                                    hipStream_t st);

}  // namespace ds
