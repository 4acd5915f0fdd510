// ds_prefill.hpp -- internal interface of the MFMA (many-row) path: LayerNorm rows, the fused-epilogue
// GEMM and attention over the cache for many new rows per sequence.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ds_device.hpp"

namespace ds {

enum GemmEpi { EPI_QKV = 0, EPI_OPROJ = 1, EPI_FF1 = 2, EPI_FF2 = 3 };

// C[M][N] = A[M][K] W[N][K]^T + bias, then by epilogue (T: the layer's 16-bit type, fp16 or bf16;
// the half_t pointers below then hold T elements):
//   EPI_QKV   columns [0,H) -> out T [M][H] (q); [H,2H) and [2H,3H) -> k_cache / v_cache rows
//             d_len[b] + t of sequence b = m / tokens, t = m % tokens, head-major [B][heads][cap][D]
//   EPI_OPROJ out fp32 [M][N] = resid T [M][N] + C
//   EPI_FF1   out T [M][N] = GeLU(C)
//   EPI_FF2   out T [M][N] = resid fp32 [M][N] + C
// A, W, bias: T, K a multiple of 64, M*K*2 and N*K*2 below 2^31 bytes.
struct GemmArgs {
  const half_t* a;
  const half_t* w;
  const half_t* bias;
  void* out;
  const void* resid;
  half_t* k_cache;
  half_t* v_cache;
  const int32_t* d_len;
  int M, N, K;
  int tokens, heads, head_dim, cap, hidden;
  int gelu_tanh;
  int tiles_m, tiles_n;  // set by the launcher
  // int8 weights (skinny path only): codes [N][K] and fp16 scales [N][K/group] in place of w
  const int8_t* wq;
  const half_t* wscale;
  int group;
  // skinny QKV launch with an int8 cache: k and v as fp32 [M][2H] here instead of into the cache
  // (quantized afterwards, one scale per head row); null otherwise
  float* kv_new;
  // skinny QKV launch: zeroes these attention merge counters (and the split counters below) first
  uint32_t* attn_counters;
  int n_counters;
  // skinny launches with K split over workgroups: per-column-block partial tiles and arrival
  // counters (zero at rest: the last arriver of a block resets its counter)
  float* sk_part;
  uint32_t* sk_cnt;
  int n_sk_cnt;
};

// Attention of `tokens` new rows per sequence over keys 0..d_len[b]+tokens-1 of the cache (the new
// rows already appended at d_len[b]..), causal or not; d_len is the length before this step. The
// 16-bit pointers hold the layer's type (fp16, or bf16 with bf16 set at launch).
struct AttnPrefillArgs {
  const half_t* q;        // [batch*tokens][H]
  const half_t* k_cache;  // [batch][heads][cap][head_dim]
  const half_t* v_cache;
  const int32_t* d_len;
  half_t* ctx;            // [batch*tokens][H]
  // an int8 cache: k_cache and v_cache hold int8 codes and these their fp16 row scales
  // [batch][heads][cap] (the kernel dequantizes while staging); null for a 16-bit cache
  const void* k_scale;
  const void* v_scale;
  int batch, tokens, heads, head_dim, cap, causal;
  float scale;            // 1/sqrt(head_dim)
};

// Tile configuration for an M x N x K product on `cus` compute units.
int gemm_pick(int M, int N, int K, int cus);
hipError_t launch_gemm(GemmEpi epi, bool bf16, const GemmArgs& a, int cfg, hipStream_t st);
// LayerNorm of `rows` rows of H elements (fp32 input, or the 16-bit type) into the 16-bit type
// (bf16 when bf16 is set, else fp16; gamma and beta in that type). With d_len, the same launch also
// advances the cache lengths (d_len[b] += ntok for b < batch, unless that would pass cap): for a
// LayerNorm that runs after every reader of the lengths in the step.
hipError_t launch_ln_rows(bool bf16, bool in_f32, const void* x, const void* g, const void* b, void* out, int rows,
                          int H, float eps, hipStream_t st, int32_t* d_len = nullptr, int batch = 0, int ntok = 0,
                          int cap = 0);
hipError_t launch_attn_prefill(bool bf16, const AttnPrefillArgs& a, hipStream_t st);
// The same product and epilogues for M <= 16 rows (decode of a few sequences): every weight row is
// streamed once, with 16-bit weights (w: fp16, or bf16 with bf16 set) or int8 codes and group-64
// scales (wq, wscale, group; fp16 activations).
hipError_t launch_skinny(GemmEpi epi, bool int8_weights, bool bf16, const GemmArgs& a, int cus, hipStream_t st);
constexpr int kSkinnyMaxRows = 16;
constexpr int kSkinnyMaxSplit = 8;  // K splits over workgroups at most
// Workspace of the split skinny launches for products of up to n_max columns.
inline size_t skinny_part_bytes(int n_max) { return (size_t)((n_max + 15) / 16) * kSkinnyMaxSplit * 64 * 16; }
inline size_t skinny_cnt_bytes(int n_max) { return (size_t)((n_max + 15) / 16) * 4; }

}  // namespace ds
