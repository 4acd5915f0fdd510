// ds_stack.hpp -- internal interface of the persistent multi-layer decode kernel.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ds_launch.hpp"

namespace ds {

// The LM head at the end of a stack: final LayerNorm parameters and the [V][H] weight (borrowed).
struct StackHead {
  const void *ln_g, *ln_b, *w, *s;
  int V;
};

// One layer as the persistent kernel sees it: weights (borrowed) and its bound KV cache.
struct StackLayer {
  const void *ln1_g, *ln1_b, *w_qkv, *b_qkv, *s_qkv, *w_o, *b_o, *s_o;
  const void *ln2_g, *ln2_b, *w_ff1, *b_ff1, *s_ff1, *w_ff2, *b_ff2, *s_ff2;
  void* k;
  void* v;
  int32_t* d_len;
  void* ks;  // an int8 cache: fp16 row scales of K and V [batch][heads][cap]; null otherwise
  void* vs;
};

// sync[] layout in 32-bit words, at the start of the caller-owned state buffer. Workgroups never
// wait for each other at a barrier: every value that crosses workgroups is stored together with a
// tag naming the launch, the layer and the phase that produced it, and a consumer polls until the
// tags it needs are current. kSyncLaunch holds the launch counter (seeded per stack, advanced by the
// last workgroup out, kLaunchBits wide); kSyncExit counts finished workgroups; kSyncError is raised
// by any wait that timed out, and a launch that finds it raised leaves before any store.
// kSyncArgmax holds the greedy-decoding keys of the LM head: two slots (launch parity) of
// kStackMaxBatch 64-bit keys; a launch takes the slot of its counter's parity and clears the other
// for the next launch.
constexpr int kSyncLine = 64;
constexpr int kStackMaxBatch = 4;
enum {
  kSyncLaunch = 0,
  kSyncExit = kSyncLine,
  kSyncError = 2 * kSyncLine,
  kSyncArgmax = 3 * kSyncLine,
  kSyncWords = 4 * kSyncLine,
};
constexpr uint32_t kSyncBytes = kSyncWords * 4;  // the layer table follows (256-byte aligned)
constexpr int kLaunchBits = 19;
constexpr uint32_t kLaunchMask = (1u << kLaunchBits) - 1u;
constexpr int kStackMaxLayers = 511;  // layer * 8 + phase fits the tag's 12 low bits

// Tag of values produced in layer l (< 512) by phase ph (< 8) of launch `launch`. The top bit is
// always set, so zero-filled memory never holds a current tag; within any 2^19 consecutive launches
// of one stack no two tags are equal (the host clears the workspace before the counter comes round).
__host__ __device__ inline uint32_t stack_tag(uint32_t launch, int l, int ph) {
  return 0x80000000u | ((launch & kLaunchMask) << 12) | (uint32_t)(l * 8 + ph);
}
enum { TAG_Q = 0, TAG_PART = 1, TAG_CTX = 2, TAG_X2 = 3, TAG_F = 4, TAG_Y = 5 };

// Workgroup shape: kStackSyncWaves waves stage activations, reduce, run the epilogues and attention
// and exchange tagged values; kStackWorkers waves stream the weights and compute the row dot products.
constexpr int kStackSyncWaves = 4;
constexpr int kStackWorkers = 8;
constexpr int kStackWaves = kStackSyncWaves + kStackWorkers;
constexpr int kStackThreads = 64 * kStackWaves;  // one workgroup per CU
constexpr int kStackChunk = 64;                  // cache rows per attention work item
constexpr int kStackLdsMax = 160 * 1024;

// Rows of an N-row projection per workgroup tile. FF1's tiles hold an even number of rows, so
// that the fp16 stacks can exchange its outputs as packed pairs (both rows of a pair are produced
// by one workgroup).
__host__ __device__ inline int stack_tile_rows(int N, int G, bool even) {
  const int r = (N + G - 1) / G;
  return even ? (r + 1) & ~1 : r;
}

// int8 group scales (fp16) the workgroup stages for its largest phase: its row tile of each
// projection (and of the LM head's V rows) times the scales per row of that matrix.
__host__ __device__ inline uint32_t stack_scale_halves(int H, int F, int V, int G, int group, int group_mlp) {
  const uint32_t q = (uint32_t)stack_tile_rows(3 * H, G, false) * (uint32_t)(H / group);
  const uint32_t o = (uint32_t)stack_tile_rows(H, G, false) * (uint32_t)(H / group);
  const uint32_t f1 = (uint32_t)stack_tile_rows(F, G, true) * (uint32_t)(H / group_mlp);
  const uint32_t f2 = (uint32_t)stack_tile_rows(H, G, false) * (uint32_t)(F / group_mlp);
  const uint32_t hd = V > 0 ? (uint32_t)stack_tile_rows(V, G, false) * (uint32_t)(H / group) : 0u;
  uint32_t m = q > o ? q : o;
  m = m > f1 ? m : f1;
  m = m > f2 ? m : f2;
  return m > hd ? m : hd;
}

// Dynamic LDS layout of one workgroup (byte offsets; the activation rows start at 0). Identical on
// the host and the device.
struct StackLds {
  uint32_t raw;     // LayerNorm input rows (fp32), then gamma and beta, inside the activation region
  uint32_t slots;   // per-(row, worker, batch row) partial sums
  uint32_t scales;  // int8 scales of the current row tile
  uint32_t wtab;    // the four weight-matrix pointers of every layer (8 bytes each)
  uint32_t layers;  // a copy of every layer's StackLayer (the sync waves' parameters)
  uint32_t lens;    // every layer's cache lengths at launch, 4 per layer (constant during the launch)
  uint32_t res;     // this workgroup's rows of x2, then of the layer output (fp32, res_n each)
  uint32_t res_n;
  uint32_t lnp;     // LayerNorm gamma and beta, prefetched: LN1 (or the LM head's) area, then LN2's
  uint32_t total;
};

__host__ __device__ inline uint32_t stack_align(uint32_t v) { return (v + 255u) & ~255u; }

// wsize: weight element bytes (4, 2, 1); bm: batch rows of the kernel variant (1 or 4); group: the
// smallest int8 scale group of the stack's matrices (sizes the staged scales). The
// activation region also holds the attention scratch (per-wave partials, then the chunk partials
// of the merge), which is never live at the same time as staged activations.
__host__ __device__ inline StackLds stack_lds_layout(int wsize, int bm, int H, int F, int rows_per_wg, int nchunk,
                                                     int D, uint32_t scale_halves, int n_layers) {
  // the weight table holds 4 entries per layer and one for the LM head
  StackLds L{};
  const uint32_t lt = wsize == 4 ? 4u : 2u;
  const uint32_t kmax = (uint32_t)(H > F ? H : F);
  uint32_t region = (uint32_t)bm * kmax * lt;
  const uint32_t ln = (uint32_t)bm * (uint32_t)H * (lt + 4u) + 2u * (uint32_t)H * lt;  // rows, fp32 copy, gamma/beta
  const uint32_t attn = (uint32_t)kStackSyncWaves * D * 4u + (uint32_t)nchunk * (D + 2) * 4u;
  if (ln > region) region = ln;
  if (attn > region) region = attn;
  L.raw = (uint32_t)bm * (uint32_t)H * lt;
  L.slots = stack_align(region);
  L.scales = stack_align(L.slots + (uint32_t)rows_per_wg * kStackWorkers * bm * 4u);
  const uint32_t sc = wsize == 1 ? scale_halves * 2u : 0u;
  L.wtab = stack_align(L.scales + sc);
  L.layers = stack_align(L.wtab + ((uint32_t)n_layers * 4u + 1u) * 8u);
  L.lens = stack_align(L.layers + (uint32_t)n_layers * (uint32_t)sizeof(StackLayer));
  L.res = stack_align(L.lens + (uint32_t)n_layers * 4u * 4u);
  L.res_n = (uint32_t)rows_per_wg * (uint32_t)bm;
  L.lnp = stack_align(L.res + 2u * L.res_n * 4u);
  L.total = stack_align(L.lnp + 2u * 2u * (uint32_t)H * lt);
  return L;
}

// A tagged value: the float's bits and the tag of the phase that stored it (one 8-byte store).
struct StackArgs {
  const StackLayer* layers;
  int n_layers;
  const void* x;   // [B][H] stack input (activation type)
  void* y;         // [B][H] stack output (activation type)
  int B, H, nh, d, F, cap, group, group_mlp;  // int8 scale groups: W_qkv, W_o, LM head; W_ff1, W_ff2
  int kv8;         // the caches hold int8 codes with fp16 row scales (StackLayer ks, vs)
  float eps;
  int gelu_tanh;
  // workspace: tagged values (8 bytes each)
  uint2* q;        // [B][H]
  uint2* knew;     // [B][H] the new K row of every head
  uint2* vnew;     // [B][H]
  uint2* part;     // [B][nh][nchunk][d + 2] attention partials (max, sum, acc[d])
  uint2* ctx;      // [B][H]
  uint2* x2;       // [B][H]
  uint2* f;        // [B][F]
  uint2* ybuf;     // [B][H] layer outputs (the last one only when the LM head runs)
  uint32_t* sync;  // kSync* words
  // the LM head (V == 0: none); head != 0: this launch runs it after the last layer
  int head, V;
  const void *head_g, *head_b, *head_w, *head_s;
  float* logits;    // [B][V] fp32, or null
  int32_t* tokens;  // [B] greedy choices
  int G;           // workgroups (all co-resident)
  int nchunk;      // attention chunks of kStackChunk rows over the capacity
  StackLds lds;
  uint64_t timeout_ticks;  // per wait, in 100 MHz wall-clock ticks
};

// The largest per-workgroup row tile among the four projections (and the LM head's V rows) for a
// grid of G workgroups.
int stack_rows_per_wg(int H, int F, int V, int G);
// Slices per worker group of the persistent kernel for these widths (1 or 5).
int stack_group_slices(Dt wdt, int H, int F);
hipError_t stack_max_groups(Dt wdt, Dt adt, bool kv8, int B, int GS, size_t lds, int* groups);
hipError_t launch_stack_decode(Dt wdt, Dt adt, const StackArgs& a, hipStream_t st);

}  // namespace ds
