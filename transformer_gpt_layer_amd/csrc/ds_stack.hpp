// ds_stack.hpp -- internal interface of the persistent multi-layer decode kernel.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ds_launch.hpp"

namespace ds {

// One layer as the persistent kernel sees it: weights (borrowed) and its bound KV cache.
struct StackLayer {
  const void *ln1_g, *ln1_b, *w_qkv, *b_qkv, *s_qkv, *w_o, *b_o, *s_o;
  const void *ln2_g, *ln2_b, *w_ff1, *b_ff1, *s_ff1, *w_ff2, *b_ff2, *s_ff2;
  void* k;
  void* v;
  int32_t* d_len;
};

// sync[] layout in 32-bit words (library-owned, zero at rest). Barrier arrivals spread over
// kSyncGroups counters, each on its own 256-byte line; the last arrival of a group bumps the top
// counter, the last top arrival publishes the barrier's epoch in the release flag.
constexpr int kSyncGroups = 16;
constexpr int kSyncLine = 64;
enum {
  kSyncSub = 0,
  kSyncTop = kSyncGroups * kSyncLine,
  kSyncFlag = kSyncTop + kSyncLine,
  kSyncExit = kSyncFlag + kSyncLine,
  kSyncError = kSyncExit + kSyncLine,
  kSyncAttn = kSyncError + kSyncLine,  // then B*nh attention-merge counters
};

// Workgroup shape: kStackSyncWaves waves stage activations, reduce, run the epilogues, attention
// and the grid barriers; kStackWorkers waves stream the weights and compute the row dot products.
constexpr int kStackSyncWaves = 4;
constexpr int kStackWorkers = 12;
constexpr int kStackWaves = kStackSyncWaves + kStackWorkers;
constexpr int kStackThreads = 64 * kStackWaves;  // one workgroup per CU
constexpr int kStackChunk = 64;                  // cache rows per attention work item
constexpr int kStackLdsMax = 160 * 1024;

// Dynamic LDS layout of one workgroup (byte offsets; the activation rows start at 0). Identical on
// the host and the device.
struct StackLds {
  uint32_t raw;     // LayerNorm input rows (fp32), then gamma and beta, inside the activation region
  uint32_t slots;   // per-(row, worker, batch row) partial sums
  uint32_t scales;  // int8 scales of the current row tile
  uint32_t wtab;    // the four weight-matrix pointers of every layer (8 bytes each)
  uint32_t total;
};

__host__ __device__ inline uint32_t stack_align(uint32_t v) { return (v + 255u) & ~255u; }

// wsize: weight element bytes (4, 2, 1); bm: batch rows of the kernel variant (1 or 4). The
// activation region also holds the attention scratch (per-wave partials, then the chunk partials
// of the merge), which is never live at the same time as staged activations.
__host__ __device__ inline StackLds stack_lds_layout(int wsize, int bm, int H, int F, int rows_per_wg, int nchunk,
                                                     int D, int group, int n_layers) {
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
  const uint32_t sc = wsize == 1 ? (uint32_t)rows_per_wg * (kmax / (uint32_t)group) * 2u : 0u;
  L.wtab = stack_align(L.scales + sc);
  L.total = stack_align(L.wtab + (uint32_t)n_layers * 4u * 8u);
  return L;
}

struct StackArgs {
  const StackLayer* layers;
  int n_layers;
  const void* x;   // [B][H] stack input (activation type)
  void* y;         // [B][H] stack output
  int B, H, nh, d, F, cap, group;
  float eps;
  int gelu_tanh;
  // workspace
  float* q;        // [B][H]
  float* part;     // [B][nh][nchunk][d + 2]
  void* ctx;       // [B][H] activation type
  float* x2;       // [B][H]
  void* f;         // [B][F] activation type
  void* ybuf0;     // [B][H] activation type, layer outputs alternate between the two
  void* ybuf1;
  uint32_t* sync;  // kSync* words, then B*nh attention counters
  int G;           // workgroups (all co-resident)
  int nchunk;      // attention chunks of kStackChunk rows over the capacity
  StackLds lds;
  uint64_t timeout_ticks;  // per wait, in 100 MHz wall-clock ticks
};

// The largest per-workgroup row tile among the four projections for a grid of G workgroups.
int stack_rows_per_wg(int H, int F, int G);
hipError_t stack_max_groups(Dt wdt, Dt adt, int B, size_t lds, int* groups);
hipError_t launch_stack_decode(Dt wdt, Dt adt, const StackArgs& a, hipStream_t st);

}  // namespace ds
