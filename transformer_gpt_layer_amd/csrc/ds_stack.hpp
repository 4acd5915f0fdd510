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
  uint64_t timeout_ticks;  // per grid-barrier wait, in 100 MHz wall-clock ticks
};

constexpr int kStackChunk = 64;    // cache rows per attention work item
constexpr int kStackThreads = 512;  // 8 wave64 per workgroup, one workgroup per CU
constexpr int kStackWaves = kStackThreads / 64;

// Dynamic LDS bytes of one workgroup and the workgroup count the device can keep co-resident.
size_t stack_lds_bytes(Dt wdt, int B, int H, int F, int rows_per_wg);
hipError_t stack_max_groups(Dt wdt, Dt adt, int B, size_t lds, int* groups);
hipError_t launch_stack_decode(Dt wdt, Dt adt, const StackArgs& a, size_t lds, hipStream_t st);
// The largest per-workgroup row tile among the four projections for a grid of G workgroups.
int stack_rows_per_wg(int H, int F, int G);
// LDS the attention merge stages (it reuses the start of the dynamic LDS).
size_t stack_merge_bytes(int nchunk, int head_dim);

}  // namespace ds
