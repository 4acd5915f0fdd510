// kernels_stack.hip -- persistent decode of a whole layer stack in one launch.
//
// Computes, for every layer in turn, the four fusion regions of one transformer layer described on
// the page "DeepSpeed Inference 内核优化深度解析" (blog.gitcode.com), section 三 3.2 (LN + QKV GeMM +
// bias; attention over the cache with the head transform folded into its addressing; the output
// GeMM with bias and residual; LN + FF1 + bias + GELU; FF2 + bias + residual). Section 三 3.1 puts the
// fusion boundaries where partial results must meet (the all-reduce points); here those are the
// grid-wide barriers between phases.
//
// gfx950 design. One cooperative launch keeps one 8-wave workgroup per CU resident for the whole
// step. Each projection is cut into per-workgroup row tiles; a tile is one contiguous range of the
// row-major matrix, cut into 1 KB "slices" (one 16-byte load per lane of a wave64), and each wave
// owns a contiguous block of slices, so every phase is balanced whatever its shape. As soon as a
// workgroup has stored a phase's results it issues the weight loads of its next tile into
// registers: weights do not depend on activations, so HBM keeps streaming through the epilogue,
// the grid barrier and the next phase's staging. The loads complete in issue order, so waiting
// until at most that many are outstanding (s_waitcnt vmcnt(N)) proves the earlier stores done
// without waiting for the prefetch. Activations that cross workgroups are written and read with
// sc1 buffer operations (at the device coherence point, past the per-XCD L2 copies); barrier
// arrivals are agent-scope atomics spread over 16 counters. Every barrier wait is bounded by a
// wall-clock timeout that raises an error flag, after which every workgroup leaves the kernel.
#include "ds_device.hpp"
#include "ds_stack.hpp"

namespace ds {
namespace {

constexpr int NW = kStackWaves;
constexpr int kAuxCoherent = 16;         // sc1
constexpr int kAuxStream = 2;            // nt
constexpr int kRsrcFlags = 0x00020000;   // raw buffer, 32-bit dword format
constexpr uint32_t kOutOfRange = 0x7ffffff0u;  // a buffer offset past every descriptor: loads return 0
// Weight slices (16 B per lane) a wave holds in registers: 25 covers a whole row tile of the
// GPT-Neo-2.7B shapes on 256 workgroups; int8 slices also carry a scale and widen in registers.
template <typename WT> struct MaxSlices { static constexpr int value = 25; };
template <> struct MaxSlices<int8_t> { static constexpr int value = 16; };

typedef __amdgpu_buffer_rsrc_t rsrc_t;

__device__ __forceinline__ rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, kRsrcFlags);
}
__device__ __forceinline__ u32x4 coh_load16(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kAuxCoherent);
}
__device__ __forceinline__ uint32_t coh_load4(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, kAuxCoherent);
}
__device__ __forceinline__ void coh_store4(rsrc_t r, uint32_t off, uint32_t v) {
  __builtin_amdgcn_raw_buffer_store_b32(v, r, off, 0, kAuxCoherent);
}

// coherent scalar access in the activation type
template <typename AT> __device__ __forceinline__ float coh_ld_act(rsrc_t r, uint32_t idx);
template <> __device__ __forceinline__ float coh_ld_act<float>(rsrc_t r, uint32_t idx) {
  return as_f32(coh_load4(r, idx * 4));
}
template <> __device__ __forceinline__ float coh_ld_act<half_t>(rsrc_t r, uint32_t idx) {
  const uint16_t h = __builtin_amdgcn_raw_buffer_load_b16(r, idx * 2, 0, kAuxCoherent);
  return (float)__builtin_bit_cast(half_t, h);
}
template <typename AT> __device__ __forceinline__ void coh_st_act(rsrc_t r, uint32_t idx, float v);
template <> __device__ __forceinline__ void coh_st_act<float>(rsrc_t r, uint32_t idx, float v) {
  coh_store4(r, idx * 4, __builtin_bit_cast(uint32_t, v));
}
template <> __device__ __forceinline__ void coh_st_act<half_t>(rsrc_t r, uint32_t idx, float v) {
  __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(uint16_t, (half_t)v), r, idx * 2, 0, kAuxCoherent);
}

template <typename T> __device__ __forceinline__ float ldp(const void* p, int i) {
  return (float)reinterpret_cast<const T*>(p)[i];
}

// s_waitcnt with only the vector-memory counter limited to N (gfx9 encoding: vmcnt in bits
// [3:0] and [15:14], expcnt [6:4] and lgkmcnt [11:8] left at their maxima).
template <int N> __device__ __forceinline__ void wait_vm_at_most() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
  asm volatile("" ::: "memory");
}

// Workgroup barrier that waits only for LDS traffic, not for outstanding global loads.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt((15) | (3 << 14) | (7 << 4) | (0 << 8));  // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Block-wide sums of two values at once; `red2` is NW float2 of LDS.
__device__ __forceinline__ float2_t block_sum2(float2_t v, float2_t* red2, int tid) {
  v.x = wave_sum(v.x);
  v.y = wave_sum(v.y);
  lds_barrier();
  if ((tid & 63) == 0) red2[tid >> 6] = v;
  lds_barrier();
  float2_t s = {0.f, 0.f};
#pragma unroll
  for (int w = 0; w < NW; ++w) s += red2[w];
  return s;
}

// ------------------------------------------------------------------ grid barrier
// Arrive at barrier `epoch` (1, 2, ...): one atomic add per workgroup on its group's counter; the
// last of a group adds to the top counter; the last top arrival publishes the epoch. The caller
// has made its own stores complete (vmcnt) before this.
__device__ __forceinline__ void grid_arrive(uint32_t* sync, uint32_t epoch, int g, int G, int tid) {
  lds_barrier();
  if (tid == 0) {
    const int ng = G < kSyncGroups ? G : kSyncGroups;
    const int gi = g % ng;
    const uint32_t members = (uint32_t)((G - gi + ng - 1) / ng);
    const uint32_t old = __hip_atomic_fetch_add(sync + kSyncSub + gi * kSyncLine, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (old == epoch * members - 1u) {
      const uint32_t top = __hip_atomic_fetch_add(sync + kSyncTop, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (top == epoch * (uint32_t)ng - 1u) __hip_atomic_store(sync + kSyncFlag, epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// Wait until barrier `epoch` is released; false (for the whole workgroup) on timeout or a raised
// error flag.
__device__ __forceinline__ bool grid_wait(uint32_t* sync, uint32_t epoch, uint64_t timeout, int* s_flag, int tid) {
  if (tid == 0) {
    int ok = 1;
    const uint64_t t0 = wall_clock64();
    while (__hip_atomic_load(sync + kSyncFlag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < epoch) {
      if (__hip_atomic_load(sync + kSyncError, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u ||
          wall_clock64() - t0 > timeout) {
        __hip_atomic_store(sync + kSyncError, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        ok = 0;
        break;
      }
      __builtin_amdgcn_s_sleep(2);
    }
    *s_flag = ok;
  }
  lds_barrier();
  return *s_flag != 0;
}

// ------------------------------------------------------------------ weight tiles
// A tile is rows [r0, r0+nr) of a row-major [N][K] matrix: one contiguous range of nr*K elements,
// cut into slices of 64*E elements. K is a multiple of the slice, so slice s of the tile starts
// at element r0*K + s*64E and lies in tile row s / (K/64E). Wave w owns the contiguous block of
// slices [w*M, min(T, (w+1)*M)), M = ceil(T/NW), and holds up to MaxSlices<WT> of them in
// registers at a time (one "round").
template <typename WT> struct WRegs {
  static constexpr int N = MaxSlices<WT>::value;
  // loads one round issues: the slices, plus their scales for int8
  static constexpr int kLoads = sizeof(WT) == 1 ? 2 * N : N;
  u32x4 w[N];
  float sc[N];
};

struct Block {
  int s0, cnt;
};
__device__ __forceinline__ Block wave_block(int T, int wave) {
  const int M = (T + NW - 1) / NW;
  const int s0 = wave * M;
  const int e = min(T, s0 + M);
  return Block{s0, e > s0 ? e - s0 : 0};
}

// Issue exactly WRegs<WT>::kLoads loads: slices [s, s + n) of the tile (n <= N) into R, and
// out-of-range loads (which return zero and touch no memory) for the rest, so that the number of
// loads in flight after this call is known at compile time. Buffer loads keep one per-lane offset
// register for all of them, and the descriptor's size bounds every access to the matrix.
template <typename WT>
__device__ __forceinline__ void issue_slices(WRegs<WT>& R, const WT* __restrict__ W, const half_t* __restrict__ S,
                                             int N, int K, int group, int r0, int s, int n, int lane) {
  constexpr int E = WTraits<WT>::E, SL = kWave * E;
  const rsrc_t rw = make_rsrc(W, (uint32_t)((size_t)N * K * sizeof(WT)));
  const uint32_t first = (uint32_t)((size_t)r0 * K + (size_t)s * SL);  // element index of slice s
  const uint32_t voff = (uint32_t)(lane * E * sizeof(WT));
  // int8 scales (unused otherwise): fp16 [N][K/group], the lane's group at (lane*E/group)
  const rsrc_t rs = make_rsrc(S, sizeof(WT) == 1 ? (uint32_t)((size_t)N * (K / group) * 2) : 0u);
  const uint32_t svoff = sizeof(WT) == 1 ? (uint32_t)((lane * E / group) * 2) : 0u;
#pragma unroll
  for (int i = 0; i < WRegs<WT>::N; ++i) {
    const uint32_t e0 = first + (uint32_t)(i * SL);
    const bool in = i < n;
    R.w[i] = __builtin_amdgcn_raw_buffer_load_b128(rw, voff, in ? e0 * (uint32_t)sizeof(WT) : kOutOfRange, kAuxStream);
    if constexpr (sizeof(WT) == 1) {
      const uint16_t h = __builtin_amdgcn_raw_buffer_load_b16(rs, svoff, in ? (e0 / group) * 2 : kOutOfRange, 0);
      R.sc[i] = (float)__builtin_bit_cast(half_t, h);
    }
  }
}

// Round 0 of this wave's block. Always issues WRegs<WT>::kLoads loads (an empty tile gets only
// out-of-range ones).
template <typename WT>
__device__ __forceinline__ void prefetch_tile(WRegs<WT>& R, const WT* W, const half_t* S, int N, int K, int group,
                                              int r0, int nr, int wave, int lane) {
  constexpr int SL = kWave * WTraits<WT>::E;
  const Block bl = wave_block(nr > 0 ? nr * (K / SL) : 0, wave);
  issue_slices<WT>(R, W, S, N, K, group, r0, bl.s0, min(bl.cnt, WRegs<WT>::N), lane);
}

template <int BM>
__device__ __forceinline__ void flush_rows(float (&acc)[BM], float* slots, int rl, int wave, int lane) {
#pragma unroll
  for (int b = 0; b < BM; ++b) {
    const float v = wave_sum(acc[b]);
    if (lane == 0) slots[(rl * NW + wave) * BM + b] = v;
    acc[b] = 0.f;
  }
}

// Row sums of the tile into slots[row][wave][b] (round 0 must already be in R; later rounds are
// loaded here). act holds BM staged rows of K elements.
template <typename WT, int BM>
__device__ __forceinline__ void gemv_tile(WRegs<WT>& R, const WT* __restrict__ W, const half_t* __restrict__ S,
                                          int N, int K, int group, int r0, int nr,
                                          const typename WTraits<WT>::LT* act, float* slots, int wave, int lane) {
  typedef typename WTraits<WT>::LT LT;
  constexpr int E = WTraits<WT>::E, SL = kWave * E;
  const int Sper = K / SL;
  const Block bl = wave_block(nr * Sper, wave);
  if (bl.cnt <= 0) return;
  float acc[BM];
#pragma unroll
  for (int b = 0; b < BM; ++b) acc[b] = 0.f;
  int rl = bl.s0 / Sper, ks = bl.s0 - rl * Sper;
  constexpr int NS = WRegs<WT>::N;
  for (int done = 0; done < bl.cnt; done += NS) {
    const int n = min(NS, bl.cnt - done);
    if (done > 0) issue_slices<WT>(R, W, S, N, K, group, r0, bl.s0 + done, n, lane);
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      if (i < n) {
        const LT* ap = act + ks * SL + lane * E;
#pragma unroll
        for (int b = 0; b < BM; ++b) {
          if constexpr (sizeof(WT) == 4) {
            acc[b] = dot4_f32(R.w[i], *reinterpret_cast<const float4_t*>(ap + b * K), acc[b]);
          } else if constexpr (sizeof(WT) == 2) {
            acc[b] = dot8_f16(R.w[i], *reinterpret_cast<const u32x4*>(ap + b * K), acc[b]);
          } else {
            acc[b] = fmaf(dot16_i8(R.w[i], *reinterpret_cast<const u32x4*>(ap + b * K),
                                   *reinterpret_cast<const u32x4*>(ap + b * K + 8)),
                          R.sc[i], acc[b]);
          }
        }
        if (++ks == Sper) {
          flush_rows<BM>(acc, slots, rl, wave, lane);
          ks = 0;
          ++rl;
        }
      }
    }
  }
  if (ks != 0) flush_rows<BM>(acc, slots, rl, wave, lane);
}

// ------------------------------------------------------------------ activation staging
constexpr int kStageUnroll = 4;  // 16-byte loads a thread has in flight while staging

// Copy B rows of K elements of type IT (written by other workgroups: coherent loads) into LDS as
// LT, zero-filling rows B..BM-1.
template <typename IT, typename LT, int BM>
__device__ __forceinline__ void stage_plain(const void* in, int B, int K, LT* act, int tid) {
  constexpr int V = 16 / (int)sizeof(IT);
  const rsrc_t r = make_rsrc(in, (uint32_t)(B * K * sizeof(IT)));
  const int nvec = BM * K / V;
  for (int j0 = tid; j0 < nvec; j0 += kStackThreads * kStageUnroll) {
    u32x4 raw[kStageUnroll];
#pragma unroll
    for (int u = 0; u < kStageUnroll; ++u) {
      const int j = j0 + u * kStackThreads;
      const uint32_t off = (uint32_t)(j * V * sizeof(IT));
      raw[u] = coh_load16(r, j < nvec ? off : kOutOfRange);  // rows past B are out of range: zero
    }
#pragma unroll
    for (int u = 0; u < kStageUnroll; ++u) {
      const int j = j0 + u * kStackThreads;
      if (j >= nvec) break;
      if constexpr (sizeof(IT) == sizeof(LT)) {
        *reinterpret_cast<u32x4*>(act + j * V) = raw[u];
      } else {  // float input to half LDS
        act[j * V + 0] = (LT)as_f32(raw[u].x);
        act[j * V + 1] = (LT)as_f32(raw[u].y);
        act[j * V + 2] = (LT)as_f32(raw[u].z);
        act[j * V + 3] = (LT)as_f32(raw[u].w);
      }
    }
  }
}

// LayerNorm B rows (biased variance, two passes) into LDS as LT. The raw rows are first copied
// to `raw` (BM*K floats of LDS) so that both passes read LDS, not global memory.
template <typename IT, typename LT, typename AT, int BM>
__device__ __forceinline__ void stage_ln(const void* in, int B, int K, const AT* __restrict__ g,
                                         const AT* __restrict__ beta, float eps, LT* act, float* raw, float2_t* red2,
                                         int tid) {
  constexpr int V = 16 / (int)sizeof(IT);
  const rsrc_t r = make_rsrc(in, (uint32_t)(B * K * sizeof(IT)));
  const int nvec = B * K / V;
  for (int j0 = tid; j0 < nvec; j0 += kStackThreads * kStageUnroll) {
    u32x4 v[kStageUnroll];
#pragma unroll
    for (int u = 0; u < kStageUnroll; ++u) {
      const int j = j0 + u * kStackThreads;
      v[u] = coh_load16(r, j < nvec ? (uint32_t)(j * 16) : kOutOfRange);
    }
#pragma unroll
    for (int u = 0; u < kStageUnroll; ++u) {
      const int j = j0 + u * kStackThreads;
      if (j >= nvec) break;
      if constexpr (sizeof(IT) == 4) {
        *reinterpret_cast<u32x4*>(raw + j * V) = v[u];
      } else {
        const uint32_t ww[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          const half2_t p = as_half2(ww[h]);
          raw[j * V + 2 * h] = (float)p.x;
          raw[j * V + 2 * h + 1] = (float)p.y;
        }
      }
    }
  }
  lds_barrier();
#pragma unroll
  for (int b = 0; b < BM; ++b) {
    if (b >= B) {
      for (int k = tid; k < K; k += kStackThreads) act[b * K + k] = (LT)0.f;
      continue;
    }
    // one block reduction of the sums of d = x - x[0] and d^2: var = (sum d^2 - (sum d)^2 / K) / K;
    // shifting by an element of the row keeps the subtraction well conditioned
    const float* xr = raw + b * K;
    const float c0 = xr[0];
    float s1 = 0.f, s2 = 0.f;
    for (int k = tid; k < K; k += kStackThreads) {
      const float d = xr[k] - c0;
      s1 += d;
      s2 += d * d;
    }
    float2_t tot = block_sum2(float2_t{s1, s2}, red2, tid);
    const float dm = tot.x / K;
    const float mean = c0 + dm;
    const float var = fmaxf(tot.y / K - dm * dm, 0.f);
    const float rstd = rsqrtf(var + eps);
    for (int k = tid; k < K; k += kStackThreads)
      act[b * K + k] = (LT)((xr[k] - mean) * rstd * (float)g[k] + (float)beta[k]);
  }
}

// ------------------------------------------------------------------ attention work items
// An item is (sequence b, head j, chunk c of kStackChunk cache rows). Lanes split a row into
// 16-byte pieces (LPK lanes per row), a wave covers KPI rows per load, NW waves cover NW*KPI.
template <typename AT, int D> struct AttnShape {
  static constexpr int EK = 16 / (int)sizeof(AT);
  static constexpr int LPK = D / EK;
  static constexpr int KPI = kWave / LPK;
  static constexpr int NIT = (kStackChunk + NW * KPI - 1) / (NW * KPI);
};

template <typename AT, int D> struct AttnRegs {
  u32x4 k[AttnShape<AT, D>::NIT], v[AttnShape<AT, D>::NIT];
  static constexpr int kLoads = 2 * AttnShape<AT, D>::NIT;
};

__device__ __forceinline__ void item_coords(const StackArgs& a, int item, int& b, int& j, int& c) {
  c = item % a.nchunk;
  j = (item / a.nchunk) % a.nh;
  b = item / (a.nchunk * a.nh);
}

// Issue exactly AttnRegs::kLoads loads: the item's past rows (before the new one, written by
// earlier launches); rows outside the item or not yet filled load as zero (out of range).
template <typename AT, int D>
__device__ __forceinline__ void attn_prefetch(AttnRegs<AT, D>& A, const StackLayer& L, const StackArgs& a, int item,
                                              int tid) {
  typedef AttnShape<AT, D> S;
  const int nitems = a.B * a.nh * a.nchunk;
  int b = 0, j = 0, c = 0;
  if (item < nitems) item_coords(a, item, b, j, c);
  const int len = item < nitems ? L.d_len[b] : 0;
  const int wave = tid >> 6, lane = tid & 63;
  const uint32_t bytes = (uint32_t)((size_t)a.B * a.nh * a.cap * D * sizeof(AT));
  const rsrc_t rk = make_rsrc(L.k, bytes), rv = make_rsrc(L.v, bytes);
  const size_t head = (((size_t)b * a.nh + j) * a.cap) * D;
  const int e0 = (lane % S::LPK) * S::EK;
#pragma unroll
  for (int it = 0; it < S::NIT; ++it) {
    const int key = c * kStackChunk + (it * NW + wave) * S::KPI + lane / S::LPK;
    const bool past = item < nitems && key < len && key < a.cap && key < (c + 1) * kStackChunk;
    const uint32_t off = past ? (uint32_t)((head + (size_t)key * D + e0) * sizeof(AT)) : kOutOfRange;
    A.k[it] = __builtin_amdgcn_raw_buffer_load_b128(rk, off, 0, 0);
    A.v[it] = __builtin_amdgcn_raw_buffer_load_b128(rv, off, 0, 0);
  }
}

// One item: scores of q against the chunk's rows, wave-reduced max and sum, the exp-weighted V
// sum; the partial (max, sum, acc[D]) goes to the workspace, and the workgroup that completes the
// last chunk of a (sequence, head) merges the partials into ctx (log-sum-exp).
template <typename AT, int D>
__device__ __forceinline__ void attn_item(AttnRegs<AT, D>& A, const StackLayer& L, const StackArgs& a, int item,
                                          bool prefetched, float* s_m, float* s_l, float* s_acc, float* s_part,
                                          int* s_flag, int tid) {
  typedef AttnShape<AT, D> S;
  constexpr int EK = S::EK, LPK = S::LPK, KPI = S::KPI, NIT = S::NIT;
  const float kNeg = -1e30f;
  int b, j, c;
  item_coords(a, item, b, j, c);
  const int len = L.d_len[b];
  int nkeys = len + 1;
  if (nkeys > a.cap) nkeys = a.cap;
  const int nvalid = (nkeys + kStackChunk - 1) / kStackChunk;
  if (c >= nvalid) return;
  const int wave = tid >> 6, lane = tid & 63;
  const int H = a.nh * D;
  const size_t head = (((size_t)b * a.nh + j) * a.cap) * D;
  const uint32_t bytes = (uint32_t)((size_t)a.B * a.nh * a.cap * D * sizeof(AT));
  const rsrc_t rk = make_rsrc(L.k, bytes), rv = make_rsrc(L.v, bytes);
  const int e0 = (lane % LPK) * EK;

  if (!prefetched) attn_prefetch<AT, D>(A, L, a, item, tid);
  // the new row (position len) was written by the QKV phase of this launch: coherent loads
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    const int key = c * kStackChunk + (it * NW + wave) * KPI + lane / LPK;
    if (key == len && key < a.cap) {
      const uint32_t off = (uint32_t)((head + (size_t)key * D + e0) * sizeof(AT));
      A.k[it] = coh_load16(rk, off);
      A.v[it] = coh_load16(rv, off);
    }
  }
  const rsrc_t rq = make_rsrc(a.q, (uint32_t)(a.B * H * 4));
  const float qs = 1.4426950408889634f / sqrtf((float)D);  // log2(e)/sqrt(d): scores feed exp2
  float qv[EK];
#pragma unroll
  for (int e = 0; e < EK; ++e) qv[e] = as_f32(coh_load4(rq, (uint32_t)((b * H + j * D + e0 + e) * 4))) * qs;

  float sc[NIT];
  bool valid[NIT];
  float m = kNeg;
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    const int key = c * kStackChunk + (it * NW + wave) * KPI + lane / LPK;
    valid[it] = key < nkeys && key < (c + 1) * kStackChunk;
    float p = 0.f;
    if constexpr (sizeof(AT) == 4) {
      p = qv[0] * as_f32(A.k[it].x) + qv[1] * as_f32(A.k[it].y) + qv[2] * as_f32(A.k[it].z) + qv[3] * as_f32(A.k[it].w);
    } else {
      const uint32_t wv[4] = {A.k[it].x, A.k[it].y, A.k[it].z, A.k[it].w};
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        const half2_t kk = as_half2(wv[h]);
        p += qv[2 * h] * (float)kk.x + qv[2 * h + 1] * (float)kk.y;
      }
    }
    p = group_sum<LPK>(p);
    sc[it] = valid[it] ? p : kNeg;
    m = fmaxf(m, sc[it]);
  }
  m = wave_max(m);
  float l = 0.f, acc[EK];
#pragma unroll
  for (int e = 0; e < EK; ++e) acc[e] = 0.f;
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    const float p = valid[it] ? exp2f(sc[it] - m) : 0.f;
    l += p;
    if constexpr (sizeof(AT) == 4) {
      acc[0] += p * as_f32(A.v[it].x);
      acc[1] += p * as_f32(A.v[it].y);
      acc[2] += p * as_f32(A.v[it].z);
      acc[3] += p * as_f32(A.v[it].w);
    } else {
      const uint32_t wv[4] = {A.v[it].x, A.v[it].y, A.v[it].z, A.v[it].w};
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        const half2_t vv = as_half2(wv[h]);
        acc[2 * h] += p * (float)vv.x;
        acc[2 * h + 1] += p * (float)vv.y;
      }
    }
  }
#pragma unroll
  for (int off = LPK; off < kWave; off <<= 1) {
    l += __shfl_xor(l, off, kWave);
#pragma unroll
    for (int e = 0; e < EK; ++e) acc[e] += __shfl_xor(acc[e], off, kWave);
  }
  lds_barrier();  // LDS scratch of a previous item is free
  if (lane < LPK) {
#pragma unroll
    for (int e = 0; e < EK; ++e) s_acc[wave * D + e0 + e] = acc[e];
    if (lane == 0) {
      s_m[wave] = m;
      s_l[wave] = l;
    }
  }
  lds_barrier();
  float M = kNeg;
#pragma unroll
  for (int w = 0; w < NW; ++w) M = fmaxf(M, s_m[w]);
  float f[NW];
#pragma unroll
  for (int w = 0; w < NW; ++w) f[w] = s_l[w] > 0.f ? exp2f(s_m[w] - M) : 0.f;
  const size_t pbase = ((size_t)b * a.nh + j) * a.nchunk;
  const rsrc_t rp = make_rsrc(a.part, (uint32_t)((size_t)a.B * a.nh * a.nchunk * (D + 2) * 4));
  if (tid < D) {
    float v = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) v += f[w] * s_acc[w * D + tid];
    coh_store4(rp, (uint32_t)(((pbase + c) * (D + 2) + 2 + tid) * 4), __builtin_bit_cast(uint32_t, v));
  }
  if (tid == 0) {
    float Ls = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) Ls += f[w] * s_l[w];
    coh_store4(rp, (uint32_t)(((pbase + c) * (D + 2)) * 4), __builtin_bit_cast(uint32_t, M));
    coh_store4(rp, (uint32_t)(((pbase + c) * (D + 2) + 1) * 4), __builtin_bit_cast(uint32_t, Ls));
  }
  wait_vm_at_most<0>();
  lds_barrier();
  uint32_t* cnt = a.sync + kSyncAttn + b * a.nh + j;
  if (tid == 0)
    *s_flag = __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == (uint32_t)(nvalid - 1);
  lds_barrier();
  if (!*s_flag) return;
  // last chunk of this (sequence, head): all partials in one parallel load, then the merge
  const int nw = nvalid * (D + 2);
  for (int i = tid; i < nw; i += kStackThreads) s_part[i] = as_f32(coh_load4(rp, (uint32_t)((pbase * (D + 2) + i) * 4)));
  lds_barrier();
  if (tid < D) {
    float MM = kNeg;
    for (int cc = 0; cc < nvalid; ++cc) MM = fmaxf(MM, s_part[cc * (D + 2)]);
    float Lsum = 0.f, Acc = 0.f;
    for (int cc = 0; cc < nvalid; ++cc) {
      const float* pc = s_part + cc * (D + 2);
      const float w = pc[1] > 0.f ? exp2f(pc[0] - MM) : 0.f;
      Lsum += w * pc[1];
      Acc += w * pc[2 + tid];
    }
    const rsrc_t rc = make_rsrc(a.ctx, (uint32_t)(a.B * H * sizeof(AT)));
    coh_st_act<AT>(rc, (uint32_t)(b * H + j * D + tid), Acc / Lsum);
  }
  if (tid == 0) __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace

// ------------------------------------------------------------------ the persistent kernel
template <typename WT, typename AT, int BM, int D>
__global__ __launch_bounds__(kStackThreads, 1) void stack_decode_kernel(const StackArgs a) {
  typedef typename WTraits<WT>::LT LT;
  constexpr int kWLoads = WRegs<WT>::kLoads;
  constexpr int kALoads = AttnRegs<AT, D>::kLoads;
  extern __shared__ __align__(16) unsigned char smem[];
  __shared__ float2_t red2[NW];
  __shared__ float s_m[NW], s_l[NW];
  __shared__ int s_flag;
  const int H = a.H, F = a.F, B = a.B, G = a.G, g = blockIdx.x;
  const int KMAX = H > F ? H : F;
  size_t act_bytes = (size_t)BM * KMAX * sizeof(LT);
  const size_t ln_bytes = (size_t)BM * H * (sizeof(LT) + 4);
  if (ln_bytes > act_bytes) act_bytes = ln_bytes;
  LT* act = reinterpret_cast<LT*>(smem);
  float* raw = reinterpret_cast<float*>(smem + (size_t)BM * H * sizeof(LT));  // LayerNorm input rows
  float* slots = reinterpret_cast<float*>(smem + act_bytes);
  float* s_acc = slots;                                  // attention: NW x D floats
  float* s_part = reinterpret_cast<float*>(smem);        // attention merge: nchunk x (D + 2) floats
  // Thread indices are re-derived through an opaque copy at every phase: otherwise the compiler
  // hoists every per-thread address of every phase out of the layer loop and keeps them all live.
  int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  auto fresh = [&]() {
    int t = threadIdx.x;
    asm volatile("" : "+v"(t));
    tid = t;
    wave = t >> 6;
    lane = t & 63;
  };

  // per-workgroup row tiles of each projection
  const int rq = (3 * H + G - 1) / G, ro = (H + G - 1) / G, r1 = (F + G - 1) / G;
  const int q0 = min(3 * H, g * rq), nq = min(3 * H, q0 + rq) - q0;
  const int o0 = min(H, g * ro), no = min(H, o0 + ro) - o0;
  const int f0 = min(F, g * r1), nf = min(F, f0 + r1) - f0;
  const int y0 = o0, ny = no;
  const int nitems = B * a.nh * a.nchunk;

  WRegs<WT> R;
  AttnRegs<AT, D> A;
  uint32_t epoch = 0;
  auto slot_clear = [&](int nr) {
    for (int i = tid; i < nr * NW * BM; i += kStackThreads) slots[i] = 0.f;
  };
  auto row_sum = [&](int rl, int b) {
    const float* p = slots + rl * NW * BM + b;
    float s = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) s += p[w * BM];
    return s;
  };
  // after a phase's stores and the next prefetch: stores done, then arrive and wait
  auto barrier = [&](auto wait_stores) -> bool {
    wait_stores();
    ++epoch;
    grid_arrive(a.sync, epoch, g, G, tid);
    return grid_wait(a.sync, epoch, a.timeout_ticks, &s_flag, tid);
  };

  {
    const StackLayer& L0 = a.layers[0];
    prefetch_tile<WT>(R, (const WT*)L0.w_qkv, (const half_t*)L0.s_qkv, 3 * H, H, a.group, q0, nq, wave, lane);
  }

  for (int l = 0; l < a.n_layers; ++l) {
    const StackLayer& L = a.layers[l];
    const void* xin = (l == 0) ? a.x : ((l & 1) ? a.ybuf0 : a.ybuf1);
    void* yout = (l == a.n_layers - 1) ? a.y : ((l & 1) ? a.ybuf1 : a.ybuf0);

    // ---- region 1: LN1 + QKV + bias; q -> workspace, k/v -> cache row d_len[b]
    fresh();
    // epilogue inputs first: they travel with the staging loads instead of after the GEMV
    float pb = 0.f, pr = 0.f;
    int plen = 0;
    if (tid < nq * B) {
      const int rl = tid / B, b = tid - rl * B;
      pb = ldp<AT>(L.b_qkv, q0 + rl);
      plen = L.d_len[b];
    }
    slot_clear(nq);
    stage_ln<AT, LT, AT, BM>(xin, B, H, (const AT*)L.ln1_g, (const AT*)L.ln1_b, a.eps, act, raw, red2, tid);
    lds_barrier();
    if (nq > 0) gemv_tile<WT, BM>(R, (const WT*)L.w_qkv, (const half_t*)L.s_qkv, 3 * H, H, a.group, q0, nq, act, slots, wave, lane);
    lds_barrier();
    {
      const rsrc_t rqo = make_rsrc(a.q, (uint32_t)(B * H * 4));
      const uint32_t cache_bytes = (uint32_t)((size_t)B * a.nh * a.cap * D * sizeof(AT));
      const rsrc_t rk = make_rsrc(L.k, cache_bytes), rv = make_rsrc(L.v, cache_bytes);
      for (int t = tid; t < nq * B; t += kStackThreads) {
        const int rl = t / B, b = t - rl * B, n = q0 + rl;
        const float z = row_sum(rl, b) + (t == tid ? pb : ldp<AT>(L.b_qkv, n));
        if (n < H) {
          coh_store4(rqo, (uint32_t)((b * H + n) * 4), __builtin_bit_cast(uint32_t, z));
        } else {
          const int m = n < 2 * H ? n - H : n - 2 * H, j = m / D, e = m - j * D;
          const int pos = t == tid ? plen : L.d_len[b];
          if (pos >= 0 && pos < a.cap) coh_st_act<AT>(n < 2 * H ? rk : rv, (uint32_t)((((size_t)b * a.nh + j) * a.cap + pos) * D + e), z);
        }
      }
    }
    asm volatile("" ::: "memory");
    attn_prefetch<AT, D>(A, L, a, g, tid);
    if (!barrier([] { wait_vm_at_most<kALoads>(); })) return;

    // ---- region 2: attention over the cache, chunk partials merged by the last chunk
    fresh();
    for (int item = g; item < nitems; item += G)
      attn_item<AT, D>(A, L, a, item, item == g, s_m, s_l, s_acc, s_part, &s_flag, tid);
    asm volatile("" ::: "memory");
    prefetch_tile<WT>(R, (const WT*)L.w_o, (const half_t*)L.s_o, H, H, a.group, o0, no, wave, lane);
    if (!barrier([] { wait_vm_at_most<kWLoads>(); })) return;

    // ---- output projection + bias + residual: x2 = x + Wo ctx + bo
    fresh();
    {
      const rsrc_t rx = make_rsrc(xin, (uint32_t)(B * H * sizeof(AT)));
      if (tid < no * B) {
        const int rl = tid / B, b = tid - rl * B;
        pb = ldp<AT>(L.b_o, o0 + rl);
        pr = coh_ld_act<AT>(rx, (uint32_t)(b * H + o0 + rl));
      }
    }
    slot_clear(no);
    stage_plain<AT, LT, BM>(a.ctx, B, H, act, tid);
    lds_barrier();
    if (no > 0) gemv_tile<WT, BM>(R, (const WT*)L.w_o, (const half_t*)L.s_o, H, H, a.group, o0, no, act, slots, wave, lane);
    lds_barrier();
    {
      const rsrc_t rx = make_rsrc(xin, (uint32_t)(B * H * sizeof(AT)));
      const rsrc_t rx2 = make_rsrc(a.x2, (uint32_t)(B * H * 4));
      for (int t = tid; t < no * B; t += kStackThreads) {
        const int rl = t / B, b = t - rl * B, n = o0 + rl;
        const float z = row_sum(rl, b) + (t == tid ? pb : ldp<AT>(L.b_o, n));
        const float xr = t == tid ? pr : coh_ld_act<AT>(rx, (uint32_t)(b * H + n));
        coh_store4(rx2, (uint32_t)((b * H + n) * 4), __builtin_bit_cast(uint32_t, xr + z));
      }
    }
    asm volatile("" ::: "memory");
    prefetch_tile<WT>(R, (const WT*)L.w_ff1, (const half_t*)L.s_ff1, F, H, a.group, f0, nf, wave, lane);
    if (!barrier([] { wait_vm_at_most<kWLoads>(); })) return;

    // ---- region 3: LN2 + FF1 + bias + GeLU
    fresh();
    if (tid < nf * B) pb = ldp<AT>(L.b_ff1, f0 + tid / B);
    slot_clear(nf);
    stage_ln<float, LT, AT, BM>(a.x2, B, H, (const AT*)L.ln2_g, (const AT*)L.ln2_b, a.eps, act, raw, red2, tid);
    lds_barrier();
    if (nf > 0) gemv_tile<WT, BM>(R, (const WT*)L.w_ff1, (const half_t*)L.s_ff1, F, H, a.group, f0, nf, act, slots, wave, lane);
    lds_barrier();
    {
      const rsrc_t rf = make_rsrc(a.f, (uint32_t)(B * F * sizeof(AT)));
      for (int t = tid; t < nf * B; t += kStackThreads) {
        const int rl = t / B, b = t - rl * B, n = f0 + rl;
        const float z = row_sum(rl, b) + (t == tid ? pb : ldp<AT>(L.b_ff1, n));
        coh_st_act<AT>(rf, (uint32_t)(b * F + n), gelu(z, a.gelu_tanh != 0));
      }
    }
    asm volatile("" ::: "memory");
    prefetch_tile<WT>(R, (const WT*)L.w_ff2, (const half_t*)L.s_ff2, H, F, a.group, y0, ny, wave, lane);
    if (!barrier([] { wait_vm_at_most<kWLoads>(); })) return;

    // ---- region 4: FF2 + bias + residual: y = x2 + W2 f + b2
    fresh();
    {
      const rsrc_t rx2 = make_rsrc(a.x2, (uint32_t)(B * H * 4));
      if (tid < ny * B) {
        const int rl = tid / B, b = tid - rl * B;
        pb = ldp<AT>(L.b_ff2, y0 + rl);
        pr = as_f32(coh_load4(rx2, (uint32_t)((b * H + y0 + rl) * 4)));
      }
    }
    slot_clear(ny);
    stage_plain<AT, LT, BM>(a.f, B, F, act, tid);
    lds_barrier();
    if (ny > 0) gemv_tile<WT, BM>(R, (const WT*)L.w_ff2, (const half_t*)L.s_ff2, H, F, a.group, y0, ny, act, slots, wave, lane);
    lds_barrier();
    {
      const rsrc_t rx2 = make_rsrc(a.x2, (uint32_t)(B * H * 4));
      const rsrc_t ry = make_rsrc(yout, (uint32_t)(B * H * sizeof(AT)));
      for (int t = tid; t < ny * B; t += kStackThreads) {
        const int rl = t / B, b = t - rl * B, n = y0 + rl;
        const float z = row_sum(rl, b) + (t == tid ? pb : ldp<AT>(L.b_ff2, n));
        const float xr = t == tid ? pr : as_f32(coh_load4(rx2, (uint32_t)((b * H + n) * 4)));
        coh_st_act<AT>(ry, (uint32_t)(b * H + n), xr + z);
      }
    }
    asm volatile("" ::: "memory");
    if (l + 1 < a.n_layers) {
      const StackLayer& Ln = a.layers[l + 1];
      prefetch_tile<WT>(R, (const WT*)Ln.w_qkv, (const half_t*)Ln.s_qkv, 3 * H, H, a.group, q0, nq, wave, lane);
      if (!barrier([] { wait_vm_at_most<kWLoads>(); })) return;
    } else {
      if (!barrier([] { wait_vm_at_most<0>(); })) return;
    }
  }

  // every layer has attended: advance the cache lengths, then the last workgroup out resets the
  // barrier state for the next launch
  if (g == 0 && tid < B)
    for (int l = 0; l < a.n_layers; ++l) {
      int32_t* dl = a.layers[l].d_len;
      if (dl[tid] + 1 <= a.cap) dl[tid] += 1;
    }
  if (tid == 0) {
    const uint32_t out = __hip_atomic_fetch_add(a.sync + kSyncExit, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (out == (uint32_t)G - 1) {
      for (int i = 0; i < kSyncGroups; ++i)
        __hip_atomic_store(a.sync + kSyncSub + i * kSyncLine, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(a.sync + kSyncTop, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(a.sync + kSyncFlag, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(a.sync + kSyncExit, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// ------------------------------------------------------------------ host-side launch helpers
int stack_rows_per_wg(int H, int F, int G) {
  int r = (3 * H + G - 1) / G;
  r = max(r, (H + G - 1) / G);
  r = max(r, (F + G - 1) / G);
  return r;
}

size_t stack_lds_bytes(Dt wdt, int B, int H, int F, int rows_per_wg) {
  const int BM = B <= 1 ? 1 : 4;
  const size_t lt = wdt == F32 ? 4 : 2;
  const size_t kmax = (size_t)(H > F ? H : F);
  size_t act = BM * kmax * lt;
  if ((size_t)BM * H * (lt + 4) > act) act = (size_t)BM * H * (lt + 4);  // LayerNorm rows in fp32 too
  size_t slots = (size_t)rows_per_wg * kStackWaves * BM * 4;
  if (slots < (size_t)kStackWaves * 128 * 4) slots = (size_t)kStackWaves * 128 * 4;  // attention scratch
  return act + slots;
}

// The attention merge stages nchunk x (head_dim + 2) floats in the activation area.
size_t stack_merge_bytes(int nchunk, int head_dim) { return (size_t)nchunk * (head_dim + 2) * 4; }

template <typename WT, typename AT, int BM, int D>
static const void* kernel_ptr() {
  return reinterpret_cast<const void*>(&stack_decode_kernel<WT, AT, BM, D>);
}

// Instantiated variants: batch tiles of 1 or 4 rows (2..4 sequences use the 4-row tile).
static const void* pick(Dt wdt, Dt adt, int B, int D) {
  const bool one = B <= 1;
#define DS_PICK(WT_, AT_)                                                                       \
  {                                                                                              \
    if (D == 64) return one ? kernel_ptr<WT_, AT_, 1, 64>() : kernel_ptr<WT_, AT_, 4, 64>();     \
    return one ? kernel_ptr<WT_, AT_, 1, 128>() : kernel_ptr<WT_, AT_, 4, 128>();               \
  }
  if (wdt == F16 && adt == F16) DS_PICK(half_t, half_t)
  if (wdt == I8 && adt == F16) DS_PICK(int8_t, half_t)
  if (wdt == F32 && adt == F32 && one) {
    if (D == 64) return kernel_ptr<float, float, 1, 64>();
    return kernel_ptr<float, float, 1, 128>();
  }
#undef DS_PICK
  return nullptr;
}

hipError_t stack_max_groups(Dt wdt, Dt adt, int B, size_t lds, int* groups) {
  // head_dim does not change the register or LDS footprint enough to matter: query d = 128
  const void* k = pick(wdt, adt, B, 128);
  if (!k) return hipErrorInvalidValue;
  int per_cu = 0, dev = 0;
  hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k, kStackThreads, lds);
  if (e != hipSuccess) return e;
  if ((e = hipGetDevice(&dev)) != hipSuccess) return e;
  int cus = 0;
  if ((e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess) return e;
  if (per_cu > 1) per_cu = 1;
  *groups = per_cu * cus;
  return hipSuccess;
}

hipError_t launch_stack_decode(Dt wdt, Dt adt, const StackArgs& a, size_t lds, hipStream_t st) {
  const void* k = pick(wdt, adt, a.B, a.d);
  if (!k) return hipErrorInvalidValue;
  StackArgs args = a;
  void* params[] = {&args};
  return hipLaunchCooperativeKernel(k, dim3(a.G), dim3(kStackThreads), params, (unsigned)lds, st);
}

}  // namespace ds
