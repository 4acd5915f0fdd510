// kernels_stack.hip -- persistent decode of a whole layer stack in one launch.
//
// Computes, for every layer in turn, the four fusion regions of one transformer layer described on
// the page "DeepSpeed Inference 内核优化深度解析" (blog.gitcode.com), section 三 3.2 (LN + QKV GeMM +
// bias; attention over the cache with the head transform folded into its addressing; the output
// GeMM with bias and residual; LN + FF1 + bias + GELU; FF2 + bias + residual). Section 三 3.1 puts the
// fusion boundaries where partial results must meet (the all-reduce points); here those are the
// points where a phase waits for the values of the previous one, produced by other workgroups.
//
// gfx950 design. One cooperative launch keeps one 12-wave workgroup per CU resident for the whole
// step. Each projection is cut into per-workgroup row tiles; a tile is one contiguous range of the
// row-major matrix, cut into 1 KB "slices" (one 16-byte load per lane of a wave64).
//
// The waves are specialized so that HBM never waits for the step's serial parts:
//  - 8 worker waves own contiguous blocks of each tile and walk the fixed sequence of all their
//    slices of all layers. Each keeps kRing slices in flight in a rotating set of registers: a
//    slice is multiplied with the staged activation (LDS) the moment it is consumed, and its
//    registers at once load the slice kRing places further on, whatever phase or layer that is.
//    Workers issue nothing but these loads, so their in-order load counter only ever waits for
//    the oldest slice; row partial sums go to LDS.
//  - 4 sync waves stage each phase's activation (LayerNorm included), reduce the workers' partial
//    sums, run the epilogues (bias, residual, GeLU, the q/k/v scatter) and compute attention over
//    the cache.
// So weight streaming continues straight through the waits between phases, the activation
// staging and the epilogues. A value that crosses workgroups is stored as a (value, tag) pair,
// the tag naming the launch, layer and phase that produced it, with sc1 buffer operations (at the
// device coherence point, past the per-XCD L2 copies); a consumer polls exactly the pairs it
// reads until their tags are current, so the grid never meets at a barrier. Every wait, in LDS or
// on other workgroups' values, is bounded by a wall-clock timeout that raises the error flag,
// after which every wave leaves the kernel.
#include <type_traits>

#include "ds_device.hpp"
#include "ds_stack.hpp"

namespace ds {
namespace {

constexpr int NS = kStackSyncWaves;
constexpr int NT = NS * kWave;             // sync threads
constexpr int NWK = kStackWorkers;
// Weight slices a worker keeps in flight: 24 for fp16 weights and one batch row (24 KB per wave,
// 192 KB per CU), 16 for fp32; variants with four batch rows or int8 weights (two 16-byte
// activation reads per row) keep 12. Twelve waves per workgroup (three per SIMD) leave every wave
// up to 168 VGPRs: the sync waves' attention and staging then run without register spills, whose
// reloads from scratch memory (queued behind the weight stream) cost 9 % of the step at sixteen
// waves and 128 VGPRs. 288 KB in flight per CU streamed no faster than 192 KB.
template <typename WT, int BM> struct Ring { static constexpr int value = (sizeof(WT) == 1 || BM == 4) ? 12 : (sizeof(WT) == 2 ? 24 : 16); };
constexpr int kAuxCoherent = 16;           // sc1
constexpr int kAuxStream = 2;              // nt
constexpr int kRsrcFlags = 0x00020000;     // raw buffer, 32-bit dword format
constexpr uint32_t kOutOfRange = 0x7ffffff0u;  // a buffer offset past every descriptor: loads return 0

typedef __amdgpu_buffer_rsrc_t rsrc_t;

// Buffer descriptors must be wave-uniform (SGPRs). Pointers read from the layer table arrive in
// VGPRs as far as the compiler knows, which would wrap every buffer access in a waterfall loop, so
// the pointer and the size pass through readfirstlane (free for values already in SGPRs).
__device__ __forceinline__ rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  const uint64_t u = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)u);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(u >> 32));
  void* q = reinterpret_cast<void*>(((uint64_t)hi << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(q, (short)0, (int)__builtin_amdgcn_readfirstlane(bytes), kRsrcFlags);
}
__device__ __forceinline__ u32x4 coh_load16(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kAuxCoherent);
}
__device__ __forceinline__ void coh_store4(rsrc_t r, uint32_t off, uint32_t v) {
  __builtin_amdgcn_raw_buffer_store_b32(v, r, off, 0, kAuxCoherent);
}

// coherent scalar store in the activation type
template <typename AT> __device__ __forceinline__ void coh_st_act(rsrc_t r, uint32_t idx, float v);
template <> __device__ __forceinline__ void coh_st_act<float>(rsrc_t r, uint32_t idx, float v) {
  coh_store4(r, idx * 4, __builtin_bit_cast(uint32_t, v));
}
template <> __device__ __forceinline__ void coh_st_act<half_t>(rsrc_t r, uint32_t idx, float v) {
  __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(uint16_t, (half_t)v), r, idx * 2, 0, kAuxCoherent);
}
template <> __device__ __forceinline__ void coh_st_act<bf16_t>(rsrc_t r, uint32_t idx, float v) {
  __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(uint16_t, (bf16_t)v), r, idx * 2, 0, kAuxCoherent);
}

template <typename T> __device__ __forceinline__ float ldp(const void* p, int i) {
  return (float)reinterpret_cast<const T*>(p)[i];
}

// Element i of a T array as raw bits, converted later by cvraw. A wave waits for a load at the
// first use of its value, and that wait also covers every earlier store of the wave (on this ISA
// one counter tracks both): converting at the use point keeps an early-issued load from making the
// wave wait for the acknowledgements of the tagged stores it has just made.
template <typename T> __device__ __forceinline__ uint32_t ldraw(const void* p, int i) {
  if constexpr (sizeof(T) == 2) return (uint32_t)reinterpret_cast<const uint16_t*>(p)[i];
  else return reinterpret_cast<const uint32_t*>(p)[i];
}
template <typename T> __device__ __forceinline__ float cvraw(uint32_t u) {
  if constexpr (sizeof(T) == 2) return lo16<T>(u);
  else return __builtin_bit_cast(float, u);
}

// s_waitcnt with only the vector-memory counter limited to N (gfx9 encoding: vmcnt in bits
// [3:0] and [15:14], expcnt [6:4] and lgkmcnt [11:8] left at their maxima).
template <int N> __device__ __forceinline__ void wait_vm_at_most() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
  asm volatile("" ::: "memory");
}
__device__ __forceinline__ void wait_lgkm0() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt((15) | (3 << 14) | (7 << 4) | (0 << 8));
  asm volatile("" ::: "memory");
}

// ------------------------------------------------------------------ workgroup control block
// LDS words shared by the sync and worker waves of one workgroup.
struct Ctl {
  uint32_t act_ready;    // 1 + sequence number of the phase whose activation is staged
  uint32_t done[NWK];    // phases each worker has finished (its partial sums are in LDS)
  uint32_t sbar;         // sync-wave barrier arrivals
  uint32_t abort;        // set when any wait of this workgroup failed
  uint32_t launch;       // launch counter (tags of this launch)
  float red[NS][12];     // LayerNorm per wave and row (up to 4): two sums, or count, mean, deviations
  float m[NS], l[NS];    // attention: per-wave max and sum
  int tab[NWK][5][8];    // per worker and phase (4: the LM head): the block geometry (see worker_table)
  uint64_t best[kStackMaxBatch];  // LM head: this workgroup's largest argmax key per sequence
};

// Fields of a worker's phase-table entry.
enum { T_CNT = 0, T_BASE = 1, T_BYTES = 2, T_K = 3, T_SPER = 4, T_RL0 = 5, T_KS0 = 6, T_GRP = 7 };

__device__ __forceinline__ uint32_t lds_ld(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ void lds_st(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

__device__ __forceinline__ void raise_abort(Ctl& c, uint32_t* sync) {
  lds_st(&c.abort, 1u);
  __hip_atomic_store(sync + kSyncError, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The grid error flag is a global load, which waits behind the CU's queue of weight loads: a
// waiting loop reads it once every kErrorEvery rounds, so that it does not delay the loop's
// reaction to the value it waits for (the wall-clock timeout is checked every round).
constexpr uint32_t kErrorEvery = 64;

// Spin until pred() holds; false on this workgroup's abort, the grid error flag or a timeout
// (which raises both). Only lane 0 of the wave polls (the other lanes would only add LDS traffic
// that the workers' activation reads queue behind); the outcome is broadcast to the wave.
template <typename Pred>
__device__ __forceinline__ bool spin_until(Ctl& c, const StackArgs& a, Pred pred) {
  int ok = 1;
  if (__lane_id() == 0 && !pred()) {
    const uint64_t t0 = wall_clock64();
    for (uint32_t it = 1;; ++it) {
      __builtin_amdgcn_s_sleep(2);
      if (pred()) break;
      if (lds_ld(&c.abort) != 0u) {
        ok = 0;
        break;
      }
      if (wall_clock64() - t0 > a.timeout_ticks ||
          (it % kErrorEvery == 0 &&
           __hip_atomic_load(a.sync + kSyncError, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u)) {
        raise_abort(c, a.sync);
        ok = 0;
        break;
      }
    }
  }
  asm volatile("" ::: "memory");
  return __builtin_amdgcn_readfirstlane(ok) != 0;
}

// The workers' wait: LDS only (a global load here would also wait for the whole weight ring, as
// loads complete in order); grid errors reach a worker through the abort word the sync waves set.
template <typename Pred>
__device__ __forceinline__ bool worker_spin(Ctl& c, const StackArgs& a, Pred pred) {
  int ok = 1;
  if (__lane_id() == 0 && !pred()) {
    const uint64_t t0 = wall_clock64();
    for (;;) {
      __builtin_amdgcn_s_sleep(1);
      if (pred()) break;
      if (lds_ld(&c.abort) != 0u) {
        ok = 0;
        break;
      }
      if (wall_clock64() - t0 > a.timeout_ticks) {
        raise_abort(c, a.sync);
        ok = 0;
        break;
      }
    }
  }
  asm volatile("" ::: "memory");
  return __builtin_amdgcn_readfirstlane(ok) != 0;
}

// Barrier of the NS sync waves only (the workers never join it). `sb` counts these barriers.
__device__ __forceinline__ bool sync_bar(Ctl& c, const StackArgs& a, uint32_t& sb, int st) {
  ++sb;
  wait_lgkm0();
  if ((st & 63) == 0) __hip_atomic_fetch_add(&c.sbar, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  const uint32_t target = sb * (uint32_t)NS;
  const bool ok = spin_until(c, a, [&] { return lds_ld(&c.sbar) >= target; });
  asm volatile("" ::: "memory");
  return ok;
}

// ------------------------------------------------------------------ tagged values across workgroups
// A value that crosses workgroups is one 8-byte store: the float's bits, then the tag of the phase
// that produced it. Stores and loads go through sc1 (the device coherence point, past the per-XCD
// L2s). A consumer re-reads the pairs whose tag is not yet the expected one, so workgroups never
// meet at a barrier: each phase waits for exactly the values it reads.
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ void tstore(rsrc_t r, uint32_t idx, float v, uint32_t tag) {
  const u32x2 pv = {__builtin_bit_cast(uint32_t, v), tag};
  __builtin_amdgcn_raw_buffer_store_b64(pv, r, idx * 8u, 0, kAuxCoherent);
}

// Two 16-bit values (fp16 or bf16, rounded from fp32) packed in the value word of one tagged 8-byte
// store (element 2i low, 2i+1 high).
template <typename AT>
__device__ __forceinline__ void tstore_pair(rsrc_t r, uint32_t pair, float lo, float hi, uint32_t tag) {
  const u32x2 pv = {pack16<AT>(lo, hi), tag};
  __builtin_amdgcn_raw_buffer_store_b64(pv, r, pair * 8u, 0, kAuxCoherent);
}

__device__ __forceinline__ bool grid_error(const StackArgs& a) {
  return __hip_atomic_load(a.sync + kSyncError, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u;
}

constexpr int kPollUnroll = 8;  // 16-byte loads (two tagged values each) a thread keeps in flight
constexpr int kPollWide = 10;   // the same for the LayerNorm rows past the register path and for f:
                                // one round for 5120 values (hidden 5120, or ffn 10240 as pairs)

// Wait until the tagged values [0, n) at src all carry `tag`, handing each one once to put(i, v).
// Threads st, st+NT, ... of the sync waves share the work.
template <int U = kPollUnroll, typename Put>
__device__ __forceinline__ bool poll_range(Ctl& c, const StackArgs& a, const uint2* src, int n, uint32_t tag, int st,
                                           Put put) {
  const rsrc_t r = make_rsrc(src, (uint32_t)n * 8u);
  const int nv = (n + 1) >> 1;
  for (int j0 = st; j0 < nv; j0 += NT * U) {
    bool need[U];
#pragma unroll
    for (int u = 0; u < U; ++u) need[u] = j0 + u * NT < nv;
    uint64_t t0 = 0;
    for (int round = 0;; ++round) {
      u32x4 v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) v[u] = coh_load16(r, need[u] ? (uint32_t)((j0 + u * NT) * 16) : kOutOfRange);
      bool stale = false;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (!need[u]) continue;
        const int i = 2 * (j0 + u * NT);
        const bool second = i + 1 < n;
        if (v[u].y == tag && (!second || v[u].w == tag)) {
          put(i, as_f32(v[u].x));
          if (second) put(i + 1, as_f32(v[u].z));
          need[u] = false;
        } else {
          stale = true;
        }
      }
      if (!stale) break;
      if (round == 0) {
        t0 = wall_clock64();
      } else if (wall_clock64() - t0 > a.timeout_ticks || lds_ld(&c.abort) != 0u ||
                 ((uint32_t)round % kErrorEvery == 0 && grid_error(a))) {
        raise_abort(c, a.sync);
        return false;
      }
      __builtin_amdgcn_s_sleep(1);
    }
  }
  return true;
}

// One lane's run of `cnt` consecutive tagged values (cnt even), polled until current.
template <int CNT>
__device__ __forceinline__ bool poll_lane(Ctl& c, const StackArgs& a, rsrc_t r, uint32_t first, uint32_t tag,
                                          float (&out)[CNT]) {
  static_assert(CNT % 2 == 0, "pairs of tagged values");
  bool need[CNT / 2];
#pragma unroll
  for (int u = 0; u < CNT / 2; ++u) need[u] = true;
  uint64_t t0 = 0;
  for (int round = 0;; ++round) {
    bool stale = false;
    u32x4 v[CNT / 2];
#pragma unroll
    for (int u = 0; u < CNT / 2; ++u) v[u] = coh_load16(r, need[u] ? (first + 2u * u) * 8u : kOutOfRange);
#pragma unroll
    for (int u = 0; u < CNT / 2; ++u) {
      if (!need[u]) continue;
      if (v[u].y == tag && v[u].w == tag) {
        out[2 * u] = as_f32(v[u].x);
        out[2 * u + 1] = as_f32(v[u].z);
        need[u] = false;
      } else {
        stale = true;
      }
    }
    if (!stale) return true;
    if (round == 0) {
      t0 = wall_clock64();
    } else if (wall_clock64() - t0 > a.timeout_ticks || lds_ld(&c.abort) != 0u ||
               ((uint32_t)round % kErrorEvery == 0 && grid_error(a))) {
      raise_abort(c, a.sync);
      return false;
    }
    __builtin_amdgcn_s_sleep(1);
  }
}

// ------------------------------------------------------------------ row tiles
// Phase ph (0 QKV, 1 O, 2 FF1, 3 FF2, 4 the LM head) of workgroup g: rows [r0, r0+nr) of the [N][K]
// matrix, one contiguous range of nr*K elements cut into slices of SL elements (K is a multiple of
// SL), so slice s lies in tile row s / (K/SL). Worker w owns the contiguous block [s0, s0+cnt), whose
// ends are multiples of GS slices (GS divides K/SL: a group of GS slices never straddles a row).
struct Geo {
  int N, K, r0, nr, s0, cnt;
};

__device__ __forceinline__ Geo phase_geo(const StackArgs& a, int SL, int GS, int g, int w, int ph) {
  const int H = a.H, F = a.F, G = a.G;
  Geo p;
  p.N = ph == 0 ? 3 * H : (ph == 2 ? F : (ph == 4 ? a.V : H));
  p.K = ph == 3 ? F : H;
  const int rows = stack_tile_rows(p.N, G, ph == 2);
  p.r0 = min(p.N, g * rows);
  p.nr = min(p.N, p.r0 + rows) - p.r0;
  const int T = p.nr * (p.K / SL);
  const int M = ((T + NWK - 1) / NWK + GS - 1) / GS * GS;
  p.s0 = min(T, w * M);
  p.cnt = min(T, p.s0 + M) - p.s0;
  return p;
}

__device__ __forceinline__ const void* phase_w(const StackLayer& L, int ph) {
  return ph == 0 ? L.w_qkv : ph == 1 ? L.w_o : ph == 2 ? L.w_ff1 : L.w_ff2;
}

// ------------------------------------------------------------------ worker waves
template <int BM>
__device__ __forceinline__ void flush_rows(float (&acc)[BM], float* slots, int rl, int w, int lane) {
#pragma unroll
  for (int b = 0; b < BM; ++b) {
    const float v = wave_sum_dpp(acc[b]);
    if (lane == 0) slots[(rl * NWK + w) * BM + b] = v;
    acc[b] = 0.f;
  }
}

// Lane p (0..4) of worker w fills the table entry of phase p, counting in groups of GS slices: group
// count, byte offset of the block's first slice in the matrix, matrix bytes, K, groups per row, first
// row and group-in-row.
template <typename WT, int GS>
__device__ __forceinline__ void worker_table(const StackArgs& a, Ctl& c, int g, int w, int lane) {
  constexpr int SL = kWave * WTraits<WT>::E;
  if (lane < 5) {
    const Geo p = phase_geo(a, SL, GS, g, w, lane);
    int* t = c.tab[w][lane];
    const int sper = p.K / SL;
    t[T_CNT] = p.cnt / GS;
    t[T_BASE] = (int)(((size_t)p.r0 * p.K + (size_t)p.s0 * SL) * sizeof(WT));
    t[T_BYTES] = (int)((size_t)p.N * p.K * sizeof(WT));
    t[T_K] = p.K;
    t[T_SPER] = sper / GS;
    t[T_RL0] = p.s0 / sper;
    t[T_KS0] = (p.s0 - (p.s0 / sper) * sper) / GS;
    t[T_GRP] = lane == 2 || lane == 3 ? a.group_mlp : a.group;  // int8 scale group of the phase's matrix
  }
  wait_lgkm0();
}

__device__ __forceinline__ int tab_ld(const Ctl& c, int w, int ph, int f) {
  return __builtin_amdgcn_readfirstlane(c.tab[w][ph][f]);
}

// Weight-matrix pointer of step p (layer p / 4, phase p % 4; p = 4 L is the LM head) from the LDS
// table, made wave-uniform.
__device__ __forceinline__ const void* wtab_ld(const uint64_t* wtab, int p) {
  const uint64_t u = wtab[p];
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)u);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(u >> 32));
  return reinterpret_cast<const void*>(((uint64_t)hi << 32) | lo);
}

// A worker walks its sequence of groups (GS consecutive 1 KB slices of one row) with a ring of RG
// groups in flight: each group is multiplied with the staged activation as soon as all its slices
// have landed (GS LDS reads, then GS products, back to back), and only then are the group's
// registers refilled with the group RG places further on, whatever phase or layer that is. The
// bookkeeping runs once per group, which is what bounds a worker's pace through slices that have
// already landed (the first groups of a phase were loaded during the exchange before it).
template <typename WT, int BM, int GS>
__device__ __forceinline__ void worker(const StackArgs& a, Ctl& c, const typename WTraits<WT>::LT* act, float* slots,
                                       const half_t* scl, const uint64_t* wtab, int g, int w, int lane) {
  typedef typename WTraits<WT>::LT LT;
  constexpr int E = WTraits<WT>::E, SL = kWave * E;
  constexpr int RG = Ring<WT, BM>::value / GS > 0 ? Ring<WT, BM>::value / GS : 1;  // groups in flight
  constexpr uint32_t SLB = (uint32_t)(SL * sizeof(WT));  // bytes of one slice
  constexpr uint32_t GB = SLB * GS;                     // bytes of one group
  // The worker's steps: p = 4 l + ph for the four projections of layer l, then p = 4 L for the LM
  // head when this launch runs it; gi(p) names the step's entry in the phase table.
  const int L = a.n_layers;
  const int P = 4 * L + (a.head ? 1 : 0);
  auto gi = [&](int p) { return p < 4 * L ? (p & 3) : 4; };
  worker_table<WT, GS>(a, c, g, w, lane);
  const int per_layer = tab_ld(c, w, 0, T_CNT) + tab_ld(c, w, 1, T_CNT) + tab_ld(c, w, 2, T_CNT) + tab_ld(c, w, 3, T_CNT);
  const int total = L * per_layer + (a.head ? tab_ld(c, w, 4, T_CNT) : 0);  // groups

  // issue cursor: the next group to load (step ip, group is of icnt)
  int ip = 0, is = 0, icnt = tab_ld(c, w, 0, T_CNT);
  while (ip < P && icnt == 0) {
    ++ip;
    icnt = ip < P ? tab_ld(c, w, gi(ip), T_CNT) : 0;
  }
  const void* iw = wtab_ld(wtab, ip < P ? ip : 0);
  uint32_t ibytes = (uint32_t)tab_ld(c, w, ip < P ? gi(ip) : 0, T_BYTES);
  uint32_t ioff = (uint32_t)tab_ld(c, w, ip < P ? gi(ip) : 0, T_BASE);
  const uint32_t voff = (uint32_t)(lane * 16);

  // consume cursor: the next group to multiply (step cp, group cs of ccnt; row rl, group ks of Sper)
  int cp = 0, cs = 0, ccnt = tab_ld(c, w, 0, T_CNT);
  int K = tab_ld(c, w, 0, T_K), Sper = tab_ld(c, w, 0, T_SPER);
  int rl = tab_ld(c, w, 0, T_RL0), ks = tab_ld(c, w, 0, T_KS0);
  int grp = tab_ld(c, w, 0, T_GRP), spr = K / grp;  // int8: scale group and scales per row
  // int8: the group of element x of a row is x / grp = mulhi(x, ceil(2^32 / grp)), exact while
  // x * grp < 2^32 (stack creation checks row length x group against that bound)
  uint32_t ginv = (uint32_t)(((1ull << 32) + (uint64_t)grp - 1) / (uint64_t)grp);
  bool wait_act = true;
  // leave step cp [finished or empty], publishing it, and move to the next non-empty one
  auto c_advance = [&]() {
    for (;;) {
      wait_lgkm0();  // this wave's slot writes are in LDS before the flag says so
      if (lane == 0) lds_st(&c.done[w], (uint32_t)(cp + 1));
      if (++cp >= P) return;
      ccnt = tab_ld(c, w, gi(cp), T_CNT);
      if (ccnt > 0) break;
    }
    const int t = gi(cp);
    cs = 0;
    K = tab_ld(c, w, t, T_K);
    Sper = tab_ld(c, w, t, T_SPER);
    rl = tab_ld(c, w, t, T_RL0);
    ks = tab_ld(c, w, t, T_KS0);
    grp = tab_ld(c, w, t, T_GRP);
    spr = K / grp;
    ginv = (uint32_t)(((1ull << 32) + (uint64_t)grp - 1) / (uint64_t)grp);
    wait_act = true;
  };
  if (ccnt == 0) c_advance();

  float acc[BM];
#pragma unroll
  for (int b = 0; b < BM; ++b) acc[b] = 0.f;

  // issue one group: GS loads of the next group, or out-of-range loads (read nothing) past the end
#define DS_ISSUE(dst)                                                                                \
  {                                                                                                  \
    const bool live = ip < P;                                                                        \
    const rsrc_t r = make_rsrc(iw, ibytes);                                                          \
    _Pragma("unroll") for (int k = 0; k < GS; ++k) dst[k] =                                          \
        __builtin_amdgcn_raw_buffer_load_b128(r, voff, live ? ioff + (uint32_t)k * SLB : kOutOfRange, kAuxStream); \
    ioff += GB;                                                                                      \
    if (live && ++is >= icnt) {                                                                      \
      is = 0;                                                                                        \
      do {                                                                                           \
        ++ip;                                                                                        \
        icnt = ip < P ? tab_ld(c, w, gi(ip), T_CNT) : 0;                                             \
      } while (ip < P && icnt == 0);                                                                 \
      if (ip < P) {                                                                                  \
        iw = wtab_ld(wtab, ip);                                                                      \
        ibytes = (uint32_t)tab_ld(c, w, gi(ip), T_BYTES);                                            \
        ioff = (uint32_t)tab_ld(c, w, gi(ip), T_BASE);                                               \
      }                                                                                              \
    }                                                                                                \
  }

  u32x4 ring[RG][GS];
#pragma unroll
  for (int u = 0; u < RG; ++u) DS_ISSUE(ring[u])

  bool ok = true;
  for (int pos = 0; pos < total && ok;) {
#pragma unroll
    for (int u = 0; u < RG; ++u) {
      if (pos < total && ok) {
        // the cursor is wave-uniform; say so, so that its bookkeeping stays in scalar registers
        ks = __builtin_amdgcn_readfirstlane(ks);
        rl = __builtin_amdgcn_readfirstlane(rl);
        cs = __builtin_amdgcn_readfirstlane(cs);
        wait_vm_at_most<(RG - 1) * GS>();  // exactly RG groups are in flight: the oldest has landed
        if (wait_act) {
          const uint32_t need = (uint32_t)(cp + 1);
          ok = worker_spin(c, a, [&] { return lds_ld(&c.act_ready) >= need; });
          wait_act = false;
        }
        if (ok) {
          const LT* ap = act + ks * (GS * SL) + lane * E;
#pragma unroll
          for (int k = 0; k < GS; ++k) {
            float sc = 1.f;
            if constexpr (sizeof(WT) == 1)
              sc = (float)scl[rl * spr + __umulhi((uint32_t)((ks * GS + k) * SL + lane * E), ginv)];
#pragma unroll
            for (int b = 0; b < BM; ++b) {
              const LT* apk = ap + k * SL + b * K;
              if constexpr (sizeof(WT) == 4) {
                acc[b] = dot4_f32(ring[u][k], *reinterpret_cast<const float4_t*>(apk), acc[b]);
              } else if constexpr (sizeof(WT) == 2) {
                acc[b] = dot8<WT>(ring[u][k], *reinterpret_cast<const u32x4*>(apk), acc[b]);
              } else {
                acc[b] = fmaf(dot16_i8(ring[u][k], *reinterpret_cast<const u32x4*>(apk),
                                       *reinterpret_cast<const u32x4*>(apk + 8)),
                              sc, acc[b]);
              }
            }
          }
          if (++ks == Sper) {
            flush_rows<BM>(acc, slots, rl, w, lane);
            ks = 0;
            ++rl;
          }
          if (++cs == ccnt) {
            if (ks != 0) flush_rows<BM>(acc, slots, rl, w, lane);
            c_advance();
          }
        }
        ++pos;
      }
      DS_ISSUE(ring[u])
    }
  }
#undef DS_ISSUE
  wait_vm_at_most<0>();
}

// ------------------------------------------------------------------ sync waves: staging
// LayerNorm B rows (biased variance) into LDS as LT. gamma and beta (this layer's, in AT) are
// already in LDS at gb (gamma, then beta: prefetched a phase earlier); fill() puts the rows into
// `raw` as fp32. Then one reduction of the shifted sums of all rows and the normalized rows.
template <typename LT, typename AT, int BM, typename Fill>
__device__ __forceinline__ bool stage_ln(Ctl& c, const StackArgs& a, uint32_t& sb, int B, int K, LT* act, float* raw,
                                         const AT* gb, int st, Fill fill) {
  if (!fill()) return false;
  if (!sync_bar(c, a, sb, st)) return false;
  // sums of d = x - x[0] and d^2 per row: var = (sum d^2 - (sum d)^2 / K) / K; shifting by an
  // element of the row keeps the subtraction well conditioned
  float s1[BM], s2[BM];
#pragma unroll
  for (int b = 0; b < BM; ++b) {
    s1[b] = 0.f;
    s2[b] = 0.f;
    if (b < B) {
      const float* xr = raw + b * K;
      const float c0 = xr[0];
      for (int k = st; k < K; k += NT) {
        const float d = xr[k] - c0;
        s1[b] += d;
        s2[b] += d * d;
      }
    }
    s1[b] = wave_sum_dpp(s1[b]);
    s2[b] = wave_sum_dpp(s2[b]);
  }
  if ((st & 63) == 0) {
#pragma unroll
    for (int b = 0; b < BM; ++b) {
      c.red[st >> 6][2 * b] = s1[b];
      c.red[st >> 6][2 * b + 1] = s2[b];
    }
  }
  if (!sync_bar(c, a, sb, st)) return false;
#pragma unroll
  for (int b = 0; b < BM; ++b) {
    if (b >= B) {
      for (int k = st; k < K; k += NT) act[b * K + k] = (LT)0.f;
      continue;
    }
    float t1 = 0.f, t2 = 0.f;
#pragma unroll
    for (int wv = 0; wv < NS; ++wv) {
      t1 += c.red[wv][2 * b];
      t2 += c.red[wv][2 * b + 1];
    }
    const float* xr = raw + b * K;
    const float dm = t1 / K;
    const float mean = xr[0] + dm;
    const float rstd = rsqrtf(fmaxf(t2 / K - dm * dm, 0.f) + a.eps);
    for (int k = st; k < K; k += NT) act[b * K + k] = (LT)((xr[k] - mean) * rstd * (float)gb[k] + (float)gb[K + k]);
  }
  return true;
}

// The caller's B rows of K elements (AT, written before the launch) as fp32 into raw.
template <typename AT>
__device__ __forceinline__ void load_rows_plain(const void* in, int B, int K, float* raw, int st) {
  constexpr int V = 16 / (int)sizeof(AT);
  const rsrc_t r = make_rsrc(in, (uint32_t)(B * K * sizeof(AT)));
  const int nvec = B * K / V;
  for (int j0 = st; j0 < nvec; j0 += NT * kPollUnroll) {
    u32x4 v[kPollUnroll];
#pragma unroll
    for (int u = 0; u < kPollUnroll; ++u) {
      const int j = j0 + u * NT;
      v[u] = __builtin_amdgcn_raw_buffer_load_b128(r, j < nvec ? (uint32_t)(j * 16) : kOutOfRange, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < kPollUnroll; ++u) {
      const int j = j0 + u * NT;
      if (j >= nvec) break;
      if constexpr (sizeof(AT) == 4) {
        *reinterpret_cast<u32x4*>(raw + j * V) = v[u];
      } else {
        const uint32_t ww[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          raw[j * V + 2 * h] = lo16<AT>(ww[h]);
          raw[j * V + 2 * h + 1] = hi16<AT>(ww[h]);
        }
      }
    }
  }
}

// ------------------------------------------------------------------ sync waves: LayerNorm in registers
// When the B rows fit kLnPairs pairs per sync thread, each thread keeps the pairs it fetched in
// registers (pair j = st + u NT holds elements 2j, 2j + 1 of the flattened [B][K] rows), reduces
// them, and writes its normalized pairs: one barrier and no round trip of the rows through LDS.
constexpr int kLnPairs = 5;  // 2560 elements: more would spill the sync waves' registers

// Pairwise update of (count, mean, sum of squared deviations) (Chan, Golub and LeVeque).
__device__ __forceinline__ void chan_merge(float& n, float& m, float& q, float n2, float m2, float q2) {
  const float nn = n + n2;
  if (nn > 0.f) {
    const float d = m2 - m, f = n2 / nn;
    q += q2 + d * d * n * f;
    m += d * f;
    n = nn;
  }
}

// The tagged pairs of [0, n) (n even) owned by thread st into x, polled until current.
template <int PU>
__device__ __forceinline__ bool poll_regs(Ctl& c, const StackArgs& a, const uint2* src, int n, uint32_t tag, int st,
                                          float (&x)[PU][2]) {
  const rsrc_t r = make_rsrc(src, (uint32_t)n * 8u);
  const int nv = n >> 1;
  bool need[PU];
#pragma unroll
  for (int u = 0; u < PU; ++u) need[u] = st + u * NT < nv;
  uint64_t t0 = 0;
  for (int round = 0;; ++round) {
    u32x4 v[PU];
#pragma unroll
    for (int u = 0; u < PU; ++u) v[u] = coh_load16(r, need[u] ? (uint32_t)((st + u * NT) * 16) : kOutOfRange);
    bool stale = false;
#pragma unroll
    for (int u = 0; u < PU; ++u) {
      if (!need[u]) continue;
      if (v[u].y == tag && v[u].w == tag) {
        x[u][0] = as_f32(v[u].x);
        x[u][1] = as_f32(v[u].z);
        need[u] = false;
      } else {
        stale = true;
      }
    }
    if (!stale) break;
    if (round == 0) {
      t0 = wall_clock64();
    } else if (wall_clock64() - t0 > a.timeout_ticks || lds_ld(&c.abort) != 0u ||
               ((uint32_t)round % kErrorEvery == 0 && grid_error(a))) {
      raise_abort(c, a.sync);
      return false;
    }
    __builtin_amdgcn_s_sleep(1);
  }
  return true;
}

// The caller's rows (AT, written before the launch): thread st's pairs of [0, n) into x.
template <typename AT, int PU>
__device__ __forceinline__ void load_regs_plain(const void* in, int n, int st, float (&x)[PU][2]) {
  const rsrc_t r = make_rsrc(in, (uint32_t)(n * sizeof(AT)));
  const int nv = n >> 1;
#pragma unroll
  for (int u = 0; u < PU; ++u) {
    const int j = st + u * NT;
    const uint32_t off = j < nv ? (uint32_t)(j * 2 * sizeof(AT)) : kOutOfRange;
    if constexpr (sizeof(AT) == 2) {
      const uint32_t h = __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
      x[u][0] = lo16<AT>(h);
      x[u][1] = hi16<AT>(h);
    } else {
      const u32x2 w = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
      x[u][0] = as_f32(w.x);
      x[u][1] = as_f32(w.y);
    }
  }
}

// LayerNorm (biased variance) of B rows of K elements held as pairs in registers, into act as LT;
// the rows come from `plain` (the caller's input) when it is given, else from the tagged values at
// `tagged`. gamma and beta are already in LDS at gb (gamma, then beta: prefetched a phase earlier);
// their reads are issued before the rows' poll, whose latency covers them.
template <typename LT, typename AT, int BM, int PU>
__device__ __forceinline__ bool stage_ln_regs(Ctl& c, const StackArgs& a, uint32_t& sb, int B, int K, const AT* gb,
                                              LT* act, int st, const void* plain, const uint2* tagged, uint32_t tag) {
  const int n = B * K, nv = n >> 1;
  // the thread's gamma and beta pairs (LDS reads, overlapping the rows' poll)
  u32x2 gw[PU], bw[PU];  // fp16: the pair in .x; fp32: the two values
#pragma unroll
  for (int u = 0; u < PU; ++u) {
    const int j = st + u * NT;
    const int e = j < nv ? 2 * j % K : 0;
    if constexpr (sizeof(AT) == 2) {
      gw[u].x = *reinterpret_cast<const uint32_t*>(gb + e);
      bw[u].x = *reinterpret_cast<const uint32_t*>(gb + K + e);
    } else {
      gw[u] = *reinterpret_cast<const u32x2*>(gb + e);
      bw[u] = *reinterpret_cast<const u32x2*>(gb + K + e);
    }
  }
  float x[PU][2];
  if (plain)
    load_regs_plain<AT, PU>(plain, n, st, x);
  else if (!poll_regs<PU>(c, a, tagged, n, tag, st, x))
    return false;
  // per thread and row: count, mean and squared deviations of its values (two passes in registers),
  // then merged across the wave
  float sn[BM], sm[BM], sq[BM];
#pragma unroll
  for (int b = 0; b < BM; ++b) {
    float s = 0.f, cnt = 0.f;
#pragma unroll
    for (int u = 0; u < PU; ++u) {
      const int j = st + u * NT;
      if (j < nv && (BM == 1 || 2 * j / K == b)) {
        s += x[u][0] + x[u][1];
        cnt += 2.f;
      }
    }
    const float m = cnt > 0.f ? s / cnt : 0.f;
    float q = 0.f;
#pragma unroll
    for (int u = 0; u < PU; ++u) {
      const int j = st + u * NT;
      if (j < nv && (BM == 1 || 2 * j / K == b)) {
        const float d0 = x[u][0] - m, d1 = x[u][1] - m;
        q += d0 * d0 + d1 * d1;
      }
    }
    sn[b] = cnt;
    sm[b] = m;
    sq[b] = q;
  }
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1)
#pragma unroll
    for (int b = 0; b < BM; ++b) {
      const float n2 = __shfl_xor(sn[b], off, kWave), m2 = __shfl_xor(sm[b], off, kWave);
      const float q2 = __shfl_xor(sq[b], off, kWave);
      chan_merge(sn[b], sm[b], sq[b], n2, m2, q2);
    }
  if ((st & 63) == 0) {
#pragma unroll
    for (int b = 0; b < BM; ++b) {
      c.red[st >> 6][3 * b] = sn[b];
      c.red[st >> 6][3 * b + 1] = sm[b];
      c.red[st >> 6][3 * b + 2] = sq[b];
    }
  }
  if (!sync_bar(c, a, sb, st)) return false;
  float mean[BM], rstd[BM];
#pragma unroll
  for (int b = 0; b < BM; ++b) {
    float tn = 0.f, tm = 0.f, tq = 0.f;
#pragma unroll
    for (int wv = 0; wv < NS; ++wv) chan_merge(tn, tm, tq, c.red[wv][3 * b], c.red[wv][3 * b + 1], c.red[wv][3 * b + 2]);
    mean[b] = tm;
    rstd[b] = rsqrtf(fmaxf(tq / (float)K, 0.f) + a.eps);
  }
#pragma unroll
  for (int u = 0; u < PU; ++u) {
    const int j = st + u * NT;
    if (j >= nv) continue;
    const int b = BM == 1 ? 0 : 2 * j / K;
    float g0, g1, b0, b1;
    if constexpr (sizeof(AT) == 2) {
      g0 = lo16<AT>(gw[u].x);
      g1 = hi16<AT>(gw[u].x);
      b0 = lo16<AT>(bw[u].x);
      b1 = hi16<AT>(bw[u].x);
    } else {
      g0 = as_f32(gw[u].x);
      g1 = as_f32(gw[u].y);
      b0 = as_f32(bw[u].x);
      b1 = as_f32(bw[u].y);
    }
    float mb = mean[0], rb_ = rstd[0];
#pragma unroll
    for (int bb = 1; bb < BM; ++bb)
      if (bb == b) {
        mb = mean[bb];
        rb_ = rstd[bb];
      }
    act[2 * j] = (LT)((x[u][0] - mb) * rb_ * g0 + b0);
    act[2 * j + 1] = (LT)((x[u][1] - mb) * rb_ * g1 + b1);
  }
  for (int i = n + st; i < BM * K; i += NT) act[i] = (LT)0.f;  // activation rows past B
  return true;
}

// int8: the fp16 scales of the phase's row tile, [nr][K/group], into LDS.
__device__ __forceinline__ void stage_scales(const void* s, int r0, int nr, int K, int group, half_t* scl, int st) {
  const int n = nr * (K / group);
  const size_t e0 = (size_t)r0 * (K / group);
  const half_t* src = static_cast<const half_t*>(s) + e0;
  int done = 0;
  if ((e0 & 7) == 0) {
    // 16-byte loads, kScaleVec per thread issued before any is written: one memory round trip
    // per kScaleVec * NT vectors (a round trip is long while the workers stream)
    constexpr int kScaleVec = 4;
    const int nv = n >> 3;
    const rsrc_t r = make_rsrc(src, (uint32_t)n * 2u);
    for (int j0 = 0; j0 < nv; j0 += kScaleVec * NT) {
      u32x4 v[kScaleVec];
#pragma unroll
      for (int u = 0; u < kScaleVec; ++u) {
        const int j = j0 + st + u * NT;
        v[u] = __builtin_amdgcn_raw_buffer_load_b128(r, j < nv ? (uint32_t)(j * 16) : kOutOfRange, 0, 0);
      }
#pragma unroll
      for (int u = 0; u < kScaleVec; ++u) {
        const int j = j0 + st + u * NT;
        if (j < nv) *reinterpret_cast<u32x4*>(scl + j * 8) = v[u];
      }
    }
    done = nv * 8;
  }
  for (int i = done + st; i < n; i += NT) scl[i] = src[i];
}

// ------------------------------------------------------------------ sync waves: attention
// An item is (sequence b, head j, chunk c of kStackChunk cache rows). Lanes split a row into
// 16-byte pieces (LPK lanes per row), a wave covers KPI rows per load, NS waves cover NS*KPI.
template <typename AT, int D> struct AttnShape {
  static constexpr int EK = 16 / (int)sizeof(AT);
  static constexpr int LPK = D / EK;
  static constexpr int KPI = kWave / LPK;
  static constexpr int NIT = (kStackChunk + NS * KPI - 1) / (NS * KPI);
};

// The attention items of one layer: (sequence b, head j, chunk cc) for the chunks that hold keys,
// numbered densely over the longest sequence's chunk count so that workgroups get at most one
// item each whenever there are fewer items than workgroups, whatever the cache capacity.
struct AttnItem {
  int b, j, cc;
  bool valid;
};
__device__ __forceinline__ int attn_nvalid(const StackArgs& a, int len) {
  int nkeys = len + 1;
  if (nkeys > a.cap) nkeys = a.cap;
  return (nkeys + kStackChunk - 1) / kStackChunk;
}
__device__ __forceinline__ AttnItem attn_item(const StackArgs& a, const int32_t* lens, int nvmax, int item) {
  AttnItem it;
  it.cc = item % nvmax;
  it.j = (item / nvmax) % a.nh;
  it.b = item / (nvmax * a.nh);
  it.valid = it.cc < attn_nvalid(a, lens[it.b]);
  return it;
}

// Loads of an item's past rows (written by earlier launches) straight from the cache into kr, vr;
// KT is the cache's element type (the activation type, or int8 with the rows' fp16 scales, which
// land in ksc, vsc).
template <typename KT, int D>
__device__ __forceinline__ void attn_load(const StackArgs& a, const StackLayer& L, int len, const AttnItem& it, int st,
                                          u32x4 (&kr)[AttnShape<KT, D>::NIT], u32x4 (&vr)[AttnShape<KT, D>::NIT],
                                          float (&ksc)[AttnShape<KT, D>::NIT], float (&vsc)[AttnShape<KT, D>::NIT]) {
  typedef AttnShape<KT, D> S;
  constexpr int EK = S::EK, LPK = S::LPK, KPI = S::KPI, NIT = S::NIT;
  const int wave = st >> 6, lane = st & 63;
  const size_t hrow = ((size_t)it.b * a.nh + it.j) * a.cap;  // the head's first cache row
  const size_t head = hrow * D;
  const uint32_t bytes = (uint32_t)((size_t)a.B * a.nh * a.cap * D * sizeof(KT));
  const rsrc_t rk = make_rsrc(L.k, bytes), rv = make_rsrc(L.v, bytes);
  const int e0 = (lane % LPK) * EK;
#pragma unroll
  for (int i = 0; i < NIT; ++i) {
    const int key = it.cc * kStackChunk + (i * NS + wave) * KPI + lane / LPK;
    const bool past = key < len && key < a.cap && key < (it.cc + 1) * kStackChunk;
    const uint32_t off = past ? (uint32_t)((head + (size_t)key * D + e0) * sizeof(KT)) : kOutOfRange;
    kr[i] = __builtin_amdgcn_raw_buffer_load_b128(rk, off, 0, 0);
    vr[i] = __builtin_amdgcn_raw_buffer_load_b128(rv, off, 0, 0);
    ksc[i] = vsc[i] = 0.f;
    if constexpr (sizeof(KT) == 1) {
      if (past) {
        ksc[i] = (float)__builtin_bit_cast(half_t, static_cast<const uint16_t*>(L.ks)[hrow + key]);
        vsc[i] = (float)__builtin_bit_cast(half_t, static_cast<const uint16_t*>(L.vs)[hrow + key]);
      }
    }
  }
}

// Largest value over aligned groups of G lanes; every lane gets its group's maximum.
template <int G> __device__ __forceinline__ float group_max(float v) {
#pragma unroll
  for (int off = G / 2; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, kWave));
  return v;
}

// One item's partial: scores of q against the chunk's rows (the past rows in kr, vr from
// attn_load, the new row at position len from this launch's tagged K/V), wave-reduced max and sum,
// the exp-weighted V sum; (max, sum, acc[D]) is stored tagged for the workgroup that merges the
// (sequence, head). With an int8 cache (KT int8) the item that holds the new row quantizes it
// (one fp16 scale per row: the row's amax over its lanes, the quantizer rule of i8_code), stores
// the codes and scales into the cache for later launches, and attends over the dequantized row.
template <typename KT, int D>
__device__ __forceinline__ bool attn_partial(Ctl& c, const StackArgs& a, uint32_t& sb, const StackLayer& L, int len,
                                             const AttnItem& ai, uint32_t tag_q, uint32_t tag_part, float* s_acc, int st,
                                             u32x4 (&kr)[AttnShape<KT, D>::NIT], u32x4 (&vr)[AttnShape<KT, D>::NIT],
                                             float (&ksc)[AttnShape<KT, D>::NIT], float (&vsc)[AttnShape<KT, D>::NIT]) {
  typedef AttnShape<KT, D> S;
  constexpr int EK = S::EK, LPK = S::LPK, KPI = S::KPI, NIT = S::NIT;
  const float kNeg = -1e30f;
  const int cc = ai.cc, j = ai.j, b = ai.b;
  int nkeys = len + 1;
  if (nkeys > a.cap) nkeys = a.cap;
  const int wave = st >> 6, lane = st & 63;
  const int H = a.nh * D;
  const int e0 = (lane % LPK) * EK;
  // q of this head, this lane's EK elements
  const rsrc_t rq = make_rsrc(a.q, (uint32_t)(a.B * H * 8));
  float qv[EK];
  if (!poll_lane<EK>(c, a, rq, (uint32_t)(b * H + j * D + e0), tag_q, qv)) return false;
  const float qs = 1.4426950408889634f / sqrtf((float)D);  // log2(e)/sqrt(d): scores feed exp2
#pragma unroll
  for (int e = 0; e < EK; ++e) qv[e] *= qs;
  // the new row (position len) of this launch
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    const int key = cc * kStackChunk + (it * NS + wave) * KPI + lane / LPK;
    if (key == len && key < a.cap) {
      const rsrc_t rkn = make_rsrc(a.knew, (uint32_t)(a.B * H * 8)), rvn = make_rsrc(a.vnew, (uint32_t)(a.B * H * 8));
      if constexpr (sizeof(KT) == 1) {
        // the key's LPK lanes hold its D values: amax over them, the row scale (from amax / 127 in
        // double, as the quantizer rounds it), the codes as rint(x * (1 / scale)) in fp32: the
        // product is within two fp32 ulps of x / scale, so a code differs from the double rule's
        // only where x / scale lies that close to a half-integer (the projection's values are
        // fp32 and differ from exact ones by more anyway); K, then V (polled one after the other:
        // both rows' values at once would spill the sync waves' registers)
        const size_t row = ((size_t)b * a.nh + j) * a.cap + key;
        auto quantize = [&](rsrc_t src, void* cache, void* scales, u32x4& codes, float& scale) -> bool {
          float xn[EK];
          if (!poll_lane<EK>(c, a, src, (uint32_t)(b * H + j * D + e0), tag_q, xn)) return false;
          float am = 0.f;
#pragma unroll
          for (int e = 0; e < EK; ++e) am = fmaxf(am, fabsf(xn[e]));
          am = group_max<LPK>(am);
          const uint16_t bits = f64_to_f16_bits_rne((double)am / 127.0);
          const float sv = (float)f16_bits_to_f64(bits);
          const float rs = sv == 0.f ? 0.f : 1.f / sv;
          uint32_t w[4];
#pragma unroll
          for (int h = 0; h < 4; ++h) {
            w[h] = 0u;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const int32_t code = (int32_t)fminf(127.f, fmaxf(-127.f, rintf(xn[4 * h + q] * rs)));
              w[h] |= ((uint32_t)code & 0xffu) << (8 * q);
            }
          }
          codes = u32x4{w[0], w[1], w[2], w[3]};
          scale = sv;
          *reinterpret_cast<u32x4*>(static_cast<int8_t*>(cache) + row * D + e0) = codes;
          if (lane % LPK == 0) static_cast<uint16_t*>(scales)[row] = bits;
          return true;
        };
        if (!quantize(rkn, L.k, L.ks, kr[it], ksc[it])) return false;
        if (!quantize(rvn, L.v, L.vs, vr[it], vsc[it])) return false;
      } else {
        float kn[EK], vn[EK];
        if (!poll_lane<EK>(c, a, rkn, (uint32_t)(b * H + j * D + e0), tag_q, kn)) return false;
        if (!poll_lane<EK>(c, a, rvn, (uint32_t)(b * H + j * D + e0), tag_q, vn)) return false;
        if constexpr (sizeof(KT) == 4) {
          kr[it] = u32x4{__builtin_bit_cast(uint32_t, kn[0]), __builtin_bit_cast(uint32_t, kn[1]),
                         __builtin_bit_cast(uint32_t, kn[2]), __builtin_bit_cast(uint32_t, kn[3])};
          vr[it] = u32x4{__builtin_bit_cast(uint32_t, vn[0]), __builtin_bit_cast(uint32_t, vn[1]),
                         __builtin_bit_cast(uint32_t, vn[2]), __builtin_bit_cast(uint32_t, vn[3])};
        } else {
          kr[it] = u32x4{pack16<KT>(kn[0], kn[1]), pack16<KT>(kn[2], kn[3]), pack16<KT>(kn[4], kn[5]),
                         pack16<KT>(kn[6], kn[7])};
          vr[it] = u32x4{pack16<KT>(vn[0], vn[1]), pack16<KT>(vn[2], vn[3]), pack16<KT>(vn[4], vn[5]),
                         pack16<KT>(vn[6], vn[7])};
        }
      }
    }
  }

  float sc[NIT];
  bool valid[NIT];
  float m = kNeg;
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    const int key = cc * kStackChunk + (it * NS + wave) * KPI + lane / LPK;
    valid[it] = key < nkeys && key < (cc + 1) * kStackChunk;
    float p = 0.f;
    if constexpr (sizeof(KT) == 4) {
      p = qv[0] * as_f32(kr[it].x) + qv[1] * as_f32(kr[it].y) + qv[2] * as_f32(kr[it].z) + qv[3] * as_f32(kr[it].w);
    } else if constexpr (sizeof(KT) == 2) {
      const uint32_t wv[4] = {kr[it].x, kr[it].y, kr[it].z, kr[it].w};
#pragma unroll
      for (int h = 0; h < 4; ++h) p += qv[2 * h] * lo16<KT>(wv[h]) + qv[2 * h + 1] * hi16<KT>(wv[h]);
    } else {
      const uint32_t wv[4] = {kr[it].x, kr[it].y, kr[it].z, kr[it].w};
#pragma unroll
      for (int h = 0; h < 4; ++h)
#pragma unroll
        for (int q = 0; q < 4; ++q) p += qv[4 * h + q] * i8_at(wv[h], q);
      p *= ksc[it];
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
    if constexpr (sizeof(KT) == 4) {
      acc[0] += p * as_f32(vr[it].x);
      acc[1] += p * as_f32(vr[it].y);
      acc[2] += p * as_f32(vr[it].z);
      acc[3] += p * as_f32(vr[it].w);
    } else if constexpr (sizeof(KT) == 2) {
      const uint32_t wv[4] = {vr[it].x, vr[it].y, vr[it].z, vr[it].w};
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        acc[2 * h] += p * lo16<KT>(wv[h]);
        acc[2 * h + 1] += p * hi16<KT>(wv[h]);
      }
    } else {
      const float pv = p * vsc[it];
      const uint32_t wv[4] = {vr[it].x, vr[it].y, vr[it].z, vr[it].w};
#pragma unroll
      for (int h = 0; h < 4; ++h)
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[4 * h + q] += pv * i8_at(wv[h], q);
    }
  }
#pragma unroll
  for (int off = LPK; off < kWave; off <<= 1) {
    l += __shfl_xor(l, off, kWave);
#pragma unroll
    for (int e = 0; e < EK; ++e) acc[e] += __shfl_xor(acc[e], off, kWave);
  }
  if (!sync_bar(c, a, sb, st)) return false;  // the scratch of a previous item is free
  if (lane < LPK) {
#pragma unroll
    for (int e = 0; e < EK; ++e) s_acc[wave * D + e0 + e] = acc[e];
    if (lane == 0) {
      c.m[wave] = m;
      c.l[wave] = l;
    }
  }
  if (!sync_bar(c, a, sb, st)) return false;
  float M = kNeg;
#pragma unroll
  for (int wv = 0; wv < NS; ++wv) M = fmaxf(M, c.m[wv]);
  float f[NS];
#pragma unroll
  for (int wv = 0; wv < NS; ++wv) f[wv] = c.l[wv] > 0.f ? exp2f(c.m[wv] - M) : 0.f;
  const size_t pbase = ((size_t)b * a.nh + j) * a.nchunk;
  const rsrc_t rp = make_rsrc(a.part, (uint32_t)((size_t)a.B * a.nh * a.nchunk * (D + 2) * 8));
  if (st < D) {
    float v = 0.f;
#pragma unroll
    for (int wv = 0; wv < NS; ++wv) v += f[wv] * s_acc[wv * D + st];
    tstore(rp, (uint32_t)((pbase + cc) * (D + 2) + 2 + st), v, tag_part);
  }
  if (st == 0) {
    float Ls = 0.f;
#pragma unroll
    for (int wv = 0; wv < NS; ++wv) Ls += f[wv] * c.l[wv];
    tstore(rp, (uint32_t)((pbase + cc) * (D + 2)), M, tag_part);
    tstore(rp, (uint32_t)((pbase + cc) * (D + 2) + 1), Ls, tag_part);
  }
  return true;
}

// Merge of one (sequence b, head j): every chunk's partial (log-sum-exp) into ctx, rounded to AT
// as the per-layer path stores it.
template <typename AT, int D>
__device__ __forceinline__ bool attn_merge(Ctl& c, const StackArgs& a, uint32_t& sb, const int32_t* lens, int b, int j,
                                           uint32_t tag_part, uint32_t tag_ctx, float* s_part, int st) {
  const float kNeg = -1e30f;
  int nkeys = lens[b] + 1;
  if (nkeys > a.cap) nkeys = a.cap;
  const int nvalid = (nkeys + kStackChunk - 1) / kStackChunk;
  const int H = a.nh * D;
  const size_t pbase = ((size_t)b * a.nh + j) * a.nchunk;
  if (!sync_bar(c, a, sb, st)) return false;  // s_part (LDS) of a previous merge is free
  if (!poll_range(c, a, a.part + pbase * (D + 2), nvalid * (D + 2), tag_part, st,
                  [&](int i, float v) { s_part[i] = v; }))
    return false;
  if (!sync_bar(c, a, sb, st)) return false;
  if (st < D) {
    float MM = kNeg;
    for (int ci = 0; ci < nvalid; ++ci) MM = fmaxf(MM, s_part[ci * (D + 2)]);
    float Lsum = 0.f, Acc = 0.f;
    for (int ci = 0; ci < nvalid; ++ci) {
      const float* pc = s_part + ci * (D + 2);
      const float wgt = pc[1] > 0.f ? exp2f(pc[0] - MM) : 0.f;
      Lsum += wgt * pc[1];
      Acc += wgt * pc[2 + st];
    }
    const rsrc_t rc = make_rsrc(a.ctx, (uint32_t)(a.B * H * 8));
    tstore(rc, (uint32_t)(b * H + j * D + st), (float)(AT)(Acc / Lsum), tag_ctx);
  }
  return true;
}

// gamma and beta of a LayerNorm (K values of AT each) into LDS at dst (gamma, then beta) by
// direct-to-LDS loads, 1 KB per wave instruction, so that no register waits for them: the phase
// they are issued in hides their latency. K * sizeof(AT) is a whole number of KB (hidden is a
// multiple of the 1 KB weight slice's element count).
template <typename AT>
__device__ __forceinline__ void prefetch_ln(const void* gam, const void* beta, int K, AT* dst, int st) {
  const uint32_t bytes = (uint32_t)K * (uint32_t)sizeof(AT);
  const int nkb = (int)(bytes >> 10);
  const int wave = __builtin_amdgcn_readfirstlane(st >> 6), lane = st & 63;
  const rsrc_t rg = make_rsrc(gam, bytes), rb = make_rsrc(beta, bytes);
  unsigned char* d = reinterpret_cast<unsigned char*>(dst);
  for (int k = wave; k < 2 * nkb; k += NS) {
    const bool second = k >= nkb;
    const uint32_t off = (uint32_t)((second ? k - nkb : k) * 1024 + lane * 16);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(second ? rb : rg, lds_ptr(d + k * 1024), 16, off, 0, 0, 0);
  }
}

// ------------------------------------------------------------------ sync waves: the phase loop
template <typename WT, typename AT, int BM, int D, bool KV8>
__device__ __forceinline__ void sync_side(const StackArgs& a, Ctl& c, unsigned char* smem, int g, int st_in,
                                          uint32_t launch) {
  typedef typename WTraits<WT>::LT LT;
  LT* act = reinterpret_cast<LT*>(smem);
  float* raw = reinterpret_cast<float*>(smem + a.lds.raw);
  AT* lnp1 = reinterpret_cast<AT*>(smem + a.lds.lnp);  // LN1's (or the LM head's) gamma, then beta
  AT* lnp2 = lnp1 + 2 * a.H;                            // LN2's
  float* slots = reinterpret_cast<float*>(smem + a.lds.slots);
  half_t* scl = reinterpret_cast<half_t*>(smem + a.lds.scales);
  float* res_x2 = reinterpret_cast<float*>(smem + a.lds.res);        // this workgroup's x2 rows
  float* res_y = res_x2 + a.lds.res_n;                                  // and its layer-output rows
  float* s_acc = reinterpret_cast<float*>(smem);                       // attention: NS x D floats
  float* s_part = reinterpret_cast<float*>(smem) + NS * D;             // merge: nchunk x (D + 2) floats
  const int H = a.H, F = a.F, B = a.B, G = a.G;
  // Thread indices are re-derived through an opaque copy at every phase: otherwise the compiler
  // hoists every per-thread address of every phase out of the layer loop and keeps them all live.
  int st = st_in;
  auto fresh = [&]() {
    int t = st_in;
    asm volatile("" : "+v"(t));
    st = t;
  };
  uint32_t sb = 0;
  typedef typename std::conditional<KV8, int8_t, AT>::type KT;  // the cache's element type
  typedef AttnShape<KT, D> AS;
  u32x4 kr[AS::NIT], vr[AS::NIT];    // the past rows of the current attention item
  float ksc[AS::NIT], vsc[AS::NIT];  // and their row scales (an int8 cache)

  // LayerNorm of the B rows of H into act with the gamma and beta prefetched at gb, from `plain` (the
  // caller's input) when given, else from the tagged values at `tagged`: in registers when the rows
  // fit, else through LDS
  auto layer_norm = [&](const AT* gb, const void* plain, const uint2* tagged, uint32_t tag)
                        __attribute__((always_inline)) -> bool {
    if (B * H <= 2 * NT * kLnPairs)
      return stage_ln_regs<LT, AT, BM, kLnPairs>(c, a, sb, B, H, gb, act, st, plain, tagged, tag);
    return stage_ln<LT, AT, BM>(c, a, sb, B, H, act, raw, gb, st, [&]() {
      if (plain) {
        load_rows_plain<AT>(plain, B, H, raw, st);
        return true;
      }
      return poll_range<kPollWide>(c, a, tagged, B * H, tag, st, [&](int i, float v) { raw[i] = v; });
    });
  };

  // per-workgroup row tiles of each projection (the same split the workers use)
  const int rq = stack_tile_rows(3 * H, G, false), ro = stack_tile_rows(H, G, false), r1 = stack_tile_rows(F, G, true);
  const int q0 = min(3 * H, g * rq), nq = min(3 * H, q0 + rq) - q0;
  const int o0 = min(H, g * ro), no = min(H, o0 + ro) - o0;
  const int f0 = min(F, g * r1), nf = min(F, f0 + r1) - f0;
  const int y0 = o0, ny = no;

  auto row_sum = [&](int rl, int b) {
    const float* p = slots + rl * NWK * BM + b;
    float s = 0.f;
#pragma unroll
    for (int w = 0; w < NWK; ++w) s += p[w * BM];
    return s;
  };
  // Epilogue operands of this thread's first row are requested when its phase begins, so that
  // their memory latency (long while the workers stream) passes during the staging and the
  // workers' products instead of after them; later rows (t >= NT) load in the loop.
  auto pre_ld = [&](const void* bias, int r0, int nr) { return st < nr * B ? ldraw<AT>(bias, r0 + st / B) : 0u; };
  auto clear_slots = [&](int nr) {
    for (int i = st; i < nr * NWK * BM; i += NT) slots[i] = 0.f;
  };
  auto zero_rows = [&](int K) {  // activation rows past B
    for (int i = B * K + st; i < BM * K; i += NT) act[i] = (LT)0.f;
  };
  // publish the staged activation of phase `seq`, request the phase's epilogue operands (`issue`:
  // their loads queue behind the weight stream, which the sync waves wait out anyway), then wait for
  // every worker to finish the phase
  auto hand_over = [&](uint32_t seq, auto issue) -> bool {
    // this wave's LayerNorm prefetch of the previous phase has landed in LDS before the barrier
    // (its later loads, the staging polls, have already been waited for)
    wait_vm_at_most<0>();
    if (!sync_bar(c, a, sb, st)) return false;
    if (st == 0) lds_st(&c.act_ready, seq + 1u);
    issue();
    bool ok = spin_until(c, a, [&] {
      bool all = true;
#pragma unroll
      for (int w = 0; w < NWK; ++w) all = all && lds_ld(&c.done[w]) >= seq + 1u;
      return all;
    });
    asm volatile("" ::: "memory");
    return ok;
  };

  prefetch_ln<AT>(reinterpret_cast<const StackLayer*>(smem + a.lds.layers)[0].ln1_g,
                  reinterpret_cast<const StackLayer*>(smem + a.lds.layers)[0].ln1_b, H, lnp1, st);
  wait_vm_at_most<0>();
  if (!sync_bar(c, a, sb, st)) return;
  for (int l = 0; l < a.n_layers; ++l) {
    const StackLayer& L = reinterpret_cast<const StackLayer*>(smem + a.lds.layers)[l];
    const int32_t* lens = reinterpret_cast<const int32_t*>(smem + a.lds.lens) + l * 4;  // d_len[b] at launch
    const bool last = l == a.n_layers - 1;
    const uint32_t seq0 = (uint32_t)l * 4u;
    const uint32_t t_q = stack_tag(launch, l, TAG_Q), t_part = stack_tag(launch, l, TAG_PART);
    const uint32_t t_ctx = stack_tag(launch, l, TAG_CTX), t_x2 = stack_tag(launch, l, TAG_X2);
    const uint32_t t_f = stack_tag(launch, l, TAG_F), t_y = stack_tag(launch, l, TAG_Y);

    // attention items of this layer (chunks with keys, over the longest sequence)
    int nvmax = 1;
    for (int b = 0; b < B; ++b) nvmax = max(nvmax, attn_nvalid(a, lens[b]));
    const int nitems = B * a.nh * nvmax;

    // ---- region 1: LN1 + QKV + bias; q, k, v tagged; k, v also into the cache row d_len[b]
    fresh();
    uint32_t pre_q = 0u;
    const int pre_pos = lens[st % B];
    if (!sync_bar(c, a, sb, st)) return;  // the previous epilogue's slot reads are done
    clear_slots(nq);
    if constexpr (sizeof(WT) == 1) stage_scales(L.s_qkv, q0, nq, H, a.group, scl, st);
    if (!layer_norm(lnp1, l == 0 ? a.x : nullptr, a.ybuf, l == 0 ? 0u : stack_tag(launch, l - 1, TAG_Y)))
      return;
    if (!hand_over(seq0, [&] {
          pre_q = pre_ld(L.b_qkv, q0, nq);
          prefetch_ln<AT>(L.ln2_g, L.ln2_b, H, lnp2, st);  // LN2 reads it after the next hand-over
        }))
      return;
    {
      const rsrc_t rqo = make_rsrc(a.q, (uint32_t)(B * H * 8));
      const rsrc_t rkn = make_rsrc(a.knew, (uint32_t)(B * H * 8)), rvn = make_rsrc(a.vnew, (uint32_t)(B * H * 8));
      const uint32_t cache_bytes = (uint32_t)((size_t)B * a.nh * a.cap * D * sizeof(AT));
      const rsrc_t rk = make_rsrc(L.k, cache_bytes), rv = make_rsrc(L.v, cache_bytes);
      for (int t = st; t < nq * B; t += NT) {
        const int rl = t / B, b = t - rl * B, n = q0 + rl;
        const float z = row_sum(rl, b) + (t == st ? cvraw<AT>(pre_q) : ldp<AT>(L.b_qkv, n));
        if (n < H) {
          tstore(rqo, (uint32_t)(b * H + n), z, t_q);
        } else {
          const int m = n < 2 * H ? n - H : n - 2 * H, j = m / D, e = m - j * D;
          if constexpr (KV8) {
            // the attention item of the new row quantizes it and writes the cache
            tstore(n < 2 * H ? rkn : rvn, (uint32_t)(b * H + m), z, t_q);
          } else {
            const float zr = (float)(AT)z;  // the value the cache holds
            tstore(n < 2 * H ? rkn : rvn, (uint32_t)(b * H + m), zr, t_q);
            const int pos = t == st ? pre_pos : lens[b];
            if (pos >= 0 && pos < a.cap)
              coh_st_act<AT>(n < 2 * H ? rk : rv, (uint32_t)((((size_t)b * a.nh + j) * a.cap + pos) * D + e), z);
          }
        }
      }
    }

    // ---- region 2: attention over the cache; first every partial of this workgroup, then the
    // merges it owns, so that no merge waits on a partial queued behind it. Items go to workgroups
    // in order (workgroup g takes items g, g + G, ...) and merges from the last workgroup down, so
    // that the merges land on the workgroups with the fewest items (or none).
    fresh();
    for (int item = g; item < nitems; item += G) {
      const AttnItem it = attn_item(a, lens, nvmax, item);
      if (!it.valid) continue;
      attn_load<KT, D>(a, L, lens[it.b], it, st, kr, vr, ksc, vsc);
      if (!attn_partial<KT, D>(c, a, sb, L, lens[it.b], it, t_q, t_part, s_acc, st, kr, vr, ksc, vsc)) return;
    }
    for (int m = G - 1 - g; m < B * a.nh; m += G)
      if (!attn_merge<AT, D>(c, a, sb, lens, m / a.nh, m % a.nh, t_part, t_ctx, s_part, st)) return;

    // ---- output projection + bias + residual: x2 = x + Wo ctx + bo
    fresh();
    uint32_t pre_o = 0u;
    if (!sync_bar(c, a, sb, st)) return;  // the attention scratch (same LDS) and the slots are free
    clear_slots(no);
    if constexpr (sizeof(WT) == 1) stage_scales(L.s_o, o0, no, H, a.group, scl, st);
    zero_rows(H);
    if (!poll_range(c, a, a.ctx, B * H, t_ctx, st, [&](int i, float v) { act[i] = (LT)v; })) return;
    if (!hand_over(seq0 + 1u, [&] { pre_o = pre_ld(L.b_o, o0, no); })) return;
    {
      const rsrc_t rx2 = make_rsrc(a.x2, (uint32_t)(B * H * 8));
      for (int t = st; t < no * B; t += NT) {
        const int rl = t / B, b = t - rl * B, n = o0 + rl;
        const float z = row_sum(rl, b) + (t == st ? cvraw<AT>(pre_o) : ldp<AT>(L.b_o, n));
        const float xr = l == 0 ? ldp<AT>(a.x, b * H + n) : res_y[t];
        const float v = xr + z;
        res_x2[t] = v;
        tstore(rx2, (uint32_t)(b * H + n), v, t_x2);
      }
    }

    // ---- region 3: LN2 + FF1 + bias + GeLU
    fresh();
    uint32_t pre_f0 = 0u, pre_f1 = 0u;
    if (!sync_bar(c, a, sb, st)) return;  // the previous epilogue's slot reads are done
    clear_slots(nf);
    if constexpr (sizeof(WT) == 1) stage_scales(L.s_ff1, f0, nf, H, a.group_mlp, scl, st);
    if (!layer_norm(lnp2, nullptr, a.x2, t_x2)) return;
    if (!hand_over(seq0 + 2u, [&] {
          // the next layer's LN1 (or the LM head's final LayerNorm) reads it after the next hand-over
          if (!last)
            prefetch_ln<AT>(reinterpret_cast<const StackLayer*>(smem + a.lds.layers)[l + 1].ln1_g,
                            reinterpret_cast<const StackLayer*>(smem + a.lds.layers)[l + 1].ln1_b, H, lnp1, st);
          else if (a.head)
            prefetch_ln<AT>(a.head_g, a.head_b, H, lnp1, st);
          // fp16: this thread's first pair of rows; otherwise its first row
          pre_f0 = sizeof(AT) == 2 ? (st < (nf / 2) * B ? ldraw<AT>(L.b_ff1, f0 + 2 * (st / B)) : 0u)
                                   : pre_ld(L.b_ff1, f0, nf);
          pre_f1 = sizeof(AT) == 2 && st < (nf / 2) * B ? ldraw<AT>(L.b_ff1, f0 + 2 * (st / B) + 1) : 0u;
        }))
      return;
    {
      const rsrc_t rf = make_rsrc(a.f, (uint32_t)(B * F * 8));
      if constexpr (sizeof(AT) == 2) {
        // 16-bit f: pairs of rows (f0 and nf are even) in one tagged store each, half the bytes the
        // FF2 staging polls
        for (int t = st; t < (nf / 2) * B; t += NT) {
          const int pl = t / B, b = t - pl * B, rl = 2 * pl, n = f0 + rl;
          const float b0 = t == st ? cvraw<AT>(pre_f0) : ldp<AT>(L.b_ff1, n);
          const float b1 = t == st ? cvraw<AT>(pre_f1) : ldp<AT>(L.b_ff1, n + 1);
          tstore_pair<AT>(rf, (uint32_t)((b * F + n) / 2), gelu(row_sum(rl, b) + b0, a.gelu_tanh != 0),
                          gelu(row_sum(rl + 1, b) + b1, a.gelu_tanh != 0), t_f);
        }
      } else {
        for (int t = st; t < nf * B; t += NT) {
          const int rl = t / B, b = t - rl * B, n = f0 + rl;
          const float z = row_sum(rl, b) + (t == st ? cvraw<AT>(pre_f0) : ldp<AT>(L.b_ff1, n));
          tstore(rf, (uint32_t)(b * F + n), (float)(AT)gelu(z, a.gelu_tanh != 0), t_f);
        }
      }
    }

    // ---- region 4: FF2 + bias + residual: y = x2 + W2 f + b2
    fresh();
    uint32_t pre_y = 0u;
    if (!sync_bar(c, a, sb, st)) return;  // the LayerNorm rows (same LDS) and the slots are free
    clear_slots(ny);
    if constexpr (sizeof(WT) == 1) stage_scales(L.s_ff2, y0, ny, F, a.group_mlp, scl, st);
    zero_rows(F);
    if constexpr (sizeof(AT) == 2) {
      // pair i holds f elements 2i and 2i + 1 of the [B][F] rows, already in the staged type
      static_assert(__is_same(LT, AT), "16-bit activations are staged in their own type");
      if (!poll_range<kPollWide>(c, a, a.f, B * F / 2, t_f, st, [&](int i, float v) {
            reinterpret_cast<uint32_t*>(act)[i] = __builtin_bit_cast(uint32_t, v);
          }))
        return;
    } else if (!poll_range(c, a, a.f, B * F, t_f, st, [&](int i, float v) { act[i] = (LT)v; })) {
      return;
    }
    if (!hand_over(seq0 + 3u, [&] { pre_y = pre_ld(L.b_ff2, y0, ny); })) return;
    {
      const rsrc_t ryt = make_rsrc(a.ybuf, (uint32_t)(B * H * 8));
      const rsrc_t ry = make_rsrc(a.y, (uint32_t)(B * H * sizeof(AT)));
      for (int t = st; t < ny * B; t += NT) {
        const int rl = t / B, b = t - rl * B, n = y0 + rl;
        const float z = row_sum(rl, b) + (t == st ? cvraw<AT>(pre_y) : ldp<AT>(L.b_ff2, n));
        const float v = (float)(AT)(res_x2[t] + z);
        res_y[t] = v;
        if (last) coh_st_act<AT>(ry, (uint32_t)(b * H + n), v);
        if (!last || a.head) tstore(ryt, (uint32_t)(b * H + n), v, t_y);
      }
    }
  }

  // ---- the LM head: final LayerNorm of the last layer's output, logits = W_vocab h, greedy choice
  uint64_t* keys = reinterpret_cast<uint64_t*>(a.sync + kSyncArgmax) + (launch & 1u) * kStackMaxBatch;
  if (a.head) {
    fresh();
    const int rv = stack_tile_rows(a.V, G, false);
    const int v0 = min(a.V, g * rv), nv = min(a.V, v0 + rv) - v0;
    if (!sync_bar(c, a, sb, st)) return;  // the previous epilogue's slot reads are done
    clear_slots(nv);
    if constexpr (sizeof(WT) == 1) stage_scales(a.head_s, v0, nv, H, a.group, scl, st);
    const uint32_t t_last = stack_tag(launch, a.n_layers - 1, TAG_Y);
    if (!layer_norm(lnp1, nullptr, a.ybuf, t_last)) return;
    if (!hand_over(4u * (uint32_t)a.n_layers, [] {})) return;
    // each logit as a 64-bit key that orders like (value, -index): the order-preserving bits of the
    // float above the inverted row index, so the largest key is the largest logit at its smallest
    // index (both zeros count as +0)
    uint64_t best[BM];
#pragma unroll
    for (int b = 0; b < BM; ++b) best[b] = 0ull;
    for (int t = st; t < nv * B; t += NT) {
      const int rl = t / B, b = t - rl * B, n = v0 + rl;
      const float z = row_sum(rl, b);
      if (a.logits) a.logits[(size_t)b * a.V + n] = z;
      const uint32_t u = z == 0.f ? 0u : __builtin_bit_cast(uint32_t, z);
      const uint32_t ord = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
      const uint64_t key = ((uint64_t)ord << 32) | (uint64_t)(0xffffffffu - (uint32_t)n);
#pragma unroll
      for (int bb = 0; bb < BM; ++bb)
        if (bb == b && key > best[bb]) best[bb] = key;
    }
    // the workgroup's largest key per sequence (LDS atomics), then one device atomic per sequence
    if (st < BM) c.best[st] = 0ull;
    if (!sync_bar(c, a, sb, st)) return;
#pragma unroll
    for (int b = 0; b < BM; ++b)
      if (b < B && best[b] != 0ull) __hip_atomic_fetch_max(&c.best[b], best[b], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    if (!sync_bar(c, a, sb, st)) return;
    if (st < B && nv > 0)
      (void)__hip_atomic_fetch_max(keys + st, c.best[st], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }

  // every store of this workgroup is complete; the last workgroup out advances the cache lengths
  // (every other one has finished reading them) and the launch counter, and hands out the greedy
  // choices (every workgroup's argmax key is in, each added before its workgroup counted itself out)
  wait_vm_at_most<0>();
  if (!sync_bar(c, a, sb, st)) return;
  if (st == 0) {
    const uint32_t out = __hip_atomic_fetch_add(a.sync + kSyncExit, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (out == (uint32_t)G - 1) {
      if (a.head)
        for (int b = 0; b < B; ++b) {
          const uint64_t key = __hip_atomic_load(keys + b, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          a.tokens[b] = (int32_t)(0xffffffffu - (uint32_t)key);
        }
      for (int l = 0; l < a.n_layers; ++l)
        for (int b = 0; b < B; ++b) {
          int32_t* dl = a.layers[l].d_len + b;
          const int v = __hip_atomic_load(dl, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          if (v + 1 <= a.cap) __hip_atomic_store(dl, v + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      __hip_atomic_store(a.sync + kSyncExit, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(a.sync + kSyncLaunch, (launch + 1u) & kLaunchMask, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}
}  // namespace

// ------------------------------------------------------------------ the persistent kernel
template <typename WT, typename AT, int BM, int D, int GS, bool KV8>
__global__ __launch_bounds__(kStackThreads, 1) void stack_decode_kernel(const StackArgs a) {
  typedef typename WTraits<WT>::LT LT;
  extern __shared__ __align__(16) unsigned char smem[];
  __shared__ Ctl c;
  uint64_t* wtab = reinterpret_cast<uint64_t*>(smem + a.lds.wtab);
  for (int i = threadIdx.x; i < a.n_layers * 4; i += kStackThreads)
    wtab[i] = reinterpret_cast<uint64_t>(phase_w(a.layers[i >> 2], i & 3));
  if (threadIdx.x == 0) wtab[a.n_layers * 4] = reinterpret_cast<uint64_t>(a.head_w);
  // The layer table and the cache lengths in LDS: the sync waves read them inside their chain,
  // where a global load would wait behind the CU's queue of weight loads.
  static_assert(sizeof(StackLayer) % 4 == 0, "layer table in words");
  {
    constexpr int kWords = (int)(sizeof(StackLayer) / 4);
    uint32_t* dst = reinterpret_cast<uint32_t*>(smem + a.lds.layers);
    const uint32_t* src = reinterpret_cast<const uint32_t*>(a.layers);
    for (int i = threadIdx.x; i < a.n_layers * kWords; i += kStackThreads) dst[i] = src[i];
    int32_t* lens = reinterpret_cast<int32_t*>(smem + a.lds.lens);
    for (int i = threadIdx.x; i < a.n_layers * 4; i += kStackThreads)
      lens[i] = (i & 3) < a.B ? a.layers[i >> 2].d_len[i & 3] : 0;
  }
  if (threadIdx.x == 0) {
    c.act_ready = 0u;
    for (int w = 0; w < NWK; ++w) c.done[w] = 0u;
    c.sbar = 0u;
    c.launch = __hip_atomic_load(a.sync + kSyncLaunch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    // an earlier launch of this stack timed out and the state has not been reset yet: this launch
    // would run under that launch's number, so it leaves before storing anything
    c.abort = __hip_atomic_load(a.sync + kSyncError, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u ? 1u : 0u;
  }
  __syncthreads();
  if (c.abort != 0u) return;
  // the argmax keys of the next launch (the other parity) start at zero; no workgroup of this
  // launch touches them
  if (blockIdx.x == 0 && threadIdx.x < kStackMaxBatch) {
    uint64_t* next = reinterpret_cast<uint64_t*>(a.sync + kSyncArgmax) + ((c.launch + 1u) & 1u) * kStackMaxBatch;
    __hip_atomic_store(next + threadIdx.x, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int lane = threadIdx.x & 63;
  if (wave < NS) {
    const uint32_t launch = __builtin_amdgcn_readfirstlane(c.launch);
    sync_side<WT, AT, BM, D, KV8>(a, c, smem, blockIdx.x, (int)threadIdx.x, launch);
    if (lds_ld(&c.abort) == 0u) return;
    raise_abort(c, a.sync);  // a failed sync wave releases the workers
  } else {
    worker<WT, BM, GS>(a, c, reinterpret_cast<const LT*>(smem), reinterpret_cast<float*>(smem + a.lds.slots),
                   reinterpret_cast<const half_t*>(smem + a.lds.scales), wtab, blockIdx.x, wave - NS, lane);
  }
}

// ------------------------------------------------------------------ host-side launch helpers
int stack_rows_per_wg(int H, int F, int V, int G) {
  int r = (3 * H + G - 1) / G;
  r = max(r, (H + G - 1) / G);
  r = max(r, stack_tile_rows(F, G, true));
  r = max(r, stack_tile_rows(V, G, false));
  return r;
}

template <typename WT, typename AT, int BM, int D, int GS, bool KV8 = false>
static const void* kernel_ptr() {
  return reinterpret_cast<const void*>(&stack_decode_kernel<WT, AT, BM, D, GS, KV8>);
}

// Slices per worker group: 5 when every row of the stack's products (K = hidden or ffn) holds a
// multiple of 5 slices (the GPT-Neo-2.7B and 13B widths), else 1.
int stack_group_slices(Dt wdt, int H, int F) {
  const int sl = wdt == F32 ? 256 : (wdt == I8 ? 1024 : 512);
  return (H / sl) % 5 == 0 && (F / sl) % 5 == 0 ? 5 : 1;
}

// Instantiated variants: batch tiles of 1 or 4 rows (2..4 sequences use the 4-row tile), head_dim 64
// or 128, groups of 1 or 5 slices; an int8 cache with fp16 or bf16 activations.
static const void* pick(Dt wdt, Dt adt, bool kv8, int B, int D, int GS) {
  const bool one = B <= 1;
#define DS_PICK_G(WT_, AT_, G_, K_)                                                                           \
  {                                                                                                            \
    if (D == 64) return one ? kernel_ptr<WT_, AT_, 1, 64, G_, K_>() : kernel_ptr<WT_, AT_, 4, 64, G_, K_>();   \
    return one ? kernel_ptr<WT_, AT_, 1, 128, G_, K_>() : kernel_ptr<WT_, AT_, 4, 128, G_, K_>();             \
  }
#define DS_PICK_K(WT_, AT_, K_)              \
  {                                          \
    if (GS == 5) DS_PICK_G(WT_, AT_, 5, K_)  \
    DS_PICK_G(WT_, AT_, 1, K_)               \
  }
#define DS_PICK(WT_, AT_)                         \
  {                                               \
    if (kv8) DS_PICK_K(WT_, AT_, true)            \
    DS_PICK_K(WT_, AT_, false)                    \
  }
  if (kv8 && adt != F16 && adt != BF16) return nullptr;
  if (wdt == F16 && adt == F16) DS_PICK(half_t, half_t)
  if (wdt == I8 && adt == F16) DS_PICK(int8_t, half_t)
  if (wdt == BF16 && adt == BF16) DS_PICK(bf16_t, bf16_t)
  if (wdt == F32 && adt == F32 && one) {
    if (GS == 5) return D == 64 ? kernel_ptr<float, float, 1, 64, 5>() : kernel_ptr<float, float, 1, 128, 5>();
    return D == 64 ? kernel_ptr<float, float, 1, 64, 1>() : kernel_ptr<float, float, 1, 128, 1>();
  }
#undef DS_PICK
#undef DS_PICK_K
#undef DS_PICK_G
  return nullptr;
}

hipError_t stack_max_groups(Dt wdt, Dt adt, bool kv8, int B, int GS, size_t lds, int* groups) {
  // head_dim does not change the register or LDS footprint enough to matter: query d = 128
  const void* k = pick(wdt, adt, kv8, B, 128, GS);
  if (!k) return hipErrorInvalidValue;
  int per_cu = 0, dev = 0;
  hipError_t e = hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k, kStackThreads, lds);
  if (e != hipSuccess) return e;
  if ((e = hipGetDevice(&dev)) != hipSuccess) return e;
  int cus = 0;
  if ((e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess) return e;
  if (per_cu > 1) per_cu = 1;
  *groups = per_cu * cus;
  return hipSuccess;
}

hipError_t launch_stack_decode(Dt wdt, Dt adt, const StackArgs& a, hipStream_t st) {
  const void* k = pick(wdt, adt, a.kv8 != 0, a.B, a.d, stack_group_slices(wdt, a.H, a.F));
  if (!k) return hipErrorInvalidValue;
  hipError_t e = hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)a.lds.total);
  if (e != hipSuccess) return e;
  StackArgs args = a;
  void* params[] = {&args};
  return hipLaunchCooperativeKernel(k, dim3(a.G), dim3(kStackThreads), params, (unsigned)a.lds.total, st);
}

}  // namespace ds
