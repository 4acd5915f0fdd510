// kernels_stack.hip -- persistent decode of a whole layer stack in one launch.
//
// Computes, for every layer in turn, the four fusion regions of one transformer layer described on
// the page "DeepSpeed Inference 内核优化深度解析" (blog.gitcode.com), section 三 3.2 (LN + QKV GeMM +
// bias; attention over the cache with the head transform folded into its addressing; the output
// GeMM with bias and residual; LN + FF1 + bias + GELU; FF2 + bias + residual). Section 三 3.1 puts the
// fusion boundaries where partial results must meet (the all-reduce points); here those are the
// grid-wide barriers between phases.
//
// gfx950 design. One cooperative launch keeps one 16-wave workgroup per CU resident for the whole
// step. Each projection is cut into per-workgroup row tiles; a tile is one contiguous range of the
// row-major matrix, cut into 1 KB "slices" (one 16-byte load per lane of a wave64).
//
// The waves are specialized so that HBM never waits for the step's serial parts:
//  - 12 worker waves own contiguous blocks of each tile and walk the fixed sequence of all their
//    slices of all layers. Each keeps kRing slices in flight in a rotating set of registers: a
//    slice is multiplied with the staged activation (LDS) the moment it is consumed, and its
//    registers at once load the slice kRing places further on, whatever phase or layer that is.
//    Workers issue nothing but these loads, so their in-order load counter only ever waits for
//    the oldest slice; row partial sums go to LDS.
//  - 4 sync waves stage each phase's activation (LayerNorm included), reduce the workers' partial
//    sums, run the epilogues (bias, residual, GeLU, the q/k/v scatter), compute attention over
//    the cache and take the grid barriers.
// So weight streaming continues straight through the barriers, the activation staging and the
// epilogues. Activations that cross workgroups are written and read with sc1 buffer operations
// (at the device coherence point, past the per-XCD L2 copies); barrier arrivals are agent-scope
// atomics spread over 16 counters. Every wait, in LDS or on the grid, is bounded by a wall-clock
// timeout that raises the error flag, after which every wave leaves the kernel.
#include "ds_device.hpp"
#include "ds_stack.hpp"

namespace ds {
namespace {

constexpr int NS = kStackSyncWaves;
constexpr int NT = NS * kWave;             // sync threads
constexpr int NWK = kStackWorkers;
// Weight slices a worker keeps in flight: 24 for fp16 weights and one batch row (24 KB per wave,
// 288 KB per CU), 16 for fp32; variants with four batch rows or int8 weights (two 16-byte
// activation reads per row) keep 12 so that a 128-VGPR wave still holds everything.
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
  int ok;                // grid-barrier outcome, broadcast to the sync waves
  int flag;              // attention: this workgroup completed a (sequence, head)
  float red[NS][8];      // LayerNorm sums: (sum, sum of squares) for up to 4 rows, per wave
  float m[NS], l[NS];    // attention: per-wave max and sum
  int tab[NWK][4][8];    // per worker and phase: the block geometry (see worker_table)
};

// Fields of a worker's phase-table entry.
enum { T_CNT = 0, T_BASE = 1, T_BYTES = 2, T_K = 3, T_SPER = 4, T_RL0 = 5, T_KS0 = 6 };

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

// Spin until pred() holds; false on this workgroup's abort, the grid error flag or a timeout
// (which raises both). Only lane 0 of the wave polls (the other lanes would only add LDS traffic
// that the workers' activation reads queue behind); the outcome is broadcast to the wave.
template <typename Pred>
__device__ __forceinline__ bool spin_until(Ctl& c, const StackArgs& a, Pred pred) {
  int ok = 1;
  if (__lane_id() == 0 && !pred()) {
    const uint64_t t0 = wall_clock64();
    for (;;) {
      __builtin_amdgcn_s_sleep(2);
      if (pred()) break;
      if (lds_ld(&c.abort) != 0u) {
        ok = 0;
        break;
      }
      if (wall_clock64() - t0 > a.timeout_ticks ||
          __hip_atomic_load(a.sync + kSyncError, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u) {
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

// ------------------------------------------------------------------ grid barrier
// Arrive at barrier `epoch` (1, 2, ...): one atomic add per workgroup on its group's counter; the
// last of a group adds to the top counter; the last top arrival publishes the epoch. Then wait for
// the release. Called by one thread after every sync wave's stores have completed.
__device__ __forceinline__ bool grid_arrive_wait(Ctl& c, const StackArgs& a, uint32_t epoch, int g) {
  uint32_t* sync = a.sync;
  const int G = a.G;
  const int ng = G < kSyncGroups ? G : kSyncGroups;
  const int gi = g % ng;
  const uint32_t members = (uint32_t)((G - gi + ng - 1) / ng);
  const uint32_t old = __hip_atomic_fetch_add(sync + kSyncSub + gi * kSyncLine, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (old == epoch * members - 1u) {
    const uint32_t top = __hip_atomic_fetch_add(sync + kSyncTop, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (top == epoch * (uint32_t)ng - 1u) __hip_atomic_store(sync + kSyncFlag, epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  const uint64_t t0 = wall_clock64();
  while (__hip_atomic_load(sync + kSyncFlag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < epoch) {
    if (__hip_atomic_load(sync + kSyncError, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u ||
        lds_ld(&c.abort) != 0u || wall_clock64() - t0 > a.timeout_ticks) {
      raise_abort(c, sync);
      return false;
    }
    __builtin_amdgcn_s_sleep(2);
  }
  return true;
}

// ------------------------------------------------------------------ row tiles
// Phase ph (0 QKV, 1 O, 2 FF1, 3 FF2) of workgroup g: rows [r0, r0+nr) of the [N][K] matrix, one
// contiguous range of nr*K elements cut into slices of SL elements (K is a multiple of SL), so
// slice s lies in tile row s / (K/SL). Worker w owns the contiguous block [s0, s0+cnt).
struct Geo {
  int N, K, r0, nr, s0, cnt;
};

__device__ __forceinline__ Geo phase_geo(const StackArgs& a, int SL, int g, int w, int ph) {
  const int H = a.H, F = a.F, G = a.G;
  Geo p;
  p.N = ph == 0 ? 3 * H : (ph == 2 ? F : H);
  p.K = ph == 3 ? F : H;
  const int rows = (p.N + G - 1) / G;
  p.r0 = min(p.N, g * rows);
  p.nr = min(p.N, p.r0 + rows) - p.r0;
  const int T = p.nr * (p.K / SL);
  const int M = (T + NWK - 1) / NWK;
  p.s0 = min(T, w * M);
  p.cnt = min(T, p.s0 + M) - p.s0;
  return p;
}

__device__ __forceinline__ const void* phase_w(const StackLayer& L, int ph) {
  return ph == 0 ? L.w_qkv : ph == 1 ? L.w_o : ph == 2 ? L.w_ff1 : L.w_ff2;
}
__device__ __forceinline__ const void* phase_s(const StackLayer& L, int ph) {
  return ph == 0 ? L.s_qkv : ph == 1 ? L.s_o : ph == 2 ? L.s_ff1 : L.s_ff2;
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

// Lane p (0..3) of worker w fills the table entry of phase p: slice count, byte offset of the
// block's first slice in the matrix, matrix bytes, K, slices per row, first row and slice-in-row.
template <typename WT>
__device__ __forceinline__ void worker_table(const StackArgs& a, Ctl& c, int g, int w, int lane) {
  constexpr int SL = kWave * WTraits<WT>::E;
  if (lane < 4) {
    const Geo p = phase_geo(a, SL, g, w, lane);
    int* t = c.tab[w][lane];
    const int sper = p.K / SL;
    t[T_CNT] = p.cnt;
    t[T_BASE] = (int)(((size_t)p.r0 * p.K + (size_t)p.s0 * SL) * sizeof(WT));
    t[T_BYTES] = (int)((size_t)p.N * p.K * sizeof(WT));
    t[T_K] = p.K;
    t[T_SPER] = sper;
    t[T_RL0] = p.s0 / sper;
    t[T_KS0] = p.s0 - (p.s0 / sper) * sper;
  }
  wait_lgkm0();
}

__device__ __forceinline__ int tab_ld(const Ctl& c, int w, int ph, int f) {
  return __builtin_amdgcn_readfirstlane(c.tab[w][ph][f]);
}

// Weight-matrix pointer of (layer, phase) from the LDS table, made wave-uniform.
__device__ __forceinline__ const void* wtab_ld(const uint64_t* wtab, int l, int ph) {
  const uint64_t u = wtab[l * 4 + ph];
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)u);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(u >> 32));
  return reinterpret_cast<const void*>(((uint64_t)hi << 32) | lo);
}

template <typename WT, int BM>
__device__ __forceinline__ void worker(const StackArgs& a, Ctl& c, const typename WTraits<WT>::LT* act, float* slots,
                                       const half_t* scl, const uint64_t* wtab, int g, int w, int lane) {
  typedef typename WTraits<WT>::LT LT;
  constexpr int E = WTraits<WT>::E, SL = kWave * E;
  constexpr int kRing = Ring<WT, BM>::value;
  constexpr uint32_t SLB = (uint32_t)(SL * sizeof(WT));  // bytes of one slice
  const int L = a.n_layers;
  worker_table<WT>(a, c, g, w, lane);
  const int per_layer = tab_ld(c, w, 0, T_CNT) + tab_ld(c, w, 1, T_CNT) + tab_ld(c, w, 2, T_CNT) + tab_ld(c, w, 3, T_CNT);
  const int total = L * per_layer;

  // issue cursor: the next slice to load (layer il, phase iph, slice is of icnt)
  int il = 0, iph = 0, is = 0, icnt = tab_ld(c, w, 0, T_CNT);
  while (il < L && icnt == 0) {
    if (++iph == 4) {
      iph = 0;
      ++il;
    }
    icnt = tab_ld(c, w, iph, T_CNT);
  }
  const void* iw = wtab_ld(wtab, il < L ? il : 0, il < L ? iph : 0);
  uint32_t ibytes = (uint32_t)tab_ld(c, w, iph, T_BYTES);
  uint32_t ioff = (uint32_t)tab_ld(c, w, iph, T_BASE);
  const uint32_t voff = (uint32_t)(lane * 16);

  // consume cursor: the next slice to multiply (layer cl, phase cph, slice cs of ccnt)
  int cl = 0, cph = 0, cs = 0, ccnt = tab_ld(c, w, 0, T_CNT);
  int K = tab_ld(c, w, 0, T_K), Sper = tab_ld(c, w, 0, T_SPER);
  int rl = tab_ld(c, w, 0, T_RL0), ks = tab_ld(c, w, 0, T_KS0);
  bool wait_act = true;
  // leave phase (cl, cph) [finished or empty], publishing it, and move to the next non-empty one
  auto c_advance = [&]() {
    for (;;) {
      wait_lgkm0();  // this wave's slot writes are in LDS before the flag says so
      if (lane == 0) lds_st(&c.done[w], (uint32_t)(cl * 4 + cph + 1));
      if (++cph == 4) {
        cph = 0;
        ++cl;
      }
      if (cl >= L) return;
      ccnt = tab_ld(c, w, cph, T_CNT);
      if (ccnt > 0) break;
    }
    cs = 0;
    K = tab_ld(c, w, cph, T_K);
    Sper = tab_ld(c, w, cph, T_SPER);
    rl = tab_ld(c, w, cph, T_RL0);
    ks = tab_ld(c, w, cph, T_KS0);
    wait_act = true;
  };
  if (ccnt == 0) c_advance();

  float acc[BM];
#pragma unroll
  for (int b = 0; b < BM; ++b) acc[b] = 0.f;

  // issue one load: the next slice, or an out-of-range load (reads nothing) past the end
#define DS_ISSUE(dst)                                                                            \
  {                                                                                              \
    const bool live = il < L;                                                                    \
    const rsrc_t r = make_rsrc(iw, ibytes);                                                      \
    dst = __builtin_amdgcn_raw_buffer_load_b128(r, voff, live ? ioff : kOutOfRange, kAuxStream); \
    ioff += SLB;                                                                                 \
    if (live && ++is >= icnt) {                                                                  \
      is = 0;                                                                                    \
      do {                                                                                       \
        if (++iph == 4) {                                                                        \
          iph = 0;                                                                               \
          ++il;                                                                                  \
        }                                                                                        \
        icnt = tab_ld(c, w, iph, T_CNT);                                                         \
      } while (il < L && icnt == 0);                                                             \
      if (il < L) {                                                                              \
        iw = wtab_ld(wtab, il, iph);                                                             \
        ibytes = (uint32_t)tab_ld(c, w, iph, T_BYTES);                                           \
        ioff = (uint32_t)tab_ld(c, w, iph, T_BASE);                                              \
      }                                                                                          \
    }                                                                                            \
  }

  u32x4 ring[kRing];
#pragma unroll
  for (int u = 0; u < kRing; ++u) DS_ISSUE(ring[u])

  bool ok = true;
  for (int pos = 0; pos < total && ok;) {
#pragma unroll
    for (int u = 0; u < kRing; ++u) {
      if (pos < total && ok) {
        // the cursor is wave-uniform; say so, so that its bookkeeping stays in scalar registers
        ks = __builtin_amdgcn_readfirstlane(ks);
        rl = __builtin_amdgcn_readfirstlane(rl);
        cs = __builtin_amdgcn_readfirstlane(cs);
        wait_vm_at_most<kRing - 1>();  // exactly kRing loads are in flight: the oldest has landed
        if (wait_act) {
          const uint32_t need = (uint32_t)(cl * 4 + cph + 1);
          ok = worker_spin(c, a, [&] { return lds_ld(&c.act_ready) >= need; });
          wait_act = false;
        }
        if (ok) {
          const LT* ap = act + ks * SL + lane * E;
          float sc = 1.f;
          if constexpr (sizeof(WT) == 1) sc = (float)scl[rl * (K / a.group) + (ks * SL + lane * E) / a.group];
#pragma unroll
          for (int b = 0; b < BM; ++b) {
            if constexpr (sizeof(WT) == 4) {
              acc[b] = dot4_f32(ring[u], *reinterpret_cast<const float4_t*>(ap + b * K), acc[b]);
            } else if constexpr (sizeof(WT) == 2) {
              acc[b] = dot8_f16(ring[u], *reinterpret_cast<const u32x4*>(ap + b * K), acc[b]);
            } else {
              acc[b] = fmaf(dot16_i8(ring[u], *reinterpret_cast<const u32x4*>(ap + b * K),
                                     *reinterpret_cast<const u32x4*>(ap + b * K + 8)),
                            sc, acc[b]);
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
constexpr int kStageUnroll = 4;  // 16-byte loads a thread has in flight while staging

// Copy B rows of K elements of type IT (written by other workgroups: coherent loads) into LDS as
// LT, zero-filling rows B..BM-1.
template <typename IT, typename LT, int BM>
__device__ __forceinline__ void stage_plain(const void* in, int B, int K, LT* act, int st) {
  constexpr int V = 16 / (int)sizeof(IT);
  const rsrc_t r = make_rsrc(in, (uint32_t)(B * K * sizeof(IT)));
  const int nvec = BM * K / V;
  for (int j0 = st; j0 < nvec; j0 += NT * kStageUnroll) {
    u32x4 raw[kStageUnroll];
#pragma unroll
    for (int u = 0; u < kStageUnroll; ++u) {
      const int j = j0 + u * NT;
      raw[u] = coh_load16(r, j < nvec ? (uint32_t)(j * 16) : kOutOfRange);  // rows past B: zero
    }
#pragma unroll
    for (int u = 0; u < kStageUnroll; ++u) {
      const int j = j0 + u * NT;
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

// LayerNorm B rows (biased variance) into LDS as LT. gamma and beta (this layer's, in AT) are
// loaded as 16-byte vectors before the rows, so their latency hides under the rows' loads, and land
// in LDS next to the fp32 copy of the rows (`raw`); then one reduction of the shifted sums of all
// rows and the normalized rows.
template <typename IT, typename LT, typename AT, int BM>
__device__ __forceinline__ bool stage_ln(Ctl& c, const StackArgs& a, uint32_t& sb, const void* in, int B, int K,
                                         const AT* __restrict__ gam, const AT* __restrict__ beta, LT* act, float* raw,
                                         AT* gb, int st) {
  constexpr int V = 16 / (int)sizeof(IT);
  constexpr int VG = 16 / (int)sizeof(AT);
  constexpr int kGB = 2;  // gamma/beta vectors per thread issued ahead of the rows
  const int ngv = K / VG;
  {
    const rsrc_t rg = make_rsrc(gam, (uint32_t)(K * sizeof(AT))), rb = make_rsrc(beta, (uint32_t)(K * sizeof(AT)));
    u32x4 gv[kGB], bv[kGB];
#pragma unroll
    for (int u = 0; u < kGB; ++u) {
      const int j = st + u * NT;
      const uint32_t off = j < ngv ? (uint32_t)(j * 16) : kOutOfRange;
      gv[u] = __builtin_amdgcn_raw_buffer_load_b128(rg, off, 0, 0);
      bv[u] = __builtin_amdgcn_raw_buffer_load_b128(rb, off, 0, 0);
    }
    const rsrc_t r = make_rsrc(in, (uint32_t)(B * K * sizeof(IT)));
    const int nvec = B * K / V;
    for (int j0 = st; j0 < nvec; j0 += NT * kStageUnroll) {
      u32x4 v[kStageUnroll];
#pragma unroll
      for (int u = 0; u < kStageUnroll; ++u) {
        const int j = j0 + u * NT;
        v[u] = coh_load16(r, j < nvec ? (uint32_t)(j * 16) : kOutOfRange);
      }
#pragma unroll
      for (int u = 0; u < kStageUnroll; ++u) {
        const int j = j0 + u * NT;
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
#pragma unroll
    for (int u = 0; u < kGB; ++u) {
      const int j = st + u * NT;
      if (j < ngv) {
        *reinterpret_cast<u32x4*>(gb + j * VG) = gv[u];
        *reinterpret_cast<u32x4*>(gb + K + j * VG) = bv[u];
      }
    }
    for (int j = st + kGB * NT; j < ngv; j += NT) {  // rows longer than kGB*NT vectors
      *reinterpret_cast<u32x4*>(gb + j * VG) = __builtin_amdgcn_raw_buffer_load_b128(rg, (uint32_t)(j * 16), 0, 0);
      *reinterpret_cast<u32x4*>(gb + K + j * VG) = __builtin_amdgcn_raw_buffer_load_b128(rb, (uint32_t)(j * 16), 0, 0);
    }
  }
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
    s1[b] = wave_sum(s1[b]);
    s2[b] = wave_sum(s2[b]);
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

// int8: the fp16 scales of the phase's row tile, [nr][K/group], into LDS.
__device__ __forceinline__ void stage_scales(const void* s, int r0, int nr, int K, int group, half_t* scl, int st) {
  const int n = nr * (K / group);
  const half_t* src = static_cast<const half_t*>(s) + (size_t)r0 * (K / group);
  for (int i = st; i < n; i += NT) scl[i] = src[i];
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

// One item: scores of q against the chunk's rows, wave-reduced max and sum, the exp-weighted V
// sum; the partial (max, sum, acc[D]) goes to the workspace, and the workgroup that completes the
// last chunk of a (sequence, head) merges the partials into ctx (log-sum-exp).
template <typename AT, int D>
__device__ __forceinline__ bool attn_item(Ctl& c, const StackArgs& a, uint32_t& sb, const StackLayer& L, int item, float* s_acc,
                          float* s_part, int st) {
  typedef AttnShape<AT, D> S;
  constexpr int EK = S::EK, LPK = S::LPK, KPI = S::KPI, NIT = S::NIT;
  const float kNeg = -1e30f;
  const int cc = item % a.nchunk;
  const int j = (item / a.nchunk) % a.nh;
  const int b = item / (a.nchunk * a.nh);
  const int len = L.d_len[b];
  int nkeys = len + 1;
  if (nkeys > a.cap) nkeys = a.cap;
  const int nvalid = (nkeys + kStackChunk - 1) / kStackChunk;
  if (cc >= nvalid) return true;
  const int wave = st >> 6, lane = st & 63;
  const int H = a.nh * D;
  const size_t head = (((size_t)b * a.nh + j) * a.cap) * D;
  const uint32_t bytes = (uint32_t)((size_t)a.B * a.nh * a.cap * D * sizeof(AT));
  const rsrc_t rk = make_rsrc(L.k, bytes), rv = make_rsrc(L.v, bytes);
  const int e0 = (lane % LPK) * EK;
  // rows of the chunk; the new row (position len) was written by the QKV phase of this launch, so
  // every row is read with coherent loads
  u32x4 kr[NIT], vr[NIT];
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    const int key = cc * kStackChunk + (it * NS + wave) * KPI + lane / LPK;
    const bool in = key < nkeys && key < (cc + 1) * kStackChunk;
    const uint32_t off = in ? (uint32_t)((head + (size_t)key * D + e0) * sizeof(AT)) : kOutOfRange;
    kr[it] = coh_load16(rk, off);
    vr[it] = coh_load16(rv, off);
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
    const int key = cc * kStackChunk + (it * NS + wave) * KPI + lane / LPK;
    valid[it] = key < nkeys && key < (cc + 1) * kStackChunk;
    float p = 0.f;
    if constexpr (sizeof(AT) == 4) {
      p = qv[0] * as_f32(kr[it].x) + qv[1] * as_f32(kr[it].y) + qv[2] * as_f32(kr[it].z) + qv[3] * as_f32(kr[it].w);
    } else {
      const uint32_t wv[4] = {kr[it].x, kr[it].y, kr[it].z, kr[it].w};
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
      acc[0] += p * as_f32(vr[it].x);
      acc[1] += p * as_f32(vr[it].y);
      acc[2] += p * as_f32(vr[it].z);
      acc[3] += p * as_f32(vr[it].w);
    } else {
      const uint32_t wv[4] = {vr[it].x, vr[it].y, vr[it].z, vr[it].w};
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
  const rsrc_t rp = make_rsrc(a.part, (uint32_t)((size_t)a.B * a.nh * a.nchunk * (D + 2) * 4));
  if (st < D) {
    float v = 0.f;
#pragma unroll
    for (int wv = 0; wv < NS; ++wv) v += f[wv] * s_acc[wv * D + st];
    coh_store4(rp, (uint32_t)(((pbase + cc) * (D + 2) + 2 + st) * 4), __builtin_bit_cast(uint32_t, v));
  }
  if (st == 0) {
    float Ls = 0.f;
#pragma unroll
    for (int wv = 0; wv < NS; ++wv) Ls += f[wv] * c.l[wv];
    coh_store4(rp, (uint32_t)(((pbase + cc) * (D + 2)) * 4), __builtin_bit_cast(uint32_t, M));
    coh_store4(rp, (uint32_t)(((pbase + cc) * (D + 2) + 1) * 4), __builtin_bit_cast(uint32_t, Ls));
  }
  wait_vm_at_most<0>();
  if (!sync_bar(c, a, sb, st)) return false;
  uint32_t* cnt = a.sync + kSyncAttn + b * a.nh + j;
  if (st == 0)
    c.flag = __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == (uint32_t)(nvalid - 1);
  if (!sync_bar(c, a, sb, st)) return false;
  if (!c.flag) return true;
  // last chunk of this (sequence, head): all partials in one parallel load, then the merge
  const int nw = nvalid * (D + 2);
  for (int i = st; i < nw; i += NT) s_part[i] = as_f32(coh_load4(rp, (uint32_t)((pbase * (D + 2) + i) * 4)));
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
    const rsrc_t rc = make_rsrc(a.ctx, (uint32_t)(a.B * H * sizeof(AT)));
    coh_st_act<AT>(rc, (uint32_t)(b * H + j * D + st), Acc / Lsum);
  }
  if (st == 0) __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return true;
}

// ------------------------------------------------------------------ sync waves: the phase loop
template <typename WT, typename AT, int BM, int D>
__device__ __forceinline__ void sync_side(const StackArgs& a, Ctl& c, unsigned char* smem, int g, int st_in) {
  typedef typename WTraits<WT>::LT LT;
  LT* act = reinterpret_cast<LT*>(smem);
  float* raw = reinterpret_cast<float*>(smem + a.lds.raw);
  AT* gb = reinterpret_cast<AT*>(smem + a.lds.raw + (uint32_t)BM * a.H * 4u);  // LayerNorm gamma, then beta
  float* slots = reinterpret_cast<float*>(smem + a.lds.slots);
  half_t* scl = reinterpret_cast<half_t*>(smem + a.lds.scales);
  float* s_acc = reinterpret_cast<float*>(smem);                   // attention: NS x D floats
  float* s_part = reinterpret_cast<float*>(smem) + NS * D;         // merge: nchunk x (D + 2) floats
  const int H = a.H, F = a.F, B = a.B, G = a.G;
  // Thread indices are re-derived through an opaque copy at every phase: otherwise the compiler
  // hoists every per-thread address of every phase out of the layer loop and keeps them all live.
  int st = st_in;
  auto fresh = [&]() {
    int t = st_in;
    asm volatile("" : "+v"(t));
    st = t;
  };
  uint32_t sb = 0, epoch = 0;
  const int nitems = B * a.nh * a.nchunk;

  // per-workgroup row tiles of each projection (the same split the workers use)
  const int rq = (3 * H + G - 1) / G, ro = (H + G - 1) / G, r1 = (F + G - 1) / G;
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
  auto clear_slots = [&](int nr) {
    for (int i = st; i < nr * NWK * BM; i += NT) slots[i] = 0.f;
  };
  // publish the staged activation of phase `seq`, then wait for every worker to finish it
  auto hand_over = [&](uint32_t seq) -> bool {
    if (!sync_bar(c, a, sb, st)) return false;
    if (st == 0) lds_st(&c.act_ready, seq + 1u);
    bool ok = spin_until(c, a, [&] {
      bool all = true;
#pragma unroll
      for (int w = 0; w < NWK; ++w) all = all && lds_ld(&c.done[w]) >= seq + 1u;
      return all;
    });
    asm volatile("" ::: "memory");
    return ok;
  };
  // after this phase's stores: every sync wave's stores complete, one arrival, the release
  auto grid_barrier = [&]() -> bool {
    wait_vm_at_most<0>();
    if (!sync_bar(c, a, sb, st)) return false;
    ++epoch;
    if (st == 0) c.ok = grid_arrive_wait(c, a, epoch, g) ? 1 : 0;
    if (!sync_bar(c, a, sb, st)) return false;
    return c.ok != 0;
  };

  for (int l = 0; l < a.n_layers; ++l) {
    const StackLayer& L = a.layers[l];
    // layer outputs alternate between the two buffers; the pointers are selected as values (a
    // select of two field addresses would make the compiler keep the arguments in scratch)
    uintptr_t yb0 = reinterpret_cast<uintptr_t>(a.ybuf0), yb1 = reinterpret_cast<uintptr_t>(a.ybuf1);
    uintptr_t xa = reinterpret_cast<uintptr_t>(a.x), ya = reinterpret_cast<uintptr_t>(a.y);
    asm volatile("" : "+s"(yb0), "+s"(yb1), "+s"(xa), "+s"(ya));
    const void* xin = reinterpret_cast<const void*>((l == 0) ? xa : ((l & 1) ? yb0 : yb1));
    void* yout = reinterpret_cast<void*>((l == a.n_layers - 1) ? ya : ((l & 1) ? yb1 : yb0));
    const uint32_t seq0 = (uint32_t)l * 4u;

    // ---- region 1: LN1 + QKV + bias; q -> workspace, k/v -> cache row d_len[b]
    fresh();
    clear_slots(nq);
    if constexpr (sizeof(WT) == 1) stage_scales(L.s_qkv, q0, nq, H, a.group, scl, st);
    if (!stage_ln<AT, LT, AT, BM>(c, a, sb, xin, B, H, (const AT*)L.ln1_g, (const AT*)L.ln1_b, act, raw, gb, st)) return;
    if (!hand_over(seq0)) return;
    {
      const rsrc_t rqo = make_rsrc(a.q, (uint32_t)(B * H * 4));
      const uint32_t cache_bytes = (uint32_t)((size_t)B * a.nh * a.cap * D * sizeof(AT));
      const rsrc_t rk = make_rsrc(L.k, cache_bytes), rv = make_rsrc(L.v, cache_bytes);
      for (int t = st; t < nq * B; t += NT) {
        const int rl = t / B, b = t - rl * B, n = q0 + rl;
        const float z = row_sum(rl, b) + ldp<AT>(L.b_qkv, n);
        if (n < H) {
          coh_store4(rqo, (uint32_t)((b * H + n) * 4), __builtin_bit_cast(uint32_t, z));
        } else {
          const int m = n < 2 * H ? n - H : n - 2 * H, j = m / D, e = m - j * D;
          const int pos = L.d_len[b];
          if (pos >= 0 && pos < a.cap) coh_st_act<AT>(n < 2 * H ? rk : rv, (uint32_t)((((size_t)b * a.nh + j) * a.cap + pos) * D + e), z);
        }
      }
    }
    if (!grid_barrier()) return;

    // ---- region 2: attention over the cache, chunk partials merged by the last chunk
    fresh();
    for (int item = g; item < nitems; item += G)
      if (!attn_item<AT, D>(c, a, sb, L, item, s_acc, s_part, st)) return;
    if (!grid_barrier()) return;

    // ---- output projection + bias + residual: x2 = x + Wo ctx + bo
    fresh();
    if (!sync_bar(c, a, sb, st)) return;  // the attention scratch (same LDS) is no longer read
    clear_slots(no);
    if constexpr (sizeof(WT) == 1) stage_scales(L.s_o, o0, no, H, a.group, scl, st);
    stage_plain<AT, LT, BM>(a.ctx, B, H, act, st);
    if (!hand_over(seq0 + 1u)) return;
    {
      const rsrc_t rx = make_rsrc(xin, (uint32_t)(B * H * sizeof(AT)));
      const rsrc_t rx2 = make_rsrc(a.x2, (uint32_t)(B * H * 4));
      for (int t = st; t < no * B; t += NT) {
        const int rl = t / B, b = t - rl * B, n = o0 + rl;
        const float z = row_sum(rl, b) + ldp<AT>(L.b_o, n);
        coh_store4(rx2, (uint32_t)((b * H + n) * 4), __builtin_bit_cast(uint32_t, coh_ld_act<AT>(rx, (uint32_t)(b * H + n)) + z));
      }
    }
    if (!grid_barrier()) return;

    // ---- region 3: LN2 + FF1 + bias + GeLU
    fresh();
    clear_slots(nf);
    if constexpr (sizeof(WT) == 1) stage_scales(L.s_ff1, f0, nf, H, a.group, scl, st);
    if (!stage_ln<float, LT, AT, BM>(c, a, sb, a.x2, B, H, (const AT*)L.ln2_g, (const AT*)L.ln2_b, act, raw, gb, st)) return;
    if (!hand_over(seq0 + 2u)) return;
    {
      const rsrc_t rf = make_rsrc(a.f, (uint32_t)(B * F * sizeof(AT)));
      for (int t = st; t < nf * B; t += NT) {
        const int rl = t / B, b = t - rl * B, n = f0 + rl;
        const float z = row_sum(rl, b) + ldp<AT>(L.b_ff1, n);
        coh_st_act<AT>(rf, (uint32_t)(b * F + n), gelu(z, a.gelu_tanh != 0));
      }
    }
    if (!grid_barrier()) return;

    // ---- region 4: FF2 + bias + residual: y = x2 + W2 f + b2
    fresh();
    clear_slots(ny);
    if constexpr (sizeof(WT) == 1) stage_scales(L.s_ff2, y0, ny, F, a.group, scl, st);
    stage_plain<AT, LT, BM>(a.f, B, F, act, st);
    if (!hand_over(seq0 + 3u)) return;
    {
      const rsrc_t rx2 = make_rsrc(a.x2, (uint32_t)(B * H * 4));
      const rsrc_t ry = make_rsrc(yout, (uint32_t)(B * H * sizeof(AT)));
      for (int t = st; t < ny * B; t += NT) {
        const int rl = t / B, b = t - rl * B, n = y0 + rl;
        const float z = row_sum(rl, b) + ldp<AT>(L.b_ff2, n);
        coh_st_act<AT>(ry, (uint32_t)(b * H + n), as_f32(coh_load4(rx2, (uint32_t)((b * H + n) * 4))) + z);
      }
    }
    if (!grid_barrier()) return;
  }

  // every layer has attended: advance the cache lengths, then the last workgroup out resets the
  // barrier state for the next launch
  if (g == 0 && st < B)
    for (int l = 0; l < a.n_layers; ++l) {
      int32_t* dl = a.layers[l].d_len;
      if (dl[st] + 1 <= a.cap) dl[st] += 1;
    }
  if (st == 0) {
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

}  // namespace

// ------------------------------------------------------------------ the persistent kernel
template <typename WT, typename AT, int BM, int D>
__global__ __launch_bounds__(kStackThreads, 1) void stack_decode_kernel(const StackArgs a) {
  typedef typename WTraits<WT>::LT LT;
  extern __shared__ __align__(16) unsigned char smem[];
  __shared__ Ctl c;
  uint64_t* wtab = reinterpret_cast<uint64_t*>(smem + a.lds.wtab);
  for (int i = threadIdx.x; i < a.n_layers * 4; i += kStackThreads)
    wtab[i] = reinterpret_cast<uint64_t>(phase_w(a.layers[i >> 2], i & 3));
  if (threadIdx.x == 0) {
    c.act_ready = 0u;
    for (int w = 0; w < NWK; ++w) c.done[w] = 0u;
    c.sbar = 0u;
    c.abort = 0u;
    c.ok = 0;
    c.flag = 0;
  }
  __syncthreads();
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int lane = threadIdx.x & 63;
  if (wave < NS) {
    sync_side<WT, AT, BM, D>(a, c, smem, blockIdx.x, (int)threadIdx.x);
    if (lds_ld(&c.abort) == 0u) return;
    raise_abort(c, a.sync);  // a failed sync wave releases the workers
  } else {
    worker<WT, BM>(a, c, reinterpret_cast<const LT*>(smem), reinterpret_cast<float*>(smem + a.lds.slots),
                   reinterpret_cast<const half_t*>(smem + a.lds.scales), wtab, blockIdx.x, wave - NS, lane);
  }
}

// ------------------------------------------------------------------ host-side launch helpers
int stack_rows_per_wg(int H, int F, int G) {
  int r = (3 * H + G - 1) / G;
  r = max(r, (H + G - 1) / G);
  r = max(r, (F + G - 1) / G);
  return r;
}

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
  const void* k = pick(wdt, adt, a.B, a.d);
  if (!k) return hipErrorInvalidValue;
  hipError_t e = hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)a.lds.total);
  if (e != hipSuccess) return e;
  StackArgs args = a;
  void* params[] = {&args};
  return hipLaunchCooperativeKernel(k, dim3(a.G), dim3(kStackThreads), params, (unsigned)a.lds.total, st);
}

}  // namespace ds
