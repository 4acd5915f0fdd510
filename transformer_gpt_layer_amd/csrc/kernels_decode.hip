// kernels_decode.hip -- the fused skinny-GEMV kernels and KV-cache attention of one layer step.
//
// Source: the customized transformer-block inference kernels of the page "DeepSpeed Inference
// 内核优化深度解析" (blog.gitcode.com), section 三: region 1 (input LayerNorm + Q/K/V GeMM + bias),
// region 2 (head transform folded into attention), region 3 (FF + LayerNorm + bias + residual +
// GELU), region 4 (bias + residual); section 三 3.3 names the mechanisms (on-chip staging of the
// normalized vector, intra-warp reductions, a vector-matrix GeMM schedule with fused epilogues).
//
// gfx950 design: every weight byte is streamed once from HBM with 16-byte non-temporal loads,
// each wave64 owns R output rows and splits the reduction dimension across its 64 lanes, the
// (normalized) activation rows of a batch group sit in LDS, partial sums are reduced across the
// wave with DPP/permute shuffles, and bias / residual / GeLU / KV scatter run in the epilogue.
#include "ds_device.hpp"
#include "ds_gemv.hpp"
#include "ds_launch.hpp"

namespace ds {

constexpr int kLdsActBytes = 64 * 1024;  // activation staging budget per workgroup

template <typename T> __device__ __forceinline__ float ldf(const void* p, size_t i) {
  return to_f32(reinterpret_cast<const T*>(p)[i]);
}

// ------------------------------------------------------------------ fused GEMV kernel
// grid.x: row blocks of 4 waves x R rows; grid.y: activation-row groups of BM rows.
template <typename WT, typename AT, int KIND, int BM, int R>
__global__ __launch_bounds__(256) void gemv_kernel(const GemvArgs a) {
  typedef typename WTraits<WT>::LT LT;
  constexpr int E = WTraits<WT>::E;
  constexpr bool kLN = (KIND == KIND_QKV || KIND == KIND_FF1);
  extern __shared__ __align__(16) unsigned char smem_raw[];
  LT* act = reinterpret_cast<LT*>(smem_raw);
  __shared__ float red[4];
  __shared__ float s_mean[BM], s_rstd[BM];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int K = a.k, N = a.n;
  const int row0 = (blockIdx.x * 4 + wave) * R;
  const int r0 = blockIdx.y * BM;
  const int nb = min(BM, a.rows - r0);

  if (KIND == KIND_QKV && blockIdx.x == 0 && blockIdx.y == 0)
    for (int i = tid; i < a.rows * a.heads; i += 256) a.attn_counters[i] = 0u;

  // LayerNorm statistics of each activation row (two passes over the row, biased variance)
  if constexpr (kLN) {
    for (int b = 0; b < nb; ++b) {
      const size_t base = (size_t)(r0 + b) * K;
      float s = 0.f;
      for (int i = tid; i < K; i += 256)
        s += (KIND == KIND_QKV) ? ldf<AT>(a.in, base + i) : ldf<float>(a.in, base + i);
      const float mean = block_sum256(s, red) / K;
      float v = 0.f;
      for (int i = tid; i < K; i += 256) {
        const float x = ((KIND == KIND_QKV) ? ldf<AT>(a.in, base + i) : ldf<float>(a.in, base + i)) - mean;
        v += x * x;
      }
      const float var = block_sum256(v, red) / K;
      if (tid == 0) {
        s_mean[b] = mean;
        s_rstd[b] = rsqrtf(var + a.eps);
      }
    }
  }

  // activation chunk length: a multiple of the per-iteration span 64*E
  int KC = kLdsActBytes / (BM * (int)sizeof(LT));
  KC = KC / (kWave * E) * (kWave * E);
  if (KC > K) KC = K;

  float acc[R][BM];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int b = 0; b < BM; ++b) acc[r][b] = 0.f;

  const int nrows = N - row0;
  for (int kbeg = 0; kbeg < K; kbeg += KC) {
    const int kend = min(K, kbeg + KC), len = kend - kbeg;
    __syncthreads();  // LN statistics ready / previous chunk consumed
    for (int idx = tid; idx < BM * len; idx += 256) {
      const int b = idx / len, kk = idx - b * len, kg = kbeg + kk;
      float v = 0.f;
      if (b < nb) {
        const size_t at = (size_t)(r0 + b) * K + kg;
        if constexpr (KIND == KIND_QKV) v = ldf<AT>(a.in, at);
        else v = ldf<float>(a.in, at);
        if constexpr (kLN) v = (v - s_mean[b]) * s_rstd[b] * ldf<AT>(a.ln_g, kg) + ldf<AT>(a.ln_b, kg);
      }
      act[b * KC + kk] = (LT)v;
    }
    __syncthreads();
    if (nrows > 0)
      gemv_rows<WT, R, BM, 4>(reinterpret_cast<const WT*>(a.w), reinterpret_cast<const half_t*>(a.s),
                              K, a.group, row0, nrows, kbeg, kend, act, KC, acc, lane);
  }
  if (nrows <= 0) return;

#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int b = 0; b < BM; ++b) acc[r][b] = wave_sum(acc[r][b]);

#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int b = 0; b < BM; ++b) {
      if (lane != r * BM + b || r >= nrows || b >= nb) continue;
      const int n = row0 + r, rr = r0 + b;
      const float z = acc[r][b] + ldf<AT>(a.bias, n);
      if constexpr (KIND == KIND_QKV) {
        const int H = a.hidden, d = a.head_dim;
        if (n < H) {
          a.q_out[(size_t)rr * H + n] = z;
        } else if (a.kv_new) {
          a.kv_new[(size_t)rr * 2 * H + (n - H)] = z;  // quantized into the int8 cache by kv_store_i8
        } else {
          const int seq = rr / a.tokens, t = rr - seq * a.tokens;
          const int pos = a.d_len[seq] + t;
          const int m = (n < 2 * H) ? n - H : n - 2 * H;
          const int j = m / d, e = m - j * d;
          if (pos >= 0 && pos < a.cap) {
            AT* cache = reinterpret_cast<AT*>(n < 2 * H ? a.k_cache : a.v_cache);
            cache[(((size_t)seq * a.heads + j) * a.cap + pos) * d + e] = from_f32<AT>(z);
          }
        }
      } else if constexpr (KIND == KIND_OPROJ) {
        reinterpret_cast<float*>(a.out)[(size_t)rr * N + n] = ldf<AT>(a.resid, (size_t)rr * N + n) + z;
      } else if constexpr (KIND == KIND_FF1) {
        reinterpret_cast<float*>(a.out)[(size_t)rr * N + n] = gelu(z, a.gelu_tanh != 0);
      } else {
        reinterpret_cast<AT*>(a.out)[(size_t)rr * N + n] =
            from_f32<AT>(ldf<float>(a.resid, (size_t)rr * N + n) + z);
      }
    }
}

template <typename WT, typename AT, int KIND, int BM>
static hipError_t launch_gemv_bm(const GemvArgs& a, hipStream_t st) {
  constexpr int R = 2;
  typedef typename WTraits<WT>::LT LT;
  constexpr int E = WTraits<WT>::E;
  int KC = kLdsActBytes / (BM * (int)sizeof(LT));
  KC = KC / (kWave * E) * (kWave * E);
  if (KC > a.k) KC = a.k;
  const size_t lds = (size_t)BM * KC * sizeof(LT);
  dim3 grid((a.n + 4 * R - 1) / (4 * R), (a.rows + BM - 1) / BM);
  hipLaunchKernelGGL((gemv_kernel<WT, AT, KIND, BM, R>), grid, dim3(256), lds, st, a);
  return hipGetLastError();
}

template <typename WT, typename AT, int KIND>
static hipError_t launch_gemv_kind(const GemvArgs& a, hipStream_t st) {
  if (a.rows >= 8) return launch_gemv_bm<WT, AT, KIND, 8>(a, st);
  if (a.rows >= 4) return launch_gemv_bm<WT, AT, KIND, 4>(a, st);
  if (a.rows >= 2) return launch_gemv_bm<WT, AT, KIND, 2>(a, st);
  return launch_gemv_bm<WT, AT, KIND, 1>(a, st);
}

template <typename WT, typename AT>
static hipError_t launch_gemv_t(GemvKind kind, const GemvArgs& a, hipStream_t st) {
  switch (kind) {
    case KIND_QKV: return launch_gemv_kind<WT, AT, KIND_QKV>(a, st);
    case KIND_OPROJ: return launch_gemv_kind<WT, AT, KIND_OPROJ>(a, st);
    case KIND_FF1: return launch_gemv_kind<WT, AT, KIND_FF1>(a, st);
    case KIND_FF2: return launch_gemv_kind<WT, AT, KIND_FF2>(a, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_gemv(Dt wdt, Dt adt, GemvKind kind, const GemvArgs& a, hipStream_t st) {
  if (wdt == F32 && adt == F32) return launch_gemv_t<float, float>(kind, a, st);
  if (wdt == F16 && adt == F16) return launch_gemv_t<half_t, half_t>(kind, a, st);
  if (wdt == I8 && adt == F16) return launch_gemv_t<int8_t, half_t>(kind, a, st);
  if (wdt == BF16 && adt == BF16) return launch_gemv_t<bf16_t, bf16_t>(kind, a, st);
  return hipErrorInvalidValue;
}

// ------------------------------------------------------------------ decode attention
// Region 2: for one (row, head) and one chunk of cached positions, q.K/sqrt(d) scores, a
// wave-reduced max and sum, and the exp-weighted V sum; the last chunk workgroup to finish merges
// the chunk partials (log-sum-exp) into ctx. grid = (nchunk, heads, rows).
// QT: the type of q and ctx (float: q, ctx; fp16 or bf16: q16, ctx16), independent of the cache's AT.
template <typename AT, int D, int C, typename QT = float>
__global__ __launch_bounds__(256) void attn_decode_kernel(const AttnArgs a) {
  constexpr bool QH = sizeof(QT) == 2;
  constexpr int EK = 16 / (int)sizeof(AT);  // elements per 16-byte load
  constexpr int LPK = D / EK;               // lanes per key
  constexpr int KPI = kWave / LPK;          // keys per wave per load
  constexpr int KPS = 4 * KPI;              // keys per workgroup step
  constexpr int PF = 4;                     // steps whose K and V loads a wave keeps in flight
  static_assert(C % KPS == 0, "chunk of whole steps");
  const float kNeg = -1e30f;
  __shared__ float s_m[4], s_l[4];
  __shared__ float s_acc[4][D];
  __shared__ int s_last;

  const int c = blockIdx.x, j = blockIdx.y, rr = blockIdx.z;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int seq = rr / a.tokens, t = rr - seq * a.tokens;
  const int len0 = a.d_len[seq];
  int nkeys = a.causal ? len0 + t + 1 : len0 + a.tokens;
  if (nkeys > a.cap) nkeys = a.cap;
  // chunks of equal length (whole steps), so that no workgroup is left with a sliver of the keys:
  // the launch's count, fewer when there are under 64 keys per chunk
  const int nch = min(a.nchunk, (nkeys + 63) / 64);
  const int cs = ((nkeys + nch - 1) / nch + KPS - 1) / KPS * KPS;
  const int nvalid = (nkeys + cs - 1) / cs;
  if (c >= nvalid) return;
  const int kb = c * cs, ke = min(kb + cs, nkeys);
  const int nsteps = (ke - kb + KPS - 1) / KPS;
  const int H = a.heads * D;

  // q slice of this lane, scaled by log2(e)/sqrt(d) so that scores feed exp2 directly
  const int e0 = (lane % LPK) * EK;
  const float qs = 1.4426950408889634f / sqrtf((float)D);
  float qv[EK];
#pragma unroll
  for (int e = 0; e < EK; ++e) {
    const size_t qi = (size_t)rr * H + j * D + e0 + e;
    if constexpr (QH) qv[e] = (float)reinterpret_cast<const QT*>(a.q16)[qi] * qs;
    else qv[e] = a.q[qi] * qs;
  }

  // K and V rows of this (sequence, head) as buffers ending at the last key: loads past it, and
  // the out-of-chunk requests of the last steps, read zeros
  const size_t head_base = (((size_t)seq * a.heads + j) * a.cap) * D;
  const uint32_t hbytes = (uint32_t)((size_t)nkeys * D * sizeof(AT));
  const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<AT*>(reinterpret_cast<const AT*>(a.k_cache) + head_base), (short)0, (int)hbytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<AT*>(reinterpret_cast<const AT*>(a.v_cache) + head_base), (short)0, (int)hbytes, 0x00020000);
  const int kl = wave * KPI + lane / LPK;  // this lane's key within a step
  u32x4 kr[PF], vr[PF];
  float ksc[PF], vsc[PF];  // an int8 cache: the keys' fp16 row scales
  const uint16_t* ksp = static_cast<const uint16_t*>(a.k_scale) + ((size_t)seq * a.heads + j) * a.cap;
  const uint16_t* vsp = static_cast<const uint16_t*>(a.v_scale) + ((size_t)seq * a.heads + j) * a.cap;
  auto issue = [&](int step, int slot) {
    const int key = kb + step * KPS + kl;
    const bool live = step < nsteps && key < ke;
    const uint32_t off = live ? (uint32_t)(((size_t)key * D + e0) * sizeof(AT)) : 0x80000000u;
    kr[slot] = __builtin_amdgcn_raw_buffer_load_b128(rk, off, 0, 0);
    vr[slot] = __builtin_amdgcn_raw_buffer_load_b128(rv, off, 0, 0);
    if constexpr (sizeof(AT) == 1) {
      ksc[slot] = live ? (float)__builtin_bit_cast(half_t, ksp[key]) : 0.f;
      vsc[slot] = live ? (float)__builtin_bit_cast(half_t, vsp[key]) : 0.f;
    }
  };
#pragma unroll
  for (int q = 0; q < PF; ++q) issue(q, q);

  // online softmax over this lane's keys: running max m, weight sum l, weighted V sum acc
  float m = kNeg, l = 0.f, acc[EK];
#pragma unroll
  for (int e = 0; e < EK; ++e) acc[e] = 0.f;
  for (int i = 0; i < nsteps; i += PF) {
#pragma unroll
    for (int q = 0; q < PF; ++q) {
      if (i + q < nsteps) {
        const int key = kb + (i + q) * KPS + kl;
        float p = 0.f;
        if constexpr (sizeof(AT) == 4) {
          p = qv[0] * as_f32(kr[q].x) + qv[1] * as_f32(kr[q].y) + qv[2] * as_f32(kr[q].z) + qv[3] * as_f32(kr[q].w);
        } else if constexpr (sizeof(AT) == 2) {
          const uint32_t wv[4] = {kr[q].x, kr[q].y, kr[q].z, kr[q].w};
#pragma unroll
          for (int h = 0; h < 4; ++h) p += qv[2 * h] * lo16<AT>(wv[h]) + qv[2 * h + 1] * hi16<AT>(wv[h]);
        } else {
          const uint32_t wv[4] = {kr[q].x, kr[q].y, kr[q].z, kr[q].w};
#pragma unroll
          for (int h = 0; h < 4; ++h)
#pragma unroll
            for (int b = 0; b < 4; ++b) p += qv[4 * h + b] * i8_at(wv[h], b);
          p *= ksc[q];
        }
        p = group_sum<LPK>(p);
        if (key < ke) {
          const float mn = fmaxf(m, p);
          const float cf = exp2f(m - mn), w = exp2f(p - mn);
          m = mn;
          l = l * cf + w;
          if constexpr (sizeof(AT) == 4) {
            acc[0] = acc[0] * cf + w * as_f32(vr[q].x);
            acc[1] = acc[1] * cf + w * as_f32(vr[q].y);
            acc[2] = acc[2] * cf + w * as_f32(vr[q].z);
            acc[3] = acc[3] * cf + w * as_f32(vr[q].w);
          } else if constexpr (sizeof(AT) == 2) {
            const uint32_t wv[4] = {vr[q].x, vr[q].y, vr[q].z, vr[q].w};
#pragma unroll
            for (int h = 0; h < 4; ++h) {
              acc[2 * h] = acc[2 * h] * cf + w * lo16<AT>(wv[h]);
              acc[2 * h + 1] = acc[2 * h + 1] * cf + w * hi16<AT>(wv[h]);
            }
          } else {
            const uint32_t wv[4] = {vr[q].x, vr[q].y, vr[q].z, vr[q].w};
            const float ws = w * vsc[q];
#pragma unroll
            for (int h = 0; h < 4; ++h)
#pragma unroll
              for (int b = 0; b < 4; ++b) acc[4 * h + b] = acc[4 * h + b] * cf + ws * i8_at(wv[h], b);
          }
        }
      }
      issue(i + q + PF, q);
    }
  }
  __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): the requests past the end
  // rescale every key slot to the wave's max, then reduce over the slots (lanes with equal
  // lane % LPK)
  const float mw = wave_max(m);
  const float sw = exp2f(m - mw);
  l *= sw;
#pragma unroll
  for (int e = 0; e < EK; ++e) acc[e] *= sw;
  m = mw;
#pragma unroll
  for (int off = LPK; off < kWave; off <<= 1) {
    l += __shfl_xor(l, off, kWave);
#pragma unroll
    for (int e = 0; e < EK; ++e) acc[e] += __shfl_xor(acc[e], off, kWave);
  }
  if (lane < LPK) {
#pragma unroll
    for (int e = 0; e < EK; ++e) s_acc[wave][e0 + e] = acc[e];
    if (lane == 0) {
      s_m[wave] = m;
      s_l[wave] = l;
    }
  }
  __syncthreads();

  // workgroup partial: merge the four waves
  float* part = a.part + (((size_t)rr * a.heads + j) * a.nchunk + c) * (D + 2);
  const float M = fmaxf(fmaxf(s_m[0], s_m[1]), fmaxf(s_m[2], s_m[3]));
  float f[4];
#pragma unroll
  for (int w = 0; w < 4; ++w) f[w] = s_l[w] > 0.f ? exp2f(s_m[w] - M) : 0.f;
  // Partials are stored at device scope (written through past this XCD's L2) and every store is
  // acknowledged before the arrival count moves, so the merging workgroup, reading them at device
  // scope, sees them without an L2 write-back or invalidation of the whole cache.
  if (tid < D)
    __hip_atomic_store(part + 2 + tid, f[0] * s_acc[0][tid] + f[1] * s_acc[1][tid] + f[2] * s_acc[2][tid] + f[3] * s_acc[3][tid],
                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (tid == 0) {
    __hip_atomic_store(part, M, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(part + 1, f[0] * s_l[0] + f[1] * s_l[1] + f[2] * s_l[2] + f[3] * s_l[3], __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
  }
  __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): this thread's stores are acknowledged
  __syncthreads();
  uint32_t* cnt = a.counters + (size_t)rr * a.heads + j;
  if (tid == 0)
    s_last = __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == (uint32_t)(nvalid - 1);
  __syncthreads();
  if (!s_last) return;

  // last workgroup of this (row, head): log-sum-exp merge of the nvalid chunk partials
  const float* p0 = a.part + ((size_t)rr * a.heads + j) * a.nchunk * (D + 2);
  if (tid < D) {
    float MM = kNeg;
    auto ld = [](const float* p) { return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); };
    for (int cc = 0; cc < nvalid; ++cc) MM = fmaxf(MM, ld(p0 + (size_t)cc * (D + 2)));
    float L = 0.f, A = 0.f;
    for (int cc = 0; cc < nvalid; ++cc) {
      const float* pc = p0 + (size_t)cc * (D + 2);
      const float lc = ld(pc + 1);
      const float w = lc > 0.f ? exp2f(ld(pc) - MM) : 0.f;
      L += w * lc;
      A += w * ld(pc + 2 + tid);
    }
    if constexpr (QH) reinterpret_cast<QT*>(a.ctx16)[(size_t)rr * H + j * D + tid] = (QT)(A / L);
    else a.ctx[(size_t)rr * H + j * D + tid] = A / L;
  }
  if (tid == 0) *cnt = 0u;
}

constexpr int kAttnChunk = 64;       // positions per workgroup for few (row, head) pairs
constexpr int kAttnChunkWide = 256;  // and for many: fewer workgroups and partials to merge

// Chunks per (row, head) for a launch. With 64-position chunks (few pairs), as many as the
// capacity has. With wide chunks, between ceil(cap / 512) and nmax (the workspace's slots) the count
// whose workgroups spread most evenly over the CUs, the fewest among equals: the 13B batch-8
// step (320 pairs, capacity 1088) runs 4 chunks (1280 workgroups, 5 per CU) instead of 5 (6.25).
int attn_chunks_for(int rows, int heads, int cap, int chunk, int nmax, int cus) {
  if (chunk != kAttnChunkWide || cus <= 0) return nmax;
  const long pairs = (long)rows * heads;
  int best = nmax;
  long best_num = 0, best_den = 1;  // imbalance ceil(pairs n / cus) cus / (pairs n)
  for (int n = max(1, (cap + 511) / 512); n <= nmax; ++n) {
    const long wg = pairs * n, num = (wg + cus - 1) / cus * cus;
    if (best_num == 0 || num * best_den < best_num * wg) {
      best = n;
      best_num = num;
      best_den = wg;
    }
  }
  return best;
}

int attn_chunk_for(int rows, int heads, int cap) {
  (void)cap;
  return (long)rows * heads >= 256 ? kAttnChunkWide : kAttnChunk;
}

template <typename AT, int D, int C, typename QT>
static hipError_t launch_attn_t(const AttnArgs& a, hipStream_t st) {
  dim3 grid(a.nchunk, a.heads, a.rows);
  hipLaunchKernelGGL((attn_decode_kernel<AT, D, C, QT>), grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

template <typename AT, typename QT>
static hipError_t launch_attn_d(const AttnArgs& a, hipStream_t st) {
  const bool wide = a.chunk == kAttnChunkWide;
  if (!wide && a.chunk != kAttnChunk) return hipErrorInvalidValue;
  if (a.head_dim == 64)
    return wide ? launch_attn_t<AT, 64, kAttnChunkWide, QT>(a, st) : launch_attn_t<AT, 64, kAttnChunk, QT>(a, st);
  if (a.head_dim == 128)
    return wide ? launch_attn_t<AT, 128, kAttnChunkWide, QT>(a, st) : launch_attn_t<AT, 128, kAttnChunk, QT>(a, st);
  return hipErrorInvalidValue;
}

hipError_t launch_attn_decode_16(bool bf16, const AttnArgs& a, hipStream_t st) {
  if (a.k_scale) return bf16 ? launch_attn_d<int8_t, bf16_t>(a, st) : launch_attn_d<int8_t, half_t>(a, st);
  return bf16 ? launch_attn_d<bf16_t, bf16_t>(a, st) : launch_attn_d<half_t, half_t>(a, st);
}

hipError_t launch_attn_decode(Dt adt, const AttnArgs& a, hipStream_t st) {
  if (a.k_scale) return adt == F16 || adt == BF16 ? launch_attn_d<int8_t, float>(a, st) : hipErrorInvalidValue;
  if (adt == F32) return launch_attn_d<float, float>(a, st);
  if (adt == F16) return launch_attn_d<half_t, float>(a, st);
  if (adt == BF16) return launch_attn_d<bf16_t, float>(a, st);
  return hipErrorInvalidValue;
}

}  // namespace ds
