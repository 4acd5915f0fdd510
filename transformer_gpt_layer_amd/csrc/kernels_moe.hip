// kernels_moe.hip -- the MoE expert FF of one step: the gate, the routing of tokens to experts,
// the chosen experts' two products and the weighted combination.
//
// Source: "DeepSpeed MoE 大规模稀疏模型推理实战指南" (blog.gitcode.com), the MoE sections: a
// number of experts per MoE layer, and the layer types 'standard' and 'residual' (PR-MoE). The
// pages do not give the gate; this library's reading is stated with ds_moe_desc in ds_layer.h.
//
// gfx950 design: a decode step is bound by streaming the chosen experts' weights, so the tokens of
// a step are grouped by expert and each chosen expert's W1 and W2 rows are read exactly once per
// step, whatever the number of tokens that chose it. The experts' products reuse the wave GEMV
// core of the dense path (16-byte weight loads, activations of up to BM tokens in LDS). The
// residual MLP of the 'residual' type is one more expert that every token takes with weight 1.
// Each token's expert outputs are kept apart and summed in slot order by the last kernel, so the
// result does not depend on the order in which workgroups finish.
#include "ds_device.hpp"
#include "ds_gemv.hpp"
#include "ds_launch.hpp"

namespace ds {
namespace {

constexpr int kMoeLdsAct = 64 * 1024;  // activation staging budget of an expert workgroup

template <typename T> __device__ __forceinline__ float ldm(const void* p, size_t i) {
  return to_f32(reinterpret_cast<const T*>(p)[i]);
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const uint32_t lo = __shfl_xor((uint32_t)v, off, kWave), hi = __shfl_xor((uint32_t)(v >> 32), off, kWave);
    const uint64_t o = ((uint64_t)hi << 32) | lo;
    v = o > v ? o : v;
  }
  return v;
}

// Route table in the workspace: [0] the number of used experts, then used[U], cnt[U], start[U]
// (U = the launch's bound on used experts) and pairs[P]: the (token, slot) pairs of each used
// expert, in token order, at pairs[start[u] ...].
struct Route {
  int32_t* n_used;
  int32_t *used, *cnt, *start, *pairs;
  __device__ Route(int32_t* r, int U) : n_used(r), used(r + 1), cnt(r + 1 + U), start(r + 1 + 2 * U), pairs(r + 1 + 3 * U) {}
};

// ------------------------------------------------------------------ gate
// One workgroup per token: LayerNorm of x2 (biased variance, two passes over the row in LDS), h
// rounded to the staged type LT and stored for the experts, the E gate logits from that same
// rounded h (each wave takes every fourth expert, its lanes 16-byte pieces of the gate row), then
// in one wave the softmax and the top-k: k rounds of a wave-wide maximum of 64-bit keys (the
// probability's bits above the inverted expert index: the largest probability, and the smallest
// index among equal ones), each lane keeping a bit mask of its experts already taken.
template <typename AT, typename LT>
__global__ __launch_bounds__(256) void moe_gate_kernel(const MoeArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  float* xs = reinterpret_cast<float*>(smem);  // [H]: the row, then h as the experts see it
  float* lg = xs + a.H;                        // [E]: logits, then exp(logit - max)
  __shared__ float red[4];
  const int t = blockIdx.x, tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int H = a.H, E = a.E, K = a.k, KS = a.KS;
  const size_t row = (size_t)t * H;

  float s = 0.f;
  for (int i = tid; i < H; i += 256) {
    const float v = ldm<AT>(a.x2, row + i);
    xs[i] = v;
    s += v;
  }
  const float mean = block_sum256(s, red) / (float)H;
  float v2 = 0.f;
  for (int i = tid; i < H; i += 256) {
    const float d = xs[i] - mean;
    v2 += d * d;
  }
  const float rstd = rsqrtf(block_sum256(v2, red) / (float)H + a.eps);
  LT* hrow = reinterpret_cast<LT*>(a.h) + row;
  for (int i = tid; i < H; i += 256) {
    const LT hv = (LT)((xs[i] - mean) * rstd * ldm<AT>(a.ln_g, i) + ldm<AT>(a.ln_b, i));
    hrow[i] = hv;
    xs[i] = (float)hv;
  }
  __syncthreads();

  constexpr int EK = 16 / (int)sizeof(AT);
  for (int e = wave; e < E; e += 4) {
    const AT* g = reinterpret_cast<const AT*>(a.w_gate) + (size_t)e * H;
    float acc = 0.f;
    for (int k = lane * EK; k < H; k += kWave * EK) {
      const u32x4 w = ld16(g + k);
      const uint32_t w4[4] = {w.x, w.y, w.z, w.w};
      if constexpr (sizeof(AT) == 4) {
#pragma unroll
        for (int h = 0; h < 4; ++h) acc += as_f32(w4[h]) * xs[k + h];
      } else {
#pragma unroll
        for (int h = 0; h < 4; ++h) acc += lo16<AT>(w4[h]) * xs[k + 2 * h] + hi16<AT>(w4[h]) * xs[k + 2 * h + 1];
      }
    }
    acc = wave_sum(acc);
    if (lane == 0) lg[e] = acc;
  }
  __syncthreads();
  if (wave != 0) return;

  float m = -3.0e38f;
  for (int e = lane; e < E; e += kWave) m = fmaxf(m, lg[e]);
  m = wave_max(m);
  float sum = 0.f;
  for (int e = lane; e < E; e += kWave) {
    const float p = expf(lg[e] - m);
    lg[e] = p;
    sum += p;
  }
  sum = wave_sum(sum);
  uint32_t taken = 0u;  // bit j: expert lane + 64 j has been chosen
  int esel[kMoeMaxK];
  float psel[kMoeMaxK];
  float ptot = 0.f;
#pragma unroll
  for (int i = 0; i < kMoeMaxK; ++i) {
    esel[i] = 0;
    psel[i] = 0.f;
    if (i >= K) continue;
    uint64_t best = 0ull;
    for (int e = lane, j = 0; e < E; e += kWave, ++j) {
      if (taken & (1u << j)) continue;
      const uint64_t key = ((uint64_t)__builtin_bit_cast(uint32_t, lg[e]) << 32) | (uint64_t)(0xffffffffu - (uint32_t)e);
      best = key > best ? key : best;
    }
    best = wave_max_u64(best);
    const int e = (int)(0xffffffffu - (uint32_t)best);
    if ((e & (kWave - 1)) == lane) taken |= 1u << (e / kWave);
    esel[i] = e;
    psel[i] = lg[e] / sum;
    ptot += psel[i];
  }
  if (lane == 0) {
#pragma unroll
    for (int i = 0; i < kMoeMaxK; ++i) {
      if (i >= K) continue;
      const float w = a.combine ? psel[i] : psel[i] / ptot;
      a.sel[(size_t)t * KS + i] = esel[i];
      a.wgt[(size_t)t * KS + i] = w;
      if (a.sel_out) a.sel_out[(size_t)t * K + i] = esel[i];
      if (a.wgt_out) a.wgt_out[(size_t)t * K + i] = w;
    }
    if (KS > K) {  // the residual MLP: expert index E, weight 1
      a.sel[(size_t)t * KS + K] = E;
      a.wgt[(size_t)t * KS + K] = 1.f;
    }
  }
}

// ------------------------------------------------------------------ routing
// One workgroup. Expert e (of NE = E + residual) counts its pairs; exclusive scans over the
// experts (four consecutive experts per thread) give each used expert its slot u and its first
// pair; each expert then lists its pairs in token order. Deterministic, no atomics.
__device__ __forceinline__ int block_excl_scan(int v, int* wsum, int& total) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  int x = v;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int y = __shfl_up(x, off, kWave);
    if (lane >= off) x += y;
  }
  __syncthreads();
  if (lane == kWave - 1) wsum[wave] = x;
  __syncthreads();
  int before = 0;
  total = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    if (w < wave) before += wsum[w];
    total += wsum[w];
  }
  return before + x - v;
}

__global__ __launch_bounds__(256) void moe_route_kernel(const MoeArgs a) {
  __shared__ int s_sel[kMoeMaxPairs];
  __shared__ int wsum[4];
  const int tid = threadIdx.x;
  const int P = a.T * a.KS, NE = a.E + (a.residual ? 1 : 0);
  Route R(a.route, a.umax);
  for (int p = tid; p < P; p += 256) s_sel[p] = a.sel[p];
  __syncthreads();
  int cnt[4], flag[4], csum = 0, fsum = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = 4 * tid + q;
    int c = 0;
    if (e < NE)
      for (int p = 0; p < P; ++p) c += s_sel[p] == e ? 1 : 0;
    cnt[q] = c;
    flag[q] = c > 0 ? 1 : 0;
    csum += c;
    fsum += flag[q];
  }
  int ctot = 0, ftot = 0;
  int c0 = block_excl_scan(csum, wsum, ctot);
  int f0 = block_excl_scan(fsum, wsum, ftot);
  if (tid == 0) *R.n_used = ftot;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = 4 * tid + q;
    if (flag[q]) {
      R.used[f0] = e;
      R.cnt[f0] = cnt[q];
      R.start[f0] = c0;
      int j = c0;
      for (int p = 0; p < P; ++p)
        if (s_sel[p] == e) R.pairs[j++] = p;
    }
    c0 += cnt[q];
    f0 += flag[q];
  }
}

// ------------------------------------------------------------------ the experts' products
// grid.x: blocks of 4 waves x R weight rows; grid.y: used-expert slot u (blocks past the number of
// used experts leave at once). A block takes its expert's tokens BM at a time: their activation
// rows (FF1: h of the token; FF2: f of the pair) are staged in LDS as LT, K in chunks that fit the
// LDS budget, and every weight row of the block is streamed once per BM tokens. FF1's epilogue adds
// b1 and applies GeLU into f (fp32); FF2's adds b2 into z (fp32), one row per (token, slot) pair.
template <typename WT, typename AT, bool FF1, int BM, int R>
__global__ __launch_bounds__(256) void moe_ffn_kernel(const MoeArgs a) {
  typedef typename WTraits<WT>::LT LT;
  constexpr int E8 = WTraits<WT>::E;
  extern __shared__ __align__(16) unsigned char smem_raw[];
  LT* act = reinterpret_cast<LT*>(smem_raw);
  const int u = blockIdx.y;
  Route RT(a.route, a.umax);
  if (u >= *RT.n_used) return;
  const int e = RT.used[u], cnt = RT.cnt[u], first = RT.start[u];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int H = a.H, F = a.F, KS = a.KS;
  const int N = FF1 ? F : H, K = FF1 ? H : F;
  const bool res = e >= a.E;
  const size_t mat = (size_t)F * H;
  const WT* W;
  const half_t* S = nullptr;
  const void* bias;
  size_t boff;
  if (FF1) {
    W = static_cast<const WT*>(res ? a.r_w1 : a.w1) + (res ? 0 : (size_t)e * mat);
    if (sizeof(WT) == 1) S = static_cast<const half_t*>(res ? a.r_s1 : a.s1) + (res ? 0 : (size_t)e * (mat / a.group));
    bias = res ? a.r_b1 : a.b1;
    boff = res ? 0 : (size_t)e * F;
  } else {
    W = static_cast<const WT*>(res ? a.r_w2 : a.w2) + (res ? 0 : (size_t)e * mat);
    if (sizeof(WT) == 1) S = static_cast<const half_t*>(res ? a.r_s2 : a.s2) + (res ? 0 : (size_t)e * (mat / a.group));
    bias = res ? a.r_b2 : a.b2;
    boff = res ? 0 : (size_t)e * H;
  }
  const int row0 = (blockIdx.x * 4 + wave) * R;
  const int nrows = N - row0;
  int KC = kMoeLdsAct / (BM * (int)sizeof(LT));
  KC = KC / (kWave * E8) * (kWave * E8);
  if (KC > K) KC = K;

  for (int c0 = 0; c0 < cnt; c0 += BM) {
    const int nb = min(BM, cnt - c0);
    float acc[R][BM];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int b = 0; b < BM; ++b) acc[r][b] = 0.f;
    for (int kbeg = 0; kbeg < K; kbeg += KC) {
      const int kend = min(K, kbeg + KC), len = kend - kbeg;
      __syncthreads();  // the previous chunk's activation rows are consumed
      for (int idx = tid; idx < BM * len; idx += 256) {
        const int b = idx / len, kk = idx - b * len;
        LT v = (LT)0.f;
        if (b < nb) {
          const int p = RT.pairs[first + c0 + b];
          if (FF1) v = reinterpret_cast<const LT*>(a.h)[(size_t)(p / KS) * H + kbeg + kk];
          else v = (LT)a.f[(size_t)p * F + kbeg + kk];
        }
        act[b * KC + kk] = v;
      }
      __syncthreads();
      if (nrows > 0) gemv_rows<WT, R, BM, 4>(W, S, K, a.group, row0, nrows, kbeg, kend, act, KC, acc, lane);
    }
    if (nrows > 0) {
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int b = 0; b < BM; ++b) acc[r][b] = wave_sum(acc[r][b]);
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int b = 0; b < BM; ++b) {
          if (lane != r * BM + b || r >= nrows || b >= nb) continue;
          const int n = row0 + r, p = RT.pairs[first + c0 + b];
          const float z = acc[r][b] + ldm<AT>(bias, boff + n);
          if (FF1) a.f[(size_t)p * F + n] = gelu(z, a.gelu_tanh != 0);
          else a.z[(size_t)p * H + n] = z;
        }
    }
  }
}

// ------------------------------------------------------------------ combination
// One workgroup per token: y = x2 + sum over its slots, in slot order, of weight x expert output.
template <typename AT>
__global__ __launch_bounds__(256) void moe_combine_kernel(const MoeArgs a) {
  const int t = blockIdx.x, H = a.H, KS = a.KS;
  for (int c = threadIdx.x; c < H; c += 256) {
    float v = ldm<AT>(a.x2, (size_t)t * H + c);
    for (int i = 0; i < KS; ++i) v += a.wgt[(size_t)t * KS + i] * a.z[((size_t)t * KS + i) * H + c];
    reinterpret_cast<AT*>(a.y)[(size_t)t * H + c] = from_f32<AT>(v);
  }
}

template <typename WT, typename AT, bool FF1, int BM>
hipError_t launch_ffn_bm(const MoeArgs& a, hipStream_t st) {
  constexpr int R = 2;
  typedef typename WTraits<WT>::LT LT;
  constexpr int E8 = WTraits<WT>::E;
  const int K = FF1 ? a.H : a.F, N = FF1 ? a.F : a.H;
  int KC = kMoeLdsAct / (BM * (int)sizeof(LT));
  KC = KC / (kWave * E8) * (kWave * E8);
  if (KC > K) KC = K;
  dim3 grid((N + 4 * R - 1) / (4 * R), a.umax);
  hipLaunchKernelGGL((moe_ffn_kernel<WT, AT, FF1, BM, R>), grid, dim3(256), (size_t)BM * KC * sizeof(LT), st, a);
  return hipGetLastError();
}

template <typename WT, typename AT, bool FF1>
hipError_t launch_ffn(const MoeArgs& a, hipStream_t st) {
  // tokens per expert are known only on the device: the batch tile covers every token of the
  // step up to 8, larger counts loop over tiles of 8
  if (a.T >= 5) return launch_ffn_bm<WT, AT, FF1, 8>(a, st);
  if (a.T >= 3) return launch_ffn_bm<WT, AT, FF1, 4>(a, st);
  if (a.T == 2) return launch_ffn_bm<WT, AT, FF1, 2>(a, st);
  return launch_ffn_bm<WT, AT, FF1, 1>(a, st);
}

template <typename WT, typename AT>
hipError_t launch_moe_t(const MoeArgs& a, hipStream_t st, MoeKernelHook hook, void* hook_ctx) {
  typedef typename WTraits<WT>::LT LT;
  const size_t lds_gate = ((size_t)a.H + (size_t)a.E) * sizeof(float);
  hipLaunchKernelGGL((moe_gate_kernel<AT, LT>), dim3(a.T), dim3(256), lds_gate, st, a);
  if (hipError_t e = hipGetLastError()) return e;
  if (hook) hook(hook_ctx, st, 0);
  hipLaunchKernelGGL(moe_route_kernel, dim3(1), dim3(256), 0, st, a);
  if (hipError_t e = hipGetLastError()) return e;
  if (hook) hook(hook_ctx, st, 1);
  if (hipError_t e = launch_ffn<WT, AT, true>(a, st)) return e;
  if (hook) hook(hook_ctx, st, 2);
  if (hipError_t e = launch_ffn<WT, AT, false>(a, st)) return e;
  if (hook) hook(hook_ctx, st, 3);
  hipLaunchKernelGGL((moe_combine_kernel<AT>), dim3(a.T), dim3(256), 0, st, a);
  if (hipError_t e = hipGetLastError()) return e;
  if (hook) hook(hook_ctx, st, 4);
  return hipSuccess;
}

}  // namespace

hipError_t launch_moe(Dt wdt, Dt adt, const MoeArgs& a, hipStream_t st, MoeKernelHook hook, void* hook_ctx) {
  if (wdt == F16 && adt == F16) return launch_moe_t<half_t, half_t>(a, st, hook, hook_ctx);
  if (wdt == BF16 && adt == BF16) return launch_moe_t<bf16_t, bf16_t>(a, st, hook, hook_ctx);
  if (wdt == I8 && adt == F16) return launch_moe_t<int8_t, half_t>(a, st, hook, hook_ctx);
  if (wdt == F32 && adt == F32) return launch_moe_t<float, float>(a, st, hook, hook_ctx);
  return hipErrorInvalidValue;
}

}  // namespace ds
