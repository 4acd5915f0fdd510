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
// grid (T, ceil(E / kGateExperts)): every workgroup normalizes its token's row (biased variance,
// two passes over the row in LDS; the workgroups of one token compute the same h), the first one
// stores h rounded to the staged type LT for the experts, and each wave takes kGateExperts / 4
// experts of the block, its lanes 16-byte pieces of the gate rows, against that same rounded h.
constexpr int kGateExperts = 4;

template <typename AT, typename LT>
__global__ __launch_bounds__(256) void moe_gate_kernel(const MoeArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  float* xs = reinterpret_cast<float*>(smem);  // [H]: the row, then h as the experts see it
  __shared__ float red[4];
  const int t = blockIdx.x, tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int H = a.H, E = a.E;
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
    if (blockIdx.y == 0) hrow[i] = hv;
    xs[i] = (float)hv;
  }
  __syncthreads();
  constexpr int EK = 16 / (int)sizeof(AT);
  const int e_end = min(E, (int)(blockIdx.y + 1) * kGateExperts);
  for (int e = blockIdx.y * kGateExperts + wave; e < e_end; e += 4) {
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
    if (lane == 0) a.logits[(size_t)t * E + e] = acc;
  }
}

// ------------------------------------------------------------------ top-k per token
// One wave per token (the routing workgroup's four waves take every fourth token): the softmax
// of the token's logits and k rounds of a wave-wide maximum of 64-bit keys (the probability's bits
// above the inverted expert index: the largest probability, the smallest index among equal ones),
// each lane keeping a bit mask of its experts already taken; then the combine weights.
__device__ void moe_topk_token(const MoeArgs& a, int t, int lane) {
  const int E = a.E, K = a.k, KS = a.KS;
  const float* lg = a.logits + (size_t)t * E;
  // the lane's logits (experts lane + 64 j) read once, all loads in flight together, then their
  // probabilities kept in registers for the k rounds
  constexpr int kPerLane = (kMoeMaxExperts + kWave - 1) / kWave;
  float pv[kPerLane];
#pragma unroll
  for (int j = 0; j < kPerLane; ++j) pv[j] = lane + kWave * j < E ? lg[lane + kWave * j] : -3.0e38f;
  float m = -3.0e38f;
#pragma unroll
  for (int j = 0; j < kPerLane; ++j) m = fmaxf(m, pv[j]);
  m = wave_max(m);
  float sum = 0.f;
#pragma unroll
  for (int j = 0; j < kPerLane; ++j) {
    if (lane + kWave * j < E) {
      pv[j] = expf(pv[j] - m);
      sum += pv[j];
    }
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
#pragma unroll
    for (int j = 0; j < kPerLane; ++j) {
      const int e = lane + kWave * j;
      if (e >= E || (taken & (1u << j))) continue;
      const uint64_t key = ((uint64_t)__builtin_bit_cast(uint32_t, pv[j]) << 32) | (uint64_t)(0xffffffffu - (uint32_t)e);
      best = key > best ? key : best;
    }
    best = wave_max_u64(best);
    const int e = (int)(0xffffffffu - (uint32_t)best);
    if ((e & (kWave - 1)) == lane) taken |= 1u << (e / kWave);
    esel[i] = e;
    psel[i] = __builtin_bit_cast(float, (uint32_t)(best >> 32)) / sum;
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
// One workgroup: the top-k of every token first, then expert e (of NE = E + residual) counts its
// pairs; exclusive scans over the
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
  for (int t = tid >> 6; t < a.T; t += 4) moe_topk_token(a, t, tid & 63);
  __syncthreads();  // every sel written by this workgroup is visible to it
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
// grid.x: blocks of (4 / KW) row groups of R weight rows; grid.y: used-expert slot u (blocks past
// the number of used experts leave at once). The KW waves of a row group split K (whole 64-lane
// steps; the last wave takes the remainder) and add their partial sums through LDS in wave order.
// A block takes its expert's tokens in tiles of BM, BM the smallest of 1, 2, 4, 8 that holds the
// expert's token count (chosen on the device; more than 8 loop over tiles of 8): their activation
// rows (FF1: h of the token; FF2: f of the pair, both already LT) are staged in LDS with 16-byte
// copies, K in chunks that fit the LDS budget, and every weight row of the block is streamed once
// per tile. FF1's epilogue adds b1 and applies GeLU into f (rounded to LT, as the fp16 GEMM path
// stores it); FF2's adds b2 into z (fp32), one row per (token, slot) pair.
template <typename WT, typename AT, bool FF1, int R, int KW, int BM>
__device__ __forceinline__ void ffn_tiles(const MoeArgs& a, const Route& RT, int first, int cnt, const WT* W,
                                          const half_t* S, const void* bias, size_t boff, unsigned char* smem) {
  typedef typename WTraits<WT>::LT LT;
  constexpr int E8 = WTraits<WT>::E, STEP = kWave * E8;
  constexpr int RG = 4 / KW;  // row groups per block
  LT* act = reinterpret_cast<LT*>(smem);
  float* red = reinterpret_cast<float*>(smem + a.lds_act);  // [4 waves][R][BM] partial sums
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int rg = wave / KW, kp = wave % KW;
  const int H = a.H, F = a.F, KS = a.KS;
  const int N = FF1 ? F : H, K = FF1 ? H : F;
  const int row0 = (blockIdx.x * RG + rg) * R;
  const int nrows = N - row0;
  // K chunk: the whole row when it fits, else whole K-split steps (the budget holds at least
  // 4096 two-byte or 2048 four-byte elements of 8 rows, a multiple of 4 x 512 and 4 x 256)
  int KC = a.lds_act / (BM * (int)sizeof(LT));
  KC = KC >= K ? K : KC / (KW * STEP) * (KW * STEP);
  for (int c0 = 0; c0 < cnt; c0 += BM) {
    const int nb = min(BM, cnt - c0);
    float acc[R][BM];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int b = 0; b < BM; ++b) acc[r][b] = 0.f;
    for (int kbeg = 0; kbeg < K; kbeg += KC) {
      const int kend = min(K, kbeg + KC), len = kend - kbeg;
      __syncthreads();  // the previous chunk's activation rows (and partial sums) are consumed
      // 16-byte copies: 8 LT elements (4 for fp32) per thread and step; len is a multiple of 64
      constexpr int V = 16 / (int)sizeof(LT);
      const int nv = len / V;
      for (int idx = tid; idx < BM * nv; idx += 256) {
        const int b = idx / nv, c = (idx - b * nv) * V;
        u32x4 v = u32x4{0u, 0u, 0u, 0u};
        if (b < nb) {
          const int p = RT.pairs[first + c0 + b];
          if (FF1) v = ld16(reinterpret_cast<const LT*>(a.h) + (size_t)(p / KS) * H + kbeg + c);
          else v = ld16(reinterpret_cast<const LT*>(a.f) + (size_t)p * F + kbeg + c);
        }
        *reinterpret_cast<u32x4*>(act + b * KC + c) = v;
      }
      __syncthreads();
      if (nrows > 0) {
        // this wave's share of the chunk: whole steps, the last wave the remainder
        const int steps = (len + STEP - 1) / STEP, per = (steps + KW - 1) / KW;
        const int kb = kbeg + min(len, kp * per * STEP), ke = kbeg + min(len, (kp + 1) * per * STEP);
        if (kb < ke) gemv_rows<WT, R, BM, 4>(W, S, K, a.group, row0, nrows, kb, ke, act + (kb - kbeg), KC, acc, lane);
      }
    }
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int b = 0; b < BM; ++b) acc[r][b] = wave_sum(acc[r][b]);
    if constexpr (KW > 1) {
      if (lane == 0) {
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
          for (int b = 0; b < BM; ++b) red[(wave * R + r) * BM + b] = acc[r][b];
      }
      __syncthreads();
      if (kp == 0) {
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
          for (int b = 0; b < BM; ++b) {
            float t = 0.f;
#pragma unroll
            for (int q = 0; q < KW; ++q) t += red[((wave + q) * R + r) * BM + b];
            acc[r][b] = t;
          }
      }
    }
    if (nrows > 0 && kp == 0) {
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int b = 0; b < BM; ++b) {
          if (lane != r * BM + b || r >= nrows || b >= nb) continue;
          const int n = row0 + r, p = RT.pairs[first + c0 + b];
          const float z = acc[r][b] + ldm<AT>(bias, boff + n);
          if (FF1) {
            reinterpret_cast<LT*>(a.f)[(size_t)p * F + n] = (LT)gelu(z, a.gelu_tanh != 0);
          } else if (a.KS == 1) {
            // one slot per token (top-1 without the residual MLP): the combination is this slot
            // alone, written here as the combination kernel would (pair p is token p)
            float v = ldm<AT>(a.x2, (size_t)p * H + n);
            v += a.wgt[p] * z;
            reinterpret_cast<AT*>(a.y)[(size_t)p * H + n] = from_f32<AT>(v);
          } else {
            a.z[(size_t)p * H + n] = z;
          }
        }
    }
  }
}

template <typename WT, typename AT, bool FF1, int R, int KW>
__global__ __launch_bounds__(256) void moe_ffn_kernel(const MoeArgs a) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  const int u = blockIdx.y;
  Route RT(a.route, a.umax);
  if (u >= *RT.n_used) return;
  const int e = RT.used[u], cnt = RT.cnt[u], first = RT.start[u];
  const bool res = e >= a.E;
  const size_t mat = (size_t)a.F * a.H;
  const WT* W;
  const half_t* S = nullptr;
  const void* bias;
  size_t boff;
  if (FF1) {
    W = static_cast<const WT*>(res ? a.r_w1 : a.w1) + (res ? 0 : (size_t)e * mat);
    if (sizeof(WT) == 1) S = static_cast<const half_t*>(res ? a.r_s1 : a.s1) + (res ? 0 : (size_t)e * (mat / a.group));
    bias = res ? a.r_b1 : a.b1;
    boff = res ? 0 : (size_t)e * a.F;
  } else {
    W = static_cast<const WT*>(res ? a.r_w2 : a.w2) + (res ? 0 : (size_t)e * mat);
    if (sizeof(WT) == 1) S = static_cast<const half_t*>(res ? a.r_s2 : a.s2) + (res ? 0 : (size_t)e * (mat / a.group));
    bias = res ? a.r_b2 : a.b2;
    boff = res ? 0 : (size_t)e * a.H;
  }
  // the tile that holds the expert's tokens (cnt is the same for the whole block)
  if (cnt <= 1) ffn_tiles<WT, AT, FF1, R, KW, 1>(a, RT, first, cnt, W, S, bias, boff, smem_raw);
  else if (cnt <= 2) ffn_tiles<WT, AT, FF1, R, KW, 2>(a, RT, first, cnt, W, S, bias, boff, smem_raw);
  else if (cnt <= 4) ffn_tiles<WT, AT, FF1, R, KW, 4>(a, RT, first, cnt, W, S, bias, boff, smem_raw);
  else ffn_tiles<WT, AT, FF1, R, KW, 8>(a, RT, first, cnt, W, S, bias, boff, smem_raw);
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

template <typename WT, typename AT, bool FF1, int R, int KW>
hipError_t launch_ffn_kw(const MoeArgs& a0, hipStream_t st) {
  typedef typename WTraits<WT>::LT LT;
  constexpr int RG = 4 / KW;
  MoeArgs a = a0;
  const int N = FF1 ? a.F : a.H, K = FF1 ? a.H : a.F;
  // activation rows for the largest tile any expert of this step can need (its token count is at
  // most the step's), within the budget: small tiles leave room for more workgroups per CU
  const int bm_max = a.T >= 5 ? 8 : (a.T >= 3 ? 4 : a.T);
  const size_t need = (size_t)bm_max * K * sizeof(LT);
  a.lds_act = (int)((need < (size_t)kMoeLdsAct ? need : (size_t)kMoeLdsAct) + 15) / 16 * 16;
  const size_t lds = (size_t)a.lds_act + 4 * R * 8 * sizeof(float);  // and the waves' partial sums
  dim3 grid((N + RG * R - 1) / (RG * R), a.umax);
  hipLaunchKernelGGL((moe_ffn_kernel<WT, AT, FF1, R, KW>), grid, dim3(256), lds, st, a);
  return hipGetLastError();
}

template <typename WT, typename AT, bool FF1>
hipError_t launch_ffn(const MoeArgs& a, hipStream_t st) {
  // few output rows over a long K (FF2: N = hidden, K = ffn): the four waves of a workgroup split
  // K over 4 rows, so that the launch has many workgroups while each stages its activation rows
  // for 4 weight rows; otherwise four row groups of 2 rows each (8 rows per staged activation)
  const int N = FF1 ? a.F : a.H, K = FF1 ? a.H : a.F;
  if (K >= 2 * N || N < 4096) return launch_ffn_kw<WT, AT, FF1, 4, 4>(a, st);
  return launch_ffn_kw<WT, AT, FF1, 2, 1>(a, st);
}

template <typename WT, typename AT>
hipError_t launch_moe_t(const MoeArgs& a, hipStream_t st, MoeKernelHook hook, void* hook_ctx) {
  typedef typename WTraits<WT>::LT LT;
  const size_t lds_gate = (size_t)a.H * sizeof(float);
  hipLaunchKernelGGL((moe_gate_kernel<AT, LT>), dim3(a.T, (a.E + kGateExperts - 1) / kGateExperts), dim3(256),
                     lds_gate, st, a);
  if (hipError_t e = hipGetLastError()) return e;
  if (hook) hook(hook_ctx, st, 0);
  hipLaunchKernelGGL(moe_route_kernel, dim3(1), dim3(256), 0, st, a);
  if (hipError_t e = hipGetLastError()) return e;
  if (hook) hook(hook_ctx, st, 1);
  if (hipError_t e = launch_ffn<WT, AT, true>(a, st)) return e;
  if (hook) hook(hook_ctx, st, 2);
  if (hipError_t e = launch_ffn<WT, AT, false>(a, st)) return e;
  if (hook) hook(hook_ctx, st, 3);
  if (a.KS > 1) {  // with one slot per token FF2 wrote y itself
    hipLaunchKernelGGL((moe_combine_kernel<AT>), dim3(a.T), dim3(256), 0, st, a);
    if (hipError_t e = hipGetLastError()) return e;
  }
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
