// ds_gemv.hpp -- the wave GEMV core shared by the per-layer GEMV kernels and the MoE expert
// kernels: one wave64 owns R weight rows, its lanes split K in 16-byte pieces (E elements), and
// the BM activation rows it meets sit in LDS.
#pragma once
#include "ds_device.hpp"

namespace ds {

// ------------------------------------------------------------------ wave GEMV core
// acc[r][b] += sum_{k in [kbeg,kend)} W[row0 + r][k] * act[b][k - kbeg]   (one wave, 64 lanes)
template <typename WT, int R, int BM, int U>
__device__ __forceinline__ void gemv_rows(const WT* __restrict__ W, const half_t* __restrict__ S,
                                          int K, int group, int row0, int nrows, int kbeg, int kend,
                                          const typename WTraits<WT>::LT* act, int act_stride,
                                          float (&acc)[R][BM], int lane) {
  typedef typename WTraits<WT>::LT LT;
  constexpr int E = WTraits<WT>::E;
  constexpr int STEP = kWave * E;
  const WT* wrow[R];
  const half_t* srow[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int row = row0 + (r < nrows ? r : nrows - 1);  // surplus rows re-read a valid row
    wrow[r] = W + (size_t)row * K;
    srow[r] = S ? S + (size_t)row * (K / group) : nullptr;
  }
  int k = kbeg + lane * E;
  auto consume = [&](const u32x4 (&w)[R], const float (&sc)[R], int kk) {
#pragma unroll
    for (int b = 0; b < BM; ++b) {
      const LT* ap = act + b * act_stride + (kk - kbeg);
      if constexpr (sizeof(WT) == 4) {
        const float4_t a4 = *reinterpret_cast<const float4_t*>(ap);
#pragma unroll
        for (int r = 0; r < R; ++r) acc[r][b] = dot4_f32(w[r], a4, acc[r][b]);
      } else if constexpr (sizeof(WT) == 2) {
        const u32x4 a8 = *reinterpret_cast<const u32x4*>(ap);
#pragma unroll
        for (int r = 0; r < R; ++r) acc[r][b] = dot8<WT>(w[r], a8, acc[r][b]);
      } else {
        const u32x4 a0 = *reinterpret_cast<const u32x4*>(ap);
        const u32x4 a1 = *reinterpret_cast<const u32x4*>(ap + 8);
#pragma unroll
        for (int r = 0; r < R; ++r) acc[r][b] = fmaf(dot16_i8(w[r], a0, a1), sc[r], acc[r][b]);
      }
    }
  };
  for (; k + (U - 1) * STEP < kend; k += U * STEP) {
    u32x4 w[U][R];
    float sc[U][R];
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int r = 0; r < R; ++r) {
        w[u][r] = ld_stream16(wrow[r] + k + u * STEP);
        if constexpr (sizeof(WT) == 1) sc[u][r] = (float)srow[r][(k + u * STEP) / group];
        else sc[u][r] = 1.f;
      }
#pragma unroll
    for (int u = 0; u < U; ++u) consume(w[u], sc[u], k + u * STEP);
  }
  for (; k < kend; k += STEP) {
    u32x4 w[R];
    float sc[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      w[r] = ld_stream16(wrow[r] + k);
      if constexpr (sizeof(WT) == 1) sc[r] = (float)srow[r][k / group];
      else sc[r] = 1.f;
    }
    consume(w, sc, k);
  }
}

}  // namespace ds
