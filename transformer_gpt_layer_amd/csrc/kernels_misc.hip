// kernels_misc.hip -- KV-cache append, length advance, and the group-wise int8 weight quantizer.
//
// Source: int8 inference with group-wise quantization settings (quantize_groups) on the page
// "DeepSpeed Inference 内核优化深度解析" (blog.gitcode.com), section 五 5.2; the KV cache bounded by
// max_out_tokens (same page, section 四 4.2).
#include "ds_device.hpp"
#include "ds_launch.hpp"

namespace ds {

// ------------------------------------------------------------------ KV append
// k_new/v_new [batch][ntok][H] -> cache [batch][heads][cap][d] at rows d_len[b] + t (16 bytes per
// thread). Rows at or past capacity are skipped.
template <typename AT>
__global__ __launch_bounds__(256) void kv_append_kernel(const AT* __restrict__ kn, const AT* __restrict__ vn,
                                                        AT* kc, AT* vc, const int32_t* d_len, int batch,
                                                        int ntok, int heads, int d, int cap) {
  constexpr int EK = 16 / (int)sizeof(AT);
  const int H = heads * d;
  const size_t nvec = (size_t)batch * ntok * H / EK;
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= nvec) return;
  const size_t el = i * EK;
  const int b = (int)(el / ((size_t)ntok * H));
  const size_t rem = el - (size_t)b * ntok * H;
  const int t = (int)(rem / H), m = (int)(rem - (size_t)t * H);
  const int j = m / d, e = m - j * d;
  const int pos = d_len[b] + t;
  if (pos < 0 || pos >= cap) return;
  const size_t at = (((size_t)b * heads + j) * cap + pos) * d + e;
  *reinterpret_cast<u32x4*>(kc + at) = ld16(kn + el);
  *reinterpret_cast<u32x4*>(vc + at) = ld16(vn + el);
}

// ------------------------------------------------------------------ int8 KV rows
// One wave per (row r = b * ntok + t, head j, K or V): the head's d values of the new row (IT:
// fp32 from a projection epilogue, or the activation type for an append), their amax (exact in
// float), the row's fp16 scale and int8 codes (i8_code: the group-wise quantizer's rule with one
// group per row), into the cache row d_len[b] + t and its scale. Rows at or past capacity are
// skipped. d is 64 or 128: a lane holds one or two values.
template <typename IT>
__global__ __launch_bounds__(256) void kv_store_i8_kernel(const IT* __restrict__ ksrc, const IT* __restrict__ vsrc,
                                                          int stride, int8_t* kc, int8_t* vc, uint16_t* ks, uint16_t* vs,
                                                          const int32_t* d_len, int batch, int ntok, int heads, int d,
                                                          int cap) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const size_t item = (size_t)blockIdx.x * 4 + wave;  // (r * heads + j) * 2 + m
  if (item >= (size_t)batch * ntok * heads * 2) return;
  const int m = (int)(item & 1u);
  const size_t rj = item >> 1;
  const int j = (int)(rj % heads);
  const size_t r = rj / heads;
  const int b = (int)(r / ntok), t = (int)(r - (size_t)b * ntok);
  const int pos = d_len[b] + t;
  if (pos < 0 || pos >= cap) return;
  const IT* src = (m ? vsrc : ksrc) + r * stride + (size_t)j * d;
  const float x0 = lane < d ? to_f32(src[lane]) : 0.f;
  const float x1 = lane + 64 < d ? to_f32(src[lane + 64]) : 0.f;
  const float amax = wave_max(fmaxf(fabsf(x0), fabsf(x1)));
  const uint16_t sb = f64_to_f16_bits_rne((double)amax / 127.0);
  const double sv = f16_bits_to_f64(sb);
  const size_t row = ((size_t)b * heads + j) * cap + pos;
  int8_t* dst = (m ? vc : kc) + row * d;
  if (lane < d) dst[lane] = (int8_t)i8_code((double)x0, sv);
  if (lane + 64 < d) dst[lane + 64] = (int8_t)i8_code((double)x1, sv);
  if (lane == 0) (m ? vs : ks)[row] = sb;
}

hipError_t launch_kv_store_i8(Dt it, const void* ksrc, const void* vsrc, int stride, void* kc, void* vc, void* ks,
                              void* vs, const int32_t* d_len, int batch, int ntok, int heads, int head_dim, int cap,
                              hipStream_t st) {
  const size_t items = (size_t)batch * ntok * heads * 2;
  if (items == 0) return hipSuccess;
  const unsigned blocks = (unsigned)((items + 3) / 4);
  int8_t *k8 = static_cast<int8_t*>(kc), *v8 = static_cast<int8_t*>(vc);
  uint16_t *ks16 = static_cast<uint16_t*>(ks), *vs16 = static_cast<uint16_t*>(vs);
  if (it == F32)
    hipLaunchKernelGGL(kv_store_i8_kernel<float>, dim3(blocks), dim3(256), 0, st, (const float*)ksrc, (const float*)vsrc,
                       stride, k8, v8, ks16, vs16, d_len, batch, ntok, heads, head_dim, cap);
  else if (it == F16)
    hipLaunchKernelGGL(kv_store_i8_kernel<half_t>, dim3(blocks), dim3(256), 0, st, (const half_t*)ksrc,
                       (const half_t*)vsrc, stride, k8, v8, ks16, vs16, d_len, batch, ntok, heads, head_dim, cap);
  else if (it == BF16)
    hipLaunchKernelGGL(kv_store_i8_kernel<bf16_t>, dim3(blocks), dim3(256), 0, st, (const bf16_t*)ksrc,
                       (const bf16_t*)vsrc, stride, k8, v8, ks16, vs16, d_len, batch, ntok, heads, head_dim, cap);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

// Zero fill of a 16-byte aligned buffer whose size is a multiple of 16 bytes (a kernel rather than a
// memset node, so that it replays correctly inside captured graphs).
__global__ __launch_bounds__(256) void fill_zero_kernel(u32x4* p, size_t n16) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += (size_t)gridDim.x * 256)
    p[i] = u32x4{0u, 0u, 0u, 0u};
}

hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t st) {
  const size_t n16 = bytes / 16;
  if (n16 == 0) return hipSuccess;
  size_t blocks = (n16 + 255) / 256;
  if (blocks > 2048) blocks = 2048;
  hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)blocks), dim3(256), 0, st, static_cast<u32x4*>(p), n16);
  return hipGetLastError();
}

// A bounded GPU-side wait of `ticks` periods of the 100 MHz wall clock (one thread).
__global__ void delay_kernel(uint64_t ticks) {
  const uint64_t t0 = wall_clock64();
  while (wall_clock64() - t0 < ticks) __builtin_amdgcn_s_sleep(8);
}

hipError_t launch_delay(uint32_t microseconds, hipStream_t st) {
  hipLaunchKernelGGL(delay_kernel, dim3(1), dim3(1), 0, st, (uint64_t)microseconds * 100u);
  return hipGetLastError();
}

__global__ void len_advance_kernel(int32_t* d_len, int batch, int ntok, int cap) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b < batch && d_len[b] + ntok <= cap) d_len[b] += ntok;
}

hipError_t launch_kv_append(Dt adt, const void* k_new, const void* v_new, void* kc, void* vc,
                            const int32_t* d_len, int batch, int ntok, int heads, int head_dim,
                            int cap, hipStream_t st) {
  const size_t el = (size_t)batch * ntok * heads * head_dim;
  const int ek = adt == F32 ? 4 : 8;
  const size_t nvec = el / ek;
  if (nvec == 0) return hipSuccess;
  const unsigned blocks = (unsigned)((nvec + 255) / 256);
  if (adt == F32)
    hipLaunchKernelGGL(kv_append_kernel<float>, dim3(blocks), dim3(256), 0, st, (const float*)k_new,
                       (const float*)v_new, (float*)kc, (float*)vc, d_len, batch, ntok, heads, head_dim, cap);
  else  // fp16 and bf16: a copy of 16-bit elements
    hipLaunchKernelGGL(kv_append_kernel<half_t>, dim3(blocks), dim3(256), 0, st, (const half_t*)k_new,
                       (const half_t*)v_new, (half_t*)kc, (half_t*)vc, d_len, batch, ntok, heads, head_dim, cap);
  return hipGetLastError();
}

// Streaming read of a whole buffer: each workgroup reads a contiguous 32 KB span per pass (every
// thread eight nontemporal 16-byte loads in flight, 4 KB apart), folds what it read into one word,
// and each workgroup folds its words into *out with one atomic XOR, so the loads cannot be dropped.
// 2048 workgroups of 256 threads cover all CUs.
constexpr int kProbeGroups = 2048, kProbeThreads = 256, kProbeUnroll = 8;
__global__ __launch_bounds__(kProbeThreads) void read_probe_kernel(const u32x4* __restrict__ p, size_t n16, uint32_t* out) {
  constexpr size_t span = (size_t)kProbeThreads * kProbeUnroll;
  const size_t stride = (size_t)gridDim.x * span;
  size_t i = (size_t)blockIdx.x * span + threadIdx.x;
  uint32_t acc = 0;
  for (; i + (kProbeUnroll - 1) * kProbeThreads < n16; i += stride) {
    u32x4 v[kProbeUnroll];
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) v[u] = __builtin_nontemporal_load(p + i + u * kProbeThreads);
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  // the last, partial span: its pieces below n16
  for (int u = 0; u < kProbeUnroll; ++u) {
    const size_t j = i + (size_t)u * kProbeThreads;
    if (i < n16 && j < n16) {
      const u32x4 v = __builtin_nontemporal_load(p + j);
      acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
  }
  __shared__ uint32_t wg;
  if (threadIdx.x == 0) wg = 0u;
  __syncthreads();
  __hip_atomic_fetch_xor(&wg, acc, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  __syncthreads();
  if (threadIdx.x == 0) __hip_atomic_fetch_xor(out, wg, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

hipError_t launch_read_probe(const void* buf, size_t bytes, uint32_t* out, hipStream_t st) {
  hipLaunchKernelGGL(read_probe_kernel, dim3(kProbeGroups), dim3(kProbeThreads), 0, st, static_cast<const u32x4*>(buf),
                     bytes / 16, out);
  return hipGetLastError();
}

hipError_t launch_len_advance(int32_t* d_len, int batch, int ntok, int cap, hipStream_t st) {
  hipLaunchKernelGGL(len_advance_kernel, dim3((batch + 63) / 64), dim3(64), 0, st, d_len, batch, ntok, cap);
  return hipGetLastError();
}

// ------------------------------------------------------------------ int8 quantizer
// One thread per (row, group): amax in double, scale = fp16_RNE(amax/127), codes = clamp(rint(w/s)).
__global__ __launch_bounds__(256) void quantize_i8_kernel(const float* __restrict__ w, int8_t* __restrict__ q,
                                                          uint16_t* __restrict__ s, int n, int k, int group) {
  const int ng = k / group;
  const size_t gi = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (gi >= (size_t)n * ng) return;
  const size_t row = gi / ng, g = gi - row * ng;
  const float* src = w + row * k + g * group;
  int8_t* dst = q + row * k + g * group;
  double amax = 0.0;
  for (int i = 0; i < group; i += 4) {
    const float4_t v = *reinterpret_cast<const float4_t*>(src + i);
    amax = fmax(amax, fabs((double)v.x));
    amax = fmax(amax, fabs((double)v.y));
    amax = fmax(amax, fabs((double)v.z));
    amax = fmax(amax, fabs((double)v.w));
  }
  const uint16_t sb = f64_to_f16_bits_rne(amax / 127.0);
  s[gi] = sb;
  const double sv = f16_bits_to_f64(sb);
  for (int i = 0; i < group; i += 16) {
    uint32_t words[4];
#pragma unroll
    for (int wq = 0; wq < 4; ++wq) {
      uint32_t word = 0;
#pragma unroll
      for (int bq = 0; bq < 4; ++bq) {
        double c = sv == 0.0 ? 0.0 : rint((double)src[i + wq * 4 + bq] / sv);
        c = fmin(127.0, fmax(-127.0, c));
        word |= ((uint32_t)(int32_t)c & 0xffu) << (8 * bq);
      }
      words[wq] = word;
    }
    *reinterpret_cast<u32x4*>(dst + i) = u32x4{words[0], words[1], words[2], words[3]};
  }
}

// w = q * s through the same int8 -> fp16 conversion the GEMV kernels use (16 codes per thread; a
// run of 16 never straddles a scale group, whose size is a multiple of 16). OT: fp32, or fp16 (the
// product rounded once: the operand of the many-row GEMM for int8 layers).
template <typename OT>
__global__ __launch_bounds__(256) void dequantize_i8_kernel(const int8_t* __restrict__ q, const uint16_t* __restrict__ s,
                                                            OT* __restrict__ w, int n, int k, int group) {
  const size_t v = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (v >= (size_t)n * k / 16) return;
  const size_t el = v * 16, row = el / k, col = el - row * k;
  const float sc = (float)__builtin_bit_cast(half_t, s[row * (k / group) + col / group]);
  const u32x4 raw = ld16(q + el);
  const uint32_t words[4] = {raw.x ^ 0x80808080u, raw.y ^ 0x80808080u, raw.z ^ 0x80808080u, raw.w ^ 0x80808080u};
  float o[16];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const half2_t lo = i8pair_to_half2(words[i], false), hi = i8pair_to_half2(words[i], true);
    o[4 * i + 0] = (float)lo.x * sc;
    o[4 * i + 1] = (float)lo.y * sc;
    o[4 * i + 2] = (float)hi.x * sc;
    o[4 * i + 3] = (float)hi.y * sc;
  }
  if constexpr (sizeof(OT) == 4) {
#pragma unroll
    for (int e = 0; e < 16; ++e) w[el + e] = o[e];
  } else {
    uint32_t p[8];
#pragma unroll
    for (int e = 0; e < 8; ++e)
      p[e] = (uint32_t)__builtin_bit_cast(uint16_t, (OT)o[2 * e]) |
             ((uint32_t)__builtin_bit_cast(uint16_t, (OT)o[2 * e + 1]) << 16);
    u32x4* dst = reinterpret_cast<u32x4*>(w + el);
    dst[0] = u32x4{p[0], p[1], p[2], p[3]};
    dst[1] = u32x4{p[4], p[5], p[6], p[7]};
  }
}

hipError_t launch_quantize_i8(const float* w, int8_t* q, uint16_t* s, int n, int k, int group, hipStream_t st) {
  const size_t groups = (size_t)n * (k / group);
  if (groups == 0) return hipSuccess;
  hipLaunchKernelGGL(quantize_i8_kernel, dim3((unsigned)((groups + 255) / 256)), dim3(256), 0, st, w, q, s, n, k, group);
  return hipGetLastError();
}

hipError_t launch_dequantize_i8(const int8_t* q, const uint16_t* s, float* w, int n, int k, int group, hipStream_t st) {
  const size_t vecs = (size_t)n * k / 16;
  if (vecs == 0) return hipSuccess;
  hipLaunchKernelGGL(dequantize_i8_kernel<float>, dim3((unsigned)((vecs + 255) / 256)), dim3(256), 0, st, q, s, w, n, k,
                     group);
  return hipGetLastError();
}

hipError_t launch_dequantize_i8_f16(const int8_t* q, const uint16_t* s, half_t* w, int n, int k, int group,
                                    hipStream_t st) {
  const size_t vecs = (size_t)n * k / 16;
  if (vecs == 0) return hipSuccess;
  if (k % 16 || group % 16) return hipErrorInvalidValue;
  hipLaunchKernelGGL(dequantize_i8_kernel<half_t>, dim3((unsigned)((vecs + 255) / 256)), dim3(256), 0, st, q, s, w, n, k,
                     group);
  return hipGetLastError();
}

}  // namespace ds
