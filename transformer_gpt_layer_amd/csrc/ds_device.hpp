// ds_device.hpp -- device helpers shared by the gfx950 kernels of libdslayer.so:
// 16-byte vector loads, wave64 reductions, fp16 and bf16 packing, int8 -> fp16 conversion, GeLU.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ds {

typedef _Float16 half_t;
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16_t;
typedef __bf16 bf162_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float2_t __attribute__((ext_vector_type(2)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// ---------------------------------------------------------------- loads
// Weight streams are read once per step: mark them non-temporal so they do not evict the small,
// reused activation and cache lines from L2.
__device__ __forceinline__ u32x4 ld_stream16(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }

template <typename T> __device__ __forceinline__ float to_f32(T v) { return static_cast<float>(v); }

// ---------------------------------------------------------------- wave64 reductions
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, kWave));
  return v;
}
// Sum over the wave with DPP lane moves instead of LDS permutes: prefix sums within each 16-lane
// row (row_shr 1, 2, 4, 8), then row 0's total into row 1 and row 2's into row 3 (row_bcast:15),
// then rows 0-1's total into rows 2-3 (row_bcast:31); lane 63 ends with the wave total, which
// readlane hands to every lane. Lanes whose DPP source lies outside the row keep adding 0.
template <int kCtrl, int kRowMask> __device__ __forceinline__ float dpp_add(float v) {
  return v + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), kCtrl, kRowMask, 0xf, false));
}
__device__ __forceinline__ float wave_sum_dpp(float v) {
  v = dpp_add<0x111, 0xf>(v);  // row_shr:1
  v = dpp_add<0x112, 0xf>(v);  // row_shr:2
  v = dpp_add<0x114, 0xf>(v);  // row_shr:4
  v = dpp_add<0x118, 0xf>(v);  // row_shr:8
  v = dpp_add<0x142, 0xa>(v);  // row_bcast:15 into rows 1 and 3
  v = dpp_add<0x143, 0xc>(v);  // row_bcast:31 into rows 2 and 3
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}

// Sum over aligned groups of G lanes (G a power of two <= 64); every lane gets its group's sum.
template <int G> __device__ __forceinline__ float group_sum(float v) {
#pragma unroll
  for (int off = G / 2; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

// Block-wide sum for a 256-thread block; `red` is 4 floats of LDS. All threads get the result.
__device__ __forceinline__ float block_sum256(float v, float* red) {
  v = wave_sum(v);
  const int wave = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[wave] = v;
  __syncthreads();
  return red[0] + red[1] + red[2] + red[3];
}

// ---------------------------------------------------------------- fp16 packing
// Bit casts take their operand by value: __builtin_bit_cast applied directly to an ext-vector
// component (v.y) reads the vector's first component instead, so components are copied first.
__device__ __forceinline__ half2_t as_half2(uint32_t u) { return __builtin_bit_cast(half2_t, u); }
__device__ __forceinline__ float as_f32(uint32_t u) { return __builtin_bit_cast(float, u); }

__device__ __forceinline__ bf162_t as_bf162(uint32_t u) { return __builtin_bit_cast(bf162_t, u); }

// Two packed 16-bit values (element 0 in the low half) of type T as floats, and back (RNE).
// bf16 widens exactly by a 16-bit shift.
template <typename T> __device__ __forceinline__ float lo16(uint32_t u) {
  if constexpr (__is_same(T, half_t)) return (float)as_half2(u).x;
  else return as_f32(u << 16);
}
template <typename T> __device__ __forceinline__ float hi16(uint32_t u) {
  if constexpr (__is_same(T, half_t)) return (float)as_half2(u).y;
  else return as_f32(u & 0xffff0000u);
}
template <typename T> __device__ __forceinline__ uint32_t pack16(float lo, float hi) {
  if constexpr (__is_same(T, half_t)) {
    const half2_t h = {(half_t)lo, (half_t)hi};
    return __builtin_bit_cast(uint32_t, h);
  } else {
    const bf162_t h = {(bf16_t)lo, (bf16_t)hi};
    return __builtin_bit_cast(uint32_t, h);
  }
}

// dot of 8 bf16 weights (one 16-byte load) with 8 bf16 activations, accumulated in fp32
__device__ __forceinline__ float dot8_bf16(u32x4 w, u32x4 a, float acc) {
  acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf162(w.x), as_bf162(a.x), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf162(w.y), as_bf162(a.y), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf162(w.z), as_bf162(a.z), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf162(w.w), as_bf162(a.w), acc, false);
  return acc;
}

// dot of 8 fp16 weights (one 16-byte load) with 8 fp16 activations, accumulated in fp32
__device__ __forceinline__ float dot8_f16(u32x4 w, u32x4 a, float acc) {
  acc = __builtin_amdgcn_fdot2(as_half2(w.x), as_half2(a.x), acc, false);
  acc = __builtin_amdgcn_fdot2(as_half2(w.y), as_half2(a.y), acc, false);
  acc = __builtin_amdgcn_fdot2(as_half2(w.z), as_half2(a.z), acc, false);
  acc = __builtin_amdgcn_fdot2(as_half2(w.w), as_half2(a.w), acc, false);
  return acc;
}

// dot of 8 16-bit weights with 8 activations of the same type (fp16 or bf16)
template <typename T> __device__ __forceinline__ float dot8(u32x4 w, u32x4 a, float acc);
template <> __device__ __forceinline__ float dot8<half_t>(u32x4 w, u32x4 a, float acc) { return dot8_f16(w, a, acc); }
template <> __device__ __forceinline__ float dot8<bf16_t>(u32x4 w, u32x4 a, float acc) { return dot8_bf16(w, a, acc); }

// An LDS address for the direct-to-LDS buffer loads (the generic pointer of a __shared__ object
// carries its LDS offset in the low 32 bits).
typedef __attribute__((address_space(3))) void lds_void;
__device__ __forceinline__ lds_void* lds_ptr(const void* p) {
  return reinterpret_cast<lds_void*>(reinterpret_cast<uintptr_t>(p));
}

// int8 -> fp16, exactly: with the byte offset to unsigned u = q + 128, the fp16 bit pattern
// 0x6400 | u encodes 1024 + u (in [1024, 2048) the fp16 spacing is 1), so subtracting
// 1152 = 1024 + 128 leaves q exactly. Two bytes of `w` (selected by `hi`) become one half2.
// One v_perm_b32 builds both halves: over the byte string {0x64 x 4 (bytes 4-7), w (bytes 0-3)}
// it picks bytes (u0, 0x64, u1, 0x64) from the low (selector 0x04010400) or high (0x04030402)
// pair of w.
__device__ __forceinline__ half2_t i8pair_to_half2(uint32_t w_biased, bool hi) {
  const uint32_t bits = __builtin_amdgcn_perm(0x64646464u, w_biased, hi ? 0x04030402u : 0x04010400u);
  const half2_t off = {(half_t)1152.0f, (half_t)1152.0f};
  return as_half2(bits) - off;
}

// dot of 16 int8 codes (one 16-byte load) with 16 fp16 activations (two 16-byte LDS reads),
// fp32 accumulation; the group scale is applied by the caller.
__device__ __forceinline__ float dot16_i8(u32x4 w, u32x4 a0, u32x4 a1) {
  const uint32_t flip = 0x80808080u;  // q + 128 for every byte
  uint32_t w0 = w.x ^ flip, w1 = w.y ^ flip, w2 = w.z ^ flip, w3 = w.w ^ flip;
  float acc = 0.f;
  acc = __builtin_amdgcn_fdot2(i8pair_to_half2(w0, false), as_half2(a0.x), acc, false);
  acc = __builtin_amdgcn_fdot2(i8pair_to_half2(w0, true), as_half2(a0.y), acc, false);
  acc = __builtin_amdgcn_fdot2(i8pair_to_half2(w1, false), as_half2(a0.z), acc, false);
  acc = __builtin_amdgcn_fdot2(i8pair_to_half2(w1, true), as_half2(a0.w), acc, false);
  acc = __builtin_amdgcn_fdot2(i8pair_to_half2(w2, false), as_half2(a1.x), acc, false);
  acc = __builtin_amdgcn_fdot2(i8pair_to_half2(w2, true), as_half2(a1.y), acc, false);
  acc = __builtin_amdgcn_fdot2(i8pair_to_half2(w3, false), as_half2(a1.z), acc, false);
  acc = __builtin_amdgcn_fdot2(i8pair_to_half2(w3, true), as_half2(a1.w), acc, false);
  return acc;
}

// dot of 4 fp32 weights with 4 fp32 activations
__device__ __forceinline__ float dot4_f32(u32x4 w, float4_t a, float acc) {
  acc = fmaf(as_f32(w.x), a.x, acc);
  acc = fmaf(as_f32(w.y), a.y, acc);
  acc = fmaf(as_f32(w.z), a.z, acc);
  acc = fmaf(as_f32(w.w), a.w, acc);
  return acc;
}

// ---------------------------------------------------------------- int8 quantization
// IEEE 754 binary16 bits of a double, round to nearest, ties to even, built directly on the
// double's bit fields: keep 10 fraction bits below the leading one (fewer in the subnormal range
// below 2^-14), round on the discarded bits, and let a carry ripple into the exponent field.
__device__ inline uint16_t f64_to_f16_bits_rne(double v) {
  const uint64_t u = (uint64_t)__double_as_longlong(v);
  const uint16_t sign = (uint16_t)((u >> 48) & 0x8000u);
  const uint64_t mag = u & 0x7fffffffffffffffull;
  if (mag >= 0x7ff0000000000000ull) return sign | (mag > 0x7ff0000000000000ull ? 0x7e00u : 0x7c00u);
  if (mag == 0) return sign;
  const int e = (int)(mag >> 52) - 1023;
  if (e > 15) return sign | 0x7c00u;
  if (e < -25) return sign;  // below 2^-25, half the smallest subnormal: rounds to zero
  const uint64_t m = (mag & ((1ull << 52) - 1)) | (1ull << 52);  // doubles this small are normal
  const int shift = (e >= -14) ? 42 : 42 + (-14 - e);
  uint64_t q = m >> shift;
  const uint64_t rem = m & ((1ull << shift) - 1), halfway = 1ull << (shift - 1);
  if (rem > halfway || (rem == halfway && (q & 1))) ++q;
  uint32_t bits = (e >= -14) ? (uint32_t)(((e + 14) << 10) + q) : (uint32_t)q;
  if (bits >= 0x7c00u) bits = 0x7c00u;
  return sign | (uint16_t)bits;
}

__device__ __forceinline__ double f16_bits_to_f64(uint16_t h) {
  return (double)(float)__builtin_bit_cast(half_t, h);
}

// Byte i (0..3) of w as a signed int8 value.
__device__ __forceinline__ float i8_at(uint32_t w, int i) { return (float)(int)(int8_t)(uint8_t)(w >> (8 * i)); }

// One value's int8 code under the fp16 scale sv (as a double): clamp(rint(x / sv), -127, 127),
// 0 for a zero scale. With amax in double and sv = fp16_RNE(amax / 127) this is the group-wise
// weight quantizer's rule; the KV cache uses it with one group per cached row of one head.
__device__ __forceinline__ int32_t i8_code(double x, double sv) {
  const double c = sv == 0.0 ? 0.0 : rint(x / sv);
  return (int32_t)fmin(127.0, fmax(-127.0, c));
}

// ---------------------------------------------------------------- GeLU
// u * Phi(u) = u/2 (1 + erf(u / sqrt 2)), or the tanh approximation
// u/2 (1 + tanh(sqrt(2/pi) (u + 0.044715 u^3))); erf and tanh come from the ROCm device library.
__device__ __forceinline__ float gelu(float u, bool tanh_form) {
  if (tanh_form) {
    const float c = 0.7978845608028654f;  // sqrt(2/pi)
    return 0.5f * u * (1.f + tanhf(c * (u + 0.044715f * u * u * u)));
  }
  return 0.5f * u * (1.f + erff(u * 0.7071067811865476f));
}

// ---------------------------------------------------------------- weight element traits
// E: weight elements per 16-byte load; LT: type of the staged activation the weights meet.
template <typename WT> struct WTraits;
template <> struct WTraits<float> { static constexpr int E = 4; typedef float LT; };
template <> struct WTraits<half_t> { static constexpr int E = 8; typedef half_t LT; };
template <> struct WTraits<bf16_t> { static constexpr int E = 8; typedef bf16_t LT; };
template <> struct WTraits<int8_t> { static constexpr int E = 16; typedef half_t LT; };

// ---------------------------------------------------------------- stores in the activation type
template <typename T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ half_t from_f32<half_t>(float v) { return (half_t)v; }
template <> __device__ __forceinline__ bf16_t from_f32<bf16_t>(float v) { return (bf16_t)v; }

}  // namespace ds
