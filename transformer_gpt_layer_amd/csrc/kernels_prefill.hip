// kernels_prefill.hip -- the many-row path of one layer (prefill, or decode with a large batch) on
// gfx950 matrix cores, for fp16 weights and activations, or bf16 ones (the GEMM, skinny GEMM,
// LayerNorm and attention kernels take the 16-bit type as a template parameter; int8 weights go
// with fp16 activations).
//
// The layer is the one of the page "DeepSpeed Inference 内核优化深度解析" (blog.gitcode.com), section
// 三 3.2, with its four fusion regions. With many rows per weight the projections are dense GEMMs
// (the QKV, output, FF1 and FF2 GeMMs of section 三 3.2), so they run on MFMA; the regions' element-
// wise work rides in the GEMM epilogues:
//   ln_rows       LayerNorm of each row into a 16-bit copy (the A operand of the next GEMM)
//   gemm QKV      h Wqkv^T + b; q to the workspace, k and v straight into the head-major cache
//                 rows d_len[b] + t (the head "transform" of region 2 done by addressing)
//   attn_prefill  causal attention over the cache, flash style (online softmax), on MFMA
//   gemm OPROJ    x + ctx Wo^T + bo -> x2 (fp32)                              (region 3 start)
//   gemm FF1      GeLU(h2 W1^T + b1) -> f (16-bit)                            (region 3)
//   gemm FF2      x2 + f W2^T + b2 -> y                                       (region 4)
// The attention mask follows the triangular_masking option of the inference-config table on the
// page "DeepSpeed MoE 大规模稀疏模型推理实战指南" (blog.gitcode.com): with it, the row at absolute
// position p sees the keys 0..p; without it, every key of its sequence.
//
// GEMM design. C[M][N] = A[M][K] W[N][K]^T with both operands K-contiguous, which is the operand
// order v_mfma_f32_16x16x32_f16 wants (lane l holds row l%16, k 8(l/16)..+7 of either operand).
// A workgroup of four waves owns a 128 x BN tile, each wave a 64 x BN/2 quarter. K advances 64 at a
// time (whole 128-byte lines of each row) through an LDS ring filled by buffer loads that write LDS
// directly (no VGPR round trip); one barrier per k-step both publishes a stage and frees the
// oldest. LDS rows are 128 bytes with the 16-byte chunk index XOR-ed by row % 8, so the MFMA
// operand reads (16 rows, one chunk) hit distinct banks. Tiles are numbered so that the workgroups the dispatcher sends to
// one XCD (every 8th) hold consecutive tiles, which share their weight columns in that XCD's L2.
#include "ds_device.hpp"
#include "ds_launch.hpp"
#include "ds_prefill.hpp"

namespace ds {
namespace prefill {

typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int kRsrcFlags = 0x00020000;    // raw buffer, 32-bit dword format
constexpr uint32_t kOutOfRange = 0x80000000u;  // a buffer offset past every valid range: loads give 0

__device__ __forceinline__ rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, kRsrcFlags);
}


// s_waitcnt vmcnt(n) for 0 <= n <= 15 (expcnt and lgkmcnt left unconstrained); larger n waits
// for 15, which is stricter and therefore still correct.
template <int N> __device__ __forceinline__ void wait_vm() {
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
template <int N> __device__ __forceinline__ void wait_vm_upto(int n) {
  if constexpr (N == 0) {
    wait_vm<0>();
  } else {
    if (n >= N) wait_vm<N>();
    else wait_vm_upto<N - 1>(n);
  }
}
// s_waitcnt vmcnt(n) for a wave-uniform n (n above 47 waits for 47).
__device__ __forceinline__ void wait_vm_dyn(int n) { wait_vm_upto<47>(n); }

// Workgroup barrier that waits only for this wave's LDS operations, not for its outstanding global
// loads (a __syncthreads() would also drain the prefetched stages of the GEMM ring).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
}

// ------------------------------------------------------------------ LayerNorm rows
// One wave per row with 16-byte input loads: the mean, then the biased variance around it, then
// (x - mean) rstd g + b written as fp16. The second and third passes re-read the row from cache.
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

// The 16-bit activation type T of a layer on this path (fp16, or bf16 for bf16 layers): its
// vectors and its 16 x 16 x 32 product (both forms take the same operand layout on gfx950).
template <typename T> struct Act16;
template <> struct Act16<half_t> { typedef half8_t v8; typedef half4_t v4; };
template <> struct Act16<bf16_t> { typedef bf16x8_t v8; typedef bf16x4_t v4; };
template <typename T>
__device__ __forceinline__ float4_t mfma_16x16x32(typename Act16<T>::v8 a, typename Act16<T>::v8 b, float4_t c) {
  if constexpr (sizeof(T) == 2 && __is_same(T, bf16_t)) return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  else return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

template <int V, typename T> __device__ __forceinline__ void ld_halves(const T* p, float (&v)[V]) {
  if constexpr (V == 8) {
    const typename Act16<T>::v8 h = *reinterpret_cast<const typename Act16<T>::v8*>(p);
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = (float)h[e];
  } else {
    const typename Act16<T>::v4 h = *reinterpret_cast<const typename Act16<T>::v4*>(p);
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = (float)h[e];
  }
}
template <int V, typename IT> __device__ __forceinline__ void ld_row(const IT* p, float (&v)[V]) {
  if constexpr (sizeof(IT) == 4) {
    const float4_t f = *reinterpret_cast<const float4_t*>(p);
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = f[e];
  } else {
    ld_halves<V, IT>(p, v);
  }
}
template <int V, typename T> __device__ __forceinline__ void st_halves(T* p, const float (&v)[V]) {
  if constexpr (V == 8) {
    typename Act16<T>::v8 h;
#pragma unroll
    for (int e = 0; e < 8; ++e) h[e] = (T)v[e];
    *reinterpret_cast<typename Act16<T>::v8*>(p) = h;
  } else {
    typename Act16<T>::v4 h;
#pragma unroll
    for (int e = 0; e < 4; ++e) h[e] = (T)v[e];
    *reinterpret_cast<typename Act16<T>::v4*>(p) = h;
  }
}

template <typename T, typename IT>
__global__ __launch_bounds__(256) void ln_rows_kernel(const IT* __restrict__ x, const T* __restrict__ g,
                                                      const T* __restrict__ beta, T* __restrict__ out,
                                                      int rows, int H, float eps) {
  constexpr int V = 16 / (int)sizeof(IT);  // elements per 16-byte load
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (row >= rows) return;
  const IT* xr = x + (size_t)row * H;
  float v[V];
  float s = 0.f;
  for (int k = lane * V; k < H; k += kWave * V) {
    ld_row<V>(xr + k, v);
#pragma unroll
    for (int e = 0; e < V; ++e) s += v[e];
  }
  const float mean = wave_sum(s) / (float)H;
  float q = 0.f;
  for (int k = lane * V; k < H; k += kWave * V) {
    ld_row<V>(xr + k, v);
#pragma unroll
    for (int e = 0; e < V; ++e) q += (v[e] - mean) * (v[e] - mean);
  }
  const float rstd = rsqrtf(wave_sum(q) / (float)H + eps);
  T* o = out + (size_t)row * H;
  for (int k = lane * V; k < H; k += kWave * V) {
    float gv[V], bv[V];
    ld_row<V>(xr + k, v);
    ld_halves<V>(g + k, gv);
    ld_halves<V>(beta + k, bv);
#pragma unroll
    for (int e = 0; e < V; ++e) v[e] = (v[e] - mean) * rstd * gv[e] + bv[e];
    st_halves<V>(o + k, v);
  }
}

// A few rows (a decode step): one 256-thread workgroup per row holds the whole row in registers
// (up to NR 16-byte vectors per thread), so the statistics take one pass and one round trip: sums
// of d = x - x[0] and d^2 give the mean and the biased variance (shifting by an element of the row
// keeps the subtraction well conditioned).
// Optional length advance folded into a LayerNorm launch that runs after every reader of the
// lengths in this step: d_len[b] += ntok for b < batch, unless that would pass cap.
struct LenAdvance {
  int32_t* d_len;
  int batch, ntok, cap;
};
__device__ __forceinline__ void len_advance(const LenAdvance& la) {
  if (la.d_len && blockIdx.x == 0)
    for (int b = threadIdx.x; b < la.batch; b += blockDim.x)
      if (la.d_len[b] + la.ntok <= la.cap) la.d_len[b] += la.ntok;
}

// One wave per row with the whole row in registers (NR 16-byte pieces per lane): one pass over
// memory, exact two-pass statistics on the registers.
template <typename T, typename IT, int NR>
__global__ __launch_bounds__(256) void ln_rows_reg_kernel(const IT* __restrict__ x, const T* __restrict__ g,
                                                          const T* __restrict__ beta, T* __restrict__ out,
                                                          int rows, int H, float eps, const LenAdvance la) {
  constexpr int V = 16 / (int)sizeof(IT);
  len_advance(la);
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (row >= rows) return;
  const IT* xr = x + (size_t)row * H;
  const int nv = H / V;
  float v[NR][V];
#pragma unroll
  for (int j = 0; j < NR; ++j) {
    const int i = lane + j * kWave;
    if (i < nv) ld_row<V>(xr + i * V, v[j]);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < NR; ++j)
    if (lane + j * kWave < nv)
#pragma unroll
      for (int e = 0; e < V; ++e) s += v[j][e];
  const float mean = wave_sum(s) / (float)H;
  float q = 0.f;
#pragma unroll
  for (int j = 0; j < NR; ++j)
    if (lane + j * kWave < nv)
#pragma unroll
      for (int e = 0; e < V; ++e) q += (v[j][e] - mean) * (v[j][e] - mean);
  const float rstd = rsqrtf(wave_sum(q) / (float)H + eps);
  T* o = out + (size_t)row * H;
#pragma unroll
  for (int j = 0; j < NR; ++j) {
    const int i = lane + j * kWave;
    if (i < nv) {
      float gv[V], bv[V];
      ld_halves<V>(g + i * V, gv);
      ld_halves<V>(beta + i * V, bv);
#pragma unroll
      for (int e = 0; e < V; ++e) v[j][e] = (v[j][e] - mean) * rstd * gv[e] + bv[e];
      st_halves<V>(o + i * V, v[j]);
    }
  }
}

template <typename T, typename IT, int NR>
__global__ __launch_bounds__(256) void ln_row_wg_kernel(const IT* __restrict__ x, const T* __restrict__ g,
                                                       const T* __restrict__ beta, T* __restrict__ out, int H,
                                                       float eps, const LenAdvance la) {
  constexpr int V = 16 / (int)sizeof(IT);
  len_advance(la);
  __shared__ float red[2][4];
  const int tid = threadIdx.x, row = blockIdx.x;
  const IT* xr = x + (size_t)row * H;
  const int nv = H / V;
  float v[NR][V], gv[NR][V], bv[NR][V];
#pragma unroll
  for (int j = 0; j < NR; ++j) {
    const int i = tid + j * 256;
    if (i < nv) {
      ld_row<V>(xr + i * V, v[j]);
      ld_halves<V>(g + i * V, gv[j]);
      ld_halves<V>(beta + i * V, bv[j]);
    }
  }
  const float c0 = (float)xr[0];
  float s1 = 0.f, s2 = 0.f;
#pragma unroll
  for (int j = 0; j < NR; ++j)
    if (tid + j * 256 < nv)
#pragma unroll
      for (int e = 0; e < V; ++e) {
        const float d = v[j][e] - c0;
        s1 += d;
        s2 += d * d;
      }
  s1 = wave_sum(s1);
  s2 = wave_sum(s2);
  if ((tid & 63) == 0) {
    red[0][tid >> 6] = s1;
    red[1][tid >> 6] = s2;
  }
  __syncthreads();
  const float t1 = red[0][0] + red[0][1] + red[0][2] + red[0][3];
  const float t2 = red[1][0] + red[1][1] + red[1][2] + red[1][3];
  const float dm = t1 / (float)H;
  const float mean = c0 + dm;
  const float rstd = rsqrtf(fmaxf(t2 / (float)H - dm * dm, 0.f) + eps);
  T* o = out + (size_t)row * H;
#pragma unroll
  for (int j = 0; j < NR; ++j) {
    const int i = tid + j * 256;
    if (i < nv) {
#pragma unroll
      for (int e = 0; e < V; ++e) v[j][e] = (v[j][e] - mean) * rstd * gv[j][e] + bv[j][e];
      st_halves<V>(o + i * V, v[j]);
    }
  }
}

// ------------------------------------------------------------------ GEMM
// Workgroup tile BM x BN, four waves in a 2 x 2 grid (each a (BM/2) x (BN/2) quarter of 16 x 16
// MFMA blocks), k-steps of 64 staged through an ST-deep LDS ring by direct-to-LDS buffer loads.
// Each k-step is two halves of 32: the operand reads of one half are issued between the products
// of the other, and one barrier per k-step both publishes the next stage and frees the last one.
constexpr int kBK = 64;

// KG = 2 splits every k-step between two groups of four waves (one 32-wide half each) and adds
// the two partial tiles through LDS at the end: two waves per SIMD with one workgroup per CU.
constexpr int gemm_threads(int kg, int nwn) { return kWave * 2 * nwn * kg; }

template <int BM, int BN, int ST, int KG, int NWN = 2> struct GemmShape {
  static constexpr int NWM = 2, NQ = NWM * NWN;    // waves of one k-group: NWM x NWN grid
  static constexpr int THREADS = gemm_threads(KG, NWN);
  static constexpr int WM = BM / NWM, WN = BN / NWN;  // one wave's part
  static constexpr int FM = WM / 16, FN = WN / 16;  // 16x16 MFMA blocks per wave
  static constexpr int A_BYTES = BM * kBK * 2;
  static constexpr int STAGE = (BM + BN) * kBK * 2;
  static constexpr int LDS = ST * STAGE;
  static_assert(BM % (8 * NQ) == 0 && BN % (8 * NQ) == 0 && WM % 16 == 0 && WN % 16 == 0, "tile shape");
  static_assert(ST >= 2, "the ring needs two stages");
  static_assert(KG == 1 || (KG == 2 && LDS >= NQ * FM * FN * 1024), "the partial tiles must fit the ring");
};

// Swizzled byte offset of (row, 16-byte chunk) in a 128-byte-row LDS tile: chunk c of row r sits
// at position c ^ (r % 8), so 16 consecutive rows read at one chunk spread over all banks.
__device__ __forceinline__ uint32_t swz(int row, int chunk) {
  return (uint32_t)(row * 128 + ((chunk ^ (row & 7)) << 4));
}

// This wave's loads of one stage. Wave load j of the workgroup (j = wave + 4u) fills bytes
// [1024 j, 1024 j + 1024) of the stage with 8 rows of 128 bytes: A rows m0 + 8j + 0..7 for
// j < BM/8, then W rows n0 + 8(j - BM/8) + 0..7. Lane L carries row L/8, logical chunk
// (L%8) ^ (L/8), which lands at physical chunk L%8, as swz() expects; va / vw are the lane's byte
// offsets for u = 0 at k = 0. Rows past the matrix lie past the descriptor's size and load zeros.
// A k-step past the end (valid false) is requested out of range: it loads zeros into a stage that
// is never read, and keeps the number of loads per step fixed.
// With two wave groups, group 0 loads the A rows and group 1 the W rows (wave is then the index
// within the group).
template <int BM, int BN, bool DO_A, bool DO_W, int NQ>
__device__ __forceinline__ void issue_stage(unsigned char* stage, int wave, uint32_t koff, bool valid,
                                            const GemmArgs& g, uint32_t va, uint32_t vw, uint32_t row_step) {
  const rsrc_t ra = make_rsrc(g.a, (uint32_t)((size_t)g.M * g.K * 2));
  const rsrc_t rw = make_rsrc(g.w, (uint32_t)((size_t)g.N * g.K * 2));
  if constexpr (DO_A) {
#pragma unroll
    for (int u = 0; u < BM / (8 * NQ); ++u)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, lds_ptr(stage + (wave + NQ * u) * 1024), 16,
                                               valid ? va + u * row_step + koff : kOutOfRange, 0, 0, 0);
  }
  if constexpr (DO_W) {
#pragma unroll
    for (int u = 0; u < BN / (8 * NQ); ++u)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, lds_ptr(stage + BM * 128 + (wave + NQ * u) * 1024), 16,
                                               valid ? vw + u * row_step + koff : kOutOfRange, 0, 0, 0);
  }
}

// One wave's operands of one 32-wide half (ks) of a stage: FM A blocks and FN W blocks of 16 rows;
// lane l takes row l%16, k-chunk l/16 (8 halves), the MFMA operand layout.
template <typename T, typename S>
__device__ __forceinline__ void read_half(const unsigned char* stage, int ks, int arow, int brow, int fch,
                                          typename Act16<T>::v8 (&af)[S::FM], typename Act16<T>::v8 (&bf)[S::FN]) {
  typedef typename Act16<T>::v8 V8;
#pragma unroll
  for (int a = 0; a < S::FM; ++a)
    af[a] = *reinterpret_cast<const V8*>(stage + swz(arow + 16 * a, 4 * ks + fch));
#pragma unroll
  for (int b = 0; b < S::FN; ++b)
    bf[b] = *reinterpret_cast<const V8*>(stage + S::A_BYTES + swz(brow + 16 * b, 4 * ks + fch));
}

// The products of one half, with the FM + FN operand reads issued just before (for the other half)
// spread between them: one read after every second product.
template <typename T, typename S>
__device__ __forceinline__ void mfma_half(float4_t (&acc)[S::FM][S::FN], const typename Act16<T>::v8 (&af)[S::FM],
                                          const typename Act16<T>::v8 (&bf)[S::FN]) {
#pragma unroll
  for (int a = 0; a < S::FM; ++a)
#pragma unroll
    for (int b = 0; b < S::FN; ++b)
      acc[a][b] = mfma_16x16x32<T>(af[a], bf[b], acc[a][b]);
#pragma unroll
  for (int i = 0; i < S::FM + S::FN; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);  // two MFMAs
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
  }
  constexpr int rest = S::FM * S::FN - 2 * (S::FM + S::FN);
  static_assert(rest >= 0, "too few products per half to cover its reads");
  if constexpr (rest > 0) __builtin_amdgcn_sched_group_barrier(0x008, rest, 0);
}

template <typename T, int EPI>
__device__ __forceinline__ void epilogue_store(const GemmArgs& g, int m, int n, float acc) {
  if (m >= g.M || n >= g.N) return;
  const float z = acc + (float)reinterpret_cast<const T*>(g.bias)[n];
  if constexpr (EPI == EPI_QKV) {
    const int H = g.hidden;
    if (n < H) {
      static_cast<T*>(g.out)[(size_t)m * H + n] = (T)z;
    } else if (g.kv_new) {
      g.kv_new[(size_t)m * 2 * H + (n - H)] = z;
    } else {
      int nn = n - H;
      T* cache = reinterpret_cast<T*>(nn < H ? g.k_cache : g.v_cache);
      nn = nn < H ? nn : nn - H;
      const int j = nn / g.head_dim, e = nn - j * g.head_dim;
      const int b = m / g.tokens, t = m - b * g.tokens;
      const int pos = g.d_len[b] + t;
      if (pos >= 0 && pos < g.cap)  // the host rejects a full cache; a bad device length writes nothing
        cache[(((size_t)b * g.heads + j) * g.cap + pos) * g.head_dim + e] = (T)z;
    }
  } else if constexpr (EPI == EPI_OPROJ) {
    const size_t i = (size_t)m * g.N + n;
    static_cast<float*>(g.out)[i] = (float)static_cast<const T*>(g.resid)[i] + z;
  } else if constexpr (EPI == EPI_FF1) {
    static_cast<T*>(g.out)[(size_t)m * g.N + n] = (T)gelu(z, g.gelu_tanh != 0);
  } else {
    const size_t i = (size_t)m * g.N + n;
    static_cast<T*>(g.out)[i] = (T)(static_cast<const float*>(g.resid)[i] + z);
  }
}

// Epilogue of one wave's FM x FN blocks of 16 x 16 at rows mb.., columns nb..: lane l holds
// C[16a + 4(l/16) + r][16b + l%16]. Column terms (bias, destination) are computed once per column
// and row terms once per row.
template <typename T, int EPI, int FM, int FN>
__device__ __forceinline__ void epilogue(const GemmArgs& g, int mb, int nb, const float4_t (&acc)[FM][FN], int lane) {
  const T* gbias = reinterpret_cast<const T*>(g.bias);
  T* kc = reinterpret_cast<T*>(g.k_cache);
  T* vc = reinterpret_cast<T*>(g.v_cache);
  const int frow = lane & 15, fch = lane >> 4;
  float bias[FN];
  size_t col[FN];  // EPI_QKV: offset within the q row or within a sequence's head-major cache block
  int kind[FN];  // EPI_QKV: 0 q, 1 k cache, 2 v cache; all: -1 past N
#pragma unroll
  for (int b = 0; b < FN; ++b) {
    const int n = nb + 16 * b + frow;
    kind[b] = -1;
    col[b] = n;
    bias[b] = 0.f;
    if (n < g.N) {
      bias[b] = (float)gbias[n];
      kind[b] = 0;
      if constexpr (EPI == EPI_QKV) {
        const int H = g.hidden;
        if (n >= H) {
          int nn = n - H;
          kind[b] = nn < H ? 1 : 2;
          nn = nn < H ? nn : nn - H;
          const int j = nn / g.head_dim;
          col[b] = (size_t)j * g.cap * g.head_dim + (nn - j * g.head_dim);
        }
      }
    }
  }
#pragma unroll
  for (int a = 0; a < FM; ++a)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = mb + 16 * a + 4 * fch + r;
      if (m >= g.M) continue;
      if constexpr (EPI == EPI_QKV) {
        const int H = g.hidden;
        const int bb = m / g.tokens, t = m - bb * g.tokens;
        const int pos = g.d_len[bb] + t;
        // the host rejects a full cache; a bad device length writes no cache row
        const bool okc = pos >= 0 && pos < g.cap;
        const size_t rc = ((size_t)bb * g.heads * g.cap + (okc ? pos : 0)) * g.head_dim;
        T* q = static_cast<T*>(g.out) + (size_t)m * H;
#pragma unroll
        for (int b = 0; b < FN; ++b) {
          const float zf = acc[a][b][r] + bias[b];
          if (kind[b] == 0) q[col[b]] = (T)zf;
          else if (kind[b] > 0 && g.kv_new) g.kv_new[(size_t)m * 2 * H + (nb + 16 * b + frow - H)] = zf;
          else if (kind[b] > 0 && okc) (kind[b] == 1 ? kc : vc)[rc + col[b]] = (T)zf;
        }
      } else {
        const size_t row = (size_t)m * g.N;
#pragma unroll
        for (int b = 0; b < FN; ++b) {
          if (kind[b] < 0) continue;
          const float z = acc[a][b][r] + bias[b];
          const size_t i = row + col[b];
          if constexpr (EPI == EPI_OPROJ) {
            static_cast<float*>(g.out)[i] = (float)static_cast<const T*>(g.resid)[i] + z;
          } else if constexpr (EPI == EPI_FF1) {
            static_cast<T*>(g.out)[i] = (T)gelu(z, g.gelu_tanh != 0);
          } else {
            static_cast<T*>(g.out)[i] = (T)(static_cast<const float*>(g.resid)[i] + z);
          }
        }
      }
    }
}

// Loads of one stage by this wave (both operands, or its group's operand with two groups).
template <int BM, int BN, int KG, int NQ>
__device__ __forceinline__ void issue_mine(unsigned char* stage, int q, int grp, int j, int nk, const GemmArgs& g,
                                           uint32_t va, uint32_t vw, uint32_t row_step) {
  const uint32_t koff = (uint32_t)(j * kBK * 2);
  if constexpr (KG == 1) {
    issue_stage<BM, BN, true, true, NQ>(stage, q, koff, j < nk, g, va, vw, row_step);
  } else {
    if (grp == 0) issue_stage<BM, BN, true, false, NQ>(stage, q, koff, j < nk, g, va, vw, row_step);
    else issue_stage<BM, BN, false, true, NQ>(stage, q, koff, j < nk, g, va, vw, row_step);
  }
}

template <typename T, int BM, int BN, int ST, int KG, int NWN, int EPI>
__global__ __launch_bounds__(gemm_threads(KG, NWN)) void gemm_kernel(const GemmArgs g) {
  typedef GemmShape<BM, BN, ST, KG, NWN> S;
  typedef typename Act16<T>::v8 V8;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: load set-up stays scalar
  const int q = wave % S::NQ, grp = wave / S::NQ;  // wave of the k-group; k-group (KG = 2)
  const int wm = q % S::NWM, wn = q / S::NWM;

  // XCD-aware tile order: workgroup i runs on XCD i % 8; give each XCD a contiguous tile range.
  const int ntiles = g.tiles_m * g.tiles_n, i = blockIdx.x;
  const int x = i & 7, per = ntiles >> 3, rem = ntiles & 7;
  const int t = x * per + min(x, rem) + (i >> 3);
  const int tm = t % g.tiles_m, tn = t / g.tiles_m;
  const int m0 = tm * BM, n0 = tn * BN;
  const int K = g.K;

  const int lr = lane >> 3, lc = (lane & 7) ^ lr;
  const uint32_t row_step = (uint32_t)(8 * S::NQ * K * 2);  // NQ wave loads = 8 NQ rows
  const uint32_t va = (uint32_t)(((size_t)(m0 + 8 * q + lr) * K + lc * 8) * 2);
  const uint32_t vw = (uint32_t)(((size_t)(n0 + 8 * q + lr) * K + lc * 8) * 2);
  // this wave's wave loads per stage
  const int nl = KG == 1 ? (BM + BN) / (8 * S::NQ) : (grp == 0 ? BM / (8 * S::NQ) : BN / (8 * S::NQ));
  const int nk = K / kBK;
  float4_t acc[S::FM][S::FN];
#pragma unroll
  for (int a = 0; a < S::FM; ++a)
#pragma unroll
    for (int b = 0; b < S::FN; ++b) acc[a][b] = float4_t{0.f, 0.f, 0.f, 0.f};

  // k-step j lives in stage j % ST. Every step requests exactly one stage (out of range past the
  // end), so when step kt+1's stage must be complete, the loads allowed in flight are always the
  // ST - 2 stages requested after it.
#pragma unroll
  for (int s = 0; s < ST; ++s) issue_mine<BM, BN, KG, S::NQ>(smem + s * S::STAGE, q, grp, s, nk, g, va, vw, row_step);

  const int fch = lane >> 4;
  const int arow = wm * S::WM + (lane & 15), brow = wn * S::WN + (lane & 15);
  V8 a0[S::FM], b0[S::FN], a1[S::FM], b1[S::FN];
  wait_vm_dyn((ST - 1) * nl);
  lds_barrier();
  if constexpr (KG == 1) {
    read_half<T, S>(smem, 0, arow, brow, fch, a0, b0);
    for (int kt = 0; kt + 1 < nk; ++kt) {
      unsigned char* cur = smem + (kt % ST) * S::STAGE;
      read_half<T, S>(cur, 1, arow, brow, fch, a1, b1);
      mfma_half<T, S>(acc, a0, b0);
      // step kt+1's stage is in LDS and every wave has finished reading step kt's
      wait_vm_dyn((ST - 2) * nl);
      lds_barrier();
      issue_mine<BM, BN, KG, S::NQ>(cur, q, grp, kt + ST, nk, g, va, vw, row_step);
      read_half<T, S>(smem + ((kt + 1) % ST) * S::STAGE, 0, arow, brow, fch, a0, b0);
      mfma_half<T, S>(acc, a1, b1);
    }
    read_half<T, S>(smem + ((nk - 1) % ST) * S::STAGE, 1, arow, brow, fch, a1, b1);
    mfma_half<T, S>(acc, a0, b0);
    mfma_half<T, S>(acc, a1, b1);
  } else {
    // this group's half of step kt+1 is read under the products of step kt
    auto step = [&](int kt, V8 (&xa)[S::FM], V8 (&xb)[S::FN], V8 (&ya)[S::FM], V8 (&yb)[S::FN]) {
      wait_vm_dyn((ST - 2) * nl);
      lds_barrier();
      issue_mine<BM, BN, KG, S::NQ>(smem + (kt % ST) * S::STAGE, q, grp, kt + ST, nk, g, va, vw, row_step);
      read_half<T, S>(smem + ((kt + 1) % ST) * S::STAGE, grp, arow, brow, fch, ya, yb);
      mfma_half<T, S>(acc, xa, xb);
    };
    read_half<T, S>(smem, grp, arow, brow, fch, a0, b0);
    int kt = 0;
    for (; kt + 2 < nk; kt += 2) {
      step(kt, a0, b0, a1, b1);
      step(kt + 1, a1, b1, a0, b0);
    }
    if (kt + 1 < nk) {
      step(kt, a0, b0, a1, b1);
      mfma_half<T, S>(acc, a1, b1);
    } else {
      mfma_half<T, S>(acc, a0, b0);
    }
  }
  wait_vm<0>();  // the out-of-range requests past the end

  if constexpr (KG == 2) {
    // group 1 hands its partial tile to group 0 through the (now idle) ring
    float4_t* red = reinterpret_cast<float4_t*>(smem) + q * (S::FM * S::FN * 64) + lane;
    lds_barrier();
    if (grp == 1) {
#pragma unroll
      for (int a = 0; a < S::FM; ++a)
#pragma unroll
        for (int b = 0; b < S::FN; ++b) red[(a * S::FN + b) * 64] = acc[a][b];
    }
    lds_barrier();
    if (grp == 1) return;
#pragma unroll
    for (int a = 0; a < S::FM; ++a)
#pragma unroll
      for (int b = 0; b < S::FN; ++b) acc[a][b] += red[(a * S::FN + b) * 64];
  }
  epilogue<T, EPI, S::FM, S::FN>(g, m0 + wm * S::WM, n0 + wn * S::WN, acc, lane);
}

// ------------------------------------------------------------------ attention over the cache
// One workgroup per (sequence b, head j, 64 consecutive new rows); wave w owns rows 16w..16w+15.
// Computed transposed so that MFMA results feed the next MFMA without a layout change:
//   S^T[key][row] = K Q^T    (A = K rows from LDS, B = q rows from registers)
//   O^T[d][row]  += V^T P^T  (A = V^T, B = the probabilities, already in B layout)
// In S^T's accumulator layout a lane holds four keys of one row (column), and O^T's accumulators
// in a lane also all belong to that row, so the online-softmax rescale is per lane. V stays
// row-major in LDS; its transposed operand comes from ds_read_b64_tr_b16, which hands lane i of a
// 16-lane group element i%4 of the 8 bytes addressed by lane 4e + i/4 as its element e (checked
// on the device with an in-bounds probe).
constexpr int kAttnRows = 64, kAttnKeys = 64;

template <int D> struct AttnShape {
  static constexpr int KROW = D * 2;                     // bytes of one K row in LDS
  static constexpr int VROW = D * 2 + 32;                // bytes of one V row (padded: the four
                                                         // keys of a transposed read hit distinct banks)
  static constexpr int K_BYTES = kAttnKeys * KROW;
  static constexpr int LDS = K_BYTES + kAttnKeys * VROW;
};

typedef short short4_t __attribute__((ext_vector_type(4)));
typedef short short8_t __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) short4_t lds_short4;
__device__ __forceinline__ short4_t lds_read_tr16(const unsigned char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4*)(reinterpret_cast<uintptr_t>(p)));
}

template <int D> constexpr size_t attn_lds_bytes() { return (size_t)AttnShape<D>::LDS; }

template <typename T, int D, bool KV8>
__global__ __launch_bounds__(256) void attn_prefill_kernel(const AttnPrefillArgs g) {
  typedef AttnShape<D> S;
  typedef typename Act16<T>::v8 V8;
  constexpr int NCH = D / 8;  // 16-byte chunks per K row
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  unsigned char* Ks = smem;
  unsigned char* Vs = smem + S::K_BYTES;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int qtiles = (g.tokens + kAttnRows - 1) / kAttnRows;
  // causal tiles further down see more keys: launch them first so that the long ones do not
  // start last
  const int qt = qtiles - 1 - (int)(blockIdx.x % qtiles), bj = blockIdx.x / qtiles;
  const int j = bj % g.heads, b = bj / g.heads;
  const int H = g.heads * D;
  const int len = min(max(g.d_len[b], 0), g.cap);  // rows already in the cache before this call
  const int t0 = qt * kAttnRows;
  const int tlast = min(t0 + kAttnRows, g.tokens) - 1;
  const int kend = min(len + g.tokens, g.cap);      // keys present after this call's append
  const int kmax = g.causal ? min(len + tlast + 1, kend) : kend;  // keys any row of this tile can see
  const int frow = lane & 15, grp = lane >> 4;
  const int trow = t0 + 16 * wave + frow;     // this lane's row (column of S^T and O^T)
  const bool row_ok = trow < g.tokens;
  const int vis = g.causal ? len + trow + 1 : kend;  // keys visible to this lane's row

  // q of this lane's row as B operand: Q^T[k = d][n = row], d = 32 s + 8 grp + 0..7
  V8 qf[D / 32];
  {
    const T* qr = reinterpret_cast<const T*>(g.q) + ((size_t)b * g.tokens + (row_ok ? trow : 0)) * H + (size_t)j * D;
#pragma unroll
    for (int s = 0; s < D / 32; ++s) {
      qf[s] = *reinterpret_cast<const V8*>(qr + 32 * s + 8 * grp);
      if (!row_ok) qf[s] = V8{};
    }
  }
  const float qscale = g.scale * 1.4426950408889634f;  // softmax in base 2
  float4_t o[D / 16];
#pragma unroll
  for (int f = 0; f < D / 16; ++f) o[f] = float4_t{0.f, 0.f, 0.f, 0.f};
  float mrun = -1e30f, lrun = 0.f;

  const size_t hrow = ((size_t)b * g.heads + j) * g.cap;  // first cache row of this (sequence, head)
  const T* kbase = reinterpret_cast<const T*>(g.k_cache) + hrow * D;
  const T* vbase = reinterpret_cast<const T*>(g.v_cache) + hrow * D;
  // an int8 cache: 8 codes of a row times its scale become one 16-byte piece of 16-bit values
  auto deq8 = [&](const void* cache, const void* scales, int key, int ch) -> u32x4 {
    const uint2 c = *reinterpret_cast<const uint2*>(static_cast<const int8_t*>(cache) + (hrow + key) * D + ch * 8);
    const float s = (float)static_cast<const half_t*>(scales)[hrow + key];
    V8 v;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t w = e < 4 ? c.x : c.y;
      v[e] = (T)((float)(int8_t)(w >> (8 * (e & 3))) * s);
    }
    return __builtin_bit_cast(u32x4, v);
  };
  // each thread carries NT 16-byte pieces of K and of V of a key tile; the next tile's pieces
  // are requested before the current tile's products, so their latency hides behind them
  constexpr int NT = kAttnKeys * NCH / 256;
  static_assert(NT * 256 == kAttnKeys * NCH, "whole pieces per thread");
  u32x4 kpre[NT], vpre[NT];
  auto fetch = [&](int k0) {
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      const int c = tid + 256 * i, kr = c / NCH, ch = c - kr * NCH, key = k0 + kr;
      kpre[i] = u32x4{0u, 0u, 0u, 0u};
      vpre[i] = u32x4{0u, 0u, 0u, 0u};
      if (key < kend) {
        if constexpr (KV8) {
          kpre[i] = deq8(g.k_cache, g.k_scale, key, ch);
          vpre[i] = deq8(g.v_cache, g.v_scale, key, ch);
        } else {
          kpre[i] = *reinterpret_cast<const u32x4*>(kbase + (size_t)key * D + ch * 8);
          vpre[i] = *reinterpret_cast<const u32x4*>(vbase + (size_t)key * D + ch * 8);
        }
      }
    }
  };
  if (kmax > 0) fetch(0);
  for (int k0 = 0; k0 < kmax; k0 += kAttnKeys) {
    __syncthreads();  // the previous tile is no longer read
    // stage K [key][d] (chunk-swizzled) and V [key][d] (padded rows); keys at or past kend are zeros
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      const int c = tid + 256 * i, kr = c / NCH, ch = c - kr * NCH;
      *reinterpret_cast<u32x4*>(Ks + kr * S::KROW + ((ch ^ (kr & 7)) << 4)) = kpre[i];
      *reinterpret_cast<u32x4*>(Vs + kr * S::VROW + ch * 16) = vpre[i];
    }
    __syncthreads();
    if (k0 + kAttnKeys < kmax) fetch(k0 + kAttnKeys);

    // S^T for 64 keys: four 16-key blocks; lane holds keys 16 f + 4 grp + r of its row
    float4_t st[4];
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      st[f] = float4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < D / 32; ++s) {
        const int kr = 16 * f + frow, ch = 4 * s + grp;
        const V8 kf = *reinterpret_cast<const V8*>(Ks + kr * S::KROW + ((ch ^ (kr & 7)) << 4));
        st[f] = mfma_16x16x32<T>(kf, qf[s], st[f]);
      }
    }
    float tmax = -1e30f;
#pragma unroll
    for (int f = 0; f < 4; ++f)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = k0 + 16 * f + 4 * grp + r;
        const float sv = key < vis ? st[f][r] * qscale : -1e30f;
        st[f][r] = sv;
        tmax = fmaxf(tmax, sv);
      }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16, kWave));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32, kWave));
    const float mnew = fmaxf(mrun, tmax);
    const float corr = exp2f(mrun - mnew);
    float psum = 0.f;
    V8 pf[2];
#pragma unroll
    for (int f = 0; f < 4; ++f)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float p = st[f][r] <= -1e29f ? 0.f : exp2f(st[f][r] - mnew);
        psum += p;
        pf[f >> 1][(f & 1) * 4 + r] = (T)p;
      }
    psum += __shfl_xor(psum, 16, kWave);
    psum += __shfl_xor(psum, 32, kWave);
    lrun = lrun * corr + psum;
    mrun = mnew;
#pragma unroll
    for (int f = 0; f < D / 16; ++f) o[f] *= corr;
    // O^T += V^T P^T: B element e of lane group grp is key 32 s + 4 grp + e (e < 4) or
    // 32 s + 16 + 4 grp + (e - 4), matching the st layout; A (V^T, d = 16 f + lane % 16) takes
    // the same keys: in each transposed read, lane frow of the group addresses key
    // 32 s + 16 h + 4 grp + frow / 4 at d = 16 f + 4 (frow % 4), h = 0 for e < 4, 1 for e >= 4.
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int f = 0; f < D / 16; ++f) {
        const unsigned char* va = Vs + (32 * s + 4 * grp + (frow >> 2)) * S::VROW + (16 * f + 4 * (frow & 3)) * 2;
        const short4_t lo = lds_read_tr16(va);
        const short4_t hi = lds_read_tr16(va + 16 * S::VROW);
        const short8_t vv = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        o[f] = mfma_16x16x32<T>(__builtin_bit_cast(V8, vv), pf[s], o[f]);
      }
  }
  if (!row_ok) return;
  const float inv = 1.f / lrun;
  T* cr = reinterpret_cast<T*>(g.ctx) + ((size_t)b * g.tokens + trow) * H + (size_t)j * D;
#pragma unroll
  for (int f = 0; f < D / 16; ++f)
#pragma unroll
    for (int r = 0; r < 4; ++r) cr[16 * f + 4 * grp + r] = (T)(o[f][r] * inv);
}


// ------------------------------------------------------------------ skinny GEMM (M <= 16 rows)
// A decode step of a few rows is bound by streaming the weights, so each weight row is read once
// and the rows of the step ride along on MFMA: a workgroup owns 16 output columns (16 rows of W)
// and its waves split K. Per 32-wide k step the 16 W rows are the B operand (lane l: row l%16,
// k chunk l/16) and the activation rows the A operand (rows past M are zeros);
// v_mfma_f32_16x16x32_f16 leaves C[4(l/16)+i][l%16] in lane l. int8 weights: a lane takes 16 codes
// (k 16j..16j+15, j = l/16) of a 64-k block (one quantization group); the block's two MFMAs take
// k 16j..16j+7 and then 16j+8..16j+15 in lane group j (the sum over k does not depend on that
// order), the activations are loaded in the same order, the codes become fp16 exactly, and the
// block's product is scaled by the row's group scale before accumulating.
__device__ __forceinline__ half8_t i8x8_to_half8(uint32_t lo, uint32_t hi) {
  const uint32_t flip = 0x80808080u;  // q + 128 for every byte
  lo ^= flip;
  hi ^= flip;
  const half2_t p0 = i8pair_to_half2(lo, false), p1 = i8pair_to_half2(lo, true);
  const half2_t p2 = i8pair_to_half2(hi, false), p3 = i8pair_to_half2(hi, true);
  half8_t h;
  h[0] = p0.x; h[1] = p0.y; h[2] = p1.x; h[3] = p1.y;
  h[4] = p2.x; h[5] = p2.y; h[6] = p3.x; h[7] = p3.y;
  return h;
}

constexpr int kSkinnyMaxWaves = 8;  // waves (K splits) per workgroup at most

// The weight rows reach LDS as whole 128-byte lines through direct-to-LDS loads (8 rows x 128 B per
// wave load, the XOR-swizzled layout of the tiled GEMM) and the B operands are read back from LDS:
// loading them in the operand layout directly would fetch 64-byte halves of 16 rows per load.
// Each wave owns a private ring of R stages (16 rows x 128 B of W each: 64 k for fp16, 128 k for
// int8) and the matching activation loads in registers; every load is a buffer load, so rows past
// N and stages past the wave's range read zeros (activation rows past M are not loaded at all),
// and each stage issues the same number of loads, which keeps the in-order load counter arithmetic
// fixed. Products with few column blocks also split K over workgroups. The launcher picks the
// split and the waves per workgroup so that every workgroup of the launch is resident at once and
// the CUs carry equal shares.
constexpr int kSkR = 2;          // stages in flight per wave: deeper rings (3, 4, 6) measured slower
constexpr int kSkMinStages = 8;  // stages per wave worth a wave of its own

// A1: at most 8 activation rows, so one activation load per 64 k (fp16) or two per 128 k (int8)
// fill the operands of both MFMA halves of a stage: lanes of rows 8-15 (whose products are
// discarded) load the second half of rows 0-7, which a row rotate by 8 lanes hands to rows 0-7.
template <typename T, bool I8, int EPI, bool A1, int R = kSkR>
__global__ __launch_bounds__(64 * kSkinnyMaxWaves) void skinny_dma_kernel(const GemmArgs g) {
  static_assert(!I8 || sizeof(T) == 2, "int8 weights with fp16 activations");
  typedef typename Act16<T>::v8 V8;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int lane = threadIdx.x & 63, KS = blockDim.x >> 6;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane & 15, j = lane >> 4;
  // workgroup = (column block cb, K part sp); its waves split the part
  const int split = g.n_sk_cnt > 0 ? max(1, g.tiles_n) : 1;
  const int cb = blockIdx.x / split, sp = blockIdx.x - cb * split;
  const int n0 = cb * 16;
  if (EPI == EPI_QKV && blockIdx.x == 0) {
    if (g.attn_counters)
      for (int i = threadIdx.x; i < g.n_counters; i += blockDim.x) g.attn_counters[i] = 0u;
    if (g.sk_cnt)
      for (int i = threadIdx.x; i < g.n_sk_cnt; i += blockDim.x) g.sk_cnt[i] = 0u;
  }
  const int K = g.K;
  constexpr int SK = I8 ? 128 : 64;               // k per stage
  // loads per stage: 2 W line-sets, the activation loads, one scale load (int8)
  constexpr int LPS = I8 ? (A1 ? 5 : 7) : (A1 ? 3 : 4);
  const int kq = K / split / KS, kb = sp * (K / split) + w * kq, ns = kq / SK;
  const uint32_t wrow = (uint32_t)(I8 ? K : 2 * K);  // bytes per weight row
  const rsrc_t rw = make_rsrc(I8 ? (const void*)g.wq : (const void*)g.w, (uint32_t)((size_t)g.N * wrow));
  const rsrc_t ra = make_rsrc(g.a, (uint32_t)((size_t)g.M * K * 2));
  const rsrc_t rs = make_rsrc(g.wscale, I8 ? (uint32_t)((size_t)g.N * (K / 64) * 2) : 0u);
  unsigned char* ring = smem + w * (R * 2048);
  // W: wave load u of a stage covers rows n0 + 8u + L/8, logical chunk (L%8) ^ (L/8)
  const int lr = lane >> 3, lc = (lane & 7) ^ lr;
  const uint32_t w_off = (uint32_t)(n0 + lr) * wrow + (uint32_t)(I8 ? kb : 2 * kb) + lc * 16;
  // A: row r; fp16 step s of a stage takes k 32s + 8j .. +8; int8 group g takes 64g + 16j .. +16.
  // With A1, lanes of rows 8-15 take the second step (group) of row r - 8.
  const int ar = A1 ? (r & 7) : r;
  const uint32_t a_off = (uint32_t)((ar * K + kb) * 2) + (uint32_t)(I8 ? 32 * j : 16 * j) +
                         (A1 && r >= 8 ? (I8 ? 128u : 64u) : 0u);
  // int8: the scales of the stage's two 64-k groups, adjacent fp16 values (4-byte aligned: K/64
  // and kb/64 are even)
  const uint32_t s_off = (uint32_t)((n0 + r) * (K / 64) + kb / 64) * 2;
  constexpr int NA = I8 ? (A1 ? 2 : 4) : (A1 ? 1 : 2);  // activation loads per stage
  u32x4 av[R][NA];
  uint32_t sc[R];
  // lanes of rows past M issue no activation loads (their operand rows are zeros)
  const bool arow = ar < g.M;
  auto issue = [&](int i, int slot) {
    const bool ok = i < ns;
    const uint32_t wk = (uint32_t)i * 128u;  // W bytes per row per stage: 128 for fp16 and int8
#pragma unroll
    for (int u = 0; u < 2; ++u)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, lds_ptr(ring + slot * 2048 + u * 1024), 16,
                                               ok ? w_off + (uint32_t)(8 * u) * wrow + wk : kOutOfRange, 0, 0, 0);
    const uint32_t ak = (uint32_t)(i * SK * 2);
#pragma unroll
    for (int t = 0; t < NA; ++t) {
      // fp16: step t at +64 t; int8: group t / 2 at +128 (t / 2), its second 16 bytes at +16
      const uint32_t at = I8 ? (uint32_t)(128 * (t >> 1) + 16 * (t & 1)) : (uint32_t)(64 * t);
      av[slot][t] = u32x4{0u, 0u, 0u, 0u};
      if (arow) av[slot][t] = __builtin_amdgcn_raw_buffer_load_b128(ra, ok ? a_off + ak + at : kOutOfRange, 0, 0);
    }
    if constexpr (I8) sc[slot] = __builtin_amdgcn_raw_buffer_load_b32(rs, ok ? s_off + (uint32_t)i * 4u : kOutOfRange, 0, 0);
  };
  float4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < R; ++i) issue(i, i);
  for (int i = 0; i < ns; i += R) {
#pragma unroll
    for (int q = 0; q < R; ++q) {
      // stage i + q complete; the R - 1 stages requested after it may stay in flight
      wait_vm<(R - 1) * LPS>();
      const unsigned char* st = ring + q * 2048;
      if (i + q < ns) {
        // the activation operands of the stage's two halves (fp16 steps, int8 groups)
        u32x4 op[I8 ? 4 : 2];
        if constexpr (A1) {
#pragma unroll
          for (int t = 0; t < NA; ++t) {
            op[t] = av[q][t];
#pragma unroll
            for (int e = 0; e < 4; ++e)  // row_ror:8
              op[NA + t][e] = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)av[q][t][e], 0x128, 0xf, 0xf, false);
          }
        } else {
#pragma unroll
          for (int t = 0; t < NA; ++t) op[t] = av[q][t];
        }
        if constexpr (!I8) {
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            const V8 b = *reinterpret_cast<const V8*>(st + swz(r, 4 * t + j));
            acc = mfma_16x16x32<T>(__builtin_bit_cast(V8, op[t]), b, acc);
          }
        } else {
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            const u32x4 c = *reinterpret_cast<const u32x4*>(st + swz(r, 4 * t + j));
            float4_t p = {0.f, 0.f, 0.f, 0.f};
            p = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, op[2 * t]), i8x8_to_half8(c.x, c.y), p, 0, 0, 0);
            p = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, op[2 * t + 1]), i8x8_to_half8(c.z, c.w), p, 0, 0, 0);
            const half2_t sp2 = as_half2(sc[q]);
            const float scale = (float)(t == 0 ? sp2.x : sp2.y);
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[e] = fmaf(p[e], scale, acc[e]);
          }
        }
      }
      // the slot's operands are in registers before its refill is requested
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
      issue(i + q + R, q);
    }
  }
  wait_vm<0>();  // the out-of-range requests past the end
  // sum the waves' K ranges (each wave's partial tile in the first 1 KB of its own ring, which
  // nothing else touches once its loads have landed), then the epilogue of C[4 j + e][n0 + r]
  reinterpret_cast<float4_t*>(ring)[lane] = acc;
  __syncthreads();
  if (w != 0) return;
  for (int v = 1; v < KS; ++v) {
    const float4_t o = reinterpret_cast<const float4_t*>(smem + v * (R * 2048))[lane];
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[e] += o[e];
  }
  if (split > 1) {
    // K split over workgroups: publish this part's tile (device-scope stores, complete before the
    // arrival is counted); the last of the block's parts to arrive adds all parts in part order,
    // so the sum does not depend on arrival order, resets the counter and runs the epilogue
    // the block's parts: split x 1 KB, 16 bytes per lane, written and read at the device coherence
    // point (sc1), past the per-XCD L2s
    const rsrc_t rp = make_rsrc(g.sk_part + (size_t)cb * split * 256, (uint32_t)(split * 1024));
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, acc), rp, (uint32_t)(sp * 1024 + lane * 16), 0, 16);
    __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): the stores have completed
    __shared__ uint32_t arrived;
    if (lane == 0) arrived = __hip_atomic_fetch_add(g.sk_cnt + cb, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    if (*(volatile uint32_t*)&arrived != (uint32_t)(split - 1)) return;
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[e] = 0.f;
    for (int q = 0; q < split; ++q) {
      const float4_t o = __builtin_bit_cast(float4_t, __builtin_amdgcn_raw_buffer_load_b128(rp, (uint32_t)(q * 1024 + lane * 16), 0, 16));
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[e] += o[e];
    }
    if (lane == 0) __hip_atomic_store(g.sk_cnt + cb, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) epilogue_store<T, EPI>(g, 4 * j + e, n0 + r, acc[e]);
}

// Resident workgroups per CU of a skinny variant with `waves` waves (the runtime's occupancy
// figure: registers, LDS and wave slots), cached per variant and wave count.
template <typename T, bool I8, int EPI, bool A1>
int skinny_slots(int waves) {
  static int cache[kSkinnyMaxWaves + 1] = {};
  int& c = cache[waves];
  if (c == 0) {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, reinterpret_cast<const void*>(&skinny_dma_kernel<T, I8, EPI, A1>),
                                                     64 * waves, (size_t)waves * kSkR * 2048) != hipSuccess)
      n = 0;
    c = n > 0 ? n : -1;
  }
  return c;
}

// Split and waves per workgroup of a skinny launch, best first by: the largest per-CU count of
// workgroups relative to their number (every workgroup resident at once, so no CU runs a second
// round while the others idle), fewer K splits, more waves. Measured on the 13B FF2 product (320
// column blocks, K 20480): 1280 workgroups of four waves, all resident, 45 us; of eight waves (four
// resident per CU, a second round for one per CU) 50 us.
struct SkPlan {
  int split = 0, ks = 0, per_cu = 0;
};
template <typename T, bool I8, int EPI, bool A1>
SkPlan skinny_plan(const GemmArgs& a, int cus) {
  const int kq = I8 ? 128 : 64;  // k per stage
  const int nblk = (a.N + 15) / 16;
  // never split the QKV product, whose first workgroup clears the split counters
  const bool can_split = EPI != EPI_QKV && a.sk_part && a.sk_cnt && nblk <= a.n_sk_cnt;
  SkPlan best;
  for (int split = 1; split <= (can_split ? kSkinnyMaxSplit : 1); split *= 2) {
    if (a.K % (split * kq) != 0) continue;
    const int kp = a.K / split, nwg = nblk * split, per_cu = (nwg + cus - 1) / cus;
    for (int ks = kSkinnyMaxWaves; ks >= 1; ks >>= 1) {
      if (kp % (ks * kq) != 0 || kp / (ks * kq) < kSkMinStages || skinny_slots<T, I8, EPI, A1>(ks) < per_cu) continue;
      const bool better = best.split == 0 || (long)per_cu * best.split < (long)best.per_cu * split;
      if (better) best = SkPlan{split, ks, per_cu};
      break;  // the most waves that fit this split
    }
  }
  if (best.split == 0) {  // nothing fits one round: the most waves that divide K
    int ks = kSkinnyMaxWaves;
    while (ks > 1 && (a.K % (ks * kq) != 0 || a.K / (ks * kq) < kSkMinStages)) ks >>= 1;
    if (a.K % (ks * kq) == 0) best = SkPlan{1, ks, 0};
  }
  return best;
}

template <typename T, bool I8, int EPI, bool A1>
hipError_t launch_skinny_t(const GemmArgs& a, int cus, hipStream_t st) {
  const SkPlan p = skinny_plan<T, I8, EPI, A1>(a, cus);
  if (p.split == 0) return hipErrorInvalidValue;
  const int nblk = (a.N + 15) / 16;
  GemmArgs g = a;
  g.tiles_n = p.split;
  if (p.split == 1 && EPI != EPI_QKV) g.n_sk_cnt = 0;
  const size_t lds = (size_t)p.ks * kSkR * 2048;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&skinny_dma_kernel<T, I8, EPI, A1>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((skinny_dma_kernel<T, I8, EPI, A1>), dim3(nblk * p.split), dim3(64 * p.ks), lds, st, g);
  return hipGetLastError();
}

template <typename T, int BM, int BN, int ST, int KG, int NWN, int EPI>
hipError_t launch_gemm_t(const GemmArgs& a0, hipStream_t st) {
  typedef GemmShape<BM, BN, ST, KG, NWN> S;
  GemmArgs a = a0;
  a.tiles_m = (a.M + BM - 1) / BM;
  a.tiles_n = (a.N + BN - 1) / BN;
  // above the default 64 KB of dynamic LDS; set on every launch (cheap, and per device)
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&gemm_kernel<T, BM, BN, ST, KG, NWN, EPI>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, S::LDS);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((gemm_kernel<T, BM, BN, ST, KG, NWN, EPI>), dim3(a.tiles_m * a.tiles_n), dim3(S::THREADS), S::LDS, st, a);
  return hipGetLastError();
}

// The tile configurations:
//   0: 128 x 160, two-stage ring, four waves, two workgroups per CU, for products with at least
//      two such tiles per CU (the next tiles' loads overlap the current ones' products);
//   1: 128 x 160, three-stage ring, two groups of four waves splitting each k-step, one workgroup
//      per CU, for products with at most one such tile per CU (deeper prefetch, two waves per SIMD);
//   2: 256 x 256, two-stage ring, eight waves of 128 x 64, one workgroup per CU: half the bytes
//      loaded per FLOP of 128 x 160 (the ring's loads set the pace), for products that come out
//      at 85-100 % of one such tile per CU.
template <typename T, int EPI>
hipError_t launch_gemm_epi(const GemmArgs& a, int cfg, hipStream_t st) {
  switch (cfg) {
    case 0: return launch_gemm_t<T, 128, 160, 2, 1, 2, EPI>(a, st);
    case 1: return launch_gemm_t<T, 128, 160, 3, 2, 2, EPI>(a, st);
    case 2: return launch_gemm_t<T, 256, 256, 2, 1, 4, EPI>(a, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace prefill

using namespace prefill;

// Measured on the GPT-Neo-2.7B prefill products (2048 rows): configuration 0 runs the 768- and
// 1024-tile products 1.1x-1.4x faster than 1, and 1 the 256-tile ones 1.2x-1.3x faster than 0;
// configuration 2 runs QKV (240 tiles of 256 x 256) 1.33x faster than 0, and FF1 (320 such
// tiles, a second round for 64) 1.3x slower.
int gemm_pick(int M, int N, int K, int cus) {
  (void)K;
  const long t256 = (long)((M + 255) / 256) * ((N + 255) / 256);
  if (M % 256 == 0 && N % 256 == 0 && t256 <= cus && 20 * t256 >= 17 * (long)cus) return 2;
  const long tiles = (long)((M + 127) / 128) * ((N + 159) / 160);
  return tiles <= cus ? 1 : 0;
}

template <int E>
hipError_t launch_skinny_e(bool i8, bool bf16, const GemmArgs& a, int cus, hipStream_t st) {
  const bool a1 = a.M <= 8;  // one activation load serves both halves of a stage
  if (i8) return a1 ? launch_skinny_t<half_t, true, E, true>(a, cus, st) : launch_skinny_t<half_t, true, E, false>(a, cus, st);
  if (bf16) return a1 ? launch_skinny_t<bf16_t, false, E, true>(a, cus, st) : launch_skinny_t<bf16_t, false, E, false>(a, cus, st);
  return a1 ? launch_skinny_t<half_t, false, E, true>(a, cus, st) : launch_skinny_t<half_t, false, E, false>(a, cus, st);
}

hipError_t launch_skinny(GemmEpi epi, bool int8_weights, bool bf16, const GemmArgs& a, int cus, hipStream_t st) {
  if (a.M <= 0 || a.N <= 0) return hipSuccess;
  if (a.M > kSkinnyMaxRows || (int8_weights && bf16)) return hipErrorInvalidValue;
  switch (epi) {
    case EPI_QKV: return launch_skinny_e<EPI_QKV>(int8_weights, bf16, a, cus, st);
    case EPI_OPROJ: return launch_skinny_e<EPI_OPROJ>(int8_weights, bf16, a, cus, st);
    case EPI_FF1: return launch_skinny_e<EPI_FF1>(int8_weights, bf16, a, cus, st);
    case EPI_FF2: return launch_skinny_e<EPI_FF2>(int8_weights, bf16, a, cus, st);
  }
  return hipErrorInvalidValue;
}

template <typename T>
hipError_t launch_gemm_type(GemmEpi epi, const GemmArgs& a, int cfg, hipStream_t st) {
  switch (epi) {
    case EPI_QKV: return launch_gemm_epi<T, EPI_QKV>(a, cfg, st);
    case EPI_OPROJ: return launch_gemm_epi<T, EPI_OPROJ>(a, cfg, st);
    case EPI_FF1: return launch_gemm_epi<T, EPI_FF1>(a, cfg, st);
    case EPI_FF2: return launch_gemm_epi<T, EPI_FF2>(a, cfg, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_gemm(GemmEpi epi, bool bf16, const GemmArgs& a, int cfg, hipStream_t st) {
  if (a.M <= 0 || a.N <= 0) return hipSuccess;
  if (a.K < kBK || a.K % kBK) return hipErrorInvalidValue;
  return bf16 ? launch_gemm_type<bf16_t>(epi, a, cfg, st) : launch_gemm_type<half_t>(epi, a, cfg, st);
}

template <typename T>
hipError_t launch_ln_rows_t(bool in_f32, const void* x, const T* g, const T* b, T* out, int rows, int H, float eps,
                            hipStream_t st, int32_t* d_len, int batch, int ntok, int cap) {
  if (rows <= 0) return hipSuccess;
  const LenAdvance la{d_len, batch, ntok, cap};
  constexpr int kNR = 8;  // 16-byte vectors per thread of the workgroup-per-row kernel
  if (rows < 64 && H <= 256 * kNR * (in_f32 ? 4 : 8)) {
    if (in_f32)
      hipLaunchKernelGGL((ln_row_wg_kernel<T, float, kNR>), dim3(rows), dim3(256), 0, st, static_cast<const float*>(x), g, b, out, H, eps, la);
    else
      hipLaunchKernelGGL((ln_row_wg_kernel<T, T, kNR>), dim3(rows), dim3(256), 0, st, static_cast<const T*>(x), g, b, out, H, eps, la);
    return hipGetLastError();
  }
  const dim3 grid((rows + 3) / 4);
  // register-resident wave-per-row kernel: 16-byte pieces per lane, the fewest of 4, 8, 12, 16
  // that hold the row
  const int pieces = (H / (in_f32 ? 4 : 8) + kWave - 1) / kWave;
  if (pieces <= 16) {
#define DS_LNR(NR)                                                                                                   \
  if (pieces <= NR) {                                                                                                \
    if (in_f32)                                                                                                      \
      hipLaunchKernelGGL((ln_rows_reg_kernel<T, float, NR>), grid, dim3(256), 0, st, static_cast<const float*>(x), g, b, \
                         out, rows, H, eps, la);                                                                     \
    else                                                                                                             \
      hipLaunchKernelGGL((ln_rows_reg_kernel<T, T, NR>), grid, dim3(256), 0, st, static_cast<const T*>(x), g, \
                         b, out, rows, H, eps, la);                                                                  \
    return hipGetLastError();                                                                                        \
  }
    DS_LNR(4)
    DS_LNR(8)
    DS_LNR(12)
    DS_LNR(16)
#undef DS_LNR
  }
  if (in_f32)
    hipLaunchKernelGGL((ln_rows_kernel<T, float>), grid, dim3(256), 0, st, static_cast<const float*>(x), g, b, out, rows, H, eps);
  else
    hipLaunchKernelGGL((ln_rows_kernel<T, T>), grid, dim3(256), 0, st, static_cast<const T*>(x), g, b, out, rows, H, eps);
  if (hipError_t e = hipGetLastError()) return e;
  if (d_len) return launch_len_advance(d_len, batch, ntok, cap, st);
  return hipSuccess;
}

hipError_t launch_ln_rows(bool bf16, bool in_f32, const void* x, const void* g, const void* b, void* out, int rows,
                          int H, float eps, hipStream_t st, int32_t* d_len, int batch, int ntok, int cap) {
  if (bf16)
    return launch_ln_rows_t<bf16_t>(in_f32, x, static_cast<const bf16_t*>(g), static_cast<const bf16_t*>(b),
                                    static_cast<bf16_t*>(out), rows, H, eps, st, d_len, batch, ntok, cap);
  return launch_ln_rows_t<half_t>(in_f32, x, static_cast<const half_t*>(g), static_cast<const half_t*>(b),
                                  static_cast<half_t*>(out), rows, H, eps, st, d_len, batch, ntok, cap);
}

template <typename T, int D>
static void launch_attn_prefill_t(const AttnPrefillArgs& a, dim3 grid, hipStream_t st) {
  if (a.k_scale) hipLaunchKernelGGL((attn_prefill_kernel<T, D, true>), grid, dim3(256), attn_lds_bytes<D>(), st, a);
  else hipLaunchKernelGGL((attn_prefill_kernel<T, D, false>), grid, dim3(256), attn_lds_bytes<D>(), st, a);
}

hipError_t launch_attn_prefill(bool bf16, const AttnPrefillArgs& a, hipStream_t st) {
  const int qtiles = (a.tokens + kAttnRows - 1) / kAttnRows;
  const dim3 grid(a.batch * a.heads * qtiles);
  if (a.batch <= 0 || a.tokens <= 0) return hipSuccess;
  if ((a.k_scale == nullptr) != (a.v_scale == nullptr)) return hipErrorInvalidValue;
  if (a.head_dim == 128) {
    if (bf16) launch_attn_prefill_t<bf16_t, 128>(a, grid, st);
    else launch_attn_prefill_t<half_t, 128>(a, grid, st);
  } else if (a.head_dim == 64) {
    if (bf16) launch_attn_prefill_t<bf16_t, 64>(a, grid, st);
    else launch_attn_prefill_t<half_t, 64>(a, grid, st);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace ds
