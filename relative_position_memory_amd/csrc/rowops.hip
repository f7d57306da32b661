// Row kernels: post-norm LayerNorm, the memory ring copy, and a float fill.
#include "txl_internal.h"

namespace txl {
namespace {

__device__ inline float block_sum(float x, float* red) {
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o, 64);
  const int w = threadIdx.x / 64, lane = threadIdx.x % 64;
  __syncthreads();
  if (lane == 0) red[w] = x;
  __syncthreads();
  float t = 0.f;
  for (int i = 0; i < (int)(blockDim.x / 64); ++i) t += red[i];
  return t;
}

// LayerNorm(Linear(a) + h) of the N-layer procedure (section 3.3): the input
// y already holds a W_o^T + h in fp32.  Mean and biased variance over D.
__device__ inline float wave_sum(float x) {
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}

// One wavefront per row, four rows per block: no block-level synchronisation.
template <typename T>
__global__ __launch_bounds__(256) void layer_norm_kernel(const float* __restrict__ y,
                                                         const T* __restrict__ gamma,
                                                         const T* __restrict__ beta, float eps,
                                                         int64_t rows, int64_t D,
                                                         T* __restrict__ out) {
  const int64_t row = (int64_t)blockIdx.x * 4 + threadIdx.x / 64;
  const int lane = threadIdx.x & 63;
  if (row >= rows) return;
  const float* x = y + row * D;
  float s = 0.f;
  for (int64_t c = lane; c < D; c += 64) s += x[c];
  const float mean = wave_sum(s) / (float)D;
  float v = 0.f;
  for (int64_t c = lane; c < D; c += 64) {
    const float t = x[c] - mean;
    v += t * t;
  }
  const float var = wave_sum(v) / (float)D;
  const float inv = rsqrtf(var + eps);
  T* o = out + row * D;
  for (int64_t c = lane; c < D; c += 64)
    Elt<T>::store(o + c, (x[c] - mean) * inv * Elt<T>::load(gamma + c) + Elt<T>::load(beta + c));
}

// The same LayerNorm for any D <= 64 NE: lane l keeps elements l + 64 k of its
// row (and of gamma and beta) in registers, all loaded before the reductions.
template <typename T, int NE>
__global__ __launch_bounds__(256) void layer_norm_reg_kernel(const float* __restrict__ y,
                                                             const T* __restrict__ gamma,
                                                             const T* __restrict__ beta,
                                                             float eps, int64_t rows, int D,
                                                             T* __restrict__ out) {
  const int64_t row = (int64_t)blockIdx.x * 4 + threadIdx.x / 64;
  const int lane = threadIdx.x & 63;
  if (row >= rows) return;
  const float* x = y + row * D;
  float v[NE], ga[NE], be[NE];
#pragma unroll
  for (int k = 0; k < NE; ++k) {
    const int c = lane + 64 * k, cc = c < D ? c : D - 1;
    v[k] = c < D ? x[cc] : 0.f;
    ga[k] = Elt<T>::load(gamma + cc);
    be[k] = Elt<T>::load(beta + cc);
  }
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < NE; ++k) s += v[k];
  const float mean = wave_sum(s) / (float)D;
  float q = 0.f;
#pragma unroll
  for (int k = 0; k < NE; ++k) {
    v[k] = lane + 64 * k < D ? v[k] - mean : 0.f;
    q += v[k] * v[k];
  }
  const float inv = rsqrtf(wave_sum(q) / (float)D + eps);
  T* o = out + row * D;
#pragma unroll
  for (int k = 0; k < NE; ++k)
    if (lane + 64 * k < D) Elt<T>::store(o + lane + 64 * k, v[k] * inv * ga[k] + be[k]);
}

// Four consecutive elements as floats / from floats (16-byte aligned fp32,
// 8-byte aligned bf16).
__device__ inline float4 load4(const float* p) { return *(const float4*)p; }
__device__ inline float4 load4(const uint16_t* p) {
  const uint2 w = *(const uint2*)p;
  return make_float4(__builtin_bit_cast(float, w.x << 16),
                     __builtin_bit_cast(float, w.x & 0xffff0000u),
                     __builtin_bit_cast(float, w.y << 16),
                     __builtin_bit_cast(float, w.y & 0xffff0000u));
}
__device__ inline void store4(float* p, float4 v) { *(float4*)p = v; }
__device__ inline void store4(uint16_t* p, float4 v) {
  const uint32_t lo = (uint32_t)f32_to_bf16(v.x) | ((uint32_t)f32_to_bf16(v.y) << 16);
  const uint32_t hi = (uint32_t)f32_to_bf16(v.z) | ((uint32_t)f32_to_bf16(v.w) << 16);
  *(uint2*)p = make_uint2(lo, hi);
}

// The same LayerNorm for D = 256 NV (NV <= 8) with aligned rows: each lane keeps
// NV 4-element chunks (chunk lane + 64 k) of its row, and of gamma and beta, in
// registers; every load is issued before the two reductions, so one memory
// round trip serves the row.
template <typename T, int NV>
__global__ __launch_bounds__(256) void layer_norm_vec_kernel(const float* __restrict__ y,
                                                             const T* __restrict__ gamma,
                                                             const T* __restrict__ beta,
                                                             float eps, int64_t rows,
                                                             T* __restrict__ out) {
  constexpr int D = 256 * NV;
  const int64_t row = (int64_t)blockIdx.x * 4 + threadIdx.x / 64;
  const int lane = threadIdx.x & 63;
  if (row >= rows) return;
  const float* x = y + row * D;
  float4 v[NV], ga[NV], be[NV];
#pragma unroll
  for (int k = 0; k < NV; ++k) {
    const int c = 4 * (lane + 64 * k);
    v[k] = load4(x + c);
    ga[k] = load4(gamma + c);
    be[k] = load4(beta + c);
  }
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < NV; ++k) s += (v[k].x + v[k].y) + (v[k].z + v[k].w);
  const float mean = wave_sum(s) / (float)D;
  float q = 0.f;
#pragma unroll
  for (int k = 0; k < NV; ++k) {
    v[k].x -= mean; v[k].y -= mean; v[k].z -= mean; v[k].w -= mean;
    q += (v[k].x * v[k].x + v[k].y * v[k].y) + (v[k].z * v[k].z + v[k].w * v[k].w);
  }
  const float inv = rsqrtf(wave_sum(q) / (float)D + eps);
  T* o = out + row * D;
#pragma unroll
  for (int k = 0; k < NV; ++k) {
    const float4 r = make_float4(v[k].x * inv * ga[k].x + be[k].x, v[k].y * inv * ga[k].y + be[k].y,
                                 v[k].z * inv * ga[k].z + be[k].z, v[k].w * inv * ga[k].w + be[k].w);
    store4(o + 4 * (lane + 64 * k), r);
  }
}

// out = LayerNorm(sum_p parts[p] + resid) * gamma + beta for D = 256 NV with
// aligned rows: the K-split partial sums of the output projection, the residual
// and the LayerNorm in one pass, laid out as layer_norm_vec_kernel (one wave per
// row, NV 4-element chunks per lane).  y, when not NULL, receives the fp32 sum.
template <typename T, int NV>
__global__ __launch_bounds__(256) void layer_norm_parts_kernel(
    const float* __restrict__ parts, int nparts, int64_t pstride, const T* __restrict__ resid,
    const T* __restrict__ gamma, const T* __restrict__ beta, float eps, int64_t rows,
    T* __restrict__ out, float* __restrict__ y) {
  constexpr int D = 256 * NV;
  const int64_t row = (int64_t)blockIdx.x * 4 + threadIdx.x / 64;
  const int lane = threadIdx.x & 63;
  if (row >= rows) return;
  float4 v[NV], ga[NV], be[NV];
#pragma unroll
  for (int k = 0; k < NV; ++k) {
    const int c = 4 * (lane + 64 * k);
    v[k] = load4(resid + row * D + c);
    ga[k] = load4(gamma + c);
    be[k] = load4(beta + c);
  }
#pragma unroll 2
  for (int p = 0; p < nparts; ++p) {
    const float* src = parts + p * pstride + row * D;
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      const float4 a = load4(src + 4 * (lane + 64 * k));
      v[k].x += a.x; v[k].y += a.y; v[k].z += a.z; v[k].w += a.w;
    }
  }
  if (y) {
#pragma unroll
    for (int k = 0; k < NV; ++k) store4(y + row * D + 4 * (lane + 64 * k), v[k]);
  }
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < NV; ++k) s += (v[k].x + v[k].y) + (v[k].z + v[k].w);
  const float mean = wave_sum(s) / (float)D;
  float q = 0.f;
#pragma unroll
  for (int k = 0; k < NV; ++k) {
    v[k].x -= mean; v[k].y -= mean; v[k].z -= mean; v[k].w -= mean;
    q += (v[k].x * v[k].x + v[k].y * v[k].y) + (v[k].z * v[k].z + v[k].w * v[k].w);
  }
  const float inv = rsqrtf(wave_sum(q) / (float)D + eps);
  T* o = out + row * D;
#pragma unroll
  for (int k = 0; k < NV; ++k) {
    const float4 r = make_float4(v[k].x * inv * ga[k].x + be[k].x, v[k].y * inv * ga[k].y + be[k].y,
                                 v[k].z * inv * ga[k].z + be[k].z, v[k].w * inv * ga[k].w + be[k].w);
    store4(o + 4 * (lane + 64 * k), r);
  }
}

// One row of D elements per (t, b), copied with `V`-byte words.
template <typename V>
__global__ __launch_bounds__(256) void ring_copy_kernel(char* ring, int64_t cap, int64_t slot0,
                                                        const char* src, int64_t src_rows,
                                                        int64_t row0, int64_t row_bytes) {
  const int64_t t = blockIdx.x, b = blockIdx.y;
  int64_t slot = slot0 + t;
  slot %= cap;
  V* dst = (V*)(ring + (b * cap + slot) * row_bytes);
  const V* s = (const V*)(src + (b * src_rows + row0 + t) * row_bytes);
  const int64_t n = row_bytes / (int64_t)sizeof(V);
  for (int64_t c = threadIdx.x; c < n; c += blockDim.x) dst[c] = s[c];
}

// The same copy as one flat list of V-sized items (16 bytes when the rows allow,
// else 4; row r = b n + t, chunk c of cpr): each thread moves RC_U items, all
// loaded before any is stored (ring and src never overlap); an item index past
// the end repeats the last item, whose identical value is then written twice.
// 32-bit index arithmetic (the caller checks the item count).
constexpr int RC_U = 4;
template <typename V>
__global__ __launch_bounds__(256) void ring_copy_flat_kernel(char* __restrict__ ring, uint32_t cap,
                                                             uint32_t slot0,
                                                             const char* __restrict__ src,
                                                             uint32_t src_rows, uint32_t row0,
                                                             uint32_t n, uint32_t cpr,
                                                             uint32_t total, int64_t rb) {
  const uint32_t i0 = blockIdx.x * (256u * RC_U) + threadIdx.x;
  V v[RC_U];
  int64_t dst[RC_U];
#pragma unroll
  for (int u = 0; u < RC_U; ++u) {
    const uint32_t i = i0 + 256u * u;
    const uint32_t ic = i < total ? i : total - 1;
    const uint32_t row = ic / cpr, c = ic - row * cpr;
    const uint32_t b = row / n, t = row - b * n;
    const uint32_t slot = (slot0 + t) % cap;
    v[u] = *(const V*)(src + ((int64_t)b * src_rows + row0 + t) * rb + (int64_t)sizeof(V) * c);
    dst[u] = ((int64_t)b * cap + slot) * rb + (int64_t)sizeof(V) * c;
  }
#pragma unroll
  for (int u = 0; u < RC_U; ++u) *(V*)(ring + dst[u]) = v[u];
}

// Padded row copies (PadJob): a block is 4 waves of PAD_RPW rows of one job.
// Lane l moves the 4-byte words l, l + 64, l + 128, l + 192 of each of its
// wave's rows (one 1 KB block of each row at a time), so every load and store
// instruction covers 256 contiguous bytes, and all of a block's loads (16 per
// lane) are issued before its stores; a source index past the width is clamped
// and its value replaced by zero, so every load is unconditional.  Rows past
// the job repeat its last row (the same values written twice).  32-bit index
// arithmetic (the launch checks the sizes).
constexpr int PAD_RPW = 4;
struct PadJobsK {
  PadJob j[PAD_MAX];
  uint32_t block_end[PAD_MAX];  // inclusive prefix sums of the jobs' blocks
  int n;
};

__device__ inline const uint32_t* pad_src_row(const RowGather& a, uint32_t r) {
  const uint32_t per = (uint32_t)(a.mem_len + a.cur_rows), len = (uint32_t)a.mem_len;
  const uint32_t b = r / per, t = r - b * per;
  if (t < len) {
    uint32_t slot = (uint32_t)a.mem_start + t;
    if (slot >= (uint32_t)a.mem_cap) slot -= (uint32_t)a.mem_cap;
    return (const uint32_t*)((const uint16_t*)a.mem + ((int64_t)b * a.mem_cap + slot) * a.lda);
  }
  return (const uint32_t*)((const uint16_t*)a.cur + ((int64_t)b * a.cur_rows + (t - len)) * a.lda);
}

__global__ __launch_bounds__(256) void pad_rows_kernel(PadJobsK J) {
  int jn = 0;
  while (jn + 1 < J.n && blockIdx.x >= J.block_end[jn]) ++jn;
  const PadJob& p = J.j[jn];
  const uint32_t blk = blockIdx.x - (jn ? J.block_end[jn - 1] : 0u);
  const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const uint32_t R = (uint32_t)p.R, r0 = (blk * 4 + wave) * PAD_RPW;
  const uint32_t wdst = (uint32_t)(p.Cpad / 2), wsrc = (uint32_t)(p.C / 2);
  uint32_t* drow[PAD_RPW];
#pragma unroll
  for (int i = 0; i < PAD_RPW; ++i)
    drow[i] = (uint32_t*)(p.dst + (int64_t)(r0 + i < R ? r0 + i : R - 1) * p.Cpad);
  if (p.src.cur == nullptr && p.src.mem == nullptr) {  // rows of zeros
    for (uint32_t c = lane; c < wdst; c += 64)
#pragma unroll
      for (int i = 0; i < PAD_RPW; ++i) drow[i][c] = 0u;
    return;
  }
  const uint32_t* srow[PAD_RPW];
#pragma unroll
  for (int i = 0; i < PAD_RPW; ++i) srow[i] = pad_src_row(p.src, r0 + i < R ? r0 + i : R - 1);
  for (uint32_t c0 = 0; c0 < wdst; c0 += 256) {
    uint32_t v[PAD_RPW][4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t c = c0 + lane + 64 * k, cs = c < wsrc ? c : wsrc - 1;
#pragma unroll
      for (int i = 0; i < PAD_RPW; ++i) v[i][k] = srow[i][cs];
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t c = c0 + lane + 64 * k;
      if (c < wdst) {
#pragma unroll
        for (int i = 0; i < PAD_RPW; ++i) drow[i][c] = c < wsrc ? v[i][k] : 0u;
      }
    }
  }
}

__global__ void fill_kernel(float* p, int64_t n, float v) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    p[i] = v;
}

}  // namespace

hipError_t launch_layer_norm(int dtype, const float* y, const void* gamma, const void* beta,
                             float eps, int64_t rows, int64_t D, void* out, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  const unsigned blocks = (unsigned)((rows + 3) / 4);
  const uintptr_t al = (uintptr_t)gamma | (uintptr_t)beta | (uintptr_t)out;
  if (D % 256 == 0 && D <= 2048 && ((uintptr_t)y % 16) == 0 && al % (dtype == 0 ? 16 : 8) == 0) {
#define TXL_LN_VEC(NV)                                                                        \
  if (D == 256 * NV) {                                                                        \
    if (dtype == 0)                                                                           \
      hipLaunchKernelGGL((layer_norm_vec_kernel<float, NV>), dim3(blocks), dim3(256), 0, s, y, \
                         (const float*)gamma, (const float*)beta, eps, rows, (float*)out);    \
    else                                                                                      \
      hipLaunchKernelGGL((layer_norm_vec_kernel<uint16_t, NV>), dim3(blocks), dim3(256), 0, s, \
                         y, (const uint16_t*)gamma, (const uint16_t*)beta, eps, rows,          \
                         (uint16_t*)out);                                                     \
    return hipGetLastError();                                                                 \
  }
    TXL_LN_VEC(1) TXL_LN_VEC(2) TXL_LN_VEC(3) TXL_LN_VEC(4)
    TXL_LN_VEC(5) TXL_LN_VEC(6) TXL_LN_VEC(7) TXL_LN_VEC(8)
#undef TXL_LN_VEC
  }
  if (D <= 1024) {
#define TXL_LN_REG(NE)                                                                        \
  if (D <= 64 * NE) {                                                                         \
    if (dtype == 0)                                                                           \
      hipLaunchKernelGGL((layer_norm_reg_kernel<float, NE>), dim3(blocks), dim3(256), 0, s, y, \
                         (const float*)gamma, (const float*)beta, eps, rows, (int)D,          \
                         (float*)out);                                                        \
    else                                                                                      \
      hipLaunchKernelGGL((layer_norm_reg_kernel<uint16_t, NE>), dim3(blocks), dim3(256), 0,   \
                         s, y, (const uint16_t*)gamma, (const uint16_t*)beta, eps, rows,       \
                         (int)D, (uint16_t*)out);                                             \
    return hipGetLastError();                                                                 \
  }
    TXL_LN_REG(2) TXL_LN_REG(4) TXL_LN_REG(8) TXL_LN_REG(16)
#undef TXL_LN_REG
  }
  if (dtype == 0)
    hipLaunchKernelGGL(layer_norm_kernel<float>, dim3(blocks), dim3(256), 0, s, y,
                       (const float*)gamma, (const float*)beta, eps, rows, D, (float*)out);
  else
    hipLaunchKernelGGL(layer_norm_kernel<uint16_t>, dim3(blocks), dim3(256), 0, s, y,
                       (const uint16_t*)gamma, (const uint16_t*)beta, eps, rows, D,
                       (uint16_t*)out);
  return hipGetLastError();
}

bool layer_norm_parts_ok(int dtype, const float* parts, int64_t pstride, const void* resid,
                         const void* gamma, const void* beta, int64_t D, const void* out,
                         const float* y) {
  const uintptr_t f = (uintptr_t)parts | (uintptr_t)y;
  const uintptr_t t = (uintptr_t)resid | (uintptr_t)gamma | (uintptr_t)beta | (uintptr_t)out;
  return D % 256 == 0 && D <= 2048 && pstride % 4 == 0 && f % 16 == 0 &&
         t % (dtype == 0 ? 16 : 8) == 0;
}

hipError_t launch_layer_norm_parts(int dtype, const float* parts, int nparts, int64_t pstride,
                                   const void* resid, const void* gamma, const void* beta,
                                   float eps, int64_t rows, int64_t D, void* out, float* y,
                                   hipStream_t s) {
  if (nparts < 1 || !layer_norm_parts_ok(dtype, parts, pstride, resid, gamma, beta, D, out, y))
    return hipErrorInvalidValue;
  if (rows == 0) return hipSuccess;
  const unsigned blocks = (unsigned)((rows + 3) / 4);
#define TXL_LNP(NV)                                                                            \
  if (D == 256 * NV) {                                                                         \
    if (dtype == 0)                                                                            \
      hipLaunchKernelGGL((layer_norm_parts_kernel<float, NV>), dim3(blocks), dim3(256), 0, s,   \
                         parts, nparts, pstride, (const float*)resid, (const float*)gamma,     \
                         (const float*)beta, eps, rows, (float*)out, y);                       \
    else                                                                                       \
      hipLaunchKernelGGL((layer_norm_parts_kernel<uint16_t, NV>), dim3(blocks), dim3(256), 0,   \
                         s, parts, nparts, pstride, (const uint16_t*)resid,                     \
                         (const uint16_t*)gamma, (const uint16_t*)beta, eps, rows,              \
                         (uint16_t*)out, y);                                                   \
    return hipGetLastError();                                                                  \
  }
  TXL_LNP(1) TXL_LNP(2) TXL_LNP(3) TXL_LNP(4) TXL_LNP(5) TXL_LNP(6) TXL_LNP(7) TXL_LNP(8)
#undef TXL_LNP
  return hipErrorInvalidValue;
}

hipError_t launch_ring_copy(int dtype, void* ring, int64_t cap, int64_t slot0, const void* src,
                            int64_t src_rows, int64_t row0, int64_t n, int64_t B, int64_t D,
                            hipStream_t s) {
  if (n == 0 || B == 0) return hipSuccess;
  const int64_t es = dtype == 0 ? 4 : 2;
  const int64_t rb = D * es;
  const uintptr_t al = (uintptr_t)ring | (uintptr_t)src;
  dim3 grid((unsigned)n, (unsigned)B);
  const bool wide = rb % 16 == 0 && al % 16 == 0;
  const int64_t isz = wide ? 16 : 4;
  const int64_t total = n * B * (rb / isz);
  const bool fits = total < 0x7fffffffLL && cap < 0x7fffffffLL && slot0 < cap &&
                    src_rows + row0 < 0x7fffffffLL;
  if ((wide || (rb % 4 == 0 && al % 4 == 0)) && fits) {
    const unsigned blocks = (unsigned)((total + 256 * RC_U - 1) / (256 * RC_U));
    if (wide)
      hipLaunchKernelGGL(ring_copy_flat_kernel<int4>, dim3(blocks), dim3(256), 0, s, (char*)ring,
                         (uint32_t)cap, (uint32_t)slot0, (const char*)src, (uint32_t)src_rows,
                         (uint32_t)row0, (uint32_t)n, (uint32_t)(rb / 16), (uint32_t)total, rb);
    else
      hipLaunchKernelGGL(ring_copy_flat_kernel<int>, dim3(blocks), dim3(256), 0, s, (char*)ring,
                         (uint32_t)cap, (uint32_t)slot0, (const char*)src, (uint32_t)src_rows,
                         (uint32_t)row0, (uint32_t)n, (uint32_t)(rb / 4), (uint32_t)total, rb);
  } else if (rb % 16 == 0 && al % 16 == 0)
    hipLaunchKernelGGL(ring_copy_kernel<int4>, grid, dim3(64), 0, s, (char*)ring, cap, slot0,
                       (const char*)src, src_rows, row0, rb);
  else if (rb % 4 == 0 && al % 4 == 0)
    hipLaunchKernelGGL(ring_copy_kernel<int>, grid, dim3(256), 0, s, (char*)ring, cap, slot0,
                       (const char*)src, src_rows, row0, rb);
  else
    hipLaunchKernelGGL(ring_copy_kernel<short>, grid, dim3(256), 0, s, (char*)ring, cap, slot0,
                       (const char*)src, src_rows, row0, rb);
  return hipGetLastError();
}

bool pad_job_ok(const PadJob& j) {
  const RowGather& a = j.src;
  if (j.R < 0 || j.Cpad < 2 || (j.Cpad & 1) || !j.dst) return false;
  if ((uintptr_t)j.dst % 4 || j.R * j.Cpad >= ((int64_t)1 << 31)) return false;
  if (a.cur == nullptr && a.mem == nullptr) return true;  // zeros
  if (j.C < 2 || j.C > j.Cpad || (j.C & 1)) return false;
  const uintptr_t al = (uintptr_t)a.cur | (a.mem_len ? (uintptr_t)a.mem : 0);
  if (a.lda < j.C || (a.lda & 1) || al % 4) return false;
  const int64_t per = a.mem_len + a.cur_rows;
  if (per <= 0 || a.mem_len < 0 || a.cur_rows < 0 || per >= 0x7fffffff) return false;
  if (a.mem_len > 0 && (a.mem_cap > 0x7fffffff || a.mem_start < 0 || a.mem_start >= a.mem_cap))
    return false;
  return true;
}

hipError_t launch_pad_rows(const PadJob* jobs, int n, hipStream_t s) {
  if (n < 0 || n > PAD_MAX) return hipErrorInvalidValue;
  PadJobsK k{};
  uint32_t blocks = 0;
  for (int i = 0; i < n; ++i) {
    if (!pad_job_ok(jobs[i])) return hipErrorInvalidValue;
    if (jobs[i].R == 0) continue;
    k.j[k.n] = jobs[i];
    blocks += (uint32_t)((jobs[i].R + 4 * PAD_RPW - 1) / (4 * PAD_RPW));
    k.block_end[k.n++] = blocks;
  }
  if (k.n == 0) return hipSuccess;
  hipLaunchKernelGGL(pad_rows_kernel, dim3(blocks), dim3(256), 0, s, k);
  return hipGetLastError();
}

hipError_t launch_fill_f32(float* p, int64_t n, float value, hipStream_t s) {
  if (n == 0) return hipSuccess;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(fill_kernel, dim3((unsigned)blocks), dim3(256), 0, s, p, n, value);
  return hipGetLastError();
}

}  // namespace txl
