// Element kernels of the layer step's backward pass (Transformer-XL section 3.3,
// the N-layer procedure: h_out = LayerNorm(a W_o^T + h_in) with the biased
// variance; section 3.2: the memory's gradient is stopped).  The products of
// the backward run through the strided GEMM; these kernels cover the
// LayerNorm backward, the copies and the gather of [memory ; h_in].
#include "txl_internal.h"

#include <type_traits>

namespace txl {
namespace {

template <typename E>
__device__ inline float ldE(const void* p, int64_t off) {
  return Elt<E>::load((const E*)p + off);
}

template <typename E>
__global__ void to_f32_kernel(const void* src, float* dst, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    dst[i] = ldE<E>(src, i);
}

__global__ void zero_f32_kernel(float* p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    p[i] = 0.f;
}

__device__ inline float block_sum(float v, float* red) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  __syncthreads();
  if (lane == 0) red[w] = v;
  __syncthreads();
  float t = 0.f;
  for (int i = 0; i < (int)(blockDim.x >> 6); ++i) t += red[i];
  return t;
}

// One row per workgroup: mean and 1/sigma of y, and
//   dy = (dyhat - mean(dyhat) - yhat mean(dyhat yhat)) / sigma,  dyhat = dh_out gamma.
template <typename E>
__global__ __launch_bounds__(256) void ln_bwd_rows_kernel(const float* y, const void* gamma,
                                                          const void* dh_out, int64_t D, float eps,
                                                          float* dy, float* mean_out,
                                                          float* rstd_out) {
  __shared__ float red[4];
  const int64_t m = blockIdx.x;
  const float* yr = y + m * D;
  float s = 0.f;
  for (int64_t c = threadIdx.x; c < D; c += blockDim.x) s += yr[c];
  const float mu = block_sum(s, red) / (float)D;
  float v = 0.f;
  for (int64_t c = threadIdx.x; c < D; c += blockDim.x) v += (yr[c] - mu) * (yr[c] - mu);
  const float rstd = rsqrtf(block_sum(v, red) / (float)D + eps);
  float s1 = 0.f, s2 = 0.f;
  for (int64_t c = threadIdx.x; c < D; c += blockDim.x) {
    const float g = ldE<E>(dh_out, m * D + c) * ldE<E>(gamma, c);
    s1 += g;
    s2 += g * (yr[c] - mu) * rstd;
  }
  const float m1 = block_sum(s1, red) / (float)D;
  const float m2 = block_sum(s2, red) / (float)D;
  for (int64_t c = threadIdx.x; c < D; c += blockDim.x) {
    const float g = ldE<E>(dh_out, m * D + c) * ldE<E>(gamma, c);
    const float yh = (yr[c] - mu) * rstd;
    dy[m * D + c] = (g - m1 - yh * m2) * rstd;
  }
  if (threadIdx.x == 0) {
    mean_out[m] = mu;
    rstd_out[m] = rstd;
  }
}

// dgamma[c] += sum over a chunk of rows of dh_out yhat, dbeta[c] += sum of dh_out
template <typename E>
__global__ __launch_bounds__(256) void ln_bwd_cols_kernel(const float* y, const float* mean,
                                                          const float* rstd, const void* dh_out,
                                                          int64_t M, int64_t D, int64_t rows,
                                                          float* dgamma, float* dbeta) {
  const int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (c >= D) return;
  const int64_t m0 = (int64_t)blockIdx.y * rows;
  const int64_t m1 = m0 + rows < M ? m0 + rows : M;
  float sg = 0.f, sb = 0.f;
  for (int64_t m = m0; m < m1; ++m) {
    const float g = ldE<E>(dh_out, m * D + c);
    sg += g * (y[m * D + c] - mean[m]) * rstd[m];
    sb += g;
  }
  atomicAdd(dgamma + c, sg);
  atomicAdd(dbeta + c, sb);
}

// ctx[b][t] = t < len ? ring[b][(start + t) % cap] : h[b][t - len]   (rows of D elements),
// in groups of G consecutive elements of a row (16-byte copies when D % G == 0 and
// the three buffers are 16-byte aligned, else G = 1).
template <typename E, int G>
__global__ void gather_ctx_kernel(const void* ring, int64_t cap, int64_t start, int64_t len,
                                  const void* h, int64_t B, int64_t L, int64_t D, void* ctx) {
  typedef typename std::conditional<G == 1, E, uint4>::type V;
  const int64_t T = len + L, DG = D / G, n = B * T * DG;
  for (int64_t x = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; x < n;
       x += (int64_t)gridDim.x * blockDim.x) {
    const int64_t c = x % DG, bt = x / DG, t = bt % T, b = bt / T;
    int64_t slot = start + t;
    slot = slot >= cap ? slot - cap : slot;
    ((V*)ctx)[x] = t < len ? ((const V*)ring)[(b * cap + slot) * DG + c]
                           : ((const V*)h)[(b * L + (t - len)) * DG + c];
  }
}

struct ZeroList {
  float* p[16];
  int64_t end[16];  // running element counts
  int n;
};

// Grid-stride over the concatenation of the buffers.
__global__ void zero_many_kernel(ZeroList z) {
  const int64_t total = z.end[z.n - 1];
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    int b = 0;
    while (i >= z.end[b]) ++b;
    z.p[b][i - (b ? z.end[b - 1] : 0)] = 0.f;
  }
}

unsigned grid_for(int64_t n) {
  const int64_t g = (n + 255) / 256;
  return (unsigned)(g < 4096 ? (g > 0 ? g : 1) : 4096);
}

}  // namespace

hipError_t launch_zero_many(float* const* p, const int64_t* count, int n, hipStream_t s) {
  if (n < 1 || n > 16) return hipErrorInvalidValue;
  ZeroList z{};
  int64_t acc = 0;
  for (int b = 0; b < n; ++b) {
    if (count[b] < 0) return hipErrorInvalidValue;
    z.p[b] = p[b];
    acc += count[b];
    z.end[b] = acc;
  }
  z.n = n;
  if (acc == 0) return hipSuccess;
  hipLaunchKernelGGL(zero_many_kernel, dim3(grid_for(acc)), dim3(256), 0, s, z);
  return hipGetLastError();
}

hipError_t launch_to_f32(int dtype, const void* src, float* dst, int64_t n, hipStream_t s) {
  if (dtype == 1)
    hipLaunchKernelGGL(to_f32_kernel<uint16_t>, dim3(grid_for(n)), dim3(256), 0, s, src, dst, n);
  else
    hipLaunchKernelGGL(to_f32_kernel<float>, dim3(grid_for(n)), dim3(256), 0, s, src, dst, n);
  return hipGetLastError();
}

hipError_t launch_ln_bwd(int dtype, const float* y, const void* gamma, const void* dh_out,
                         int64_t M, int64_t D, float eps, float* dy, float* mean, float* rstd,
                         float* dgamma, float* dbeta, hipStream_t s, bool zeroed) {
  if (!zeroed) {
    hipLaunchKernelGGL(zero_f32_kernel, dim3(grid_for(D)), dim3(256), 0, s, dgamma, D);
    hipLaunchKernelGGL(zero_f32_kernel, dim3(grid_for(D)), dim3(256), 0, s, dbeta, D);
  }
  if (M > 0x7fffffffLL) return hipErrorInvalidValue;
  const int64_t rows = 16;  // enough row chunks to fill the GPU
  const dim3 gc((unsigned)((D + 255) / 256), (unsigned)((M + rows - 1) / rows));
  if (dtype == 1) {
    hipLaunchKernelGGL(ln_bwd_rows_kernel<uint16_t>, dim3((unsigned)M), dim3(256), 0, s, y, gamma,
                       dh_out, D, eps, dy, mean, rstd);
    hipLaunchKernelGGL(ln_bwd_cols_kernel<uint16_t>, gc, dim3(256), 0, s, y, mean, rstd, dh_out, M,
                       D, rows, dgamma, dbeta);
  } else {
    hipLaunchKernelGGL(ln_bwd_rows_kernel<float>, dim3((unsigned)M), dim3(256), 0, s, y, gamma,
                       dh_out, D, eps, dy, mean, rstd);
    hipLaunchKernelGGL(ln_bwd_cols_kernel<float>, gc, dim3(256), 0, s, y, mean, rstd, dh_out, M, D,
                       rows, dgamma, dbeta);
  }
  return hipGetLastError();
}

hipError_t launch_gather_ctx(int dtype, const void* ring, int64_t cap, int64_t start, int64_t len,
                             const void* h, int64_t B, int64_t L, int64_t D, void* ctx,
                             hipStream_t s) {
  const int64_t n = B * (len + L) * D;
  const int64_t per16 = dtype == 1 ? 8 : 4;  // elements per 16 bytes
  const bool vec = D % per16 == 0 &&
                   (((uintptr_t)ring | (uintptr_t)h | (uintptr_t)ctx) % 16) == 0;
  if (vec && dtype == 1)
    hipLaunchKernelGGL((gather_ctx_kernel<uint16_t, 8>), dim3(grid_for(n / 8)), dim3(256), 0, s,
                       ring, cap, start, len, h, B, L, D, ctx);
  else if (vec)
    hipLaunchKernelGGL((gather_ctx_kernel<float, 4>), dim3(grid_for(n / 4)), dim3(256), 0, s, ring,
                       cap, start, len, h, B, L, D, ctx);
  else if (dtype == 1)
    hipLaunchKernelGGL((gather_ctx_kernel<uint16_t, 1>), dim3(grid_for(n)), dim3(256), 0, s, ring,
                       cap, start, len, h, B, L, D, ctx);
  else
    hipLaunchKernelGGL((gather_ctx_kernel<float, 1>), dim3(grid_for(n)), dim3(256), 0, s, ring,
                       cap, start, len, h, B, L, D, ctx);
  return hipGetLastError();
}

}  // namespace txl
