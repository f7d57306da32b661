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
template <typename T>
__global__ __launch_bounds__(256) void layer_norm_kernel(const float* __restrict__ y,
                                                         const T* __restrict__ gamma,
                                                         const T* __restrict__ beta, float eps,
                                                         int64_t D, T* __restrict__ out) {
  __shared__ float red[4];
  const int64_t row = blockIdx.x;
  const float* x = y + row * D;
  float s = 0.f;
  for (int64_t c = threadIdx.x; c < D; c += blockDim.x) s += x[c];
  const float mean = block_sum(s, red) / (float)D;
  float v = 0.f;
  for (int64_t c = threadIdx.x; c < D; c += blockDim.x) {
    const float t = x[c] - mean;
    v += t * t;
  }
  const float var = block_sum(v, red) / (float)D;
  const float inv = rsqrtf(var + eps);
  T* o = out + row * D;
  for (int64_t c = threadIdx.x; c < D; c += blockDim.x)
    Elt<T>::store(o + c, (x[c] - mean) * inv * Elt<T>::load(gamma + c) + Elt<T>::load(beta + c));
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

__global__ void fill_kernel(float* p, int64_t n, float v) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    p[i] = v;
}

}  // namespace

hipError_t launch_layer_norm(int dtype, const float* y, const void* gamma, const void* beta,
                             float eps, int64_t rows, int64_t D, void* out, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  if (dtype == 0)
    hipLaunchKernelGGL(layer_norm_kernel<float>, dim3((unsigned)rows), dim3(256), 0, s, y,
                       (const float*)gamma, (const float*)beta, eps, D, (float*)out);
  else
    hipLaunchKernelGGL(layer_norm_kernel<uint16_t>, dim3((unsigned)rows), dim3(256), 0, s, y,
                       (const uint16_t*)gamma, (const uint16_t*)beta, eps, D, (uint16_t*)out);
  return hipGetLastError();
}

hipError_t launch_ring_copy(int dtype, void* ring, int64_t cap, int64_t slot0, const void* src,
                            int64_t src_rows, int64_t row0, int64_t n, int64_t B, int64_t D,
                            hipStream_t s) {
  if (n == 0 || B == 0) return hipSuccess;
  const int64_t es = dtype == 0 ? 4 : 2;
  const int64_t rb = D * es;
  const uintptr_t al = (uintptr_t)ring | (uintptr_t)src;
  dim3 grid((unsigned)n, (unsigned)B);
  if (rb % 16 == 0 && al % 16 == 0)
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

hipError_t launch_fill_f32(float* p, int64_t n, float value, hipStream_t s) {
  if (n == 0) return hipSuccess;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(fill_kernel, dim3((unsigned)blocks), dim3(256), 0, s, p, n, value);
  return hipGetLastError();
}

}  // namespace txl
