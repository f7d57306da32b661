// Batched GEMM with arbitrary element strides, fp32 accumulation and output.
// It serves the backward pass, whose products take operands transposed and
// strided in every way (P^T dO, dS^T qc, dY^T X, dY W): a 64 x 64 output tile
// per workgroup of 256 threads, each thread a 4 x 4 block, K in steps of 16
// staged through LDS (operands widened to fp32 on the way in).
#include "txl_internal.h"

namespace txl {
namespace {

constexpr int TM = 64, TN = 64, TK = 16;

template <typename T>
__device__ inline float ld(const void* p, int64_t off) {
  return Elt<T>::load((const T*)p + off);
}

template <typename TA, typename TB>
__global__ __launch_bounds__(256) void gemm_strided_kernel(StridedGemm g, int ksplit) {
  __shared__ float As[TK][TM + 4];
  __shared__ float Bs[TK][TN + 4];
  const int tid = threadIdx.x;
  // blockIdx.z = batch * ksplit + split; split s takes the s-th share of K and
  // adds its partial sums atomically (C was zeroed or holds the term to add to)
  const int64_t z = blockIdx.z / ksplit;
  const int split = blockIdx.z % ksplit;
  const int64_t kchunk = ((g.K + ksplit - 1) / ksplit + TK - 1) / TK * TK;
  const int64_t kbeg = split * kchunk, kend = kbeg + kchunk < g.K ? kbeg + kchunk : g.K;
  const int64_t m0 = (int64_t)blockIdx.y * TM, n0 = (int64_t)blockIdx.x * TN;
  const int64_t zq = z / g.zdiv, zr = z % g.zdiv;
  const int64_t abase = zq * g.A.s1 + zr * g.A.s2;
  const int64_t bbase = zq * g.B.s1 + zr * g.B.s2;
  const int tm = tid / 16, tn = tid % 16;  // this thread's rows 4 tm .., columns 4 tn ..
  float acc[4][4] = {};
  for (int64_t k0 = kbeg; k0 < kend; k0 += TK) {
    // stage A[m0 .. +64][k0 .. +16] and B[k0 .. +16][n0 .. +64] (zero outside)
    for (int e = tid; e < TK * TM; e += 256) {
      const int kk = e / TM, mm = e % TM;
      const int64_t m = m0 + mm, k = k0 + kk;
      As[kk][mm] = (m < g.M && k < kend) ? ld<TA>(g.A.p, abase + m * g.A.si + k * g.A.sj) : 0.f;
    }
    for (int e = tid; e < TK * TN; e += 256) {
      const int kk = e / TN, nn = e % TN;
      const int64_t n = n0 + nn, k = k0 + kk;
      Bs[kk][nn] = (n < g.N && k < kend) ? ld<TB>(g.B.p, bbase + k * g.B.si + n * g.B.sj) : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < TK; ++kk) {
      float a[4], b[4];
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        a[x] = As[kk][4 * tm + x];
        b[x] = Bs[kk][4 * tn + x];
      }
#pragma unroll
      for (int x = 0; x < 4; ++x)
#pragma unroll
        for (int y = 0; y < 4; ++y) acc[x][y] += a[x] * b[y];
    }
    __syncthreads();
  }
  const int64_t cbase = zq * g.c1 + zr * g.c2;
#pragma unroll
  for (int x = 0; x < 4; ++x) {
    const int64_t m = m0 + 4 * tm + x;
    if (m >= g.M) continue;
#pragma unroll
    for (int y = 0; y < 4; ++y) {
      const int64_t n = n0 + 4 * tn + y;
      if (n >= g.N) continue;
      float* c = g.C + cbase + m * g.cm + n * g.cn;
      const float v = g.alpha * acc[x][y];
      if (ksplit > 1)
        atomicAdd(c, v);
      else
        *c = g.accumulate ? *c + v : v;
    }
  }
}

// C = 0 before split-K partial sums are added to it
__global__ void zero_c_kernel(StridedGemm g) {
  const int64_t n = g.M * g.N;
  for (int64_t z = 0; z < g.batch; ++z) {
    const int64_t base = (z / g.zdiv) * g.c1 + (z % g.zdiv) * g.c2;
    for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < n;
         e += (int64_t)gridDim.x * blockDim.x)
      g.C[base + (e / g.N) * g.cm + (e % g.N) * g.cn] = 0.f;
  }
}

}  // namespace

hipError_t launch_gemm_strided(const StridedGemm& g, hipStream_t s) {
  if (g.M <= 0 || g.N <= 0 || g.batch <= 0) return hipSuccess;
  if (g.zdiv <= 0 || g.batch > 65535 || (g.N + TN - 1) / TN > 0x7fffffff ||
      (g.M + TM - 1) / TM > 65535)
    return hipErrorInvalidValue;
  // Split K when the tiles alone leave the GPU short of workgroups (about four
  // per CU wanted), each split at least 256 deep; the splits add atomically.
  const int64_t tiles = ((g.N + TN - 1) / TN) * ((g.M + TM - 1) / TM) * g.batch;
  int64_t ks = (1024 + tiles - 1) / tiles;
  if (ks > g.K / 256) ks = g.K / 256;
  if (ks > 16) ks = 16;
  if (ks < 1 || g.batch * ks > 65535) ks = 1;
  if (ks > 1 && !g.accumulate) {
    hipLaunchKernelGGL(zero_c_kernel, dim3(256), dim3(256), 0, s, g);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const dim3 grid((unsigned)((g.N + TN - 1) / TN), (unsigned)((g.M + TM - 1) / TM),
                  (unsigned)(g.batch * ks));
  const int k = (int)ks;
  if (g.a_dtype == 0 && g.b_dtype == 0)
    hipLaunchKernelGGL((gemm_strided_kernel<float, float>), grid, dim3(256), 0, s, g, k);
  else if (g.a_dtype == 0 && g.b_dtype == 1)
    hipLaunchKernelGGL((gemm_strided_kernel<float, uint16_t>), grid, dim3(256), 0, s, g, k);
  else if (g.a_dtype == 1 && g.b_dtype == 0)
    hipLaunchKernelGGL((gemm_strided_kernel<uint16_t, float>), grid, dim3(256), 0, s, g, k);
  else
    hipLaunchKernelGGL((gemm_strided_kernel<uint16_t, uint16_t>), grid, dim3(256), 0, s, g, k);
  return hipGetLastError();
}

}  // namespace txl
