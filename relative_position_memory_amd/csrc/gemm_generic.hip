// Projection GEMM, generic path (fp32 storage, or bf16 of any alignment):
//   C[m][n] = sum_k A[m][k] * W[n][k]     (y = x W^T, the pages' convention)
// with the row gather of RowGather (memory ring rows, then current rows) and
// the epilogues of Epilogue.  SIMT, 64x64 tiles, fp32 arithmetic.
#include "txl_internal.h"
#include "gemm_common.h"

namespace txl {
namespace {

constexpr int TM = 64, TN = 64, TK = 16;

template <typename T>
__global__ __launch_bounds__(256) void gemm_generic_kernel(GemmArgs g) {
  __shared__ float As[TK][TM + 4];
  __shared__ float Ws[TK][TN + 4];
  const int tid = threadIdx.x;
  const int tx = tid % 16, ty = tid / 16;
  const int64_t m0 = (int64_t)blockIdx.y * TM, n0 = (int64_t)blockIdx.x * TN;

  // loader: thread loads 4 consecutive k of one A row and of one W row
  const int lr = tid / 4, lk = (tid % 4) * 4;
  const int64_t am = m0 + lr, wn = n0 + lr;
  const T* arow = am < g.M ? (const T*)gather_row(g.a, am, sizeof(T)) : nullptr;
  const T* wrow = wn < g.N ? (const T*)weight_row(g.w, wn, sizeof(T)) : nullptr;

  float acc[4][4];
#pragma unroll
  for (int x = 0; x < 4; ++x)
#pragma unroll
    for (int y = 0; y < 4; ++y) acc[x][y] = 0.f;

  for (int64_t k0 = 0; k0 < g.K; k0 += TK) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int64_t kk = k0 + lk + e;
      As[lk + e][lr] = (arow && kk < g.K) ? Elt<T>::load(arow + kk) : 0.f;
      Ws[lk + e][lr] = (wrow && kk < g.K) ? Elt<T>::load(wrow + kk) : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < TK; ++kk) {
      float av[4], wv[4];
#pragma unroll
      for (int x = 0; x < 4; ++x) { av[x] = As[kk][ty * 4 + x]; wv[x] = Ws[kk][tx * 4 + x]; }
#pragma unroll
      for (int x = 0; x < 4; ++x)
#pragma unroll
        for (int y = 0; y < 4; ++y) acc[x][y] += av[x] * wv[y];
    }
    __syncthreads();
  }
#pragma unroll
  for (int x = 0; x < 4; ++x)
#pragma unroll
    for (int y = 0; y < 4; ++y) {
      const int64_t m = m0 + ty * 4 + x, n = n0 + tx * 4 + y;
      if (m < g.M && n < g.N) epilogue_store<T>(g, m, n, acc[x][y]);
    }
}

}  // namespace

hipError_t launch_gemm_generic(int dtype, const GemmArgs& g, hipStream_t s) {
  dim3 grid((unsigned)((g.N + TN - 1) / TN), (unsigned)((g.M + TM - 1) / TM));
  if (dtype == 0)
    hipLaunchKernelGGL(gemm_generic_kernel<float>, grid, dim3(256), 0, s, g);
  else
    hipLaunchKernelGGL(gemm_generic_kernel<uint16_t>, grid, dim3(256), 0, s, g);
  return hipGetLastError();
}

}  // namespace txl
