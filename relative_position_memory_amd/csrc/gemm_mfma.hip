// Projection GEMM, bf16 matrix-core path for gfx950:
//   C[m][n] = sum_k A[m][k] * W[n][k]      (y = x W^T, fp32 accumulation)
// A's rows are gathered (memory ring rows, then the current rows: the extended
// context [SG(m) o h] of Transformer-XL section 3.2 is never materialised).
//
// 128 x 128 output tile per workgroup of 4 waves (2 x 2), each wave 64 x 64 =
// 2 x 2 blocks of v_mfma_f32_32x32x16_bf16.  K is walked 64 at a time through
// double-buffered LDS (row pitch 72 bf16: 16-byte reads without bank conflicts);
// the next step's tiles are prefetched into registers while the current one
// is multiplied.  Both operands are K-contiguous, so every MFMA fragment is one
// 16-byte LDS read.
#include "gemm_common.h"

namespace txl {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;

constexpr int GBM = 128, GBN = 128, GBK = 64, GKP = 72;
constexpr int NXCD = 8;

struct __align__(16) GSmem {
  uint16_t A[2][GBM * GKP];
  uint16_t W[2][GBN * GKP];
};

__device__ inline uint4 keep_if(uint4 v, bool keep) {
  const uint32_t k = keep ? 0xffffffffu : 0u;
  return make_uint4(v.x & k, v.y & k, v.z & k, v.w & k);
}

__global__ __launch_bounds__(256, 2) void gemm_mfma_kernel(GemmArgs g, int ntm, int ntn) {
  extern __shared__ __align__(16) char smem_raw[];
  GSmem& sm = *(GSmem*)smem_raw;

  // Row tiles of A are spread over the XCDs (block n runs on XCD n % 8); the
  // column tiles of one row tile run consecutively on the same XCD, so that
  // XCD's L2 serves the A tile to all of them.
  const int xcd = blockIdx.x % NXCD, k_on = blockIdx.x / NXCD;
  const int tm = (k_on / ntn) * NXCD + xcd;
  const int tn = k_on % ntn;
  if (tm >= ntm) return;
  const int64_t m0 = (int64_t)tm * GBM, n0 = (int64_t)tn * GBN;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int li = lane & 31, lh = lane >> 5;
  const int wm = wave >> 1, wn = wave & 1;
  const int K = (int)g.K;

  // loader: 16-byte chunk c of rows (tid >> 3) + 32 x, x = 0..3, of both tiles
  const int c = tid & 7;
  const uint16_t* arow[4];
  const uint16_t* wrow[4];
  bool aval[4], wval[4];
#pragma unroll
  for (int x = 0; x < 4; ++x) {
    const int64_t m = m0 + (tid >> 3) + 32 * x;
    const int64_t n = n0 + (tid >> 3) + 32 * x;
    aval[x] = m < g.M;
    wval[x] = n < g.N;
    arow[x] = (const uint16_t*)gather_row(g.a, aval[x] ? m : g.M - 1, 2);
    wrow[x] = (const uint16_t*)weight_row(g.w, wval[x] ? n : g.N - 1, 2);
  }
  uint4 ra[4], rw[4];
  auto load = [&](int k0) {
    const int kc = k0 + 8 * c;
    const int kk = kc < K ? kc : K - 8;  // clamped into the row; masked at store
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      ra[x] = *(const uint4*)(arow[x] + kk);
      rw[x] = *(const uint4*)(wrow[x] + kk);
    }
  };
  auto store = [&](int buf, int k0) {
    const bool kin = k0 + 8 * c < K;
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      const int row = (tid >> 3) + 32 * x;
      *(uint4*)&sm.A[buf][row * GKP + 8 * c] = keep_if(ra[x], kin && aval[x]);
      *(uint4*)&sm.W[buf][row * GKP + 8 * c] = keep_if(rw[x], kin && wval[x]);
    }
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int x = 0; x < 16; ++x) acc[i][j][x] = 0.f;

  const int nk = (K + GBK - 1) / GBK;
  load(0);
  store(0, 0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) load((kt + 1) * GBK);
#pragma unroll
    for (int s = 0; s < GBK / 16; ++s) {
      bf16x8 af[2], wf[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        af[i] = *(const bf16x8*)&sm.A[buf][(wm * 64 + 32 * i + li) * GKP + 16 * s + 8 * lh];
        wf[i] = *(const bf16x8*)&sm.W[buf][(wn * 64 + 32 * i + li) * GKP + 16 * s + 8 * lh];
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], wf[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) store(buf ^ 1, (kt + 1) * GBK);
    __syncthreads();
  }

  // ---- epilogue: lane (column li of block j, half lh), reg x -> row 8 (x/4) + 4 lh + x%4
  const int64_t per = g.a.mem_len + g.a.cur_rows;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int64_t n = n0 + wn * 64 + 32 * j + li;
    if (n >= g.N) continue;
    uint16_t* hcol = nullptr;  // EPI_HEADS: destination of (b = 0, t = 0) for column n
    if (g.e.mode == EPI_HEADS) {
      const int64_t which = n / g.e.HD, nn = n - which * g.e.HD;
      const int64_t head = nn / g.e.d, cc = nn - head * g.e.d;
      hcol = (uint16_t*)(which ? g.e.dst1 : g.e.dst0) + head * g.e.sh + cc;
    }
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int x4 = 0; x4 < 4; ++x4) {
        const int64_t mb = m0 + wm * 64 + 32 * i + 8 * x4 + 4 * lh;
        int64_t b = mb / per, t = mb - b * per;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int64_t m = mb + e;
          if (m < g.M) {
            const float v = acc[i][j][4 * x4 + e];
            if (g.e.mode == EPI_HEADS) {
              hcol[b * g.e.sb + t * g.e.st] = f32_to_bf16(v);
            } else {
              const uint16_t* res = (const uint16_t*)g.e.resid + m * g.N + n;
              g.e.y[m * g.N + n] = v + bf16_to_f32(*res);
            }
          }
          if (++t == per) { t = 0; ++b; }
        }
      }
  }
}

}  // namespace

bool gemm_mfma_supported(const GemmArgs& g) {
  if (g.K % 8 != 0 || g.K < 8 || g.a.lda % 8 != 0 || g.w.ldw % 8 != 0) return false;
  const uintptr_t al = (uintptr_t)g.a.cur | (uintptr_t)g.w.W0 | (uintptr_t)g.w.W1 |
                       (g.a.mem_len ? (uintptr_t)g.a.mem : 0);
  if (al % 16) return false;
  if (g.K > 0x7fffffffLL) return false;
  return true;
}

hipError_t launch_gemm_mfma(const GemmArgs& g, hipStream_t s) {
  const int ntm = (int)((g.M + GBM - 1) / GBM);
  const int ntn = (int)((g.N + GBN - 1) / GBN);
  const int64_t nblocks = (int64_t)NXCD * ((ntm + NXCD - 1) / NXCD) * ntn;
  const size_t smem = sizeof(GSmem);
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)gemm_mfma_kernel,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  hipLaunchKernelGGL(gemm_mfma_kernel, dim3((unsigned)nblocks), dim3(256), smem, s, g, ntm, ntn);
  return hipGetLastError();
}

}  // namespace txl
