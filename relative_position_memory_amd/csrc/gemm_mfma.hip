// Projection GEMMs, bf16 matrix-core path for gfx950:
//   C[m][n] = sum_k A[m][k] * W[n][k]      (y = x W^T, fp32 accumulation)
// A's rows are gathered (memory ring rows, then the current rows: the extended
// context [SG(m) o h] of Transformer-XL section 3.2 is never materialised).
//
// (64 MI) x 128 output tile per workgroup of 4 waves (2 x 2), each wave
// (32 MI) x 64 = MI x 2 blocks of v_mfma_f32_32x32x16_bf16 (MI = 2 for large
// grids, 1 when 128-row tiles would leave CUs idle).  K is walked 64 at a time
// through double-buffered LDS (row pitch 72 bf16: 16-byte reads without bank
// conflicts).  Global loads run two K-steps ahead in two register sets, so a
// step's tiles have a whole step of compute to arrive before they are staged.
// Both operands are K-contiguous, so every MFMA fragment is one 16-byte LDS read.
//
// One launch may carry up to four independent problems (the layer step's q,
// k/v and r projections share K and run as one grid).
#include "gemm_common.h"

namespace txl {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;

constexpr int GBN = 128, GBK = 64, GKP = 72;
constexpr int NXCD = 8;
constexpr int MAXP = 4;

template <int MI>
struct __align__(16) GSmem {
  uint16_t A[2][64 * MI * GKP];
  uint16_t W[2][GBN * GKP];
};

struct GemmBatch {
  GemmArgs g[MAXP];
  int ntm[MAXP], ntn[MAXP];
  int block_end[MAXP];  // inclusive prefix sums of the problems' block counts
  int n;
};

__device__ inline uint4 keep_if(uint4 v, bool keep) {
  const uint32_t k = keep ? 0xffffffffu : 0u;
  return make_uint4(v.x & k, v.y & k, v.z & k, v.w & k);
}

// 16-byte chunk c = tid % 8 of A rows (tid / 8) + 32 x, x < 2 MI, and of
// W rows (tid / 8) + 32 x, x < 4.
template <int MI>
struct Regs {
  uint4 a[2 * MI], w[4];
};

template <int MI>
struct Loader {
  const uint16_t* arow[2 * MI];
  const uint16_t* wrow[4];
  bool aval[2 * MI], wval[4];
  int c, K, tid;

  __device__ void load(Regs<MI>& r, int k0) const {
    const int kc = k0 + 8 * c;
    const int kk = kc < K ? kc : K - 8;  // clamped into the row; masked at store
#pragma unroll
    for (int x = 0; x < 2 * MI; ++x) r.a[x] = *(const uint4*)(arow[x] + kk);
#pragma unroll
    for (int x = 0; x < 4; ++x) r.w[x] = *(const uint4*)(wrow[x] + kk);
  }
  __device__ void store(GSmem<MI>& sm, int buf, const Regs<MI>& r, int k0) const {
    const bool kin = k0 + 8 * c < K;
#pragma unroll
    for (int x = 0; x < 2 * MI; ++x)
      *(uint4*)&sm.A[buf][((tid >> 3) + 32 * x) * GKP + 8 * c] = keep_if(r.a[x], kin && aval[x]);
#pragma unroll
    for (int x = 0; x < 4; ++x)
      *(uint4*)&sm.W[buf][((tid >> 3) + 32 * x) * GKP + 8 * c] = keep_if(r.w[x], kin && wval[x]);
  }
};

template <int MI>
__device__ inline void mma_step(const GSmem<MI>& sm, int buf, int wm, int wn, int li, int lh,
                                f32x16 (&acc)[MI][2]) {
#pragma unroll
  for (int s = 0; s < GBK / 16; ++s) {
    bf16x8 af[MI], wf[2];
#pragma unroll
    for (int i = 0; i < MI; ++i)
      af[i] = *(const bf16x8*)&sm.A[buf][(wm * 32 * MI + 32 * i + li) * GKP + 16 * s + 8 * lh];
#pragma unroll
    for (int j = 0; j < 2; ++j)
      wf[j] = *(const bf16x8*)&sm.W[buf][(wn * 64 + 32 * j + li) * GKP + 16 * s + 8 * lh];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], wf[j], acc[i][j], 0, 0, 0);
  }
}

template <int MI>
__global__ __launch_bounds__(256, 2) void gemm_mfma_kernel(GemmBatch bt) {
  constexpr int BM = 64 * MI;
  extern __shared__ __align__(16) char smem_raw[];
  GSmem<MI>& sm = *(GSmem<MI>*)smem_raw;

  int p = 0;
  while (p + 1 < bt.n && (int)blockIdx.x >= bt.block_end[p]) ++p;
  const GemmArgs& g = bt.g[p];
  const int ntm = bt.ntm[p], ntn = bt.ntn[p];
  const int bid = (int)blockIdx.x - (p ? bt.block_end[p - 1] : 0);
  // Row tiles of A are spread over the XCDs (block n runs on XCD n % 8; every
  // problem's block range starts at a multiple of 8); the column tiles of one
  // row tile run consecutively on the same XCD, whose L2 then serves the A tile
  // to all of them.
  const int xcd = bid % NXCD, k_on = bid / NXCD;
  const int tm = (k_on / ntn) * NXCD + xcd;
  const int tn = k_on % ntn;
  if (tm >= ntm) return;
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * GBN;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int li = lane & 31, lh = lane >> 5;
  const int wm = wave >> 1, wn = wave & 1;

  Loader<MI> ld;
  ld.c = tid & 7;
  ld.K = (int)g.K;
  ld.tid = tid;
#pragma unroll
  for (int x = 0; x < 2 * MI; ++x) {
    const int64_t m = m0 + (tid >> 3) + 32 * x;
    ld.aval[x] = m < g.M;
    ld.arow[x] = (const uint16_t*)gather_row(g.a, ld.aval[x] ? m : g.M - 1, 2);
  }
#pragma unroll
  for (int x = 0; x < 4; ++x) {
    const int64_t n = n0 + (tid >> 3) + 32 * x;
    ld.wval[x] = n < g.N;
    ld.wrow[x] = (const uint16_t*)weight_row(g.w, ld.wval[x] ? n : g.N - 1, 2);
  }

  f32x16 acc[MI][2];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int x = 0; x < 16; ++x) acc[i][j][x] = 0.f;

  // Invariant at the top of step kt: LDS buffer kt%2 holds tile kt, register
  // set (kt+1)%2 holds (or is receiving) tile kt+1, set kt%2 is free.
  const int nk = (ld.K + GBK - 1) / GBK;
  Regs<MI> r0, r1;
  ld.load(r0, 0);
  if (nk > 1) ld.load(r1, GBK);
  ld.store(sm, 0, r0, 0);
  __syncthreads();
  for (int kt = 0; kt < nk; kt += 2) {
    if (kt + 2 < nk) ld.load(r0, (kt + 2) * GBK);
    mma_step<MI>(sm, 0, wm, wn, li, lh, acc);
    if (kt + 1 < nk) ld.store(sm, 1, r1, (kt + 1) * GBK);
    __syncthreads();
    if (kt + 1 >= nk) break;
    if (kt + 3 < nk) ld.load(r1, (kt + 3) * GBK);
    mma_step<MI>(sm, 1, wm, wn, li, lh, acc);
    if (kt + 2 < nk) ld.store(sm, 0, r0, (kt + 2) * GBK);
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
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int x4 = 0; x4 < 4; ++x4) {
        const int64_t mb = m0 + wm * 32 * MI + 32 * i + 8 * x4 + 4 * lh;
        int64_t b = mb / per, t = mb - b * per;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int64_t m = mb + e;
          if (m < g.M) {
            const float v = acc[i][j][4 * x4 + e];
            if (g.e.mode == EPI_HEADS) {
              hcol[b * g.e.sb + t * g.e.st] = __builtin_bit_cast(uint16_t, (__bf16)v);
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

template <int MI>
hipError_t launch_mi(const GemmArgs* gs, int n, hipStream_t s) {
  constexpr int BM = 64 * MI;
  GemmBatch bt{};
  int64_t total = 0;
  for (int p = 0; p < n; ++p) {
    bt.g[p] = gs[p];
    bt.ntm[p] = (int)((gs[p].M + BM - 1) / BM);
    bt.ntn[p] = (int)((gs[p].N + GBN - 1) / GBN);
    total += (int64_t)NXCD * ((bt.ntm[p] + NXCD - 1) / NXCD) * bt.ntn[p];
    if (total > 0x7fffffffLL) return hipErrorInvalidValue;
    bt.block_end[p] = (int)total;
  }
  bt.n = n;
  if (total == 0) return hipSuccess;
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)gemm_mfma_kernel<MI>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)sizeof(GSmem<MI>));
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  hipLaunchKernelGGL(gemm_mfma_kernel<MI>, dim3((unsigned)total), dim3(256), sizeof(GSmem<MI>),
                     s, bt);
  return hipGetLastError();
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

hipError_t launch_gemm_mfma_multi(const GemmArgs* gs, int n, hipStream_t s, int num_cus) {
  if (n < 1 || n > MAXP) return hipErrorInvalidValue;
  // 128-row tiles when they still give every CU two workgroups, else 64-row tiles
  int64_t tiles128 = 0;
  for (int p = 0; p < n; ++p) tiles128 += ((gs[p].M + 127) / 128) * ((gs[p].N + GBN - 1) / GBN);
  if (tiles128 >= 2LL * num_cus) return launch_mi<2>(gs, n, s);
  return launch_mi<1>(gs, n, s);
}

hipError_t launch_gemm_mfma(const GemmArgs& g, hipStream_t s, int num_cus) {
  return launch_gemm_mfma_multi(&g, 1, s, num_cus);
}

}  // namespace txl
