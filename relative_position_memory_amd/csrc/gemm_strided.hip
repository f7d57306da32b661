// Batched GEMM with arbitrary element strides, fp32 accumulation and output.
// It serves the backward pass, whose products take operands transposed and
// strided in every way (P^T dO, dS^T qc, dY^T X, dY W).  Two kernels over the
// same 64 x 64 output tiles and K split:
//  * fp32: 256 threads, each a 4 x 4 block, K in steps of 16 staged through LDS
//    (operands widened to fp32 on the way in);
//  * bf16 matrix cores (StridedGemm::bf16_mfma): 4 waves, each one 32 x 32
//    block of v_mfma_f32_32x32x16_bf16, K in steps of 128.  Each operand is read
//    along whichever of its axes is contiguous (8 consecutive k of one row, or
//    4 consecutive rows at 2 k), rounded to bf16 in registers and written to LDS
//    k-contiguous, so the fragment reads are 16-byte rows.  The next step's
//    global loads are in flight during the current step's products.
#include "txl_internal.h"

namespace txl {
namespace {

constexpr int TM = 64, TN = 64, TK = 16;
constexpr int MK = 128;  // matrix-core K step (measured: 128 beats 32 and 64)

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;

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

__device__ inline uint32_t pack_bf16_pair(float lo, float hi) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){lo, hi}, bf16x2));
}

// n consecutive elements (n = 4 or 8) at element offset off, widened to fp32;
// off is a multiple of 4 (fp32) or of n (bf16), so the loads are 16 or 8 bytes.
template <typename T, int n>
__device__ inline void ld_vec(const void* p, int64_t off, float* v);
template <>
__device__ inline void ld_vec<float, 8>(const void* p, int64_t off, float* v) {
  const float4 a = *(const float4*)((const float*)p + off);
  const float4 b = *(const float4*)((const float*)p + off + 4);
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}
template <>
__device__ inline void ld_vec<float, 4>(const void* p, int64_t off, float* v) {
  const float4 a = *(const float4*)((const float*)p + off);
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
}
template <>
__device__ inline void ld_vec<uint16_t, 8>(const void* p, int64_t off, float* v) {
  const uint4 a = *(const uint4*)((const uint16_t*)p + off);
  const uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    v[2 * e] = bf16_to_f32((uint16_t)(w[e] & 0xffffu));
    v[2 * e + 1] = bf16_to_f32((uint16_t)(w[e] >> 16));
  }
}
template <>
__device__ inline void ld_vec<uint16_t, 4>(const void* p, int64_t off, float* v) {
  const uint2 a = *(const uint2*)((const uint16_t*)p + off);
  v[0] = bf16_to_f32((uint16_t)(a.x & 0xffffu));
  v[1] = bf16_to_f32((uint16_t)(a.x >> 16));
  v[2] = bf16_to_f32((uint16_t)(a.y & 0xffffu));
  v[3] = bf16_to_f32((uint16_t)(a.y >> 16));
}

// Operand staging flags: bit 0 = read 4 consecutive rows at 2 k (the row axis is
// contiguous), else 8 consecutive k of one row; bit 1 = the vector loads are
// aligned (checked on the host).
constexpr int ST_ROWS = 1, ST_VEC = 2;

// One thread's share of a 64 x KS block of X(row, k) = p[base + row sr + k sk]
// (rows r0.., k k0..; zero outside R rows and kend), as KS / 32 units of 4
// packed bf16 pairs.  Unit u = tid + 256 x.
template <typename T, int KS>
__device__ inline void stage_load(const void* p, int64_t base, int64_t sr, int64_t sk, int64_t R,
                                  int64_t r0, int64_t k0, int64_t kend, int flags, int tid,
                                  uint32_t (&w)[KS / 32][4]) {
#pragma unroll
  for (int x = 0; x < KS / 32; ++x) {
    const int u = tid + 256 * x;
    if (!(flags & ST_ROWS)) {  // row r0 + u / (KS / 8), k = k0 + 8 (u % (KS / 8)) + e
      const int64_t r = r0 + u / (KS / 8), k = k0 + 8 * (u % (KS / 8));
      float v[8];
      if ((flags & ST_VEC) && r < R && k + 8 <= kend) {
        ld_vec<T, 8>(p, base + r * sr + k, v);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e)
          v[e] = (r < R && k + e < kend) ? ld<T>(p, base + r * sr + (k + e) * sk) : 0.f;
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) w[x][e] = pack_bf16_pair(v[2 * e], v[2 * e + 1]);
    } else {  // rows r0 + 4 (u % 16) + i, k = k0 + 2 (u / 16) + {0, 1}
      const int64_t r = r0 + 4 * (u & 15), k = k0 + 2 * (u >> 4);
      float v0[4], v1[4];
      if ((flags & ST_VEC) && r + 4 <= R) {
        if (k < kend) ld_vec<T, 4>(p, base + r + k * sk, v0);
        else v0[0] = v0[1] = v0[2] = v0[3] = 0.f;
        if (k + 1 < kend) ld_vec<T, 4>(p, base + r + (k + 1) * sk, v1);
        else v1[0] = v1[1] = v1[2] = v1[3] = 0.f;
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          v0[i] = (r + i < R && k < kend) ? ld<T>(p, base + (r + i) * sr + k * sk) : 0.f;
          v1[i] = (r + i < R && k + 1 < kend) ? ld<T>(p, base + (r + i) * sr + (k + 1) * sk) : 0.f;
        }
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) w[x][i] = pack_bf16_pair(v0[i], v1[i]);
    }
  }
}

// LDS block [64][KS + 8], k contiguous
template <int KS>
__device__ inline void stage_store(uint16_t* Xs, int flags, int tid, const uint32_t (&w)[KS / 32][4]) {
  constexpr int P = KS + 8;
#pragma unroll
  for (int x = 0; x < KS / 32; ++x) {
    const int u = tid + 256 * x;
    if (!(flags & ST_ROWS)) {
      *(uint4*)(Xs + (u / (KS / 8)) * P + 8 * (u % (KS / 8))) =
          make_uint4(w[x][0], w[x][1], w[x][2], w[x][3]);
    } else {
      const int r = 4 * (u & 15), k = 2 * (u >> 4);
#pragma unroll
      for (int i = 0; i < 4; ++i) *(uint32_t*)(Xs + (r + i) * P + k) = w[x][i];
    }
  }
}

template <typename TA, typename TB, int KS>
__global__ __launch_bounds__(256) void gemm_strided_mfma_kernel(StridedGemm g, int ksplit, int fa,
                                                                int fb) {
  constexpr int P = KS + 8;
  __shared__ __align__(16) uint16_t As[TM * P];
  __shared__ __align__(16) uint16_t Bs[TN * P];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t z = blockIdx.z / ksplit;
  const int split = blockIdx.z % ksplit;
  const int64_t kchunk = ((g.K + ksplit - 1) / ksplit + KS - 1) / KS * KS;
  const int64_t kbeg = split * kchunk, kend = kbeg + kchunk < g.K ? kbeg + kchunk : g.K;
  const int64_t m0 = (int64_t)blockIdx.y * TM, n0 = (int64_t)blockIdx.x * TN;
  const int64_t zq = z / g.zdiv, zr = z % g.zdiv;
  const int64_t abase = zq * g.A.s1 + zr * g.A.s2;
  const int64_t bbase = zq * g.B.s1 + zr * g.B.s2;
  // A is staged as X(row m, k), B as X(row n, k)
  uint32_t wa[KS / 32][4], wb[KS / 32][4];
  if (kbeg < kend) {
    stage_load<TA, KS>(g.A.p, abase, g.A.si, g.A.sj, g.M, m0, kbeg, kend, fa, tid, wa);
    stage_load<TB, KS>(g.B.p, bbase, g.B.sj, g.B.si, g.N, n0, kbeg, kend, fb, tid, wb);
  }
  const int wm = wave >> 1, wn = wave & 1;
  // fragment rows: lane l supplies row l % 32 of its wave's block, k 8 (l / 32) .. + 8
  const uint16_t* af = As + (32 * wm + (lane & 31)) * P + 8 * (lane >> 5);
  const uint16_t* bfp = Bs + (32 * wn + (lane & 31)) * P + 8 * (lane >> 5);
  f32x16 acc;
#pragma unroll
  for (int x = 0; x < 16; ++x) acc[x] = 0.f;
  for (int64_t k0 = kbeg; k0 < kend; k0 += KS) {
    __syncthreads();  // the previous step's fragment reads are done
    stage_store<KS>(As, fa, tid, wa);
    stage_store<KS>(Bs, fb, tid, wb);
    __syncthreads();
    if (k0 + KS < kend) {
      stage_load<TA, KS>(g.A.p, abase, g.A.si, g.A.sj, g.M, m0, k0 + KS, kend, fa, tid, wa);
      stage_load<TB, KS>(g.B.p, bbase, g.B.sj, g.B.si, g.N, n0, k0 + KS, kend, fb, tid, wb);
    }
#pragma unroll
    for (int s = 0; s < KS / 16; ++s) {
      const bf16x8 a = *(const bf16x8*)(af + 16 * s);
      const bf16x8 b = *(const bf16x8*)(bfp + 16 * s);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc, 0, 0, 0);
    }
  }
  // lane l, register x: row 32 wm + 8 (x / 4) + 4 (l / 32) + x % 4, column 32 wn + l % 32
  const int64_t n = n0 + 32 * wn + (lane & 31);
  if (n >= g.N) return;
  const int64_t cbase = zq * g.c1 + zr * g.c2;
#pragma unroll
  for (int x = 0; x < 16; ++x) {
    const int64_t m = m0 + 32 * wm + 8 * (x >> 2) + 4 * (lane >> 5) + (x & 3);
    if (m >= g.M) continue;
    float* c = g.C + cbase + m * g.cm + n * g.cn;
    const float v = g.alpha * acc[x];
    if (ksplit > 1)
      atomicAdd(c, v);
    else
      *c = g.accumulate ? *c + v : v;
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

// Staging flags of an operand read as X(row, k) = p[... + row sr + k sk] (see stage_load).
int stage_flags(const StridedOperand& o, int64_t sr, int64_t sk, int dtype) {
  const uintptr_t p = (uintptr_t)o.p;
  if (sk == 1) {  // 8 consecutive k: 16-byte loads at offsets that are multiples of 4 / 8
    const int64_t q = dtype == 0 ? 4 : 8;
    const bool vec = p % 16 == 0 && sr % q == 0 && o.s1 % q == 0 && o.s2 % q == 0;
    return vec ? ST_VEC : 0;
  }
  if (sr == 1) {  // 4 consecutive rows: 16 (fp32) or 8 (bf16) bytes at multiples of 4
    const bool vec = p % (dtype == 0 ? 16 : 8) == 0 && sk % 4 == 0 && o.s1 % 4 == 0 &&
                     o.s2 % 4 == 0;
    return ST_ROWS | (vec ? ST_VEC : 0);
  }
  return 0;  // neither axis contiguous: element loads
}

template <int KS>
void launch_mfma_variant(const StridedGemm& g, dim3 grid, int k, int fa, int fb, hipStream_t s) {
  if (g.a_dtype == 0 && g.b_dtype == 0)
    hipLaunchKernelGGL((gemm_strided_mfma_kernel<float, float, KS>), grid, dim3(256), 0, s, g, k, fa,
                       fb);
  else if (g.a_dtype == 0 && g.b_dtype == 1)
    hipLaunchKernelGGL((gemm_strided_mfma_kernel<float, uint16_t, KS>), grid, dim3(256), 0, s, g, k,
                       fa, fb);
  else if (g.a_dtype == 1 && g.b_dtype == 0)
    hipLaunchKernelGGL((gemm_strided_mfma_kernel<uint16_t, float, KS>), grid, dim3(256), 0, s, g, k,
                       fa, fb);
  else
    hipLaunchKernelGGL((gemm_strided_mfma_kernel<uint16_t, uint16_t, KS>), grid, dim3(256), 0, s, g,
                       k, fa, fb);
}

hipError_t launch_gemm_strided(const StridedGemm& g, hipStream_t s) {
  if (g.M <= 0 || g.N <= 0 || g.batch <= 0) return hipSuccess;
  if (g.zdiv <= 0 || g.batch > 65535 || (g.N + TN - 1) / TN > 0x7fffffff ||
      (g.M + TM - 1) / TM > 65535)
    return hipErrorInvalidValue;
  // Split K when the tiles alone leave the GPU short of workgroups (about two per
  // CU for the matrix-core kernel, four for the fp32 one), each split at least 256
  // deep; the splits add atomically.
  const int64_t wg_target = g.bf16_mfma ? 512 : 1024;
  const int64_t tiles = ((g.N + TN - 1) / TN) * ((g.M + TM - 1) / TM) * g.batch;
  int64_t ks = (wg_target + tiles - 1) / tiles;
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
  if (g.bf16_mfma) {
    const int fa = stage_flags(g.A, g.A.si, g.A.sj, g.a_dtype);
    const int fb = stage_flags(g.B, g.B.sj, g.B.si, g.b_dtype);
    launch_mfma_variant<MK>(g, grid, k, fa, fb, s);
    return hipGetLastError();
  }
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
