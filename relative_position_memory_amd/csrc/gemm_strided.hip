// Batched GEMM with arbitrary element strides, fp32 accumulation and output.
// It serves the backward pass, whose products take operands transposed and
// strided in every way (P^T dO, dS^T qc, dY^T X, dY W).  Two kernels:
//  * fp32: 64 x 64 output tiles, 256 threads, each a 4 x 4 block, K in steps of
//    16 staged through LDS (operands widened to fp32 on the way in);
//  * bf16 matrix cores (StridedGemm::bf16_mfma): 64 x 64 or 128 x 128 tiles, 4
//    waves of v_mfma_f32_16x16x32_bf16, K in steps of 64.  Each operand is read
//    in 16-byte pieces along whichever of its axes is contiguous (8 consecutive
//    k of one row, or 8 consecutive rows at one k), rounded to bf16 and stored
//    to LDS as read: [row][k] or [k][row].  The fragments of a [k][row] tile
//    come through transposing LDS reads (ds_read_b64_tr_b16), those of a
//    [row][k] tile through two 8-byte reads in the same k order, so no layout
//    is transposed on the way in.  The next step's global loads are in flight
//    during the current step's products.
// Both split K across workgroups (atomic fp32 sums) when the tiles alone leave
// the GPU short of workgroups.
#include "txl_internal.h"

namespace txl {
namespace {

constexpr int TM = 64, TN = 64, TK = 16;
constexpr int KS = 64;  // matrix-core K step

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef short v4s __attribute__((ext_vector_type(4)));

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

// Operand staging flags: bit 0 = the row axis is contiguous (pieces of 8 rows at
// one k, tile [k][row]), else pieces of 8 k of one row (tile [row][k]); bit 1 =
// the 16-byte (bf16) or 2 x 16-byte (fp32) loads are aligned (checked on the host).
constexpr int ST_ROWS = 1, ST_VEC = 2;

// LDS tile of an R-row operand: [R][KS + 8] or [KS][R + 8] bf16
template <int R>
constexpr int tile_elems() {
  return R * (KS + 8) > KS * (R + 8) ? R * (KS + 8) : KS * (R + 8);
}

// A staged 8-element piece as loaded: fp32 keeps its two 16-byte loads (eight
// floats), bf16 its one; it is rounded to bf16 only when stored to LDS, so the
// wait for the loads falls after the products issued in between.
template <typename T> struct Raw;
template <> struct Raw<float> {
  float4 a, b;
  // elements e with bit e of keep clear become 0
  __device__ void mask(uint32_t keep) {
    a.x = keep & 1 ? a.x : 0.f; a.y = keep & 2 ? a.y : 0.f;
    a.z = keep & 4 ? a.z : 0.f; a.w = keep & 8 ? a.w : 0.f;
    b.x = keep & 16 ? b.x : 0.f; b.y = keep & 32 ? b.y : 0.f;
    b.z = keep & 64 ? b.z : 0.f; b.w = keep & 128 ? b.w : 0.f;
  }
  __device__ uint4 packed() const {
    return make_uint4(pack_bf16_pair(a.x, a.y), pack_bf16_pair(a.z, a.w),
                      pack_bf16_pair(b.x, b.y), pack_bf16_pair(b.z, b.w));
  }
  __device__ void load(const void* p, int64_t off) {
    a = *(const float4*)((const float*)p + off);
    b = *(const float4*)((const float*)p + off + 4);
  }
  __device__ void set(const float* v) {
    a = make_float4(v[0], v[1], v[2], v[3]);
    b = make_float4(v[4], v[5], v[6], v[7]);
  }
};
template <> struct Raw<uint16_t> {
  uint4 a;
  __device__ void mask(uint32_t keep) {
    auto m2 = [&](int e) { return (keep >> e & 1 ? 0x0000ffffu : 0u) | (keep >> (e + 1) & 1 ? 0xffff0000u : 0u); };
    a.x &= m2(0); a.y &= m2(2); a.z &= m2(4); a.w &= m2(6);
  }
  __device__ uint4 packed() const { return a; }
  __device__ void load(const void* p, int64_t off) { a = *(const uint4*)((const uint16_t*)p + off); }
  __device__ void set(const float* v) {
    a = make_uint4(pack_bf16_pair(v[0], v[1]), pack_bf16_pair(v[2], v[3]),
                   pack_bf16_pair(v[4], v[5]), pack_bf16_pair(v[6], v[7]));
  }
};

// This thread's pieces of the R x KS block of X(row, k) = p[base + row sr + k sk]
// (rows r0.., k k0..; zero outside Rmax rows and kend), 8 elements each.  Piece
// q = tid + 256 x: rows-contiguous: k q / (R / 8), rows 8 (q % (R / 8)) ..;
// else row q / (KS / 8), k 8 (q % (KS / 8)) ..
// When the whole block is inside and the layout allows 16-byte loads (a
// condition uniform over the workgroup) every piece is one unconditional load,
// so all of them are in flight together; otherwise each piece is checked, and
// loaded element by element where it crosses an edge.
template <typename T, int R>
__device__ inline void stage_load(const void* p, int64_t base, int64_t sr, int64_t sk, int64_t Rmax,
                                  int64_t r0, int64_t k0, int64_t kend, int flags, int tid,
                                  Raw<T> (&w)[R * KS / 2048]) {
  if ((flags & ST_VEC) && r0 + R <= Rmax && k0 + KS <= kend) {
#pragma unroll
    for (int x = 0; x < R * KS / 2048; ++x) {
      const int q = tid + 256 * x;
      if (flags & ST_ROWS) {
        const int64_t k = k0 + q / (R / 8), r = r0 + 8 * (q % (R / 8));
        w[x].load(p, base + r + k * sk);
      } else {
        const int64_t r = r0 + q / (KS / 8), k = k0 + 8 * (q % (KS / 8));
        w[x].load(p, base + r * sr + k);
      }
    }
    return;
  }
#pragma unroll
  for (int x = 0; x < R * KS / 2048; ++x) {
    const int q = tid + 256 * x;
    float v[8];
    if (flags & ST_ROWS) {
      const int64_t k = k0 + q / (R / 8), r = r0 + 8 * (q % (R / 8));
      if ((flags & ST_VEC) && k < kend && r + 8 <= Rmax) {
        ld_vec<T, 8>(p, base + r + k * sk, v);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e)
          v[e] = (k < kend && r + e < Rmax) ? ld<T>(p, base + (r + e) * sr + k * sk) : 0.f;
      }
    } else {
      const int64_t r = r0 + q / (KS / 8), k = k0 + 8 * (q % (KS / 8));
      if ((flags & ST_VEC) && r < Rmax && k + 8 <= kend) {
        ld_vec<T, 8>(p, base + r * sr + k, v);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e)
          v[e] = (r < Rmax && k + e < kend) ? ld<T>(p, base + r * sr + (k + e) * sk) : 0.f;
      }
    }
    w[x].set(v);
  }
}

// Causal mask of this thread's pieces of the block at rows r0, k k0 (see
// StridedGemm::causal_off): element (row, k) is kept when row <= k + off.
template <typename T, int R>
__device__ inline void stage_causal(int flags, int tid, int64_t r0, int64_t k0, int64_t off,
                                    Raw<T> (&w)[R * KS / 2048]) {
#pragma unroll
  for (int x = 0; x < R * KS / 2048; ++x) {
    const int q = tid + 256 * x;
    uint32_t keep = 0;
    if (flags & ST_ROWS) {  // rows r .. r + 7 at one k
      const int64_t k = k0 + q / (R / 8), r = r0 + 8 * (q % (R / 8));
#pragma unroll
      for (int e = 0; e < 8; ++e) keep |= (r + e <= k + off ? 1u : 0u) << e;
    } else {  // k .. k + 7 of one row
      const int64_t r = r0 + q / (KS / 8), k = k0 + 8 * (q % (KS / 8));
#pragma unroll
      for (int e = 0; e < 8; ++e) keep |= (r <= k + e + off ? 1u : 0u) << e;
    }
    w[x].mask(keep);
  }
}

template <typename T, int R>
__device__ inline void stage_store(uint16_t* Xs, int flags, int tid, const Raw<T> (&w)[R * KS / 2048]) {
#pragma unroll
  for (int x = 0; x < R * KS / 2048; ++x) {
    const int q = tid + 256 * x;
    const uint4 pk = w[x].packed();
    if (flags & ST_ROWS)
      *(uint4*)(Xs + (q / (R / 8)) * (R + 8) + 8 * (q % (R / 8))) = pk;
    else
      *(uint4*)(Xs + (q / (KS / 8)) * (KS + 8) + 8 * (q % (KS / 8))) = pk;
  }
}

// 16x16x32 operand fragment of rows rb .. rb + 15 and k 32 s .. 32 s + 31 of a
// staged tile: lane (g, n) gets row rb + n at k index 8 g + 4 h + e <-> k
// 32 s + 16 h + 4 g + e (h, e < 2, 4), the order the transposing reads produce.
template <int R>
__device__ inline bf16x8 frag(const uint16_t* Xs, int flags, int rb, int s, int g4, int n16) {
  if (flags & ST_ROWS) {
    constexpr int P = R + 8;
    const uint16_t* p = Xs + (32 * s + 4 * g4 + (n16 >> 2)) * P + rb + 4 * (n16 & 3);
    const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s*)p);
    const v4s hi =
        __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s*)(p + 16 * P));
    const v4s both[2] = {lo, hi};
    return *(const bf16x8*)both;
  }
  constexpr int P = KS + 8;
  const uint16_t* p = Xs + (rb + n16) * P + 32 * s + 4 * g4;
  const uint2 lo = *(const uint2*)p, hi = *(const uint2*)(p + 16);
  return __builtin_bit_cast(bf16x8, make_uint4(lo.x, lo.y, hi.x, hi.y));
}

// Output tile RM x RN; wave (wm, wn) of the 2 x 2 waves owns (RM / 32) x (RN / 32)
// blocks of 16 x 16 at rows RM / 2 wm + 16 x, columns RN / 2 wn + 16 y.
// AR, BR: the ST_ROWS bit of A's and B's staging flags, fixed per instantiation
// (fa, fb supply the ST_VEC bit), so a kernel carries only its layouts' code.
template <typename TA, typename TB, int RM, int RN, int AR, int BR>
__global__ __launch_bounds__(256, RM * RN <= 128 * 64 ? 2 : 1) void gemm_strided_mfma_kernel(StridedGemm g, int ksplit, int fa_in,
                                                                int fb_in) {
  const int fa = (AR ? ST_ROWS : 0) | (fa_in & ST_VEC), fb = (BR ? ST_ROWS : 0) | (fb_in & ST_VEC);
  constexpr int XM = RM / 32, XN = RN / 32;
  __shared__ __align__(16) uint16_t As[tile_elems<RM>()];
  __shared__ __align__(16) uint16_t Bs[tile_elems<RN>()];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g4 = lane >> 4, n16 = lane & 15;
  const int64_t z = blockIdx.z / ksplit;
  const int split = blockIdx.z % ksplit;
  const int64_t kchunk = ((g.K + ksplit - 1) / ksplit + KS - 1) / KS * KS;
  int64_t kbeg = split * kchunk;
  const int64_t kend = kbeg + kchunk < g.K ? kbeg + kchunk : g.K;
  const int64_t m0 = (int64_t)blockIdx.y * RM, n0 = (int64_t)blockIdx.x * RN;
  // causal A: the steps before the first k that sees row m0 hold no visible pair
  if (g.causal_on) {
    const int64_t kmin = (m0 - g.causal_off) > 0 ? (m0 - g.causal_off) / KS * KS : 0;
    kbeg = kbeg > kmin ? kbeg : (kmin < kend ? kmin : kend);
  }
  const int64_t zq = z / g.zdiv, zr = z % g.zdiv;
  const int64_t abase = zq * g.A.s1 + zr * g.A.s2;
  const int64_t bbase = zq * g.B.s1 + zr * g.B.s2;
  // A is staged as X(row m, k), B as X(row n, k)
  Raw<TA> wa[RM * KS / 2048];
  Raw<TB> wb[RN * KS / 2048];
  if (kbeg < kend) {
    stage_load<TA, RM>(g.A.p, abase, g.A.si, g.A.sj, g.M, m0, kbeg, kend, fa, tid, wa);
    stage_load<TB, RN>(g.B.p, bbase, g.B.sj, g.B.si, g.N, n0, kbeg, kend, fb, tid, wb);
  }
  const int wm = wave >> 1, wn = wave & 1;
  f32x4 acc[XM][XN];
#pragma unroll
  for (int x = 0; x < XM; ++x)
#pragma unroll
    for (int y = 0; y < XN; ++y) acc[x][y] = {0.f, 0.f, 0.f, 0.f};
  for (int64_t k0 = kbeg; k0 < kend; k0 += KS) {
    __syncthreads();  // the previous step's fragment reads are done
    // (a step that reaches past the diagonal: pairs not visible are zeroed)
    if (g.causal_on && m0 + RM - 1 > k0 + g.causal_off)
      stage_causal<TA, RM>(fa, tid, m0, k0, g.causal_off, wa);
    stage_store<TA, RM>(As, fa, tid, wa);
    stage_store<TB, RN>(Bs, fb, tid, wb);
    __syncthreads();
    if (k0 + KS < kend) {
      stage_load<TA, RM>(g.A.p, abase, g.A.si, g.A.sj, g.M, m0, k0 + KS, kend, fa, tid, wa);
      stage_load<TB, RN>(g.B.p, bbase, g.B.sj, g.B.si, g.N, n0, k0 + KS, kend, fb, tid, wb);
    }
#pragma unroll
    for (int s = 0; s < KS / 32; ++s) {
      bf16x8 af[XM], bfr[XN];
#pragma unroll
      for (int x = 0; x < XM; ++x) af[x] = frag<RM>(As, fa, RM / 2 * wm + 16 * x, s, g4, n16);
#pragma unroll
      for (int y = 0; y < XN; ++y) bfr[y] = frag<RN>(Bs, fb, RN / 2 * wn + 16 * y, s, g4, n16);
#pragma unroll
      for (int x = 0; x < XM; ++x)
#pragma unroll
        for (int y = 0; y < XN; ++y)
          acc[x][y] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[x], bfr[y], acc[x][y], 0, 0, 0);
    }
  }
  // lane (g4, n16), register e of block (x, y): row RM / 2 wm + 16 x + 4 g4 + e,
  // column RN / 2 wn + 16 y + n16
  const int64_t cbase = zq * g.c1 + zr * g.c2;
#pragma unroll
  for (int y = 0; y < XN; ++y) {
    const int64_t n = n0 + RN / 2 * wn + 16 * y + n16;
    if (n >= g.N) continue;
#pragma unroll
    for (int x = 0; x < XM; ++x)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int64_t m = m0 + RM / 2 * wm + 16 * x + 4 * g4 + e;
        if (m >= g.M) continue;
        float* c = g.C + cbase + m * g.cm + n * g.cn;
        const float v = g.alpha * acc[x][y][e];
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

// Staging flags of an operand read as X(row, k) = p[... + row sr + k sk] (see stage_load).
int stage_flags(const StridedOperand& o, int64_t sr, int64_t sk, int dtype) {
  const uintptr_t p = (uintptr_t)o.p;
  const int64_t q = dtype == 0 ? 4 : 8;  // elements per aligned 16-byte load
  if (sk == 1) {  // 8 consecutive k: offsets row sr + k (k % 8 == 0)
    const bool vec = p % 16 == 0 && sr % q == 0 && o.s1 % q == 0 && o.s2 % q == 0;
    return vec ? ST_VEC : 0;
  }
  if (sr == 1) {  // 8 consecutive rows: offsets row + k sk (row % 8 == 0)
    const bool vec = p % 16 == 0 && sk % q == 0 && o.s1 % q == 0 && o.s2 % q == 0;
    return ST_ROWS | (vec ? ST_VEC : 0);
  }
  return 0;  // neither axis contiguous: element loads
}

template <int RM, int RN, int AR, int BR>
void launch_mfma_layout(const StridedGemm& g, dim3 grid, int k, int fa, int fb, hipStream_t s) {
  if (g.a_dtype == 0 && g.b_dtype == 0)
    hipLaunchKernelGGL((gemm_strided_mfma_kernel<float, float, RM, RN, AR, BR>), grid, dim3(256), 0,
                       s, g, k, fa, fb);
  else if (g.a_dtype == 0 && g.b_dtype == 1)
    hipLaunchKernelGGL((gemm_strided_mfma_kernel<float, uint16_t, RM, RN, AR, BR>), grid, dim3(256),
                       0, s, g, k, fa, fb);
  else if (g.a_dtype == 1 && g.b_dtype == 0)
    hipLaunchKernelGGL((gemm_strided_mfma_kernel<uint16_t, float, RM, RN, AR, BR>), grid, dim3(256),
                       0, s, g, k, fa, fb);
  else
    hipLaunchKernelGGL((gemm_strided_mfma_kernel<uint16_t, uint16_t, RM, RN, AR, BR>), grid,
                       dim3(256), 0, s, g, k, fa, fb);
}

template <int RM, int RN>
void launch_mfma_variant(const StridedGemm& g, dim3 grid, int k, int fa, int fb, hipStream_t s) {
  const bool ar = fa & ST_ROWS, br = fb & ST_ROWS;
  if (ar && br) launch_mfma_layout<RM, RN, 1, 1>(g, grid, k, fa, fb, s);
  else if (ar) launch_mfma_layout<RM, RN, 1, 0>(g, grid, k, fa, fb, s);
  else if (br) launch_mfma_layout<RM, RN, 0, 1>(g, grid, k, fa, fb, s);
  else launch_mfma_layout<RM, RN, 0, 0>(g, grid, k, fa, fb, s);
}

hipError_t launch_gemm_strided(const StridedGemm& g, hipStream_t s) {
  if (g.M <= 0 || g.N <= 0 || g.batch <= 0) return hipSuccess;
  if (g.zdiv <= 0 || g.batch > 65535) return hipErrorInvalidValue;
  // matrix cores: 128 x 128 tiles when both output sides reach 128, 128 x 64
  // when only the rows do (the key-major products dk, dv of a head: N = d)
  const bool big = g.bf16_mfma && g.M >= 128 && g.N >= 128;
  const bool tall = g.bf16_mfma && !big && g.M >= 128;
  const int64_t tm = big || tall ? 128 : 64, tn = big ? 128 : 64;
  if ((g.N + tn - 1) / tn > 0x7fffffff || (g.M + tm - 1) / tm > 65535) return hipErrorInvalidValue;
  // Split K when the tiles alone leave the GPU short of workgroups (about one per
  // CU for the matrix-core kernel, four for the fp32 one; measured), each split at
  // least 256 deep; the splits add atomically.
  const int64_t wg_target = g.bf16_mfma ? 256 : 1024;
  const int64_t tiles = ((g.N + tn - 1) / tn) * ((g.M + tm - 1) / tm) * g.batch;
  int64_t ks = (wg_target + tiles - 1) / tiles;
  if (ks > g.K / 256) ks = g.K / 256;
  if (ks > 16) ks = 16;
  if (ks < 1 || g.batch * ks > 65535) ks = 1;
  if (ks > 1 && !g.accumulate) {
    hipLaunchKernelGGL(zero_c_kernel, dim3(1024), dim3(256), 0, s, g);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const dim3 grid((unsigned)((g.N + tn - 1) / tn), (unsigned)((g.M + tm - 1) / tm),
                  (unsigned)(g.batch * ks));
  const int k = (int)ks;
  if (g.bf16_mfma) {
    const int fa = stage_flags(g.A, g.A.si, g.A.sj, g.a_dtype);
    const int fb = stage_flags(g.B, g.B.sj, g.B.si, g.b_dtype);
    if (big)
      launch_mfma_variant<128, 128>(g, grid, k, fa, fb, s);
    else if (tall)
      launch_mfma_variant<128, 64>(g, grid, k, fa, fb, s);
    else
      launch_mfma_variant<64, 64>(g, grid, k, fa, fb, s);
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
