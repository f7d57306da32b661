// Element kernels of the layer step's backward pass (Transformer-XL section 3.3,
// the N-layer procedure: h_out = LayerNorm(a W_o^T + h_in) with the biased
// variance; section 3.2: the memory's gradient is stopped).  The products of
// the backward run through the strided GEMM; these kernels cover the
// LayerNorm backward, the copies and the gather of [memory ; h_in].
#include "txl_internal.h"

#include <algorithm>
#include <type_traits>

namespace txl {
namespace {

// two floats -> bf16 pair (low half = lo), round to nearest even
__device__ inline uint32_t pack2_bf16(float lo, float hi) {
  return (uint32_t)f32_to_bf16(lo) | ((uint32_t)f32_to_bf16(hi) << 16);
}

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
// LayerNorm backward with the row in registers, for D = 256 NJ: one wave per row,
// lane l holding columns 256 j + 4 l .. + 3 (16-byte loads), the four row sums
// as DPP wave reductions, the next row of the wave loaded before this one is
// reduced.  dy fp32 (and, when dyb is set, as bf16 rows of pitch ldyb).  Each
// workgroup adds its rows' dgamma and dbeta terms over its four waves and writes
// them to part[block][0 / 1][D]; ln_part_sum_kernel adds the blocks.
template <typename E, int NJ>
__global__ __launch_bounds__(256) void ln_bwd_fused_kernel(const float* __restrict__ y,
                                                           const void* __restrict__ gamma,
                                                           const void* __restrict__ dh_out,
                                                           int M, float eps, float* __restrict__ dy,
                                                           uint16_t* __restrict__ dyb, int64_t ldyb,
                                                           float* __restrict__ part) {
  __shared__ float red[4][2][256 * NJ];
  constexpr int D = 256 * NJ;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  float gm[NJ][4], dg[NJ][4], db[NJ][4];
#pragma unroll
  for (int j = 0; j < NJ; ++j)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      gm[j][e] = ldE<E>(gamma, 256 * j + 4 * lane + e);
      dg[j][e] = 0.f;
      db[j][e] = 0.f;
    }
  auto load = [&](int m, float (&yv)[NJ][4], float (&hv)[NJ][4]) {
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int64_t o = (int64_t)m * D + 256 * j + 4 * lane;
      const float4 a = *(const float4*)(y + o);
      yv[j][0] = a.x; yv[j][1] = a.y; yv[j][2] = a.z; yv[j][3] = a.w;
      if constexpr (std::is_same<E, float>::value) {
        const float4 b = *(const float4*)((const float*)dh_out + o);
        hv[j][0] = b.x; hv[j][1] = b.y; hv[j][2] = b.z; hv[j][3] = b.w;
      } else {
        const uint2 b = *(const uint2*)((const uint16_t*)dh_out + o);
        hv[j][0] = bf16_to_f32((uint16_t)(b.x & 0xffffu)); hv[j][1] = bf16_to_f32((uint16_t)(b.x >> 16));
        hv[j][2] = bf16_to_f32((uint16_t)(b.y & 0xffffu)); hv[j][3] = bf16_to_f32((uint16_t)(b.y >> 16));
      }
    }
  };
  const int stride = gridDim.x * 4;
  int m = blockIdx.x * 4 + wave;
  float yv[NJ][4], hv[NJ][4], yn[NJ][4], hn[NJ][4];
  load(m < M ? m : M - 1, yv, hv);
  for (; m < M; m += stride) {
    const int mn = m + stride < M ? m + stride : m;
    load(mn, yn, hn);
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) s += yv[j][e];
    const float mu = wave_allsum(s) / (float)D;
    float v = 0.f;
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) v += (yv[j][e] - mu) * (yv[j][e] - mu);
    const float rstd = rsqrtf(wave_allsum(v) / (float)D + eps);
    float s1 = 0.f, s2 = 0.f;
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float yh = (yv[j][e] - mu) * rstd;
        const float g = hv[j][e] * gm[j][e];
        s1 += g;
        s2 += g * yh;
        dg[j][e] += hv[j][e] * yh;
        db[j][e] += hv[j][e];
        yv[j][e] = yh;  // (y hat from here on)
      }
    const float m1 = wave_allsum(s1) / (float)D, m2 = wave_allsum(s2) / (float)D;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      float o[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) o[e] = (hv[j][e] * gm[j][e] - m1 - yv[j][e] * m2) * rstd;
      const int64_t c = 256 * j + 4 * lane;
      *(float4*)(dy + (int64_t)m * D + c) = make_float4(o[0], o[1], o[2], o[3]);
      if (dyb)
        *(uint2*)(dyb + (int64_t)m * ldyb + c) = make_uint2(pack2_bf16(o[0], o[1]), pack2_bf16(o[2], o[3]));
    }
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        yv[j][e] = yn[j][e];
        hv[j][e] = hn[j][e];
      }
  }
#pragma unroll
  for (int j = 0; j < NJ; ++j)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      red[wave][0][256 * j + 4 * lane + e] = dg[j][e];
      red[wave][1][256 * j + 4 * lane + e] = db[j][e];
    }
  __syncthreads();
  for (int c = tid; c < 2 * D; c += 256) {
    const int w2 = c / D, cc = c - w2 * D;
    part[(int64_t)blockIdx.x * 2 * D + c] = red[0][w2][cc] + red[1][w2][cc] + red[2][w2][cc] +
                                            red[3][w2][cc];
  }
}

// dgamma[c] = sum_b part[b][0][c], dbeta[c] = sum_b part[b][1][c]: a workgroup
// takes 16 of the 2 D columns; thread (g, c) adds blocks 16 g' .. of its group g
// (all 16 loads issued at once, indexes clamped), then the 16 groups add in LDS.
__global__ __launch_bounds__(256) void ln_part_sum_kernel(const float* __restrict__ part, int blocks,
                                                          int D, float* __restrict__ dgamma,
                                                          float* __restrict__ dbeta) {
  __shared__ float red[16][17];
  const int tid = threadIdx.x, cl = tid & 15, pg = tid >> 4;
  const int c0 = blockIdx.x * 16 + cl;
  const int c = c0 < 2 * D ? c0 : 2 * D - 1;
  const int per = (blocks + 15) / 16;  // <= 16 (blocks <= LN_BWD_BLOCKS)
  float v[16];
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const int b = pg * per + k;
    const int bb = b < blocks ? b : blocks - 1;
    v[k] = part[(int64_t)bb * 2 * D + c];
  }
  float a = 0.f;
#pragma unroll
  for (int k = 0; k < 16; ++k) a += (k < per && pg * per + k < blocks) ? v[k] : 0.f;
  red[pg][cl] = a;
  __syncthreads();
  if (pg == 0 && c0 < 2 * D) {
    float t = 0.f;
#pragma unroll
    for (int g = 0; g < 16; ++g) t += red[g][cl];
    if (c0 < D) dgamma[c0] = t;
    else dbeta[c0 - D] = t;
  }
}

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

// Transposing pack to bf16: dst[r][k] = bf16(src[r + k * sk]) for r < R, k < K,
// and 0 for K <= k < Kp (row pitch Kp): a 64 x 64 block per workgroup passes
// through LDS, read along r (contiguous in src) and written along k.  Every
// load is issued (indexes past the ends are clamped, their values zeroed).
// One 64 x 64 tile of destination rows r0.., columns c0.. of a pack job per
// block: dst[r][c] = source element (r, c) converted to bf16 for c < C, zero for
// C <= c < Cpad.  A transposed job reads element (r, c) at src[c sk + r] and
// passes the tile through LDS; a rows job reads src[(r / rpb) sb + (r % rpb) ld
// + c] directly.  Jobs marked vec (every row and pitch 16-byte aligned, R, C
// and Cpad multiples of 8) move 16 bytes per access, both in and out; the
// others go element by element.  Out-of-range addresses are clamped and their
// values replaced, so every load of a tile is issued unconditionally.
__device__ inline float pk_ld(const void* p, int64_t i, int dtype) {
  return dtype ? bf16_to_f32(((const uint16_t*)p)[i]) : ((const float*)p)[i];
}
// first byte of source row c of a transposed job (0 <= c < C)
__device__ inline const char* pk_row(const PackJob& J, int64_t c) {
  const int64_t es = J.dtype ? 2 : 4;
  if (!J.gather) return (const char*)J.src + c * J.sk * es;
  // (32-bit: launch_pack checks that the context's rows fit)
  const uint32_t cc = (uint32_t)c, per = (uint32_t)J.per, b = cc / per, t = cc - b * per;
  if (t < (uint32_t)J.len) {
    uint32_t slot = (uint32_t)J.start + t;
    slot = slot >= (uint32_t)J.cap ? slot - (uint32_t)J.cap : slot;
    return (const char*)J.src + ((int64_t)b * J.cap + slot) * J.sk * es;
  }
  return (const char*)J.h + ((int64_t)b * J.h_rows + (t - (uint32_t)J.len)) * J.sk * es;
}

__global__ __launch_bounds__(256) void pack_kernel(PackJobs jobs) {
  __shared__ float t[64][65];
  int jn = 0;
  while (jn + 1 < jobs.n && (int64_t)blockIdx.x >= jobs.j[jn].tile_end) ++jn;
  const PackJob& J = jobs.j[jn];
  const int64_t tile = (int64_t)blockIdx.x - (jn ? jobs.j[jn - 1].tile_end : 0);
  const int64_t ntc = (J.Cpad + 63) / 64;
  const int64_t r0 = (tile / ntc) * 64, c0 = (tile % ntc) * 64;
  const int tid = threadIdx.x;
  if (J.vec) {
    if (J.trans) {
      // source rows are c: 64 of them, 64 r each, into t[c - c0][r - r0]
      if (J.dtype == 0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int cl = tid / 16 + 16 * i, rl = 4 * (tid % 16);
          const int64_t c = c0 + cl, r = r0 + rl;
          const bool ok = c < J.C && r < J.R;
          const float4 v = *(const float4*)((const float*)pk_row(J, ok ? c : 0) + (ok ? r : 0));
          t[cl][rl] = ok ? v.x : 0.f; t[cl][rl + 1] = ok ? v.y : 0.f;
          t[cl][rl + 2] = ok ? v.z : 0.f; t[cl][rl + 3] = ok ? v.w : 0.f;
        }
      } else {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const int cl = tid / 8 + 32 * i, rl = 8 * (tid % 8);
          const int64_t c = c0 + cl, r = r0 + rl;
          const bool ok = c < J.C && r < J.R;
          const uint4 v = *(const uint4*)((const uint16_t*)pk_row(J, ok ? c : 0) + (ok ? r : 0));
          const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            t[cl][rl + 2 * e] = ok ? bf16_to_f32((uint16_t)(w[e] & 0xffffu)) : 0.f;
            t[cl][rl + 2 * e + 1] = ok ? bf16_to_f32((uint16_t)(w[e] >> 16)) : 0.f;
          }
        }
      }
      __syncthreads();
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int rl = tid / 8 + 32 * i, cl = 8 * (tid % 8);
        const int64_t r = r0 + rl, c = c0 + cl;
        if (r >= J.R || c >= J.Cpad) continue;
        uint32_t w[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = pack2_bf16(t[cl + 2 * e][rl], t[cl + 2 * e + 1][rl]);
        *(uint4*)(J.dst + r * J.ldd + c) = make_uint4(w[0], w[1], w[2], w[3]);
      }
      if (J.dst2) {  // the same tile in rows form: 8 r of one source row c per thread
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const int cl = tid / 8 + 32 * i, rl = 8 * (tid % 8);
          const int64_t c = c0 + cl, r = r0 + rl;
          if (c >= J.C || r >= J.R) continue;
          const int64_t b = c / J.per2, tt = c - b * J.per2;
          if (tt < J.skip2) continue;
          uint32_t w[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) w[e] = pack2_bf16(t[cl][rl + 2 * e], t[cl][rl + 2 * e + 1]);
          *(uint4*)(J.dst2 + (b * (J.per2 - J.skip2) + tt - J.skip2) * J.ldd2 + r) =
              make_uint4(w[0], w[1], w[2], w[3]);
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int rl = tid / 8 + 32 * i, cl = 8 * (tid % 8);
        const int64_t r = r0 + rl, c = c0 + cl;
        if (r >= J.R || c >= J.Cpad) continue;
        const bool ok = c < J.C;
        const int64_t off = (r / J.rpb) * J.sb + (r % J.rpb) * J.ld + (ok ? c : 0);
        uint4 o;
        if (J.dtype == 0) {
          const float4 a = *(const float4*)((const float*)J.src + off);
          const float4 b = *(const float4*)((const float*)J.src + off + 4);
          o = make_uint4(pack2_bf16(a.x, a.y), pack2_bf16(a.z, a.w), pack2_bf16(b.x, b.y),
                         pack2_bf16(b.z, b.w));
        } else {
          o = *(const uint4*)((const uint16_t*)J.src + off);
        }
        if (!ok) o = make_uint4(0u, 0u, 0u, 0u);
        *(uint4*)(J.dst + r * J.ldd + c) = o;
      }
    }
    return;
  }
  // element by element
  if (J.trans) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int cl = tid / 64 + 4 * i, rl = tid % 64;
      const int64_t c = c0 + cl, r = r0 + rl;
      const bool ok = c < J.C && r < J.R;
      const float v = pk_ld(pk_row(J, ok ? c : 0), ok ? r : 0, J.dtype);
      t[cl][rl] = ok ? v : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int rl = tid / 64 + 4 * i, cl = tid % 64;
      const int64_t r = r0 + rl, c = c0 + cl;
      if (r < J.R && c < J.Cpad) J.dst[r * J.ldd + c] = f32_to_bf16(t[cl][rl]);
    }
    if (J.dst2) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int cl = tid / 64 + 4 * i, rl = tid % 64;
        const int64_t c = c0 + cl, r = r0 + rl;
        if (c >= J.C || r >= J.R) continue;
        const int64_t b = c / J.per2, tt = c - b * J.per2;
        if (tt >= J.skip2)
          J.dst2[(b * (J.per2 - J.skip2) + tt - J.skip2) * J.ldd2 + r] = f32_to_bf16(t[cl][rl]);
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int rl = tid / 64 + 4 * i, cl = tid % 64;
      const int64_t r = r0 + rl, c = c0 + cl;
      if (r >= J.R || c >= J.Cpad) continue;
      const bool ok = c < J.C;
      const float v = pk_ld(J.src, (r / J.rpb) * J.sb + (r % J.rpb) * J.ld + (ok ? c : 0), J.dtype);
      J.dst[r * J.ldd + c] = ok ? f32_to_bf16(v) : (uint16_t)0;
    }
  }
}

// dst[i] = sum over s < parts of src[s n + i] for each job, four elements per
// thread (16-byte loads when the job's n and pointers allow), every part's load
// issued before the first add (indexes of parts past the job's clamped, their
// values dropped).
constexpr int SJ_MAX = 8;
struct SumJobsK {
  const float* src[SJ_MAX];
  float* dst[SJ_MAX];
  int64_t n[SJ_MAX];
  int64_t item_end[SJ_MAX];  // inclusive prefix sums of (n + 3) / 4
  const void* resid[SJ_MAX];  // optional residual added to the sum
  int parts[SJ_MAX], vec[SJ_MAX], rbf[SJ_MAX];
  int nj;
};

__device__ inline float sum_resid(const SumJobsK& J, int j, int64_t i) {
  if (!J.resid[j]) return 0.f;
  return J.rbf[j] ? bf16_to_f32(((const uint16_t*)J.resid[j])[i]) : ((const float*)J.resid[j])[i];
}

__global__ __launch_bounds__(256) void sum_partials_kernel(SumJobsK J) {
  const int64_t items = J.item_end[J.nj - 1];
  for (int64_t it = (int64_t)blockIdx.x * 256 + threadIdx.x; it < items;
       it += (int64_t)gridDim.x * 256) {
    int j = 0;
    while (j + 1 < J.nj && it >= J.item_end[j]) ++j;
    const int64_t i = 4 * (it - (j ? J.item_end[j - 1] : 0)), n = J.n[j];
    const float* src = J.src[j];
    const int parts = J.parts[j];
    if (J.vec[j]) {
      float4 v[16];
#pragma unroll
      for (int p = 0; p < 16; ++p) v[p] = *(const float4*)(src + (p < parts ? p : parts - 1) * n + i);
      float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
      for (int p = 0; p < 16; ++p)
        if (p < parts) {
          acc.x += v[p].x; acc.y += v[p].y; acc.z += v[p].z; acc.w += v[p].w;
        }
      if (J.resid[j]) {
        acc.x += sum_resid(J, j, i); acc.y += sum_resid(J, j, i + 1);
        acc.z += sum_resid(J, j, i + 2); acc.w += sum_resid(J, j, i + 3);
      }
      *(float4*)(J.dst[j] + i) = acc;
    } else {
      for (int e = 0; e < 4 && i + e < n; ++e) {
        float a = 0.f;
        for (int p = 0; p < parts; ++p) a += src[p * n + i + e];
        J.dst[j][i + e] = a + sum_resid(J, j, i + e);
      }
    }
  }
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

bool ln_bwd_fused_ok(int64_t M, int64_t D) {
  return D % 256 == 0 && D >= 256 && D <= 1024 && M >= 1 && M * D < 0x7fffffffLL;
}

size_t ln_bwd_part_bytes(int64_t M, int64_t D) {
  const int64_t blocks = std::min<int64_t>((M + 3) / 4, LN_BWD_BLOCKS);
  return (size_t)(blocks * 2 * D) * sizeof(float);
}

hipError_t launch_ln_bwd_fused(int dtype, const float* y, const void* gamma, const void* dh_out,
                               int64_t M, int64_t D, float eps, float* dy, uint16_t* dyb,
                               int64_t ldyb, float* part, float* dgamma, float* dbeta,
                               hipStream_t s) {
  if (!ln_bwd_fused_ok(M, D) || !part || (dyb && (ldyb < D || ldyb % 4 || (uintptr_t)dyb % 8)) ||
      (uintptr_t)y % 16 || (uintptr_t)dy % 16 || (uintptr_t)dh_out % 16)
    return hipErrorInvalidValue;
  const int blocks = (int)std::min<int64_t>((M + 3) / 4, LN_BWD_BLOCKS);
  const int nj = (int)(D / 256);
  auto go = [&](auto tag, auto njc) {
    using E = decltype(tag);
    constexpr int NJ = decltype(njc)::value;
    hipLaunchKernelGGL((ln_bwd_fused_kernel<E, NJ>), dim3((unsigned)blocks), dim3(256), 0, s, y,
                       gamma, dh_out, (int)M, eps, dy, dyb, ldyb, part);
  };
  if (dtype == 1) {
    if (nj == 1) go(uint16_t{}, std::integral_constant<int, 1>{});
    else if (nj == 2) go(uint16_t{}, std::integral_constant<int, 2>{});
    else if (nj == 3) go(uint16_t{}, std::integral_constant<int, 3>{});
    else go(uint16_t{}, std::integral_constant<int, 4>{});
  } else {
    if (nj == 1) go(float{}, std::integral_constant<int, 1>{});
    else if (nj == 2) go(float{}, std::integral_constant<int, 2>{});
    else if (nj == 3) go(float{}, std::integral_constant<int, 3>{});
    else go(float{}, std::integral_constant<int, 4>{});
  }
  static_assert(LN_BWD_BLOCKS <= 256, "ln_part_sum_kernel adds at most 16 x 16 blocks");
  hipLaunchKernelGGL(ln_part_sum_kernel, dim3((unsigned)((2 * D + 15) / 16)), dim3(256), 0, s,
                     part, blocks, (int)D, dgamma, dbeta);
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

PackJob pack_rows(const void* src, int dtype, int64_t R, int64_t C, int64_t Cpad, int64_t rpb,
                  int64_t sb, int64_t ld, uint16_t* dst, int64_t ldd) {
  PackJob j{};
  j.src = src; j.dtype = dtype; j.trans = 0;
  j.R = R; j.C = C; j.Cpad = Cpad; j.rpb = rpb; j.sb = sb; j.ld = ld;
  j.dst = dst; j.ldd = ldd;
  return j;
}

PackJob pack_trans(const void* src, int dtype, int64_t R, int64_t C, int64_t Cpad, int64_t sk,
                   uint16_t* dst, int64_t ldd) {
  PackJob j{};
  j.src = src; j.dtype = dtype; j.trans = 1;
  j.R = R; j.C = C; j.Cpad = Cpad; j.rpb = 1; j.sk = sk;
  j.dst = dst; j.ldd = ldd;
  return j;
}

PackJob pack_trans_ctx(const void* ring, int64_t cap, int64_t start, int64_t len, const void* h,
                       int64_t h_rows, int64_t B, int dtype, int64_t R, int64_t Cpad, int64_t sk,
                       uint16_t* dst, int64_t ldd) {
  PackJob j = pack_trans(ring, dtype, R, B * (len + h_rows), Cpad, sk, dst, ldd);
  j.gather = 1;
  j.h = h;
  j.per = len + h_rows;
  j.len = len;
  j.cap = cap;
  j.start = start;
  j.h_rows = h_rows;
  return j;
}

hipError_t launch_pack(const PackJob* js, int n, hipStream_t s) {
  for (int base = 0; base < n; base += PJ_MAX) {
    PackJobs b{};
    int64_t tiles = 0;
    for (int x = 0; x < PJ_MAX && base + x < n; ++x) {
      PackJob j = js[base + x];
      if (j.R < 0 || j.C < 0 || j.Cpad < j.C || j.ldd < j.Cpad || j.rpb < 1 ||
          (j.dtype != 0 && j.dtype != 1) || (j.C > 0 && j.R > 0 && !j.src))
        return hipErrorInvalidValue;
      const int64_t es = j.dtype ? 2 : 4, al = 16 / es;  // elements per 16 bytes
      if (j.gather && (!j.trans || j.per < 1 || j.len < 0 || j.len > j.cap || j.start < 0 ||
                       j.start >= (j.cap > 0 ? j.cap : 1) || (j.per > j.len && !j.h) ||
                       j.C > 0x7fffffffLL || j.cap > 0x7fffffffLL))
        return hipErrorInvalidValue;
      const uintptr_t src = (uintptr_t)j.src | (j.gather ? (uintptr_t)j.h : 0), dst = (uintptr_t)j.dst;
      bool vec = j.Cpad % 8 == 0 && j.ldd % 8 == 0 && dst % 16 == 0 && src % 16 == 0;
      if (j.dst2 && (!j.trans || j.per2 < 1 || j.skip2 < 0 || j.skip2 >= j.per2 || j.ldd2 < j.R))
        return hipErrorInvalidValue;
      if (j.trans)
        vec = vec && j.R % 8 == 0 && j.sk % al == 0 &&
              (!j.dst2 || ((uintptr_t)j.dst2 % 16 == 0 && j.ldd2 % 8 == 0));
      else
        vec = vec && j.C % 8 == 0 && j.ld % al == 0 && j.sb % al == 0;
      j.vec = vec ? 1 : 0;
      tiles += ((j.R + 63) / 64) * ((j.Cpad + 63) / 64);
      if (tiles > 0x7fffffffLL) return hipErrorInvalidValue;
      j.tile_end = tiles;
      b.j[x] = j;
      b.n = x + 1;
    }
    if (tiles == 0) continue;
    hipLaunchKernelGGL(pack_kernel, dim3((unsigned)tiles), dim3(256), 0, s, b);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_sum_partials_multi(const SumJob* jobs, int n, hipStream_t s) {
  if (n < 1 || n > SJ_MAX) return hipErrorInvalidValue;
  SumJobsK J{};
  int64_t items = 0;
  int nj = 0;
  for (int x = 0; x < n; ++x) {
    const SumJob& b = jobs[x];
    if (b.parts < 1 || b.parts > 16 || b.n < 0 || (b.n > 0 && (!b.src || !b.dst)))
      return hipErrorInvalidValue;
    if (b.n == 0) continue;
    J.src[nj] = b.src;
    J.dst[nj] = b.dst;
    J.n[nj] = b.n;
    J.parts[nj] = b.parts;
    J.resid[nj] = b.resid;
    J.rbf[nj] = b.resid_bf16 ? 1 : 0;
    J.vec[nj] = b.n % 4 == 0 && (uintptr_t)b.src % 16 == 0 && (uintptr_t)b.dst % 16 == 0;
    items += (b.n + 3) / 4;
    J.item_end[nj++] = items;
  }
  if (nj == 0) return hipSuccess;
  J.nj = nj;
  const unsigned grid = (unsigned)std::min<int64_t>((items + 255) / 256, 65536);
  hipLaunchKernelGGL(sum_partials_kernel, dim3(grid), dim3(256), 0, s, J);
  return hipGetLastError();
}

hipError_t launch_sum_partials(const float* src, int parts, int64_t n, float* dst, hipStream_t s) {
  const SumJob j = {src, parts, n, dst, nullptr, 0};
  return launch_sum_partials_multi(&j, 1, s);
}

}  // namespace txl
