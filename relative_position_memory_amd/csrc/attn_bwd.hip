// Backward pass of the relative-position attention (Transformer-XL, section
// 3.3: score with content and position terms and the global biases u and v;
// Appendix B: key j of query i at distance mem_len + i - j), d <= 64, fp32 math.
//
//   P = softmax(s),  dP_ij = dO_i . v_j,  dS_ij = P_ij (dP_ij - sum_j' P_ij' dP_ij')
//   dq_i = scale sum_j dS_ij (k_j + r_{mem_len+i-j}),  du, dv: the two parts summed
//   dv_j = sum_i P_ij dO_i,  dk_j = scale sum_i dS_ij (q_i + u)
//   dr_p = scale sum over pairs at distance p of dS_ij (q_i + v)
//
// attn_bwd_rows_kernel: one workgroup per 64 queries of one (batch, head).  A
// first walk over the key tiles keeps the running maximum, sum of
// exponentials and sum of exponentials times dP per query (an online softmax, so
// the forward's output is not needed); a second walk forms P and dS, writes them
// to scratch and accumulates dq.  The key-side gradients are then products over
// the queries (strided GEMMs), and dr sums dS along the diagonals
// (attn_bwd_dr_kernel).
#include "txl_internal.h"

namespace txl {
namespace {

constexpr int BQ = 64, BK = 64, DP = 64, LD = DP + 1;

struct BwdSmem {
  float QC[BQ][LD];          // q + u (this block's queries)
  float QP[BQ][LD];          // q + v
  float G[BQ][LD];           // dO
  float K[BK][LD];           // key tile
  float V[BK][LD];           // value tile
  float RW[BQ + BK][LD];     // r rows of the tile pair's distances, local row w <-> ii - jj + 63
  float DS[BQ][BK + 1];      // dS of the tile pair
};

template <typename E>
__device__ inline float ldE(const void* p, int64_t off) {
  return Elt<E>::load((const E*)p + off);
}

template <typename E>
__global__ __launch_bounds__(256) void attn_bwd_rows_kernel(AttnBwdArgs a) {
  extern __shared__ __align__(16) char smem_raw[];
  BwdSmem& sm = *(BwdSmem*)smem_raw;
  const int tid = threadIdx.x;
  const int H = (int)a.H, L = (int)a.L, len = (int)a.mem_len, d = (int)a.d;
  const int T = len + L;
  const int z = blockIdx.y, b = z / H, h = z % H;
  const int i0 = blockIdx.x * BQ;
  const int ti = tid / 16, tj = tid % 16;  // pairs (4 ti + x, 4 tj + y)
  const int imax = i0 + BQ - 1 < L - 1 ? i0 + BQ - 1 : L - 1;
  const int nkb = (len + imax) / BK + 1;  // key tiles up to the last query's last key
  const int64_t prow0 = ((int64_t)z * L) * T;  // row (b, h, 0) of P and dS

  // queries, dO, and the scratch copies of q + u, q + v
  for (int e = tid; e < BQ * DP; e += 256) {
    const int ii = e / DP, c = e % DP, i = i0 + ii;
    float qv = 0.f, g = 0.f, qc = 0.f, qp = 0.f;
    if (i < L && c < d) {
      qv = ldE<E>(a.q, (int64_t)b * a.q_sb + (int64_t)i * a.q_st + (int64_t)h * a.q_sh + c);
      const int64_t go = (int64_t)b * a.do_sb + (int64_t)i * a.do_st + (int64_t)h * a.do_sh + c;
      g = a.dout_f32 ? ((const float*)a.dout)[go] : ldE<E>(a.dout, go);
      qc = qv + ldE<E>(a.u, (int64_t)h * d + c);
      qp = qv + ldE<E>(a.vb, (int64_t)h * d + c);
    }
    sm.QC[ii][c] = qc;
    sm.QP[ii][c] = qp;
    sm.G[ii][c] = g;
    if (i < L) {
      a.qc[((int64_t)z * L + i) * DP + c] = qc;
      a.qp[((int64_t)z * L + i) * DP + c] = qp;
    }
  }

  auto load_tiles = [&](int j0) {
    for (int e = tid; e < BK * DP; e += 256) {
      const int jj = e / DP, c = e % DP, j = j0 + jj;
      float kv = 0.f, vv = 0.f;
      if (j < T && c < d) {
        const int64_t off = (int64_t)b * a.kv_sb + (int64_t)j * a.kv_st + (int64_t)h * a.kv_sh + c;
        kv = ldE<E>(a.k, off);
        vv = ldE<E>(a.v, off);
      }
      sm.K[jj][c] = kv;
      sm.V[jj][c] = vv;
    }
    // distance of local row w: len + i0 - j0 - 63 + w
    const int dbase = len + i0 - j0 - (BK - 1);
    for (int e = tid; e < (BQ + BK) * DP; e += 256) {
      const int w = e / DP, c = e % DP, dist = dbase + w;
      float rv = 0.f;
      if (dist >= 0 && dist < T && c < d)
        rv = ldE<E>(a.r, (int64_t)dist * a.r_sp + (int64_t)h * a.r_sh + c);
      sm.RW[w][c] = rv;
    }
  };
  // scores (scaled) and dP of this thread's 16 pairs; masked pairs: -inf and 0
  auto pair_terms = [&](int j0, float (&s)[4][4], float (&dp)[4][4]) {
#pragma unroll
    for (int x = 0; x < 4; ++x)
#pragma unroll
      for (int y = 0; y < 4; ++y) s[x][y] = dp[x][y] = 0.f;
    for (int c = 0; c < DP; ++c) {
      float qc[4], qp[4], g[4], kk[4], vv[4], rr[7];
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        qc[x] = sm.QC[4 * ti + x][c];
        qp[x] = sm.QP[4 * ti + x][c];
        g[x] = sm.G[4 * ti + x][c];
        kk[x] = sm.K[4 * tj + x][c];
        vv[x] = sm.V[4 * tj + x][c];
      }
#pragma unroll
      for (int w = 0; w < 7; ++w) rr[w] = sm.RW[4 * ti - 4 * tj + w + (BK - 1) - 3][c];
#pragma unroll
      for (int x = 0; x < 4; ++x)
#pragma unroll
        for (int y = 0; y < 4; ++y) {
          s[x][y] += qc[x] * kk[y] + qp[x] * rr[x - y + 3];
          dp[x][y] += g[x] * vv[y];
        }
    }
#pragma unroll
    for (int x = 0; x < 4; ++x)
#pragma unroll
      for (int y = 0; y < 4; ++y) {
        const int i = i0 + 4 * ti + x, j = j0 + 4 * tj + y;
        const bool ok = i < L && j < T && j <= len + i;
        s[x][y] = ok ? s[x][y] * a.scale : -INFINITY;
        dp[x][y] = ok ? dp[x][y] : 0.f;
      }
  };
  // sum / max over the 16 threads of a query row (consecutive lanes)
  auto row_sum = [](float v) {
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) v += __shfl_xor(v, o, 16);
    return v;
  };
  auto row_max = [](float v) {
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) v = fmaxf(v, __shfl_xor(v, o, 16));
    return v;
  };

  // ---- walk 1: running max m, sum l of exp(s - m), and sum of exp(s - m) dP -------
  float m[4], l[4], dn[4];
#pragma unroll
  for (int x = 0; x < 4; ++x) {
    m[x] = -INFINITY;
    l[x] = dn[x] = 0.f;
  }
  for (int kb = 0; kb < nkb; ++kb) {
    __syncthreads();  // previous tiles retired (and the query tiles written)
    load_tiles(kb * BK);
    __syncthreads();
    float s[4][4], dp[4][4];
    pair_terms(kb * BK, s, dp);
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      const float tmax = row_max(fmaxf(fmaxf(s[x][0], s[x][1]), fmaxf(s[x][2], s[x][3])));
      const float mn = fmaxf(m[x], tmax);
      if (mn == -INFINITY) continue;  // (uniform over the row's 16 threads)
      const float al = __expf(m[x] - mn);
      float el = 0.f, ed = 0.f;
#pragma unroll
      for (int y = 0; y < 4; ++y) {
        const float e = __expf(s[x][y] - mn);
        el += e;
        ed += e * dp[x][y];
      }
      l[x] = l[x] * al + row_sum(el);
      dn[x] = dn[x] * al + row_sum(ed);
      m[x] = mn;
    }
  }
  float lse[4], Dd[4];
#pragma unroll
  for (int x = 0; x < 4; ++x) {
    lse[x] = l[x] > 0.f ? m[x] + __logf(l[x]) : 0.f;
    Dd[x] = l[x] > 0.f ? dn[x] / l[x] : 0.f;
  }

  // ---- walk 2: P, dS (to scratch), dq ---------------------------------------------
  float dqc[4][4] = {}, dqp[4][4] = {};  // rows 4 ti + x, columns 4 tj + y
  for (int kb = 0; kb < nkb; ++kb) {
    const int j0 = kb * BK;
    __syncthreads();
    load_tiles(j0);
    __syncthreads();
    float s[4][4], dp[4][4];
    pair_terms(j0, s, dp);
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      const int i = i0 + 4 * ti + x;
      float pv[4], dsv[4];
#pragma unroll
      for (int y = 0; y < 4; ++y) {
        pv[y] = s[x][y] == -INFINITY ? 0.f : __expf(s[x][y] - lse[x]);
        dsv[y] = pv[y] * (dp[x][y] - Dd[x]);
        sm.DS[4 * ti + x][4 * tj + y] = dsv[y];
      }
      if (i < L) {
        const int jb = j0 + 4 * tj;
        float* pr = a.P + prow0 + (int64_t)i * T;
        float* sr = a.dS + prow0 + (int64_t)i * T;
#pragma unroll
        for (int y = 0; y < 4; ++y)
          if (jb + y < T) {
            pr[jb + y] = pv[y];
            sr[jb + y] = dsv[y];
          }
      }
    }
    __syncthreads();
    for (int jj = 0; jj < BK; ++jj) {
      float ds[4], kv[4];
#pragma unroll
      for (int x = 0; x < 4; ++x) ds[x] = sm.DS[4 * ti + x][jj];
#pragma unroll
      for (int y = 0; y < 4; ++y) kv[y] = sm.K[jj][4 * tj + y];
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        const float* rrow = sm.RW[4 * ti + x - jj + (BK - 1)];
#pragma unroll
        for (int y = 0; y < 4; ++y) {
          dqc[x][y] += ds[x] * kv[y];
          dqp[x][y] += ds[x] * rrow[4 * tj + y];
        }
      }
    }
  }
  // keys past the last visible one: P = dS = 0 (the key-side products read whole rows)
  for (int e = tid; e < BQ * (T - nkb * BK > 0 ? T - nkb * BK : 0); e += 256) {
    const int span = T - nkb * BK;
    const int ii = e / span, j = nkb * BK + e % span, i = i0 + ii;
    if (i < L) {
      a.P[prow0 + (int64_t)i * T + j] = 0.f;
      a.dS[prow0 + (int64_t)i * T + j] = 0.f;
    }
  }
  // dq, and this block's shares of du and dv (reduced over its queries)
#pragma unroll
  for (int x = 0; x < 4; ++x) {
    const int i = i0 + 4 * ti + x;
    if (i >= L) continue;
#pragma unroll
    for (int y = 0; y < 4; ++y) {
      const int c = 4 * tj + y;
      if (c < d) a.dq[(((int64_t)b * L + i) * H + h) * d + c] = a.scale * (dqc[x][y] + dqp[x][y]);
    }
  }
  __syncthreads();
  float* red = &sm.DS[0][0];  // [2][16][64]
#pragma unroll
  for (int y = 0; y < 4; ++y) {
    float su = 0.f, sv = 0.f;
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      su += dqc[x][y];
      sv += dqp[x][y];
    }
    red[ti * 64 + 4 * tj + y] = su;
    red[1024 + ti * 64 + 4 * tj + y] = sv;
  }
  __syncthreads();
  if (tid < 64 && tid < d) {
    float su = 0.f, sv = 0.f;
    for (int t = 0; t < 16; ++t) {
      su += red[t * 64 + tid];
      sv += red[1024 + t * 64 + tid];
    }
    atomicAdd(a.du + (int64_t)h * d + tid, a.scale * su);
    atomicAdd(a.dvb + (int64_t)h * d + tid, a.scale * sv);
  }
}

// dr_p = scale sum_b sum_i dS[b][h][i][len + i - p] qp[b][h][i]: one workgroup
// per 64 distances of one head, the pairs of each (batch, 64-query block) staged
// as a [distance][query] tile of dS gathered along its diagonals.
__global__ __launch_bounds__(256) void attn_bwd_dr_kernel(AttnBwdArgs a) {
  __shared__ float DG[64][65];   // [distance][query]
  __shared__ float QPt[64][65];  // [query][column]
  const int tid = threadIdx.x;
  const int H = (int)a.H, L = (int)a.L, len = (int)a.mem_len, d = (int)a.d;
  const int T = len + L;
  const int h = blockIdx.y, p0 = blockIdx.x * 64;
  const int tp = tid / 16, tc = tid % 16;
  float acc[4][4] = {};
  for (int b = 0; b < (int)a.B; ++b) {
    const int64_t z = (int64_t)b * H + h;
    for (int i0 = 0; i0 < L; i0 += 64) {
      // pairs exist only for p <= len + i (uniform over the workgroup)
      if (p0 > len + (i0 + 63 < L - 1 ? i0 + 63 : L - 1)) continue;
      __syncthreads();
      for (int e = tid; e < 64 * 64; e += 256) {
        const int ii = e / 64, c = e % 64, i = i0 + ii;
        QPt[ii][c] = i < L ? a.qp[(z * L + i) * DP + c] : 0.f;
        // DG: consecutive threads take consecutive distances of one query
        const int pp = e % 64, iq = e / 64, iq_abs = i0 + iq, p = p0 + pp;
        const int j = len + iq_abs - p;
        DG[pp][iq] = (iq_abs < L && p < T && j >= 0) ? a.dS[(z * L + iq_abs) * T + j] : 0.f;
      }
      __syncthreads();
      for (int ii = 0; ii < 64; ++ii) {
        float g[4], q[4];
#pragma unroll
        for (int x = 0; x < 4; ++x) g[x] = DG[4 * tp + x][ii];
#pragma unroll
        for (int y = 0; y < 4; ++y) q[y] = QPt[ii][4 * tc + y];
#pragma unroll
        for (int x = 0; x < 4; ++x)
#pragma unroll
          for (int y = 0; y < 4; ++y) acc[x][y] += g[x] * q[y];
      }
    }
  }
#pragma unroll
  for (int x = 0; x < 4; ++x) {
    const int p = p0 + 4 * tp + x;
    if (p >= T) continue;
#pragma unroll
    for (int y = 0; y < 4; ++y) {
      const int c = 4 * tc + y;
      if (c < d) a.dr[((int64_t)p * H + h) * d + c] = a.scale * acc[x][y];
    }
  }
}

__global__ void attn_bwd_zero_kernel(float* p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    p[i] = 0.f;
}

}  // namespace

size_t attn_bwd_scratch_bytes(int64_t B, int64_t H, int64_t L, int64_t mem_len) {
  const size_t T = (size_t)(mem_len + L), rows = (size_t)(B * H * L);
  auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
  return al(rows * T * 4) * 2 + al(rows * DP * 4) * 2 + 256;
}

void attn_bwd_bind(AttnBwdArgs& a, void* scratch) {
  const size_t T = (size_t)(a.mem_len + a.L), rows = (size_t)(a.B * a.H * a.L);
  auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
  char* base = (char*)(((uintptr_t)scratch + 255) & ~(uintptr_t)255);
  a.P = (float*)base;
  base += al(rows * T * 4);
  a.dS = (float*)base;
  base += al(rows * T * 4);
  a.qc = (float*)base;
  base += al(rows * DP * 4);
  a.qp = (float*)base;
}

hipError_t launch_attn_bwd(int dtype, const AttnBwdArgs& a, hipStream_t s) {
  if (a.d > DP || a.d < 1 || a.B < 1 || a.H < 1 || a.L < 1 || a.mem_len < 0)
    return hipErrorInvalidValue;
  const int64_t T = a.mem_len + a.L, H = a.H, d = a.d;
  if (a.B * a.H > 65535 || (a.L + BQ - 1) / BQ > 0x7fffffff) return hipErrorInvalidValue;
  if (!a.zeroed) {
    hipLaunchKernelGGL(attn_bwd_zero_kernel, dim3(1), dim3(256), 0, s, a.du, H * d);
    hipLaunchKernelGGL(attn_bwd_zero_kernel, dim3(1), dim3(256), 0, s, a.dvb, H * d);
  }
  hipError_t e;
  if (dtype == 1) {
    if ((e = launch_attn_bwd_rows_mfma(a, s)) != hipSuccess) return e;
  } else {
    const size_t smem = sizeof(BwdSmem);
    static bool attr_set = false;
    if (!attr_set) {
      e = hipFuncSetAttribute((const void*)attn_bwd_rows_kernel<float>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
      if (e != hipSuccess) return e;
      attr_set = true;
    }
    const dim3 grid((unsigned)((a.L + BQ - 1) / BQ), (unsigned)(a.B * a.H));
    hipLaunchKernelGGL(attn_bwd_rows_kernel<float>, grid, dim3(256), smem, s, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  // dv = P^T dO and dk = scale dS^T (q + u), per (batch, head): m = key, k = query
  StridedGemm g{};
  g.M = T; g.N = d; g.K = a.L; g.batch = a.B * a.H; g.zdiv = H;
  g.A = {a.P, H * a.L * T, a.L * T, 1, T};
  g.B = {a.dout, a.do_sb, a.do_sh, a.do_st, 1};
  g.C = a.dv; g.c1 = T * H * d; g.c2 = d; g.cm = H * d; g.cn = 1;
  g.alpha = 1.f; g.accumulate = 0; g.a_dtype = 0; g.b_dtype = (dtype == 1 && !a.dout_f32) ? 1 : 0;
  g.bf16_mfma = dtype == 1 ? 1 : 0;  // bf16 inputs: P and dS enter the products as bf16
  g.a_dtype = dtype == 1 ? 1 : 0;     // and the matrix-core rows kernel stores them so
  // (matrix-core path: the rows kernel writes P and dS only up to each query
  // block's last visible key tile; the products read key j of query i only where
  // j <= mem_len + i)
  g.causal_on = dtype == 1 ? 1 : 0;
  g.causal_off = a.mem_len;
  if ((e = launch_gemm_strided(g, s)) != hipSuccess) return e;
  g.A.p = a.dS;  // (bf16 path: P and dS are stored as bf16)
  g.B = {a.qc, H * a.L * DP, a.L * DP, DP, 1};
  g.b_dtype = 0;
  g.C = a.dk;
  g.alpha = a.scale;
  if ((e = launch_gemm_strided(g, s)) != hipSuccess) return e;
  if (dtype == 1) return launch_attn_bwd_dr_mfma(a, s);
  hipLaunchKernelGGL(attn_bwd_dr_kernel, dim3((unsigned)((T + 63) / 64), (unsigned)H), dim3(256), 0,
                     s, a);
  return hipGetLastError();
}

}  // namespace txl
