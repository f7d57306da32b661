// Backward pass of the relative-position attention on the bf16 matrix cores
// (Transformer-XL, section 3.3: score with content and position terms and the
// global biases u and v; Appendix B: key j of query i at distance mem_len+i-j).
// It replaces the fp32 rows kernel for bf16 inputs and writes the same things:
// P and dS (here as bf16 scratch, the precision in which the key-side products
// take them; only up to each query block's last visible key tile, the products
// taking the pairs past the diagonal as zero), dq, and this block's shares of du
// and dv; the gradients sum in fp32.
//
// One workgroup = 4 waves = 64 queries of one (batch, head); wave w owns queries
// 16 w .. 16 w + 15 of the block.  All products are v_mfma_f32_16x16x32_bf16 and
// keep the queries on the 16 lanes n of a block (keys / columns on the registers
// and the lane groups g), as in the forward kernel:
//
//   S^T   = K Qc^T + gather(W^T),  W^T = RW Qp^T over the wave's 80 distance rows
//           (the diagonal shift is the address of a store into a [query][key]
//           buffer, read back as the content product's accumulator)
//   dP^T  = V G^T                    (G = dO)
//   walk 1: running max, sum of exponentials, and their sum weighted by dP
//   walk 2: P = exp(S - lse), dS = P (dP - D), D = sum_j P dP;
//           dq^T += K^T dS^T  (content)  and  RW^T dSw^T  (position), where
//           dSw[i][distance row] = dS[i][key] is the inverse of the shift,
//           written into a zeroed [query][distance row] buffer.
// K^T and RW^T fragments come from their row-major tiles through transposing
// LDS reads (ds_read_b64_tr_b16); dS^T is packed from registers in the k order
// those reads produce.  (q+u) and (q+v) are scaled by scale * log2(e) before
// rounding, so the softmax runs in the exp2 domain.
#include "txl_internal.h"

namespace txl {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef short v4s __attribute__((ext_vector_type(4)));

constexpr int BQ = 64, BK = 64, DP = 64;
constexpr int KPI = DP + 8;        // bf16 pitch of the K, V and r rows in LDS (144 bytes)
constexpr int RWR = 144;           // r rows staged per tile (distance rows 0 .. 143)
constexpr int SPP = 68;            // float pitch of a wave's [query][key] position buffer
constexpr int DWP = 104;           // bf16 pitch of a wave's [query][distance row] dS buffer
constexpr float LOG2E = 1.4426950408889634f;

struct __align__(16) BwdMfmaSmem {
  uint16_t K[BK * KPI];
  uint16_t V[BK * KPI];
  uint16_t RW[RWR * KPI];          // row w: distance len + i0 - j0 - 63 + w
  float Sp[4][16 * SPP];
  uint16_t Dw[4][16 * DWP];
};

__device__ inline uint32_t pack2(float lo, float hi) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){lo, hi}, bf16x2));
}
__device__ inline f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ inline bf16x8 lds_tr2(const uint16_t* p0, const uint16_t* p1) {
  const v4s a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s*)p0);
  const v4s b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s*)p1);
  const v4s ab[2] = {a, b};
  return *(const bf16x8*)ab;
}
// reductions over the four lanes of one query (n, n + 16, n + 32, n + 48)
__device__ inline float max4(float x) {
  x = fmaxf(x, __shfl_xor(x, 16, 64));
  return fmaxf(x, __shfl_xor(x, 32, 64));
}
__device__ inline float sum4(float x) {
  x += __shfl_xor(x, 16, 64);
  return x + __shfl_xor(x, 32, 64);
}

// Rows [row0, row0 + NR) of a bf16 [row][c] operand (row stride rs), columns
// 0..63 in 16-byte chunks (zero past d and outside [0, rmax)): chunk q = tid +
// 256 x is row q / 8, columns 8 (q % 8) ..  fetch_rows loads this thread's
// chunks into registers, store_rows writes them to LDS rows of KPI elements.
template <int NR>
__device__ inline void fetch_rows(const uint16_t* src, int64_t rs, int row0, int rmax, int d,
                                  bool vec, int tid, uint4 (&v)[(NR * 8 + 255) / 256]) {
#pragma unroll
  for (int x = 0; x < (NR * 8 + 255) / 256; ++x) {
    const int q = tid + 256 * x;
    const int rr = q >> 3, c0 = 8 * (q & 7), row = row0 + rr;
    v[x] = make_uint4(0u, 0u, 0u, 0u);
    if (q < NR * 8 && row >= 0 && row < rmax && c0 < d) {
      const uint16_t* p = src + (int64_t)row * rs + c0;
      if (vec && c0 + 8 <= d) {
        v[x] = *(const uint4*)p;
      } else {
        uint16_t t[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) t[e] = c0 + e < d ? p[e] : (uint16_t)0;
        v[x] = make_uint4(t[0] | ((uint32_t)t[1] << 16), t[2] | ((uint32_t)t[3] << 16),
                          t[4] | ((uint32_t)t[5] << 16), t[6] | ((uint32_t)t[7] << 16));
      }
    }
  }
}
template <int NR>
__device__ inline void store_rows(uint16_t* dst, int tid, const uint4 (&v)[(NR * 8 + 255) / 256]) {
#pragma unroll
  for (int x = 0; x < (NR * 8 + 255) / 256; ++x) {
    const int q = tid + 256 * x;
    if (q < NR * 8) *(uint4*)(dst + (q >> 3) * KPI + 8 * (q & 7)) = v[x];
  }
}

__global__ __launch_bounds__(256, 2) void attn_bwd_mfma_kernel(AttnBwdArgs a, int vec) {
  extern __shared__ __align__(16) char smem_raw[];
  BwdMfmaSmem& sm = *(BwdMfmaSmem*)smem_raw;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g4 = lane >> 4, n16 = lane & 15;
  const int H = (int)a.H, L = (int)a.L, len = (int)a.mem_len, d = (int)a.d;
  const int T = len + L;
  // one-dimensional grid, the last query blocks (the most key tiles) first
  const int nz = (int)(a.B * a.H), nqb = (L + BQ - 1) / BQ;
  const int z = (int)(blockIdx.x % nz), b = z / H, h = z % H;
  const int i0 = (nqb - 1 - (int)(blockIdx.x / nz)) * BQ;
  const int i = i0 + 16 * wave + n16;  // this lane's query
  const bool qok = i < L;
  const int imax = i0 + BQ - 1 < L - 1 ? i0 + BQ - 1 : L - 1;
  const int nkb = (len + imax) / BK + 1;
  const int64_t prow = ((int64_t)z * L + i) * T;  // row (b, h, i) of P and dS
  const float sl2 = a.scale * LOG2E;

  const uint16_t* kbase = (const uint16_t*)a.k + b * a.kv_sb + h * a.kv_sh;
  const uint16_t* vbase = (const uint16_t*)a.v + b * a.kv_sb + h * a.kv_sh;
  const uint16_t* rbase = (const uint16_t*)a.r + h * a.r_sh;

  // ---- this lane's query fragments: columns 32 s + 8 g4 + e --------------------------
  bf16x8 qcf[2], qpf[2], gf[2];
  float dot_go = 0.f;  // this lane's share of dO . o (with the forward's statistics)
  {
    const uint16_t* orow = a.o ? (const uint16_t*)a.o + b * a.o_sb + (int64_t)(qok ? i : 0) * a.o_st +
                                     h * a.o_sh
                               : nullptr;
    const uint16_t* qrow = (const uint16_t*)a.q + b * a.q_sb + (int64_t)(qok ? i : 0) * a.q_st +
                           h * a.q_sh;
    const int64_t go = b * a.do_sb + (int64_t)(qok ? i : 0) * a.do_st + h * a.do_sh;
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int c = 32 * s + 8 * g4 + e;
        const bool ok = qok && c < d;
        const float qv = ok ? bf16_to_f32(qrow[c]) : 0.f;
        const float qc = ok ? qv + bf16_to_f32(((const uint16_t*)a.u)[h * d + c]) : 0.f;
        const float qp = ok ? qv + bf16_to_f32(((const uint16_t*)a.vb)[h * d + c]) : 0.f;
        const float g = !ok ? 0.f
                            : (a.dout_f32 ? ((const float*)a.dout)[go + c]
                                          : bf16_to_f32(((const uint16_t*)a.dout)[go + c]));
        qcf[s][e] = (__bf16)(qc * sl2);
        qpf[s][e] = (__bf16)(qp * sl2);
        gf[s][e] = (__bf16)g;
        if (orow && ok) dot_go += g * bf16_to_f32(orow[c]);
        if (qok) {  // unscaled q + u, q + v for the key-side products and dr
          a.qc[((int64_t)z * L + i) * DP + c] = qc;
          a.qp[((int64_t)z * L + i) * DP + c] = qp;
        }
      }
  }

  // zero this wave's dS-by-distance buffer once: slots outside a query's 64
  // distance rows are never written and must read as 0
  for (int x = lane; x < 16 * DWP / 2; x += 64) ((uint32_t*)sm.Dw[wave])[x] = 0u;

  float* const sp = sm.Sp[wave];
  uint16_t* const dw = sm.Dw[wave];
  // transposing-read offsets (elements): lane (g4, n16) reads row 4 g4 + n16 / 4
  // (+ 16 for the second half), 8-byte piece 4 db + n16 % 4 of it
  int toff[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) toff[db] = (4 * g4 + (n16 >> 2)) * KPI + 4 * (4 * db + (n16 & 3));

  // Tile j0's K, V and r rows: fetched into registers one tile ahead (the loads
  // run during the previous tile's products), then written to LDS.
  uint4 fk[(BK * 8 + 255) / 256], fv[(BK * 8 + 255) / 256], fr[(RWR * 8 + 255) / 256];
  auto fetch = [&](int j0) {
    fetch_rows<BK>(kbase, a.kv_st, j0, T, d, vec & 1, tid, fk);
    fetch_rows<BK>(vbase, a.kv_st, j0, T, d, vec & 1, tid, fv);
    fetch_rows<RWR>(rbase, a.r_sp, len + i0 - j0 - (BK - 1), T, d, (vec & 2) != 0, tid, fr);
  };
  auto commit = [&]() {
    store_rows<BK>(sm.K, tid, fk);
    store_rows<BK>(sm.V, tid, fv);
    store_rows<RWR>(sm.RW, tid, fr);
  };
  // S^T (exp2 domain, masked to -inf) and dP^T of key tile j0: block kb, register e
  // = key j0 + 16 kb + 4 g4 + e of query i
  auto scores = [&](int j0, f32x4 (&S)[4], f32x4 (&dP)[4]) {
    f32x4 w[5];
#pragma unroll
    for (int bw = 0; bw < 5; ++bw) {
      const uint16_t* rrow = sm.RW + (16 * wave + 16 * bw + n16) * KPI + 8 * g4;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      acc = mfma(*(const bf16x8*)rrow, qpf[0], acc);
      w[bw] = mfma(*(const bf16x8*)(rrow + 32), qpf[1], acc);
    }
    // distance row 16 bw + 4 g4 + e of query n16 is key jj = n16 + 63 - 16 bw - 4 g4 - e;
    // blocks 0 and 4 hold keys jj and jj - 64 (exactly one of them in 0..63)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int jj = n16 + 63 - 4 * g4 - e;
      sp[n16 * SPP + (jj & 63)] = jj <= 63 ? w[0][e] : w[4][e];
    }
#pragma unroll
    for (int bw = 1; bw < 4; ++bw)
#pragma unroll
      for (int e = 0; e < 4; ++e) sp[n16 * SPP + n16 + 63 - 16 * bw - 4 * g4 - e] = w[bw][e];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const uint16_t* krow = sm.K + (16 * kb + n16) * KPI + 8 * g4;
      const uint16_t* vrow = sm.V + (16 * kb + n16) * KPI + 8 * g4;
      f32x4 c = *(const f32x4*)(sp + n16 * SPP + 16 * kb + 4 * g4);
      c = mfma(*(const bf16x8*)krow, qcf[0], c);
      S[kb] = mfma(*(const bf16x8*)(krow + 32), qcf[1], c);
      f32x4 p = {0.f, 0.f, 0.f, 0.f};
      p = mfma(*(const bf16x8*)vrow, gf[0], p);
      dP[kb] = mfma(*(const bf16x8*)(vrow + 32), gf[1], p);
    }
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int j = j0 + 16 * kb + 4 * g4 + e;
        if (!qok || j > len + i) S[kb][e] = -INFINITY;
      }
  };

  // ---- walk 1: running max m, sum l of exp2(S - m), and sum of exp2(S - m) dP ----------
  //      (skipped when the forward's log-sum-exp is given: then D = dO . o)
  float m = -INFINITY, l = 0.f, dn = 0.f;  // l, dn: this lane's partial sums
  fetch(0);
  const bool fwd_stats = a.lse != nullptr;
  for (int kb0 = 0; kb0 < (fwd_stats ? 0 : nkb); ++kb0) {
    const int j0 = kb0 * BK;
    __syncthreads();
    commit();
    __syncthreads();
    fetch(kb0 + 1 < nkb ? j0 + BK : 0);  // walk 2 starts again at tile 0
    f32x4 S[4], dP[4];
    scores(j0, S, dP);
    float tmax = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int e = 0; e < 4; ++e) tmax = fmaxf(tmax, S[kb][e]);
    const float mn = fmaxf(m, max4(tmax));
    if (mn != -INFINITY) {
      const float al = __builtin_amdgcn_exp2f(m - mn);  // m = -inf: 0
      float el = 0.f, ed = 0.f;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float x = S[kb][e] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(S[kb][e] - mn);
          el += x;
          ed += x * dP[kb][e];
        }
      l = l * al + el;
      dn = dn * al + ed;
      m = mn;
    }
  }
  l = sum4(l);
  dn = sum4(dn);
  dot_go = sum4(dot_go);
  const float lse = fwd_stats ? (qok ? a.lse[(int64_t)z * L + i] : 0.f) : (l > 0.f ? m + __log2f(l) : 0.f);
  const float Dd = fwd_stats ? dot_go : (l > 0.f ? dn / l : 0.f);

  // ---- walk 2: P, dS (to scratch), dq = scale (K^T dS^T + RW^T dSw^T) -------------------
  f32x4 dqc[4], dqp[4];  // rows = columns 16 db + 4 g4 + e, lane = query n16
#pragma unroll
  for (int db = 0; db < 4; ++db) dqc[db] = dqp[db] = {0.f, 0.f, 0.f, 0.f};
  for (int kb0 = 0; kb0 < nkb; ++kb0) {
    const int j0 = kb0 * BK;
    __syncthreads();
    commit();
    __syncthreads();
    if (kb0 + 1 < nkb) fetch(j0 + BK);
    f32x4 S[4], dP[4];
    scores(j0, S, dP);
    f32x4 dS[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float p = S[kb][e] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(S[kb][e] - lse);
        dS[kb][e] = p * (dP[kb][e] - Dd);
        S[kb][e] = p;
      }
    if (qok) {  // bf16 rows of P and dS (they enter the key-side products as bf16)
      uint16_t* prow_p = (uint16_t*)a.P + prow;
      uint16_t* prow_s = (uint16_t*)a.dS + prow;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const int j = j0 + 16 * kb + 4 * g4;  // 4 consecutive keys j .. j + 3
        if ((T & 3) == 0) {  // 8-byte aligned
          if (j < T) {
            *(uint2*)(prow_p + j) = make_uint2(pack2(S[kb][0], S[kb][1]), pack2(S[kb][2], S[kb][3]));
            *(uint2*)(prow_s + j) =
                make_uint2(pack2(dS[kb][0], dS[kb][1]), pack2(dS[kb][2], dS[kb][3]));
          }
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (j + e < T) {
              prow_p[j + e] = __builtin_bit_cast(uint16_t, (__bf16)S[kb][e]);
              prow_s[j + e] = __builtin_bit_cast(uint16_t, (__bf16)dS[kb][e]);
            }
        }
      }
    }
    // dS by distance row: key jj of query n16 is row n16 + 63 - jj
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        dw[n16 * DWP + n16 + 63 - (16 * kb + 4 * g4 + e)] =
            __builtin_bit_cast(uint16_t, (__bf16)dS[kb][e]);
    // content: k index 8 g4 + 4 kb' + e of key half hh <-> key 32 hh + 16 kb' + 4 g4 + e
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const uint4 pk = make_uint4(pack2(dS[2 * hh][0], dS[2 * hh][1]), pack2(dS[2 * hh][2], dS[2 * hh][3]),
                                  pack2(dS[2 * hh + 1][0], dS[2 * hh + 1][1]),
                                  pack2(dS[2 * hh + 1][2], dS[2 * hh + 1][3]));
      const bf16x8 dsb = __builtin_bit_cast(bf16x8, pk);
      const uint16_t* kt = sm.K + 32 * hh * KPI;
#pragma unroll
      for (int db = 0; db < 4; ++db)
        dqc[db] = mfma(lds_tr2(kt + toff[db], kt + 16 * KPI + toff[db]), dsb, dqc[db]);
    }
    // position: distance rows 32 hh + 16 kb' + 4 g4 + e of the wave's window (rows
    // 16 wave ..), the same k order on both sides
#pragma unroll
    for (int hh = 0; hh < 3; ++hh) {
      const uint16_t* drow = dw + n16 * DWP + 32 * hh + 4 * g4;
      const uint2 lo = *(const uint2*)drow, hi = *(const uint2*)(drow + 16);
      const bf16x8 dsw = __builtin_bit_cast(bf16x8, make_uint4(lo.x, lo.y, hi.x, hi.y));
      const uint16_t* rt = sm.RW + (16 * wave + 32 * hh) * KPI;
#pragma unroll
      for (int db = 0; db < 4; ++db)
        dqp[db] = mfma(lds_tr2(rt + toff[db], rt + 16 * KPI + toff[db]), dsw, dqp[db]);
    }
  }

  // (keys past the block's last visible key tile are left unwritten: the key-side
  // products take P and dS as zero past the diagonal, and the position gradient
  // reads visible pairs only)
  // dq, and this block's shares of du and dv
  if (qok) {
    float* dqrow = a.dq + (((int64_t)b * L + i) * H + h) * d;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int c = 16 * db + 4 * g4 + e;
        if (c < d) dqrow[c] = a.scale * (dqc[db][e] + dqp[db][e]);
      }
  }
  __syncthreads();
  float* red = &sm.Sp[0][0];  // [2][4 waves][64 columns]
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float su = dqc[db][e], sv = dqp[db][e];  // rows past L hold zeros
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) {
        su += __shfl_xor(su, o, 64);
        sv += __shfl_xor(sv, o, 64);
      }
      if (n16 == 0) {
        red[wave * 64 + 16 * db + 4 * g4 + e] = su;
        red[256 + wave * 64 + 16 * db + 4 * g4 + e] = sv;
      }
    }
  __syncthreads();
  if (tid < d) {
    float su = 0.f, sv = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      su += red[w * 64 + tid];
      sv += red[256 + w * 64 + tid];
    }
    atomicAdd(a.du + (int64_t)h * d + tid, a.scale * su);
    atomicAdd(a.dvb + (int64_t)h * d + tid, a.scale * sv);
  }
}

// dr_p = scale sum over (b, i) of dS[b][h][i][len + i - p] (q_i + v): the pairs at
// distance p lie on a diagonal of dS.  Workgroup (distance block, head, split)
// takes the (batch, 64-query block) items split, split + nsplit, ...: per item
// it gathers the diagonals into a [distance][query] tile and (q + v) into a
// [column][query] tile (bf16 in LDS), and wave w multiplies distances 16 w ..
// 16 w + 15 by all 64 columns.  With nsplit > 1 the partial sums are added
// atomically into dr (cleared before).
constexpr int DGP = 64 + 8;  // bf16 pitch of both tiles

__global__ __launch_bounds__(256) void attn_bwd_dr_mfma_kernel(AttnBwdArgs a, int nsplit) {
  __shared__ __align__(16) uint16_t DG[64 * DGP];
  __shared__ __align__(16) uint16_t QT[64 * DGP];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g4 = lane >> 4, n16 = lane & 15;
  const int H = (int)a.H, L = (int)a.L, len = (int)a.mem_len, d = (int)a.d;
  const int T = len + L;
  const int p0 = blockIdx.x * 64, h = blockIdx.y, split = blockIdx.z;
  const int nqb = (L + 63) / 64, items = (int)a.B * nqb;
  f32x4 acc[4];
#pragma unroll
  for (int cb = 0; cb < 4; ++cb) acc[cb] = {0.f, 0.f, 0.f, 0.f};
  // items with a pair at these distances, in this split's order
  auto next_item = [&](int it) {
    for (; it < items; it += nsplit) {
      const int i0 = (it % nqb) * 64, ilast = i0 + 63 < L - 1 ? i0 + 63 : L - 1;
      if (p0 <= len + ilast) break;
    }
    return it;
  };
  // this thread's gathers of one item: unit u = tid + 256 x covers distances /
  // columns 4 (u % 16) .. + 3 of queries i0 + 2 (u / 16), + 1.  Every load is
  // issued unconditionally (indexes clamped into the tensors, the values of
  // pairs outside the block dropped when staged): a per-lane test around each
  // load made every load wait for the one before it.
  struct Gath {
    uint16_t raw[2][2][4];
    float4 qf[2][2];
  };
  auto gather = [&](int it, Gath& G) {
    const int b = it / nqb, i0 = (it % nqb) * 64;
    const int64_t z = (int64_t)b * H + h;
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      const int u = tid + 256 * x;
      const int f4 = 4 * (u & 15), ii = 2 * (u >> 4);
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        const int i = i0 + ii + r, ic = i < L ? i : L - 1;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int p = p0 + f4 + e, j = len + ic - p;
          const int jc = j < 0 ? 0 : (j < T ? j : T - 1);
          G.raw[x][r][e] = ((const uint16_t*)a.dS)[(z * L + ic) * T + jc];
        }
        G.qf[x][r] = *(const float4*)(a.qp + (z * L + ic) * DP + f4);
      }
    }
  };
  // the next item's gathers are in flight while this one is staged and multiplied
  int it = next_item(split);
  Gath cur;
  if (it < items) gather(it, cur);
  while (it < items) {
    const int nit = next_item(it + nsplit);
    Gath nxt;
    if (nit < items) gather(nit, nxt);
    const int i0 = (it % nqb) * 64;
    __syncthreads();  // the previous item's tiles are read
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      const int u = tid + 256 * x;
      const int f4 = 4 * (u & 15), ii = 2 * (u >> 4);
      float v[2][4], w[2][4];
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        const int i = i0 + ii + r;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int p = p0 + f4 + e, j = len + i - p;
          v[r][e] = (i < L && p < T && j >= 0) ? bf16_to_f32(cur.raw[x][r][e]) : 0.f;
        }
        const bool iok = i < L;
        w[r][0] = iok ? cur.qf[x][r].x : 0.f; w[r][1] = iok ? cur.qf[x][r].y : 0.f;
        w[r][2] = iok ? cur.qf[x][r].z : 0.f; w[r][3] = iok ? cur.qf[x][r].w : 0.f;
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        *(uint32_t*)(DG + (f4 + e) * DGP + ii) = pack2(v[0][e], v[1][e]);
        *(uint32_t*)(QT + (f4 + e) * DGP + ii) = pack2(w[0][e], w[1][e]);
      }
    }
    __syncthreads();
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const bf16x8 af = *(const bf16x8*)(DG + (16 * wave + n16) * DGP + 32 * s + 8 * g4);
#pragma unroll
      for (int cb = 0; cb < 4; ++cb)
        acc[cb] = mfma(af, *(const bf16x8*)(QT + (16 * cb + n16) * DGP + 32 * s + 8 * g4), acc[cb]);
    }
    if (nit < items) cur = nxt;
    it = nit;
  }
  // lane (g4, n16) of block cb: distance p0 + 16 wave + 4 g4 + e, column 16 cb + n16
#pragma unroll
  for (int cb = 0; cb < 4; ++cb)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int p = p0 + 16 * wave + 4 * g4 + e, c = 16 * cb + n16;
      if (p < T && c < d) {
        float* o = a.dr + ((int64_t)p * H + h) * d + c;
        const float v = a.scale * acc[cb][e];
        if (nsplit > 1)
          atomicAdd(o, v);
        else
          *o = v;
      }
    }
}

__global__ void zero_kernel(float* p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    p[i] = 0.f;
}

}  // namespace

hipError_t launch_attn_bwd_dr_mfma(const AttnBwdArgs& a, hipStream_t s) {
  const int64_t T = a.mem_len + a.L, nqb = (a.L + 63) / 64, items = a.B * nqb;
  const int64_t blocks = ((T + 63) / 64) * a.H;
  if (blocks > 0x7fffffffLL || a.H > 65535) return hipErrorInvalidValue;
  // enough workgroups for the GPU (about four per CU), each with several items
  int64_t nsplit = (1024 + blocks - 1) / blocks;
  nsplit = nsplit < items ? nsplit : items;
  nsplit = nsplit < 1 ? 1 : (nsplit > 65535 ? 65535 : nsplit);
  if (nsplit > 1 && !a.zeroed) {
    const int64_t n = T * a.H * a.d;
    const int64_t zb = (n + 255) / 256 < 1024 ? (n + 255) / 256 : 1024;
    hipLaunchKernelGGL(zero_kernel, dim3((unsigned)zb), dim3(256), 0, s, a.dr, n);
  }
  hipLaunchKernelGGL(attn_bwd_dr_mfma_kernel, dim3((unsigned)((T + 63) / 64), (unsigned)a.H,
                                                   (unsigned)nsplit),
                     dim3(256), 0, s, a, (int)nsplit);
  return hipGetLastError();
}

hipError_t launch_attn_bwd_rows_mfma(const AttnBwdArgs& a, hipStream_t s) {
  const size_t smem = sizeof(BwdMfmaSmem);
  static bool attr_set = false;
  if (!attr_set) {
    const hipError_t e = hipFuncSetAttribute((const void*)attn_bwd_mfma_kernel,
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  // 16-byte row loads when every row start of k / v (resp. r) is 16-byte aligned
  const uintptr_t kv = (uintptr_t)a.k | (uintptr_t)a.v;
  const bool kv_vec = kv % 16 == 0 && a.kv_sb % 8 == 0 && a.kv_st % 8 == 0 && a.kv_sh % 8 == 0;
  const bool r_vec = (uintptr_t)a.r % 16 == 0 && a.r_sp % 8 == 0 && a.r_sh % 8 == 0;
  const int64_t nblk = ((a.L + BQ - 1) / BQ) * a.B * a.H;
  if (nblk > 0x7fffffffLL) return hipErrorInvalidValue;
  const dim3 grid((unsigned)nblk);
  hipLaunchKernelGGL(attn_bwd_mfma_kernel, grid, dim3(256), smem, s, a,
                     (kv_vec ? 1 : 0) | (r_vec ? 2 : 0));
  return hipGetLastError();
}

}  // namespace txl
