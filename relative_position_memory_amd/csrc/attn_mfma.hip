// Relative-position attention over segment-level memory, bf16 matrix-core path
// for gfx950 (Transformer-XL, section 3.3: the A^rel score with terms (a)-(d);
// Appendix B: distances 0 .. M+L-1, key j of query i at distance mem_len+i-j).
//
// One workgroup = 4 waves = 128 queries of one (batch row, head); each wave owns
// 32 queries and walks the key tiles (64 keys) up to its last visible key with
// an online softmax in the exp2 domain.  Per key tile and wave:
//
//   position term  W^T = r_win . Qp^T : a 96 x 32 MFMA product of the r rows of
//                  the 95 distances the tile can need (reversed order) with the
//                  wave's queries (q+v) -> written to a wave-private LDS buffer.
//                  Row ii of W (query ii) is stored with pitch P = 101 floats;
//                  the score of (query ii, key jj) sits at window index
//                  31 - ii + jj, i.e. at flat offset ii*(P-1) + jj + 31 : read
//                  back with pitch P-1 the diagonal "relative shift" becomes a
//                  plain aligned 16-byte read (the padded-reshape idea of the
//                  shift, done in LDS addresses instead of memory copies).
//   content term   S^T = K . Qc^T  (q+u), with the position term loaded as the
//                  MFMA accumulator, so the sum of the four terms costs no ALU op.
//   softmax        S^T keeps one query per lane: row max and row sum are in-lane
//                  (plus one exchange between the two lane halves).
//   P.V            O^T = V^T . P^T, V staged transposed in LDS.
//
// The scale 1/sqrt(d) and log2(e) are folded into (q+u) and (q+v) before they
// are rounded to bf16, so the softmax is exp2(S - max) with no extra multiply.
#include "txl_internal.h"

namespace txl {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;

constexpr int NW = 4;           // waves per workgroup
constexpr int BQW = 32;         // queries per wave
constexpr int BQ = NW * BQW;    // queries per workgroup
constexpr int BK = 64;          // keys per tile
constexpr int DP = 64;          // head size padded for the MFMA k-loop
constexpr int KP = 72;          // Ks / Rs row pitch (bf16): 144 B, 16B-aligned, conflict-free
constexpr int VP = 68;          // Vt row pitch (bf16): 136 B, 8B-aligned, conflict-free
constexpr int RROWS = BQ + BK;  // staged r rows: distances dist_lo .. dist_lo+191
constexpr int WP = 101;         // W row pitch (floats); read pitch WP-1 = 100
constexpr int WBUF = 1 + BQW * WP + 3;  // one wave's W buffer (floats), 16B multiple
constexpr float LOG2E = 1.4426950408889634f;

struct __align__(16) Smem {
  uint16_t Ks[BK * KP];      // K tile, [key][c]
  uint16_t Vt[DP * VP];      // V tile transposed, [c][key]
  uint16_t Rs[RROWS * KP];   // r rows of the window union, [row][c], natural order
  float Wb[NW * WBUF];       // position-term windows, one per wave
};

__device__ inline bf16x8 lds_b128(const uint16_t* p) { return *(const bf16x8*)p; }
__device__ inline bf16x8 lds_2xb64(const uint16_t* p0, const uint16_t* p1) {
  const bf16x4 a = *(const bf16x4*)p0, b = *(const bf16x4*)p1;
  return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

// 8 consecutive bf16 of a head row starting at element c0 (< d); zeros past d.
__device__ inline uint4 load_chunk(const uint16_t* row, int c0, int d, bool valid) {
  uint4 z = {0u, 0u, 0u, 0u};
  if (!valid || c0 >= d) return z;
  if (c0 + 8 <= d) return *(const uint4*)(row + c0);
  uint16_t t[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) t[e] = (c0 + e < d) ? row[c0 + e] : (uint16_t)0;
  uint4 o;
  o.x = t[0] | ((uint32_t)t[1] << 16);
  o.y = t[2] | ((uint32_t)t[3] << 16);
  o.z = t[4] | ((uint32_t)t[5] << 16);
  o.w = t[6] | ((uint32_t)t[7] << 16);
  return o;
}

// Registers holding one key tile on its way from HBM to LDS.
struct TileRegs {
  uint4 k[2];     // two 16B chunks of K
  uint4 v[2];     // V rows 2p and 2p+1, chunk cv
  uint4 r[6];     // six 16B chunks of the r window
};

__device__ inline void load_tile(TileRegs& tr, const AttnArgs& a, const uint16_t* kb,
                                 const uint16_t* vbp, const uint16_t* rb, int64_t j0,
                                 int64_t dist_lo, int64_t T, int tid) {
  const int d = (int)a.d;
#pragma unroll
  for (int x = 0; x < 2; ++x) {
    const int idx = tid + 256 * x;
    const int key = idx >> 3, c = idx & 7;
    const int64_t j = j0 + key;
    tr.k[x] = load_chunk(kb + j * a.kv_st, 8 * c, d, j < T);
  }
  {
    const int cv = tid & 7, p = tid >> 3;
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      const int64_t j = j0 + 2 * p + x;
      tr.v[x] = load_chunk(vbp + j * a.kv_st, 8 * cv, d, j < T);
    }
  }
#pragma unroll
  for (int x = 0; x < 6; ++x) {
    const int idx = tid + 256 * x;
    const int row = idx >> 3, c = idx & 7;
    const int64_t dist = dist_lo + row;
    tr.r[x] = load_chunk(rb + dist * a.r_sp, 8 * c, d, dist >= 0 && dist < T);
  }
}

__device__ inline void store_tile(Smem& sm, const TileRegs& tr, int tid) {
#pragma unroll
  for (int x = 0; x < 2; ++x) {
    const int idx = tid + 256 * x;
    const int key = idx >> 3, c = idx & 7;
    *(uint4*)&sm.Ks[key * KP + 8 * c] = tr.k[x];
  }
  {
    const int cv = tid & 7, p = tid >> 3;
    const uint32_t* v0 = (const uint32_t*)&tr.v[0];
    const uint32_t* v1 = (const uint32_t*)&tr.v[1];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      // elements 2w (low halves) and 2w+1 (high halves) of keys 2p and 2p+1
      const uint32_t lo = (v0[w] & 0xffffu) | (v1[w] << 16);
      const uint32_t hi = (v0[w] >> 16) | (v1[w] & 0xffff0000u);
      *(uint32_t*)&sm.Vt[(8 * cv + 2 * w) * VP + 2 * p] = lo;
      *(uint32_t*)&sm.Vt[(8 * cv + 2 * w + 1) * VP + 2 * p] = hi;
    }
  }
#pragma unroll
  for (int x = 0; x < 6; ++x) {
    const int idx = tid + 256 * x;
    const int row = idx >> 3, c = idx & 7;
    *(uint4*)&sm.Rs[row * KP + 8 * c] = tr.r[x];
  }
}

__global__ __launch_bounds__(256, 1) void attn_mfma_kernel(AttnArgs a, int nqt, int groups) {
  extern __shared__ __align__(16) char smem_raw[];
  Smem& sm = *(Smem*)smem_raw;

  // All query tiles of one (batch, head) are consecutive, longest first, so
  // they run together and share K, V and r through L2.
  const int g = blockIdx.x / nqt;
  const int qt = nqt - 1 - (int)(blockIdx.x % nqt);
  if (g >= groups) return;
  const int64_t b = g / a.H, hd = g % a.H;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int li = lane & 31, lh = lane >> 5;
  const int d = (int)a.d;
  const int64_t L = a.L, len = a.mem_len, T = len + L;
  const int64_t q0 = (int64_t)qt * BQ;
  const int64_t i0w = q0 + wave * BQW;

  const uint16_t* kb = (const uint16_t*)a.k + b * a.kv_sb + hd * a.kv_sh;
  const uint16_t* vbp = (const uint16_t*)a.v + b * a.kv_sb + hd * a.kv_sh;
  const uint16_t* rb = (const uint16_t*)a.r + hd * a.r_sh;

  // ---- this lane's query (column li of the MFMA B operand), pre-scaled ----------
  bf16x8 qc[4], qp[4];
  {
    const int64_t i = i0w + li;
    const uint16_t* qrow = (const uint16_t*)a.q + b * a.q_sb + i * a.q_st + hd * a.q_sh;
    const uint16_t* ur = (const uint16_t*)a.u + hd * d;
    const uint16_t* vr = (const uint16_t*)a.vb + hd * d;
    const float sl2 = a.scale * LOG2E;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int c0 = 16 * s + 8 * lh;
      const uint4 raw = load_chunk(qrow, c0, d, i < L);
      const uint16_t* rv = (const uint16_t*)&raw;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int c = c0 + e;
        float x = bf16_to_f32(rv[e]);
        const float uu = c < d ? bf16_to_f32(ur[c]) : 0.f;
        const float vv = c < d ? bf16_to_f32(vr[c]) : 0.f;
        qc[s][e] = (__bf16)(c < d ? (x + uu) * sl2 : 0.f);
        qp[s][e] = (__bf16)(c < d ? (x + vv) * sl2 : 0.f);
      }
    }
  }

  const int64_t imax_wg = (q0 + BQ - 1 < L - 1) ? q0 + BQ - 1 : L - 1;
  const int n_kt = (int)((len + imax_wg) / BK) + 1;
  const bool wave_has_rows = i0w < L;
  const int64_t imax_w = (i0w + BQW - 1 < L - 1) ? i0w + BQW - 1 : L - 1;
  const int kt_w = wave_has_rows ? (int)((len + imax_w) / BK) : -1;

  float m_run = -INFINITY, l_run = 0.f;
  f32x16 acc[2];
#pragma unroll
  for (int x = 0; x < 16; ++x) { acc[0][x] = 0.f; acc[1][x] = 0.f; }

  float* wb = sm.Wb + wave * WBUF;
  float* srow_base = nullptr;
  if (a.scores) srow_base = a.scores + ((b * a.H + hd) * L) * T;

  TileRegs tr;
  load_tile(tr, a, kb, vbp, rb, 0, len + q0 - BK, T, tid);

  for (int kt = 0; kt < n_kt; ++kt) {
    const int64_t j0 = (int64_t)kt * BK;
    __syncthreads();
    store_tile(sm, tr, tid);
    __syncthreads();
    if (kt + 1 < n_kt) {
      const int64_t j1 = j0 + BK;
      load_tile(tr, a, kb, vbp, rb, j1, len + q0 - j1 - BK, T, tid);
    }
    if (kt > kt_w) continue;

    const int64_t Dw = len + i0w - j0;  // distance of (query 0, key 0) of this wave's tile

    // ---- position term: W^T[w''][ii] = r[Dw + 31 - w''] . qp[ii], w'' in [0, 96) ----
#pragma unroll
    for (int blk = 0; blk < 3; ++blk) {
      f32x16 w;
#pragma unroll
      for (int x = 0; x < 16; ++x) w[x] = 0.f;
      // A-row li of block blk is distance Dw + 31 - 32 blk - li, staged at row
      // dist - (len + q0 - j0 - 64), which lies in [0, 191]
      const int rrow = BQW * wave + 95 - 32 * blk - li;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const bf16x8 ar = lds_b128(&sm.Rs[rrow * KP + 16 * s + 8 * lh]);
        w = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ar, qp[s], w, 0, 0, 0);
      }
      // lane (query li, half lh), reg x -> window index 32 blk + 8 (x/4) + 4 lh + x%4
#pragma unroll
      for (int x = 0; x < 16; ++x)
        wb[1 + li * WP + 32 * blk + 8 * (x >> 2) + 4 * lh + (x & 3)] = w[x];
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    // ---- content term with the gathered position term as accumulator ------------
    f32x16 sc[2];
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2) {
#pragma unroll
      for (int x4 = 0; x4 < 4; ++x4) {
        // keys jj = 32 kb2 + 8 x4 + 4 lh + t, t = 0..3 -> flat 32 + 100 li + jj
        const f32x4 sp = *(const f32x4*)&wb[32 + (WP - 1) * li + 32 * kb2 + 8 * x4 + 4 * lh];
        sc[kb2][4 * x4 + 0] = sp[0];
        sc[kb2][4 * x4 + 1] = sp[1];
        sc[kb2][4 * x4 + 2] = sp[2];
        sc[kb2][4 * x4 + 3] = sp[3];
      }
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const bf16x8 ak = lds_b128(&sm.Ks[(32 * kb2 + li) * KP + 16 * s + 8 * lh]);
        sc[kb2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ak, qc[s], sc[kb2], 0, 0, 0);
      }
    }

    // ---- causal mask (tiles that reach past the wave's first query only) --------
    if (j0 + BK - 1 > len + i0w) {
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
        for (int x = 0; x < 16; ++x) {
          const int jj = 32 * kb2 + 8 * (x >> 2) + 4 * lh + (x & 3);
          if (jj - li > Dw) sc[kb2][x] = -INFINITY;
        }
    }
    if (srow_base) {
      const int64_t i = i0w + li;
      if (i < L) {
        float* srow = srow_base + i * T;
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
          for (int x = 0; x < 16; ++x) {
            const int64_t j = j0 + 32 * kb2 + 8 * (x >> 2) + 4 * lh + (x & 3);
            if (j < T) srow[j] = sc[kb2][x] * (1.0f / LOG2E);
          }
      }
    }

    // ---- online softmax (exp2 domain), one query per lane --------------------------
    float tmax = -INFINITY;
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
      for (int x = 0; x < 16; ++x) tmax = fmaxf(tmax, sc[kb2][x]);
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
    const float m_new = fmaxf(m_run, tmax);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    m_run = m_new;
    float psum = 0.f;
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
      for (int x = 0; x < 16; ++x) {
        const float p = __builtin_amdgcn_exp2f(sc[kb2][x] - m_new);
        sc[kb2][x] = p;
        psum += p;
      }
    l_run = l_run * alpha + psum;
#pragma unroll
    for (int x = 0; x < 16; ++x) {
      acc[0][x] *= alpha;
      acc[1][x] *= alpha;
    }

    // ---- O^T += V^T . P^T ------------------------------------------------------------
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      bf16x8 pb;
      const int kb2 = s >> 1, v0 = 8 * (s & 1);
#pragma unroll
      for (int e = 0; e < 8; ++e) pb[e] = (__bf16)sc[kb2][v0 + e];
#pragma unroll
      for (int db = 0; db < 2; ++db) {
        const uint16_t* vrow = &sm.Vt[(32 * db + li) * VP + 16 * s + 4 * lh];
        const bf16x8 av = lds_2xb64(vrow, vrow + 8);
        acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, pb, acc[db], 0, 0, 0);
      }
    }
  }

  // ---- epilogue: out[i][c] = acc / l -------------------------------------------------
  if (!wave_has_rows) return;
  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  const int64_t i = i0w + li;
  if (i >= L) return;
  const float inv = 1.f / l_tot;
  uint16_t* orow = (uint16_t*)a.out + b * a.o_sb + i * a.o_st + hd * a.o_sh;
#pragma unroll
  for (int db = 0; db < 2; ++db)
#pragma unroll
    for (int x = 0; x < 16; ++x) {
      const int c = 32 * db + 8 * (x >> 2) + 4 * lh + (x & 3);
      if (c < d) orow[c] = f32_to_bf16(acc[db][x] * inv);
    }
}

}  // namespace

bool attn_mfma_supported(const AttnArgs& a) {
  if (a.d > DP) return false;
  const uintptr_t al = (uintptr_t)a.q | (uintptr_t)a.k | (uintptr_t)a.v | (uintptr_t)a.r;
  if (al % 16) return false;
  const int64_t st[] = {a.q_sb, a.q_st, a.q_sh, a.kv_sb, a.kv_st, a.kv_sh, a.r_sp, a.r_sh};
  for (int64_t s : st)
    if (s % 8) return false;
  return true;
}

hipError_t launch_attn_mfma(const AttnArgs& a, int num_cus, hipStream_t s) {
  (void)num_cus;
  const int nqt = (int)((a.L + BQ - 1) / BQ);
  const int groups = (int)(a.B * a.H);
  const int64_t nblocks = (int64_t)nqt * groups;
  const size_t smem = sizeof(Smem);
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)attn_mfma_kernel,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  hipLaunchKernelGGL(attn_mfma_kernel, dim3((unsigned)nblocks), dim3(256), smem, s, a, nqt,
                     groups);
  return hipGetLastError();
}

}  // namespace txl
