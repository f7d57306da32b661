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
//                  Row ii of W (query ii) is stored with pitch P = 69 floats;
//                  the score of (query ii, key jj) sits at window index
//                  31 - ii + jj, i.e. at flat offset ii*(P-1) + jj + 31 : read
//                  back with pitch P-1 the diagonal "relative shift" becomes a
//                  plain aligned 16-byte read (the padded-reshape idea of the
//                  shift, done in LDS addresses instead of memory copies).
//                  Only the 64 window entries a row reads are written, so the
//                  rows may overlap and the buffer stays small enough for two
//                  workgroups per CU.
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
constexpr int WP = 69;          // W row pitch (floats); read pitch WP-1 = 68 (= 4 mod 32)
constexpr int WBUF = 2208;      // one wave's W buffer (floats): 1 + 31*69 + 94 - 31 < 2208
constexpr float LOG2E = 1.4426950408889634f;
constexpr int NXCD = 8;         // accelerator dies (XCDs), one L2 each

struct __align__(16) Smem {
  uint16_t Ks[BK * KP];      // K tile, [key][c]
  uint16_t Vt[DP * VP];      // V tile transposed, [c][key]
  uint16_t Rs[RROWS * KP];   // r rows of the window union, [row][c], natural order
  float Wb[NW * WBUF];       // position-term windows, one per wave
};

// fp32 -> bf16 bits with the hardware conversion (round to nearest even)
__device__ inline uint16_t bf16_bits(float x) { return __builtin_bit_cast(uint16_t, (__bf16)x); }

__device__ inline bf16x8 lds_b128(const uint16_t* p) { return *(const bf16x8*)p; }
__device__ inline bf16x8 lds_2xb64(const uint16_t* p0, const uint16_t* p1) {
  const bf16x4 a = *(const bf16x4*)p0, b = *(const bf16x4*)p1;
  return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Column mask of a 16-byte chunk starting at column c0: all-ones words for
// columns < d, zero words past d (d is not necessarily a multiple of 8).
__device__ inline uint4 chunk_mask(int c0, int d) {
  uint32_t w[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const uint32_t lo = (c0 + 2 * e < d) ? 0x0000ffffu : 0u;
    const uint32_t hi = (c0 + 2 * e + 1 < d) ? 0xffff0000u : 0u;
    w[e] = lo | hi;
  }
  return make_uint4(w[0], w[1], w[2], w[3]);
}
__device__ inline uint4 and4(uint4 a, uint4 m, bool keep) {
  const uint32_t k = keep ? 0xffffffffu : 0u;
  return make_uint4(a.x & m.x & k, a.y & m.y & k, a.z & m.z & k, a.w & m.w & k);
}

// Registers holding one key tile on its way from HBM to LDS.  The loads are
// unconditional (addresses clamped into the tensor); rows and columns that
// are out of range are zeroed when the tile is written to LDS, after the wait
// that the write needs anyway, so no load is waited for early.
struct TileRegs {
  uint4 k[2];  // two 16B chunks of K
  uint4 v[2];  // V rows 2p and 2p+1, chunk cv
  uint4 r[6];  // six 16B chunks of the r window
};

struct TileGeom {
  const uint16_t* kb;
  const uint16_t* vb;
  const uint16_t* rb;
  int kv_st, r_sp;  // strides (elements)
  int T;            // keys
  int cl_max;       // last loadable chunk index (d_load / 8 - 1)
};

__device__ inline void load_tile(TileRegs& tr, const TileGeom& g, int j0, int dist_lo, int tid) {
  const int c = tid & 7;
  const int cl = c < g.cl_max ? c : g.cl_max;
#pragma unroll
  for (int x = 0; x < 2; ++x) {
    const int j = j0 + (tid >> 3) + 32 * x;
    const int jc = j < g.T ? j : g.T - 1;
    tr.k[x] = *(const uint4*)(g.kb + (int64_t)jc * g.kv_st + 8 * cl);
  }
  // V: key pair p = tid & 31 (fastest, so the transposed LDS writes are
  // conflict-free), chunk cv = tid >> 5
  const int cv = tid >> 5;
  const int cvl = cv < g.cl_max ? cv : g.cl_max;
#pragma unroll
  for (int x = 0; x < 2; ++x) {
    const int j = j0 + 2 * (tid & 31) + x;
    const int jc = j < g.T ? j : g.T - 1;
    tr.v[x] = *(const uint4*)(g.vb + (int64_t)jc * g.kv_st + 8 * cvl);
  }
#pragma unroll
  for (int x = 0; x < 6; ++x) {
    const int dist = dist_lo + (tid >> 3) + 32 * x;
    const int dc = dist < 0 ? 0 : (dist < g.T ? dist : g.T - 1);
    tr.r[x] = *(const uint4*)(g.rb + (int64_t)dc * g.r_sp + 8 * cl);
  }
}

__device__ inline void store_tile(Smem& sm, const TileRegs& tr, const TileGeom& g, uint4 cmask,
                                  uint4 cmask_v, bool full_cols, int j0, int dist_lo, int tid) {
  const int c = tid & 7;
  const int p = tid & 31, cv = tid >> 5;
  // interior tile with all 64 columns live: no masking at all (wave-uniform)
  if (full_cols && j0 + BK <= g.T && dist_lo >= 0 && dist_lo + RROWS <= g.T) {
#pragma unroll
    for (int x = 0; x < 2; ++x)
      *(uint4*)&sm.Ks[((tid >> 3) + 32 * x) * KP + 8 * c] = tr.k[x];
    const uint32_t* v0 = (const uint32_t*)&tr.v[0];
    const uint32_t* v1 = (const uint32_t*)&tr.v[1];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      *(uint32_t*)&sm.Vt[(8 * cv + 2 * w) * VP + 2 * p] = (v0[w] & 0xffffu) | (v1[w] << 16);
      *(uint32_t*)&sm.Vt[(8 * cv + 2 * w + 1) * VP + 2 * p] = (v0[w] >> 16) | (v1[w] & 0xffff0000u);
    }
#pragma unroll
    for (int x = 0; x < 6; ++x)
      *(uint4*)&sm.Rs[((tid >> 3) + 32 * x) * KP + 8 * c] = tr.r[x];
    return;
  }
#pragma unroll
  for (int x = 0; x < 2; ++x) {
    const int key = (tid >> 3) + 32 * x;
    *(uint4*)&sm.Ks[key * KP + 8 * c] = and4(tr.k[x], cmask, j0 + key < g.T);
  }
  {
    const uint4 a0 = and4(tr.v[0], cmask_v, j0 + 2 * p < g.T);
    const uint4 a1 = and4(tr.v[1], cmask_v, j0 + 2 * p + 1 < g.T);
    const uint32_t* v0 = (const uint32_t*)&a0;
    const uint32_t* v1 = (const uint32_t*)&a1;
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
    const int row = (tid >> 3) + 32 * x;
    const int dist = dist_lo + row;
    *(uint4*)&sm.Rs[row * KP + 8 * c] = and4(tr.r[x], cmask, dist >= 0 && dist < g.T);
  }
}

__global__ __launch_bounds__(256, 2) void attn_mfma_kernel(AttnArgs a, int nqt, int groups) {
  extern __shared__ __align__(16) char smem_raw[];
  Smem& sm = *(Smem*)smem_raw;

  // Workgroups are dispatched to the 8 XCDs round-robin by id, and each XCD has
  // its own L2.  Block id n runs on XCD n % 8 as its (n / 8)-th block; that
  // XCD takes the (batch, head) groups g = x, x + 8, ... with their query tiles
  // consecutive and longest first, so the tiles of a group run together on
  // one L2 and share its K, V and r.  With a key split, the nsplit workgroups
  // of one query tile are consecutive as well.
  const int nsplit = a.nsplit;
  const int nper = nqt * nsplit;
  const int xcd = blockIdx.x % NXCD, k_on = blockIdx.x / NXCD;
  const int g = (k_on / nper) * NXCD + xcd;
  const int qt = nqt - 1 - (k_on % nper) / nsplit;
  const int split = (k_on % nper) % nsplit;
  if (g >= groups) return;
  const int64_t b = g / a.H, hd = g % a.H;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int li = lane & 31, lh = lane >> 5;
  const int d = (int)a.d;
  const int L = (int)a.L, len = (int)a.mem_len, T = len + L;
  const int q0 = qt * BQ;
  const int i0w = q0 + wave * BQW;

  TileGeom tg;
  tg.kb = (const uint16_t*)a.k + b * a.kv_sb + hd * a.kv_sh;
  tg.vb = (const uint16_t*)a.v + b * a.kv_sb + hd * a.kv_sh;
  tg.rb = (const uint16_t*)a.r + hd * a.r_sh;
  tg.kv_st = (int)a.kv_st;
  tg.r_sp = (int)a.r_sp;
  tg.T = T;
  tg.cl_max = (int)(a.d_load / 8) - 1;
  const uint4 cmask = chunk_mask(8 * (tid & 7), d);
  const uint4 cmask_v = chunk_mask(8 * (tid >> 5), d);
  const bool full_cols = d == DP;

  // key tiles of this workgroup: all tiles up to the last query's last key,
  // or this split's share of them
  const int imax_wg = (q0 + BQ - 1 < L - 1) ? q0 + BQ - 1 : L - 1;
  const int n_kt = (len + imax_wg) / BK + 1;
  const int kt_lo = (split * n_kt) / nsplit, kt_hi = ((split + 1) * n_kt) / nsplit;
  const bool wave_has_rows = i0w < L;
  const int imax_w = (i0w + BQW - 1 < L - 1) ? i0w + BQW - 1 : L - 1;
  const int kt_w = wave_has_rows ? (len + imax_w) / BK : -1;

  TileRegs tr;
  if (kt_lo < kt_hi) load_tile(tr, tg, kt_lo * BK, len + q0 - kt_lo * BK - BK, tid);

  // ---- this lane's query (column li of the MFMA B operand), pre-scaled ----------
  bf16x8 qc[4], qp[4];
  {
    const int i = i0w + li;
    const int ic = i < L ? i : L - 1;
    const uint16_t* qrow = (const uint16_t*)a.q + b * a.q_sb + (int64_t)ic * a.q_st + hd * a.q_sh;
    const uint16_t* ur = (const uint16_t*)a.u + hd * d;
    const uint16_t* vr = (const uint16_t*)a.vb + hd * d;
    const float sl2 = a.scale * LOG2E;
    // u and v rows: 16-byte loads when they are aligned, else element by element
    const bool uv_vec = (d % 8 == 0) && ((((uintptr_t)a.u) | ((uintptr_t)a.vb)) % 16 == 0);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int c0 = 16 * s + 8 * lh;
      const int cc = c0 / 8 < tg.cl_max ? c0 : 8 * tg.cl_max;
      const uint4 raw = *(const uint4*)(qrow + cc);
      const uint16_t* rv = (const uint16_t*)&raw;
      uint16_t uh[8], vh[8];
      if (uv_vec && c0 < d) {
        *(uint4*)uh = *(const uint4*)(ur + c0);
        *(uint4*)vh = *(const uint4*)(vr + c0);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          uh[e] = c0 + e < d ? ur[c0 + e] : (uint16_t)0;
          vh[e] = c0 + e < d ? vr[c0 + e] : (uint16_t)0;
        }
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const bool ok = c0 + e < d && i < L;
        const float x = bf16_to_f32(rv[e]);
        qc[s][e] = (__bf16)(ok ? (x + bf16_to_f32(uh[e])) * sl2 : 0.f);
        qp[s][e] = (__bf16)(ok ? (x + bf16_to_f32(vh[e])) * sl2 : 0.f);
      }
    }
  }

  float m_run = -INFINITY, l_run = 0.f;
  f32x16 acc[2];
#pragma unroll
  for (int x = 0; x < 16; ++x) { acc[0][x] = 0.f; acc[1][x] = 0.f; }

  float* wb = sm.Wb + wave * WBUF;
  float* srow_base = nullptr;
  if (a.scores) srow_base = a.scores + ((b * a.H + hd) * a.L) * (int64_t)T;

  for (int kt = kt_lo; kt < kt_hi; ++kt) {
    const int j0 = kt * BK;
    __syncthreads();
    store_tile(sm, tr, tg, cmask, cmask_v, full_cols, j0, len + q0 - j0 - BK, tid);
    __syncthreads();
    if (kt + 1 < kt_hi) load_tile(tr, tg, j0 + BK, len + q0 - j0 - 2 * BK, tid);
    if (kt > kt_w) continue;

    const int Dw = len + i0w - j0;  // distance of (query 0, key 0) of this wave's tile

    // ---- position term: W^T[w''][ii] = r[Dw + 31 - w''] . qp[ii], w'' in [0, 96) ----
    // A-row li of block blk is distance Dw + 31 - 32 blk - li, staged at row
    // dist - (len + q0 - j0 - 64), which lies in [0, 191].
    {
      f32x16 w[3];
#pragma unroll
      for (int blk = 0; blk < 3; ++blk)
#pragma unroll
        for (int x = 0; x < 16; ++x) w[blk][x] = 0.f;
      // all twelve A fragments first, so their LDS latency overlaps
      bf16x8 ar[3][4];
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int blk = 0; blk < 3; ++blk)
          ar[blk][s] = lds_b128(&sm.Rs[(BQW * wave + 95 - 32 * blk - li) * KP + 16 * s + 8 * lh]);
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int blk = 0; blk < 3; ++blk)
          w[blk] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ar[blk][s], qp[s], w[blk], 0, 0, 0);
      // lane (query li, half lh), reg x -> window index w'' = 32 blk + 8 (x/4) + 4 lh + x%4;
      // row li reads w'' in [31 - li, 94 - li] only, and only those are written:
      // all of block 1, the part of block 0 with w'' >= 31 - li and the part of
      // block 2 with w'' <= 94 - li.  The other values of blocks 0 and 2 go to a
      // per-lane dump slot (floats 0..31 of the buffer are never read), which
      // keeps the writes branch-free.
      float* wrow = wb + 1 + li * WP + 4 * lh;
      float* dump = wb + li;
      const int c_l = li + 4 * lh;
#pragma unroll
      for (int x = 0; x < 16; ++x) {
        const int off = 8 * (x >> 2) + (x & 3);
        wrow[32 + off] = w[1][x];
        *(c_l + off >= 31 ? wrow + off : dump) = w[0][x];
        *(c_l + off <= 30 ? wrow + 64 + off : dump) = w[2][x];
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    // ---- content term with the gathered position term as accumulator ------------
    f32x16 sc[2];
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
      for (int x4 = 0; x4 < 4; ++x4) {
        // keys jj = 32 kb2 + 8 x4 + 4 lh + t, t = 0..3 -> flat 32 + 100 li + jj
        const f32x4 sp = *(const f32x4*)&wb[32 + (WP - 1) * li + 32 * kb2 + 8 * x4 + 4 * lh];
#pragma unroll
        for (int t = 0; t < 4; ++t) sc[kb2][4 * x4 + t] = sp[t];
      }
    {
      bf16x8 ak[2][4];
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2)
          ak[kb2][s] = lds_b128(&sm.Ks[(32 * kb2 + li) * KP + 16 * s + 8 * lh]);
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2)
          sc[kb2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ak[kb2][s], qc[s], sc[kb2], 0, 0, 0);
    }

    // ---- causal mask (tiles that reach past the wave's first query only) --------
    if (j0 + BK - 1 > len + i0w) {
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
        for (int x = 0; x < 16; ++x) {
          const int jj = 32 * kb2 + 8 * (x >> 2) + 4 * lh + (x & 3);
          sc[kb2][x] = (jj - li > Dw) ? -INFINITY : sc[kb2][x];
        }
    }
    if (srow_base) {
      const int i = i0w + li;
      if (i < L) {
        float* srow = srow_base + (int64_t)i * T;
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
          for (int x = 0; x < 16; ++x) {
            const int j = j0 + 32 * kb2 + 8 * (x >> 2) + 4 * lh + (x & 3);
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
    // a split's tiles can hide every key of a query so far: keep the max at
    // -inf then, with zero weights and no NaN from (-inf) - (-inf)
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
    m_run = m_new;
    float psum = 0.f;
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
      for (int x = 0; x < 16; ++x) {
        const float p = __builtin_amdgcn_exp2f(sc[kb2][x] - m_use);
        sc[kb2][x] = p;
        psum += p;
      }
    l_run = l_run * alpha + psum;
    // the running max rarely moves after the first tiles: rescale only if it did
    if (__any(alpha != 1.f)) {
#pragma unroll
      for (int x = 0; x < 16; ++x) {
        acc[0][x] *= alpha;
        acc[1][x] *= alpha;
      }
    }

    // ---- O^T += V^T . P^T ------------------------------------------------------------
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      bf16x8 pb;
      const int kb2 = s >> 1, v0 = 8 * (s & 1);
#pragma unroll
      for (int e = 0; e < 8; ++e) pb[e] = (__bf16)sc[kb2][v0 + e];
      bf16x8 av[2];
#pragma unroll
      for (int db = 0; db < 2; ++db) {
        const uint16_t* vrow = &sm.Vt[(32 * db + li) * VP + 16 * s + 4 * lh];
        av[db] = lds_2xb64(vrow, vrow + 8);
      }
#pragma unroll
      for (int db = 0; db < 2; ++db)
        acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[db], pb, acc[db], 0, 0, 0);
    }
  }

  // ---- epilogue: out[i][c] = acc / l -------------------------------------------------
  if (!wave_has_rows) return;
  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  const int i = i0w + li;
  if (i >= L) return;
  if (nsplit > 1) {
    // unnormalised partial of this split: acc (all 64 columns), max and sum
    const int64_t row = ((int64_t)split * groups + g) * a.L + i;
    float* pa = a.part_acc + row * DP;
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int x4 = 0; x4 < 4; ++x4) {
        const int c = 32 * db + 8 * x4 + 4 * lh;
        *(f32x4*)(pa + c) = {acc[db][4 * x4], acc[db][4 * x4 + 1], acc[db][4 * x4 + 2],
                             acc[db][4 * x4 + 3]};
      }
    if (lh == 0) {
      a.part_ml[2 * row] = m_run;
      a.part_ml[2 * row + 1] = l_tot;
    }
    return;
  }
  const float inv = 1.f / l_tot;
  uint16_t* orow = (uint16_t*)a.out + b * a.o_sb + (int64_t)i * a.o_st + hd * a.o_sh;
  const bool vec = ((d & 3) == 0) && (((uintptr_t)a.out & 7) == 0) && ((a.o_sb & 3) == 0) &&
                   ((a.o_st & 3) == 0) && ((a.o_sh & 3) == 0);
  if (vec) {
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int x4 = 0; x4 < 4; ++x4) {
        const int c = 32 * db + 8 * x4 + 4 * lh;
        if (c < d) {
          uint2 pk;
          pk.x = bf16_bits(acc[db][4 * x4] * inv) |
                 ((uint32_t)bf16_bits(acc[db][4 * x4 + 1] * inv) << 16);
          pk.y = bf16_bits(acc[db][4 * x4 + 2] * inv) |
                 ((uint32_t)bf16_bits(acc[db][4 * x4 + 3] * inv) << 16);
          *(uint2*)(orow + c) = pk;
        }
      }
  } else {
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int x = 0; x < 16; ++x) {
        const int c = 32 * db + 8 * (x >> 2) + 4 * lh + (x & 3);
        if (c < d) orow[c] = bf16_bits(acc[db][x] * inv);
      }
  }
}

// Log-sum-exp merge of the key splits of one (query, batch*head) per wavefront:
//   out = sum_s 2^(m_s - M) acc_s / sum_s 2^(m_s - M) l_s,  M = max_s m_s.
// Split 0 holds key 0, visible to every query, so M is finite.
__global__ __launch_bounds__(64) void attn_split_merge_kernel(AttnArgs a) {
  const int64_t i = blockIdx.x, g = blockIdx.y;
  const int c = threadIdx.x;
  const int64_t G = a.B * a.H;
  float M = -INFINITY;
  for (int s = 0; s < a.nsplit; ++s) M = fmaxf(M, a.part_ml[2 * ((s * G + g) * a.L + i)]);
  float num = 0.f, den = 0.f;
  for (int s = 0; s < a.nsplit; ++s) {
    const int64_t row = (s * G + g) * a.L + i;
    const float w = __builtin_amdgcn_exp2f(a.part_ml[2 * row] - M);
    den += w * a.part_ml[2 * row + 1];
    num += w * a.part_acc[row * DP + c];
  }
  if (c < a.d) {
    const int64_t b = g / a.H, hd = g % a.H;
    uint16_t* orow = (uint16_t*)a.out + b * a.o_sb + i * a.o_st + hd * a.o_sh;
    orow[c] = bf16_bits(num / den);
  }
}

}  // namespace

int attn_mfma_plan_splits(const AttnArgs& a, int num_cus) {
  // split the keys only when the query tiles cannot give every CU two workgroups
  const int64_t nqt = (a.L + BQ - 1) / BQ;
  const int64_t base = nqt * a.B * a.H;
  if (base >= 2LL * num_cus) return 1;
  const int64_t imax0 = (BQ - 1 < a.L - 1) ? BQ - 1 : a.L - 1;
  const int64_t tiles0 = (a.mem_len + imax0) / BK + 1;  // fewest tiles of any query tile
  int64_t ns = (2LL * num_cus + base - 1) / base;
  // at least two key tiles per split: with one, each workgroup's fixed start-up
  // (q, u, v and the first tile) outweighs its work
  if (ns > tiles0 / 2) ns = tiles0 / 2;
  if (ns > 16) ns = 16;
  return ns < 2 ? 1 : (int)ns;
}

size_t attn_split_bytes(const AttnArgs& a, int nsplit) {
  if (nsplit <= 1) return 0;
  const size_t rows = (size_t)nsplit * (size_t)(a.B * a.H) * (size_t)a.L;
  return rows * DP * sizeof(float) + rows * 2 * sizeof(float) + 256;
}

bool attn_mfma_supported(const AttnArgs& a) {
  if (a.d > DP || a.d_load % 8 != 0 || a.d_load > DP) return false;
  if (a.mem_len + a.L > 0x7fffffffLL - 2 * BQ) return false;
  // 32-bit element offsets inside a (batch, head) slab
  if ((a.mem_len + a.L) * (a.kv_st > a.r_sp ? a.kv_st : a.r_sp) > 0x7fffffffLL) return false;
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
  const int nsplit = a.nsplit > 1 ? a.nsplit : 1;
  const int64_t nblocks = (int64_t)nqt * nsplit * NXCD * ((groups + NXCD - 1) / NXCD);
  const size_t smem = sizeof(Smem);
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)attn_mfma_kernel,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  AttnArgs aa = a;
  aa.nsplit = nsplit;
  hipLaunchKernelGGL(attn_mfma_kernel, dim3((unsigned)nblocks), dim3(256), smem, s, aa, nqt,
                     groups);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || nsplit == 1) return e;
  hipLaunchKernelGGL(attn_split_merge_kernel, dim3((unsigned)a.L, (unsigned)groups), dim3(64),
                     0, s, aa);
  return hipGetLastError();
}

}  // namespace txl
