// Relative-position attention over segment-level memory, bf16 matrix-core path
// for gfx950 (Transformer-XL, section 3.3: the A^rel score with terms (a)-(d);
// Appendix B: distances 0 .. M+L-1, key j of query i at distance mem_len+i-j).
//
// One workgroup = 4 waves = 128 queries of one (batch row, head); each wave owns
// 32 queries as two groups of 16 and walks the 64-key tiles up to its last
// visible key with an online softmax in the exp2 domain.  All products are
// v_mfma_f32_16x16x32_bf16.  Per key tile and 16-query group:
//
//   position term  W^T = r_win . Qp^T: the 80 r rows of the distances the tile
//                  can need (16 + 64 - 1, rounded up) against the group's
//                  (q+v).  Lane (g, n) holds four consecutive window rows of
//                  query n; window row rho of query n is the distance of key
//                  jj = rho - 15 + n, so each value is stored in key jj's slot
//                  of a [query][key] LDS buffer (row pitch 68 floats): the
//                  diagonal "relative shift" is a per-lane address offset on
//                  the store side and the reads are aligned 16-byte loads.
//   content term   S^T = K . Qc^T (q+u), accumulated onto the gathered
//                  position term, so the four terms add inside the MFMA.
//   softmax        lane (g, n) holds 16 of query n's 64 scores; row max and the
//                  running sum are kept per lane and combined over the four
//                  lanes of a query (lane xor 16, 32).
//   P.V            O^T = V^T . P^T.  V stays row-major in LDS and its fragments
//                  are read with ds_read_b64_tr_b16 (a transposing LDS read).
//
// K, V and the r rows reach LDS straight from global memory (global_load_lds,
// no register staging).  r lives in a ring of four 64-distance blocks indexed
// by (distance - mem_len) mod 256: successive key tiles move the window by one
// block, so each tile loads only 64 new r rows.  Every 128-byte row stores its
// 16-byte chunk c in slot c ^ ((row >> 1) & 7) (V: c ^ (row & 6)), which keeps
// the fragment reads free of bank conflicts.
//
// The scale 1/sqrt(d) and log2(e) are folded into (q+u) and (q+v) before they
// are rounded to bf16, so the softmax is exp2(S - max) with no extra multiply.
#include "txl_internal.h"

#include <algorithm>
#include <atomic>
#include <functional>
#include <mutex>
#include <vector>

namespace txl {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef short v4s __attribute__((ext_vector_type(4)));

constexpr int NW = 4;           // waves per workgroup
constexpr int BQW = 32;         // queries per wave (two groups of 16)
constexpr int BQ = NW * BQW;    // queries per workgroup
constexpr int BK = 64;          // keys per tile
constexpr int DP = 64;          // head size padded for the MFMA k-loop
constexpr int RRING = 4 * BK;   // r ring rows (four 64-distance blocks)
constexpr int WGF = 16 * 64;    // a wave's S_p buffer (floats): 16 queries x 64 keys
constexpr float LOG2E = 1.4426950408889634f;
constexpr int NXCD = 8;         // accelerator dies (XCDs), one L2 each
#ifndef TXL_ATTN_SCHED
#define TXL_ATTN_SCHED 1
#endif

// 80 KB: two workgroups fill a CU's 160 KB.
struct __align__(16) Smem {
  uint16_t K[2][BK * DP];    // key tiles (double-buffered), [key][c], swizzled 16-byte chunks
  uint16_t V[2][BK * DP];    // value tiles (double-buffered), [key][c], swizzled
  uint16_t R[RRING * DP];    // r ring, row (distance - mem_len) mod 256, swizzled
  float W[NW][WGF];          // gathered position term of one 16-query group, per wave
};

// fp32 -> bf16 bits with the hardware conversion (round to nearest even)
__device__ inline uint16_t bf16_bits(float x) { return __builtin_bit_cast(uint16_t, (__bf16)x); }
// two floats -> packed bf16 pair (low half = lo), one v_cvt_pk_bf16_f32
__device__ inline uint32_t pack2(float lo, float hi) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){lo, hi}, bf16x2));
}

// The LDS has 64 banks of 4 bytes; a 128-byte row covers half of them.
// 16-byte slot of chunk c in row r of K and r: c ^ swz(r) (16 consecutive rows
// read at one chunk hit 16 distinct 16-byte bank groups).
__device__ inline int swz(int r) { return (r >> 1) & 7; }
// V: c ^ swzv(r).  A transposing read of 8 rows x 4 eight-byte pieces (two
// chunks) is conflict-free when the rows of one parity use four different
// chunk pairs.
__device__ inline int swzv(int r) { return r & 6; }

__device__ inline void dma16(const uint16_t* src, uint16_t* lds) {
  __builtin_amdgcn_global_load_lds((const void __attribute__((address_space(1)))*)src,
                                   (void __attribute__((address_space(3)))*)lds, 16, 0, 0);
}
__device__ inline void wait_dma() { __builtin_amdgcn_s_waitcnt(0x3f70); }  // vmcnt(0)
// Workgroup barrier for LDS written by this workgroup's waves and for the
// LDS-direct loads each wave has already waited for.
__device__ inline void barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n s_barrier" ::: "memory"); }

__device__ inline bf16x8 lds_b128(const uint16_t* p) { return *(const bf16x8*)p; }
__device__ inline bf16x8 lds_tr2(const uint16_t* p0, const uint16_t* p1) {
  const v4s a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s*)p0);
  const v4s b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s*)p1);
  const v4s ab[2] = {a, b};
  return *(const bf16x8*)ab;
}
// Reductions over the lanes n, n + 16, n + 32, n + 48 (one query of a 16 x 16
// block) with the gfx950 lane-swap instructions: permlane16_swap(v, v) yields the
// value of lane ^ 16 in one of its two results, permlane32_swap that of lane ^ 32.
__device__ inline float max4(float x) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  auto p = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  x = fmaxf(__builtin_bit_cast(float, (uint32_t)p[0]), __builtin_bit_cast(float, (uint32_t)p[1]));
  const uint32_t w = __builtin_bit_cast(uint32_t, x);
  auto q = __builtin_amdgcn_permlane32_swap(w, w, false, false);
  return fmaxf(__builtin_bit_cast(float, (uint32_t)q[0]), __builtin_bit_cast(float, (uint32_t)q[1]));
}
__device__ inline float sum4(float x) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  auto p = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  x = __builtin_bit_cast(float, (uint32_t)p[0]) + __builtin_bit_cast(float, (uint32_t)p[1]);
  const uint32_t w = __builtin_bit_cast(uint32_t, x);
  auto q = __builtin_amdgcn_permlane32_swap(w, w, false, false);
  return __builtin_bit_cast(float, (uint32_t)q[0]) + __builtin_bit_cast(float, (uint32_t)q[1]);
}
__device__ inline f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// ---- pieces shared by the 128- and the 64-query kernels -------------------------------

// LDS-direct loads of one (batch, head)'s key, value and r rows.  Instruction x
// (0, 1) of a wave fills tile rows 16 wave + 8 x .. + 7: lane -> row + lane / 8,
// 16-byte slot lane % 8 (chunk slot ^ swz, V: ^ swzv); chunks past d_load repeat
// a real one (times q = 0).  Interior tiles address from a uniform tile base
// plus the lane's fixed offset; rows past the ends are clamped (they feed masked
// scores only).  Keys may sit in a ring (row (kv_start + j) % kv_cap); without
// one the cap is past every key, so the row is j.
struct TileLoads {
  const uint16_t *kb, *vb, *rb;
  int kv_st, r_sp, T, len, kvs, kvc, wave;
  int drow[2], dch[2], dchv[2], ko[2], vo[2], ro[2];

  __device__ TileLoads(const AttnArgs& a, int64_t b, int64_t hd, int wave_, int lane) {
    kb = (const uint16_t*)a.k + b * a.kv_sb + hd * a.kv_sh;
    vb = (const uint16_t*)a.v + b * a.kv_sb + hd * a.kv_sh;
    rb = (const uint16_t*)a.r + hd * a.r_sh;
    kv_st = (int)a.kv_st;
    r_sp = (int)a.r_sp;
    len = (int)a.mem_len;
    T = len + (int)a.L;
    kvs = a.kv_cap > 0 ? (int)a.kv_start : 0;
    kvc = a.kv_cap > 0 ? (int)a.kv_cap : 0x7fffffff - BK;
    wave = wave_;
    const int cl_max = (int)(a.d_load / 8) - 1;  // last readable 16-byte chunk of a row
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      drow[x] = 16 * wave + 8 * x + (lane >> 3);
      const int c = (lane & 7) ^ swz(drow[x]), cv = (lane & 7) ^ swzv(drow[x]);
      dch[x] = 8 * (c < cl_max ? c : cl_max);
      dchv[x] = 8 * (cv < cl_max ? cv : cl_max);
      ko[x] = drow[x] * kv_st + dch[x];  // this lane's element offsets within a tile
      vo[x] = drow[x] * kv_st + dchv[x];
      ro[x] = drow[x] * r_sp + dch[x];
    }
  }
  __device__ void kv(const uint16_t* base, uint16_t* lds, int j0, const int (&off)[2],
                     const int (&ch)[2]) const {
    int p0 = kvs + j0;
    p0 = p0 >= kvc ? p0 - kvc : p0;
    if (j0 + BK <= T && p0 + BK <= kvc) {
      const uint16_t* tb = base + p0 * kv_st;
#pragma unroll
      for (int x = 0; x < 2; ++x) dma16(tb + off[x], lds + (16 * wave + 8 * x) * DP);
    } else {
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        const int j = j0 + drow[x] < T ? j0 + drow[x] : T - 1;
        int p = kvs + j;
        p = p >= kvc ? p - kvc : p;
        dma16(base + p * kv_st + ch[x], lds + (16 * wave + 8 * x) * DP);
      }
    }
  }
  // keys j0 .. j0 + 63 into a K or a V tile
  __device__ void k(uint16_t* lds, int j0) const { kv(kb, lds, j0, ko, dch); }
  __device__ void v(uint16_t* lds, int j0) const { kv(vb, lds, j0, vo, dchv); }
  // r rows of relative distances e0 .. e0 + 63 (e = distance - mem_len, e0 % 64 ==
  // 0) into a ring of RING rows indexed by e mod RING
  template <int RING>
  __device__ void r(uint16_t* ring, int e0) const {
    uint16_t* dst = ring + ((e0 & (RING - 1)) + 16 * wave) * DP;
    const int dist0 = len + e0;
    if (dist0 >= 0 && dist0 + BK <= T) {
      const uint16_t* tb = rb + dist0 * r_sp;
#pragma unroll
      for (int x = 0; x < 2; ++x) dma16(tb + ro[x], dst + 8 * x * DP);
    } else {
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        int dist = dist0 + drow[x];
        dist = dist < 0 ? 0 : (dist < T ? dist : T - 1);
        dma16(rb + dist * r_sp + dch[x], dst + 8 * x * DP);
      }
    }
  }
};

// K fragment (16x16x32 A operand) of k-step s: row 16 kb + n16, chunk 4 s + g4
__device__ inline int k_frag(int n16, int g4, int s) { return n16 * DP + 8 * ((4 * s + g4) ^ swz(n16)); }
// V^T through transposing reads: lane (g4, n16) of a 16-lane group reads key row
// 4 g4 + n16 / 4 (+ 32 h + 16 kb'), columns 16 db + 4 (n16 % 4) .. + 3
__device__ inline int v_frag(int n16, int g4, int db) {
  const int vrow = 4 * g4 + (n16 >> 2);
  const int piece = 4 * db + (n16 & 3);  // 8-byte piece of the row
  return vrow * DP + 8 * ((piece >> 1) ^ swzv(vrow)) + 4 * (piece & 1);
}

// (q_i + u) and (q_i + v) of query i as the B operands of k-steps 0 and 1 (lane
// (g4, n16): columns 32 s + 8 g4 .. + 7), scaled by scale * log2(e) before they
// are rounded to bf16; zero past d and for i >= L.
__device__ inline void query_operands(const AttnArgs& a, int64_t b, int64_t hd, int i, int g4,
                                      bf16x8 (&qc)[2], bf16x8 (&qp)[2]) {
  const int d = (int)a.d, L = (int)a.L;
  const int cl_max = (int)(a.d_load / 8) - 1;
  const uint16_t* ur = (const uint16_t*)a.u + hd * d;
  const uint16_t* vr = (const uint16_t*)a.vb + hd * d;
  const float sl2 = a.scale * LOG2E;
  const bool uv_vec = (d % 8 == 0) && ((((uintptr_t)a.u) | ((uintptr_t)a.vb)) % 16 == 0);
  const int ic = i < L ? i : L - 1;
  const uint16_t* qrow = (const uint16_t*)a.q + b * a.q_sb + (int64_t)ic * a.q_st + hd * a.q_sh;
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const int c0 = 32 * s + 8 * g4;
    const int cc = c0 / 8 < cl_max ? c0 : 8 * cl_max;
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

// out[i][c] = acc * inv for query i < L: lane (g4, n16) of block db holds columns
// 16 db + 4 g4 .. + 3
__device__ inline void write_out(const AttnArgs& a, int64_t b, int64_t hd, int i, int g4,
                                 const f32x4 (&acc)[4], float inv) {
  const int d = (int)a.d;
  uint16_t* orow = (uint16_t*)a.out + b * a.o_sb + (int64_t)i * a.o_st + hd * a.o_sh;
  const bool vec = ((d & 3) == 0) && (((uintptr_t)a.out & 7) == 0) && ((a.o_sb & 3) == 0) &&
                   ((a.o_st & 3) == 0) && ((a.o_sh & 3) == 0);
#pragma unroll
  for (int db = 0; db < 4; ++db) {
    const int c = 16 * db + 4 * g4;
    if (vec) {
      if (c < d)
        *(uint2*)(orow + c) = make_uint2(pack2(acc[db][0] * inv, acc[db][1] * inv),
                                         pack2(acc[db][2] * inv, acc[db][3] * inv));
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (c + e < d) orow[c + e] = bf16_bits(acc[db][e] * inv);
    }
  }
}

// LSE: also write each query's log-sum-exp (AttnArgs::lse).  A separate
// instantiation, so the plain forward's code is untouched by it.
template <bool LSE>
__global__ __launch_bounds__(256, 2) void attn_mfma_kernel(AttnArgs a, int nqt, int groups) {
  extern __shared__ __align__(16) char smem_raw[];
  Smem& sm = *(Smem*)smem_raw;

  // Workgroups are dispatched to the 8 XCDs round-robin by id, and each XCD has
  // its own L2.  Block id n runs on XCD n % 8 as its (n / 8)-th block; XCD x
  // owns the (batch, head) groups g = x, x + 8, ..., so their K, V and r stay in
  // one L2.  Each XCD issues the plan's work classes in order (all its groups of
  // one class, then the next): the longest parts start first and the short ones
  // fill the tail.
  const int gpx = (groups + NXCD - 1) / NXCD;  // groups per XCD
  const int xcd = blockIdx.x % NXCD, k_on = blockIdx.x / NXCD;
  const int cls = k_on / gpx;
  const int g = (k_on % gpx) * NXCD + xcd;
  const int qt = a.plan.ncls > 0 ? a.plan.cls_qt[cls] : nqt - 1 - cls;
  const int part = a.plan.ncls > 0 ? a.plan.cls_part[cls] : 0;
  const int nparts = a.plan.ncls > 0 ? a.plan.nparts[qt] : 1;
  if (g >= groups) return;
  const int64_t b = g / a.H, hd = g % a.H;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar address math
  const int g4 = lane >> 4, n16 = lane & 15;  // 16x16 MFMA lane coordinates
  const int L = (int)a.L, len = (int)a.mem_len, T = len + L;
  const int q0 = qt * BQ;
  const int i0w = q0 + wave * BQW;

  // key tiles of this workgroup: all tiles up to the last query's last key,
  // or this part's share of them
  const int imax_wg = (q0 + BQ - 1 < L - 1) ? q0 + BQ - 1 : L - 1;
  const int n_kt = (len + imax_wg) / BK + 1;
  const int kt_lo = (part * n_kt) / nparts, kt_hi = ((part + 1) * n_kt) / nparts;
  const bool wave_has_rows = i0w < L;
  const int imax_w = (i0w + BQW - 1 < L - 1) ? i0w + BQW - 1 : L - 1;
  const int kt_w = wave_has_rows ? (len + imax_w) / BK : -1;

  const TileLoads ld(a, b, hd, wave, lane);

  // ---- fragment offsets (elements / floats), fixed for the whole walk -----------------
  int koff[2], voff[4];
#pragma unroll
  for (int s = 0; s < 2; ++s) koff[s] = k_frag(n16, g4, s);
#pragma unroll
  for (int db = 0; db < 4; ++db) voff[db] = v_frag(n16, g4, db);
  // Gathered position term S_p[query n][key jj] of one 16-query group: row n of
  // 64 floats, 16-byte chunk c of it in slot (c + 4 n + 3 (n / 4)) % 16.  Both
  // the 16-byte reads (16 queries at one chunk) and the 4-byte stores (64 lanes,
  // 64 distinct banks for every (bw, e)) are then free of bank conflicts.  Lane
  // (g4, n16) holds window rows 16 bw + 4 g4 + e of query n16, window row rho
  // being the distance of key jj = rho - 15 + n16.
  float* const wbuf = sm.W[wave];
  const int sprot = 4 * n16 + 3 * (n16 >> 2);
  auto sp_slot = [&](int jj) { return n16 * 64 + ((((jj >> 2) + sprot) & 15) << 2) + (jj & 3); };
  // r fragments: union block u (0..5) of the wave's 96 window rows, row rho =
  // n16 is relative distance i0w - j0 + 31 - 16 u - n16, stored at ring row
  // (that) mod 256; roff[u] is its s = 0 offset, s = 1 is roff[u] ^ 32.
  int roff[6];

  // ---- first tile: K, V and the three r blocks of its window (issued before the
  //      query loads, so the two global round trips overlap) -----------------------
  if (kt_lo < kt_hi) {
    const int j0 = kt_lo * BK;
    ld.k(sm.K[kt_lo & 1], j0);
    ld.v(sm.V[kt_lo & 1], j0);
#pragma unroll
    for (int blk = 0; blk < 3; ++blk) ld.r<RRING>(sm.R, q0 - j0 - BK + BK * blk);
    // ring offsets of the union blocks for this tile
#pragma unroll
    for (int u = 0; u < 6; ++u) {
      const int e = i0w - j0 + 31 - 16 * u - n16;
      const int rr = e & (RRING - 1);
      roff[u] = rr * DP + 8 * (g4 ^ swz(rr));
    }
  }

  // ---- this lane's queries, pre-scaled: group gm holds query i0w + 16 gm + n16,
  //      k-step s columns 32 s + 8 g4 .. + 7 ---------------------------------------------
  bf16x8 qc[2][2], qp[2][2];
#pragma unroll
  for (int gm = 0; gm < 2; ++gm) query_operands(a, b, hd, i0w + 16 * gm + n16, g4, qc[gm], qp[gm]);

  // Softmax state per query: the reference s_off that the position product
  // subtracts from every score through its accumulator's initial value (so the
  // scores arrive as S - s_off and P = exp2 of them), and lim, how far above
  // s_off a score may go before the reference moves: -inf until the query has
  // seen a key, then TAU.  The reference is a maximum of the scores seen when it
  // was set, so P stays below 2^TAU and moves are rare.  acc_l accumulates the
  // row sums of P with the matrix core (a ones operand).
  constexpr float TAU = 8.f;
  float s_off[2] = {0.f, 0.f}, lim[2] = {-INFINITY, -INFINITY};
  f32x4 acc[2][4], acc_l[2];
#pragma unroll
  for (int gm = 0; gm < 2; ++gm) {
    acc_l[gm] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int db = 0; db < 4; ++db) acc[gm][db] = {0.f, 0.f, 0.f, 0.f};
  }
  const bf16x8 ones = __builtin_bit_cast(bf16x8, make_uint4(0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u));

  float* srow_base = nullptr;
  if (a.scores) srow_base = a.scores + ((b * a.H + hd) * a.L) * (int64_t)T;

  // One barrier per tile.  At the top of tile kt every wave has waited for its
  // own loads of tile kt, and the barrier makes them visible and retires tile
  // kt - 1 in every wave; then tile kt + 1's K and V go to the other buffers and
  // its new r block to the ring slot only tile kt - 1 used, so the loads run a
  // whole tile ahead of their use.
  for (int kt = kt_lo; kt < kt_hi; ++kt) {
    const int j0 = kt * BK;
    wait_dma();
    barrier();
    if (kt + 1 < kt_hi) {
      ld.k(sm.K[(kt + 1) & 1], j0 + BK);
      ld.v(sm.V[(kt + 1) & 1], j0 + BK);
      ld.r<RRING>(sm.R, q0 - j0 - 2 * BK);  // the block the next tile adds
    }
    const uint16_t* Kt = sm.K[kt & 1];
    const uint16_t* Vt = sm.V[kt & 1];
    const bool work = kt <= kt_w;
    const int Dw = len + i0w - j0;  // distance of (query i0w, key j0)
    f32x4 sc[2][4];
    if (work) {
      // ---- r and K fragments first, so their LDS latency overlaps ---------------------
      bf16x8 rf[6][2], kf[4][2];
#pragma unroll
      for (int u = 0; u < 6; ++u) {
        rf[u][0] = lds_b128(sm.R + roff[u]);
        rf[u][1] = lds_b128(sm.R + (roff[u] ^ 32));
      }
#pragma unroll
      for (int kbk = 0; kbk < 4; ++kbk)
#pragma unroll
        for (int s = 0; s < 2; ++s) kf[kbk][s] = lds_b128(Kt + kbk * 16 * DP + koff[s]);
      // ---- position terms of both groups; group 1's products run while group 0's
      //      shifted stores and reads go through LDS --------------------------------------
      f32x4 wv[2][5];
      auto pos = [&](int gm) {
#pragma unroll
        for (int bw = 0; bw < 5; ++bw) {
          const int u = bw + 1 - gm;
          f32x4 w = {-s_off[gm], -s_off[gm], -s_off[gm], -s_off[gm]};
          w = mfma(rf[u][0], qp[gm][0], w);
          wv[gm][bw] = mfma(rf[u][1], qp[gm][1], w);
        }
      };
      auto store_w = [&](int gm) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int jj = 4 * g4 + e - 15 + n16;  // key of block 0, in -15 .. 15
          wbuf[sp_slot(jj & (BK - 1))] = jj >= 0 ? wv[gm][0][e] : wv[gm][4][e];
        }
#pragma unroll
        for (int bw = 1; bw < 4; ++bw)
#pragma unroll
          for (int e = 0; e < 4; ++e) wbuf[sp_slot(16 * bw + 4 * g4 + e - 15 + n16)] = wv[gm][bw][e];
      };
      f32x4 cw[2][4];
      auto read_w = [&](int gm) {
#pragma unroll
        for (int kbk = 0; kbk < 4; ++kbk)
          cw[gm][kbk] = *(const f32x4*)(wbuf + n16 * 64 + (((4 * kbk + g4 + sprot) & 15) << 2));
      };
      pos(0);
      store_w(0);
      pos(1);
      read_w(0);
      store_w(1);  // (after group 0's reads: one wave's LDS operations complete in order)
      read_w(1);
#pragma unroll
      for (int gm = 0; gm < 2; ++gm)
#pragma unroll
        for (int kbk = 0; kbk < 4; ++kbk) {
          f32x4 c = cw[gm][kbk];
          c = mfma(kf[kbk][0], qc[gm][0], c);
          c = mfma(kf[kbk][1], qc[gm][1], c);
          sc[gm][kbk] = c;
        }
    }
    // the next tile's union blocks sit one ring block lower
#pragma unroll
    for (int u = 0; u < 6; ++u) roff[u] = (roff[u] - BK * DP) & (RRING * DP - 1);
    if (!work) continue;

    // ---- causal mask (tiles that reach past the wave's first query only) --------------
    if (j0 + BK - 1 > len + i0w) {
#pragma unroll
      for (int gm = 0; gm < 2; ++gm)
#pragma unroll
        for (int kbk = 0; kbk < 4; ++kbk)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int jj = 16 * kbk + 4 * g4 + e;
            sc[gm][kbk][e] = (jj - n16 > Dw + 16 * gm) ? -INFINITY : sc[gm][kbk][e];
          }
    }
    if (srow_base) {
#pragma unroll
      for (int gm = 0; gm < 2; ++gm) {
        const int i = i0w + 16 * gm + n16;
        if (i < L) {
          float* srow = srow_base + (int64_t)i * T;
#pragma unroll
          for (int kbk = 0; kbk < 4; ++kbk)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int j = j0 + 16 * kbk + 4 * g4 + e;
              if (j < T) srow[j] = (sc[gm][kbk][e] + s_off[gm]) * (1.0f / LOG2E);
            }
        }
      }
    }

    // ---- online softmax (exp2 domain); query n16 of group gm lives in lanes
    //      n16 + 16 g4, g4 = 0..3.  The scores are S - s_off.  While none exceeds
    //      its query's limit (the common case after the first tile) P = exp2 of
    //      them as they are; otherwise the queries over their limit move s_off to
    //      their new maximum and rescale what they have accumulated. ---------------
    float lmax[2];
#pragma unroll
    for (int gm = 0; gm < 2; ++gm) {
      lmax[gm] = -INFINITY;
#pragma unroll
      for (int kbk = 0; kbk < 4; ++kbk)
#pragma unroll
        for (int e = 0; e < 4; ++e) lmax[gm] = fmaxf(lmax[gm], sc[gm][kbk][e]);
    }
    if (__any(lmax[0] > lim[0] || lmax[1] > lim[1])) {
#pragma unroll
      for (int gm = 0; gm < 2; ++gm) {
        const float tmax = max4(lmax[gm]);  // this query's largest S - s_off in the tile
        const bool move = tmax > lim[gm];
        const float delta = move ? tmax : 0.f;
        // rescale by 2^(old reference - new one); nothing is accumulated yet
        // while lim is -inf, and the factor is finite either way
        const float alpha = __builtin_amdgcn_exp2f(-delta);
#pragma unroll
        for (int kbk = 0; kbk < 4; ++kbk)
#pragma unroll
          for (int e = 0; e < 4; ++e) sc[gm][kbk][e] -= delta;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc_l[gm][e] *= alpha;
#pragma unroll
          for (int db = 0; db < 4; ++db) acc[gm][db][e] *= alpha;
        }
        s_off[gm] += delta;
        if (move) lim[gm] = TAU;
      }
    }
    // ---- P = exp2(S - s_off) packed to bf16, and O^T += V^T . P^T.  The V^T
    //      fragments do not depend on P, so their reads go out before the
    //      exponentials; group 1's exponentials are interleaved with group 0's
    //      products (the hints below), so the vector unit and the matrix core
    //      work at the same time within this wave.  Raised issue priority while
    //      this wave feeds the matrix core. ---------------------------------------------
    __builtin_amdgcn_s_setprio(1);
    bf16x8 vf[2][4];
#pragma unroll
    for (int db = 0; db < 4; ++db) vf[0][db] = lds_tr2(Vt + voff[db], Vt + 16 * DP + voff[db]);
    bf16x8 pb[2][2];
    auto exp_pack = [&](int gm) {
#pragma unroll
      for (int kbk = 0; kbk < 4; ++kbk)
#pragma unroll
        for (int e = 0; e < 4; ++e) sc[gm][kbk][e] = __builtin_amdgcn_exp2f(sc[gm][kbk][e]);
      // P^T operand of key half h: k index 8 g4 + 4 kb' + e <-> key 32 h + 16 kb' + 4 g4 + e
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint32_t w0 = pack2(sc[gm][2 * h][0], sc[gm][2 * h][1]);
        const uint32_t w1 = pack2(sc[gm][2 * h][2], sc[gm][2 * h][3]);
        const uint32_t w2 = pack2(sc[gm][2 * h + 1][0], sc[gm][2 * h + 1][1]);
        const uint32_t w3 = pack2(sc[gm][2 * h + 1][2], sc[gm][2 * h + 1][3]);
        const uint4 pk = make_uint4(w0, w1, w2, w3);
        pb[gm][h] = __builtin_bit_cast(bf16x8, pk);
      }
    };
    exp_pack(0);
#pragma unroll
    for (int db = 0; db < 4; ++db)
      vf[1][db] = lds_tr2(Vt + 32 * DP + voff[db], Vt + 48 * DP + voff[db]);
    exp_pack(1);
#pragma unroll
    for (int gm = 0; gm < 2; ++gm)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
#pragma unroll
        for (int db = 0; db < 4; ++db) acc[gm][db] = mfma(vf[h][db], pb[gm][h], acc[gm][db]);
        acc_l[gm] = mfma(ones, pb[gm][h], acc_l[gm]);
      }
#if TXL_ATTN_SCHED
    // schedule: group 0's exponentials and packing, then each of group 0's ten
    // products followed by up to three of group 1's vector instructions, then
    // group 1's products
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);    // V reads, half 0
    __builtin_amdgcn_sched_group_barrier(0x402, 24, 0);   // exp + pack, group 0
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);    // V reads, half 1
#pragma unroll
    for (int x = 0; x < 10; ++x) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x402, 3, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 10, 0);
#endif
    __builtin_amdgcn_s_setprio(0);
  }

  // ---- a part of a split query tile writes its unnormalised state (acc, its
  //      reference and row sum) in one block per (slot, group), laid out by lane
  //      so that each access covers whole lines:
  //        acc  [wave][gm][db][pair][lane] x 2 floats (pair 0: elements 0, 1)
  //        m, l [wave][gm][n16] x 2 floats
  //      and attn_part_merge_kernel, launched after this kernel on the same
  //      stream, merges the parts (the kernel boundary orders the partials'
  //      stores before its loads).  The part that holds key 0 has a finite
  //      reference for every query. ---------------------------------------------------
  float l_tot[2] = {acc_l[0][0], acc_l[1][0]};
  if (nparts > 1) {
    const int64_t slot0 = a.plan.slot0[qt];
    float* pa = a.part_acc + ((slot0 + part) * groups + g) * (BQ * DP);
    float* pm = a.part_ml + ((slot0 + part) * groups + g) * (BQ * 2);
#pragma unroll
    for (int gm = 0; gm < 2; ++gm) {
      if (!wave_has_rows || i0w + 16 * gm + n16 >= L) continue;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int pr = 0; pr < 2; ++pr)
          *(float2*)(pa + ((((wave * 2 + gm) * 4 + db) * 2 + pr) * 64 + lane) * 2) =
              make_float2(acc[gm][db][2 * pr], acc[gm][db][2 * pr + 1]);
      if (g4 == 0)
        *(float2*)(pm + ((wave * 2 + gm) * 16 + n16) * 2) =
            make_float2(lim[gm] == -INFINITY ? -INFINITY : s_off[gm], l_tot[gm]);
    }
    return;
  }

  // ---- epilogue: out[i][c] = acc / l, lane (g4, n16) of block db holds query
  //      i0w + 16 gm + n16, columns 16 db + 4 g4 .. + 3 -------------------------------------
  if (!wave_has_rows) return;
#pragma unroll
  for (int gm = 0; gm < 2; ++gm) {
    const int i = i0w + 16 * gm + n16;
    if (i >= L) continue;
    if constexpr (LSE) {
      if (g4 == 0) a.lse[(int64_t)g * L + i] = s_off[gm] + __log2f(l_tot[gm]);
    }
    write_out(a, b, hd, i, g4, acc[gm], 1.f / l_tot[gm]);
  }
}

// ---- 64-query workgroups -------------------------------------------------------------
// The same arithmetic with one 16-query group per wave: a workgroup is 4 waves =
// 64 queries of one (batch, head), 155 registers per lane and 48 KB of LDS, so
// three workgroups share a CU (12 waves, three per SIMD) where the 128-query
// kernel fits two; more waves cover each wave's chain of dependent LDS and
// matrix steps, and the finer query tiles leave a shorter tail (a 512-query
// segment has 8 tiles of 9 .. 16 key tiles instead of 4 of 10 .. 16).
// Every buffer is single: K, V, a 2-block r ring and each wave's shifted
// position term.  Two barriers per key tile order the loads:
//   top of tile t:  K(t) and the r blocks of tile t have landed; V(t) is issued
//                   into the V buffer (its last reader was the P.V of tile t - 1)
//   middle:         V(t) has landed; every wave has read its K and r fragments,
//                   so K(t + 1) and the r block tile t + 1 adds (into the slot of
//                   tile t's upper block) are issued
// Each load has half a tile to land; the other workgroups of the CU run meanwhile.
constexpr int BQ64 = 64;        // queries per workgroup
constexpr int RR64 = 2 * BK;    // r ring rows (two 64-distance blocks)

struct __align__(16) Smem64 {
  uint16_t K[BK * DP];        // key tile, [key][c], swizzled 16-byte chunks
  uint16_t V[BK * DP];        // value tile
  uint16_t R[RR64 * DP];      // r ring, row (distance - mem_len) mod 128, swizzled
  float W[NW][WGF];           // gathered position term of the wave's 16 queries
};

template <bool LSE>
__global__ __launch_bounds__(256, 3) void attn_q64_kernel(AttnArgs a, int nqt, int groups) {
  extern __shared__ __align__(16) char smem_raw[];
  Smem64& sm = *(Smem64*)smem_raw;

  // XCD-aware order as in the 128-query kernel: XCD x owns the groups x, x + 8,
  // ...; each XCD issues all its groups' last query tile (most key tiles) first.
  const int gpx = (groups + NXCD - 1) / NXCD;
  const int xcd = blockIdx.x % NXCD, k_on = blockIdx.x / NXCD;
  const int qt = nqt - 1 - k_on / gpx;
  const int g = (k_on % gpx) * NXCD + xcd;
  if (g >= groups) return;
  const int64_t b = g / a.H, hd = g % a.H;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g4 = lane >> 4, n16 = lane & 15;
  const int L = (int)a.L, len = (int)a.mem_len, T = len + L;
  const int q0 = qt * BQ64;
  const int i0w = q0 + wave * 16;

  const int imax_wg = (q0 + BQ64 - 1 < L - 1) ? q0 + BQ64 - 1 : L - 1;
  const int n_kt = (len + imax_wg) / BK + 1;
  const bool wave_has_rows = i0w < L;
  const int imax_w = (i0w + 15 < L - 1) ? i0w + 15 : L - 1;
  const int kt_w = wave_has_rows ? (len + imax_w) / BK : -1;

  const TileLoads ld(a, b, hd, wave, lane);
  int koff[2], voff[4];
#pragma unroll
  for (int s = 0; s < 2; ++s) koff[s] = k_frag(n16, g4, s);
#pragma unroll
  for (int db = 0; db < 4; ++db) voff[db] = v_frag(n16, g4, db);
  float* const wbuf = sm.W[wave];
  const int sprot = 4 * n16 + 3 * (n16 >> 2);
  auto sp_slot = [&](int jj) { return n16 * 64 + ((((jj >> 2) + sprot) & 15) << 2) + (jj & 3); };
  // r fragments: window block bw (0..4) of the wave's 80 rows, row n16 is relative
  // distance i0w - j0 + 15 - 16 bw - n16 (key jj = 16 bw + n16' - 15 + query),
  // stored at ring row (that) mod 128
  int roff[5];

  // ---- first tile: K, V and the two r blocks of its window ----------------------------
  {
    const int j0 = 0;
    ld.k(sm.K, j0);
    ld.v(sm.V, j0);
    ld.r<RR64>(sm.R, q0 - j0 - BK);
    ld.r<RR64>(sm.R, q0 - j0);
#pragma unroll
    for (int bw = 0; bw < 5; ++bw) {
      const int e = i0w - j0 + 15 - 16 * bw - n16;
      const int rr = e & (RR64 - 1);
      roff[bw] = rr * DP + 8 * (g4 ^ swz(rr));
    }
  }

  // ---- this lane's queries, pre-scaled: query i0w + n16, k-step s columns 32 s + 8 g4 ..
  bf16x8 qc[2], qp[2];
  query_operands(a, b, hd, i0w + n16, g4, qc, qp);

  // softmax state (see the 128-query kernel): reference s_off folded into the
  // position product's accumulator, limit lim, row sums on the matrix core
  constexpr float TAU = 8.f;
  float s_off = 0.f, lim = -INFINITY;
  f32x4 acc[4], acc_l = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int db = 0; db < 4; ++db) acc[db] = {0.f, 0.f, 0.f, 0.f};
  const bf16x8 ones = __builtin_bit_cast(bf16x8, make_uint4(0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u));
  float* srow_base = nullptr;
  if (a.scores) srow_base = a.scores + ((b * a.H + hd) * a.L) * (int64_t)T;

  for (int kt = 0; kt < n_kt; ++kt) {
    const int j0 = kt * BK;
    wait_dma();
    barrier();
    if (kt > 0) ld.v(sm.V, j0);
    const bool work = kt <= kt_w;
    const int Dw = len + i0w - j0;  // distance of (query i0w, key j0)
    f32x4 sc[4];
    if (work) {
      // ---- position term through the shifted LDS stores, then the content term
      bf16x8 rf[5][2], kf[4][2];
#pragma unroll
      for (int bw = 0; bw < 5; ++bw) {
        rf[bw][0] = lds_b128(sm.R + roff[bw]);
        rf[bw][1] = lds_b128(sm.R + (roff[bw] ^ 32));
      }
#pragma unroll
      for (int kbk = 0; kbk < 4; ++kbk)
#pragma unroll
        for (int s = 0; s < 2; ++s) kf[kbk][s] = lds_b128(sm.K + kbk * 16 * DP + koff[s]);
      f32x4 wv[5];
#pragma unroll
      for (int bw = 0; bw < 5; ++bw) {
        f32x4 w = {-s_off, -s_off, -s_off, -s_off};
        w = mfma(rf[bw][0], qp[0], w);
        wv[bw] = mfma(rf[bw][1], qp[1], w);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int jj = 4 * g4 + e - 15 + n16;  // key of block 0, in -15 .. 15
        wbuf[sp_slot(jj & (BK - 1))] = jj >= 0 ? wv[0][e] : wv[4][e];
      }
#pragma unroll
      for (int bw = 1; bw < 4; ++bw)
#pragma unroll
        for (int e = 0; e < 4; ++e) wbuf[sp_slot(16 * bw + 4 * g4 + e - 15 + n16)] = wv[bw][e];
#pragma unroll
      for (int kbk = 0; kbk < 4; ++kbk) {
        f32x4 c = *(const f32x4*)(wbuf + n16 * 64 + (((4 * kbk + g4 + sprot) & 15) << 2));
        c = mfma(kf[kbk][0], qc[0], c);
        c = mfma(kf[kbk][1], qc[1], c);
        sc[kbk] = c;
      }
    }
    // middle barrier: V(kt) has landed, K(kt) and this tile's r fragments are read
    wait_dma();
    barrier();
    if (kt + 1 < n_kt) {
      ld.k(sm.K, j0 + BK);
      ld.r<RR64>(sm.R, q0 - j0 - 2 * BK);  // the block tile kt + 1 adds, over tile kt's upper one
    }
#pragma unroll
    for (int bw = 0; bw < 5; ++bw) roff[bw] = (roff[bw] - BK * DP) & (RR64 * DP - 1);
    if (!work) continue;

    if (j0 + BK - 1 > len + i0w) {
#pragma unroll
      for (int kbk = 0; kbk < 4; ++kbk)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int jj = 16 * kbk + 4 * g4 + e;
          sc[kbk][e] = (jj - n16 > Dw) ? -INFINITY : sc[kbk][e];
        }
    }
    if (srow_base) {
      const int i = i0w + n16;
      if (i < L) {
        float* srow = srow_base + (int64_t)i * T;
#pragma unroll
        for (int kbk = 0; kbk < 4; ++kbk)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int j = j0 + 16 * kbk + 4 * g4 + e;
            if (j < T) srow[j] = (sc[kbk][e] + s_off) * (1.0f / LOG2E);
          }
      }
    }
    float lmax = -INFINITY;
#pragma unroll
    for (int kbk = 0; kbk < 4; ++kbk)
#pragma unroll
      for (int e = 0; e < 4; ++e) lmax = fmaxf(lmax, sc[kbk][e]);
    if (__any(lmax > lim)) {
      const float tmax = max4(lmax);
      const bool move = tmax > lim;
      const float delta = move ? tmax : 0.f;
      const float alpha = __builtin_amdgcn_exp2f(-delta);
#pragma unroll
      for (int kbk = 0; kbk < 4; ++kbk)
#pragma unroll
        for (int e = 0; e < 4; ++e) sc[kbk][e] -= delta;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc_l[e] *= alpha;
#pragma unroll
        for (int db = 0; db < 4; ++db) acc[db][e] *= alpha;
      }
      s_off += delta;
      if (move) lim = TAU;
    }
    // ---- P = exp2(S - s_off) packed to bf16; O^T += V^T . P^T ---------------------
    __builtin_amdgcn_s_setprio(1);
    bf16x8 vf[2][4];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int db = 0; db < 4; ++db)
        vf[h][db] = lds_tr2(sm.V + 32 * h * DP + voff[db], sm.V + (32 * h + 16) * DP + voff[db]);
#pragma unroll
    for (int kbk = 0; kbk < 4; ++kbk)
#pragma unroll
      for (int e = 0; e < 4; ++e) sc[kbk][e] = __builtin_amdgcn_exp2f(sc[kbk][e]);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint32_t w0 = pack2(sc[2 * h][0], sc[2 * h][1]);
      const uint32_t w1 = pack2(sc[2 * h][2], sc[2 * h][3]);
      const uint32_t w2 = pack2(sc[2 * h + 1][0], sc[2 * h + 1][1]);
      const uint32_t w3 = pack2(sc[2 * h + 1][2], sc[2 * h + 1][3]);
      const bf16x8 pb = __builtin_bit_cast(bf16x8, make_uint4(w0, w1, w2, w3));
#pragma unroll
      for (int db = 0; db < 4; ++db) acc[db] = mfma(vf[h][db], pb, acc[db]);
      acc_l = mfma(ones, pb, acc_l);
    }
    __builtin_amdgcn_s_setprio(0);
  }

  // ---- epilogue: out[i][c] = acc / l; lane (g4, n16) of block db holds query
  //      i0w + n16, columns 16 db + 4 g4 .. + 3 -------------------------------------------
  if (!wave_has_rows) return;
  const int i = i0w + n16;
  if (i >= L) return;
  const float l_tot = acc_l[0];
  if constexpr (LSE) {
    if (g4 == 0) a.lse[(int64_t)g * L + i] = s_off + __log2f(l_tot);
  }
  write_out(a, b, hd, i, g4, acc, 1.f / l_tot);
}

// Merge of the parts of a split query tile: one wave per (query tile, group,
// 16-query block wq = 2 w + gm, 16-column block db), whose lanes take the
// writing lanes' places (lane (g4, n16) of writing wave w holds query
// 32 w + 16 gm + n16, columns 16 db + 4 g4 .. + 3), so every load covers whole
// lines:
//   out = sum_p 2^(m_p - M) acc_p / sum_p 2^(m_p - M) l_p,  M = max_p m_p.
// The references, sums and outputs of all parts (4 values per lane and part)
// are loaded at once: one memory round trip for up to 16 parts.  The part that
// holds key 0 has a finite reference for every query.
template <int MP>
__global__ __launch_bounds__(64) void attn_part_merge_kernel(AttnArgs a) {
  const int qt = a.plan.split_qt[blockIdx.x >> 5], wq = (blockIdx.x >> 2) & 7;
  const int db = blockIdx.x & 3, g = blockIdx.y;
  const int np = a.plan.nparts[qt];  // 2 .. MP
  const int wave = wq >> 1, gm = wq & 1;
  const int64_t groups = a.B * a.H;
  const int lane = threadIdx.x;
  const int g4 = lane >> 4, n16 = lane & 15;
  const int d = (int)a.d, L = (int)a.L;
  const int64_t b = g / a.H, hd = g % a.H;
  const int64_t blk0 = (int64_t)a.plan.slot0[qt] * groups + g;
  const int i = qt * BQ + wave * BQW + 16 * gm + n16;
  if (qt * BQ + wave * BQW + 16 * gm >= L) return;  // no query of this block
  if (16 * db >= d) return;                          // no column of this block
  const int moff = (wq * 16 + n16) * 2;
  // (indexes of parts past np are clamped to part 0 and their values dropped)
  float2 ml[MP], av[MP][2];
#pragma unroll
  for (int p = 0; p < MP; ++p) {
    const int64_t blk = blk0 + (int64_t)(p < np ? p : 0) * groups;
    const float2 v = *(const float2*)(a.part_ml + blk * (BQ * 2) + moff);
    const float* pa = a.part_acc + blk * (BQ * DP) + (wq * 4 * 2 * 64 + lane) * 2;
#pragma unroll
    for (int pr = 0; pr < 2; ++pr) av[p][pr] = *(const float2*)(pa + (db * 2 + pr) * 128);
    ml[p] = p < np ? v : make_float2(-INFINITY, 0.f);
  }
  float M = -INFINITY;
#pragma unroll
  for (int p = 0; p < MP; ++p) M = fmaxf(M, ml[p].x);
  float den = 0.f, o[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int p = 0; p < MP; ++p) {
    const float wgt = p < np ? __builtin_amdgcn_exp2f(ml[p].x - M) : 0.f;
    den += wgt * ml[p].y;
    o[0] += wgt * av[p][0].x;
    o[1] += wgt * av[p][0].y;
    o[2] += wgt * av[p][1].x;
    o[3] += wgt * av[p][1].y;
  }
  if (i >= L) return;
  const float inv = 1.f / den;
  if (a.lse && db == 0 && g4 == 0) a.lse[(int64_t)g * L + i] = M + __log2f(den);
  uint16_t* orow = (uint16_t*)a.out + b * a.o_sb + (int64_t)i * a.o_st + hd * a.o_sh;
  const bool vec = ((d & 3) == 0) && (((uintptr_t)a.out & 7) == 0) && ((a.o_sb & 3) == 0) &&
                   ((a.o_st & 3) == 0) && ((a.o_sh & 3) == 0);
  const int c = 16 * db + 4 * g4;
  if (vec) {
    if (c < d)
      *(uint2*)(orow + c) = make_uint2(pack2(o[0] * inv, o[1] * inv), pack2(o[2] * inv, o[3] * inv));
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (c + e < d) orow[c + e] = bf16_bits(o[e] * inv);
  }
}

}  // namespace

// ---- work plan ---------------------------------------------------------------------------
// Workgroups of one XCD run on its CUs two at a time and start in id order, so
// the kernel's time is the longest chain of work one workgroup slot receives.
// The plan splits the key axis of some query tiles into parts (each part costs
// a fixed start-up, the partial write and the merge, PART_COST tiles) so that
// a greedy list schedule of the parts, longest first, over the XCD's slots ends
// early.  The planner starts from no split and keeps taking the single change
// (one more part for one query tile) that shortens the simulated schedule most.
namespace {

#ifndef TXL_PART_COST
#define TXL_PART_COST 2.0
#endif
constexpr double PART_COST = TXL_PART_COST;

struct PlanShape {
  int nqt, gpx, slots;
  int n_kt[ATTN_MAXQT];
};

double plan_makespan(const PlanShape& sh, const int* k, std::vector<double>& sizes,
                     std::vector<double>& heap) {
  sizes.clear();
  for (int t = 0; t < sh.nqt; ++t)
    for (int p = 0; p < k[t]; ++p) {
      const int lo = p * sh.n_kt[t] / k[t], hi = (p + 1) * sh.n_kt[t] / k[t];
      sizes.push_back((hi - lo) + (k[t] > 1 ? PART_COST : 0.0));
    }
  std::sort(sizes.begin(), sizes.end(), [](double x, double y) { return x > y; });
  heap.assign(sh.slots, 0.0);  // min-heap of slot finish times
  for (double sz : sizes)
    for (int gi = 0; gi < sh.gpx; ++gi) {
      std::pop_heap(heap.begin(), heap.end(), std::greater<double>());
      heap.back() += sz;
      std::push_heap(heap.begin(), heap.end(), std::greater<double>());
    }
  return *std::max_element(heap.begin(), heap.end());
}

}  // namespace

// Kernel choice (txl_attn_variant): 0 by shape, 1 the 64-query kernel, 2 the
// 128-query kernel with its planned key splits.
std::atomic<int> g_variant{0};

AttnPlan plan_uncached(const AttnArgs& a, int num_cus, size_t budget);

// Plans are cached per shape (the search costs far more than a launch).
int attn_set_variant(int v) { return g_variant.exchange(v); }

AttnPlan attn_mfma_plan(const AttnArgs& a, int num_cus, size_t budget) {
  struct Entry { int64_t groups, L, mem_len; int cus; size_t budget; int var; AttnPlan plan; };
  static std::mutex mu;
  static Entry cache[16];
  static int n_cached = 0, next = 0;
  const int64_t groups = a.B * a.H;
  {
    std::lock_guard<std::mutex> lock(mu);
    for (int i = 0; i < n_cached; ++i) {
      const Entry& e = cache[i];
      if (e.groups == groups && e.L == a.L && e.mem_len == a.mem_len && e.cus == num_cus &&
          e.budget == budget && e.var == g_variant.load(std::memory_order_relaxed))
        return e.plan;
    }
  }
  const AttnPlan p = plan_uncached(a, num_cus, budget);
  std::lock_guard<std::mutex> lock(mu);
  cache[next] = {groups, a.L, a.mem_len, num_cus, budget, g_variant.load(std::memory_order_relaxed), p};
  next = (next + 1) % 16;
  if (n_cached < 16) ++n_cached;
  return p;
}

AttnPlan plan_uncached(const AttnArgs& a, int num_cus, size_t budget) {
  AttnPlan p{};
  const int64_t nqt = (a.L + BQ - 1) / BQ;
  const int64_t groups = a.B * a.H;
  // By shape.  A long key loop (16 or more key tiles for the last query tile)
  // with enough 128-query tiles for a full round of two per CU: the 128-query
  // kernel, whose two query groups per wave share every K, V and r fragment read
  // (a 512-token segment over a 512-token memory).  Otherwise, with enough
  // 64-query tiles for two per CU, the 64-query kernel, unsplit: finer tiles
  // and three workgroups per CU (the word model's 150-token segments, the
  // 384-token training segments).  Fewer (a long memory over few query rows):
  // the 128-query kernel, its key axis split as planned below.
  const int var = g_variant.load(std::memory_order_relaxed);
  const int64_t n_kt_last = (a.mem_len + a.L - 1) / BK + 1;
  const bool long_loop = n_kt_last >= 16 && groups * nqt >= 2 * (int64_t)num_cus;
  if (var == 1 ||
      (var == 0 && !long_loop && groups * ((a.L + BQ64 - 1) / BQ64) >= 2 * (int64_t)num_cus)) {
    p.q64 = 1;
    return p;
  }
  if (nqt > ATTN_MAXQT || groups <= 0) return p;  // default order, no split
  PlanShape sh{};
  sh.nqt = (int)nqt;
  sh.gpx = (int)((groups + NXCD - 1) / NXCD);
  sh.slots = num_cus * 2 / NXCD > 0 ? num_cus * 2 / NXCD : 1;
  for (int t = 0; t < sh.nqt; ++t) {
    const int64_t imax = (int64_t)t * BQ + BQ - 1 < a.L - 1 ? (int64_t)t * BQ + BQ - 1 : a.L - 1;
    sh.n_kt[t] = (int)((a.mem_len + imax) / BK + 1);
  }
  int k[ATTN_MAXQT];
  for (int t = 0; t < sh.nqt; ++t) k[t] = 1;
  auto bytes_of = [&](const int* kk) {
    int slots = 0, ncls = 0;
    for (int t = 0; t < sh.nqt; ++t) {
      ncls += kk[t];
      if (kk[t] > 1) slots += kk[t];
    }
    if (ncls > ATTN_MAXCLS || slots > 255) return (size_t)-1;
    const size_t rows = (size_t)slots * (size_t)groups * BQ;
    return slots ? rows * (DP + 2) * sizeof(float) + 512 : (size_t)0;
  };
  // Descent: each step takes the change (one more part for one query tile) that
  // shortens the simulated schedule most, or, when none does, splits the tile
  // with the longest parts further (the schedule may need several tiles split
  // before it shortens).  The best plan met on the way wins; a plan replaces a
  // smaller one only for a clear gain.
  std::vector<double> sizes, heap;
  double cur = plan_makespan(sh, k, sizes, heap), best = cur;
  int best_k[ATTN_MAXQT];
  for (int t = 0; t < sh.nqt; ++t) best_k[t] = k[t];
  auto can_split = [&](int t, int kk) {
    if (kk > 16 || kk > sh.n_kt[t] / 2) return false;
    const int keep = k[t];
    k[t] = kk;
    const bool ok = bytes_of(k) <= budget;
    k[t] = keep;
    return ok;
  };
  for (int step = 0; step < ATTN_MAXCLS; ++step) {
    int bt = -1;
    double bm = cur;
    for (int t = 0; t < sh.nqt; ++t) {
      if (!can_split(t, k[t] + 1)) continue;
      ++k[t];
      const double m = plan_makespan(sh, k, sizes, heap);
      --k[t];
      if (m < bm) {
        bm = m;
        bt = t;
      }
    }
    if (bt < 0) {  // no single change helps: split the longest parts further
      int longest = 0;
      for (int t = 0; t < sh.nqt; ++t) {
        const int part = (sh.n_kt[t] + k[t] - 1) / k[t];
        if (can_split(t, k[t] + 1) && part > longest) {
          longest = part;
          bt = t;
        }
      }
      if (bt < 0) break;
      ++k[bt];
      bm = plan_makespan(sh, k, sizes, heap);
    } else {
      ++k[bt];
    }
    cur = bm;
    if (cur < best * 0.99) {
      best = cur;
      for (int t = 0; t < sh.nqt; ++t) best_k[t] = k[t];
    }
  }
  for (int t = 0; t < sh.nqt; ++t) k[t] = best_k[t];
  // class list: parts longest first (ties: later query tile first), slots of split tiles
  struct Cls { int sz, qt, part; };
  std::vector<Cls> cl;
  int slot = 0;
  p.nsplit_qt = 0;
  for (int t = 0; t < sh.nqt; ++t) {
    p.nparts[t] = (uint8_t)k[t];
    p.slot0[t] = (uint8_t)(k[t] > 1 ? slot : 0);
    if (k[t] > 1) {
      slot += k[t];
      p.split_qt[p.nsplit_qt++] = (uint8_t)t;
    }
    for (int q = 0; q < k[t]; ++q) {
      const int lo = q * sh.n_kt[t] / k[t], hi = (q + 1) * sh.n_kt[t] / k[t];
      cl.push_back({hi - lo, t, q});
    }
  }
  std::stable_sort(cl.begin(), cl.end(), [](const Cls& x, const Cls& y) {
    return x.sz != y.sz ? x.sz > y.sz : x.qt > y.qt;
  });
  p.ncls = slot > 0 ? (int)cl.size() : 0;  // no split: the kernel's own order, same list
  p.slots = slot;
  for (int c = 0; c < p.ncls; ++c) {
    p.cls_qt[c] = (uint8_t)cl[c].qt;
    p.cls_part[c] = (uint8_t)cl[c].part;
  }
  return p;
}

size_t attn_plan_bytes(const AttnArgs& a, const AttnPlan& p) {
  if (p.slots <= 0) return 0;
  const size_t groups = (size_t)(a.B * a.H);
  const size_t rows = (size_t)p.slots * groups * BQ;
  return rows * (DP + 2) * sizeof(float) + 512;
}

void attn_plan_bind(AttnArgs& a, const AttnPlan& p, void* scratch) {
  a.plan = p;
  a.part_acc = nullptr;
  a.part_ml = nullptr;
  if (p.slots <= 0) return;
  const size_t groups = (size_t)(a.B * a.H);
  const size_t rows = (size_t)p.slots * groups * BQ;
  char* base = (char*)(((uintptr_t)scratch + 255) & ~(uintptr_t)255);
  a.part_acc = (float*)base;
  base += (rows * DP * sizeof(float) + 255) & ~(size_t)255;
  a.part_ml = (float*)base;
}

bool attn_mfma_supported(const AttnArgs& a) {
  if (a.d > DP || a.d_load % 8 != 0 || a.d_load > DP) return false;
  if (a.mem_len + a.L > 0x7fffffffLL - 2 * BQ) return false;
  // 32-bit element offsets inside a (batch, head) slab
  const int64_t krows = a.kv_cap > 0 ? a.kv_cap : a.mem_len + a.L;
  if (krows * a.kv_st > 0x7fffffffLL || (a.mem_len + a.L) * a.r_sp > 0x7fffffffLL) return false;
  if (a.kv_cap > 0x7fffffffLL - 2 * BK) return false;
  const uintptr_t al = (uintptr_t)a.q | (uintptr_t)a.k | (uintptr_t)a.v | (uintptr_t)a.r;
  if (al % 16) return false;
  const int64_t st[] = {a.q_sb, a.q_st, a.q_sh, a.kv_sb, a.kv_st, a.kv_sh, a.r_sp, a.r_sh};
  for (int64_t s : st)
    if (s % 8) return false;
  return true;
}

hipError_t launch_attn_mfma(const AttnArgs& a, int num_cus, hipStream_t s) {
  (void)num_cus;
  if (a.plan.q64) {
    const int nqt64 = (int)((a.L + BQ64 - 1) / BQ64);
    const int groups = (int)(a.B * a.H);
    const int64_t nblocks = (int64_t)nqt64 * NXCD * ((groups + NXCD - 1) / NXCD);
    const size_t smem = sizeof(Smem64);
    static bool attr64 = false;
    if (!attr64) {
      hipError_t e = hipFuncSetAttribute((const void*)attn_q64_kernel<false>,
                                         hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
      if (e == hipSuccess)
        e = hipFuncSetAttribute((const void*)attn_q64_kernel<true>,
                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
      if (e != hipSuccess) return e;
      attr64 = true;
    }
    if (a.lse)
      hipLaunchKernelGGL(attn_q64_kernel<true>, dim3((unsigned)nblocks), dim3(256), smem, s, a,
                         nqt64, groups);
    else
      hipLaunchKernelGGL(attn_q64_kernel<false>, dim3((unsigned)nblocks), dim3(256), smem, s, a,
                         nqt64, groups);
    return hipGetLastError();
  }
  const int nqt = (int)((a.L + BQ - 1) / BQ);
  const int groups = (int)(a.B * a.H);
  const int ncls = a.plan.ncls > 0 ? a.plan.ncls : nqt;
  const int64_t nblocks = (int64_t)ncls * NXCD * ((groups + NXCD - 1) / NXCD);
  const size_t smem = sizeof(Smem);
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)attn_mfma_kernel<false>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    if (e == hipSuccess)
      e = hipFuncSetAttribute((const void*)attn_mfma_kernel<true>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  if (a.plan.slots > 0 && (!a.part_acc || !a.part_ml)) return hipErrorInvalidValue;
  if (a.lse)
    hipLaunchKernelGGL(attn_mfma_kernel<true>, dim3((unsigned)nblocks), dim3(256), smem, s, a, nqt,
                       groups);
  else
    hipLaunchKernelGGL(attn_mfma_kernel<false>, dim3((unsigned)nblocks), dim3(256), smem, s, a, nqt,
                       groups);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.plan.slots == 0) return e;
  // one wave per (split query tile, 16-query block, 16-column block, group), the
  // part loop sized to the most parts any tile has
  int mp = 2;
  for (int t = 0; t < a.plan.nsplit_qt; ++t)
    while (mp < a.plan.nparts[a.plan.split_qt[t]]) mp *= 2;
  const dim3 mgrid((unsigned)a.plan.nsplit_qt * 32, (unsigned)groups);
  if (mp <= 2)
    hipLaunchKernelGGL(attn_part_merge_kernel<2>, mgrid, dim3(64), 0, s, a);
  else if (mp <= 4)
    hipLaunchKernelGGL(attn_part_merge_kernel<4>, mgrid, dim3(64), 0, s, a);
  else if (mp <= 8)
    hipLaunchKernelGGL(attn_part_merge_kernel<8>, mgrid, dim3(64), 0, s, a);
  else
    hipLaunchKernelGGL(attn_part_merge_kernel<16>, mgrid, dim3(64), 0, s, a);
  return hipGetLastError();
}

}  // namespace txl
