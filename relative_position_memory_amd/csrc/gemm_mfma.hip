// Projection GEMMs, bf16 matrix-core path for gfx950:
//   C[m][n] = sum_k A[m][k] * W[n][k]      (y = x W^T, fp32 accumulation)
// A's rows are gathered (memory ring rows, then the current rows: the extended
// context [SG(m) o h] of Transformer-XL section 3.2 is never materialised).
//
// Sizing for gfx950.  A CU reads LDS at ~256 B/clk (16-byte reads) but writes
// it at ~100 B/clk, and global-load latency under load exceeds one K step of
// matrix work, so:
//  * The large tile is 256 x 256 per workgroup of 8 waves (2 along m, 4 along
//    n), each wave 128 x 64 = 4 x 2 blocks of v_mfma_f32_32x32x16_bf16; per
//    16-deep k slice a wave reads 6 KB of LDS for 8 MFMAs.  A 128 x 128 tile
//    (4 waves of 64 x 64) serves grids that would leave CUs idle.
//  * When K is a multiple of 32 the tiles travel from global memory straight
//    into LDS (global_load_lds_dwordx4, no register staging) through a ring of
//    four 32-deep stages, loads running three stages ahead of the MFMAs.
//    Rows are 64 bytes; 16-byte chunk c of row r sits in slot
//    c ^ swz(r), which keeps every fragment read conflict-free.
//  * Otherwise a register-staged, double-buffered 64-deep pipeline is used.
//  * Workgroups are persistent: each walks tiles blockIdx.x, + gridDim.x, ...
//
// The product is formed transposed, C^T = W A^T: W supplies the MFMA's A
// operand and the gathered rows its B operand, so each lane owns one output
// row m; W rows are fed in a permuted order so that each lane holds 16
// consecutive output columns.  The epilogue stages the tile in LDS and writes
// whole 16-byte chunks.  One launch may carry up to four independent problems
// (the layer step's q, k/v and r projections share K and run as one grid).
#include "gemm_common.h"

namespace txl {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;

constexpr int NXCD = 8;
constexpr int MAXP = 8;
#ifndef TXL_GEMV
#define TXL_GEMV 1
#endif

struct GemmBatch {
  GemmArgs g[MAXP];
  int ntm[MAXP], ntn[MAXP];
  int block_end[MAXP];  // inclusive prefix sums of the problems' tile counts (x ks)
  int ks[MAXP];         // K splits of each output tile, >= 1 (> 1: fp32 partials)
  int n;
};

__device__ inline uint4 keep_if(uint4 v, bool keep) {
  const uint32_t k = keep ? 0xffffffffu : 0u;
  return make_uint4(v.x & k, v.y & k, v.z & k, v.w & k);
}

// two floats -> packed bf16 pair (low half = lo), one v_cvt_pk_bf16_f32
__device__ inline uint32_t pack_bf16x2(float lo, float hi) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){lo, hi}, bf16x2));
}

// Output row rho = 8 q + 4 h + t of a 32 x 32 MFMA block (q = register group,
// h = lane half, t = register in the group) is fed W row wrow_perm(rho) =
// 16 h + 4 q + t, so lane half h ends up holding the 16 consecutive columns
// 16 h .. 16 h + 15 of the block in registers 0 .. 15.
__device__ inline int wrow_perm(int rho) { return 16 * ((rho >> 2) & 1) + 4 * (rho >> 3) + (rho & 3); }

// Tile geometry: BM x BN outputs, WM x WN waves of (BM/WM) x (BN/WN).
template <int BM_, int BN_, int WM_, int WN_, int OCC_>
struct Cfg {
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_;
  static constexpr int OCC = OCC_;                // workgroups per CU
  static constexpr int NW = WM * WN;
  static constexpr int NT = 64 * NW;             // threads
  static constexpr int TI = BM / WM / 32;        // 32-row blocks of m per wave
  static constexpr int TJ = BN / WN / 32;        // 32-column blocks of n per wave
  // register-staged pipeline: 64-deep K steps, rows padded to 72 bf16
  static constexpr int RBK = 64, RKP = 72;
  static constexpr int RPP = NT / 8;             // rows per load pass (8 x 16 B per row)
  static constexpr int PA = BM / RPP, PW = BN / RPP;
  static constexpr size_t RSMEM = (size_t)2 * (BM + BN) * RKP * sizeof(uint16_t);
  // LDS-direct pipeline: 32-deep K steps (64-byte rows), NS stages
  static constexpr int DBK = 32, NS = 4;
  static constexpr int STAGE = (BM + BN) * DBK;  // bf16 elements per stage
  static constexpr int QA = BM / 16 / NW, QW = BN / 16 / NW;  // 1 KB loads per wave and stage
  static constexpr size_t DSMEM = (size_t)NS * STAGE * sizeof(uint16_t);
  // epilogue staging
  static constexpr size_t ESMEM_BF16 = (size_t)BM * (BN + 8) * sizeof(uint16_t);
  static constexpr size_t ESMEM_F32 = (size_t)BM * (BN + 4) * sizeof(float);
  static constexpr size_t ESMEM_SCALAR = (size_t)NW * 32 * (32 * TJ + 1) * sizeof(float);
};
using Big = Cfg<256, 256, 2, 4, 1>;
using Small = Cfg<128, 128, 2, 2, 2>;

enum { EPI_SCALAR = 0, EPI_STAGE_BF16 = 1, EPI_STAGE_F32 = 2 };

template <class C, int EPI>
constexpr size_t epi_smem() {
  return EPI == EPI_STAGE_BF16 ? C::ESMEM_BF16
       : EPI == EPI_STAGE_F32  ? C::ESMEM_F32
                               : C::ESMEM_SCALAR;
}
constexpr size_t cmax(size_t a, size_t b) { return a > b ? a : b; }

// Address of logical row m of the gathered A operand, 32-bit index arithmetic
// (the launch checks that every row and offset fits).
__device__ inline const uint16_t* gather_row32(const RowGather& a, int m) {
  const int per = (int)(a.mem_len + a.cur_rows), len = (int)a.mem_len;
  const int b = m / per, t = m - b * per;
  if (t < len) {
    int slot = (int)a.mem_start + t;
    if (slot >= (int)a.mem_cap) slot -= (int)a.mem_cap;
    return (const uint16_t*)a.mem + ((int64_t)b * a.mem_cap + slot) * a.lda;
  }
  return (const uint16_t*)a.cur + ((int64_t)b * a.cur_rows + (t - len)) * a.lda;
}

struct TileId {
  int p, m0, n0;
  bool valid;
};

// Tile n of the batch.  Row tiles of A are spread over the XCDs (workgroup w
// runs on XCD w % 8, the grid is a multiple of 8 and every problem's tile
// range starts at a multiple of 8, so tile n is always computed on XCD n % 8);
// the column tiles of one row tile run consecutively on the same XCD, whose L2
// then serves the A tile to all of them.  That covers the row tiles of whole
// groups of 8; the last ntm % 8 row tiles follow in plain row-major order, and
// only the problem's tile count is padded to a multiple of 8 (tile_slots).
template <class C>
__device__ inline TileId tile_id(const GemmBatch& bt, int tile, int& split) {
  TileId t;
  t.p = 0;
  while (t.p + 1 < bt.n && tile >= bt.block_end[t.p]) ++t.p;
  const int ntm = bt.ntm[t.p], ntn = bt.ntn[t.p];
  // the K splits of one output tile are consecutive slots
  const int local = tile - (t.p ? bt.block_end[t.p - 1] : 0), ks = bt.ks[t.p];
  split = local % ks;
  const int bid = local / ks;
  const int main_rows = ntm / NXCD * NXCD;
  int tm, tn;
  if (bid < main_rows * ntn) {
    const int xcd = bid % NXCD, k_on = bid / NXCD;
    tm = (k_on / ntn) * NXCD + xcd;
    tn = k_on % ntn;
  } else {
    const int r = bid - main_rows * ntn;
    tm = main_rows + r / ntn;
    tn = r % ntn;
  }
  t.valid = tm < ntm;
  t.m0 = tm * C::BM;
  t.n0 = tn * C::BN;
  return t;
}

// Grid slots of one problem in tile_id's order: its tiles, padded to a multiple of 8
// (times the problem's K splits).
inline int64_t tile_slots(int64_t ntm, int64_t ntn) {
  return (ntm * ntn + NXCD - 1) / NXCD * NXCD;
}

template <class C>
__device__ inline void zero_acc(f32x16 (&acc)[C::TJ][C::TI]) {
#pragma unroll
  for (int j = 0; j < C::TJ; ++j)
#pragma unroll
    for (int i = 0; i < C::TI; ++i)
#pragma unroll
      for (int x = 0; x < 16; ++x) acc[j][i][x] = 0.f;
}

// ---- epilogue -----------------------------------------------------------------------
// Lane (li, h) of block (j, i) holds row m0 + wm*32*TI + 32 i + li, columns
// n0 + wn*32*TJ + 32 j + 16 h + [0, 16) in registers 0..15.  The staged forms
// write the tile to LDS (whose K-loop contents are dead: the caller has passed
// a barrier after the last fragment read), then store 16-byte chunks: every
// row's columns are contiguous in the destination, so each store instruction
// covers whole cache lines.  Ends with a barrier (the next tile reuses LDS).
template <class C, int EPI>
__device__ inline void epilogue(const GemmArgs& g, int m0, int n0, char* smem,
                                const f32x16 (&acc)[C::TJ][C::TI], int tid, int wm, int wn,
                                int li, int lh, int split = -1) {
  if (EPI == EPI_STAGE_BF16) {
    constexpr int EP = C::BN + 8;  // row pitch (bf16): 16-byte aligned, conflict-free
    uint16_t* es = (uint16_t*)smem;
    // bias and activation (wave-uniform: only the feed-forward's first layer has them)
    const bool post = g.e.bias != nullptr || g.e.act != ACT_NONE;
#pragma unroll
    for (int i = 0; i < C::TI; ++i)
#pragma unroll
      for (int j = 0; j < C::TJ; ++j) {
        float v[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) v[e] = acc[j][i][e];
        if (post) {
          const int nb = n0 + wn * 32 * C::TJ + 32 * j + 16 * lh;
#pragma unroll
          for (int e = 0; e < 16; ++e)
            v[e] = nb + e < g.N ? epi_value<uint16_t>(g.e, nb + e, v[e]) : v[e];
        }
        uint32_t pk[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) pk[e] = pack_bf16x2(v[2 * e], v[2 * e + 1]);
        uint16_t* dst = es + (wm * 32 * C::TI + 32 * i + li) * EP + wn * 32 * C::TJ + 32 * j + 16 * lh;
        *(uint4*)dst = make_uint4(pk[0], pk[1], pk[2], pk[3]);
        *(uint4*)(dst + 8) = make_uint4(pk[4], pk[5], pk[6], pk[7]);
      }
    __syncthreads();
    constexpr int CPR = C::BN / 8;     // 16-byte chunks per row
    constexpr int STEP = C::NT / CPR;  // rows between a thread's chunks
    const int per = (int)(g.a.mem_len + g.a.cur_rows);
    const int HD = (int)g.e.HD, d = (int)g.e.d;
    const int c = tid % CPR;
    const int n = n0 + 8 * c;
    const int which = n >= HD, nn = n - which * HD;
    const int head = nn / d, cc = nn - head * d;
    uint16_t* colbase = (uint16_t*)(which ? g.e.dst1 : g.e.dst0) + (int64_t)head * g.e.sh + cc;
    // head-padded columns: this thread's 8 elements past d_valid are stored as zeros
    uint32_t keep[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const bool lo = g.e.d_valid <= 0 || cc + 2 * q < g.e.d_valid;
      const bool hi = g.e.d_valid <= 0 || cc + 2 * q + 1 < g.e.d_valid;
      keep[q] = (lo ? 0x0000ffffu : 0u) | (hi ? 0xffff0000u : 0u);
    }
    const int row0 = tid / CPR;
    int b = (m0 + row0) / per, t = m0 + row0 - b * per;
    for (int row = row0; row < C::BM; row += STEP) {
      if (m0 + row >= g.M) break;
      if (n < g.N) {
        const uint4 v = *(const uint4*)(es + row * EP + 8 * c);
        *(uint4*)(colbase + b * g.e.sb + ring_t(g.e, t) * g.e.st) =
            make_uint4(v.x & keep[0], v.y & keep[1], v.z & keep[2], v.w & keep[3]);
      }
      t += STEP;
      while (t >= per) { t -= per; ++b; }
    }
    __syncthreads();
  } else if (EPI == EPI_STAGE_F32) {
    // y[m][n] = acc + bias + resid[m][n] (no residual when resid is NULL; fp32
    // residual when resid_f32).  In a K-split launch split s stores its partial
    // sum to y + s M N, with neither bias nor residual.  A bf16
    // residual is loaded before the staging (a load after a store to y would wait
    // for it: the two may alias as far as the compiler knows); an fp32 residual,
    // twice the registers, after it, when the accumulators are dead, all rows of
    // this thread before the first store.  Four columns per thread: 16-byte
    // stores when N % 4 == 0 and the tensors are aligned, else element by element.
    constexpr int EP = C::BN + 4;  // row pitch (fp32)
    constexpr int CPR = C::BN / 4;
    constexpr int STEP = C::NT / CPR, RPT = C::BM / STEP;  // rows per pass, per thread
    float* es = (float*)smem;
    const int c = tid % CPR, row0 = tid / CPR;
    const int n = n0 + 4 * c;
    const int64_t N = g.N;
    const bool plain = split >= 0;  // partial of a split launch
    float* y = g.e.y + (plain ? (int64_t)split * g.M * N : 0);
    const bool rf32 = g.e.resid_f32 != 0;
    const void* resv = plain ? nullptr : g.e.resid;
    const bool vec = N % 4 == 0 && (uintptr_t)g.e.y % 16 == 0 &&
                     (uintptr_t)resv % (rf32 ? 16 : 8) == 0;
    const uint16_t* res = (const uint16_t*)resv;
    uint16_t rv[RPT][4] = {};
#pragma unroll
    for (int x = 0; x < RPT; ++x) {
      if (res == nullptr || rf32) break;
      const int64_t m = (int64_t)m0 + row0 + STEP * x < g.M ? (int64_t)m0 + row0 + STEP * x : g.M - 1;
      if (vec) {
        const int64_t nc = n < N ? n : N - 4;
        const uint2 w = *(const uint2*)(res + m * N + nc);
        rv[x][0] = (uint16_t)(w.x & 0xffffu); rv[x][1] = (uint16_t)(w.x >> 16);
        rv[x][2] = (uint16_t)(w.y & 0xffffu); rv[x][3] = (uint16_t)(w.y >> 16);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) rv[x][e] = res[m * N + (n + e < N ? n + e : N - 1)];
      }
    }
#pragma unroll
    for (int i = 0; i < C::TI; ++i)
#pragma unroll
      for (int j = 0; j < C::TJ; ++j) {
        float* dst = es + (wm * 32 * C::TI + 32 * i + li) * EP + wn * 32 * C::TJ + 32 * j + 16 * lh;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          *(float4*)(dst + 4 * e) = make_float4(acc[j][i][4 * e], acc[j][i][4 * e + 1],
                                                acc[j][i][4 * e + 2], acc[j][i][4 * e + 3]);
      }
    __syncthreads();
    float4 fr[RPT];
#pragma unroll
    for (int x = 0; x < RPT; ++x) {
      fr[x] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (resv == nullptr || !rf32) continue;
      const float* rf = (const float*)resv;
      const int64_t m = (int64_t)m0 + row0 + STEP * x < g.M ? (int64_t)m0 + row0 + STEP * x : g.M - 1;
      if (vec) {
        fr[x] = *(const float4*)(rf + m * N + (n < N ? n : N - 4));
      } else {
        fr[x].x = rf[m * N + (n < N ? n : N - 1)];
        fr[x].y = rf[m * N + (n + 1 < N ? n + 1 : N - 1)];
        fr[x].z = rf[m * N + (n + 2 < N ? n + 2 : N - 1)];
        fr[x].w = rf[m * N + (n + 3 < N ? n + 3 : N - 1)];
      }
    }
#pragma unroll
    for (int x = 0; x < RPT; ++x) {
      const int row = row0 + STEP * x;
      const int64_t m = (int64_t)m0 + row;
      if (m >= g.M || n >= N) continue;
      const float4 a4 = *(const float4*)(es + row * EP + 4 * c);
      float o[4] = {a4.x, a4.y, a4.z, a4.w};
      if (!plain) {
        const float r4[4] = {fr[x].x, fr[x].y, fr[x].z, fr[x].w};
#pragma unroll
        for (int e = 0; e < 4; ++e)
          o[e] = epi_value<uint16_t>(g.e, n + e, o[e]) + (rf32 ? r4[e] : bf16_to_f32(rv[x][e]));
      }
      float* yr = y + m * N + n;
      if (vec) {
        *(float4*)yr = make_float4(o[0], o[1], o[2], o[3]);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (n + e < N) yr[e] = o[e];
      }
    }
    __syncthreads();
  } else {
    // element by element (any layout): each wave passes one 32-row block at a
    // time through its own LDS slice, then its lanes walk the block row-major
    // (consecutive lanes take consecutive columns).
    // (the residual values of a block are loaded before its stores: see above)
    constexpr int WC = 32 * C::TJ, EPW = WC + 1, PER = 32 * WC / 64;
    float* ws = (float*)smem + (wm * C::WN + wn) * 32 * EPW;
    const int lane = tid & 63;
    const bool heads = g.e.mode == EPI_HEADS;
#pragma unroll
    for (int i = 0; i < C::TI; ++i) {
      const int64_t mb = (int64_t)m0 + wm * 32 * C::TI + 32 * i;
      const int64_t nb = (int64_t)n0 + wn * WC;
      // (the residual's form is decided once, so each loop's loads are unconditional)
      float rv[PER];
#pragma unroll
      for (int x = 0; x < PER; ++x) rv[x] = 0.f;
      if (!heads && g.e.resid != nullptr) {
        if (g.e.resid_f32) {
#pragma unroll
          for (int x = 0; x < PER; ++x) {
            const int idx = lane + 64 * x, r = idx / WC, c = idx - r * WC;
            const int64_t m = mb + r < g.M ? mb + r : g.M - 1, n = nb + c < g.N ? nb + c : g.N - 1;
            rv[x] = ((const float*)g.e.resid)[m * g.N + n];
          }
        } else {
#pragma unroll
          for (int x = 0; x < PER; ++x) {
            const int idx = lane + 64 * x, r = idx / WC, c = idx - r * WC;
            const int64_t m = mb + r < g.M ? mb + r : g.M - 1, n = nb + c < g.N ? nb + c : g.N - 1;
            rv[x] = bf16_to_f32(((const uint16_t*)g.e.resid)[m * g.N + n]);
          }
        }
      }
#pragma unroll
      for (int j = 0; j < C::TJ; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) ws[li * EPW + 32 * j + 16 * lh + e] = acc[j][i][e];
      __syncthreads();
#pragma unroll
      for (int x = 0; x < PER; ++x) {
        const int idx = lane + 64 * x, r = idx / WC, c = idx - r * WC;
        const int64_t m = mb + r, n = nb + c;
        if (m >= g.M || n >= g.N) continue;
        const float v = epi_value<uint16_t>(g.e, n, ws[r * EPW + c]);
        if (heads) {
          heads_store<uint16_t>(g, m, n, v);
        } else {
          g.e.y[m * g.N + n] = v + rv[x];
        }
      }
      __syncthreads();
    }
  }
}

// ---- LDS-direct pipeline (K % 32 == 0) ----------------------------------------------

// Swizzle of a 64-byte row: chunk c of row r lives in slot c ^ swz(r).  Sixteen
// lanes reading one chunk of rows {0-3, 16-19, 4-7, 20-23} (W, permuted) or of
// 16 consecutive rows (A) hit 16 distinct (r mod 4, slot) bank groups.
__device__ inline int swz(int r) { return ((r >> 2) + 2 * (r >> 4)) & 3; }

// s_waitcnt vmcnt(N) with expcnt and lgkmcnt left alone (gfx9 encoding: vmcnt
// bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).
template <int N>
__device__ inline void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
// wait until at most `later` stages of PER loads each are still in flight
template <int PER>
__device__ inline void wait_stages(int later) {
  if (later >= 2) wait_vm<2 * PER>();
  else if (later == 1) wait_vm<PER>();
  else wait_vm<0>();
}

// Barrier that orders LDS accesses for the compiler without waiting for the
// in-flight LDS-direct loads (each wave waits for its own loads first).
__device__ inline void lds_barrier() { asm volatile("s_barrier" ::: "memory"); }
// The same after this wave's own LDS reads have completed.
// (the LDS wait goes through the builtin so that the compiler's own wait
// tracking knows these reads are complete and does not wait again after it)
__device__ inline void lds_read_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt and expcnt left alone
  asm volatile("s_barrier" ::: "memory");
}

template <class C, int EPI>
__global__ __launch_bounds__(C::NT, C::OCC) void gemm_dma_kernel(GemmBatch bt) {
  extern __shared__ __align__(16) char smem_raw[];
  uint16_t* ring = (uint16_t*)smem_raw;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int li = lane & 31, lh = lane >> 5;
  const int wm = wave / C::WN, wn = wave % C::WN;
  const int wli = wrow_perm(li);
  // fragment rows (within the stage's A / W blocks)
  int arow_f[C::TI], wrow_f[C::TJ];
#pragma unroll
  for (int i = 0; i < C::TI; ++i) arow_f[i] = wm * 32 * C::TI + 32 * i + li;
#pragma unroll
  for (int j = 0; j < C::TJ; ++j) wrow_f[j] = wn * 32 * C::TJ + 32 * j + wli;

  for (int tile = blockIdx.x; tile < bt.block_end[bt.n - 1]; tile += gridDim.x) {
    int split;
    const TileId tl = tile_id<C>(bt, tile, split);
    if (!tl.valid) continue;
    const GemmArgs& g = bt.g[tl.p];
    const int ks = bt.ks[tl.p];
    const int m0 = tl.m0, n0 = tl.n0;
    // this split's 32-deep K steps kt0 .. kt0 + nk - 1 (at least
    // floor(steps / ksplit) >= 1)
    const int nk_all = (int)(g.K / C::DBK);
    const int kt0 = split * nk_all / ks;
    const int nk = (split + 1) * nk_all / ks - kt0;

    // This lane's source rows: load q of the wave covers stage rows 16 q' + lane/4
    // (q' = wave * Q + q), 16-byte slot lane % 4, i.e. chunk slot ^ swz(row).
    const uint16_t* asrc[C::QA];
    const uint16_t* wsrc[C::QW];
#pragma unroll
    for (int q = 0; q < C::QA; ++q) {
      const int r = 16 * (wave * C::QA + q) + (lane >> 2);
      const int m = m0 + r < g.M ? m0 + r : (int)g.M - 1;  // rows past M: never stored
      asrc[q] = gather_row32(g.a, m) + 8 * ((lane & 3) ^ swz(r)) + kt0 * C::DBK;
    }
#pragma unroll
    for (int q = 0; q < C::QW; ++q) {
      const int r = 16 * (wave * C::QW + q) + (lane >> 2);
      const int n = n0 + r < g.N ? n0 + r : (int)g.N - 1;  // columns past N: never stored
      wsrc[q] = (const uint16_t*)weight_row(g.w, n, 2) + 8 * ((lane & 3) ^ swz(r)) + kt0 * C::DBK;
    }
    auto issue = [&](int kt) {
      uint16_t* st = ring + (kt % C::NS) * C::STAGE;
#pragma unroll
      for (int q = 0; q < C::QA; ++q)
        __builtin_amdgcn_global_load_lds(
            (const void __attribute__((address_space(1)))*)(asrc[q] + kt * C::DBK),
            (void __attribute__((address_space(3)))*)(st + (wave * C::QA + q) * 16 * C::DBK), 16,
            0, 0);
#pragma unroll
      for (int q = 0; q < C::QW; ++q)
        __builtin_amdgcn_global_load_lds(
            (const void __attribute__((address_space(1)))*)(wsrc[q] + kt * C::DBK),
            (void __attribute__((address_space(3)))*)(st + C::BM * C::DBK +
                                                      (wave * C::QW + q) * 16 * C::DBK),
            16, 0, 0);
    };
    constexpr int PER_STAGE = C::QA + C::QW;  // loads per wave and stage
    static_assert(C::NS == 4, "wait_stages covers up to two later stages");

    f32x16 acc[C::TJ][C::TI];
    zero_acc<C>(acc);
    // Fragments of 16-deep half s of stage kt (lane's chunk kc of the 32-deep step).
    auto frags = [&](int kt, int s, bf16x8 (&wf)[C::TJ], bf16x8 (&af)[C::TI]) {
      const uint16_t* sa = ring + (kt % C::NS) * C::STAGE;
      const uint16_t* sw = sa + C::BM * C::DBK;
      const int kc = 2 * s + lh;
#pragma unroll
      for (int j = 0; j < C::TJ; ++j)
        wf[j] = *(const bf16x8*)&sw[wrow_f[j] * C::DBK + 8 * (kc ^ swz(wrow_f[j]))];
#pragma unroll
      for (int i = 0; i < C::TI; ++i)
        af[i] = *(const bf16x8*)&sa[arow_f[i] * C::DBK + 8 * (kc ^ swz(arow_f[i]))];
    };
    auto mfmas = [&](const bf16x8 (&wf)[C::TJ], const bf16x8 (&af)[C::TI]) {
#pragma unroll
      for (int j = 0; j < C::TJ; ++j)
#pragma unroll
        for (int i = 0; i < C::TI; ++i)
          acc[j][i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[j], af[i], acc[j][i], 0, 0, 0);
    };
#pragma unroll
    for (int s = 0; s < C::NS - 1; ++s)
      if (s < nk) issue(s);
    // Every fragment read goes out one half-step ahead of its products, so its
    // LDS latency hides behind the previous half's MFMAs.  Stage kt + 1 is
    // waited for and made visible by the barrier in the middle of step kt; the
    // barrier also retires this wave's reads of stage kt (lgkmcnt 0), whose
    // buffer the loads of stage kt + 4 then reuse.
    wait_stages<PER_STAGE>(nk - 1 < C::NS - 2 ? nk - 1 : C::NS - 2);
    lds_barrier();
    if (C::NS - 1 < nk) issue(C::NS - 1);
    bf16x8 wf0[C::TJ], af0[C::TI], wf1[C::TJ], af1[C::TI];
    // Within each half step: one MFMA, then the next half's fragment reads, then
    // the other MFMAs (the reads then have all but one MFMA of the half to land).
    // The last step is peeled off so that the products after the barrier are
    // reached only through its LDS wait and start without waiting again.
    auto pin = [&]() {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                  // MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, C::TI + C::TJ, 0);      // LDS reads
      __builtin_amdgcn_sched_group_barrier(0x008, C::TI * C::TJ - 1, 0);  // MFMA
    };
    frags(0, 0, wf0, af0);
    for (int kt = 0; kt + 1 < nk; ++kt) {
      frags(kt, 1, wf1, af1);
      mfmas(wf0, af0);
      pin();
      const int later = nk - 2 - kt < C::NS - 2 ? nk - 2 - kt : C::NS - 2;
      wait_stages<PER_STAGE>(later);
      lds_read_barrier();
      if (kt + C::NS < nk) issue(kt + C::NS);
      frags(kt + 1, 0, wf0, af0);
      mfmas(wf1, af1);
      pin();
    }
    frags(nk - 1, 1, wf1, af1);
    mfmas(wf0, af0);
    mfmas(wf1, af1);
    __syncthreads();  // all fragment reads done before the epilogue reuses LDS
    epilogue<C, EPI>(g, m0, n0, smem_raw, acc, tid, wm, wn, li, lh, ks > 1 ? split : -1);
  }
}

// ---- register-staged pipeline (any K % 8 == 0; NARROW: any even K) --------------------

// Thread t stages 8-element piece (t % 8) of A rows t/8 + RPP x and W rows
// t/8 + RPP x.  Rows whose pitch is a multiple of 8 elements (16-byte aligned)
// load each piece as one 16-byte access; NARROW rows are only 4-byte aligned
// (even K and pitches, as with d_model 410): four 4-byte accesses per piece,
// each taken only below K, so the K tail is zero-filled pair by pair.
template <class C, bool NARROW>
struct Loader {
  const uint16_t* arow[C::PA];
  const uint16_t* wrow[C::PW];
  uint32_t aval, wval;  // bit x: row x is inside the problem
  int c, K, tid;

  __device__ static uint4 piece(const uint16_t* row, int kc, int K) {
    uint32_t v[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = kc + 2 * e < K ? *(const uint32_t*)(row + kc + 2 * e) : 0u;
    return make_uint4(v[0], v[1], v[2], v[3]);
  }
  __device__ void load(uint4 (&ra)[C::PA], uint4 (&rw)[C::PW], int k0) const {
    const int kc = k0 + 8 * c;
    if (NARROW) {
#pragma unroll
      for (int x = 0; x < C::PA; ++x) ra[x] = piece(arow[x], kc, K);
#pragma unroll
      for (int x = 0; x < C::PW; ++x) rw[x] = piece(wrow[x], kc, K);
      return;
    }
    const int kk = kc < K ? kc : K - 8;  // clamped into the row; zeroed at store
#pragma unroll
    for (int x = 0; x < C::PA; ++x) ra[x] = *(const uint4*)(arow[x] + kk);
#pragma unroll
    for (int x = 0; x < C::PW; ++x) rw[x] = *(const uint4*)(wrow[x] + kk);
  }
  __device__ void store(uint16_t* sa, uint16_t* sw, const uint4 (&ra)[C::PA],
                        const uint4 (&rw)[C::PW], int k0) const {
    const bool kin = NARROW || k0 + 8 * c < K;
#pragma unroll
    for (int x = 0; x < C::PA; ++x)
      *(uint4*)&sa[((tid >> 3) + C::RPP * x) * C::RKP + 8 * c] =
          keep_if(ra[x], kin && ((aval >> x) & 1));
#pragma unroll
    for (int x = 0; x < C::PW; ++x)
      *(uint4*)&sw[((tid >> 3) + C::RPP * x) * C::RKP + 8 * c] =
          keep_if(rw[x], kin && ((wval >> x) & 1));
  }
};

template <class C, int EPI, bool NARROW>
__global__ __launch_bounds__(C::NT, C::OCC) void gemm_reg_kernel(GemmBatch bt) {
  extern __shared__ __align__(16) char smem_raw[];
  uint16_t* lds = (uint16_t*)smem_raw;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int li = lane & 31, lh = lane >> 5;
  const int wm = wave / C::WN, wn = wave % C::WN;
  const int wli = wrow_perm(li);

  for (int tile = blockIdx.x; tile < bt.block_end[bt.n - 1]; tile += gridDim.x) {
    int split;  // (always 0: the register-staged pipeline takes no K splits)
    const TileId tl = tile_id<C>(bt, tile, split);
    if (!tl.valid) continue;
    const GemmArgs& g = bt.g[tl.p];
    const int m0 = tl.m0, n0 = tl.n0;

    Loader<C, NARROW> ld;
    ld.c = tid & 7;
    ld.K = (int)g.K;
    ld.tid = tid;
    ld.aval = 0;
    ld.wval = 0;
#pragma unroll
    for (int x = 0; x < C::PA; ++x) {
      const int m = m0 + (tid >> 3) + C::RPP * x;
      const bool ok = m < g.M;
      ld.aval |= (uint32_t)ok << x;
      ld.arow[x] = gather_row32(g.a, ok ? m : (int)g.M - 1);
    }
#pragma unroll
    for (int x = 0; x < C::PW; ++x) {
      const int n = n0 + (tid >> 3) + C::RPP * x;
      const bool ok = n < g.N;
      ld.wval |= (uint32_t)ok << x;
      ld.wrow[x] = (const uint16_t*)weight_row(g.w, ok ? n : g.N - 1, 2);
    }

    f32x16 acc[C::TJ][C::TI];
    zero_acc<C>(acc);
    // At the top of step kt LDS buffer kt % 2 holds tile kt and the registers
    // hold (or are receiving) tile kt + 1; buffer (kt + 1) % 2 was last read in
    // step kt - 1, which every wave finished before the barrier that ended it.
    auto sa = [&](int buf) { return lds + buf * (C::BM + C::BN) * C::RKP; };
    auto sw = [&](int buf) { return lds + buf * (C::BM + C::BN) * C::RKP + C::BM * C::RKP; };
    const int nk = (ld.K + C::RBK - 1) / C::RBK;
    uint4 ra[C::PA], rw[C::PW];
    ld.load(ra, rw, 0);
    ld.store(sa(0), sw(0), ra, rw, 0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
      const bool more = kt + 1 < nk;
      if (more) ld.load(ra, rw, (kt + 1) * C::RBK);
      const uint16_t* A = sa(kt & 1);
      const uint16_t* W = sw(kt & 1);
#pragma unroll
      for (int s = 0; s < C::RBK / 16; ++s) {
        bf16x8 wf[C::TJ], af[C::TI];
#pragma unroll
        for (int j = 0; j < C::TJ; ++j)
          wf[j] = *(const bf16x8*)&W[(wn * 32 * C::TJ + 32 * j + wli) * C::RKP + 16 * s + 8 * lh];
#pragma unroll
        for (int i = 0; i < C::TI; ++i)
          af[i] = *(const bf16x8*)&A[(wm * 32 * C::TI + 32 * i + li) * C::RKP + 16 * s + 8 * lh];
#pragma unroll
        for (int j = 0; j < C::TJ; ++j)
#pragma unroll
          for (int i = 0; i < C::TI; ++i)
            acc[j][i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[j], af[i], acc[j][i], 0, 0, 0);
      }
      if (more) ld.store(sa((kt + 1) & 1), sw((kt + 1) & 1), ra, rw, (kt + 1) * C::RBK);
      __syncthreads();
    }
    epilogue<C, EPI>(g, m0, n0, smem_raw, acc, tid, wm, wn, li, lh);
  }
}

// ---- launch ----------------------------------------------------------------------------

// Staged epilogues write 16-byte chunks: eight bf16 columns of one head (or
// four fp32 columns of y) that are contiguous and 16-byte aligned in memory.
template <class C>
int epi_kind(const GemmArgs& g) {
  if (g.e.mode == EPI_HEADS) {
    const bool ok = g.e.d % 8 == 0 && g.e.HD % 8 == 0 && g.N % 8 == 0 && g.N <= 2 * g.e.HD &&
                    g.e.sb % 8 == 0 && g.e.sh % 8 == 0 && g.e.st % 8 == 0 &&
                    (uintptr_t)g.e.dst0 % 16 == 0 && (uintptr_t)g.e.dst1 % 16 == 0;
    return ok ? EPI_STAGE_BF16 : EPI_SCALAR;
  }
  // (any N and alignment: the fp32 epilogue falls back to single elements)
  return C::ESMEM_F32 <= 160 * 1024 / C::OCC ? EPI_STAGE_F32 : EPI_SCALAR;
}

// Operand loads: LDS-direct (K % 32 == 0, 16-byte rows), register-staged 16-byte
// pieces (K % 8 == 0), or register-staged 4-byte pairs (even K, 4-byte rows).
enum { LOAD_DMA = 0, LOAD_REG = 1, LOAD_NARROW = 2 };

template <class C, int EPI, int LOAD>
hipError_t launch_cfg(const GemmBatch& bt, int total, int num_cus, hipStream_t s) {
  constexpr bool DMA = LOAD == LOAD_DMA;
  constexpr size_t smem = cmax(DMA ? C::DSMEM : C::RSMEM, epi_smem<C, EPI>());
  const void* fn = DMA ? (const void*)gemm_dma_kernel<C, EPI>
                       : (const void*)gemm_reg_kernel<C, EPI, LOAD == LOAD_NARROW>;
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  // a multiple of 8 workgroups (one XCD each in turn), at most one round
  const int slots = (num_cus * C::OCC) / NXCD * NXCD;
  const int grid = total < slots ? total : (slots > 0 ? slots : NXCD);
  if (DMA)
    hipLaunchKernelGGL((gemm_dma_kernel<C, EPI>), dim3((unsigned)grid), dim3(C::NT), smem, s, bt);
  else
    hipLaunchKernelGGL((gemm_reg_kernel<C, EPI, LOAD == LOAD_NARROW>), dim3((unsigned)grid),
                       dim3(C::NT), smem, s, bt);
  return hipGetLastError();
}

template <class C, int LOAD>
hipError_t launch_epi(const GemmBatch& bt, int epi, int total, int num_cus, hipStream_t s) {
  if (epi == EPI_STAGE_BF16) return launch_cfg<C, EPI_STAGE_BF16, LOAD>(bt, total, num_cus, s);
  // (the fp32 staging fits only the tiles whose ESMEM_F32 fits in LDS: no other
  // instance is built)
  if constexpr (C::ESMEM_F32 <= 160 * 1024 / C::OCC)
    if (epi == EPI_STAGE_F32) return launch_cfg<C, EPI_STAGE_F32, LOAD>(bt, total, num_cus, s);
  if (epi == EPI_STAGE_F32) return hipErrorInvalidValue;
  return launch_cfg<C, EPI_SCALAR, LOAD>(bt, total, num_cus, s);
}

// 16-byte operand rows: K, both row pitches a multiple of 8 and 16-byte bases.
bool wide_rows(const GemmArgs& g) {
  const uintptr_t al = (uintptr_t)g.a.cur | (uintptr_t)g.w.W0 | (uintptr_t)g.w.W1 |
                       (g.a.mem_len ? (uintptr_t)g.a.mem : 0);
  return g.K % 8 == 0 && g.a.lda % 8 == 0 && g.w.ldw % 8 == 0 && al % 16 == 0;
}
// LDS-direct loads move whole 32-deep K steps (no tail masking).
bool dma_ok(const GemmArgs& g) { return g.K % 32 == 0 && wide_rows(g); }

template <class C>
hipError_t launch_tiles(const GemmArgs* gs, int n, int num_cus, hipStream_t s,
                        const int* ksplit = nullptr) {
  GemmBatch bt{};
  int64_t total = 0;
  int epi = -1;
  bool dma = true, wide = true, split = false;
  for (int p = 0; p < n; ++p) {
    bt.g[p] = gs[p];
    bt.ntm[p] = (int)((gs[p].M + C::BM - 1) / C::BM);
    bt.ntn[p] = (int)((gs[p].N + C::BN - 1) / C::BN);
    bt.ks[p] = ksplit && ksplit[p] > 1 ? ksplit[p] : 1;
    split = split || bt.ks[p] > 1;
    total += tile_slots(bt.ntm[p], bt.ntn[p]) * bt.ks[p];
    if (total > 0x7fffffffLL) return hipErrorInvalidValue;
    bt.block_end[p] = (int)total;
    const int k = epi_kind<C>(gs[p]);
    epi = (epi < 0 || epi == k) ? k : EPI_SCALAR;
    dma = dma && dma_ok(gs[p]);
    wide = wide && wide_rows(gs[p]);
  }
  bt.n = n;
  // K splits write fp32 partial tiles: the LDS-direct pipeline, staged fp32 epilogue
  if (split && (!dma || epi != EPI_STAGE_F32)) return hipErrorInvalidValue;
  for (int p = 0; p < n; ++p)
    if (bt.ks[p] > 1 && (gs[p].e.mode != EPI_RESID_F32 || gs[p].K / 32 < bt.ks[p]))
      return hipErrorInvalidValue;
  if (total == 0) return hipSuccess;
  if (dma) return launch_epi<C, LOAD_DMA>(bt, epi, (int)total, num_cus, s);
  if (wide) return launch_epi<C, LOAD_REG>(bt, epi, (int)total, num_cus, s);
  return launch_epi<C, LOAD_NARROW>(bt, epi, (int)total, num_cus, s);
}


// ---- skinny GEMM: at most 32 rows (decode steps) -----------------------------------------
// C = A W^T with M <= 32: the large tiles would leave almost every CU idle and
// read the weights through 256-row tiles of mostly absent rows.  Here a
// workgroup owns 32 output columns for all M rows and its 8 waves split K in
// eighths; each wave keeps 16 accumulators of v_mfma_f32_32x32x16_bf16 (W rows
// as the A operand, the gathered rows of A, zero past M, as B), so lane l holds
// row l % 32.  Operands come straight from global memory, four 16-deep k steps
// per batch with the next batch's loads issued before the current batch's
// products, so every wave keeps 8 loads in flight; the weights are read once and
// A (a few KB) is shared through L2.  The eighths are summed through LDS and the
// usual epilogue stores each output.
constexpr int SK_BN = 32, SK_NW = 8, SK_CH = 4;

struct SkinnyBatch {
  GemmArgs g[MAXP];
  int block_end[MAXP];  // inclusive prefix sums of the problems' column tiles
  int n;
};

__global__ __launch_bounds__(64 * SK_NW) void gemm_skinny_kernel(SkinnyBatch bt) {
  __shared__ float red[SK_NW][64][16];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  int p = 0;
  while (p + 1 < bt.n && (int)blockIdx.x >= bt.block_end[p]) ++p;
  const GemmArgs& g = bt.g[p];
  const int n0 = ((int)blockIdx.x - (p ? bt.block_end[p - 1] : 0)) * SK_BN;
  const int M = (int)g.M, N = (int)g.N, K = (int)g.K;
  const int r32 = lane & 31, kc = 8 * (lane >> 5);  // operand row, 8-element k chunk
  const uint16_t* arow = r32 < M ? gather_row32(g.a, r32) : nullptr;
  const uint16_t* wrow = (const uint16_t*)weight_row(g.w, n0 + r32 < N ? n0 + r32 : N - 1, 2);
  const int kq = K / SK_NW, k_lo = wave * kq + kc, nit = kq / 16;
  const bf16x8 zero8 = {};
  bf16x8 wa[2][SK_CH], xb[2][SK_CH];
  auto load = [&](bf16x8 (&w)[SK_CH], bf16x8 (&x)[SK_CH], int it0) {
#pragma unroll
    for (int c = 0; c < SK_CH; ++c) {
      if (it0 + c >= nit) break;
      const int k = k_lo + 16 * (it0 + c);
      w[c] = *(const bf16x8*)(wrow + k);
      x[c] = arow ? *(const bf16x8*)(arow + k) : zero8;
    }
  };
  f32x16 acc;
#pragma unroll
  for (int x = 0; x < 16; ++x) acc[x] = 0.f;
  auto mult = [&](const bf16x8 (&w)[SK_CH], const bf16x8 (&x)[SK_CH], int it0) {
#pragma unroll
    for (int c = 0; c < SK_CH; ++c) {
      if (it0 + c >= nit) break;
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(w[c], x[c], acc, 0, 0, 0);
    }
  };
  load(wa[0], xb[0], 0);
  for (int it0 = 0; it0 < nit; it0 += 2 * SK_CH) {
    load(wa[1], xb[1], it0 + SK_CH);
    mult(wa[0], xb[0], it0);
    load(wa[0], xb[0], it0 + 2 * SK_CH);
    mult(wa[1], xb[1], it0 + SK_CH);
  }
#pragma unroll
  for (int x = 0; x < 16; ++x) red[wave][lane][x] = acc[x];
  __syncthreads();
  // C[n][m]: lane l, register x is column n0 + 8 (x / 4) + 4 (l / 32) + x % 4, row l % 32
  for (int v = tid; v < 64 * 16; v += 64 * SK_NW) {
    const int l = v >> 4, x = v & 15;
    const int m = l & 31, n = n0 + 8 * (x >> 2) + 4 * (l >> 5) + (x & 3);
    if (m >= M || n >= N) continue;
    float sum = 0.f;
#pragma unroll
    for (int w = 0; w < SK_NW; ++w) sum += red[w][l][x];
    epilogue_store<uint16_t>(g, m, n, sum);
  }
}

// ---- matrix-vector products: at most 4 rows (one-token decode steps) -----------------
// C = A W^T with M <= 4: the products are weight-streaming, so the weights are
// read once with 16-byte coalesced loads and summed on the vector ALU.  Each
// wave computes one output column n (weight row n): its 64 lanes read
// consecutive 8-element pieces of the row (K % 8 == 0), two pieces each in
// flight (K = 1024 in one round trip), and multiply them with the matching
// pieces of the MM rows of A by bf16 pair dot products (v_dot2, fp32
// accumulation); the MM sums are then reduced across the lanes.  The wave's
// column is uniform, so its weight row is found on the scalar unit; index
// arithmetic is 32-bit (gemv_ok bounds the sizes).
constexpr int GV_WAVES = 4, GV_COLS = GV_WAVES, GV_MAXM = 4;
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ inline float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

// Weight row of output column n (see WeightPair), 32-bit.
__device__ inline const uint16_t* weight_row32(const WeightPair& w, int n) {
  const bool second = n >= (int)w.n_split;
  if (second) n -= (int)w.n_split;
  const int hp = (int)w.hd_pad, hi = (int)w.hd_in;
  if (hp > hi && hi > 0) {
    const int head = n / hp, c = n - head * hp;
    n = head * hi + (c < hi ? c : hi - 1);
  }
  return (const uint16_t*)(second ? w.W1 : w.W0) + (int64_t)n * w.ldw;
}

// epilogue_store with 32-bit index arithmetic (bf16 inputs).
__device__ inline void gemv_store(const GemmArgs& g, int m, int n, float acc) {
  const Epilogue& e = g.e;
  acc = epi_value<uint16_t>(e, n, acc);
  if (e.mode != EPI_HEADS) {
    const int64_t i = (int64_t)m * g.N + n;
    e.y[i] = acc + resid_at<uint16_t>(e, i);
    return;
  }
  const int per = (int)(g.a.mem_len + g.a.cur_rows), HD = (int)e.HD, d = (int)e.d;
  const int b = m / per, t = m - b * per;
  const int which = n / HD, nn = n - which * HD;
  const int head = nn / d, c = nn - head * d;
  int tr = t;
  if (e.t_mod > 0) {
    tr = (int)e.t_off + t;
    tr = tr >= (int)e.t_mod ? tr - (int)e.t_mod : tr;
  }
  uint16_t* p = (uint16_t*)(which ? e.dst1 : e.dst0) + b * e.sb + head * e.sh + tr * e.st + c;
  if (e.d_valid > 0 && c >= (int)e.d_valid) acc = 0.f;
  Elt<uint16_t>::store(p, acc);
  if (e.pad > e.d && c == d - 1) {
#pragma unroll
    for (int i = 1; i < 8; ++i)
      if (i <= (int)(e.pad - e.d)) Elt<uint16_t>::store(p + i, 0.f);
  }
}

template <int MM>
__global__ __launch_bounds__(64 * GV_WAVES) void gemm_gemv_kernel(SkinnyBatch bt) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  int p = 0;
  while (p + 1 < bt.n && (int)blockIdx.x >= bt.block_end[p]) ++p;
  p = __builtin_amdgcn_readfirstlane(p);
  const GemmArgs& g = bt.g[p];
  const int N = (int)g.N, K = (int)g.K;
  const int n = ((int)blockIdx.x - (p ? bt.block_end[p - 1] : 0)) * GV_COLS + wave;
  const uint16_t* wrow = weight_row32(g.w, n < N ? n : N - 1);
  const uint16_t* arow[MM];
#pragma unroll
  for (int m = 0; m < MM; ++m) arow[m] = gather_row32(g.a, m);
  float acc[MM];
#pragma unroll
  for (int m = 0; m < MM; ++m) acc[m] = 0.f;
  // a second piece past K is read at the first one's k, with A zeroed
  for (int k0 = 8 * lane; k0 < K; k0 += 2 * 8 * 64) {
    const bool has1 = k0 + 8 * 64 < K;
    const int k1 = has1 ? k0 + 8 * 64 : k0;
    const uint4 w0 = *(const uint4*)(wrow + k0), w1 = *(const uint4*)(wrow + k1);
    uint4 a0[MM], a1[MM];
#pragma unroll
    for (int m = 0; m < MM; ++m) {
      a0[m] = *(const uint4*)(arow[m] + k0);
      const uint4 x = *(const uint4*)(arow[m] + k1);
      a1[m] = has1 ? x : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int m = 0; m < MM; ++m) {
      float t = acc[m];
      t = dot2_bf16(a0[m].x, w0.x, t);
      t = dot2_bf16(a0[m].y, w0.y, t);
      t = dot2_bf16(a0[m].z, w0.z, t);
      t = dot2_bf16(a0[m].w, w0.w, t);
      t = dot2_bf16(a1[m].x, w1.x, t);
      t = dot2_bf16(a1[m].y, w1.y, t);
      t = dot2_bf16(a1[m].z, w1.z, t);
      t = dot2_bf16(a1[m].w, w1.w, t);
      acc[m] = t;
    }
  }
  // sums across the wave's 64 lanes
#pragma unroll
  for (int m = 0; m < MM; ++m) acc[m] = wave_allsum(acc[m]);
  if (lane < MM && n < N) {
    float v = acc[0];
#pragma unroll
    for (int m = 1; m < MM; ++m) v = lane == m ? acc[m] : v;
    gemv_store(g, lane, n, v);
  }
}

// Sizes the 32-bit index arithmetic of the matrix-vector kernel covers.
bool gemv_ok(const GemmArgs& g) {
  const int64_t lim = 0x7fffffffLL;
  if (g.M > GV_MAXM || g.K % 8 != 0 || !wide_rows(g)) return false;
  if (g.N > lim || g.K > lim || g.w.n_split > lim || g.a.mem_len + g.a.cur_rows > lim) return false;
  if (g.e.mode == EPI_HEADS && (g.e.HD > lim || g.e.d > lim || g.e.t_mod > lim)) return false;
  if (g.a.mem_cap > lim) return false;
  return true;
}

hipError_t launch_gemv(const GemmArgs* gs, int n, hipStream_t s) {
  SkinnyBatch bt{};
  int64_t total = 0;
  for (int p = 0; p < n; ++p) {
    bt.g[p] = gs[p];
    total += (gs[p].N + GV_COLS - 1) / GV_COLS;
    if (total > 0x7fffffffLL) return hipErrorInvalidValue;
    bt.block_end[p] = (int)total;
  }
  bt.n = n;
  if (total == 0) return hipSuccess;
  int M = 0;
  for (int p = 0; p < n; ++p) M = gs[p].M > M ? (int)gs[p].M : M;
  for (int p = 0; p < n; ++p)
    if (gs[p].M != M) return hipErrorInvalidValue;  // one row count per launch
  if (M == 0) return hipSuccess;
  const dim3 grid((unsigned)total), block(64 * GV_WAVES);
  switch (M) {
    case 1: hipLaunchKernelGGL(gemm_gemv_kernel<1>, grid, block, 0, s, bt); break;
    case 2: hipLaunchKernelGGL(gemm_gemv_kernel<2>, grid, block, 0, s, bt); break;
    case 3: hipLaunchKernelGGL(gemm_gemv_kernel<3>, grid, block, 0, s, bt); break;
    case 4: hipLaunchKernelGGL(gemm_gemv_kernel<4>, grid, block, 0, s, bt); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

bool skinny_ok(const GemmArgs& g) {
  return g.M <= 32 && g.K % (16 * SK_NW) == 0 && wide_rows(g);
}

hipError_t launch_skinny(const GemmArgs* gs, int n, hipStream_t s) {
  SkinnyBatch bt{};
  int64_t total = 0;
  for (int p = 0; p < n; ++p) {
    bt.g[p] = gs[p];
    total += (gs[p].N + SK_BN - 1) / SK_BN;
    if (total > 0x7fffffffLL) return hipErrorInvalidValue;
    bt.block_end[p] = (int)total;
  }
  bt.n = n;
  if (total == 0) return hipSuccess;
  hipLaunchKernelGGL(gemm_skinny_kernel, dim3((unsigned)total), dim3(64 * SK_NW), 0, s, bt);
  return hipGetLastError();
}

// ---- output projection + residual + LayerNorm ------------------------------------------
// h_out[m] = LayerNorm(a[m] W_o^T (+ bias) + h[m]) * gamma + beta (section 3.3: post-norm,
// mean and biased variance over D).  One workgroup owns 64 whole rows, so the
// row statistics never leave the CU and y never goes to memory.  Eight waves;
// wave w owns output columns 64 w .. 64 w + 63 (2 x 2 blocks of 32 x 32 over the
// 64 rows), so D <= 512.  K streams through the same LDS-direct ring as above:
// per 32-deep stage 4 KB of a and D x 64 B of W_o.
// RAGGED: D not a multiple of 64 (even): the waves cover Dw = D rounded up to 64
// columns (W_o rows past D repeat row D - 1), the columns past D are left out of
// the row statistics and the stores, and the residual, gamma, beta, bias and
// output rows, only 4-byte aligned, move in 4-byte words.
constexpr int LBM = 64, LNW = 8, LNT = 64 * LNW, LBK = 32, LNS = 4, LDMAX = 512;

template <bool RAGGED>
__global__ __launch_bounds__(LNT, 1) void gemm_ln_kernel(LnArgs p) {
  extern __shared__ __align__(16) char smem_raw[];
  uint16_t* ring = (uint16_t*)smem_raw;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int li = lane & 31, lh = lane >> 5;
  const int D = (int)p.D, K = (int)p.K, M = (int)p.M;
  const int m0 = blockIdx.x * LBM;
  const int Dw = RAGGED ? (D + 63) / 64 * 64 : D;  // columns the waves cover
  const int stage = (LBM + Dw) * LBK;        // bf16 elements per stage
  const bool active = wave * 64 < Dw;        // this wave owns columns
  const int wli = wrow_perm(li);

  // DMA sources: a-block loads 0..3 by waves 0..3, W loads q = wave + 8 x
  const int qa = wave < LBM / 16 ? 1 : 0;
  const int qw = (Dw / 16 - wave + LNW - 1) / LNW;  // W loads of this wave (<= 4)
  const uint16_t* asrc = nullptr;
  if (qa) {
    const int r = 16 * wave + (lane >> 2);
    const int m = m0 + r < M ? m0 + r : M - 1;  // rows past M: never stored
    asrc = (const uint16_t*)p.a + (int64_t)m * K + 8 * ((lane & 3) ^ swz(r));
  }
  const uint16_t* wsrc[4];
#pragma unroll
  for (int x = 0; x < 4; ++x) {
    const int r = 16 * (wave + LNW * x) + (lane >> 2);
    const int n = r < D ? r : D - 1;
    wsrc[x] = (const uint16_t*)p.W + (int64_t)n * K + 8 * ((lane & 3) ^ swz(r));
  }
  const int nk = K / LBK;
  auto issue = [&](int kt) {
    uint16_t* st = ring + (kt % LNS) * stage;
    if (qa)
      __builtin_amdgcn_global_load_lds(
          (const void __attribute__((address_space(1)))*)(asrc + kt * LBK),
          (void __attribute__((address_space(3)))*)(st + wave * 16 * LBK), 16, 0, 0);
#pragma unroll
    for (int x = 0; x < 4; ++x)
      if (x < qw)
        __builtin_amdgcn_global_load_lds(
            (const void __attribute__((address_space(1)))*)(wsrc[x] + kt * LBK),
            (void __attribute__((address_space(3)))*)(st + LBM * LBK + (wave + LNW * x) * 16 * LBK),
            16, 0, 0);
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int x = 0; x < 16; ++x) acc[j][i][x] = 0.f;
  for (int s = 0; s < LNS - 1; ++s)
    if (s < nk) issue(s);
  const int per = qa + qw;  // loads per stage issued by this wave (wave-uniform)
  for (int kt = 0; kt < nk; ++kt) {
    const int later = nk - 1 - kt < LNS - 2 ? nk - 1 - kt : LNS - 2;
    if (per == 5) wait_stages<5>(later);
    else if (per == 4) wait_stages<4>(later);
    else if (per == 3) wait_stages<3>(later);
    else if (per == 2) wait_stages<2>(later);
    else if (per == 1) wait_stages<1>(later);
    lds_barrier();
    if (kt + LNS - 1 < nk) issue(kt + LNS - 1);
    if (active) {
      const uint16_t* sa = ring + (kt % LNS) * stage;
      const uint16_t* sw = sa + LBM * LBK;
#pragma unroll
      for (int s = 0; s < LBK / 16; ++s) {
        const int kc = 2 * s + lh;
        bf16x8 wf[2], af[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int r = wave * 64 + 32 * j + wli;
          wf[j] = *(const bf16x8*)&sw[r * LBK + 8 * (kc ^ swz(r))];
        }
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const int r = 32 * i + li;
          af[i] = *(const bf16x8*)&sa[r * LBK + 8 * (kc ^ swz(r))];
        }
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int i = 0; i < 2; ++i)
            acc[j][i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[j], af[i], acc[j][i], 0, 0, 0);
      }
    }
  }
  __syncthreads();  // ring dead from here on

  // ---- epilogue: lane (li, h) of block (j, i) holds row 32 i + li, columns
  //      64 w + 32 j + 16 h + [0, 16).  y = acc + h, then the row statistics.
  constexpr int EP = LDMAX + 8;
  uint16_t* es = (uint16_t*)smem_raw;                        // [64][EP] bf16 output
  float* red = (float*)(smem_raw + LBM * EP * sizeof(uint16_t));  // [LNW][64]
  float rs[2] = {0.f, 0.f};
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int m = m0 + 32 * i + li;
    const int mc = m < M ? m : M - 1;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int n = wave * 64 + 32 * j + 16 * lh;
      if (!active) continue;
      uint32_t rw[8];
      if (RAGGED) {  // 4-byte words, clamped to the row (past D: dropped below)
        const uint32_t* rp = (const uint32_t*)p.resid + (int64_t)mc * (D / 2);
#pragma unroll
        for (int e = 0; e < 8; ++e) rw[e] = rp[n / 2 + e < D / 2 ? n / 2 + e : D / 2 - 1];
      } else {
        const uint4* rp = (const uint4*)((const uint16_t*)p.resid + (int64_t)mc * D + n);
        const uint4 r0 = rp[0], r1 = rp[1];
        rw[0] = r0.x; rw[1] = r0.y; rw[2] = r0.z; rw[3] = r0.w;
        rw[4] = r1.x; rw[5] = r1.y; rw[6] = r1.z; rw[7] = r1.w;
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        acc[j][i][2 * e] += bf16_to_f32((uint16_t)(rw[e] & 0xffffu));
        acc[j][i][2 * e + 1] += bf16_to_f32((uint16_t)(rw[e] >> 16));
      }
      if (p.bias) {
        uint32_t bw[8];
        if (RAGGED) {
#pragma unroll
          for (int e = 0; e < 8; ++e)
            bw[e] = ((const uint32_t*)p.bias)[n / 2 + e < D / 2 ? n / 2 + e : D / 2 - 1];
        } else {
          const uint4* bp = (const uint4*)((const uint16_t*)p.bias + n);
          const uint4 b0 = bp[0], b1 = bp[1];
          bw[0] = b0.x; bw[1] = b0.y; bw[2] = b0.z; bw[3] = b0.w;
          bw[4] = b1.x; bw[5] = b1.y; bw[6] = b1.z; bw[7] = b1.w;
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          acc[j][i][2 * e] += bf16_to_f32((uint16_t)(bw[e] & 0xffffu));
          acc[j][i][2 * e + 1] += bf16_to_f32((uint16_t)(bw[e] >> 16));
        }
      }
      if (RAGGED) {  // columns past D take no part in the statistics
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[j][i][e] = n + e < D ? acc[j][i][e] : 0.f;
      }
#pragma unroll
      for (int e = 0; e < 16; ++e) rs[i] += acc[j][i][e];
    }
  }
  // row sums: lane halves, then waves
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    rs[i] += __shfl_xor(rs[i], 32, 64);
    if (lh == 0) red[wave * 64 + 32 * i + li] = rs[i];
  }
  __syncthreads();
  float mean[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    float t = 0.f;
#pragma unroll
    for (int w = 0; w < LNW; ++w) t += red[w * 64 + 32 * i + li];
    mean[i] = t / (float)D;
  }
  __syncthreads();
  float rq[2] = {0.f, 0.f};
  if (active) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const float t = (!RAGGED || wave * 64 + 32 * j + 16 * lh + e < D) ? acc[j][i][e] - mean[i] : 0.f;
          rq[i] += t * t;
        }
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    rq[i] += __shfl_xor(rq[i], 32, 64);
    if (lh == 0) red[wave * 64 + 32 * i + li] = rq[i];
  }
  __syncthreads();
  float rstd[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    float t = 0.f;
#pragma unroll
    for (int w = 0; w < LNW; ++w) t += red[w * 64 + 32 * i + li];
    rstd[i] = rsqrtf(t / (float)D + p.eps);
  }
  if (active) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int n = wave * 64 + 32 * j + 16 * lh;
      uint32_t gw[8], bw[8];
      if (RAGGED) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int c = n / 2 + e < D / 2 ? n / 2 + e : D / 2 - 1;
          gw[e] = ((const uint32_t*)p.gamma)[c];
          bw[e] = ((const uint32_t*)p.beta)[c];
        }
      } else {
        const uint4* gp = (const uint4*)((const uint16_t*)p.gamma + n);
        const uint4* bp = (const uint4*)((const uint16_t*)p.beta + n);
        const uint4 g0 = gp[0], g1 = gp[1], b0 = bp[0], b1 = bp[1];
        gw[0] = g0.x; gw[1] = g0.y; gw[2] = g0.z; gw[3] = g0.w;
        gw[4] = g1.x; gw[5] = g1.y; gw[6] = g1.z; gw[7] = g1.w;
        bw[0] = b0.x; bw[1] = b0.y; bw[2] = b0.z; bw[3] = b0.w;
        bw[4] = b1.x; bw[5] = b1.y; bw[6] = b1.z; bw[7] = b1.w;
      }
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        uint32_t pk[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float lo = (acc[j][i][2 * e] - mean[i]) * rstd[i] *
                               bf16_to_f32((uint16_t)(gw[e] & 0xffffu)) +
                           bf16_to_f32((uint16_t)(bw[e] & 0xffffu));
          const float hi = (acc[j][i][2 * e + 1] - mean[i]) * rstd[i] *
                               bf16_to_f32((uint16_t)(gw[e] >> 16)) +
                           bf16_to_f32((uint16_t)(bw[e] >> 16));
          pk[e] = pack_bf16x2(lo, hi);
        }
        uint16_t* dst = es + (32 * i + li) * EP + n;
        *(uint4*)dst = make_uint4(pk[0], pk[1], pk[2], pk[3]);
        *(uint4*)(dst + 8) = make_uint4(pk[4], pk[5], pk[6], pk[7]);
      }
    }
  }
  __syncthreads();
  if (RAGGED) {
    // 4-byte words: wave w stores rows w, w + 8, ..., its lanes consecutive words
    for (int row = wave; row < LBM && m0 + row < M; row += LNW)
      for (int c = lane; c < D / 2; c += 64)
        ((uint32_t*)p.out)[(int64_t)(m0 + row) * (D / 2) + c] = *(const uint32_t*)(es + row * EP + 2 * c);
    return;
  }
  // 16-byte chunks: D / 8 per row, rows contiguous in h_out
  const int cpr = D / 8;
  for (int q = tid; q < LBM * cpr; q += LNT) {
    const int row = q / cpr, c = q - row * cpr;
    const int m = m0 + row;
    if (m < M)
      *(uint4*)((uint16_t*)p.out + (int64_t)m * D + 8 * c) = *(const uint4*)(es + row * EP + 8 * c);
  }
}

}  // namespace

bool gemm_mfma_supported(const GemmArgs& g) {
  // even K and row pitches, 4-byte aligned rows (16-byte rows take wider loads)
  if (g.K % 2 != 0 || g.K < 8 || g.a.lda % 2 != 0 || g.w.ldw % 2 != 0) return false;
  const uintptr_t al = (uintptr_t)g.a.cur | (uintptr_t)g.w.W0 | (uintptr_t)g.w.W1 |
                       (g.a.mem_len ? (uintptr_t)g.a.mem : 0);
  if (al % 4) return false;
  // 32-bit row/column/offset arithmetic in the kernel
  if (g.K > 0x7fffffffLL || g.M > 0x7fffffffLL - 256 || g.N > 0x7fffffffLL - 256) return false;
  if (g.e.mode == EPI_HEADS) {
    const int64_t per = g.a.mem_len + g.a.cur_rows;
    const int64_t nb = (g.M + per - 1) / per;
    const int64_t span = nb * g.e.sb + (g.N / (g.e.d > 0 ? g.e.d : 1) + 1) * g.e.sh + per * g.e.st;
    if (span > 0x7fffffffLL) return false;
  }
  return true;
}

hipError_t launch_gemm_batch(const GemmArgs* gs, const int* ksplit, int n, hipStream_t s,
                             int num_cus) {
  if (n < 1 || n > MAXP || !ksplit) return hipErrorInvalidValue;
  GemmArgs gv[MAXP];
  int nv = 0, kv[MAXP];
  for (int p = 0; p < n; ++p) {
    if (ksplit[p] < 1 || gs[p].e.mode != EPI_RESID_F32 || !dma_ok(gs[p]) ||
        !gemm_mfma_supported(gs[p]) || gs[p].K / 32 < ksplit[p] ||
        epi_kind<Small>(gs[p]) != EPI_STAGE_F32)
      return hipErrorInvalidValue;
    if (gs[p].M * gs[p].N * ksplit[p] > ((int64_t)1 << 40)) return hipErrorInvalidValue;
    if (gs[p].M == 0 || gs[p].N == 0) continue;
    gv[nv] = gs[p];
    if (ksplit[p] > 1) {  // partials carry neither bias nor residual
      gv[nv].e.resid = nullptr;
      gv[nv].e.bias = nullptr;
    }
    kv[nv++] = ksplit[p];
  }
  if (nv == 0) return hipSuccess;
  return launch_tiles<Small>(gv, nv, num_cus, s, kv);
}

hipError_t launch_gemm_splitk(const GemmArgs& g, int ksplit, hipStream_t s, int num_cus) {
  GemmArgs g1 = g;
  if (ksplit == 1) {  // one split: y = the product itself
    g1.e.resid = nullptr;
    g1.e.bias = nullptr;
  }
  return launch_gemm_batch(&g1, &ksplit, 1, s, num_cus);
}

hipError_t launch_gemm_mfma_multi(const GemmArgs* gs, int n, hipStream_t s, int num_cus) {
  if (n < 1 || n > MAXP) return hipErrorInvalidValue;
  bool gemv = true, skinny = true;
  for (int p = 0; p < n; ++p) {
    gemv = gemv && gemv_ok(gs[p]) && gs[p].M == gs[0].M;
    skinny = skinny && skinny_ok(gs[p]);
  }
  if (gemv && TXL_GEMV) return launch_gemv(gs, n, s);
  if (skinny) return launch_skinny(gs, n, s);
  // 256 x 256 tiles when they give most CUs a workgroup, else 128 x 128
  int64_t big = 0;
  for (int p = 0; p < n; ++p)
    big += ((gs[p].M + Big::BM - 1) / Big::BM) * ((gs[p].N + Big::BN - 1) / Big::BN);
  if (big >= (int64_t)num_cus * 3 / 4) return launch_tiles<Big>(gs, n, num_cus, s);
  return launch_tiles<Small>(gs, n, num_cus, s);
}

hipError_t launch_gemm_mfma(const GemmArgs& g, hipStream_t s, int num_cus) {
  return launch_gemm_mfma_multi(&g, 1, s, num_cus);
}

bool gemm_ln_supported(const LnArgs& p) {
  // D a multiple of 64, or any even D (the ragged form) up to LDMAX
  const bool ragged = p.D % 64 != 0;
  if (p.D > LDMAX || p.D < 2 || p.D % 2 != 0 || p.K % LBK != 0 || p.K < LBK) return false;
  if (p.M < 1 || p.M > 0x7fffffffLL - LBM || p.M * p.K > 0x7fffffffLL || p.M * p.D > 0x7fffffffLL)
    return false;
  const uintptr_t ops = (uintptr_t)p.a | (uintptr_t)p.W;
  const uintptr_t rows = (uintptr_t)p.resid | (uintptr_t)p.gamma | (uintptr_t)p.beta |
                         (uintptr_t)p.out | (uintptr_t)p.bias;
  return ops % 16 == 0 && rows % (ragged ? 4 : 16) == 0;
}

hipError_t launch_gemm_ln(const LnArgs& p, hipStream_t s) {
  if (!gemm_ln_supported(p)) return hipErrorInvalidValue;
  const bool ragged = p.D % 64 != 0;
  const int64_t Dw = (p.D + 63) / 64 * 64;
  const size_t ring = (size_t)LNS * (LBM + Dw) * LBK * sizeof(uint16_t);
  const size_t epi = (size_t)LBM * (LDMAX + 8) * sizeof(uint16_t) + LNW * 64 * sizeof(float);
  const size_t smem = cmax(ring, epi);
  static bool attr_set[2] = {false, false};
  const void* fn = ragged ? (const void*)gemm_ln_kernel<true> : (const void*)gemm_ln_kernel<false>;
  if (!attr_set[ragged]) {
    const size_t most = cmax((size_t)LNS * (LBM + LDMAX) * LBK * sizeof(uint16_t), epi);
    hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)most);
    if (e != hipSuccess) return e;
    attr_set[ragged] = true;
  }
  const unsigned blocks = (unsigned)((p.M + LBM - 1) / LBM);
  if (ragged)
    hipLaunchKernelGGL(gemm_ln_kernel<true>, dim3(blocks), dim3(LNT), smem, s, p);
  else
    hipLaunchKernelGGL(gemm_ln_kernel<false>, dim3(blocks), dim3(LNT), smem, s, p);
  return hipGetLastError();
}

}  // namespace txl
