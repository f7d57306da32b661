// Internal launch interfaces of libtxl.so (not part of the public ABI).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace txl {

// ---- element helpers -------------------------------------------------------------
// bf16 is carried as its 16-bit pattern; widening is a shift, narrowing rounds
// to nearest even (NaN stays NaN).
__host__ __device__ inline float bf16_to_f32(uint16_t h) {
  union { uint32_t u; float f; } x;
  x.u = (uint32_t)h << 16;
  return x.f;
}
__host__ __device__ inline uint16_t f32_to_bf16(float f) {
  union { uint32_t u; float f; } x;
  x.f = f;
  if ((x.u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((x.u >> 16) | 0x40u);
  const uint32_t bias = 0x7fffu + ((x.u >> 16) & 1u);
  return (uint16_t)((x.u + bias) >> 16);
}

// ---- wave reductions ---------------------------------------------------------------
// Sum / maximum over the 64 lanes of a wave with DPP row operations (swap within
// pairs and quads, mirror within half-rows and rows of 16, then broadcast lane 15
// of a row into the next row and lane 31 into the upper half), the total read
// from lane 63 into every lane.  Every lane of the wave must be active.
template <int CTRL, int ROWS>
__device__ inline float dpp_f32(float old, float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, old),
                                                               __builtin_bit_cast(int, v), CTRL,
                                                               ROWS, 0xf, false));
}
__device__ inline float wave_allsum(float v) {
  v += dpp_f32<0xB1, 0xf>(0.f, v);   // quad_perm [1,0,3,2]
  v += dpp_f32<0x4E, 0xf>(0.f, v);   // quad_perm [2,3,0,1]
  v += dpp_f32<0x141, 0xf>(0.f, v);  // row_half_mirror
  v += dpp_f32<0x140, 0xf>(0.f, v);  // row_mirror
  v += dpp_f32<0x142, 0xa>(0.f, v);  // row_bcast:15 into rows 1, 3
  v += dpp_f32<0x143, 0xc>(0.f, v);  // row_bcast:31 into rows 2, 3
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}
__device__ inline float wave_allmax(float v) {
  v = fmaxf(v, dpp_f32<0xB1, 0xf>(v, v));
  v = fmaxf(v, dpp_f32<0x4E, 0xf>(v, v));
  v = fmaxf(v, dpp_f32<0x141, 0xf>(v, v));
  v = fmaxf(v, dpp_f32<0x140, 0xf>(v, v));
  v = fmaxf(v, dpp_f32<0x142, 0xa>(v, v));
  v = fmaxf(v, dpp_f32<0x143, 0xc>(v, v));
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}

template <typename T> struct Elt;
template <> struct Elt<float> {
  __device__ static inline float load(const float* p) { return *p; }
  __device__ static inline void store(float* p, float v) { *p = v; }
};
template <> struct Elt<uint16_t> {
  __device__ static inline float load(const uint16_t* p) { return bf16_to_f32(*p); }
  __device__ static inline void store(uint16_t* p, float v) { *p = f32_to_bf16(v); }
};

// ---- attention ---------------------------------------------------------------------
// Work plan of the matrix-core attention.  Query tile t (128 queries) of every
// (batch, head) group has its key tiles divided among nparts[t] workgroups.  The
// work classes (query tile cls_qt[c], part cls_part[c]) are issued in list order
// (longest first) for all groups of an XCD before the next class.  ncls == 0
// means one part per query tile, last tile first.
constexpr int ATTN_MAXQT = 64, ATTN_MAXCLS = 192;
struct AttnPlan {
  int ncls;
  int slots;                       // partial slots (sum of nparts over split tiles)
  uint8_t cls_qt[ATTN_MAXCLS], cls_part[ATTN_MAXCLS];
  uint8_t nparts[ATTN_MAXQT];
  uint8_t slot0[ATTN_MAXQT];       // first partial slot of a split tile's parts
  uint8_t split_qt[ATTN_MAXQT];    // the split query tiles (nsplit_qt of them)
  int nsplit_qt;
  int q64;                         // run the 64-query kernel (no split)
};

struct AttnArgs {
  int64_t B, H, L, mem_len, d;
  const void* q; int64_t q_sb, q_st, q_sh;
  const void* k; const void* v; int64_t kv_sb, kv_st, kv_sh;
  const void* r; int64_t r_sp, r_sh;
  const void* u; const void* vb;
  float scale;
  void* out; int64_t o_sb, o_st, o_sh;
  float* scores;  // NULL or [B][H][L][T]
  // NULL, or [B][H][L]: each query's log-sum-exp of its scaled scores in the
  // exp2 domain (log2 sum_j 2^(s_ij log2 e)), for the backward (matrix-core path).
  float* lse;
  // Columns of every q/k/v/r row that may be read (>= d).  Equal to d for
  // caller-owned tensors; the layer step's own workspace rows are padded to a
  // multiple of 8 and may be read whole (columns >= d are ignored).
  int64_t d_load;
  // Split of the key axis (matrix-core path only), see AttnPlan.  Parts of a
  // split query tile write unnormalised partials; a second kernel, launched
  // after the attention on the same stream, merges them.
  // Slot s of the plan holds, per (batch, head) group, a block of
  //   part_acc: 128 queries x 64 fp32, part_ml: 128 x 2 fp32 (max in the exp2
  //   domain, sum of exponentials), in the writing lanes' order.
  AttnPlan plan;
  float* part_acc;
  float* part_ml;
  // Keys as a ring: when kv_cap > 0, key j (0 <= j < mem_len + L <= kv_cap) is
  // row (kv_start + j) % kv_cap of k and v (0 <= kv_start < kv_cap).
  int64_t kv_start, kv_cap;
};

// Row of key j in k / v (see AttnArgs::kv_start).
__host__ __device__ inline int64_t kv_row(const AttnArgs& a, int64_t j) {
  if (a.kv_cap <= 0) return j;
  const int64_t p = a.kv_start + j;
  return p >= a.kv_cap ? p - a.kv_cap : p;
}

// Work plan of the matrix-core attention for these shapes on a device with
// num_cus CUs whose partials (and counters) fit in budget bytes, and the bytes a
// plan needs (0 when it splits nothing).
AttnPlan attn_mfma_plan(const AttnArgs& a, int num_cus, size_t budget);
// Kernel choice of the bf16 matrix-core attention (txl_attn_variant); returns the old one.
int attn_set_variant(int v);
size_t attn_plan_bytes(const AttnArgs& a, const AttnPlan& p);
// Points a's partial buffers into scratch (256-byte aligned inside it).
void attn_plan_bind(AttnArgs& a, const AttnPlan& p, void* scratch);

// ---- attention backward ------------------------------------------------------------
// Gradients of the relative attention for an upstream gradient dout (same layout
// as the forward's out), d <= 64.  Inputs keep the forward's strides; every
// gradient is fp32 and dense: dq [B][L][H][d], dk, dv [B][T][H][d], dr [T][H][d],
// du, dvb [H][d].  Scratch (fp32): P and dS [B][H][L][T], qc = q + u and
// qp = q + v [B][H][L][64].
struct AttnBwdArgs {
  int64_t B, H, L, mem_len, d;
  const void* q; int64_t q_sb, q_st, q_sh;
  const void* k; const void* v; int64_t kv_sb, kv_st, kv_sh;
  const void* r; int64_t r_sp, r_sh;
  const void* u; const void* vb;
  float scale;
  const void* dout; int64_t do_sb, do_st, do_sh;
  int dout_f32;   // dout is fp32 whatever the inputs' dtype
  int zeroed;     // du, dvb and dr are already zero (the caller cleared them)
  float* dq; float* dk; float* dv; float* dr; float* du; float* dvb;
  float* P; float* dS; float* qc; float* qp;
  // Optional (matrix-core path): the forward's exp2-domain log-sum-exp per query
  // ([B][H][L], AttnArgs::lse) and its output o (bf16, strides like dout); with
  // them the softmax statistics are not recomputed and sum_j P dP = dO . o.
  const float* lse;
  const void* o; int64_t o_sb, o_st, o_sh;
};
size_t attn_bwd_scratch_bytes(int64_t B, int64_t H, int64_t L, int64_t mem_len);
// Points P, dS, qc and qp into scratch (256-byte aligned inside it).
void attn_bwd_bind(AttnBwdArgs& a, void* scratch);
hipError_t launch_attn_bwd(int dtype, const AttnBwdArgs& a, hipStream_t s);
// The per-query part of the backward (P, dS, dq, du, dv) on the bf16 matrix cores
// (bf16 q, k, v, r, u, v; d <= 64).
hipError_t launch_attn_bwd_rows_mfma(const AttnBwdArgs& a, hipStream_t s);
// dr from the stored dS and q + v on the bf16 matrix cores.
hipError_t launch_attn_bwd_dr_mfma(const AttnBwdArgs& a, hipStream_t s);

// C[z] = alpha A[z] B[z] (+ C[z] when accumulate), fp32 accumulation and output,
// any element strides.  Operand X's element (i, j) of batch z sits at
// X + (z / zdiv) * s1 + (z % zdiv) * s2 + i * si + j * sj.  dtype of A and B:
// 0 = fp32, 1 = bf16.
struct StridedOperand {
  const void* p; int64_t s1, s2, si, sj;
};
struct StridedGemm {
  int64_t M, N, K, batch, zdiv;
  StridedOperand A, B;   // A (m, k), B (k, n)
  float* C; int64_t c1, c2, cm, cn;
  float alpha;
  int accumulate;
  int a_dtype, b_dtype;
  // 1: the products may run on the bf16 matrix cores (operands rounded to bf16
  // as they are staged, fp32 accumulation); 0: fp32 throughout.
  int bf16_mfma;
  // Causal A (matrix-core path): A(m, k) is taken as 0 wherever m > k + causal_off
  // (key m is not visible to query k), whatever memory holds there, and K steps
  // with no visible pair are skipped.
  int causal_on;
  int64_t causal_off;
};
hipError_t launch_gemm_strided(const StridedGemm& g, hipStream_t s);

// Layer-step backward helpers: dtype 0 = fp32, 1 = bf16 for the non-fp32 operands.
hipError_t launch_to_f32(int dtype, const void* src, float* dst, int64_t n, hipStream_t s);
// dy of h_out = LayerNorm(y) gamma + beta for dh_out (rows of D), the rows' mean
// and 1/sigma, and dgamma, dbeta (overwritten).
// Sets n fp32 buffers (at most 16) to zero in one launch.
hipError_t launch_zero_many(float* const* p, const int64_t* count, int n, hipStream_t s);
// (dgamma and dbeta are cleared first unless zeroed)
hipError_t launch_ln_bwd(int dtype, const float* y, const void* gamma, const void* dh_out,
                         int64_t M, int64_t D, float eps, float* dy, float* mean, float* rstd,
                         float* dgamma, float* dbeta, hipStream_t s, bool zeroed = false);
// LayerNorm backward with dgamma / dbeta summed per workgroup (no atomics) for
// D = 256, 512, 768 or 1024 (ln_bwd_fused_ok): dy fp32 [M][D], and also as bf16
// rows of pitch ldyb when dyb is set; part is scratch of ln_bwd_part_bytes(M, D).
// dgamma and dbeta are written (not added to).
constexpr int LN_BWD_BLOCKS = 256;
bool ln_bwd_fused_ok(int64_t M, int64_t D);
size_t ln_bwd_part_bytes(int64_t M, int64_t D);
hipError_t launch_ln_bwd_fused(int dtype, const float* y, const void* gamma, const void* dh_out,
                               int64_t M, int64_t D, float eps, float* dy, uint16_t* dyb,
                               int64_t ldyb, float* part, float* dgamma, float* dbeta,
                               hipStream_t s);
// Conversion of fp32 or bf16 operands into bf16 rows along K for the matrix
// cores, several independent jobs per launch.  Job output: dst[r][c] (row pitch
// ldd) = element (r, c) of the source for r < R, c < C, zero for C <= c < Cpad.
// pack_rows: element (r, c) at src[(r / rpb) sb + (r % rpb) ld + c] (rows of
// several batches); pack_trans: at src[c sk + r] (a transpose).  dtype 0 = fp32
// source, 1 = bf16.  tile_end and vec are filled in by launch_pack.
struct PackJob {
  const void* src;
  int64_t R, C, Cpad, rpb, sb, ld, sk;
  uint16_t* dst;
  int64_t ldd;
  int dtype, trans, vec;
  int64_t tile_end;
  // pack_trans_ctx: source row c (pitch sk) of the context [ring ; h] of batch
  // row b = c / per, position t = c % per: ring row (start + t) mod cap of batch
  // row b for t < len (src = the ring [B][cap]), else row t - len of h [B][h_rows]
  int gather;
  const void* h;
  int64_t per, len, cap, start, h_rows;
  // transposed jobs: also the rows form, dst2[row2][r] = element (r, c) for the
  // source rows c with t = c mod per2 >= skip2, row2 = (c / per2) (per2 - skip2)
  // + t - skip2 (NULL: none)
  uint16_t* dst2;
  int64_t ldd2, per2, skip2;
};
constexpr int PJ_MAX = 16;
struct PackJobs {
  PackJob j[PJ_MAX];
  int n;
};
PackJob pack_rows(const void* src, int dtype, int64_t R, int64_t C, int64_t Cpad, int64_t rpb,
                  int64_t sb, int64_t ld, uint16_t* dst, int64_t ldd);
PackJob pack_trans(const void* src, int dtype, int64_t R, int64_t C, int64_t Cpad, int64_t sk,
                   uint16_t* dst, int64_t ldd);
// pack_trans over the context rows [ring rows (oldest first) ; h] of B batch rows
// (per = len + h_rows of them each), read where they are: dst[r][c] = context
// row c, element r.
PackJob pack_trans_ctx(const void* ring, int64_t cap, int64_t start, int64_t len, const void* h,
                       int64_t h_rows, int64_t B, int dtype, int64_t R, int64_t Cpad, int64_t sk,
                       uint16_t* dst, int64_t ldd);
hipError_t launch_pack(const PackJob* jobs, int n, hipStream_t s);
// ctx [B][len + L][D] = [ring rows (oldest first) ; h]
hipError_t launch_gather_ctx(int dtype, const void* ring, int64_t cap, int64_t start, int64_t len,
                             const void* h, int64_t B, int64_t L, int64_t D, void* ctx,
                             hipStream_t s);

// Any strides, d <= 128, fp32 math.  dtype 0 = fp32, 1 = bf16.
hipError_t launch_attn_generic(int dtype, const AttnArgs& a, hipStream_t s);
// bf16 matrix-core path: d <= 64, 16-byte aligned q/k/v/r, strides multiple of 8.
hipError_t launch_attn_mfma(const AttnArgs& a, int num_cus, hipStream_t s);
bool attn_mfma_supported(const AttnArgs& a);
// One query per (batch, head) (L == 1, no scores or lse output), bf16, d <= 64,
// 16-byte aligned k/v/r with strides a multiple of 8: keys split into parts, one
// workgroup each.  attn_decode_parts gives the parts for a device with num_cus
// CUs whose partials fit scratch_bytes (0: none fits, take another path);
// attn_decode_bytes the scratch they need (0 for one part).
bool attn_decode_supported(const AttnArgs& a);
int attn_decode_parts(const AttnArgs& a, int num_cus, size_t scratch_bytes);
size_t attn_decode_bytes(const AttnArgs& a, int nparts);
hipError_t launch_attn_decode(const AttnArgs& a, int nparts, void* scratch, hipStream_t s);

// ---- GEMM: C[m][n] = sum_k A[m][k] * W[n][k] ---------------------------------------
// Row m of A is gathered: with rows_per_batch = mem_len + cur_rows,
//   b = m / rows_per_batch, t = m % rows_per_batch,
//   t <  mem_len: ring row  mem + (b*mem_cap + (mem_start + t) % mem_cap) * lda
//   t >= mem_len: current   cur + (b*cur_rows + t - mem_len) * lda
struct RowGather {
  const void* mem; int64_t mem_cap, mem_start, mem_len;
  const void* cur; int64_t cur_rows;
  int64_t lda;
};

// Two weight matrices may be stacked along n: rows [0, n_split) of the output
// use W0, rows [n_split, N) use W1 (row n - n_split).
// Head-padded columns: when hd_pad > hd_in > 0, output column n of a weight is
// element n % hd_pad of head n / hd_pad, computed from weight row
// (n / hd_pad) * hd_in + min(n % hd_pad, hd_in - 1); the columns past hd_in
// duplicate a real one and the epilogue stores them as zeros (Epilogue::d_valid).
struct WeightPair {
  const void* W0; const void* W1; int64_t n_split; int64_t ldw;
  int64_t hd_in, hd_pad;
};

enum EpiMode { EPI_HEADS = 0, EPI_RESID_F32 = 1 };
struct Epilogue {
  int mode;
  // EPI_HEADS: column n -> tensor (n / HD), head (n % HD) / d, element (n % HD) % d,
  //   written to dst[n / HD] + b*sb + head*sh + t*st + elem, (b, t) as in RowGather.
  void* dst0; void* dst1; int64_t HD, d, sb, sh, st;
  // EPI_RESID_F32: y[m][n] = acc + resid[m][n]  (y fp32 [M][N], resid [M][N] of
  // the input dtype, or fp32 when resid_f32 below; no residual when resid is NULL).
  float* y; const void* resid;
  // EPI_HEADS into a ring: when t_mod > 0, row t is stored at (t_off + t) % t_mod
  // (0 <= t_off < t_mod, t < t_mod).
  int64_t t_off, t_mod;
  // EPI_HEADS rows padded past d: when pad > d, elements d .. pad-1 of every
  // head row are written as zeros (readers may load whole padded rows).
  int64_t pad;
  // Optional per-column bias (dtype [N], NULL = none) added to acc, then for
  // EPI_HEADS the activation act (ACT_NONE or ACT_RELU).
  const void* bias;
  int act;
  // EPI_HEADS with head-padded columns: elements d_valid .. d-1 of every head
  // row are stored as zeros (0 = every element is valid).
  int64_t d_valid;
  // EPI_RESID_F32: the residual is fp32 (else the input dtype).
  int resid_f32;
};
enum ActMode { ACT_NONE = 0, ACT_RELU = 1 };

__host__ __device__ inline int64_t ring_t(const Epilogue& e, int64_t t) {
  if (e.t_mod <= 0) return t;
  const int64_t p = e.t_off + t;
  return p >= e.t_mod ? p - e.t_mod : p;
}

struct GemmArgs {
  int64_t M, N, K;
  RowGather a;
  WeightPair w;
  Epilogue e;
};
// K-split partial products on the bf16 matrix cores, for outputs whose tiles
// alone leave the GPU short of work: y[s][m][n] = sum over K slice s of
// A[m][k] W[n][k] for s < ksplit (fp32, y + s M N; g.e.mode EPI_RESID_F32, its
// bias and residual unused).  A and W dense bf16 rows (16-byte aligned, pitches
// multiples of 8), K a multiple of 32 with K / 32 >= ksplit.  The caller sums
// the partials (launch_sum_partials).
hipError_t launch_gemm_splitk(const GemmArgs& g, int ksplit, hipStream_t s, int num_cus);
// Up to 8 such problems in one grid (128 x 128 tiles), problem p split ksplit[p]
// ways (1: y = the product, with bias and residual; more: partials as above).
hipError_t launch_gemm_batch(const GemmArgs* gs, const int* ksplit, int n, hipStream_t s,
                             int num_cus);
// dst[i] = sum_{s < parts} src[s n + i] for i < n (fp32).
hipError_t launch_sum_partials(const float* src, int parts, int64_t n, float* dst, hipStream_t s);
// The same for up to 8 independent (src, parts, n, dst) sums in one launch.
struct SumJob {
  const float* src;
  int parts;
  int64_t n;
  float* dst;
  const void* resid;  // optional: dst[i] also adds resid[i] (bf16 when resid_bf16, else fp32)
  int resid_bf16;
};
hipError_t launch_sum_partials_multi(const SumJob* jobs, int n, hipStream_t s);

hipError_t launch_gemm(int dtype, const GemmArgs& g, hipStream_t s);

// ---- row kernels -------------------------------------------------------------------
// out[m] = LayerNorm(y[m]) * gamma + beta, biased variance over D.
hipError_t launch_layer_norm(int dtype, const float* y, const void* gamma, const void* beta,
                             float eps, int64_t rows, int64_t D, void* out, hipStream_t s);
// out[m] = LayerNorm(sum_{p < nparts} parts[p pstride + m D ..] + resid[m]) * gamma
// + beta (fp32 partials, resid/gamma/beta/out of the dtype), and y[m] = that sum
// when y is not NULL.  D a multiple of 256 up to 2048, 16-byte aligned fp32
// rows (layer_norm_parts_ok).
bool layer_norm_parts_ok(int dtype, const float* parts, int64_t pstride, const void* resid,
                         const void* gamma, const void* beta, int64_t D, const void* out,
                         const float* y);
hipError_t launch_layer_norm_parts(int dtype, const float* parts, int nparts, int64_t pstride,
                                   const void* resid, const void* gamma, const void* beta,
                                   float eps, int64_t rows, int64_t D, void* out, float* y,
                                   hipStream_t s);
// ring[b][(slot0 + t) % cap] = src[b][row0 + t] for t < n, rows of D elements.
hipError_t launch_ring_copy(int dtype, void* ring, int64_t cap, int64_t slot0,
                            const void* src, int64_t src_rows, int64_t row0, int64_t n,
                            int64_t B, int64_t D, hipStream_t s);
// p[0 .. n) = value
hipError_t launch_fill_f32(float* p, int64_t n, float value, hipStream_t s);
// bf16 rows copied to a wider pitch with zero columns past the source width:
// dst[r][c] = src row r element c for c < C, 0 for C <= c < Cpad.  Source row r
// is RowGather's logical row r (the memory ring and the current rows, or one
// plain matrix); src.cur and src.mem both NULL write rows of zeros.  C, Cpad
// and the source pitch even, source rows and dst 4-byte aligned; R * Cpad below
// 2^31 (pad_job_ok).
struct PadJob {
  RowGather src;
  int64_t R, C, Cpad;
  uint16_t* dst;
};
constexpr int PAD_MAX = 8;
bool pad_job_ok(const PadJob& j);
hipError_t launch_pad_rows(const PadJob* jobs, int n, hipStream_t s);

// Static device scratch of txl_rel_attn_fwd_noalloc (static_scratch.hip): its
// size, and its address on the current device (looked up once per device).
constexpr size_t STATIC_SCRATCH_BYTES = (size_t)16 << 20;
hipError_t static_scratch_ptr(void** out);

}  // namespace txl
