// Relative-position attention for one query per (batch row, head): the
// one-token decode step (Transformer-XL section 3.3's score A^rel with terms
// (a)-(d); Appendix B: key j of the query at distance mem_len - j), bf16.
//
// The matrix-core kernel works on 128-query tiles; with one query almost all of
// its work is padding, and what remains is a dot product per key.  Here the
// T = mem_len + 1 keys of a (batch, head) are split into parts of at most
// DEC_KMAX keys, one 256-thread workgroup per part; wave w takes keys
// 32 w .. 32 w + 31 of the part.  Lane l of a wave reads the 8-column piece
// l % 8 of key rows 8 i + l / 8 (i = 0..3), so every load instruction moves
// eight whole rows (1 KB with 64 columns), and every load the wave makes (key,
// r and value rows) is issued before the first is used:
//   - (q+u) and (q+v), scaled by scale * log2(e), are staged in LDS, and each
//     lane keeps the 8 columns of its piece;
//   - a score is the sum over a group of 8 lanes (DPP swaps and a half-row
//     mirror);
//   - the part's maximum and sum of exp2(s - max) are reduced over the
//     workgroup (DPP wave reductions, LDS across waves);
//   - each lane accumulates P.V for its piece's columns over its 4 keys; the
//     lanes sharing a piece are added with a DPP row rotation, then in LDS.
// With several parts each writes (max, sum, unnormalised output) and
// attn_decode_merge_kernel, launched after it on the same stream, combines them
// (out = sum_p 2^(m_p - m) acc_p / sum_p 2^(m_p - m) l_p); with one part the
// output is written directly.
#include "txl_internal.h"

namespace txl {
namespace {

constexpr int DEC_T = 256;          // threads per workgroup
constexpr int DEC_KMAX = 128;       // keys per part at most (32 per wave)
constexpr int DEC_MAXP = 1024;      // parts per (batch, head) at most
constexpr int DEC_D = 64;           // head size bound (padded row columns read)
constexpr int DEC_REC = DEC_D + 2;  // partial record: m, l, acc[64]
constexpr int DEC_MPRE = 8;         // partial outputs prefetched per wave by the merge
constexpr float LOG2E = 1.4426950408889634f;

__device__ inline float bf_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ inline float bf_hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xffff0000u); }

// Workgroup (4 waves) maximum / sum; red holds 4 floats.
__device__ inline float block_max(float x, float* red) {
  x = wave_allmax(x);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = x;
  __syncthreads();
  return fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}
__device__ inline float block_sum(float x, float* red) {
  x = wave_allsum(x);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = x;
  __syncthreads();
  return (red[0] + red[1]) + (red[2] + red[3]);
}

// Row of key j in k / v: j itself, or (kv_start + j) % kv_cap for a ring
// (0 <= j < kv_cap); 32-bit (attn_decode_supported bounds the slab).
__device__ inline int ring_row(int kvs, int kvc, int j) {
  const int p = kvs + j;
  return p >= kvc ? p - kvc : p;
}

__global__ __launch_bounds__(DEC_T) void attn_decode_kernel(AttnArgs a, int nparts, float* part) {
  __shared__ float qs[2][DEC_D];
  __shared__ float red[4];
  __shared__ float accs[4][4][DEC_D];  // [wave][row of 16 lanes][column]
  // (32-bit index arithmetic: B H <= 65535, parts <= DEC_MAXP and
  // T <= DEC_KMAX DEC_MAXP, so parts * T < 2^31)
  const unsigned pid = blockIdx.x, g = blockIdx.y, H = (unsigned)a.H, np = (unsigned)nparts;
  const int64_t b = g / H, hd = g % H;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int d = (int)a.d, dl = (int)a.d_load;
  const int len = (int)a.mem_len, T = len + 1;
  const int j_lo = (int)(pid * (unsigned)T / np);
  const int n = (int)((pid + 1) * (unsigned)T / np) - j_lo;
  const int kvs = a.kv_cap > 0 ? (int)a.kv_start : 0;
  const int kvc = a.kv_cap > 0 ? (int)a.kv_cap : 0x7fffffff;
  const int kst = (int)a.kv_st, rsp = (int)a.r_sp;
  const uint16_t* kb = (const uint16_t*)a.k + b * a.kv_sb + hd * a.kv_sh;
  const uint16_t* vb = (const uint16_t*)a.v + b * a.kv_sb + hd * a.kv_sh;
  const uint16_t* rb = (const uint16_t*)a.r + hd * a.r_sh;

  // Loads, all unconditional (no branch between them, so none waits for
  // another): a key past the part is read as the part's first key and a piece
  // past d_load as piece 0; what such a load brings is discarded (the score
  // is masked, or it meets zero query columns, or it lands in columns >= d_load
  // that are never stored).
  const int pc = lane & 7, c0 = 8 * pc, cl = c0 < dl ? c0 : 0;
  const int kk0 = 32 * wave + (lane >> 3);  // key of load i: kk0 + 8 i
  uint4 kw[4], rw[4], vw[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int kk = kk0 + 8 * i;
    const int j = j_lo + (kk < n ? kk : 0);
    const int row = ring_row(kvs, kvc, j);
    kw[i] = *(const uint4*)(kb + (row * kst + cl));
    rw[i] = *(const uint4*)(rb + ((len - j) * rsp + cl));
    vw[i] = *(const uint4*)(vb + (row * kst + cl));
  }
  // the query with its biases, in the exp2 domain; zero past d
  if (tid < DEC_D) {
    const float sl2 = a.scale * LOG2E;
    float x = 0.f, uu = 0.f, vv = 0.f;
    if (tid < d) {
      x = bf16_to_f32(((const uint16_t*)a.q)[b * a.q_sb + hd * a.q_sh + tid]);
      uu = bf16_to_f32(((const uint16_t*)a.u)[hd * d + tid]);
      vv = bf16_to_f32(((const uint16_t*)a.vb)[hd * d + tid]);
    }
    qs[0][tid] = (x + uu) * sl2;
    qs[1][tid] = (x + vv) * sl2;
  }
  __syncthreads();
  float qc[8], qp[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    qc[e] = qs[0][c0 + e];
    qp[e] = qs[1][c0 + e];
  }

  // scores: content term against k, position term against r, summed over the
  // 8 lanes of the row group
  float sc[4];
  float mx = -INFINITY;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t k4[4] = {kw[i].x, kw[i].y, kw[i].z, kw[i].w};
    const uint32_t r4[4] = {rw[i].x, rw[i].y, rw[i].z, rw[i].w};
    float t = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      t += qc[2 * e] * bf_lo(k4[e]) + qc[2 * e + 1] * bf_hi(k4[e]);
      t += qp[2 * e] * bf_lo(r4[e]) + qp[2 * e + 1] * bf_hi(r4[e]);
    }
    t += dpp_f32<0xB1, 0xf>(0.f, t);   // quad_perm [1,0,3,2]
    t += dpp_f32<0x4E, 0xf>(0.f, t);   // quad_perm [2,3,0,1]
    t += dpp_f32<0x141, 0xf>(0.f, t);  // row_half_mirror: the 8-lane sum
    sc[i] = kk0 + 8 * i < n ? t : -INFINITY;
    mx = fmaxf(mx, sc[i]);
  }
  const float m = block_max(mx, red);
  float ls = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    sc[i] = __builtin_amdgcn_exp2f(sc[i] - m);  // 0 for a masked key
    ls += sc[i];
  }
  const float l = block_sum(pc == 0 ? ls : 0.f, red);

  // P.V for this piece's 8 columns over the lane's 4 keys
  float o[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t v4[4] = {vw[i].x, vw[i].y, vw[i].z, vw[i].w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      o[2 * e] += sc[i] * bf_lo(v4[e]);
      o[2 * e + 1] += sc[i] * bf_hi(v4[e]);
    }
  }
  // lanes l and l ^ 8 of a row of 16 share a piece: row_ror:8, then LDS
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] += dpp_f32<0x128, 0xf>(0.f, o[e]);
  if ((lane & 8) == 0) {
    float* dst = &accs[wave][lane >> 4][c0];
    *(float4*)dst = make_float4(o[0], o[1], o[2], o[3]);
    *(float4*)(dst + 4) = make_float4(o[4], o[5], o[6], o[7]);
  }
  __syncthreads();
  if (tid < DEC_D) {
    float acc = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc += accs[w][r][tid];
    if (nparts == 1) {
      if (tid < d)
        ((uint16_t*)a.out)[b * a.o_sb + hd * a.o_sh + tid] = f32_to_bf16(acc / l);
    } else {
      float* rec = part + ((int64_t)g * nparts + pid) * DEC_REC;
      rec[2 + tid] = acc;
      if (tid == 0) {
        rec[0] = m;
        rec[1] = l;
      }
    }
  }
}

// One workgroup per (batch, head): the parts' maxima and sums read in
// parallel, then wave w adds the outputs of parts w, w + 4, ... (lane = column);
// the first DEC_MPRE of those outputs are loaded together with the maxima.
__global__ __launch_bounds__(DEC_T) void attn_decode_merge_kernel(AttnArgs a, int nparts,
                                                                  const float* part) {
  __shared__ float wsh[DEC_MAXP];
  __shared__ float red[4];
  __shared__ float accs[4][DEC_D];
  const unsigned g = blockIdx.x, H = (unsigned)a.H;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t b = g / H, hd = g % H;
  const float* rec = part + (int64_t)g * nparts * DEC_REC;
  float pre[DEC_MPRE];
#pragma unroll
  for (int i = 0; i < DEC_MPRE; ++i) {
    const int p = wave + 4 * i;
    pre[i] = rec[(int64_t)(p < nparts ? p : 0) * DEC_REC + 2 + lane];
  }
  float mp[DEC_MAXP / DEC_T], lp[DEC_MAXP / DEC_T];
  float m = -INFINITY;
#pragma unroll
  for (int i = 0; i < DEC_MAXP / DEC_T; ++i) {
    const int p = tid + i * DEC_T;
    mp[i] = p < nparts ? rec[(int64_t)p * DEC_REC] : -INFINITY;
    lp[i] = p < nparts ? rec[(int64_t)p * DEC_REC + 1] : 0.f;
    m = fmaxf(m, mp[i]);
  }
  m = block_max(m, red);
  float den = 0.f;
#pragma unroll
  for (int i = 0; i < DEC_MAXP / DEC_T; ++i) {
    const int p = tid + i * DEC_T;
    if (p < nparts) {
      const float w = __builtin_amdgcn_exp2f(mp[i] - m);
      wsh[p] = w;
      den += w * lp[i];
    }
  }
  den = block_sum(den, red);  // (its barriers publish wsh)
  float num = 0.f;
#pragma unroll
  for (int i = 0; i < DEC_MPRE; ++i) {
    const int p = wave + 4 * i;
    num += p < nparts ? wsh[p] * pre[i] : 0.f;
  }
#pragma unroll 8
  for (int p = wave + 4 * DEC_MPRE; p < nparts; p += 4)
    num += wsh[p] * rec[(int64_t)p * DEC_REC + 2 + lane];
  accs[wave][lane] = num;
  __syncthreads();
  if (tid < a.d) {
    const float o = (accs[0][tid] + accs[1][tid]) + (accs[2][tid] + accs[3][tid]);
    ((uint16_t*)a.out)[b * a.o_sb + hd * a.o_sh + tid] = f32_to_bf16(o / den);
  }
}

}  // namespace

bool attn_decode_supported(const AttnArgs& a) {
  if (a.L != 1 || a.scores || a.lse) return false;
  if (a.d > DEC_D || a.d_load > DEC_D || a.d_load % 8 != 0) return false;
  if (a.mem_len + 1 > (int64_t)DEC_KMAX * DEC_MAXP) return false;
  if (a.B * a.H > 65535) return false;
  // 32-bit element offsets inside a (batch, head) slab
  const int64_t krows = a.kv_cap > 0 ? a.kv_cap : a.mem_len + 1;
  if (krows * a.kv_st + DEC_D > 0x7fffffffLL || (a.mem_len + 1) * a.r_sp + DEC_D > 0x7fffffffLL)
    return false;
  const uintptr_t al = (uintptr_t)a.k | (uintptr_t)a.v | (uintptr_t)a.r;
  if (al % 16) return false;
  const int64_t st[] = {a.kv_sb, a.kv_st, a.kv_sh, a.r_sp, a.r_sh};
  for (int64_t s : st)
    if (s % 8) return false;
  return true;
}

// Parts for this shape: at most DEC_KMAX keys each, and more (down to 64 keys a
// part) while the grid is below two workgroups per CU; 0 when the keys do not
// fit one part and there is no room for the partials (the caller then takes
// another path).
int attn_decode_parts(const AttnArgs& a, int num_cus, size_t scratch_bytes) {
  const int64_t T = a.mem_len + 1, groups = a.B * a.H;
  const int64_t min_parts = (T + DEC_KMAX - 1) / DEC_KMAX;
  int64_t fill = (2 * (int64_t)num_cus + groups - 1) / groups;
  const int64_t by_keys = (T + 63) / 64;
  fill = fill < by_keys ? fill : by_keys;
  int64_t want = fill > min_parts ? fill : min_parts;
  while (want > min_parts && attn_decode_bytes(a, (int)want) > scratch_bytes) --want;
  if (want > 1 && attn_decode_bytes(a, (int)want) > scratch_bytes) return 0;
  return (int)want;
}

size_t attn_decode_bytes(const AttnArgs& a, int nparts) {
  return nparts > 1 ? (size_t)(a.B * a.H) * nparts * DEC_REC * sizeof(float) + 256 : 0;
}

hipError_t launch_attn_decode(const AttnArgs& a, int nparts, void* scratch, hipStream_t s) {
  if (nparts < 1 || nparts > DEC_MAXP || (a.mem_len + nparts) / nparts > DEC_KMAX)
    return hipErrorInvalidValue;
  if (nparts > 1 && !scratch) return hipErrorInvalidValue;
  float* part = (float*)(((uintptr_t)scratch + 255) & ~(uintptr_t)255);
  const unsigned groups = (unsigned)(a.B * a.H);
  hipLaunchKernelGGL(attn_decode_kernel, dim3((unsigned)nparts, groups), dim3(DEC_T), 0, s, a,
                     nparts, part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || nparts == 1) return e;
  hipLaunchKernelGGL(attn_decode_merge_kernel, dim3(groups), dim3(DEC_T), 0, s, a, nparts,
                     (const float*)part);
  return hipGetLastError();
}

}  // namespace txl
