// Relative-position attention, generic path: any strides, d_head <= 128,
// fp32 or bf16 storage, fp32 arithmetic.  One wavefront per (query, head,
// batch row); it walks the visible keys 64 at a time with an online softmax.
//
// Score (Transformer-XL, section 3.3, A^rel): for key j <= mem_len + i and
// distance p = mem_len + i - j,
//   A = scale * ((q_i + u) . k_j + (q_i + v) . r_p)
// which is terms (a)+(c) plus (b)+(d); keys past the query are masked.
#include "txl_internal.h"

namespace txl {
namespace {

__device__ inline float wave_max(float x) {
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
  return x;
}
__device__ inline float wave_sum(float x) {
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}

template <typename T>
__global__ __launch_bounds__(64) void attn_generic_kernel(AttnArgs a) {
  const int64_t i = blockIdx.x, hd = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x;
  const int64_t d = a.d;
  const int64_t T_all = a.mem_len + a.L;
  const int64_t nvis = a.mem_len + i + 1;  // keys 0 .. mem_len+i are visible

  __shared__ float qc[128], qp[128], pw[64];
  const T* q = (const T*)a.q + b * a.q_sb + i * a.q_st + hd * a.q_sh;
  const T* u = (const T*)a.u + hd * d;
  const T* vb = (const T*)a.vb + hd * d;
  for (int64_t c = lane; c < d; c += 64) {
    const float qv = Elt<T>::load(q + c);
    qc[c] = qv + Elt<T>::load(u + c);   // query for terms (a) + (c)
    qp[c] = qv + Elt<T>::load(vb + c);  // query for terms (b) + (d)
  }
  __syncthreads();

  const T* kb = (const T*)a.k + b * a.kv_sb + hd * a.kv_sh;
  const T* vbase = (const T*)a.v + b * a.kv_sb + hd * a.kv_sh;
  const T* rb = (const T*)a.r + hd * a.r_sh;
  float* srow = a.scores ? a.scores + ((b * a.H + hd) * a.L + i) * T_all : nullptr;

  float m = -INFINITY, l = 0.f, acc0 = 0.f, acc1 = 0.f;
  for (int64_t j0 = 0; j0 < nvis; j0 += 64) {
    const int64_t j = j0 + lane;
    float s = -INFINITY;
    if (j < nvis) {
      const T* kj = kb + kv_row(a, j) * a.kv_st;
      const T* rp = rb + (a.mem_len + i - j) * a.r_sp;
      float acc = 0.f;
      for (int64_t c = 0; c < d; ++c)
        acc += qc[c] * Elt<T>::load(kj + c) + qp[c] * Elt<T>::load(rp + c);
      s = acc * a.scale;
    }
    if (srow && j < T_all) srow[j] = s;
    const float m_new = fmaxf(m, wave_max(s));
    const float alpha = __expf(m - m_new);
    const float p = j < nvis ? __expf(s - m_new) : 0.f;
    l = l * alpha + wave_sum(p);
    pw[lane] = p;
    __syncthreads();
    acc0 *= alpha;
    acc1 *= alpha;
    const int64_t nk = nvis - j0 < 64 ? nvis - j0 : 64;
    for (int64_t jj = 0; jj < nk; ++jj) {
      const T* vj = vbase + kv_row(a, j0 + jj) * a.kv_st;
      const float pj = pw[jj];
      if (lane < d) acc0 += pj * Elt<T>::load(vj + lane);
      if (lane + 64 < d) acc1 += pj * Elt<T>::load(vj + lane + 64);
    }
    __syncthreads();
    m = m_new;
  }
  if (srow)
    for (int64_t j = nvis + lane; j < T_all; j += 64) srow[j] = -INFINITY;
  T* o = (T*)a.out + b * a.o_sb + i * a.o_st + hd * a.o_sh;
  const float inv = 1.f / l;
  if (lane < d) Elt<T>::store(o + lane, acc0 * inv);
  if (lane + 64 < d) Elt<T>::store(o + lane + 64, acc1 * inv);
}

}  // namespace

hipError_t launch_attn_generic(int dtype, const AttnArgs& a, hipStream_t s) {
  dim3 grid((unsigned)a.L, (unsigned)a.H, (unsigned)a.B);
  if (dtype == 0)
    hipLaunchKernelGGL(attn_generic_kernel<float>, grid, dim3(64), 0, s, a);
  else
    hipLaunchKernelGGL(attn_generic_kernel<uint16_t>, grid, dim3(64), 0, s, a);
  return hipGetLastError();
}

}  // namespace txl
