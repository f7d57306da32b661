// Row gather and epilogue helpers shared by the projection GEMM kernels.
#pragma once
#include "txl_internal.h"

namespace txl {

// Address of logical row m of the gathered A operand (see RowGather).
__device__ inline const char* gather_row(const RowGather& a, int64_t m, int es) {
  const int64_t per = a.mem_len + a.cur_rows;
  const int64_t b = m / per, t = m - b * per;
  if (t < a.mem_len) {
    int64_t slot = a.mem_start + t;
    if (slot >= a.mem_cap) slot -= a.mem_cap;
    return (const char*)a.mem + (b * a.mem_cap + slot) * a.lda * es;
  }
  return (const char*)a.cur + (b * a.cur_rows + (t - a.mem_len)) * a.lda * es;
}

__device__ inline const char* weight_row(const WeightPair& w, int64_t n, int es) {
  const bool second = n >= w.n_split;
  if (second) n -= w.n_split;
  if (w.hd_pad > w.hd_in && w.hd_in > 0) {
    const int64_t head = n / w.hd_pad, c = n - head * w.hd_pad;
    n = head * w.hd_in + (c < w.hd_in ? c : w.hd_in - 1);
  }
  return (const char*)(second ? w.W1 : w.W0) + n * w.ldw * es;
}

// Destination of output element (m, n) for EPI_HEADS.
template <typename T>
__device__ inline T* heads_dst(const GemmArgs& g, int64_t m, int64_t n) {
  const Epilogue& e = g.e;
  const int64_t per = g.a.mem_len + g.a.cur_rows;
  const int64_t b = m / per, t = m - b * per;
  const int64_t which = n / e.HD, nn = n - which * e.HD;
  const int64_t head = nn / e.d, c = nn - head * e.d;
  T* base = (T*)(which ? e.dst1 : e.dst0);
  return base + b * e.sb + head * e.sh + ring_t(e, t) * e.st + c;
}

// Residual element i of an EPI_RESID_F32 output: 0 without one, else fp32 or
// the input dtype T (Epilogue::resid_f32).
template <typename T>
__device__ inline float resid_at(const Epilogue& e, int64_t i) {
  if (e.resid == nullptr) return 0.f;
  return e.resid_f32 ? ((const float*)e.resid)[i] : Elt<T>::load((const T*)e.resid + i);
}

// acc + bias[n], then the activation (EPI_HEADS) -- see Epilogue::bias.
template <typename T>
__device__ inline float epi_value(const Epilogue& e, int64_t n, float acc) {
  if (e.bias) acc += Elt<T>::load((const T*)e.bias + n);
  if (e.mode == EPI_HEADS && e.act == ACT_RELU) acc = acc > 0.f ? acc : 0.f;
  return acc;
}

// Stores element (m, n) of a head-major output (a padding element of a
// head-padded column as zero); the store of a head's last element also clears
// the row's padding past d when pad > d.
template <typename T>
__device__ inline void heads_store(const GemmArgs& g, int64_t m, int64_t n, float acc) {
  T* p = heads_dst<T>(g, m, n);
  if (g.e.d_valid > 0 && (n % g.e.HD) % g.e.d >= g.e.d_valid) acc = 0.f;
  Elt<T>::store(p, acc);
  // (padding is less than 8 elements: a fixed-trip loop)
  if (g.e.pad > g.e.d && (n % g.e.HD) % g.e.d == g.e.d - 1) {
#pragma unroll
    for (int c = 1; c < 8; ++c)
      if (c <= g.e.pad - g.e.d) Elt<T>::store(p + c, 0.f);
  }
}

template <typename T>
__device__ inline void epilogue_store(const GemmArgs& g, int64_t m, int64_t n, float acc) {
  acc = epi_value<T>(g.e, n, acc);
  if (g.e.mode == EPI_HEADS) {
    heads_store<T>(g, m, n, acc);
  } else {
    g.e.y[m * g.N + n] = acc + resid_at<T>(g.e, m * g.N + n);
  }
}

hipError_t launch_gemm_generic(int dtype, const GemmArgs& g, hipStream_t s);
hipError_t launch_gemm_mfma(const GemmArgs& g, hipStream_t s, int num_cus);
// Up to four independent problems in one grid (all must be gemm_mfma_supported).
hipError_t launch_gemm_mfma_multi(const GemmArgs* g, int n, hipStream_t s, int num_cus);
bool gemm_mfma_supported(const GemmArgs& g);

// h_out = LayerNorm(a W^T + bias + resid) * gamma + beta for bf16 rows of width D
// (D <= 512 and even, K % 32 == 0; a and W 16-byte aligned; resid, gamma, beta,
// bias and out 16-byte aligned when D % 64 == 0, else 4-byte aligned).
struct LnArgs {
  int64_t M, D, K;        // rows, width, inner size
  const void* a;          // [M][K]
  const void* W;          // [D][K]
  const void* resid;      // [M][D]
  const void* gamma;      // [D]
  const void* beta;       // [D]
  float eps;
  void* out;              // [M][D]
  const void* bias;       // [D] added before the residual, or NULL
};
bool gemm_ln_supported(const LnArgs& p);
hipError_t launch_gemm_ln(const LnArgs& p, hipStream_t s);

}  // namespace txl
