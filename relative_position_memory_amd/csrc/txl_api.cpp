// C ABI of libtxl.so: argument validation, workspace layout and launch plans.
// Every check runs before the first launch, so a failing call writes nothing.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <vector>

#include "../../include/txl.h"
#include "gemm_common.h"
#include "txl_internal.h"

namespace {

thread_local char g_detail[512] = "";
thread_local char g_msg[640] = "";

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_detail, sizeof(g_detail), fmt, ap);
  va_end(ap);
  return status;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(TXL_EHIP, "%s: %s", what, hipGetErrorString(e));
}

int64_t elt_size(int dtype) { return dtype == TXL_FP32 ? 4 : 2; }

// Byte span [lo, hi) touched by a [n0][n1][n2][d] tensor with strides s0, s1, s2.
struct Span { uintptr_t lo, hi; };
Span span4(const void* p, int64_t n0, int64_t s0, int64_t n1, int64_t s1, int64_t n2, int64_t s2,
           int64_t d, int64_t es) {
  const int64_t last = (n0 - 1) * s0 + (n1 - 1) * s1 + (n2 - 1) * s2 + d;
  return {(uintptr_t)p, (uintptr_t)p + (uintptr_t)(last * es)};
}
bool overlap(Span a, Span b) { return a.lo < b.hi && b.lo < a.hi; }

bool stride_ok(int64_t n, int64_t s, int64_t d) { return n <= 1 || s >= d; }

int num_cus() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0)
      n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

int64_t round_up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }

// Workspace layout of txl_layer_step (byte offsets, each 256-aligned).
struct WsLayout {
  int64_t dp;                      // padded head size of q/k/v/r rows
  size_t q, k, v, r, a, y, part, opart, total;  // offsets and total bytes
  // zero-padded operand copies (pad_k): context rows [B][T][Dp], R rows [T][Dp],
  // W_q, W_kE, W_v, W_kR [H d][Dp] each; W_o [D][HDp] and a [B L][HDp]
  int64_t Dp, HDp;
  size_t xa, xr, xw, xwo, xo;
};

// bf16 products over rows that are not whole 32-element K steps (d_model or
// H d not a multiple of 32) run on copies padded with zero columns to the next
// multiple of 32, which the LDS-direct product takes (its K loop moves whole
// 32-deep steps of 16-byte pieces).
int64_t pad_k(int64_t es, int64_t K) {
  return es == 2 && K % 32 != 0 && K % 2 == 0 ? round_up(K, 32) : 0;
}

// K splits of the unfused output projection y = a W_o^T + h: when its 128 x 128
// tiles would leave most of a 256-CU chip idle (a few rows, as at a long-memory
// evaluation segment), about 128 workgroups, each at least two K steps of 32
// deep; when they would fill less than half of its 512 workgroup slots, two
// (a fixed rule of the dims, so the workspace does not depend on the device).
int out_splits(const txl_layer_dims& dm) {
  const int64_t BL = dm.B * dm.L, D = dm.d_model, HD = dm.n_head * dm.d_head;
  const int64_t tiles = ((BL + 127) / 128) * ((D + 127) / 128);
  if (HD % 32 != 0) return 1;
  if (tiles >= 64) return tiles < 256 && HD >= 256 ? 2 : 1;
  int64_t ks = (128 + tiles - 1) / tiles;
  ks = std::min<int64_t>(ks, std::min<int64_t>(HD / 64, 16));
  return ks > 1 ? (int)ks : 1;
}
// part_bytes: room for the attention's key-split partials (0 when it does not split)
WsLayout ws_layout(const txl_layer_dims& dm, int64_t T, int64_t es, size_t part_bytes = 0) {
  WsLayout w;
  w.dp = round_up(dm.d_head, 8);
  const int64_t B = dm.B, H = dm.n_head, L = dm.L;
  size_t off = 0;
  auto take = [&](int64_t bytes) {
    const size_t o = off;
    off += (size_t)round_up(bytes, 256);
    return o;
  };
  w.q = take(B * H * L * w.dp * es);
  w.k = take(B * H * T * w.dp * es);
  w.v = take(B * H * T * w.dp * es);
  w.r = take(H * T * w.dp * es);
  w.a = take(B * L * H * dm.d_head * es);
  w.y = take(B * L * dm.d_model * 4);
  const int64_t D = dm.d_model, HD = H * dm.d_head;
  w.Dp = pad_k(es, D);
  w.HDp = pad_k(es, HD);
  w.xa = take(w.Dp ? B * T * w.Dp * es : 0);
  w.xr = take(w.Dp ? T * w.Dp * es : 0);
  w.xw = take(w.Dp ? 4 * HD * w.Dp * es : 0);
  w.xwo = take(w.HDp ? D * w.HDp * es : 0);
  w.xo = take(w.HDp ? B * L * w.HDp * es : 0);
  w.part = take((int64_t)part_bytes);
  // the output projection's K-split partials (bf16 layers)
  const int ks = out_splits(dm);
  w.opart = take(es == 2 && ks > 1 ? ks * B * L * dm.d_model * 4 : 0);
  w.total = off;
  return w;
}

int check_dims(const txl_layer_dims* dm) {
  if (!dm) return fail(TXL_EINVAL, "dims is NULL");
  if (dm->B < 1 || dm->L < 1 || dm->d_model < 1 || dm->n_head < 1 || dm->d_head < 1)
    return fail(TXL_EINVAL, "dims must be >= 1 (B=%lld L=%lld D=%lld H=%lld d=%lld)",
                (long long)dm->B, (long long)dm->L, (long long)dm->d_model,
                (long long)dm->n_head, (long long)dm->d_head);
  if (dm->d_head > 128) return fail(TXL_EUNSUPPORTED, "d_head %lld > 128", (long long)dm->d_head);
  if (!(dm->ln_eps >= 0.f) || !isfinite(dm->ln_eps))
    return fail(TXL_EINVAL, "ln_eps must be finite and >= 0");
  if (dm->n_head > 65535 || dm->B > 65535)
    return fail(TXL_EUNSUPPORTED, "B and n_head must be <= 65535");
  return TXL_OK;
}

int check_attn(int dtype, const txl::AttnArgs& a, int64_t r_rows) {
  if (dtype != TXL_FP32 && dtype != TXL_BF16) return fail(TXL_EUNSUPPORTED, "dtype %d", dtype);
  if (a.B < 1 || a.H < 1 || a.L < 1 || a.mem_len < 0)
    return fail(TXL_EINVAL, "B, H, L must be >= 1 and mem_len >= 0");
  if (a.d < 1) return fail(TXL_EINVAL, "d_head must be >= 1");
  if (a.d > 128) return fail(TXL_EUNSUPPORTED, "d_head %lld > 128", (long long)a.d);
  if (a.H > 65535 || a.B > 65535 || a.L > 0x7fffffffLL)
    return fail(TXL_EUNSUPPORTED, "B, H must be <= 65535 and L < 2^31");
  if (!a.q || !a.k || !a.v || !a.r || !a.u || !a.vb || !a.out)
    return fail(TXL_EINVAL, "NULL tensor pointer");
  const int64_t T = a.mem_len + a.L;
  if (r_rows < T)
    return fail(TXL_EINVAL, "r_rows %lld < mem_len + L = %lld", (long long)r_rows, (long long)T);
  const int64_t ss[] = {a.q_sb, a.q_st, a.q_sh, a.kv_sb, a.kv_st, a.kv_sh, a.r_sp, a.r_sh,
                        a.o_sb, a.o_st, a.o_sh};
  for (int64_t s : ss)
    if (s < 0) return fail(TXL_EINVAL, "negative stride");
  if (!stride_ok(a.L, a.q_st, a.d) || !stride_ok(a.H, a.q_sh, a.d) ||
      !stride_ok(T, a.kv_st, a.d) || !stride_ok(a.H, a.kv_sh, a.d) ||
      !stride_ok(T, a.r_sp, a.d) || !stride_ok(a.H, a.r_sh, a.d) ||
      !stride_ok(a.L, a.o_st, a.d) || !stride_ok(a.H, a.o_sh, a.d))
    return fail(TXL_EINVAL, "a token/head stride is below d_head");
  if (!isfinite(a.scale)) return fail(TXL_EINVAL, "scale is not finite");
  const int64_t es = elt_size(dtype);
  const Span so = span4(a.out, a.B, a.o_sb, a.L, a.o_st, a.H, a.o_sh, a.d, es);
  const Span in[] = {span4(a.q, a.B, a.q_sb, a.L, a.q_st, a.H, a.q_sh, a.d, es),
                     span4(a.k, a.B, a.kv_sb, T, a.kv_st, a.H, a.kv_sh, a.d, es),
                     span4(a.v, a.B, a.kv_sb, T, a.kv_st, a.H, a.kv_sh, a.d, es),
                     span4(a.r, 1, 0, T, a.r_sp, a.H, a.r_sh, a.d, es),
                     span4(a.u, 1, 0, 1, 0, 1, 0, a.H * a.d, es),
                     span4(a.vb, 1, 0, 1, 0, 1, 0, a.H * a.d, es)};
  for (const Span& s : in)
    if (overlap(so, s)) return fail(TXL_EINVAL, "out overlaps an input");
  if (a.scores) {
    const Span sd = {(uintptr_t)a.scores, (uintptr_t)(a.scores + a.B * a.H * a.L * T)};
    if (overlap(sd, so)) return fail(TXL_EINVAL, "scores_dbg overlaps out");
    for (const Span& s : in)
      if (overlap(sd, s)) return fail(TXL_EINVAL, "scores_dbg overlaps an input");
  }
  return TXL_OK;
}

// Bytes of key-split partials the attention's plan needs (0 = none): the
// single-query kernel's parts for one query per (batch, head), else the
// matrix-core plan's.
size_t attn_plan_bytes(int dtype, const txl::AttnArgs& a) {
  if (dtype != TXL_BF16) return 0;
  if (txl::attn_decode_supported(a))
    return txl::attn_decode_bytes(a, txl::attn_decode_parts(a, num_cus(), (size_t)-1));
  if (!txl::attn_mfma_supported(a)) return 0;
  return txl::attn_plan_bytes(a, txl::attn_mfma_plan(a, num_cus(), (size_t)-1));
}

// Bytes of key-split partials the layer step's attention needs at this memory length.
size_t layer_part_bytes(const txl_layer_dims& dm, int64_t mem_len, int dtype) {
  txl::AttnArgs a{};
  const int64_t dp = round_up(dm.d_head, 8), T = mem_len + dm.L;
  a.B = dm.B; a.H = dm.n_head; a.L = dm.L; a.mem_len = mem_len; a.d = dm.d_head;
  a.d_load = dp;
  a.q = a.k = a.v = a.r = (const void*)(uintptr_t)256;  // workspace regions are aligned
  a.q_sb = dm.n_head * dm.L * dp; a.q_st = dp; a.q_sh = dm.L * dp;
  a.kv_sb = dm.n_head * T * dp; a.kv_st = dp; a.kv_sh = T * dp;
  a.r_sp = dp; a.r_sh = T * dp;
  return attn_plan_bytes(dtype, a);
}

// Runs the attention; scratch (may be NULL) holds the key-split partials when
// the plan splits the keys and scratch_bytes covers them, else no split.
int run_attn(int dtype, txl::AttnArgs a, void* scratch, size_t scratch_bytes, hipStream_t st) {
  const int64_t T = a.mem_len + a.L;
  hipError_t e;
  if (a.scores) {
    e = txl::launch_fill_f32(a.scores, a.B * a.H * a.L * T, -INFINITY, st);
    if (e != hipSuccess) return hip_fail(e, "scores fill");
  }
  const int dec_parts = dtype == TXL_BF16 && txl::attn_decode_supported(a)
                            ? txl::attn_decode_parts(a, num_cus(), scratch ? scratch_bytes : 0)
                            : 0;
  if (dec_parts > 0) {
    e = txl::launch_attn_decode(a, dec_parts, scratch, st);
  } else if (dtype == TXL_BF16 && txl::attn_mfma_supported(a)) {
    // the best plan whose partials fit the scratch (none: no split)
    const txl::AttnPlan plan = txl::attn_mfma_plan(a, num_cus(), scratch ? scratch_bytes : 0);
    txl::attn_plan_bind(a, plan, scratch);
    e = txl::launch_attn_mfma(a, num_cus(), st);
  } else {
    e = txl::launch_attn_generic(dtype, a, st);
  }
  if (e != hipSuccess) return hip_fail(e, "attention launch");
  return TXL_OK;
}

int run_gemm(int dtype, const txl::GemmArgs& g, hipStream_t st, const char* what);

// Columns of a head-major projection over nw stacked weights of H heads of d
// rows each, stored with rows padded to dp: the GEMM produces dp columns per
// head (the ones past d from a repeated weight row, stored as zeros), so that
// every output row is whole 16-byte pieces of the workspace layout.
void head_padded_cols(txl::GemmArgs& g, int64_t nw, int64_t H, int64_t d, int64_t dp) {
  g.N = nw * H * dp;
  g.w.n_split = H * dp;
  g.w.hd_in = d;
  g.w.hd_pad = dp;
  g.e.HD = H * dp;
  g.e.d = dp;
  g.e.pad = 0;
  g.e.d_valid = d;
}

// h_out = LayerNorm(a W_o^T + h_in) * gamma + beta (section 3.3), a [B*L][H*d]
// token-major; y: fp32 [B*L][D] scratch for the unfused form.
// Whether run_out_ln takes the fused kernel (else it writes y = a W_o^T + h_in,
// fp32, before the LayerNorm).
// a_pad, wo_pad: a and W_o copied to rows of HDp (zero columns past H d), or NULL.
txl::LnArgs out_ln_args(const txl_layer_dims& dm, const void* a, const txl_layer_weights* w,
                        const void* h_in, void* h_out, const void* a_pad, const void* wo_pad,
                        int64_t HDp) {
  const int64_t BL = dm.B * dm.L, D = dm.d_model, HD = dm.n_head * dm.d_head;
  if (a_pad && wo_pad)
    return {BL, D, HDp, a_pad, wo_pad, h_in, w->ln_gamma, w->ln_beta, dm.ln_eps, h_out};
  return {BL, D, HD, a, w->W_o, h_in, w->ln_gamma, w->ln_beta, dm.ln_eps, h_out};
}
bool out_ln_fused(int dtype, const txl_layer_dims& dm, const void* a, const txl_layer_weights* w,
                  const void* h_in, void* h_out, const void* a_pad = nullptr,
                  const void* wo_pad = nullptr, int64_t HDp = 0) {
  // (a few rows, as in a decode step, go to the skinny GEMM and the row kernel)
  return dtype == TXL_BF16 && dm.B * dm.L > 32 &&
         txl::gemm_ln_supported(out_ln_args(dm, a, w, h_in, h_out, a_pad, wo_pad, HDp));
}

// need_y: y must hold a W_o^T + h_in afterwards (the unfused form writes it anyway
// unless the LayerNorm sums the K-split partials itself).
int run_out_ln(int dtype, const txl_layer_dims& dm, const void* a, const txl_layer_weights* w,
               const void* h_in, void* h_out, float* y, hipStream_t st, float* opart = nullptr,
               const void* a_pad = nullptr, const void* wo_pad = nullptr, int64_t HDp = 0,
               bool need_y = true) {
  const int64_t BL = dm.B * dm.L, D = dm.d_model, HD = dm.n_head * dm.d_head;
  // one fused kernel when the rows fit it
  const txl::LnArgs ln = out_ln_args(dm, a, w, h_in, h_out, a_pad, wo_pad, HDp);
  if (out_ln_fused(dtype, dm, a, w, h_in, h_out, a_pad, wo_pad, HDp)) {
    const hipError_t e = txl::launch_gemm_ln(ln, st);
    if (e != hipSuccess) return hip_fail(e, "output projection + LayerNorm");
    return TXL_OK;
  }
  // y = a W_o^T + h, then LayerNorm
  txl::GemmArgs g{};
  g.M = BL; g.N = D; g.K = HD;
  g.a = {nullptr, 1, 0, 0, a, BL, HD};
  g.w = {w->W_o, w->W_o, D, HD};
  g.e = {txl::EPI_RESID_F32, nullptr, nullptr, 0, 1, 0, 0, 0, y, h_in};
  if (a_pad && wo_pad) {  // the zero columns add nothing to the sums
    g.K = HDp;
    g.a = {nullptr, 1, 0, 0, a_pad, BL, HDp};
    g.w = {wo_pad, wo_pad, D, HDp};
  }
  int rc;
  const int ks = out_splits(dm);
  if (opart && ks > 1 && dtype == TXL_BF16 && txl::gemm_mfma_supported(g) && g.K % 32 == 0 &&
      (uintptr_t)g.a.cur % 16 == 0 && (uintptr_t)g.w.W0 % 16 == 0) {
    // few rows: K split into partials, summed with the residual into y
    txl::GemmArgs gp = g;
    gp.e.y = opart;
    gp.e.resid = nullptr;
    hipError_t e = txl::launch_gemm_splitk(gp, ks, st, num_cus());
    if (e != hipSuccess) return hip_fail(e, "output projection");
    float* yo = need_y ? y : nullptr;
    if (txl::layer_norm_parts_ok(dtype, opart, BL * D, h_in, w->ln_gamma, w->ln_beta, D, h_out,
                                 yo)) {
      // the partials, the residual and the LayerNorm in one pass
      e = txl::launch_layer_norm_parts(dtype, opart, ks, BL * D, h_in, w->ln_gamma, w->ln_beta,
                                       dm.ln_eps, BL, D, h_out, yo, st);
      if (e != hipSuccess) return hip_fail(e, "output projection sum + layer norm");
      return TXL_OK;
    }
    const txl::SumJob sj = {opart, ks, BL * D, y, h_in, 1};
    e = txl::launch_sum_partials_multi(&sj, 1, st);
    if (e != hipSuccess) return hip_fail(e, "output projection sum");
  } else if ((rc = run_gemm(dtype, g, st, "output projection")) != TXL_OK) {
    return rc;
  }
  const hipError_t e =
      txl::launch_layer_norm(dtype, y, w->ln_gamma, w->ln_beta, dm.ln_eps, BL, D, h_out, st);
  if (e != hipSuccess) return hip_fail(e, "layer norm");
  return TXL_OK;
}

int run_gemm(int dtype, const txl::GemmArgs& g, hipStream_t st, const char* what) {
  if (g.M == 0 || g.N == 0) return TXL_OK;
  hipError_t e;
  if (dtype == TXL_BF16 && txl::gemm_mfma_supported(g))
    e = txl::launch_gemm_mfma(g, st, num_cus());
  else
    e = txl::launch_gemm_generic(dtype, g, st);
  if (e != hipSuccess) return hip_fail(e, what);
  return TXL_OK;
}

// Workspace of txl_layer_step_kv: q [B][H][L][dp], a [B][L][H*d], y fp32
// [B][L][D], then the attention's scratch.
// (with zero-padded copies as in WsLayout: h [B L][Dp], W_q, W_kE, W_v [H d][Dp];
// W_o [D][HDp] and a [B L][HDp])
struct KvWs { size_t q, a, y, xh, xw, xwo, xo, part, total; int64_t dp, Dp, HDp; };
KvWs kv_ws_layout(const txl_layer_dims& dm, int64_t es, size_t part_bytes) {
  KvWs w;
  w.dp = round_up(dm.d_head, 8);
  size_t off = 0;
  auto take = [&](int64_t bytes) {
    const size_t o = off;
    off += (size_t)round_up(bytes, 256);
    return o;
  };
  const int64_t BL = dm.B * dm.L, D = dm.d_model, HD = dm.n_head * dm.d_head;
  w.q = take(dm.B * dm.n_head * dm.L * w.dp * es);
  w.a = take(BL * HD * es);
  w.y = take(BL * D * 4);
  w.Dp = pad_k(es, D);
  w.HDp = pad_k(es, HD);
  w.xh = take(w.Dp ? BL * w.Dp * es : 0);
  w.xw = take(w.Dp ? 3 * HD * w.Dp * es : 0);
  w.xwo = take(w.HDp ? D * w.HDp * es : 0);
  w.xo = take(w.HDp ? BL * w.HDp * es : 0);
  w.part = take((int64_t)part_bytes);
  w.total = off;
  return w;
}

}  // namespace

extern "C" {

int txl_attn_variant(int variant) {
  g_detail[0] = 0;
  if (variant < 0 || variant > 2) return fail(TXL_EINVAL, "variant %d not in 0 .. 2", variant);
  return txl::attn_set_variant(variant);
}

const char* txl_status_string(int status) {
  const char* s;
  switch (status) {
    case TXL_OK: s = "TXL_OK"; break;
    case TXL_EINVAL: s = "TXL_EINVAL: invalid argument"; break;
    case TXL_EUNSUPPORTED: s = "TXL_EUNSUPPORTED: unsupported configuration"; break;
    case TXL_EHIP: s = "TXL_EHIP: HIP runtime error"; break;
    case TXL_EWORKSPACE: s = "TXL_EWORKSPACE: workspace too small"; break;
    default: s = "unknown txl status"; break;
  }
  if (status == TXL_OK || g_detail[0] == 0) {
    snprintf(g_msg, sizeof(g_msg), "%s", s);
  } else {
    snprintf(g_msg, sizeof(g_msg), "%s (%s)", s, g_detail);
  }
  return g_msg;
}

int txl_rel_attn_fwd(void* stream, int dtype, int64_t B, int64_t H, int64_t L, int64_t mem_len,
                     int64_t d_head, const void* q, int64_t q_sb, int64_t q_st, int64_t q_sh,
                     const void* k, const void* v, int64_t kv_sb, int64_t kv_st, int64_t kv_sh,
                     const void* r, int64_t r_sp, int64_t r_sh, int64_t r_rows,
                     const void* u_bias, const void* v_bias, float scale, void* out,
                     int64_t o_sb, int64_t o_st, int64_t o_sh, float* scores_dbg,
                     void* workspace, size_t ws_bytes) {
  g_detail[0] = 0;
  txl::AttnArgs a{};
  a.B = B; a.H = H; a.L = L; a.mem_len = mem_len; a.d = d_head;
  a.q = q; a.q_sb = q_sb; a.q_st = q_st; a.q_sh = q_sh;
  a.k = k; a.v = v; a.kv_sb = kv_sb; a.kv_st = kv_st; a.kv_sh = kv_sh;
  a.r = r; a.r_sp = r_sp; a.r_sh = r_sh;
  a.u = u_bias; a.vb = v_bias; a.scale = scale;
  a.out = out; a.o_sb = o_sb; a.o_st = o_st; a.o_sh = o_sh;
  a.scores = scores_dbg;
  a.d_load = d_head;
  const int rc = check_attn(dtype, a, r_rows);
  if (rc != TXL_OK) return rc;
  if (workspace) {
    const int64_t T = mem_len + L;
    const Span sw = {(uintptr_t)workspace, (uintptr_t)workspace + ws_bytes};
    const int64_t es = elt_size(dtype);
    const Span io[] = {span4(a.out, B, o_sb, L, o_st, H, o_sh, d_head, es),
                       span4(a.q, B, q_sb, L, q_st, H, q_sh, d_head, es),
                       span4(a.k, B, kv_sb, T, kv_st, H, kv_sh, d_head, es),
                       span4(a.v, B, kv_sb, T, kv_st, H, kv_sh, d_head, es),
                       span4(a.r, 1, 0, T, r_sp, H, r_sh, d_head, es)};
    for (const Span& s : io)
      if (overlap(sw, s)) return fail(TXL_EINVAL, "workspace overlaps a tensor argument");
  }
  return run_attn(dtype, a, workspace, ws_bytes, (hipStream_t)stream);
}

int txl_rel_attn_fwd_noalloc(void* stream, int dtype, int64_t B, int64_t H, int64_t L,
                             int64_t mem_len, int64_t d_head, const void* q, int64_t q_sb,
                             int64_t q_st, int64_t q_sh, const void* k, const void* v,
                             int64_t kv_sb, int64_t kv_st, int64_t kv_sh, const void* r,
                             int64_t r_sp, int64_t r_sh, int64_t r_rows, const void* u_bias,
                             const void* v_bias, float scale, void* out, int64_t o_sb,
                             int64_t o_st, int64_t o_sh, float* scores_dbg) {
  g_detail[0] = 0;
  txl::AttnArgs a{};
  a.B = B; a.H = H; a.L = L; a.mem_len = mem_len; a.d = d_head;
  a.q = q; a.q_sb = q_sb; a.q_st = q_st; a.q_sh = q_sh;
  a.k = k; a.v = v; a.kv_sb = kv_sb; a.kv_st = kv_st; a.kv_sh = kv_sh;
  a.r = r; a.r_sp = r_sp; a.r_sh = r_sh;
  a.u = u_bias; a.vb = v_bias; a.scale = scale;
  a.out = out; a.o_sb = o_sb; a.o_st = o_st; a.o_sh = o_sh;
  a.scores = scores_dbg;
  a.d_load = d_head;
  const int rc = check_attn(dtype, a, r_rows);
  if (rc != TXL_OK) return rc;
  // the whole split plan of this shape must fit the static scratch
  const size_t need = attn_plan_bytes(dtype, a);
  if (need > txl::STATIC_SCRATCH_BYTES)
    return fail(TXL_EWORKSPACE,
                "the key split of this shape needs %zu bytes of scratch; the static scratch "
                "holds %zu (use txl_rel_attn_fwd with a workspace)",
                need, (size_t)txl::STATIC_SCRATCH_BYTES);
  void* scratch = nullptr;
  if (need > 0) {
    const hipError_t e = txl::static_scratch_ptr(&scratch);
    if (e != hipSuccess) return hip_fail(e, "static scratch address");
  }
  return run_attn(dtype, a, scratch, need, (hipStream_t)stream);
}

size_t txl_rel_attn_noalloc_max_scratch_bytes(void) { return txl::STATIC_SCRATCH_BYTES; }

size_t txl_rel_attn_workspace_bytes(int dtype, int64_t B, int64_t H, int64_t L, int64_t mem_len,
                                    int64_t d_head) {
  if ((dtype != TXL_FP32 && dtype != TXL_BF16) || B < 1 || H < 1 || L < 1 || mem_len < 0 ||
      d_head < 1 || d_head > 128)
    return 0;
  txl::AttnArgs a{};
  a.B = B; a.H = H; a.L = L; a.mem_len = mem_len; a.d = d_head; a.d_load = d_head;
  // the plan depends only on the shapes; layouts are taken as aligned head-major
  a.q = a.k = a.v = a.r = (const void*)(uintptr_t)256;
  a.q_sb = a.q_st = a.q_sh = a.kv_sb = a.kv_st = a.kv_sh = a.r_sp = a.r_sh = 64;
  return attn_plan_bytes(dtype, a);
}

int txl_attn_kernel(int dtype, int64_t B, int64_t H, int64_t L, int64_t mem_len,
                    int64_t d_head) {
  g_detail[0] = 0;
  if ((dtype != TXL_FP32 && dtype != TXL_BF16) || B < 1 || H < 1 || L < 1 || mem_len < 0 ||
      d_head < 1 || d_head > 128)
    return fail(TXL_EINVAL, "invalid sizes or dtype");
  txl::AttnArgs a{};
  a.B = B; a.H = H; a.L = L; a.mem_len = mem_len; a.d = d_head; a.d_load = d_head;
  a.q = a.k = a.v = a.r = (const void*)(uintptr_t)256;
  a.q_sb = a.q_st = a.q_sh = a.kv_sb = a.kv_st = a.kv_sh = a.r_sp = a.r_sh = 64;
  if (dtype != TXL_BF16) return TXL_ATTN_VECTOR;
  if (txl::attn_decode_supported(a)) return TXL_ATTN_ONE_QUERY;
  if (!txl::attn_mfma_supported(a)) return TXL_ATTN_VECTOR;
  const txl::AttnPlan p = txl::attn_mfma_plan(a, num_cus(), (size_t)-1);
  if (p.q64) return TXL_ATTN_Q64;
  return p.slots > 0 ? TXL_ATTN_Q128_SPLIT : TXL_ATTN_Q128;
}

size_t txl_layer_workspace_bytes(const txl_layer_dims* dims, int64_t mem_capacity, int dtype) {
  if (check_dims(dims) != TXL_OK || mem_capacity < 0) return 0;
  if (dtype != TXL_FP32 && dtype != TXL_BF16) return 0;
  return ws_layout(*dims, mem_capacity + dims->L, elt_size(dtype),
                   layer_part_bytes(*dims, mem_capacity, dtype))
      .total;
}

int txl_layer_workspace_map(const txl_layer_dims* dims, int64_t mem_len, int dtype,
                            txl_workspace_map* map) {
  g_detail[0] = 0;
  if (dtype != TXL_FP32 && dtype != TXL_BF16) return fail(TXL_EUNSUPPORTED, "dtype %d", dtype);
  const int rc = check_dims(dims);
  if (rc != TXL_OK) return rc;
  if (!map) return fail(TXL_EINVAL, "map is NULL");
  if (mem_len < 0) return fail(TXL_EINVAL, "mem_len must be >= 0");
  const WsLayout w = ws_layout(*dims, mem_len + dims->L, elt_size(dtype));
  map->q = w.q;
  map->k = w.k;
  map->v = w.v;
  map->r = w.r;
  map->a = w.a;
  map->d_pad = w.dp;
  return TXL_OK;
}

// The layer step; with lse != NULL the matrix-core attention also writes each
// query's log-sum-exp there ([B][H][L]) and *lse_written says whether it did;
// *y_written (if given) says whether the workspace holds y = a W_o^T + h_in.
static int layer_step_run(void* stream, int dtype, const txl_layer_dims* dims, const void* h_in,
                          const txl_ring* mem, const txl_layer_weights* w, const void* u_bias,
                          const void* v_bias, const void* R, int64_t R_rows, void* h_out,
                          void* workspace, size_t ws_bytes, float* lse, bool* lse_written,
                          bool* y_written = nullptr) {
  g_detail[0] = 0;
  if (lse_written) *lse_written = false;
  if (y_written) *y_written = false;
  if (dtype != TXL_FP32 && dtype != TXL_BF16) return fail(TXL_EUNSUPPORTED, "dtype %d", dtype);
  int rc = check_dims(dims);
  if (rc != TXL_OK) return rc;
  if (!mem) return fail(TXL_EINVAL, "mem is NULL");
  if (mem->capacity < 1 || mem->start < 0 || mem->start >= mem->capacity || mem->len < 0 ||
      mem->len > mem->capacity)
    return fail(TXL_EINVAL, "ring state (capacity %lld, start %lld, len %lld) is invalid",
                (long long)mem->capacity, (long long)mem->start, (long long)mem->len);
  if (!mem->data) return fail(TXL_EINVAL, "mem->data is NULL");
  if (!w || !w->W_q || !w->W_kE || !w->W_v || !w->W_kR || !w->W_o || !w->ln_gamma ||
      !w->ln_beta)
    return fail(TXL_EINVAL, "NULL weight pointer");
  if (!h_in || !h_out || !u_bias || !v_bias || !R) return fail(TXL_EINVAL, "NULL tensor pointer");
  if (!workspace) return fail(TXL_EINVAL, "workspace is NULL");
  if ((uintptr_t)workspace % 256) return fail(TXL_EINVAL, "workspace is not 256-byte aligned");
  const txl_layer_dims dm = *dims;
  const int64_t B = dm.B, L = dm.L, D = dm.d_model, H = dm.n_head, d = dm.d_head;
  const int64_t len = mem->len, T = len + L, HD = H * d;
  if (R_rows < T)
    return fail(TXL_EINVAL, "R_rows %lld < mem->len + L = %lld", (long long)R_rows, (long long)T);
  const int64_t es = elt_size(dtype);
  const size_t need =
      ws_layout(dm, mem->capacity + L, es, layer_part_bytes(dm, mem->capacity, dtype)).total;
  if (ws_bytes < need)
    return fail(TXL_EWORKSPACE, "need %zu bytes, got %zu", need, ws_bytes);
  const Span sh_in = {(uintptr_t)h_in, (uintptr_t)h_in + (uintptr_t)(B * L * D * es)};
  const Span sh_out = {(uintptr_t)h_out, (uintptr_t)h_out + (uintptr_t)(B * L * D * es)};
  const Span sring = {(uintptr_t)mem->data,
                      (uintptr_t)mem->data + (uintptr_t)(B * mem->capacity * D * es)};
  const Span sws = {(uintptr_t)workspace, (uintptr_t)workspace + ws_bytes};
  if (overlap(sh_out, sh_in)) return fail(TXL_EINVAL, "h_out aliases h_in");
  if (overlap(sh_out, sring)) return fail(TXL_EINVAL, "h_out aliases the memory");
  if (overlap(sws, sh_in) || overlap(sws, sh_out) || overlap(sws, sring))
    return fail(TXL_EINVAL, "workspace overlaps an argument");

  const WsLayout ws = ws_layout(dm, T, es);
  char* base = (char*)workspace;
  void* q = base + ws.q;
  void* k = base + ws.k;
  void* v = base + ws.v;
  void* r = base + ws.r;
  void* a = base + ws.a;
  float* y = (float*)(base + ws.y);
  const int64_t dp = ws.dp;
  hipStream_t st = (hipStream_t)stream;

  // k, v over the extended context [memory ; h] (section 3.2): the ring rows are
  // gathered by the GEMM's row loader, never copied.
  txl::GemmArgs proj[3] = {};
  txl::GemmArgs& gkv = proj[0];
  gkv.M = B * T; gkv.N = 2 * HD; gkv.K = D;
  gkv.a = {mem->data, mem->capacity, mem->start, len, h_in, L, D};
  gkv.w = {w->W_kE, w->W_v, HD, D};
  gkv.e = {txl::EPI_HEADS, k, v, HD, d, H * T * dp, T * dp, dp, nullptr, nullptr, 0, 0, dp};
  // q from the current rows only
  txl::GemmArgs& gq = proj[1];
  gq.M = B * L; gq.N = HD; gq.K = D;
  gq.a = {nullptr, 1, 0, 0, h_in, L, D};
  gq.w = {w->W_q, w->W_q, HD, D};
  gq.e = {txl::EPI_HEADS, q, q, HD, d, H * L * dp, L * dp, dp, nullptr, nullptr, 0, 0, dp};
  // r = R[0:T] W_kR^T, shared by the whole batch
  txl::GemmArgs& gr = proj[2];
  gr.M = T; gr.N = HD; gr.K = D;
  gr.a = {nullptr, 1, 0, 0, R, T, D};
  gr.w = {w->W_kR, w->W_kR, HD, D};
  gr.e = {txl::EPI_HEADS, r, r, HD, d, 0, T * dp, dp, nullptr, nullptr, 0, 0, dp};
  // d_model not a multiple of 32: the projections read zero-padded copies of the
  // context rows, R and the weights (one launch), then run K = Dp
  uint16_t* xw = (uint16_t*)(base + ws.xw);
  const int64_t Dp = ws.Dp;
  auto al4 = [](const void* p) { return (uintptr_t)p % 4 == 0; };
  const bool pin = dtype == TXL_BF16 && Dp > 0 && al4(h_in) && al4(mem->data) && al4(R) &&
                   al4(w->W_q) && al4(w->W_kE) && al4(w->W_v) && al4(w->W_kR);
  const bool pout = dtype == TXL_BF16 && ws.HDp > 0 && al4(w->W_o) && al4(a);
  if (pin || pout) {
    txl::PadJob pj[7];
    int np = 0;
    if (pin) {
      uint16_t* xa = (uint16_t*)(base + ws.xa);
      pj[np++] = {{mem->data, mem->capacity, mem->start, len, h_in, L, D}, B * T, D, Dp, xa};
      pj[np++] = {{nullptr, 1, 0, 0, R, T, D}, T, D, Dp, (uint16_t*)(base + ws.xr)};
      const void* wsrc[4] = {w->W_q, w->W_kE, w->W_v, w->W_kR};
      for (int i = 0; i < 4; ++i)
        pj[np++] = {{nullptr, 1, 0, 0, wsrc[i], HD, D}, HD, D, Dp, xw + i * HD * Dp};
      gkv.K = gq.K = gr.K = Dp;
      gkv.a = {nullptr, 1, 0, 0, xa, T, Dp};
      gq.a = {xa, T, len, L, nullptr, 0, Dp};  // rows len .. T-1 of each batch row
      gr.a = {nullptr, 1, 0, 0, base + ws.xr, T, Dp};
      gkv.w = {xw + HD * Dp, xw + 2 * HD * Dp, HD, Dp};
      gq.w = {xw, xw, HD, Dp};
      gr.w = {xw + 3 * HD * Dp, xw + 3 * HD * Dp, HD, Dp};
    }
    if (pout)
      pj[np++] = {{nullptr, 1, 0, 0, w->W_o, D, HD}, D, HD, ws.HDp, (uint16_t*)(base + ws.xwo)};
    const hipError_t e = txl::launch_pad_rows(pj, np, st);
    if (e != hipSuccess) return hip_fail(e, "padded operand copies");
  }
  head_padded_cols(gkv, 2, H, d, dp);
  head_padded_cols(gq, 1, H, d, dp);
  head_padded_cols(gr, 1, H, d, dp);
  if (dtype == TXL_BF16 && txl::gemm_mfma_supported(gkv) && txl::gemm_mfma_supported(gq) &&
      txl::gemm_mfma_supported(gr)) {
    // the three projections share K and run as one grid
    const hipError_t e = txl::launch_gemm_mfma_multi(proj, 3, st, num_cus());
    if (e != hipSuccess) return hip_fail(e, "q/kv/r projections");
  } else {
    if ((rc = run_gemm(dtype, gkv, st, "kv projection")) != TXL_OK) return rc;
    if ((rc = run_gemm(dtype, gq, st, "q projection")) != TXL_OK) return rc;
    if ((rc = run_gemm(dtype, gr, st, "r projection")) != TXL_OK) return rc;
  }
  // attention; output a [B, L, H*d] token-major for the output projection
  txl::AttnArgs at{};
  at.B = B; at.H = H; at.L = L; at.mem_len = len; at.d = d;
  at.q = q; at.q_sb = H * L * dp; at.q_st = dp; at.q_sh = L * dp;
  at.k = k; at.v = v; at.kv_sb = H * T * dp; at.kv_st = dp; at.kv_sh = T * dp;
  at.r = r; at.r_sp = dp; at.r_sh = T * dp;
  at.u = u_bias; at.vb = v_bias; at.scale = 1.0f / sqrtf((float)d);
  at.out = a; at.o_sb = L * HD; at.o_st = HD; at.o_sh = d;
  at.scores = nullptr;
  at.d_load = dp;  // workspace rows hold dp readable columns
  if (lse && dtype == TXL_BF16 && txl::attn_mfma_supported(at)) {
    at.lse = lse;
    *lse_written = true;
  }
  if ((rc = run_attn(dtype, at, base + ws.part, ws_bytes - ws.part, st)) != TXL_OK) return rc;
  if (pout) {
    // H d not a multiple of 32: a copied to rows of HDp for the output projection
    const txl::PadJob pa = {{nullptr, 1, 0, 0, a, B * L, HD}, B * L, HD, ws.HDp,
                            (uint16_t*)(base + ws.xo)};
    const hipError_t e = txl::launch_pad_rows(&pa, 1, st);
    if (e != hipSuccess) return hip_fail(e, "padded attention output");
  }
  const void* a_pad = pout ? base + ws.xo : nullptr;
  const void* wo_pad = pout ? base + ws.xwo : nullptr;
  if (y_written) *y_written = !out_ln_fused(dtype, dm, a, w, h_in, h_out, a_pad, wo_pad, ws.HDp);
  return run_out_ln(dtype, dm, a, w, h_in, h_out, y, st, (float*)(base + ws.opart), a_pad,
                    wo_pad, ws.HDp, y_written != nullptr);
}

int txl_layer_step(void* stream, int dtype, const txl_layer_dims* dims, const void* h_in,
                   const txl_ring* mem, const txl_layer_weights* w, const void* u_bias,
                   const void* v_bias, const void* R, int64_t R_rows, void* h_out,
                   void* workspace, size_t ws_bytes) {
  return layer_step_run(stream, dtype, dims, h_in, mem, w, u_bias, v_bias, R, R_rows, h_out,
                        workspace, ws_bytes, nullptr, nullptr);
}

int txl_mem_update(void* stream, int dtype, txl_ring* mem, int64_t B, int64_t d_model,
                   const void* h_new, int64_t L) {
  g_detail[0] = 0;
  if (dtype != TXL_FP32 && dtype != TXL_BF16) return fail(TXL_EUNSUPPORTED, "dtype %d", dtype);
  if (!mem || !mem->data || !h_new) return fail(TXL_EINVAL, "NULL pointer");
  if (B < 1 || d_model < 1 || L < 1) return fail(TXL_EINVAL, "B, d_model, L must be >= 1");
  if (B > 65535) return fail(TXL_EUNSUPPORTED, "B must be <= 65535");
  const int64_t M = mem->capacity;
  if (M < 1 || mem->start < 0 || mem->start >= M || mem->len < 0 || mem->len > M)
    return fail(TXL_EINVAL, "ring state (capacity %lld, start %lld, len %lld) is invalid",
                (long long)M, (long long)mem->start, (long long)mem->len);
  const int64_t es = elt_size(dtype);
  const Span sring = {(uintptr_t)mem->data, (uintptr_t)mem->data + (uintptr_t)(B * M * d_model * es)};
  const Span sh = {(uintptr_t)h_new, (uintptr_t)h_new + (uintptr_t)(B * L * d_model * es)};
  if (overlap(sring, sh)) return fail(TXL_EINVAL, "h_new overlaps the memory");
  const int64_t n = L < M ? L : M;                 // newest rows that survive
  const int64_t slot0 = (mem->start + mem->len + (L - n)) % M;
  hipError_t e = txl::launch_ring_copy(dtype, mem->data, M, slot0, h_new, L, L - n, n, B,
                                       d_model, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "ring copy");
  const int64_t tot = mem->len + L;
  const int64_t new_len = tot < M ? tot : M;
  mem->start = (mem->start + tot - new_len) % M;
  mem->len = new_len;
  return TXL_OK;
}

// ---- a stack of layers over several segments ----------------------------------------

size_t txl_stack_workspace_bytes(const txl_layer_dims* dims, int64_t mem_capacity, int dtype,
                                 int n_streams) {
  if (n_streams < 1 || n_streams > TXL_STACK_MAX_STREAMS) return 0;
  const size_t lw = txl_layer_workspace_bytes(dims, mem_capacity, dtype);
  if (lw == 0) return 0;
  const int64_t hb = round_up(dims->B * dims->L * dims->d_model * elt_size(dtype), 256);
  return (size_t)n_streams * (size_t)(round_up((int64_t)lw, 256) + 2 * hb);
}

int txl_stack_fwd(void* const* streams, int n_streams, int dtype, const txl_layer_dims* dims,
                  int64_t n_layers, int64_t n_segments, const void* h_in, txl_ring* mem,
                  const txl_layer_weights* w, const void* u_bias, const void* v_bias,
                  const void* R, int64_t R_rows, void* h_out, void* workspace,
                  size_t ws_bytes) {
  g_detail[0] = 0;
  if (dtype != TXL_FP32 && dtype != TXL_BF16) return fail(TXL_EUNSUPPORTED, "dtype %d", dtype);
  int rc = check_dims(dims);
  if (rc != TXL_OK) return rc;
  if (!streams) return fail(TXL_EINVAL, "streams is NULL");
  if (n_streams < 1 || n_streams > TXL_STACK_MAX_STREAMS)
    return fail(TXL_EINVAL, "n_streams %d not in 1 .. %d", n_streams, TXL_STACK_MAX_STREAMS);
  if (n_layers < 1 || n_segments < 1)
    return fail(TXL_EINVAL, "n_layers and n_segments must be >= 1");
  if (!h_in || !mem || !w || !u_bias || !v_bias || !R || !h_out)
    return fail(TXL_EINVAL, "NULL pointer");
  if (!workspace) return fail(TXL_EINVAL, "workspace is NULL");
  if ((uintptr_t)workspace % 256) return fail(TXL_EINVAL, "workspace is not 256-byte aligned");
  const txl_layer_dims dm = *dims;
  const int64_t B = dm.B, L = dm.L, D = dm.d_model, es = elt_size(dtype);
  const int64_t seg = B * L * D * es;  // bytes of one segment's [B][L][D]
  // every layer's arguments, before anything is enqueued
  size_t lw = 0;
  for (int64_t n = 0; n < n_layers; ++n) {
    const txl_ring& m = mem[n];
    if (m.capacity < 1 || m.start < 0 || m.start >= m.capacity || m.len < 0 ||
        m.len > m.capacity || !m.data)
      return fail(TXL_EINVAL, "ring of layer %lld: state (capacity %lld, start %lld, len %lld)",
                  (long long)n, (long long)m.capacity, (long long)m.start, (long long)m.len);
    const txl_layer_weights& wl = w[n];
    if (!wl.W_q || !wl.W_kE || !wl.W_v || !wl.W_kR || !wl.W_o || !wl.ln_gamma || !wl.ln_beta)
      return fail(TXL_EINVAL, "NULL weight pointer in layer %lld", (long long)n);
    // the longest memory this layer reads: len grows by L per segment up to the capacity
    const int64_t len_max = std::min<int64_t>(m.len + (n_segments - 1) * L, m.capacity);
    if (R_rows < len_max + L)
      return fail(TXL_EINVAL, "R_rows %lld < %lld (layer %lld's longest memory + L)",
                  (long long)R_rows, (long long)(len_max + L), (long long)n);
    lw = std::max(lw, txl_layer_workspace_bytes(dims, m.capacity, dtype));
  }
  if (lw == 0) return fail(TXL_EINVAL, "invalid layer dims");
  const int64_t hb = round_up(seg, 256);
  const int64_t per = round_up((int64_t)lw, 256) + 2 * hb;  // one stream's share
  const size_t need = (size_t)(n_streams * per);
  if (ws_bytes < need) return fail(TXL_EWORKSPACE, "need %zu bytes, got %zu", need, ws_bytes);
  const Span sin = {(uintptr_t)h_in, (uintptr_t)h_in + (uintptr_t)(n_segments * seg)};
  const Span sout = {(uintptr_t)h_out, (uintptr_t)h_out + (uintptr_t)(n_segments * seg)};
  const Span sws = {(uintptr_t)workspace, (uintptr_t)workspace + ws_bytes};
  if (overlap(sout, sin)) return fail(TXL_EINVAL, "h_out overlaps h_in");
  if (overlap(sws, sin) || overlap(sws, sout)) return fail(TXL_EINVAL, "workspace overlaps h_in or h_out");
  for (int64_t n = 0; n < n_layers; ++n) {
    const Span sr = {(uintptr_t)mem[n].data,
                     (uintptr_t)mem[n].data + (uintptr_t)(B * mem[n].capacity * D * es)};
    if (overlap(sr, sin) || overlap(sr, sout) || overlap(sr, sws))
      return fail(TXL_EINVAL, "the ring of layer %lld overlaps h_in, h_out or the workspace",
                  (long long)n);
    for (int64_t m = 0; m < n; ++m) {
      const Span so = {(uintptr_t)mem[m].data,
                       (uintptr_t)mem[m].data + (uintptr_t)(B * mem[m].capacity * D * es)};
      if (overlap(sr, so))
        return fail(TXL_EINVAL, "the rings of layers %lld and %lld overlap", (long long)m,
                    (long long)n);
    }
  }

  // Streams that get segments, and the events of the schedule: done[s & 1][n] is
  // recorded after layer n of segment s has appended its input to ring n; layer
  // n of segment s + 1 (the next stream) waits for it.  The same slot is recorded
  // again two segments later, after that wait was enqueued.
  const int ns = (int)std::min<int64_t>(n_streams, n_segments);
  struct Events {
    std::vector<hipEvent_t> v;
    ~Events() { for (hipEvent_t e : v) (void)hipEventDestroy(e); }  // released when complete
  } evs;
  auto make_event = [&](hipEvent_t* e) {
    const hipError_t x = hipEventCreateWithFlags(e, hipEventDisableTiming);
    if (x == hipSuccess) evs.v.push_back(*e);
    return x;
  };
  std::vector<hipEvent_t> done;
  hipEvent_t e_start = nullptr;
  if (ns > 1) {
    done.resize(2 * n_layers);
    for (hipEvent_t& e : done) {
      const hipError_t x = make_event(&e);
      if (x != hipSuccess) return hip_fail(x, "event create");
    }
    hipError_t x = make_event(&e_start);
    if (x == hipSuccess) x = hipEventRecord(e_start, (hipStream_t)streams[0]);
    for (int k = 1; k < ns && x == hipSuccess; ++k)
      x = hipStreamWaitEvent((hipStream_t)streams[k], e_start, 0);
    if (x != hipSuccess) return hip_fail(x, "stream start order");
  }
  char* base = (char*)workspace;
  for (int64_t s = 0; s < n_segments; ++s) {
    const int k = (int)(s % ns);
    void* st = streams[k];
    char* wsk = base + k * per;
    char* buf[2] = {wsk + round_up((int64_t)lw, 256), wsk + round_up((int64_t)lw, 256) + hb};
    const char* h = (const char*)h_in + s * seg;
    for (int64_t n = 0; n < n_layers; ++n) {
      if (ns > 1 && s > 0) {
        const hipError_t x = hipStreamWaitEvent((hipStream_t)st, done[((s - 1) & 1) * n_layers + n], 0);
        if (x != hipSuccess) return hip_fail(x, "stream wait");
      }
      void* out = n == n_layers - 1 ? (void*)((char*)h_out + s * seg) : (void*)buf[n & 1];
      rc = layer_step_run(st, dtype, dims, h, &mem[n], &w[n], u_bias, v_bias, R, R_rows, out,
                          wsk, (size_t)round_up((int64_t)lw, 256), nullptr, nullptr);
      if (rc != TXL_OK) return rc;
      rc = txl_mem_update(st, dtype, &mem[n], B, D, h, L);
      if (rc != TXL_OK) return rc;
      if (ns > 1) {
        const hipError_t x = hipEventRecord(done[(s & 1) * n_layers + n], (hipStream_t)st);
        if (x != hipSuccess) return hip_fail(x, "event record");
      }
      h = (const char*)out;
    }
  }
  // stream 0 waits for the others' last work, so that it alone orders what follows
  for (int k = 1; k < ns; ++k) {
    hipEvent_t e_end = nullptr;
    hipError_t x = make_event(&e_end);
    if (x == hipSuccess) x = hipEventRecord(e_end, (hipStream_t)streams[k]);
    if (x == hipSuccess) x = hipStreamWaitEvent((hipStream_t)streams[0], e_end, 0);
    if (x != hipSuccess) return hip_fail(x, "stream end order");
  }
  return TXL_OK;
}

// ---- evaluation with cached keys and values -----------------------------------------

size_t txl_kv_ring_bytes(const txl_layer_dims* dims, int64_t capacity, int dtype) {
  if (check_dims(dims) != TXL_OK || capacity < 1) return 0;
  if (dtype != TXL_FP32 && dtype != TXL_BF16) return 0;
  return (size_t)(dims->B * dims->n_head * capacity * round_up(dims->d_head, 8) * elt_size(dtype));
}

int txl_pos_proj(void* stream, int dtype, const txl_layer_dims* dims, const void* R,
                 int64_t R_rows, const void* W_kR, void* r_out) {
  g_detail[0] = 0;
  if (dtype != TXL_FP32 && dtype != TXL_BF16) return fail(TXL_EUNSUPPORTED, "dtype %d", dtype);
  const int rc = check_dims(dims);
  if (rc != TXL_OK) return rc;
  if (!R || !W_kR || !r_out) return fail(TXL_EINVAL, "NULL pointer");
  if (R_rows < 1 || R_rows > 0x7fffffffLL) return fail(TXL_EINVAL, "R_rows must be in 1 .. 2^31-1");
  const int64_t D = dims->d_model, H = dims->n_head, d = dims->d_head, HD = H * d;
  const int64_t dp = round_up(d, 8), es = elt_size(dtype);
  const Span so = {(uintptr_t)r_out, (uintptr_t)r_out + (uintptr_t)(H * R_rows * dp * es)};
  const Span sR = {(uintptr_t)R, (uintptr_t)R + (uintptr_t)(R_rows * D * es)};
  const Span sW = {(uintptr_t)W_kR, (uintptr_t)W_kR + (uintptr_t)(HD * D * es)};
  if (overlap(so, sR) || overlap(so, sW)) return fail(TXL_EINVAL, "r_out overlaps an input");
  txl::GemmArgs gr{};
  gr.M = R_rows; gr.N = HD; gr.K = D;
  gr.a = {nullptr, 1, 0, 0, R, R_rows, D};
  gr.w = {W_kR, W_kR, HD, D};
  gr.e = {txl::EPI_HEADS, r_out, r_out, HD, d, 0, R_rows * dp, dp, nullptr, nullptr, 0, 0, dp};
  head_padded_cols(gr, 1, H, d, dp);
  return run_gemm(dtype, gr, (hipStream_t)stream, "position projection");
}


size_t txl_layer_kv_workspace_bytes(const txl_layer_dims* dims, int64_t mem_max, int dtype) {
  if (check_dims(dims) != TXL_OK || mem_max < 0) return 0;
  if (dtype != TXL_FP32 && dtype != TXL_BF16) return 0;
  return kv_ws_layout(*dims, elt_size(dtype), layer_part_bytes(*dims, mem_max, dtype)).total;
}

int txl_layer_step_kv(void* stream, int dtype, const txl_layer_dims* dims, const void* h_in,
                      txl_kv_ring* kv, const txl_layer_weights* w, const void* u_bias,
                      const void* v_bias, const void* r, int64_t r_rows, void* h_out,
                      void* workspace, size_t ws_bytes) {
  g_detail[0] = 0;
  if (dtype != TXL_FP32 && dtype != TXL_BF16) return fail(TXL_EUNSUPPORTED, "dtype %d", dtype);
  int rc = check_dims(dims);
  if (rc != TXL_OK) return rc;
  if (!kv || !kv->k || !kv->v) return fail(TXL_EINVAL, "kv ring or its k / v is NULL");
  const txl_layer_dims dm = *dims;
  const int64_t B = dm.B, L = dm.L, D = dm.d_model, H = dm.n_head, d = dm.d_head, HD = H * d;
  const int64_t C = kv->capacity, M = kv->mem_max, len = kv->len, T = len + L;
  if (M < 0 || C < M + L || C > 0x7fffffffLL || kv->start < 0 || kv->start >= C || len < 0 ||
      len > M)
    return fail(TXL_EINVAL,
                "kv ring state (capacity %lld, mem_max %lld, start %lld, len %lld) is invalid "
                "for L = %lld (needs capacity >= mem_max + L, len <= mem_max)",
                (long long)C, (long long)M, (long long)kv->start, (long long)len, (long long)L);
  if (!w || !w->W_q || !w->W_kE || !w->W_v || !w->W_o || !w->ln_gamma || !w->ln_beta)
    return fail(TXL_EINVAL, "NULL weight pointer");
  if (!h_in || !h_out || !u_bias || !v_bias || !r) return fail(TXL_EINVAL, "NULL tensor pointer");
  if (r_rows < T)
    return fail(TXL_EINVAL, "r_rows %lld < kv->len + L = %lld", (long long)r_rows, (long long)T);
  if (!workspace) return fail(TXL_EINVAL, "workspace is NULL");
  if ((uintptr_t)workspace % 256) return fail(TXL_EINVAL, "workspace is not 256-byte aligned");
  const int64_t es = elt_size(dtype);
  const KvWs ws = kv_ws_layout(dm, es, layer_part_bytes(dm, M, dtype));
  if (ws_bytes < ws.total)
    return fail(TXL_EWORKSPACE, "need %zu bytes, got %zu", ws.total, ws_bytes);
  const int64_t dp = ws.dp;
  const size_t ring_bytes = (size_t)(B * H * C * dp * es);
  const Span sh_in = {(uintptr_t)h_in, (uintptr_t)h_in + (uintptr_t)(B * L * D * es)};
  const Span sh_out = {(uintptr_t)h_out, (uintptr_t)h_out + (uintptr_t)(B * L * D * es)};
  const Span sk = {(uintptr_t)kv->k, (uintptr_t)kv->k + ring_bytes};
  const Span sv = {(uintptr_t)kv->v, (uintptr_t)kv->v + ring_bytes};
  const Span sr = {(uintptr_t)r, (uintptr_t)r + (uintptr_t)(H * r_rows * dp * es)};
  const Span sws = {(uintptr_t)workspace, (uintptr_t)workspace + ws_bytes};
  if (overlap(sh_out, sh_in)) return fail(TXL_EINVAL, "h_out aliases h_in");
  if (overlap(sk, sv)) return fail(TXL_EINVAL, "kv->k and kv->v overlap");
  const Span outs[] = {sh_out, sk, sv, sws};
  const Span ins[] = {sh_in, sr};
  for (const Span& o : outs)
    for (const Span& i : ins)
      if (overlap(o, i)) return fail(TXL_EINVAL, "an output (h_out, k, v, workspace) overlaps an input");
  if (overlap(sws, sh_out) || overlap(sws, sk) || overlap(sws, sv) || overlap(sh_out, sk) ||
      overlap(sh_out, sv))
    return fail(TXL_EINVAL, "h_out, the ring and the workspace must not overlap");

  char* base = (char*)workspace;
  void* q = base + ws.q;
  void* a = base + ws.a;
  float* y = (float*)(base + ws.y);
  hipStream_t st = (hipStream_t)stream;

  // k, v of the L new rows straight into the ring, after the len memory rows
  txl::GemmArgs proj[2] = {};
  txl::GemmArgs& gkv = proj[0];
  gkv.M = B * L; gkv.N = 2 * HD; gkv.K = D;
  gkv.a = {nullptr, 1, 0, 0, h_in, L, D};
  gkv.w = {w->W_kE, w->W_v, HD, D};
  gkv.e = {txl::EPI_HEADS, kv->k, kv->v, HD, d, H * C * dp, C * dp, dp, nullptr, nullptr,
           (kv->start + len) % C, C, dp};
  txl::GemmArgs& gq = proj[1];
  gq.M = B * L; gq.N = HD; gq.K = D;
  gq.a = {nullptr, 1, 0, 0, h_in, L, D};
  gq.w = {w->W_q, w->W_q, HD, D};
  gq.e = {txl::EPI_HEADS, q, q, HD, d, H * L * dp, L * dp, dp, nullptr, nullptr, 0, 0, dp};
  // d_model or H d not a multiple of 32: zero-padded copies (one launch), as in
  // txl_layer_step
  auto al4 = [](const void* p) { return (uintptr_t)p % 4 == 0; };
  const bool pin = dtype == TXL_BF16 && ws.Dp > 0 && al4(h_in) && al4(w->W_q) && al4(w->W_kE) &&
                   al4(w->W_v);
  const bool pout = dtype == TXL_BF16 && ws.HDp > 0 && al4(w->W_o) && al4(a);
  if (pin || pout) {
    txl::PadJob pj[5];
    int np = 0;
    const int64_t Dp = ws.Dp;
    if (pin) {
      uint16_t* xh = (uint16_t*)(base + ws.xh);
      uint16_t* xw = (uint16_t*)(base + ws.xw);
      pj[np++] = {{nullptr, 1, 0, 0, h_in, B * L, D}, B * L, D, Dp, xh};
      const void* wsrc[3] = {w->W_q, w->W_kE, w->W_v};
      for (int i = 0; i < 3; ++i)
        pj[np++] = {{nullptr, 1, 0, 0, wsrc[i], HD, D}, HD, D, Dp, xw + i * HD * Dp};
      gkv.K = gq.K = Dp;
      gkv.a = {nullptr, 1, 0, 0, xh, L, Dp};
      gq.a = {nullptr, 1, 0, 0, xh, L, Dp};
      gkv.w = {xw + HD * Dp, xw + 2 * HD * Dp, HD, Dp};
      gq.w = {xw, xw, HD, Dp};
    }
    if (pout)
      pj[np++] = {{nullptr, 1, 0, 0, w->W_o, D, HD}, D, HD, ws.HDp, (uint16_t*)(base + ws.xwo)};
    const hipError_t e = txl::launch_pad_rows(pj, np, st);
    if (e != hipSuccess) return hip_fail(e, "padded operand copies");
  }
  head_padded_cols(gkv, 2, H, d, dp);
  head_padded_cols(gq, 1, H, d, dp);
  if (dtype == TXL_BF16 && txl::gemm_mfma_supported(gkv) && txl::gemm_mfma_supported(gq)) {
    const hipError_t e = txl::launch_gemm_mfma_multi(proj, 2, st, num_cus());
    if (e != hipSuccess) return hip_fail(e, "q/kv projections");
  } else {
    if ((rc = run_gemm(dtype, gkv, st, "kv projection")) != TXL_OK) return rc;
    if ((rc = run_gemm(dtype, gq, st, "q projection")) != TXL_OK) return rc;
  }
  // attention over the len memory keys and the L new ones, all in the ring
  txl::AttnArgs at{};
  at.B = B; at.H = H; at.L = L; at.mem_len = len; at.d = d;
  at.q = q; at.q_sb = H * L * dp; at.q_st = dp; at.q_sh = L * dp;
  at.k = kv->k; at.v = kv->v; at.kv_sb = H * C * dp; at.kv_st = dp; at.kv_sh = C * dp;
  at.kv_start = kv->start; at.kv_cap = C;
  at.r = r; at.r_sp = dp; at.r_sh = r_rows * dp;
  at.u = u_bias; at.vb = v_bias; at.scale = 1.0f / sqrtf((float)d);
  at.out = a; at.o_sb = L * HD; at.o_st = HD; at.o_sh = d;
  at.scores = nullptr;
  at.d_load = dp;  // ring, q and r rows hold dp readable columns (padding zeroed)
  if ((rc = run_attn(dtype, at, base + ws.part, ws_bytes - ws.part, st)) != TXL_OK) return rc;
  if (pout) {
    const txl::PadJob pa = {{nullptr, 1, 0, 0, a, B * L, HD}, B * L, HD, ws.HDp,
                            (uint16_t*)(base + ws.xo)};
    const hipError_t e = txl::launch_pad_rows(&pa, 1, st);
    if (e != hipSuccess) return hip_fail(e, "padded attention output");
    rc = run_out_ln(dtype, dm, a, w, h_in, h_out, y, st, nullptr, base + ws.xo, base + ws.xwo,
                    ws.HDp, false);
  } else {
    rc = run_out_ln(dtype, dm, a, w, h_in, h_out, y, st);
  }
  if (rc != TXL_OK) return rc;
  // the memory keeps the newest min(M, len + L) rows: only the ring state moves
  const int64_t new_len = T < M ? T : M;
  kv->start = (kv->start + T - new_len) % C;
  kv->len = new_len;
  return TXL_OK;
}

// ---- position-wise feed-forward ---------------------------------------------------------

// Workspace of txl_pos_ff: f = relu(x W1^T + b1) [rows][Fp], y fp32 [rows][D]
// (the unfused second layer), then, when d_model or d_inner is not a multiple of
// 32 (bf16), the zero-padded operand copies: x [rows][K1], W1 [Fp][K1] (rows past
// d_inner zero), b1 [Fp], W2 [D][Fp], with K1 = pad_k(d_model) or d_model and
// Fp = pad_k(d_inner) or d_inner.
struct FfWs { size_t f, y, xp, w1p, b1p, w2p, total; int64_t K1, Fp; bool pad; };
FfWs ff_ws_layout(int64_t rows, int64_t D, int64_t Di, int64_t es) {
  FfWs w{};
  const int64_t Dp = pad_k(es, D), Dip = pad_k(es, Di);
  w.K1 = Dp ? Dp : D;
  w.Fp = Dip ? Dip : Di;
  w.pad = (Dp > 0 || Dip > 0) && w.K1 % 32 == 0 && w.Fp % 32 == 0;
  size_t off = 0;
  auto take = [&](int64_t bytes) {
    const size_t o = off;
    off += (size_t)round_up(bytes, 256);
    return o;
  };
  w.f = take(rows * w.Fp * es);
  w.y = take(rows * D * 4);
  w.xp = take(w.pad && Dp ? rows * w.K1 * es : 0);
  w.w1p = take(w.pad ? w.Fp * w.K1 * es : 0);
  w.b1p = take(w.pad ? w.Fp * es : 0);
  w.w2p = take(w.pad ? D * w.Fp * es : 0);
  w.total = off;
  return w;
}

size_t txl_pos_ff_workspace_bytes(int64_t rows, int64_t d_model, int64_t d_inner, int dtype) {
  if ((dtype != TXL_FP32 && dtype != TXL_BF16) || rows < 1 || d_model < 1 || d_inner < 1)
    return 0;
  return ff_ws_layout(rows, d_model, d_inner, elt_size(dtype)).total;
}

int txl_pos_ff(void* stream, int dtype, int64_t rows, int64_t d_model, int64_t d_inner,
               const void* x, const void* W1, const void* b1, const void* W2, const void* b2,
               const void* ln_gamma, const void* ln_beta, float ln_eps, void* out,
               void* workspace, size_t ws_bytes) {
  g_detail[0] = 0;
  if (dtype != TXL_FP32 && dtype != TXL_BF16) return fail(TXL_EUNSUPPORTED, "dtype %d", dtype);
  if (rows < 1 || d_model < 1 || d_inner < 1)
    return fail(TXL_EINVAL, "rows, d_model, d_inner must be >= 1");
  if (rows > 0x7fffffffLL || d_model > 65535 || d_inner > 0x7fffffffLL / 8)
    return fail(TXL_EUNSUPPORTED, "sizes out of range");
  if (!x || !W1 || !b1 || !W2 || !b2 || !ln_gamma || !ln_beta || !out)
    return fail(TXL_EINVAL, "NULL tensor pointer");
  if (!(ln_eps >= 0.f) || !isfinite(ln_eps)) return fail(TXL_EINVAL, "ln_eps must be finite and >= 0");
  if (!workspace) return fail(TXL_EINVAL, "workspace is NULL");
  if ((uintptr_t)workspace % 256) return fail(TXL_EINVAL, "workspace is not 256-byte aligned");
  const size_t need = txl_pos_ff_workspace_bytes(rows, d_model, d_inner, dtype);
  if (ws_bytes < need) return fail(TXL_EWORKSPACE, "need %zu bytes, got %zu", need, ws_bytes);
  const int64_t es = elt_size(dtype), D = d_model, Di = d_inner;
  const Span sx = {(uintptr_t)x, (uintptr_t)x + (uintptr_t)(rows * D * es)};
  const Span so = {(uintptr_t)out, (uintptr_t)out + (uintptr_t)(rows * D * es)};
  const Span sws = {(uintptr_t)workspace, (uintptr_t)workspace + ws_bytes};
  const Span sw[] = {{(uintptr_t)W1, (uintptr_t)W1 + (uintptr_t)(Di * D * es)},
                     {(uintptr_t)W2, (uintptr_t)W2 + (uintptr_t)(D * Di * es)},
                     {(uintptr_t)b1, (uintptr_t)b1 + (uintptr_t)(Di * es)},
                     {(uintptr_t)b2, (uintptr_t)b2 + (uintptr_t)(D * es)},
                     {(uintptr_t)ln_gamma, (uintptr_t)ln_gamma + (uintptr_t)(D * es)},
                     {(uintptr_t)ln_beta, (uintptr_t)ln_beta + (uintptr_t)(D * es)}, sx};
  for (const Span& s : sw)
    if (overlap(so, s) || overlap(sws, s)) return fail(TXL_EINVAL, "out or workspace overlaps an input");
  if (overlap(so, sws)) return fail(TXL_EINVAL, "out overlaps the workspace");

  char* base = (char*)workspace;
  const FfWs fw = ff_ws_layout(rows, D, Di, es);
  void* f = base + fw.f;  // relu(x W1^T + b1), [rows][Di] (pitch Fp when padded)
  float* y = (float*)(base + fw.y);
  hipStream_t st = (hipStream_t)stream;
  // d_model or d_inner not a multiple of 32: both products read zero-padded copies
  // (one launch; the padded inner columns of f come out as relu(0 + 0) = 0)
  auto al4 = [](const void* p) { return (uintptr_t)p % 4 == 0; };
  const bool pad = dtype == TXL_BF16 && fw.pad && al4(x) && al4(W1) && al4(b1) && al4(W2);
  const int64_t K1 = pad ? fw.K1 : D, Fp = pad ? fw.Fp : Di;
  const void *xa = x, *w1 = W1, *bb1 = b1, *w2 = W2;
  if (pad) {
    txl::PadJob pj[5];
    int np = 0;
    if (K1 != D) {
      xa = base + fw.xp;
      pj[np++] = {{nullptr, 1, 0, 0, x, rows, D}, rows, D, K1, (uint16_t*)xa};
    }
    uint16_t* w1p = (uint16_t*)(base + fw.w1p);
    pj[np++] = {{nullptr, 1, 0, 0, W1, Di, D}, Di, D, K1, w1p};
    if (Fp > Di) pj[np++] = {{}, Fp - Di, 0, K1, w1p + Di * K1};
    pj[np++] = {{nullptr, 1, 0, 0, b1, 1, Di}, 1, Di, Fp, (uint16_t*)(base + fw.b1p)};
    pj[np++] = {{nullptr, 1, 0, 0, W2, D, Di}, D, Di, Fp, (uint16_t*)(base + fw.w2p)};
    const hipError_t e = txl::launch_pad_rows(pj, np, st);
    if (e != hipSuccess) return hip_fail(e, "feed-forward padded operands");
    w1 = w1p;
    bb1 = base + fw.b1p;
    w2 = base + fw.w2p;
  }
  txl::GemmArgs g1{};
  g1.M = rows; g1.N = Fp; g1.K = K1;
  g1.a = {nullptr, 1, 0, 0, xa, rows, K1};
  g1.w = {w1, w1, Fp, K1};
  // row-major [rows][Fp] as a single "head" of width Fp
  g1.e = {txl::EPI_HEADS, f, f, Fp, Fp, 0, 0, Fp, nullptr, nullptr, 0, 0, 0, bb1, txl::ACT_RELU};
  int rc = run_gemm(dtype, g1, st, "feed-forward first layer");
  if (rc != TXL_OK) return rc;
  txl::LnArgs ln{rows, D, Fp, f, w2, x, ln_gamma, ln_beta, ln_eps, out, b2};
  if (dtype == TXL_BF16 && rows > 32 && txl::gemm_ln_supported(ln)) {
    const hipError_t e = txl::launch_gemm_ln(ln, st);
    if (e != hipSuccess) return hip_fail(e, "feed-forward second layer + LayerNorm");
    return TXL_OK;
  }
  txl::GemmArgs g2{};
  g2.M = rows; g2.N = D; g2.K = Fp;
  g2.a = {nullptr, 1, 0, 0, f, rows, Fp};
  g2.w = {w2, w2, D, Fp};
  g2.e = {txl::EPI_RESID_F32, nullptr, nullptr, 0, 1, 0, 0, 0, y, x, 0, 0, 0, b2, txl::ACT_NONE};
  if ((rc = run_gemm(dtype, g2, st, "feed-forward second layer")) != TXL_OK) return rc;
  const hipError_t e =
      txl::launch_layer_norm(dtype, y, ln_gamma, ln_beta, ln_eps, rows, D, out, st);
  if (e != hipSuccess) return hip_fail(e, "layer norm");
  return TXL_OK;
}




// ---- attention backward -----------------------------------------------------------------

size_t txl_rel_attn_bwd_workspace_bytes(int dtype, int64_t B, int64_t H, int64_t L,
                                        int64_t mem_len, int64_t d_head) {
  if ((dtype != TXL_FP32 && dtype != TXL_BF16) || B < 1 || H < 1 || L < 1 || mem_len < 0 ||
      d_head < 1 || d_head > 64)
    return 0;
  return txl::attn_bwd_scratch_bytes(B, H, L, mem_len);
}

int txl_rel_attn_bwd(void* stream, int dtype, int64_t B, int64_t H, int64_t L, int64_t mem_len,
                     int64_t d_head, const void* q, int64_t q_sb, int64_t q_st, int64_t q_sh,
                     const void* k, const void* v, int64_t kv_sb, int64_t kv_st, int64_t kv_sh,
                     const void* r, int64_t r_sp, int64_t r_sh, int64_t r_rows,
                     const void* u_bias, const void* v_bias, float scale, const void* dout,
                     int64_t do_sb, int64_t do_st, int64_t do_sh, float* dq, float* dk, float* dv,
                     float* dr, float* du, float* dvb, void* workspace, size_t ws_bytes) {
  g_detail[0] = 0;
  // the forward's checks cover q, k, v, r, u, v and dout (in out's place)
  txl::AttnArgs f{};
  f.B = B; f.H = H; f.L = L; f.mem_len = mem_len; f.d = d_head;
  f.q = q; f.q_sb = q_sb; f.q_st = q_st; f.q_sh = q_sh;
  f.k = k; f.v = v; f.kv_sb = kv_sb; f.kv_st = kv_st; f.kv_sh = kv_sh;
  f.r = r; f.r_sp = r_sp; f.r_sh = r_sh;
  f.u = u_bias; f.vb = v_bias; f.scale = scale;
  f.out = (void*)dout; f.o_sb = do_sb; f.o_st = do_st; f.o_sh = do_sh;
  f.d_load = d_head;
  int rc = check_attn(dtype, f, r_rows);
  if (rc != TXL_OK) return rc;
  if (d_head > 64) return fail(TXL_EUNSUPPORTED, "backward: d_head %lld > 64", (long long)d_head);
  if (!dq || !dk || !dv || !dr || !du || !dvb) return fail(TXL_EINVAL, "NULL gradient pointer");
  const size_t need = txl::attn_bwd_scratch_bytes(B, H, L, mem_len);
  if (!workspace || ws_bytes < need)
    return fail(TXL_EINVAL, "workspace of %zu bytes < %zu", ws_bytes, need);
  const int64_t T = mem_len + L, es = elt_size(dtype);
  const Span outs[] = {{(uintptr_t)dq, (uintptr_t)(dq + B * L * H * d_head)},
                       {(uintptr_t)dk, (uintptr_t)(dk + B * T * H * d_head)},
                       {(uintptr_t)dv, (uintptr_t)(dv + B * T * H * d_head)},
                       {(uintptr_t)dr, (uintptr_t)(dr + T * H * d_head)},
                       {(uintptr_t)du, (uintptr_t)(du + H * d_head)},
                       {(uintptr_t)dvb, (uintptr_t)(dvb + H * d_head)},
                       {(uintptr_t)workspace, (uintptr_t)workspace + ws_bytes}};
  const Span ins[] = {span4(q, B, q_sb, L, q_st, H, q_sh, d_head, es),
                      span4(k, B, kv_sb, T, kv_st, H, kv_sh, d_head, es),
                      span4(v, B, kv_sb, T, kv_st, H, kv_sh, d_head, es),
                      span4(r, 1, 0, T, r_sp, H, r_sh, d_head, es),
                      span4(u_bias, 1, 0, 1, 0, 1, 0, H * d_head, es),
                      span4(v_bias, 1, 0, 1, 0, 1, 0, H * d_head, es),
                      span4(dout, B, do_sb, L, do_st, H, do_sh, d_head, es)};
  const int n_out = sizeof(outs) / sizeof(outs[0]);
  for (int x = 0; x < n_out; ++x) {
    for (const Span& s : ins)
      if (overlap(outs[x], s)) return fail(TXL_EINVAL, "a gradient or the workspace overlaps an input");
    for (int y = x + 1; y < n_out; ++y)
      if (overlap(outs[x], outs[y])) return fail(TXL_EINVAL, "gradients / workspace overlap");
  }
  txl::AttnBwdArgs a{};
  a.B = B; a.H = H; a.L = L; a.mem_len = mem_len; a.d = d_head;
  a.q = q; a.q_sb = q_sb; a.q_st = q_st; a.q_sh = q_sh;
  a.k = k; a.v = v; a.kv_sb = kv_sb; a.kv_st = kv_st; a.kv_sh = kv_sh;
  a.r = r; a.r_sp = r_sp; a.r_sh = r_sh;
  a.u = u_bias; a.vb = v_bias; a.scale = scale;
  a.dout = dout; a.do_sb = do_sb; a.do_st = do_st; a.do_sh = do_sh;
  a.dq = dq; a.dk = dk; a.dv = dv; a.dr = dr; a.du = du; a.dvb = dvb;
  txl::attn_bwd_bind(a, workspace);
  const hipError_t e = txl::launch_attn_bwd(dtype == TXL_BF16 ? 1 : 0, a, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "attention backward launch");
  return TXL_OK;
}


// ---- layer step backward --------------------------------------------------------------
namespace {

// K splits of a weight-gradient product summed over K rows that shares a grid
// with an unsplit product of depth Kref (da for dW_o, dh for the others): enough
// that no split is deeper than that product's tiles, at most 16 and at least 32
// rows deep.  (Splits exist only to balance that grid; each costs its partial's
// write and read.)  A fixed rule of the dims, so the workspace does not depend
// on the device.
int wg_splits(int64_t K, int64_t Kref) {
  int64_t ks = (K + Kref - 1) / std::max<int64_t>(Kref, 32);
  ks = std::min<int64_t>(ks, std::min<int64_t>(K / 32, 16));
  return ks > 1 ? (int)ks : 1;
}

// The five weight-gradient products dW [M][N] over K summed rows (K rounded up
// to 32), each with the depth Kref of the unsplit product of its grid: dW_o
// (with da: K = d_model), dW_q, dW_kE, dW_v, dW_kR (with dh: K = 3 HD).
void wg_shapes(const txl_layer_dims& dm, int64_t cap, int64_t (&sh)[5][4]) {
  const int64_t B = dm.B, L = dm.L, D = dm.d_model, HD = dm.n_head * dm.d_head, T = cap + L;
  const int64_t Kbl = round_up(B * L, 32), Kbt = round_up(B * T, 32), Kt = round_up(T, 32);
  const int64_t Kd = round_up(D, 32), Kc = round_up(3 * HD, 32);
  const int64_t v[5][4] = {{D, HD, Kbl, Kd}, {HD, D, Kbl, Kc}, {HD, D, Kbt, Kc},
                           {HD, D, Kbt, Kc}, {HD, D, Kt, Kc}};
  for (int i = 0; i < 5; ++i)
    for (int j = 0; j < 4; ++j) sh[i][j] = v[i][j];
}
// fp32 partials of one weight gradient (0 when it is not split)
int64_t wg_part_floats(int64_t M, int64_t N, int64_t K, int64_t Kref) {
  const int ks = wg_splits(K, Kref);
  return ks > 1 ? ks * M * N : 0;
}

struct BwdWs {
  size_t fwd, hout, y, dy, mean, rstd, da, dq, dk, dv, dr, ctx, lse, attn, dyb, wot, cat, wcat,
      pko, pkq, pkkv, pkr, part, lnpart, total;
};

BwdWs bwd_ws_layout(const txl_layer_dims& dm, int64_t cap, int dtype) {
  BwdWs w{};
  const int64_t B = dm.B, L = dm.L, D = dm.d_model, HD = dm.n_head * dm.d_head;
  const int64_t T = cap + L, es = elt_size(dtype);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += (bytes + 255) & ~(size_t)255;
    return o;
  };
  w.fwd = take(txl_layer_workspace_bytes(&dm, cap, dtype));
  w.hout = take((size_t)(B * L * D * es));
  w.y = take((size_t)(B * L * D) * 4);
  w.dy = take((size_t)(B * L * D) * 4);
  w.mean = take((size_t)(B * L) * 4);
  w.rstd = take((size_t)(B * L) * 4);
  w.da = take((size_t)(B * L * HD) * 4);
  w.dq = take((size_t)(B * L * HD) * 4);
  w.dk = take((size_t)(B * T * HD) * 4);
  w.dv = take((size_t)(B * T * HD) * 4);
  w.dr = take((size_t)(T * HD) * 4);
  w.ctx = take((size_t)(B * T * D * es));
  w.lse = take((size_t)(B * dm.n_head * L) * 4);
  w.attn = take(txl::attn_bwd_scratch_bytes(B, dm.n_head, L, cap));
  // bf16 layers: the input-gradient products' operands as bf16 rows along K (K
  // rounded up to 32, zero-padded): dy and W_o^T for da; [dq | dk | dv] of the
  // current rows and [W_q^T | W_kE^T | W_v^T] for dh
  const bool mc = dtype == TXL_BF16;
  const int64_t Kd = round_up(D, 32), Kc = round_up(3 * HD, 32);
  w.dyb = take(mc ? (size_t)(B * L * Kd) * 2 : 0);
  w.wot = take(mc ? (size_t)(HD * Kd) * 2 : 0);
  w.cat = take(mc ? (size_t)(B * L * Kc) * 2 : 0);
  w.wcat = take(mc ? (size_t)(D * Kc) * 2 : 0);
  // and the weight-gradient products' operands transposed to rows along the
  // summed rows (B L, B T or T, rounded up to 32): [dy^T ; a^T], [dq^T ; h_in^T],
  // [dk^T ; dv^T ; ctx^T], [dr^T ; R^T], then the K-split partial sums
  const int64_t Kbl = round_up(B * L, 32), Kbt = round_up(B * T, 32), Kt = round_up(T, 32);
  w.pko = take(mc ? (size_t)((D + HD) * Kbl) * 2 : 0);
  w.pkq = take(mc ? (size_t)((HD + D) * Kbl) * 2 : 0);
  w.pkkv = take(mc ? (size_t)((2 * HD + D) * Kbt) * 2 : 0);
  w.pkr = take(mc ? (size_t)((HD + D) * Kt) * 2 : 0);
  // (a region per split weight gradient, taken in the backward's order; all are
  // summed by one launch at the end)
  size_t part = 0;
  if (mc) {
    int64_t sh[5][4];
    wg_shapes(dm, cap, sh);
    for (const auto& x : sh) part += wg_part_floats(x[0], x[1], x[2], x[3]) * 4;
  }
  w.part = take(part);
  // per-workgroup dgamma / dbeta sums of the fused LayerNorm backward
  w.lnpart = take(txl::ln_bwd_fused_ok(B * L, D) ? txl::ln_bwd_part_bytes(B * L, D) : 0);
  w.total = off;
  return w;
}

// Arguments of y = A W^T on the matrix cores: A [M][K] and W [N][K] bf16 rows,
// y fp32 [M][N] (+ an fp32 residual when resid is set).
txl::GemmArgs mm_args(int64_t M, int64_t N, int64_t K, const uint16_t* A, const uint16_t* W,
                      float* y, const float* resid) {
  txl::GemmArgs g{};
  g.M = M; g.N = N; g.K = K;
  g.a = {nullptr, 1, 0, 0, A, M, K};
  g.w = {W, W, N, K, 0, 0};
  g.e.mode = txl::EPI_RESID_F32;
  g.e.y = y;
  g.e.resid = resid;
  g.e.resid_f32 = 1;
  return g;
}

// A weight gradient dW [M][N] = A W^T from the transposed operands A [M][K] and
// W [N][K]: appended to a GEMM batch (into its partial region when split, whose
// sum goes to sums) and the partial region advanced.
void wg_add(int64_t M, int64_t N, int64_t K, int64_t Kref, const uint16_t* A, const uint16_t* W,
            float* dW, float*& part, txl::GemmArgs* gs, int* ks, int& n, txl::SumJob* sums,
            int& nsum) {
  const int k = wg_splits(K, Kref);
  gs[n] = mm_args(M, N, K, A, W, k > 1 ? part : dW, nullptr);
  ks[n++] = k;
  if (k > 1) {
    sums[nsum++] = {part, k, M * N, dW};
    part += k * M * N;
  }
}

// C = alpha A B (+ C), A (m, k) at a + m*am + k*ak, B (k, n) at b + k*bk + n*bn, C row-major
// with row pitch ldc; batch z offsets a_z, b_z, c_z.
hipError_t sgemm(hipStream_t st, int64_t M, int64_t N, int64_t K, const void* a, int adt,
                 int64_t am, int64_t ak, const void* b, int bdt, int64_t bk, int64_t bn, float* c,
                 int64_t ldc, bool acc, int64_t batch = 1, int64_t a_z = 0, int64_t b_z = 0,
                 int64_t c_z = 0) {
  txl::StridedGemm g{};
  g.M = M; g.N = N; g.K = K; g.batch = batch; g.zdiv = 1;
  g.A = {a, a_z, 0, am, ak};
  g.B = {b, b_z, 0, bk, bn};
  g.C = c; g.c1 = c_z; g.c2 = 0; g.cm = ldc; g.cn = 1;
  g.alpha = 1.f; g.accumulate = acc ? 1 : 0;
  g.a_dtype = adt; g.b_dtype = bdt;
  g.bf16_mfma = (adt == 1 || bdt == 1) ? 1 : 0;  // a bf16 layer: bf16 products, fp32 sums
  return txl::launch_gemm_strided(g, st);
}

}  // namespace

size_t txl_layer_bwd_workspace_bytes(const txl_layer_dims* dims, int64_t mem_capacity, int dtype) {
  if (check_dims(dims) != TXL_OK || mem_capacity < 0 || dims->d_head > 64) return 0;
  if (dtype != TXL_FP32 && dtype != TXL_BF16) return 0;
  return bwd_ws_layout(*dims, mem_capacity, dtype).total;
}

// Saved state of a training forward: the layer step's workspace, then the
// attention's log-sum-exp [B][H][L].
struct SavedLayout {
  size_t fwd, lse, total;
};
static SavedLayout saved_layout(const txl_layer_dims& dm, int64_t cap, int dtype) {
  SavedLayout sl{};
  sl.fwd = 0;
  sl.lse = (txl_layer_workspace_bytes(&dm, cap, dtype) + 255) & ~(size_t)255;
  sl.total = sl.lse + (((size_t)(dm.B * dm.n_head * dm.L) * 4 + 255) & ~(size_t)255);
  return sl;
}

size_t txl_layer_saved_bytes(const txl_layer_dims* dims, int64_t mem_capacity, int dtype) {
  if (check_dims(dims) != TXL_OK || mem_capacity < 1) return 0;
  if (dtype != TXL_FP32 && dtype != TXL_BF16) return 0;
  if (txl_layer_workspace_bytes(dims, mem_capacity, dtype) == 0) return 0;
  return saved_layout(*dims, mem_capacity, dtype).total;
}

int txl_layer_step_save(void* stream, int dtype, const txl_layer_dims* dims, const void* h_in,
                        const txl_ring* mem, const txl_layer_weights* w, const void* u_bias,
                        const void* v_bias, const void* R, int64_t R_rows, void* h_out,
                        txl_layer_saved* saved) {
  g_detail[0] = 0;
  if (!saved || !saved->data || (uintptr_t)saved->data % 256)
    return fail(TXL_EINVAL, "saved state is NULL or unaligned");
  int rc = check_dims(dims);
  if (rc != TXL_OK) return rc;
  if (!mem || mem->capacity < 1) return fail(TXL_EINVAL, "ring state is invalid");
  if (dtype != TXL_FP32 && dtype != TXL_BF16) return fail(TXL_EUNSUPPORTED, "dtype %d", dtype);
  const SavedLayout sl = saved_layout(*dims, mem->capacity, dtype);
  if (saved->bytes < sl.total)
    return fail(TXL_EWORKSPACE, "saved state: need %zu bytes, got %zu", sl.total, saved->bytes);
  // the saved state must not overlap the layer's input, output or memory
  // (the workspace part of it is checked again by the step itself)
  {
    const int64_t es = elt_size(dtype), B = dims->B, L = dims->L, D = dims->d_model;
    const Span ssv = {(uintptr_t)saved->data, (uintptr_t)saved->data + saved->bytes};
    const Span others[] = {{(uintptr_t)h_in, (uintptr_t)h_in + (uintptr_t)(B * L * D * es)},
                           {(uintptr_t)h_out, (uintptr_t)h_out + (uintptr_t)(B * L * D * es)},
                           {(uintptr_t)mem->data,
                            (uintptr_t)mem->data + (uintptr_t)(B * mem->capacity * D * es)}};
    for (const Span& o : others)
      if (o.lo && overlap(ssv, o)) return fail(TXL_EINVAL, "the saved state overlaps an argument");
  }
  char* base = (char*)saved->data;
  bool has_lse = false, has_y = false;
  rc = layer_step_run(stream, dtype, dims, h_in, mem, w, u_bias, v_bias, R, R_rows, h_out,
                      base + sl.fwd, sl.lse - sl.fwd, (float*)(base + sl.lse), &has_lse, &has_y);
  saved->has_lse = has_lse ? 1 : 0;
  saved->has_y = has_y ? 1 : 0;
  // what the state belongs to (the backward checks it)
  saved->mem_data = mem->data;
  saved->mem_capacity = mem->capacity;
  saved->mem_start = mem->start;
  saved->mem_len = mem->len;
  saved->h_in = h_in;
  saved->B = dims->B;
  saved->L = dims->L;
  saved->d_model = dims->d_model;
  saved->n_head = dims->n_head;
  saved->d_head = dims->d_head;
  saved->dtype = dtype;
  return rc;
}

static int layer_bwd_run(void* stream, int dtype, const txl_layer_dims* dims, const void* h_in,
                         const txl_ring* mem, const txl_layer_weights* w, const void* u_bias,
                         const void* v_bias, const void* R, int64_t R_rows, const void* dh_out,
                         const txl_layer_saved* saved, const txl_layer_grads* g, void* workspace,
                         size_t ws_bytes) {
  g_detail[0] = 0;
  if (dtype != TXL_FP32 && dtype != TXL_BF16) return fail(TXL_EUNSUPPORTED, "dtype %d", dtype);
  int rc = check_dims(dims);
  if (rc != TXL_OK) return rc;
  if (dims->d_head > 64)
    return fail(TXL_EUNSUPPORTED, "backward: d_head %lld > 64", (long long)dims->d_head);
  if (!mem || !g || !dh_out) return fail(TXL_EINVAL, "NULL argument");
  if (!g->dh || !g->dW_q || !g->dW_kE || !g->dW_v || !g->dW_kR || !g->dW_o || !g->du ||
      !g->dv_bias || !g->dgamma || !g->dbeta)
    return fail(TXL_EINVAL, "NULL gradient pointer");
  if (!workspace || (uintptr_t)workspace % 256) return fail(TXL_EINVAL, "workspace is NULL or unaligned");
  const txl_layer_dims dm = *dims;
  const int64_t B = dm.B, L = dm.L, D = dm.d_model, H = dm.n_head, d = dm.d_head, HD = H * d;
  if (mem->capacity < 1 || mem->len < 0 || mem->len > mem->capacity)
    return fail(TXL_EINVAL, "ring state is invalid");
  const BwdWs bw = bwd_ws_layout(dm, mem->capacity, dtype);
  if (ws_bytes < bw.total) return fail(TXL_EWORKSPACE, "need %zu bytes, got %zu", bw.total, ws_bytes);
  const int64_t len = mem->len, T = len + L, es = elt_size(dtype);
  const int dt = dtype == TXL_BF16 ? 1 : 0;
  // gradients must not overlap each other, the inputs or the workspace
  const Span outs[] = {{(uintptr_t)g->dh, (uintptr_t)(g->dh + B * L * D)},
                       {(uintptr_t)g->dW_q, (uintptr_t)(g->dW_q + HD * D)},
                       {(uintptr_t)g->dW_kE, (uintptr_t)(g->dW_kE + HD * D)},
                       {(uintptr_t)g->dW_v, (uintptr_t)(g->dW_v + HD * D)},
                       {(uintptr_t)g->dW_kR, (uintptr_t)(g->dW_kR + HD * D)},
                       {(uintptr_t)g->dW_o, (uintptr_t)(g->dW_o + D * HD)},
                       {(uintptr_t)g->du, (uintptr_t)(g->du + HD)},
                       {(uintptr_t)g->dv_bias, (uintptr_t)(g->dv_bias + HD)},
                       {(uintptr_t)g->dgamma, (uintptr_t)(g->dgamma + D)},
                       {(uintptr_t)g->dbeta, (uintptr_t)(g->dbeta + D)},
                       {(uintptr_t)workspace, (uintptr_t)workspace + ws_bytes}};
  SavedLayout sl{};
  if (saved) {
    sl = saved_layout(dm, mem->capacity, dtype);
    if (!saved->data || (uintptr_t)saved->data % 256 || saved->bytes < sl.total)
      return fail(TXL_EINVAL, "saved state is NULL, unaligned or short");
    if (!w || !w->W_q || !w->W_kE || !w->W_v || !w->W_kR || !w->W_o || !w->ln_gamma ||
        !w->ln_beta || !h_in || !u_bias || !v_bias || !R || !mem->data)
      return fail(TXL_EINVAL, "NULL argument");
    if (R_rows < mem->len + L) return fail(TXL_EINVAL, "R_rows < mem->len + L");
    if (saved->mem_data != mem->data || saved->mem_capacity != mem->capacity ||
        saved->mem_start != mem->start || saved->mem_len != mem->len)
      return fail(TXL_EINVAL,
                  "the memory differs from the one the state was saved with (ring start %lld "
                  "len %lld then, %lld %lld now): run the backward before the memory update",
                  (long long)saved->mem_start, (long long)saved->mem_len, (long long)mem->start,
                  (long long)mem->len);
    if (saved->h_in != h_in || saved->dtype != dtype || saved->B != dm.B || saved->L != dm.L ||
        saved->d_model != dm.d_model || saved->n_head != dm.n_head || saved->d_head != dm.d_head)
      return fail(TXL_EINVAL, "h_in, the dims or the dtype differ from the saved forward's");
  }
  const Span ssaved = {(uintptr_t)(saved ? saved->data : nullptr),
                       (uintptr_t)(saved ? (char*)saved->data + saved->bytes : nullptr)};
  const Span ins[] = {{(uintptr_t)h_in, (uintptr_t)h_in + (uintptr_t)(B * L * D * es)},
                      {(uintptr_t)dh_out, (uintptr_t)dh_out + (uintptr_t)(B * L * D * es)},
                      {(uintptr_t)mem->data,
                       (uintptr_t)mem->data + (uintptr_t)(B * mem->capacity * D * es)}};
  const int n_out = sizeof(outs) / sizeof(outs[0]);
  for (int x = 0; x < n_out; ++x) {
    for (const Span& sp : ins)
      if (overlap(outs[x], sp)) return fail(TXL_EINVAL, "a gradient or the workspace overlaps an input");
    for (int y = x + 1; y < n_out; ++y)
      if (overlap(outs[x], outs[y])) return fail(TXL_EINVAL, "gradients / workspace overlap");
    if (saved && overlap(outs[x], ssaved))
      return fail(TXL_EINVAL, "a gradient or the workspace overlaps the saved state");
  }
  char* base = (char*)workspace;
  hipStream_t st = (hipStream_t)stream;
  // q, k, v, r and a: the saved forward's, or the forward again (which also
  // checks the remaining arguments)
  bool have_lse = false, have_y = false;
  char* fb = base + bw.fwd;
  float* lse = (float*)(base + bw.lse);
  if (saved) {
    fb = (char*)saved->data + sl.fwd;
    lse = (float*)((char*)saved->data + sl.lse);
    have_lse = saved->has_lse != 0;
    have_y = saved->has_y != 0;
  } else {
    rc = layer_step_run(stream, dtype, dims, h_in, mem, w, u_bias, v_bias, R, R_rows,
                        base + bw.hout, fb, bw.hout - bw.fwd, lse, &have_lse, &have_y);
    if (rc != TXL_OK) return rc;
  }
  const WsLayout fl = ws_layout(dm, T, es);
  const void* q = fb + fl.q;
  const void* k = fb + fl.k;
  const void* v = fb + fl.v;
  const void* r = fb + fl.r;
  const void* a = fb + fl.a;
  const int64_t dp = fl.dp;
  // y = a W_o^T + h_in: the forward's own when it wrote one (the unfused output
  // projection), else recomputed below
  float* y = have_y ? (float*)(fb + fl.y) : (float*)(base + bw.y);
  float* dy = (float*)(base + bw.dy);
  float* da = (float*)(base + bw.da);
  float* dq = (float*)(base + bw.dq);
  float* dk = (float*)(base + bw.dk);
  float* dv = (float*)(base + bw.dv);
  float* dr = (float*)(base + bw.dr);
  void* ctx = base + bw.ctx;
  const int64_t BL = B * L;
  hipError_t e;
#define TXL_TRY(x, what) do { if ((e = (x)) != hipSuccess) return hip_fail(e, what); } while (0)
  // every output that is summed into (atomically or by accumulating products),
  // cleared in one launch
  {
    // (bf16 layers store the weight gradients and da whole)
    const int64_t wz = dt == 1 ? 0 : HD * D;
    float* zp[] = {g->dgamma, g->dbeta, g->du, g->dv_bias, dr, g->dW_o, g->dW_q, g->dW_kE,
                   g->dW_v, g->dW_kR, da};
    const int64_t zn[] = {D, D, HD, HD, T * HD, wz, wz, wz, wz, wz, dt == 1 ? 0 : BL * HD};
    TXL_TRY(txl::launch_zero_many(zp, zn, 11, st), "clear");
  }
  // y = a W_o^T + h_in (the LayerNorm input), then the LayerNorm backward
  if (!have_y) {
    TXL_TRY(txl::launch_to_f32(dt, h_in, y, BL * D, st), "copy");
    TXL_TRY(sgemm(st, BL, D, HD, a, dt, HD, 1, w->W_o, dt, 1, HD, y, D, true), "y");
  }
  const int64_t Kd = round_up(D, 32), Kc = round_up(3 * HD, 32);
  const int64_t Kbl = round_up(BL, 32), Kbt = round_up(B * T, 32), Kt = round_up(T, 32);
  uint16_t* dyb = (uint16_t*)(base + bw.dyb);
  // (D a multiple of 256: one wave per row, which also writes dy's bf16 rows)
  const bool ln_fused = txl::ln_bwd_fused_ok(BL, D);
  if (ln_fused)
    TXL_TRY(txl::launch_ln_bwd_fused(dt, y, w->ln_gamma, dh_out, BL, D, dm.ln_eps, dy,
                                     dt == 1 ? dyb : nullptr, Kd, (float*)(base + bw.lnpart),
                                     g->dgamma, g->dbeta, st), "layernorm backward");
  else
    TXL_TRY(txl::launch_ln_bwd(dt, y, w->ln_gamma, dh_out, BL, D, dm.ln_eps, dy,
                               (float*)(base + bw.mean), (float*)(base + bw.rstd), g->dgamma,
                               g->dbeta, st, true), "layernorm backward");
  // dW_o = dy^T a, da = dy W_o.  bf16 layers: both on the matrix cores, from dy
  // as bf16 rows, W_o^T, dy^T and a^T packed in one launch
  float* part_next = (float*)(base + bw.part);
  txl::SumJob sums[5];
  int nsum = 0;
  if (dt == 1) {
    uint16_t* wot = (uint16_t*)(base + bw.wot);
    uint16_t* ao = (uint16_t*)(base + bw.pko);
    uint16_t* wo = ao + D * Kbl;
    const txl::PackJob jobs[] = {
        txl::pack_trans(w->W_o, 1, HD, D, Kd, HD, wot, Kd),
        txl::pack_trans(dy, 0, D, BL, Kbl, D, ao, Kbl),
        txl::pack_trans(a, 1, HD, BL, Kbl, HD, wo, Kbl),
        txl::pack_rows(dy, 0, BL, D, Kd, BL, 0, D, dyb, Kd)};
    TXL_TRY(txl::launch_pack(jobs, ln_fused ? 3 : 4, st), "operand packs");
    // da and dW_o in one grid (dW_o's partials are summed with the others at the end)
    txl::GemmArgs gs[2];
    int ks[2], n = 0;
    gs[n] = mm_args(BL, HD, Kd, dyb, wot, da, nullptr);
    ks[n++] = 1;
    wg_add(D, HD, Kbl, Kd, ao, wo, g->dW_o, part_next, gs, ks, n, sums, nsum);
    TXL_TRY(txl::launch_gemm_batch(gs, ks, n, st, num_cus()), "da, dW_o");
  } else {
    TXL_TRY(sgemm(st, D, HD, BL, dy, 0, 1, D, a, dt, HD, 1, g->dW_o, HD, true), "dW_o");
    TXL_TRY(sgemm(st, BL, HD, D, dy, 0, D, 1, w->W_o, dt, HD, 1, da, HD, true), "da");
  }
  // attention backward on the forward's head-major q, k, v, r
  txl::AttnBwdArgs ab{};
  ab.B = B; ab.H = H; ab.L = L; ab.mem_len = len; ab.d = d;
  ab.q = q; ab.q_sb = H * L * dp; ab.q_st = dp; ab.q_sh = L * dp;
  ab.k = k; ab.v = v; ab.kv_sb = H * T * dp; ab.kv_st = dp; ab.kv_sh = T * dp;
  ab.r = r; ab.r_sp = dp; ab.r_sh = T * dp;
  ab.u = u_bias; ab.vb = v_bias; ab.scale = 1.0f / sqrtf((float)d);
  ab.dout = da; ab.do_sb = L * HD; ab.do_st = HD; ab.do_sh = d; ab.dout_f32 = 1;
  ab.dq = dq; ab.dk = dk; ab.dv = dv; ab.dr = dr; ab.du = g->du; ab.dvb = g->dv_bias;
  ab.zeroed = 1;  // du, dv_bias and dr were cleared above
  if (have_lse) {  // the forward's softmax statistics and output
    ab.lse = lse;
    ab.o = a; ab.o_sb = L * HD; ab.o_st = HD; ab.o_sh = d;
  }
  txl::attn_bwd_bind(ab, base + bw.attn);
  TXL_TRY(txl::launch_attn_bwd(dt, ab, st), "attention backward");
  // projection weights: dW_q = dq^T h_in, dW_kE = dk^T ctx, dW_v = dv^T ctx, dW_kR = dr^T R
  // (bf16 layers pack ctx^T straight from the ring and h_in instead)
  if (dt != 1)
    TXL_TRY(txl::launch_gather_ctx(dt, mem->data, mem->capacity, mem->start, len, h_in, B, L, D,
                                   ctx, st), "context gather");
  // dh = dy + dq W_q + (dk W_kE + dv W_v) on the current rows (the memory's gradient is stopped)
  if (dt == 1) {
    // one launch packs the four weight gradients' operands and dh's: one product
    // over K = 3 HD, [dq | dk | dv] (bf16 rows) times [W_q^T | W_kE^T | W_v^T]
    uint16_t* cat = (uint16_t*)(base + bw.cat);
    uint16_t* wcat = (uint16_t*)(base + bw.wcat);
    uint16_t* aq = (uint16_t*)(base + bw.pkq);
    uint16_t* wq = aq + HD * Kbl;
    uint16_t* ak = (uint16_t*)(base + bw.pkkv);
    uint16_t* av = ak + HD * Kbt;
    uint16_t* wc = av + HD * Kbt;
    uint16_t* ar = (uint16_t*)(base + bw.pkr);
    uint16_t* wr = ar + HD * Kt;
    // dq, dk and dv are read once: their transposes for the weight gradients also
    // write the current rows into [dq | dk | dv] (dst2); the columns of that
    // operand past 3 HD are zeros
    txl::PackJob jobs[] = {
        txl::pack_trans(dq, 0, HD, BL, Kbl, HD, aq, Kbl),
        txl::pack_trans(h_in, 1, D, BL, Kbl, D, wq, Kbl),
        txl::pack_trans(dk, 0, HD, B * T, Kbt, HD, ak, Kbt),
        txl::pack_trans(dv, 0, HD, B * T, Kbt, HD, av, Kbt),
        txl::pack_trans_ctx(mem->data, mem->capacity, mem->start, len, h_in, L, B, 1, D, Kbt, D,
                            wc, Kbt),
        txl::pack_trans(dr, 0, HD, T, Kt, HD, ar, Kt),
        txl::pack_trans(R, 1, D, T, Kt, D, wr, Kt),
        txl::pack_trans(w->W_q, 1, D, HD, HD, D, wcat, Kc),
        txl::pack_trans(w->W_kE, 1, D, HD, HD, D, wcat + HD, Kc),
        txl::pack_trans(w->W_v, 1, D, HD, Kc - 2 * HD, D, wcat + 2 * HD, Kc),
        txl::pack_rows(dq, 0, BL, 0, Kc - 3 * HD, BL, 0, HD, cat + 3 * HD, Kc)};
    auto rows_too = [&](txl::PackJob& j, uint16_t* d2, int64_t per2, int64_t skip2) {
      j.dst2 = d2; j.ldd2 = Kc; j.per2 = per2; j.skip2 = skip2;
    };
    rows_too(jobs[0], cat, L, 0);
    rows_too(jobs[2], cat + HD, T, len);
    rows_too(jobs[3], cat + 2 * HD, T, len);
    TXL_TRY(txl::launch_pack(jobs, Kc > 3 * HD ? 11 : 10, st), "operand packs");
    // dh (its tiles the longest: first) and the four weight gradients in one grid,
    // then every split weight gradient's partials summed in one launch
    txl::GemmArgs gs[5];
    int ks[5], n = 0;
    gs[n] = mm_args(BL, D, Kc, cat, wcat, g->dh, dy);
    ks[n++] = 1;
    wg_add(HD, D, Kbt, Kc, ak, wc, g->dW_kE, part_next, gs, ks, n, sums, nsum);
    wg_add(HD, D, Kbt, Kc, av, wc, g->dW_v, part_next, gs, ks, n, sums, nsum);
    wg_add(HD, D, Kbl, Kc, aq, wq, g->dW_q, part_next, gs, ks, n, sums, nsum);
    wg_add(HD, D, Kt, Kc, ar, wr, g->dW_kR, part_next, gs, ks, n, sums, nsum);
    TXL_TRY(txl::launch_gemm_batch(gs, ks, n, st, num_cus()), "dh and weight gradients");
    if (nsum) TXL_TRY(txl::launch_sum_partials_multi(sums, nsum, st), "weight-gradient sums");
  } else {
    TXL_TRY(sgemm(st, HD, D, BL, dq, 0, 1, HD, h_in, dt, D, 1, g->dW_q, D, true), "dW_q");
    TXL_TRY(sgemm(st, HD, D, B * T, dk, 0, 1, HD, ctx, dt, D, 1, g->dW_kE, D, true), "dW_kE");
    TXL_TRY(sgemm(st, HD, D, B * T, dv, 0, 1, HD, ctx, dt, D, 1, g->dW_v, D, true), "dW_v");
    TXL_TRY(sgemm(st, HD, D, T, dr, 0, 1, HD, R, dt, D, 1, g->dW_kR, D, true), "dW_kR");
    TXL_TRY(txl::launch_to_f32(0, dy, g->dh, BL * D, st), "copy");
    TXL_TRY(sgemm(st, BL, D, HD, dq, 0, HD, 1, w->W_q, dt, D, 1, g->dh, D, true), "dh q");
    TXL_TRY(sgemm(st, L, D, HD, dk + len * HD, 0, HD, 1, w->W_kE, dt, D, 1, g->dh, D, true, B,
                  T * HD, 0, L * D), "dh k");
    TXL_TRY(sgemm(st, L, D, HD, dv + len * HD, 0, HD, 1, w->W_v, dt, D, 1, g->dh, D, true, B,
                  T * HD, 0, L * D), "dh v");
  }
#undef TXL_TRY
  return TXL_OK;
}

int txl_layer_step_bwd(void* stream, int dtype, const txl_layer_dims* dims, const void* h_in,
                       const txl_ring* mem, const txl_layer_weights* w, const void* u_bias,
                       const void* v_bias, const void* R, int64_t R_rows, const void* dh_out,
                       const txl_layer_grads* g, void* workspace, size_t ws_bytes) {
  return layer_bwd_run(stream, dtype, dims, h_in, mem, w, u_bias, v_bias, R, R_rows, dh_out,
                       nullptr, g, workspace, ws_bytes);
}

int txl_layer_step_bwd_saved(void* stream, int dtype, const txl_layer_dims* dims,
                             const void* h_in, const txl_ring* mem, const txl_layer_weights* w,
                             const void* u_bias, const void* v_bias, const void* R,
                             int64_t R_rows, const void* dh_out, const txl_layer_saved* saved,
                             const txl_layer_grads* g, void* workspace, size_t ws_bytes) {
  if (!saved) return fail(TXL_EINVAL, "saved state is NULL");
  return layer_bwd_run(stream, dtype, dims, h_in, mem, w, u_bias, v_bias, R, R_rows, dh_out,
                       saved, g, workspace, ws_bytes);
}

}  // extern "C"
