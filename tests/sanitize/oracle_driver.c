/*
 * Drives every function of the C oracle (oracle/txl_oracle.c) on small seeded
 * inputs, including the edge shapes (no memory, one query, one head of size 1,
 * a memory longer than the segment, eviction in the memory update), for a build
 * with AddressSanitizer and UndefinedBehaviorSanitizer.  It checks nothing about
 * the values (the pins do that); a sanitizer report or a non-zero exit fails.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

void txo_rel_attn(int64_t B, int64_t H, int64_t L, int64_t mem_len, int64_t d, const double* q,
                  const double* k, const double* v, const double* r, const double* u,
                  const double* vb, double scale, double* out, double* scores);
void txo_linear(int64_t rows, int64_t n_out, int64_t n_in, const double* x, const double* W,
                double* y);
void txo_layer_norm(int64_t rows, int64_t D, const double* x, const double* gamma,
                    const double* beta, double eps, double* y);
int txo_pos_ff(int64_t rows, int64_t D, int64_t Di, const double* x, const double* W1,
               const double* b1, const double* W2, const double* b2, const double* gamma,
               const double* beta, double eps, double* out);
int txo_layer_step(int64_t B, int64_t L, int64_t D, int64_t H, int64_t d, int64_t mem_len,
                   double eps, const double* h, const double* mem, const double* W_q,
                   const double* W_kE, const double* W_v, const double* W_kR, const double* W_o,
                   const double* gamma, const double* beta, const double* u, const double* vb,
                   const double* R, double* h_out, double* q_out, double* k_out, double* v_out,
                   double* r_out, double* a_out);
int txo_layer_step_rows(int64_t B, int64_t L, int64_t D, int64_t H, int64_t d, int64_t mem_len,
                        double eps, const double* h, const double* mem, const double* W_q,
                        const double* W_kE, const double* W_v, const double* W_kR,
                        const double* W_o, const double* gamma, const double* beta,
                        const double* u, const double* vb, const double* R, int64_t n_rows,
                        const int64_t* bs, const int64_t* is, double* out);
int64_t txo_mem_update(int64_t B, int64_t M, int64_t D, const double* mem, int64_t mem_len,
                       const double* h, int64_t L, double* out);

static uint64_t state = 12345;
static double rnd(void) {  /* xorshift64*, uniform in [-1, 1) */
  state ^= state >> 12;
  state ^= state << 25;
  state ^= state >> 27;
  return (double)((state * 2685821657736338717ULL) >> 11) / 4503599627370496.0 - 1.0;
}
static double* arr(int64_t n) {
  double* p = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
  for (int64_t i = 0; i < n; ++i) p[i] = rnd();
  return p;
}

static void attn_case(int64_t B, int64_t H, int64_t L, int64_t M, int64_t d) {
  const int64_t T = M + L;
  double *q = arr(B * L * H * d), *k = arr(B * T * H * d), *v = arr(B * T * H * d);
  double *r = arr(T * H * d), *u = arr(H * d), *vb = arr(H * d);
  double *out = arr(B * L * H * d), *sc = arr(B * H * L * T);
  txo_rel_attn(B, H, L, M, d, q, k, v, r, u, vb, 0.25, out, sc);
  txo_rel_attn(B, H, L, M, d, q, k, v, r, u, vb, 0.25, out, NULL);
  free(q); free(k); free(v); free(r); free(u); free(vb); free(out); free(sc);
}

static void layer_case(int64_t B, int64_t L, int64_t D, int64_t H, int64_t d, int64_t M) {
  const int64_t T = M + L, HD = H * d;
  double *h = arr(B * L * D), *mem = arr(B * M * D);
  double *Wq = arr(HD * D), *Wk = arr(HD * D), *Wv = arr(HD * D), *Wr = arr(HD * D);
  double *Wo = arr(D * HD), *g = arr(D), *be = arr(D), *u = arr(HD), *vb = arr(HD);
  double *R = arr(T * D), *ho = arr(B * L * D);
  double *qo = arr(B * L * HD), *ko = arr(B * T * HD), *vo = arr(B * T * HD);
  double *ro = arr(T * HD), *ao = arr(B * L * HD);
  if (txo_layer_step(B, L, D, H, d, M, 1e-5, h, M ? mem : NULL, Wq, Wk, Wv, Wr, Wo, g, be, u, vb,
                     R, ho, qo, ko, vo, ro, ao) != 0)
    exit(2);
  int64_t bs[3] = {0, B - 1, B / 2}, is[3] = {0, L - 1, L / 2};
  double* rows = arr(3 * D);
  if (txo_layer_step_rows(B, L, D, H, d, M, 1e-5, h, M ? mem : NULL, Wq, Wk, Wv, Wr, Wo, g, be,
                          u, vb, R, 3, bs, is, rows) != 0)
    exit(3);
  double* nm = arr(B * (M > 0 ? M : 1) * D);
  (void)txo_mem_update(B, M > 0 ? M : 1, D, M ? mem : NULL, M, h, L, nm);
  double *x = arr(5 * D), *W1 = arr(3 * D * D), *b1 = arr(3 * D), *W2 = arr(D * 3 * D);
  double *b2 = arr(D), *po = arr(5 * D), *lin = arr(5 * 3 * D);
  txo_linear(5, 3 * D, D, x, W1, lin);
  txo_layer_norm(5, D, x, g, be, 1e-5, po);
  if (txo_pos_ff(5, D, 3 * D, x, W1, b1, W2, b2, g, be, 1e-5, po) != 0) exit(4);
  free(h); free(mem); free(Wq); free(Wk); free(Wv); free(Wr); free(Wo); free(g); free(be);
  free(u); free(vb); free(R); free(ho); free(qo); free(ko); free(vo); free(ro); free(ao);
  free(rows); free(nm); free(x); free(W1); free(b1); free(W2); free(b2); free(po); free(lin);
}

int main(void) {
  attn_case(1, 2, 16, 16, 16);
  attn_case(2, 1, 1, 0, 1);
  attn_case(1, 3, 5, 0, 8);
  attn_case(1, 1, 3, 11, 4);
  layer_case(2, 9, 12, 2, 6, 7);
  layer_case(1, 1, 8, 1, 8, 0);
  layer_case(2, 4, 10, 2, 5, 13);
  puts("oracle driver done");
  return 0;
}
