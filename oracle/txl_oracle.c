/*
 * CPU oracle for Transformer-XL relative-position attention over segment-level
 * memory.  TEST INFRASTRUCTURE ONLY: it is called by the tests, by the smoke
 * check and by the CPU-baseline leg of the benchmark, never by the product
 * path.  It shares no code, header or table with the HIP library.
 *
 * Everything is fp64 and computes the plain definition written out:
 *   - no relative-shift trick, no tiling, no ring buffer, no virtual concat;
 *   - memory is passed in logical order (oldest row first);
 *   - every score A[i][j] is computed by direct indexing of the distance i-j.
 *
 * Source: Dai et al., "Transformer-XL: Attentive Language Models Beyond a
 * Fixed-Length Context" (arXiv 1901.02860v3):
 *   section 3.2 (segment-level recurrence, the extended context
 *       [SG(m) o h] and the length-M memory that spans segments),
 *   section 3.3 (the relative score A^rel with terms (a)-(d), the global
 *       biases u and v, separate W_{k,E} and W_{k,R}, and the N-layer
 *       procedure: masked softmax, Linear + residual + LayerNorm),
 *   Appendix B (the distance i-j ranges over 0 .. M+L-1; key j of query i
 *       sits at distance M+i-j, distance 0 is the query itself).
 *
 * Readings where the pages are silent (each is listed in the design notes):
 *   - the whole four-term score is multiplied by `scale` (1/sqrt(d_head));
 *   - key j is visible to query i iff j <= mem_len + i (self included);
 *   - queries come from the current rows only, keys/values from [mem ; h];
 *   - multi-head: head hd uses rows hd*d .. hd*d+d-1 of every projection;
 *   - LayerNorm is post-norm, biased variance, eps given, gamma/beta given;
 *   - no bias terms in the attention projections;
 *   - the position-wise feed-forward (section 3.3 names it, leaves its inside
 *     open) is the two-layer ReLU network with biases and a post-norm
 *     residual: LayerNorm(x + relu(x W1^T + b1) W2^T + b2);
 *   - the new memory is the last min(M, len+L) rows of [old memory ; h].
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int txo_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Threads of the parallel regions that follow (the benchmark's 1-thread run). */
void txo_set_num_threads(int n) {
#ifdef _OPENMP
    if (n >= 1) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

static double dot(const double* a, const double* b, int64_t n) {
    double s = 0.0;
    for (int64_t c = 0; c < n; ++c) s += a[c] * b[c];
    return s;
}

/*
 * Relative-position attention for B batch rows and H heads (section 3.3,
 * the A^rel equation and the N-layer procedure's masked softmax).
 *
 *   q   [B, L, H, d]            queries of the current segment
 *   k,v [B, T, H, d]            keys/values over [memory ; current], T = mem_len+L
 *   r   [T, H, d]               r[p] = W_{k,R} R_p, the projected encoding of distance p
 *   u,vb [H, d]                 global content bias u and position bias v
 *   out [B, L, H, d]
 *   scores  NULL or [B, H, L, T]: scaled score, -INFINITY where masked
 *
 * For query i and key j <= mem_len+i, with p = mem_len+i-j:
 *   A = scale * ( q_i.k_j      (a) content addressing
 *               + q_i.r_p      (b) content-dependent position bias
 *               + u.k_j        (c) global content bias
 *               + vb.r_p )     (d) global position bias
 */
void txo_rel_attn(int64_t B, int64_t H, int64_t L, int64_t mem_len, int64_t d,
                  const double* q, const double* k, const double* v,
                  const double* r, const double* u, const double* vb,
                  double scale, double* out, double* scores) {
    const int64_t T = mem_len + L;
#pragma omp parallel
    {
        double* A = (double*)malloc(sizeof(double) * (size_t)(T > 0 ? T : 1));
#pragma omp for collapse(3) schedule(dynamic, 4)
        for (int64_t b = 0; b < B; ++b)
            for (int64_t hd = 0; hd < H; ++hd)
                for (int64_t i = 0; i < L; ++i) {
                    const double* qi = q + ((b * L + i) * H + hd) * d;
                    const double* uh = u + hd * d;
                    const double* vh = vb + hd * d;
                    double amax = -INFINITY;
                    for (int64_t j = 0; j < T; ++j) {
                        if (j > mem_len + i) { A[j] = -INFINITY; continue; }
                        const int64_t p = mem_len + i - j;
                        const double* kj = k + ((b * T + j) * H + hd) * d;
                        const double* rp = r + (p * H + hd) * d;
                        const double ta = dot(qi, kj, d);
                        const double tb = dot(qi, rp, d);
                        const double tc = dot(uh, kj, d);
                        const double td = dot(vh, rp, d);
                        A[j] = scale * (ta + tb + tc + td);
                        if (A[j] > amax) amax = A[j];
                    }
                    if (scores) {
                        double* srow = scores + ((b * H + hd) * L + i) * T;
                        for (int64_t j = 0; j < T; ++j) srow[j] = A[j];
                    }
                    /* softmax over the visible keys; masked keys weigh exactly 0 */
                    double den = 0.0;
                    for (int64_t j = 0; j <= mem_len + i; ++j) {
                        A[j] = exp(A[j] - amax);
                        den += A[j];
                    }
                    double* oi = out + ((b * L + i) * H + hd) * d;
                    for (int64_t c = 0; c < d; ++c) oi[c] = 0.0;
                    for (int64_t j = 0; j <= mem_len + i; ++j) {
                        const double pj = A[j] / den;
                        const double* vj = v + ((b * T + j) * H + hd) * d;
                        for (int64_t c = 0; c < d; ++c) oi[c] += pj * vj[c];
                    }
                }
        free(A);
    }
}

/* y[m][n] = sum_c x[m][c] * W[n][c]   (the pages write projections as h W^T) */
void txo_linear(int64_t rows, int64_t n_out, int64_t n_in, const double* x,
                const double* W, double* y) {
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t m = 0; m < rows; ++m)
        for (int64_t n = 0; n < n_out; ++n)
            y[m * n_out + n] = dot(x + m * n_in, W + n * n_in, n_in);
}

/* Post-norm LayerNorm of one row: biased variance over D, then gamma, beta. */
static void layer_norm_row(int64_t D, const double* x, const double* gamma,
                           const double* beta, double eps, double* y) {
    double mean = 0.0;
    for (int64_t c = 0; c < D; ++c) mean += x[c];
    mean /= (double)D;
    double var = 0.0;
    for (int64_t c = 0; c < D; ++c) var += (x[c] - mean) * (x[c] - mean);
    var /= (double)D;
    const double inv = 1.0 / sqrt(var + eps);
    for (int64_t c = 0; c < D; ++c) y[c] = (x[c] - mean) * inv * gamma[c] + beta[c];
}

void txo_layer_norm(int64_t rows, int64_t D, const double* x, const double* gamma,
                    const double* beta, double eps, double* y) {
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < rows; ++m)
        layer_norm_row(D, x + m * D, gamma, beta, eps, y + m * D);
}

/*
 * Position-wise feed-forward of the N-layer procedure (section 3.3, the step
 * h = Positionwise-Feed-Forward(o) after the attention sublayer), per row:
 *   f   = relu(x W1^T + b1)          W1 [Di, D], b1 [Di]
 *   out = LayerNorm(x + f W2^T + b2)  W2 [D, Di], b2 [D], biased variance, eps
 *   x, out [rows, D]
 * Returns 0, or -1 if scratch allocation fails.
 */
int txo_pos_ff(int64_t rows, int64_t D, int64_t Di, const double* x, const double* W1,
               const double* b1, const double* W2, const double* b2, const double* gamma,
               const double* beta, double eps, double* out) {
    double* f = (double*)malloc(sizeof(double) * (size_t)(rows * Di));
    double* y = (double*)malloc(sizeof(double) * (size_t)(rows * D));
    if (!f || !y) {
        free(f);
        free(y);
        return -1;
    }
    txo_linear(rows, Di, D, x, W1, f);
    for (int64_t m = 0; m < rows; ++m)
        for (int64_t c = 0; c < Di; ++c) {
            const double t = f[m * Di + c] + b1[c];
            f[m * Di + c] = t > 0.0 ? t : 0.0;
        }
    txo_linear(rows, D, Di, f, W2, y);
    for (int64_t m = 0; m < rows; ++m)
        for (int64_t c = 0; c < D; ++c) y[m * D + c] += b2[c] + x[m * D + c];
    txo_layer_norm(rows, D, y, gamma, beta, eps, out);
    free(f);
    free(y);
    return 0;
}

/*
 * One layer n for one segment (section 3.3, the N-layer procedure, without
 * the position-wise feed-forward):
 *   ctx = [mem ; h]                         extended context, T = mem_len+L rows
 *   q = h W_q^T,  k = ctx W_kE^T,  v = ctx W_v^T,  r = R[0:T] W_kR^T
 *   a = masked softmax(A^rel) v             per head, heads concatenated
 *   h_out = LayerNorm(a W_o^T + h)
 *
 *   h    [B, L, D]        layer input of the current segment
 *   mem  [B, mem_len, D]  memory in logical order (oldest first); may be NULL if mem_len == 0
 *   W_q, W_kE, W_v, W_kR  [H*d, D];  W_o [D, H*d];  gamma, beta [D];  u, vb [H, d]
 *   R    [>= T, D]        row p is the encoding of distance p
 *   h_out [B, L, D]
 *   q_o, k_o, v_o, r_o, a_o: NULL, or receive q [B,L,H,d], k/v [B,T,H,d], r [T,H,d], a [B,L,H,d]
 */
int txo_layer_step(int64_t B, int64_t L, int64_t D, int64_t H, int64_t d,
                   int64_t mem_len, double eps, const double* h, const double* mem,
                   const double* W_q, const double* W_kE, const double* W_v,
                   const double* W_kR, const double* W_o, const double* gamma,
                   const double* beta, const double* u, const double* vb,
                   const double* R, double* h_out, double* q_o, double* k_o,
                   double* v_o, double* r_o, double* a_o) {
    const int64_t T = mem_len + L, HD = H * d;
    double* ctx = (double*)malloc(sizeof(double) * (size_t)(B * T * D));
    double* q = (double*)malloc(sizeof(double) * (size_t)(B * L * HD));
    double* k = (double*)malloc(sizeof(double) * (size_t)(B * T * HD));
    double* v = (double*)malloc(sizeof(double) * (size_t)(B * T * HD));
    double* r = (double*)malloc(sizeof(double) * (size_t)(T * HD));
    double* a = (double*)malloc(sizeof(double) * (size_t)(B * L * HD));
    double* y = (double*)malloc(sizeof(double) * (size_t)(B * L * D));
    if (!ctx || !q || !k || !v || !r || !a || !y) {
        free(ctx); free(q); free(k); free(v); free(r); free(a); free(y);
        return -1;
    }
    /* the extended context: memory rows, then the current rows */
    for (int64_t b = 0; b < B; ++b) {
        if (mem_len > 0)
            memcpy(ctx + b * T * D, mem + b * mem_len * D, sizeof(double) * (size_t)(mem_len * D));
        memcpy(ctx + (b * T + mem_len) * D, h + b * L * D, sizeof(double) * (size_t)(L * D));
    }
    txo_linear(B * L, HD, D, h, W_q, q);
    txo_linear(B * T, HD, D, ctx, W_kE, k);
    txo_linear(B * T, HD, D, ctx, W_v, v);
    txo_linear(T, HD, D, R, W_kR, r);
    txo_rel_attn(B, H, L, mem_len, d, q, k, v, r, u, vb, 1.0 / sqrt((double)d), a, NULL);
    txo_linear(B * L, D, HD, a, W_o, y);
    for (int64_t m = 0; m < B * L * D; ++m) y[m] += h[m];
    txo_layer_norm(B * L, D, y, gamma, beta, eps, h_out);
    if (q_o) memcpy(q_o, q, sizeof(double) * (size_t)(B * L * HD));
    if (k_o) memcpy(k_o, k, sizeof(double) * (size_t)(B * T * HD));
    if (v_o) memcpy(v_o, v, sizeof(double) * (size_t)(B * T * HD));
    if (r_o) memcpy(r_o, r, sizeof(double) * (size_t)(T * HD));
    if (a_o) memcpy(a_o, a, sizeof(double) * (size_t)(B * L * HD));
    free(ctx); free(q); free(k); free(v); free(r); free(a); free(y);
    return 0;
}

/*
 * The same layer step, evaluated only at n sampled output rows (b_s[t], i_s[t]):
 * keys and values are projected for the whole context of each sampled batch
 * row, the query, attention, output projection and LayerNorm only for the
 * sampled rows.  Same arithmetic as txo_layer_step, cheaper at full size.
 *   h_out_rows [n, D]
 */
int txo_layer_step_rows(int64_t B, int64_t L, int64_t D, int64_t H, int64_t d,
                        int64_t mem_len, double eps, const double* h, const double* mem,
                        const double* W_q, const double* W_kE, const double* W_v,
                        const double* W_kR, const double* W_o, const double* gamma,
                        const double* beta, const double* u, const double* vb,
                        const double* R, int64_t n, const int64_t* b_s,
                        const int64_t* i_s, double* h_out_rows) {
    const int64_t T = mem_len + L, HD = H * d;
    (void)B;
    double* ctx = (double*)malloc(sizeof(double) * (size_t)(T * D));
    double* k = (double*)malloc(sizeof(double) * (size_t)(T * HD));
    double* v = (double*)malloc(sizeof(double) * (size_t)(T * HD));
    double* r = (double*)malloc(sizeof(double) * (size_t)(T * HD));
    double* q = (double*)malloc(sizeof(double) * (size_t)HD);
    double* a = (double*)malloc(sizeof(double) * (size_t)HD);
    double* y = (double*)malloc(sizeof(double) * (size_t)D);
    if (!ctx || !k || !v || !r || !q || !a || !y) {
        free(ctx); free(k); free(v); free(r); free(q); free(a); free(y);
        return -1;
    }
    txo_linear(T, HD, D, R, W_kR, r);
    int64_t cur_b = -1;
    for (int64_t t = 0; t < n; ++t) {
        const int64_t b = b_s[t], i = i_s[t];
        if (b != cur_b) {
            if (mem_len > 0)
                memcpy(ctx, mem + b * mem_len * D, sizeof(double) * (size_t)(mem_len * D));
            memcpy(ctx + mem_len * D, h + b * L * D, sizeof(double) * (size_t)(L * D));
            txo_linear(T, HD, D, ctx, W_kE, k);
            txo_linear(T, HD, D, ctx, W_v, v);
            cur_b = b;
        }
        const double* hi = h + (b * L + i) * D;
        txo_linear(1, HD, D, hi, W_q, q);
        /* attention of this one query: a 1-row problem whose memory is the
         * first mem_len+i rows of the context, i.e. query 0 at mem_len' = mem_len+i */
        const int64_t ml = mem_len + i;
        txo_rel_attn(1, H, 1, ml, d, q, k, v, r, u, vb, 1.0 / sqrt((double)d), a, NULL);
        txo_linear(1, D, HD, a, W_o, y);
        for (int64_t c = 0; c < D; ++c) y[c] += hi[c];
        layer_norm_row(D, y, gamma, beta, eps, h_out_rows + t * D);
    }
    free(ctx); free(k); free(v); free(r); free(q); free(a); free(y);
    return 0;
}

/*
 * Memory update (section 3.2: cache a predefined number M of old hidden
 * states, possibly spanning several segments).  The new memory is the last
 * min(M, mem_len+L) rows of [mem ; h], in logical order.
 *   mem [B, mem_len, D], h [B, L, D], mem_out [B, M, D] (rows past the new length untouched)
 * Returns the new length.
 */
int64_t txo_mem_update(int64_t B, int64_t M, int64_t D, const double* mem,
                       int64_t mem_len, const double* h, int64_t L, double* mem_out) {
    const int64_t T = mem_len + L;
    const int64_t new_len = T < M ? T : M;
    const int64_t first = T - new_len; /* logical index in [mem ; h] of the oldest kept row */
    for (int64_t b = 0; b < B; ++b)
        for (int64_t t = 0; t < new_len; ++t) {
            const int64_t x = first + t;
            const double* src = x < mem_len ? mem + (b * mem_len + x) * D
                                            : h + (b * L + (x - mem_len)) * D;
            memcpy(mem_out + (b * M + t) * D, src, sizeof(double) * (size_t)D);
        }
    return new_len;
}
