/*
 * txl.h -- C ABI of libtxl.so: Transformer-XL relative-position attention over
 * segment-level memory (forward), the layer step that feeds it, and the memory
 * update, for AMD Instinct MI355X (gfx950).
 *
 * Source of every operation: Dai et al., "Transformer-XL: Attentive Language
 * Models Beyond a Fixed-Length Context" (arXiv 1901.02860v3), section 3.2
 * (segment-level recurrence with a length-M memory), section 3.3 (relative
 * positional encodings: the score A^rel with terms (a)-(d), the biases u and v,
 * separate W_{k,E} and W_{k,R}, and the N-layer computational procedure), and
 * Appendix B (distances range over 0 .. M+L-1).
 *
 * Conventions shared by every entry point
 *   - All tensors are device pointers (hipMalloc'd or torch-allocated memory).
 *     The library allocates no device memory; scratch comes from the caller's
 *     workspace argument (txl_rel_attn_fwd_noalloc alone uses a fixed static
 *     device array instead).
 *   - Strides are in ELEMENTS.  Element types: TXL_FP32 = float,
 *     TXL_BF16 = bfloat16 (stored as 16-bit words).  One call uses one dtype for
 *     all of its tensor arguments (scores_dbg is always float).
 *   - All work is enqueued on `stream` (a hipStream_t; NULL = the null stream).
 *     No entry point synchronises; the caller owns ordering and lifetime.
 *   - Every argument is validated before anything is enqueued, so a call that
 *     returns an error has written nothing.  No C++ exception crosses the ABI.
 *   - Weights are stored [out, in] row-major: y = x W^T, as the pages write
 *     projections (h W^T).
 */
#ifndef TXL_H
#define TXL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  TXL_OK = 0,
  TXL_EINVAL = -1,        /* null pointer, non-positive size, bad stride, aliasing  */
  TXL_EUNSUPPORTED = -2,  /* valid but not supported: dtype, d_head > 128           */
  TXL_EHIP = -3,          /* a HIP runtime call or kernel launch failed             */
  TXL_EWORKSPACE = -4     /* workspace smaller than txl_layer_workspace_bytes()     */
} txl_status;

typedef enum { TXL_FP32 = 0, TXL_BF16 = 1 } txl_dtype;

/*
 * Relative-position attention, forward (section 3.3, the A^rel equation and the
 * masked softmax of the N-layer procedure).  For batch row b, head h, query
 * i in [0, L) and key j in [0, T), T = mem_len + L (keys 0 .. mem_len-1 are the
 * memory, oldest first; keys mem_len .. T-1 are the current segment):
 *
 *   key j is visible to query i  iff  j <= mem_len + i      (the query sees itself)
 *   p = mem_len + i - j                                      (relative distance)
 *   A[i][j] = scale * ( (q_i + u_h) . k_j  +  (q_i + v_h) . r_p )
 *           = scale * ( (a) + (c) + (b) + (d) )
 *   out_i   = sum_j softmax_j(A[i][.]) v_j
 *
 * Arguments
 *   stream            hipStream_t to enqueue on.
 *   dtype             TXL_FP32 or TXL_BF16 (bf16 inputs: fp32 accumulation and
 *                     fp32 softmax state; output rounded to bf16).
 *   B, H, L           batch, heads, segment length (queries per batch row), >= 1.
 *   mem_len           valid memory rows, >= 0.
 *   d_head            head size, 1 .. 128.
 *   q                 q[b][i][h][c]  at q + b*q_sb + i*q_st + h*q_sh + c.
 *   k, v              k[b][j][h][c]  at k + b*kv_sb + j*kv_st + h*kv_sh + c
 *                     (v uses the same strides), j in [0, T).
 *   r                 r[p][h][c]     at r + p*r_sp + h*r_sh + c, p in [0, r_rows);
 *                     row p is W_{k,R} R_p, the projected encoding of distance p.
 *                     r_rows must be >= T.
 *   u_bias, v_bias    [H][d_head] dense: the global content bias u and the
 *                     global position bias v of section 3.3.
 *   scale             multiplies the whole four-term score (1/sqrt(d_head) is
 *                     the usual choice).
 *   out               out[b][i][h][c] at out + b*o_sb + i*o_st + h*o_sh + c.
 *                     Must not overlap any input.
 *   scores_dbg        NULL, or float [B][H][L][T] dense: receives A (scaled), with
 *                     -INFINITY where masked.  Debug only; it slows the call.
 *   workspace, ws_bytes  NULL/0, or device scratch of at least
 *                     txl_rel_attn_workspace_bytes() bytes (it must not overlap
 *                     any tensor argument).  When the query tiles alone would
 *                     leave the GPU unevenly loaded (few batch rows and heads,
 *                     short segments over a long memory), the matrix-core path
 *                     splits the keys of some query tiles among several
 *                     workgroups, keeps their partial softmax states (and
 *                     arrival counters) here and merges them with a
 *                     log-sum-exp.  With less workspace it takes the best split
 *                     that fits, or none; the result is the same up to
 *                     rounding.  Calls that share a workspace must not overlap.
 *
 * Layouts: any strides with the innermost (c) dimension contiguous are
 * accepted.  bf16 calls whose q/k/v/r base pointers are 16-byte aligned and
 * whose q/k/v/r strides are multiples of 8 take the matrix-core path (d_head
 * <= 64); other layouts take a generic path.  This is never an error.
 * Returns TXL_OK or a txl_status.
 */
int txl_rel_attn_fwd(void* stream, int dtype,
                     int64_t B, int64_t H, int64_t L, int64_t mem_len, int64_t d_head,
                     const void* q, int64_t q_sb, int64_t q_st, int64_t q_sh,
                     const void* k, const void* v, int64_t kv_sb, int64_t kv_st, int64_t kv_sh,
                     const void* r, int64_t r_sp, int64_t r_sh, int64_t r_rows,
                     const void* u_bias, const void* v_bias, float scale,
                     void* out, int64_t o_sb, int64_t o_st, int64_t o_sh,
                     float* scores_dbg, void* workspace, size_t ws_bytes);

/*
 * Scratch bytes txl_rel_attn_fwd can use for a key split at these sizes on the
 * current device (0: it would not split).  Returns 0 for invalid arguments too.
 */
size_t txl_rel_attn_workspace_bytes(int dtype, int64_t B, int64_t H, int64_t L,
                                    int64_t mem_len, int64_t d_head);

/*
 * txl_rel_attn_fwd for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same computation, arguments, layouts and results, without the workspace.
 * The key-split partials go to the library's static device scratch instead, a
 * file-scope array of txl_rel_attn_noalloc_max_scratch_bytes() bytes (16 MiB)
 * that every device the library runs on holds from the library's load until the
 * process ends.  The call allocates nothing and calls no allocating routine.
 *   - A shape whose split plan needs more scratch than that returns
 *     TXL_EWORKSPACE (txl_rel_attn_workspace_bytes() gives the need) and
 *     writes nothing; use txl_rel_attn_fwd with a workspace there.
 *   - Nothing in the scratch needs to start at zero: every partial is written
 *     before the same call reads it; the last call's contents stay behind.
 *   - All calls on one GPU share that GPU's scratch: calls that may overlap in
 *     time on one GPU (several streams, several host threads) race and must be
 *     ordered by the caller.
 * Returns TXL_OK or a txl_status.
 */
int txl_rel_attn_fwd_noalloc(void* stream, int dtype,
                             int64_t B, int64_t H, int64_t L, int64_t mem_len, int64_t d_head,
                             const void* q, int64_t q_sb, int64_t q_st, int64_t q_sh,
                             const void* k, const void* v, int64_t kv_sb, int64_t kv_st,
                             int64_t kv_sh, const void* r, int64_t r_sp, int64_t r_sh,
                             int64_t r_rows, const void* u_bias, const void* v_bias, float scale,
                             void* out, int64_t o_sb, int64_t o_st, int64_t o_sh,
                             float* scores_dbg);

/* Bytes of the static scratch txl_rel_attn_fwd_noalloc uses (its maximum). */
size_t txl_rel_attn_noalloc_max_scratch_bytes(void);

/*
 * Backward pass of txl_rel_attn_fwd (training with a stop-gradient memory:
 * Transformer-XL section 3.2 stops the gradient at the cached memory, so the
 * keys and values of the memory rows still get gradients here, but nothing
 * below them does; section 3.3 defines the score whose chain rule this is).
 * With P the attention weights, dP_ij = dout_i . v_j and
 * dS_ij = P_ij (dP_ij - sum_j' P_ij' dP_ij'):
 *   dq_i = scale sum_j dS_ij (k_j + r_{mem_len+i-j})
 *   dk_j = scale sum_i dS_ij (q_i + u),   dv_j = sum_i P_ij dout_i
 *   dr_p = scale sum of dS_ij (q_i + v) over the pairs at distance p
 *   du   = scale sum_ij dS_ij k_j,        dv_bias = scale sum_ij dS_ij r_{mem_len+i-j}
 *
 * Arguments as in txl_rel_attn_fwd (same layouts and strides for q, k, v, r,
 * u_bias, v_bias and scale; dout takes out's place and layout), d_head <= 64
 * (else TXL_EUNSUPPORTED).  The forward's output is not needed: the softmax
 * statistics are recomputed.  Gradients are fp32, dense and written whole:
 *   dq [B][L][H][d]  dk, dv [B][T][H][d]  dr [T][H][d]  du, dvb [H][d]
 * Precision: fp32 inputs are differentiated in fp32 throughout; bf16 inputs on
 * the bf16 matrix cores with fp32 sums, where P, dS, dout, q + u and q + v
 * enter the products rounded to bf16 (as P enters the forward's P V).
 * workspace (required): device scratch of txl_rel_attn_bwd_workspace_bytes()
 * bytes; it holds P and dS [B][H][L][T] (fp32, or bf16 for bf16 inputs).
 * Gradients, workspace and inputs must not overlap.  Returns TXL_OK or a
 * txl_status.
 */
int txl_rel_attn_bwd(void* stream, int dtype,
                     int64_t B, int64_t H, int64_t L, int64_t mem_len, int64_t d_head,
                     const void* q, int64_t q_sb, int64_t q_st, int64_t q_sh,
                     const void* k, const void* v, int64_t kv_sb, int64_t kv_st, int64_t kv_sh,
                     const void* r, int64_t r_sp, int64_t r_sh, int64_t r_rows,
                     const void* u_bias, const void* v_bias, float scale,
                     const void* dout, int64_t do_sb, int64_t do_st, int64_t do_sh,
                     float* dq, float* dk, float* dv, float* dr, float* du, float* dvb,
                     void* workspace, size_t ws_bytes);

/* Scratch bytes txl_rel_attn_bwd needs at these sizes (0 for invalid or
 * unsupported arguments). */
size_t txl_rel_attn_bwd_workspace_bytes(int dtype, int64_t B, int64_t H, int64_t L,
                                        int64_t mem_len, int64_t d_head);

/*
 * The memory of one layer (section 3.2: a length-M cache of old hidden states
 * that may span several segments), stored as a ring so that an update never
 * moves the rows it keeps.
 *   data      device [B][capacity][d_model], row pitch d_model elements.
 *   capacity  M >= 1.
 *   start     physical slot of logical row 0 (the oldest), 0 <= start < M.
 *   len       valid rows, 0 <= len <= M (0 = empty memory).
 * Logical row t (0 = oldest) of batch row b lives at data[b][(start + t) % M].
 */
typedef struct {
  void* data;
  int64_t capacity;
  int64_t start;
  int64_t len;
} txl_ring;

typedef struct {
  int64_t B;        /* batch                               */
  int64_t L;        /* segment length                      */
  int64_t d_model;  /* hidden size D                       */
  int64_t n_head;   /* H                                   */
  int64_t d_head;   /* d, 1 .. 128                         */
  float ln_eps;     /* LayerNorm epsilon (e.g. 1e-5)       */
} txl_layer_dims;

typedef struct {
  const void* W_q;       /* [H*d, D]  query projection                      */
  const void* W_kE;      /* [H*d, D]  content-key projection W_{k,E}         */
  const void* W_v;       /* [H*d, D]  value projection                      */
  const void* W_kR;      /* [H*d, D]  position-key projection W_{k,R}        */
  const void* W_o;       /* [D, H*d]  output projection ("Linear")           */
  const void* ln_gamma;  /* [D]       LayerNorm scale                        */
  const void* ln_beta;   /* [D]       LayerNorm shift                        */
} txl_layer_weights;

/*
 * Bytes of workspace txl_layer_step needs for these dims with a memory of
 * capacity mem_capacity (it covers every mem->len <= mem_capacity).
 * Returns 0 if the arguments are invalid.
 */
size_t txl_layer_workspace_bytes(const txl_layer_dims* dims, int64_t mem_capacity, int dtype);

/*
 * One Transformer-XL layer for one segment (section 3.3, the N-layer procedure,
 * without the position-wise feed-forward; section 3.2 for the context):
 *
 *   ctx   = [ memory (mem->len rows, oldest first) ; h_in (L rows) ]   per batch row
 *   q     = h_in W_q^T             k = ctx W_kE^T        v = ctx W_v^T
 *   r     = R[0 : mem->len + L] W_kR^T        (row p <-> distance p)
 *   a     = txl_rel_attn_fwd(q, k, v, r, u, v_bias, scale = 1/sqrt(d_head))
 *   h_out = LayerNorm(a W_o^T + h_in) * gamma + beta   (biased variance over D)
 *
 *   h_in      [B][L][D] dense, the layer input of the current segment.
 *   mem       the layer's memory, read only (the ring is gathered in place,
 *             never copied).  mem->data must have d_model columns.
 *   w         this layer's weights.
 *   u_bias, v_bias  [H][d] dense.
 *   R         [R_rows][D] dense, row p the encoding of distance p; R_rows >= mem->len + L.
 *   h_out     [B][L][D] dense; must not alias h_in or the memory.
 *   workspace device scratch of ws_bytes >= txl_layer_workspace_bytes(dims,
 *             mem->capacity, dtype), 256-byte aligned.  Holds q, k, v, r, a and
 *             the pre-LayerNorm sum between the kernels of this call.
 *
 * To advance the recurrence the caller then appends h_in (the layer INPUT,
 * which is what this layer reads at the next segment) with txl_mem_update on
 * the same stream.
 */
int txl_layer_step(void* stream, int dtype, const txl_layer_dims* dims,
                   const void* h_in, const txl_ring* mem, const txl_layer_weights* w,
                   const void* u_bias, const void* v_bias,
                   const void* R, int64_t R_rows, void* h_out,
                   void* workspace, size_t ws_bytes);

/*
 * Gradients of one layer step (fp32, dense), see txl_layer_step_bwd.
 */
typedef struct {
  float* dh;        /* [B][L][D]  gradient of h_in (current rows; the memory gets none) */
  float* dW_q;      /* [H*d][D]                                                        */
  float* dW_kE;     /* [H*d][D]   over the memory rows and the current rows             */
  float* dW_v;      /* [H*d][D]                                                        */
  float* dW_kR;     /* [H*d][D]                                                        */
  float* dW_o;      /* [D][H*d]                                                        */
  float* du;        /* [H][d]     content bias u                                       */
  float* dv_bias;   /* [H][d]     position bias v                                      */
  float* dgamma;    /* [D]                                                             */
  float* dbeta;     /* [D]                                                             */
} txl_layer_grads;

/* Bytes of workspace txl_layer_step_bwd needs (memory capacity mem_capacity);
 * 0 for invalid or unsupported arguments. */
size_t txl_layer_bwd_workspace_bytes(const txl_layer_dims* dims, int64_t mem_capacity, int dtype);

/*
 * Backward pass of txl_layer_step for the upstream gradient dh_out [B][L][D]
 * (same dtype as h_in): the training step with a stop-gradient memory of
 * Transformer-XL section 3.2 (the cached hidden states get no gradient, while
 * the weights collect the memory rows' contributions through k and v) over the
 * procedure of section 3.3 (projections, relative attention, output projection,
 * residual, LayerNorm with biased variance).  All arguments but dh_out, g and
 * the workspace are txl_layer_step's (same meaning and checks); d_head <= 64.
 * The call recomputes the forward in its workspace, then:
 *   dy  = LayerNorm backward of dh_out          (also dgamma, dbeta)
 *   dW_o = dy^T a,   da = dy W_o,   (dq, dk, dv, dr, du, dv_bias) = txl_rel_attn_bwd(da)
 *   dW_q = dq^T h_in,  dW_kE = dk^T ctx,  dW_v = dv^T ctx,  dW_kR = dr^T R[0:T]
 *   dh  = dy + dq W_q + (dk W_kE + dv W_v) restricted to the current rows
 * with ctx = [memory ; h_in].  Every gradient is written whole (not accumulated).
 * bf16 layers run every product on the bf16 matrix cores (operands rounded to
 * bf16, fp32 sums) and take the attention's softmax statistics from the
 * recomputed forward; fp32 layers stay in fp32 throughout.
 *   g          gradient pointers (all required; they must not overlap each other,
 *              the inputs or the workspace).
 *   workspace  device scratch of ws_bytes >= txl_layer_bwd_workspace_bytes(dims,
 *              mem->capacity, dtype), 256-byte aligned.
 * Returns TXL_OK or a txl_status.
 */
int txl_layer_step_bwd(void* stream, int dtype, const txl_layer_dims* dims,
                       const void* h_in, const txl_ring* mem, const txl_layer_weights* w,
                       const void* u_bias, const void* v_bias, const void* R, int64_t R_rows,
                       const void* dh_out, const txl_layer_grads* g,
                       void* workspace, size_t ws_bytes);

/*
 * Training without the forward recompute.  txl_layer_step_save is
 * txl_layer_step that keeps, in caller-owned device memory, what
 * txl_layer_step_bwd would otherwise recompute (q, k, v, r, the attention output
 * and, where the forward has them, its softmax statistics and LayerNorm input);
 * txl_layer_step_bwd_saved is txl_layer_step_bwd that takes them from there.
 * The arguments of the two calls must be the same (and the memory unchanged in
 * between), as in a training step: forward through the stack, then backward;
 * the backward checks the memory, h_in, dims and dtype against the save.
 *   saved->data   device memory of saved->bytes >= txl_layer_saved_bytes(dims,
 *                 mem->capacity, dtype), 256-byte aligned, not overlapping any
 *                 other argument; owned by the caller, alive until the backward.
 *   saved->has_lse, saved->has_y   written by txl_layer_step_save (host side),
 *                 read by txl_layer_step_bwd_saved.
 * The backward's workspace and results are txl_layer_step_bwd's.  Returns TXL_OK
 * or a txl_status.
 */
typedef struct {
  void*  data;
  size_t bytes;
  int    has_lse;  /* the softmax statistics are in data */
  int    has_y;    /* the fp32 LayerNorm input is in data */
  /* Written by txl_layer_step_save: the call the state belongs to.  The backward
   * re-gathers the context [memory ; h_in] from the ring, so it returns
   * TXL_EINVAL, writing nothing, when the ring (data, capacity, start, len),
   * h_in, the dims or the dtype differ -- e.g. after a txl_mem_update of that
   * ring between the two calls. */
  const void* mem_data;
  int64_t mem_capacity, mem_start, mem_len;
  const void* h_in;
  int64_t B, L, d_model, n_head, d_head;
  int     dtype;
} txl_layer_saved;

size_t txl_layer_saved_bytes(const txl_layer_dims* dims, int64_t mem_capacity, int dtype);
int txl_layer_step_save(void* stream, int dtype, const txl_layer_dims* dims, const void* h_in,
                        const txl_ring* mem, const txl_layer_weights* w, const void* u_bias,
                        const void* v_bias, const void* R, int64_t R_rows, void* h_out,
                        txl_layer_saved* saved);
int txl_layer_step_bwd_saved(void* stream, int dtype, const txl_layer_dims* dims,
                             const void* h_in, const txl_ring* mem, const txl_layer_weights* w,
                             const void* u_bias, const void* v_bias, const void* R,
                             int64_t R_rows, const void* dh_out, const txl_layer_saved* saved,
                             const txl_layer_grads* g, void* workspace, size_t ws_bytes);

/*
 * Where txl_layer_step leaves its intermediates in the workspace (section 3.3's
 * q, k, v, the projected encodings r = R W_kR^T, and the attention output a),
 * for a call with mem->len == mem_len.  After such a call the workspace holds,
 * at the returned byte offsets (T = mem_len + L, d_pad = row pitch):
 *   q [B][H][L][d_pad]   k, v [B][H][T][d_pad]   r [H][T][d_pad]   a [B][L][H*d]
 * in the call's dtype; columns d .. d_pad-1 of q, k, v, r rows are unspecified.
 * Returns TXL_OK, or TXL_EINVAL / TXL_EUNSUPPORTED for bad dims or dtype.
 */
typedef struct {
  size_t q, k, v, r, a;  /* byte offsets into the workspace          */
  int64_t d_pad;         /* row pitch in elements of q, k, v, r rows */
} txl_workspace_map;

int txl_layer_workspace_map(const txl_layer_dims* dims, int64_t mem_len, int dtype,
                            txl_workspace_map* map);

/*
 * Memory update (section 3.2): the memory becomes the last min(M, len + L)
 * rows of [memory ; h_new].  Only the newest min(L, M) rows of h_new are
 * copied (into the ring slots that follow the current content); rows that stay
 * are not moved.  mem->start and mem->len are updated on the host before the
 * call returns; the copy is enqueued on `stream`.
 *   h_new  [B][L][d_model] dense, same dtype as the ring.
 */
int txl_mem_update(void* stream, int dtype, txl_ring* mem, int64_t B, int64_t d_model,
                   const void* h_new, int64_t L);

/*
 * An n_layers stack run over n_segments consecutive segments, forward (the
 * recurrence of section 3.2 over the N-layer procedure of section 3.3; the
 * layer is txl_layer_step, the memory update txl_mem_update):
 *
 *   for s in 0 .. n_segments-1:
 *     h = h_in[s]
 *     for n in 0 .. n_layers-1:
 *       y = txl_layer_step(h, mem[n], w[n]);  txl_mem_update(mem[n], h);  h = y
 *     h_out[s] = h
 *
 * Layer n of segment s reads two things: the output of layer n-1 of segment s
 * and ring n as segment s-1 left it.  So layer n of segment s+1 and layer n+1 of
 * segment s do not depend on each other, and with more than one stream the
 * segments go round the streams (segment s on streams[s % n_streams]), each
 * layer step of segment s waiting for the memory update of the same layer in
 * segment s-1 (an event on the previous segment's stream): segment s+1 runs one
 * layer behind segment s, and the two overlap.  Every kernel reads and writes
 * what it would in the serial order above, so the results are bit-identical to
 * it for any n_streams.
 *   streams    n_streams (1 .. TXL_STACK_MAX_STREAMS) HIP streams; NULL entries
 *              are the default stream, repeats are allowed (they serialise).
 *              Streams 1.. first wait for the work already on streams[0], and
 *              streams[0] waits for their last work before the call returns, so
 *              ordering later work after streams[0] covers the whole stack.
 *   h_in       [n_segments][B][L][d_model] dense, the first layer's inputs.
 *   mem        n_layers rings (capacity, start and len each their own), updated
 *              in place, n_segments times each, as txl_mem_update does.
 *   w          n_layers layer weights;  u_bias, v_bias, R as in txl_layer_step,
 *              R_rows covering each layer's longest memory + L.
 *   h_out      [n_segments][B][L][d_model] dense, the last layer's outputs; must
 *              not overlap h_in, the rings or the workspace.
 *   workspace  >= txl_stack_workspace_bytes(dims, largest ring capacity, dtype,
 *              n_streams) bytes, 256-byte aligned: per stream one layer
 *              workspace and two [B][L][d_model] buffers for the layer outputs.
 * Every argument is checked before anything is enqueued (a failing call writes
 * nothing and leaves the rings as they were).  Returns TXL_OK or a txl_status.
 */
#define TXL_STACK_MAX_STREAMS 8
int txl_stack_fwd(void* const* streams, int n_streams, int dtype, const txl_layer_dims* dims,
                  int64_t n_layers, int64_t n_segments, const void* h_in, txl_ring* mem,
                  const txl_layer_weights* w, const void* u_bias, const void* v_bias,
                  const void* R, int64_t R_rows, void* h_out, void* workspace,
                  size_t ws_bytes);

/* Workspace bytes of txl_stack_fwd (0 for invalid dims, dtype or n_streams). */
size_t txl_stack_workspace_bytes(const txl_layer_dims* dims, int64_t mem_capacity, int dtype,
                                 int n_streams);

/*
 * ---- Evaluation with cached keys and values ---------------------------------------------
 * At evaluation the weights are fixed, so the projected keys and values of a
 * memory row (section 3.2's cached hidden states, projected by W_kE and W_v as in
 * section 3.3) and the projected encodings r = R W_kR^T do not change once
 * computed.  This path keeps the projected k and v of the memory rows in a ring
 * per layer and projects only the L new rows of each segment; r is projected
 * once (txl_pos_proj).  The result equals txl_layer_step over the hidden-state
 * memory up to rounding.  L = 1 is the per-token (decode) shape.
 *
 * A layer's key/value ring:
 *   k, v       device [B][H][capacity][d_pad] each, d_pad = d_head rounded up to 8;
 *              txl_kv_ring_bytes() bytes each.  Memory row t (0 = oldest) of batch
 *              row b, head h sits at row (start + t) % capacity.  Contents need no
 *              initialisation (rows are written before they are read).
 *   capacity   >= mem_max + L of every call (the new rows are appended behind the
 *              memory before the oldest ones are dropped).
 *   start      0 <= start < capacity.
 *   len        memory rows, 0 <= len <= mem_max (0 = empty memory).
 *   mem_max    M: after a step the memory keeps the newest min(M, len + L) rows.
 */
typedef struct {
  void* k;
  void* v;
  int64_t capacity;
  int64_t start;
  int64_t len;
  int64_t mem_max;
} txl_kv_ring;

/* Bytes of one of k, v of a ring of this capacity (0 for invalid arguments). */
size_t txl_kv_ring_bytes(const txl_layer_dims* dims, int64_t capacity, int dtype);

/*
 * r = R[0 : R_rows] W_kR^T (section 3.3's W_{k,R} R_{i-j}; row p <-> distance p)
 * into r_out [H][R_rows][d_pad] (padding columns written as zeros), dims->d_model
 * columns of R and of W_kR.  Enqueued on `stream`.  r_out must not overlap R or
 * W_kR.
 */
int txl_pos_proj(void* stream, int dtype, const txl_layer_dims* dims, const void* R,
                 int64_t R_rows, const void* W_kR, void* r_out);

/* Workspace bytes of txl_layer_step_kv for rings of this mem_max (0 if invalid). */
size_t txl_layer_kv_workspace_bytes(const txl_layer_dims* dims, int64_t mem_max, int dtype);

/*
 * One layer for one segment with cached keys and values:
 *   k, v of the L rows of h_in are projected into the ring behind its len memory
 *   rows; q = h_in W_q^T; a = attention of q over the len + L keys (relative
 *   distances through r); h_out = LayerNorm(a W_o^T + h_in) * gamma + beta.
 *   Then the ring keeps the newest min(mem_max, len + L) rows: kv->start and
 *   kv->len are updated on the host before the call returns (no data moves).
 *   h_in     [B][L][D] dense.      h_out  [B][L][D] dense, must not alias h_in.
 *   kv       this layer's ring (see above); w->W_kR is not used.
 *   r        txl_pos_proj output [H][r_rows][d_pad]; r_rows >= kv->len + L.
 *   workspace  >= txl_layer_kv_workspace_bytes(dims, kv->mem_max, dtype) bytes,
 *            256-byte aligned.
 * Errors as txl_layer_step; a failing call changes nothing.  Calls that share a
 * ring or a workspace must be ordered (one stream).
 */
int txl_layer_step_kv(void* stream, int dtype, const txl_layer_dims* dims, const void* h_in,
                      txl_kv_ring* kv, const txl_layer_weights* w, const void* u_bias,
                      const void* v_bias, const void* r, int64_t r_rows, void* h_out,
                      void* workspace, size_t ws_bytes);

/*
 * Position-wise feed-forward of the N-layer procedure (section 3.3: after the
 * attention sublayer, h = Positionwise-Feed-Forward(o); the pages leave its
 * inside open).  Read as the two-layer ReLU network with biases and a post-norm
 * residual, per row:
 *   out = LayerNorm(x + relu(x W1^T + b1) W2^T + b2) * gamma + beta   (biased variance)
 *   x, out   [rows][d_model] dense (out must not overlap any input)
 *   W1 [d_inner][d_model], b1 [d_inner], W2 [d_model][d_inner], b2, ln_gamma, ln_beta [d_model]
 *   workspace  >= txl_pos_ff_workspace_bytes() bytes, 256-byte aligned (holds the
 *            hidden activations).
 * A layer of the full stack is txl_layer_step (or txl_layer_step_kv) followed by
 * this on its output; the memory still caches the layer INPUT.
 */
size_t txl_pos_ff_workspace_bytes(int64_t rows, int64_t d_model, int64_t d_inner, int dtype);
int txl_pos_ff(void* stream, int dtype, int64_t rows, int64_t d_model, int64_t d_inner,
               const void* x, const void* W1, const void* b1, const void* W2, const void* b2,
               const void* ln_gamma, const void* ln_beta, float ln_eps, void* out,
               void* workspace, size_t ws_bytes);

/* Static text for a status, followed by the calling thread's detail of its last error. */
/*
 * Which bf16 matrix-core attention kernel txl_rel_attn_fwd and the layer steps
 * run (process-wide; the result is the same to rounding, the speed differs):
 *   0  by shape (the default): the 128-query kernel where its tiles fill at
 *      least two per CU and the last query tile has 16 or more 64-key tiles;
 *      else the 64-query kernel (three 4-wave workgroups per CU, no key split)
 *      where the shape has at least two of its 64-query tiles per CU; else the
 *      128-query kernel with its planned key splits;
 *   1  the 64-query kernel wherever the matrix-core path applies;
 *   2  the 128-query kernel with its planned key splits.
 * For tests and tuning.  Workspace sizes follow the setting in force when they
 * are asked for; a call whose workspace cannot hold the planned key-split
 * partials runs with fewer parts.  Returns the previous setting, or TXL_EINVAL.
 * Not synchronised with calls running on other host threads.
 */
int txl_attn_variant(int variant);

/*
 * Which kernel txl_rel_attn_fwd runs at these sizes, for dense head rows of
 * d_head elements in an aligned layout (the workspace of txl_layer_step, or
 * 16-byte aligned rows whose pitches are multiples of 8): one of
 * txl_attn_kernel_kind under the txl_attn_variant setting in force, or
 * TXL_EINVAL.
 */
typedef enum {
  TXL_ATTN_VECTOR = 0,       /* vector-unit kernel (fp32, or rows the matrix cores do not take) */
  TXL_ATTN_ONE_QUERY = 1,    /* single-query kernel with its key-part merge (L = 1)            */
  TXL_ATTN_Q128 = 2,         /* matrix cores, 128-query workgroups                              */
  TXL_ATTN_Q128_SPLIT = 3,   /* the same with the key axis split and a merge kernel             */
  TXL_ATTN_Q64 = 4           /* matrix cores, 64-query workgroups, three per CU                 */
} txl_attn_kernel_kind;
int txl_attn_kernel(int dtype, int64_t B, int64_t H, int64_t L, int64_t mem_len, int64_t d_head);

const char* txl_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* TXL_H */
