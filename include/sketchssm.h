/*
 * sketchssm.h -- C ABI of libsketchssm.so: the SketchSSM windowed
 * linear-attention decode path on AMD Instinct MI355X (gfx950).
 *
 * Method (SketchSSM pages: readsearch.ai listing of arXiv 2609.33051,
 * "SketchSSM: Write to the Full State, Read from a Compact Sketch", Abstract;
 * agihunt.info summary, "Confirmed" bullets "Mechanism details" and
 * "Error control"):
 *   - keys, values and gates of the current window are buffered and the full
 *     recurrent state S (d_k x d_v, fp32, one per (sequence, head) unit) is
 *     written once per window;
 *   - the same pass that writes S also stores a compact sketch: the outputs of
 *     S for r fixed, offline basis vectors b_1..b_r;
 *   - every decode step in between reads only the sketch and the buffer and
 *     rebuilds the output from query-dependent coefficients; the sketch's
 *     approximation error never reaches S.
 *
 * Notation (per unit). Token i of the window has key k_i, value v_i, gate(s)
 * and, for the delta rules, a write strength beta_i. Its transition matrix M_i
 * and update S <- M_i S + b_i k_i v_i^T are:
 *   SSM_MAMBA2 : M = a I                         , b = 1      (scalar decay a)
 *   SSM_GDN    : M = alpha (I - beta k k^T)      , b = beta   (scalar gate alpha)
 *   SSM_KDA    : M = (I - beta k k^T) Diag(alpha), b = beta   (per-channel gate alpha[d_k])
 * With S_win the state at the window start, after tau buffered tokens
 *   S_tau = A S_win + R,  A = M_tau ... M_1,  R = sum_i M_tau..M_{i+1} b_i k_i v_i^T,
 * and the exact output is y = S_tau^T q = S_win^T (A^T q) + R^T q.
 * The sketch read replaces S_win^T q~ (q~ = A^T q) by Sk^T c with c = B q~.
 *
 * Memory layouts (row-major, every pointer a DEVICE pointer owned by the
 * caller; the library keeps no pointer after a call returns):
 *   state   S   fp32  [N][H][d_k][d_v]
 *   sketch  Sk  fp32 or bf16 (ssm_dims.sketch_dtype)  [N][H][r][d_v]
 *                                        row m = S^T b_m (the output for basis vector b_m)
 *   basis   B   fp32  [H][r][d_k]        row m = b_m; rows orthonormal (not checked)
 *   k_buf       in    [N][H][W][d_k]     window buffer, slot i = token i+1 of the window
 *   v_buf       in    [N][H][W][d_v]
 *   decay_buf   fp32  [N][H][W] (Mamba-2 a, GDN alpha) or [N][H][W][d_k] (KDA alpha)
 *   beta_buf    fp32  [N][H][W] (GDN, KDA); NULL for Mamba-2
 *   q, k_t      in    [N][H][d_k]        one token per unit
 *   v_t         in    [N][H][d_v]
 *   decay_t     fp32  [N][H] or [N][H][d_k];  beta_t fp32 [N][H] or NULL
 *   y           fp32  [N][H][d_v]
 * "in" is bf16 or fp32 as ssm_dims.in_dtype says. A unit is (n, h), flat
 * index n*H + h.
 *
 * Calls are asynchronous: arguments are checked on the host, then the work is
 * enqueued on `stream` (a hipStream_t; NULL = the default stream). No call
 * allocates, frees or synchronises. Invalid arguments return a non-zero
 * status before anything is enqueued; a failed launch returns SSM_E_LAUNCH.
 * Faults inside a kernel surface at the caller's next synchronisation. No C++
 * exception crosses this interface. The detail of the last failure on the
 * calling thread is in ssm_last_error().
 *
 * Supported shapes: d_k in {16, 32, 64, 128}; d_v in {16, 32, 64, 128}; 1 <= W <= 16;
 * 1 <= r <= min(d_k, 32); N >= 0 (N = 0 is a no-op); H >= 1; N*H < 2^24, which
 * keeps every grid (one workgroup of up to 256 threads per unit) below 2^32
 * threads. Every pointer must be 16-byte aligned. Outputs must not overlap any
 * input of the same call.
 */
#ifndef SKETCHSSM_H
#define SKETCHSSM_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SSM_ABI_VERSION 5

typedef enum { SSM_MAMBA2 = 0, SSM_GDN = 1, SSM_KDA = 2 } ssm_rule;
typedef enum { SSM_IN_BF16 = 0, SSM_IN_F32 = 1 } ssm_in_dtype;
/* Storage type of the sketch. The pages leave its precision open: fp32 is the
 * default; bf16 halves the sketch bytes every decode step reads. A bf16 sketch
 * is computed in fp32 and rounded to nearest, ties to even, when it is stored. */
typedef enum { SSM_SKETCH_F32 = 0, SSM_SKETCH_BF16 = 1 } ssm_sketch_dtype;

typedef enum {
  SSM_OK = 0,
  SSM_E_NULL = 1,   /* a required pointer is NULL                          */
  SSM_E_SHAPE = 2,  /* unsupported or inconsistent dimensions               */
  SSM_E_ALIGN = 3,  /* a pointer is not 16-byte aligned                     */
  SSM_E_RANGE = 4,  /* an enum, a token count, tau or slot is out of range,
                       or beta is given for Mamba-2                         */
  SSM_E_ALIAS = 5,  /* an output overlaps an input                          */
  SSM_E_LAUNCH = 6  /* the HIP runtime refused the launch                   */
} ssm_status;

typedef struct {
  int32_t rule;      /* ssm_rule                          */
  int32_t in_dtype;  /* ssm_in_dtype of q, k, v           */
  int32_t batch;     /* N sequences                       */
  int32_t heads;     /* H heads                           */
  int32_t d_k;       /* key / state rows                  */
  int32_t d_v;       /* value / state columns             */
  int32_t window;    /* W buffered tokens per state write */
  int32_t rank;      /* r basis vectors (sketch rows)     */
  int32_t sketch_dtype; /* ssm_sketch_dtype of the sketch (0: fp32) */
} ssm_dims;

/* SSM_ABI_VERSION of the library. */
int32_t ssm_abi_version(void);

/* Static text for a status code. */
const char* ssm_status_string(int32_t status);

/* Detail of the last non-OK status returned on the calling thread ("" if none). */
const char* ssm_last_error(void);

/*
 * Token buffering. Copies the current token of every unit into window slot
 * `slot` (0-based, 0 <= slot < W): k_t -> k_buf, v_t -> v_buf,
 * decay_t -> decay_buf, beta_t -> beta_buf (beta_t and beta_buf NULL for
 * Mamba-2). Source: the pages' buffering of keys and values between state
 * writes (readsearch.ai listing, Abstract, on ReplaySSM; agihunt.info
 * "Confirmed", background bullet).
 */
ssm_status ssm_buffer_append(const ssm_dims* d,
                             const void* k_t, const void* v_t,
                             const float* decay_t, const float* beta_t,
                             void* k_buf, void* v_buf, float* decay_buf, float* beta_buf,
                             int32_t slot, void* stream);

/*
 * Window update fused with the sketch refresh. For every unit: reads S once,
 * applies the first n_tokens buffered tokens in order (S <- M_i S + b_i k_i v_i^T),
 * writes S back (only if n_tokens > 0), then, if `sketch` is not NULL, stores
 * Sk = B S (row m = S^T b_m) from the updated state. n_tokens = 0 with a sketch
 * is the refresh-only pass that creates the first sketch; sketch = NULL (basis
 * may then be NULL) is a plain windowed update with no refresh.
 * 0 <= n_tokens <= W. Source: readsearch.ai listing, Abstract (one full-state
 * read per update precomputes the basis outputs); agihunt.info "Error control"
 * (the full state is updated once per window and the sketch is refreshed in
 * the same kernel).
 * Outputs: state (in/out), sketch. Inputs: basis, the buffers.
 */
ssm_status ssm_window_update_refresh(const ssm_dims* d,
                                     float* state, void* sketch, const float* basis,
                                     const void* k_buf, const void* v_buf,
                                     const float* decay_buf, const float* beta_buf,
                                     int32_t n_tokens, void* stream);

/*
 * Sketch decode step (the per-step read). tau (1 <= tau <= W) tokens of the
 * window are valid, the current token included. For every unit:
 *   walk the buffer newest to oldest from u = q:  s_i = k_i . u,
 *   intra += b_i s_i v_i,  u <- M_i^T u;  then q~ = u, c = B q~ and
 *   y = Sk^T c + intra.
 * Reads only the sketch, the basis, q and the buffer; never the state.
 * Token append, fused: if k_t is not NULL, the current token (k_t, v_t,
 * decay_t, beta_t) is first written into slot tau-1 of the buffer and used
 * from there; if k_t is NULL, slot tau-1 must already hold it and v_t,
 * decay_t, beta_t must be NULL too. The buffers are written only in the
 * fused case. Source: readsearch.ai listing, Abstract (each decode step
 * combines the sketch vectors with query-dependent coefficients);
 * agihunt.info "Mechanism details" (within a window only the queries vary).
 * Output: y. The sketch and the state are never written.
 */
ssm_status ssm_sketch_decode_step(const ssm_dims* d,
                                  const void* sketch, const float* basis, const void* q,
                                  const void* k_t, const void* v_t,
                                  const float* decay_t, const float* beta_t,
                                  void* k_buf, void* v_buf, float* decay_buf, float* beta_buf,
                                  int32_t tau, float* y, void* stream);

/*
 * Exact full-read decode step (the comparison path: the buffered read that
 * still reads all of S each step; readsearch.ai listing, Abstract, on
 * ReplaySSM). Same walk as ssm_sketch_decode_step, then
 * y = S_win^T q~ + intra, reading the whole window-start state S_win = state.
 * Token append works as in ssm_sketch_decode_step. Output: y.
 */
ssm_status ssm_full_read_decode_step(const ssm_dims* d,
                                     const float* state, const void* q,
                                     const void* k_t, const void* v_t,
                                     const float* decay_t, const float* beta_t,
                                     void* k_buf, void* v_buf, float* decay_buf, float* beta_buf,
                                     int32_t tau, float* y, void* stream);

/*
 * Heterogeneous sketch ranks per head (the pages report an average sketch rank
 * of 8: agihunt.info "Results"), for ssm_window_update_refresh_ranked and
 * ssm_sketch_decode_step_ranked. rank_offsets is a HOST array of H + 1 int32
 * prefix offsets: head h has rank r_h = rank_offsets[h+1] - rank_offsets[h],
 * 1 <= r_h <= min(d_k, 32), rank_offsets[0] = 0, H <= 256; the array is read
 * during the call only. With R = rank_offsets[H]:
 *   basis   fp32 [R][d_k]       rows rank_offsets[h] .. +r_h are head h's basis
 *   sketch  [N][R][d_v] (fp32 or bf16) rows rank_offsets[h] .. +r_h of sequence n are
 *                               the outputs of head h's basis vectors
 * d->rank must still be a valid rank (the table decides the sizes). Every other
 * argument and behaviour is that of the uniform-rank entry point.
 */
ssm_status ssm_window_update_refresh_ranked(const ssm_dims* d, const int32_t* rank_offsets,
                                            float* state, void* sketch, const float* basis,
                                            const void* k_buf, const void* v_buf,
                                            const float* decay_buf, const float* beta_buf,
                                            int32_t n_tokens, void* stream);

ssm_status ssm_sketch_decode_step_ranked(const ssm_dims* d, const int32_t* rank_offsets,
                                         const void* sketch, const float* basis, const void* q,
                                         const void* k_t, const void* v_t,
                                         const float* decay_t, const float* beta_t,
                                         void* k_buf, void* v_buf, float* decay_buf,
                                         float* beta_buf, int32_t tau, float* y, void* stream);

/*
 * Variable-length batches over a pool of persistent slots (serving with
 * continuous batching: sequences join, leave and sit at different positions
 * of their windows). A call serves d->batch rows; row n uses slot[n] (a DEVICE
 * int32 array, or NULL for slot n) of a pool of num_slots slots:
 *   persistent, indexed by slot: state [num_slots][H][d_k][d_v], sketch
 *     [num_slots][H][r][d_v], k_buf/v_buf/decay_buf/beta_buf [num_slots][H][W]...
 *   per call, indexed by row: q, k_t, v_t, decay_t, beta_t, y [batch][H][...]
 * Per-row counts come from DEVICE int32 arrays:
 *   ssm_window_update_refresh_varlen: n_tokens[n] in [0, W] tokens to apply
 *     (0 = refresh only); any other value skips the row.
 *   ssm_sketch_decode_step_varlen: tau[n] in [1, W] as in ssm_sketch_decode_step;
 *     any other value skips the row (its y is not written).
 * A row whose slot is outside [0, num_slots) is skipped too. Rows of one call
 * must map to distinct slots (calls with repeated slots race); the device
 * arrays are not read on the host. Uniform sketch rank (d->rank). The slot and
 * count arrays need 4-byte alignment; everything else as the lockstep entry
 * points. Source: the pages' setting of large decode batches (readsearch.ai
 * listing, Abstract); the serving schedule itself is not on the pages.
 */
ssm_status ssm_window_update_refresh_varlen(const ssm_dims* d, int32_t num_slots,
                                            const int32_t* slot, const int32_t* n_tokens,
                                            float* state, void* sketch, const float* basis,
                                            const void* k_buf, const void* v_buf,
                                            const float* decay_buf, const float* beta_buf,
                                            void* stream);

ssm_status ssm_sketch_decode_step_varlen(const ssm_dims* d, int32_t num_slots,
                                         const int32_t* slot, const int32_t* tau,
                                         const void* sketch, const float* basis, const void* q,
                                         const void* k_t, const void* v_t,
                                         const float* decay_t, const float* beta_t,
                                         void* k_buf, void* v_buf, float* decay_buf,
                                         float* beta_buf, float* y, void* stream);

/*
 * One serving decode step over a slot pool in a single launch (ABI version 5).
 * Source: the pages' once-per-window state write and every-step sketch read
 * (readsearch.ai listing of arXiv 2609.33051, Abstract; agihunt.info summary,
 * "Mechanism details"), for a batch whose sequences sit at different window
 * positions; the schedule itself is not on the pages. For every batch row n
 * with slot s = slot[n] (or n when slot is NULL) and tau[n] in [1, W]:
 *   1. the current token (k_t, v_t, decay_t, beta_t of row n) is appended into
 *      window slot tau[n] - 1 of slot s;
 *   2. y[n] is the sketch read at window position tau[n], as
 *      ssm_sketch_decode_step, from sketch0 when parity[n] is 0 and from
 *      sketch1 otherwise;
 *   3. if n is one of the n_update rows listed in update_rows (DEVICE int32
 *      batch-row indices, distinct) and tau[n] == W, the window's W tokens (the
 *      current one included) are applied to state[s], and the refreshed sketch
 *      is stored in the other buffer (sketch1 when parity[n] is 0, else
 *      sketch0). A listed row with tau[n] != W is not updated.
 * The two sketch buffers let a row at tau = W read its window's sketch while
 * the same launch writes the next one; the caller flips parity[n] for the
 * row's next window. Rows with tau outside [1, W] or slot outside
 * [0, num_slots) are skipped (nothing is read for them and y[n] is not
 * written). slot, tau and parity are DEVICE int32 [batch] arrays (4-byte
 * aligned; parity required); the counts in them are not read on the host.
 * Rows must map to distinct slots. Layouts as the other _varlen entry points,
 * sketch0 and sketch1 each [num_slots][H][r][d_v] in d->sketch_dtype; uniform
 * rank. Outputs: y, state, sketch0, sketch1 and the window buffers, none of
 * which may overlap an input or each other.
 */
ssm_status ssm_decode_step_varlen(const ssm_dims* d, int32_t num_slots, const int32_t* slot,
                                  const int32_t* tau, const int32_t* parity, int32_t n_update,
                                  const int32_t* update_rows, float* state, void* sketch0,
                                  void* sketch1, const float* basis, const void* q,
                                  const void* k_t, const void* v_t, const float* decay_t,
                                  const float* beta_t, void* k_buf, void* v_buf,
                                  float* decay_buf, float* beta_buf, float* y, void* stream);

/*
 * Least-squares coefficients: the other reading of the pages' "low-rank
 * state-weighted query approximation" (readsearch.ai listing of arXiv
 * 2609.33051, Abstract). Instead of c = B q~, a step takes the c that minimises
 * || S_win^T q~ - Sk^T c || (the smallest such c when the sketch rows are
 * linearly dependent), so its output Sk^T c + R^T q is the orthogonal
 * projection of the exact window-start read on the span of the sketch rows.
 * It is never further from the exact read than the projection read, and it is
 * exact whenever S_win^T q~ lies in that span (e.g. a state of rank <= r whose
 * row space the sketch captures).
 *
 * ssm_window_update_refresh_ls: the window update as ssm_window_update_refresh,
 * then, from the updated state S and Sk = B S,
 *   sketch_q  fp32 [N][H][r][d_v]  rows orthonormal and spanning the rows of Sk
 *                                  (Gram-Schmidt; a row whose residual is below
 *                                  1e-5 of the largest Sk row norm is stored as zero)
 *   read_map  fp32 [N][H][r][d_k]  Y = sketch_q S^T
 * ssm_sketch_decode_step_ls: the step as ssm_sketch_decode_step, with
 * y = sketch_q^T (read_map q~) + R^T q. The basis is not read.
 * Requires sketch_dtype = SSM_SKETCH_F32 (else SSM_E_RANGE); uniform rank; all
 * sequences at the same window position. Outputs of the update: state,
 * sketch_q, read_map; of the step: y (and the buffers when the token is fused).
 * Per step the read moves r*(d_v + d_k)*4 bytes of sketch_q and read_map per
 * unit instead of r*d_v*4 of Sk.
 */
ssm_status ssm_window_update_refresh_ls(const ssm_dims* d, float* state, float* sketch_q,
                                        float* read_map, const float* basis, const void* k_buf,
                                        const void* v_buf, const float* decay_buf,
                                        const float* beta_buf, int32_t n_tokens, void* stream);
ssm_status ssm_sketch_decode_step_ls(const ssm_dims* d, const float* sketch_q,
                                     const float* read_map, const void* q, const void* k_t,
                                     const void* v_t, const float* decay_t,
                                     const float* beta_t, void* k_buf, void* v_buf,
                                     float* decay_buf, float* beta_buf, int32_t tau, float* y,
                                     void* stream);

/*
 * Per-token recurrent decode step (the standard decode SketchSSM is compared
 * against: readsearch.ai listing, Abstract, kernel speedups over the standard
 * vLLM baseline; agihunt.info "Confirmed", background bullet: every step reads
 * the full state). For every unit, with the current token (k_t, v_t, decay_t,
 * beta_t): S <- M S + b k v^T, S is written back, and y = S^T q is read from
 * the updated state. No window buffer and no sketch; d->window and d->rank are
 * checked but not used. Outputs: state (in/out), y.
 */
ssm_status ssm_recurrent_decode_step(const ssm_dims* d,
                                     float* state, const void* q,
                                     const void* k_t, const void* v_t,
                                     const float* decay_t, const float* beta_t,
                                     float* y, void* stream);

/*
 * Offline basis fit on the device. The pages fix the query basis offline
 * (readsearch.ai listing, Abstract; agihunt.info "Confirmed", mechanism bullet:
 * queries are compressed onto a small low-rank basis); the Mamba-2 workload's
 * recipe takes the top PCA directions of sampled queries and makes them
 * orthonormal. For every head h, with X_h = samples[h] (n_samples queries of
 * d_k entries), basis[h] receives the d->rank unit eigenvectors of the
 * uncentred second moment X_h^T X_h / n_samples with the largest eigenvalues,
 * one per row, in decreasing order of eigenvalue, orthonormal in fp32, each
 * signed so that its entry of largest magnitude (the first on a tie) is
 * positive. Rows for equal eigenvalues are some orthonormal basis of their
 * eigenspace.
 *   samples: [H][n_samples][d_k], d->in_dtype, device, read only;
 *   basis:   [H][rank][d_k] fp32, device, out: the layout the window and
 *            sketch calls read.
 * Uses heads, d_k, rank and in_dtype of d; the other fields are checked but
 * not used. 1 <= n_samples <= 2^24. The basis must not overlap the samples.
 * Setup-time work: one workgroup per head, nothing allocated.
 */
ssm_status ssm_fit_basis(const ssm_dims* d, const void* samples, int32_t n_samples,
                         float* basis, void* stream);

/*
 * Measurement aid, not a step of the method: the HBM rate that a state-sized
 * read + write reaches on this device, to set the window update's bandwidth
 * against. Streams buf in place: every value is read, multiplied by 1.0f and
 * written back, all of a thread's loads before its stores, non-temporal.
 *   buf:     fp32, device, n_tiles * 16384 floats (64 KB tiles), in/out;
 *   shape 0: the window update's access order: one 256-thread workgroup per
 *            tile seen as a 128 x 128 state; each wave holds 32 columns, lane
 *            group g of a wave the rows g, g + 8, ...; consecutive tiles go to
 *            one XCD;
 *   shape 1: two tiles per 512-thread workgroup, read as one flat run; each
 *            load instruction of the workgroup covers 8 KB contiguous.
 * 1 <= n_tiles < 2^24; shape 1 needs an even n_tiles (else SSM_E_SHAPE);
 * shape outside {0, 1} gives SSM_E_RANGE. One launch per call.
 */
ssm_status ssm_stream_probe(float* buf, int64_t n_tiles, int32_t shape, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SKETCHSSM_H */
