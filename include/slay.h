/*
 * slay.h -- C ABI of libslay: causal SLAY attention (Spherical Linearized
 * Attention with Yat kernels) on AMD Instinct MI355X (gfx950).
 *
 * Method sources (web pages; cited by title and section):
 *   - "SLAY: Geometry-Aware Spherical Linearized Attention with Yat-Kernel",
 *     arXiv 2602.04915, English abstract: q and k are normalised onto the
 *     sphere; K is written, via Bernstein's theorem, as a positive sum of
 *     u^2 exp(beta u) terms, which positive random features approximate, so
 *     attention costs O(L).
 *   - nubint.ai review of that paper, "Proposed method" (six bullets):
 *     (1) Yat kernel as a spherical similarity on unit-norm q, k; (2) the
 *     denominator linearised through its Laplace representation; (3) anchor
 *     features for the polynomial part, PRF for the exponential part;
 *     (4) Gauss-Laguerre discretisation of the integral; (5) the two feature
 *     sets fused by a random tensor sketch; (6) standard causal linear
 *     attention contraction without the L x L matrix.
 *
 * The computation, with u = q.k on unit vectors and eps > 0:
 *   K(u)    = u^2 / (2 - 2u + eps)                      (spherical Yat kernel)
 *   K_R(u)  = sum_r alpha_r u^2 exp(beta_r u),  alpha_r = w_r/(2+eps),
 *             beta_r = 2 x_r/(2+eps), (x_r, w_r) the R-point Gauss-Laguerre rule
 *   phi(x)[r*m+t] = sqrt(alpha_r/m) (a_rt . xh)^2 exp(sqrt(beta_r) g_rt . xh - beta_r/2),
 *             xh = x / max(|x|, 1e-12),  F = R*m features
 *   o_i     = phi(q_i)^T S_i / phi(q_i)^T z_i,
 *             S_i = S0 + sum_{j<=i} phi(k_j) v_j^T,  z_i = z0 + sum_{j<=i} phi(k_j)
 * The anchor vectors a_rt and PRF vectors g_rt are drawn by the caller
 * (i.i.d. N(0, I) for the estimator the pages describe) and passed in.
 *
 * Conventions for every call:
 *   - Device pointers are HIP device memory owned by the caller; the library
 *     never allocates or frees device memory and keeps no device state.
 *   - All arrays are dense and row-major with the shapes given; 16-byte
 *     aligned base pointers are required for q, k, v, x, o, phi and draws.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = default stream)
 *     and is asynchronous; nothing synchronises.  Calls are thread-safe.
 *   - Argument checking happens on the host before anything is enqueued:
 *     SLAY_E_INVALID (bad argument; nothing enqueued), SLAY_E_UNSUPPORTED
 *     (valid but not implemented; nothing enqueued), SLAY_E_DEVICE (a HIP
 *     launch error; the stream may hold part of the work).  The last error
 *     message of the calling thread is returned by slay_last_error().
 */
#ifndef SLAY_H
#define SLAY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SLAY_OK = 0,
  SLAY_E_INVALID = 1,
  SLAY_E_UNSUPPORTED = 2,
  SLAY_E_DEVICE = 3
} slay_status_t;

typedef enum { SLAY_F32 = 0, SLAY_BF16 = 1 } slay_dtype_t;

/* Feature-map parameters (review, "Proposed method" bullets 3-5).
 * anchors, prf: device arrays [n_draw_sets][R*m][d] of draw_dtype; row r*m+t
 * is the vector of feature t of Gauss-Laguerre node r.  Head h (0-based
 * index over B*H heads, or over the n_heads of a decode step) uses draw set
 * h % n_draw_sets; n_draw_sets = 1 shares one draw across all heads.
 * Limits: d in {32, 64, 128}; 1 <= R <= 16; m a multiple of 16; eps > 0. */
typedef struct {
  int32_t d;
  int32_t R;
  int32_t m;
  double eps;
  const void* anchors;
  const void* prf;
  slay_dtype_t draw_dtype;
  int32_t n_draw_sets;
  int64_t draw_set_stride; /* elements between consecutive draw sets (>= R*m*d) */
} slay_params_t;

/* Feature map phi of n_rows rows of x (abstract; review "Proposed method"
 * bullets 1, 3, 5).
 *   x   : device [n_rows][d], dtype x_dtype (must equal params->draw_dtype)
 *   phi : device [n_rows][R*m], dtype phi_dtype (f32 or bf16, RNE rounding)
 *   rows_per_head: rows belonging to one head, for draw-set selection
 *                  (row i uses set (i / rows_per_head) % n_draw_sets); must
 *                  divide n_rows; ignored (may be 0) when n_draw_sets == 1.
 * Projection on MFMA (fp32 accumulate), features in fp32, then rounded. */
slay_status_t slay_featmap(const slay_params_t* params, const void* x, slay_dtype_t x_dtype, int64_t n_rows,
                           int64_t rows_per_head, void* phi, slay_dtype_t phi_dtype, void* stream);

/* Workspace bytes slay_attn_chunked_fwd needs for this shape (0 is possible). */
size_t slay_attn_chunked_fwd_workspace_size(const slay_params_t* params, int32_t B, int32_t H, int64_t L,
                                            int32_t dv, int32_t chunk, slay_dtype_t io_dtype);

/* Causal SLAY forward (review, "Proposed method" bullet 6), chunked:
 * within a chunk of `chunk` tokens the masked block tril(phi(Q) phi(K)^T)
 * (diagonal included) is applied to v, the state of all earlier chunks adds
 * phi(q) S and phi(q) z; no L x L matrix is formed.
 *   q, k : device [B][H][L][d];  v, o : device [B][H][L][dv];  dtype io_dtype
 *          (draws must have the same dtype).  bf16: fp32 accumulation,
 *          outputs rounded to bf16 (RNE).
 *   S0, z0     : nullable device fp32 initial state [B*H][R*m][dv], [B*H][R*m]
 *                (NULL = zero state);
 *   S_out, z_out: nullable device fp32 final state, same shapes; S_out may
 *                alias S0 and z_out may alias z0 (the state carried in place).
 *   workspace  : device scratch of at least
 *                slay_attn_chunked_fwd_workspace_size(...) bytes (NULL if 0).
 * L need not be a multiple of chunk (the tail chunk is masked); L = 0 only
 * copies S0/z0 to S_out/z_out.  chunk in [1, 128].
 * Kernel families, chosen from the shape:
 *   bf16, d = dv = 64, chunk = 64, R*m <= 256: fused MFMA kernels (the
 *     feature map computed on chip), built for R*m in {64, 96, 128, 256};
 *     other R*m run the next built count on zero-padded features (no result
 *     changes; R*m above 128 needs m a multiple of 32);
 *   otherwise bf16, d in {32, 64, 128}, dv in {64, 128}, chunk a multiple of
 *     32, R*m in {128, 256, 384, 512}: wide MFMA kernels (phi(q), phi(k)
 *     written once to the workspace in bf16, the state kept on chip);
 *   every other accepted shape (fp32 included): the general kernels.
 * All three compute the same quantity; the chunk size changes only the
 * order of summation. */
slay_status_t slay_attn_chunked_fwd(const slay_params_t* params, const void* q, const void* k, const void* v,
                                    slay_dtype_t io_dtype, int32_t B, int32_t H, int64_t L, int32_t dv,
                                    int32_t chunk, const float* S0, const float* z0, void* o, float* S_out,
                                    float* z_out, void* workspace, size_t workspace_bytes, void* stream);

/* Size of the fixed device scratch behind slay_attn_chunked_fwd_noalloc. */
#define SLAY_NOALLOC_SCRATCH_BYTES (32u << 20)

/* slay_attn_chunked_fwd for callers that cannot allocate device memory
 * (code under stream capture, tight serving loops, hosts that forbid
 * allocation).  Same arguments, semantics and kernels as
 * slay_attn_chunked_fwd, without the workspace: the library uses its own
 * fixed device array of SLAY_NOALLOC_SCRATCH_BYTES bytes instead (32 MiB,
 * held on every GPU the library runs on until the process ends).  Calls whose
 * workspace would exceed it -- slay_attn_chunked_fwd_workspace_size(...) >
 * SLAY_NOALLOC_SCRATCH_BYTES -- return SLAY_E_UNSUPPORTED with nothing
 * enqueued.  Nothing is allocated or freed: not by the library, not through
 * a library it calls.  The scratch carries no state between calls (no
 * kernel reads what an earlier call left in it), but every call on one GPU
 * shares it: calls that overlap in time on one GPU (different streams or
 * threads) race and give wrong results; serialise them.  The scratch's
 * device address is looked up once per device on the first call there. */
slay_status_t slay_attn_chunked_fwd_noalloc(const slay_params_t* params, const void* q, const void* k,
                                            const void* v, slay_dtype_t io_dtype, int32_t B, int32_t H, int64_t L,
                                            int32_t dv, int32_t chunk, const float* S0, const float* z0, void* o,
                                            float* S_out, float* z_out, void* stream);

/* Workspace bytes slay_attn_varlen_fwd needs (0 for unsupported shapes). */
size_t slay_attn_varlen_fwd_workspace_size(const slay_params_t* params, int32_t n_seqs, int32_t H,
                                           int64_t total_tokens, int32_t dv, slay_dtype_t io_dtype);

/* Causal SLAY forward over a batch of sequences of different lengths (the
 * same contraction as slay_attn_chunked_fwd, review "Proposed method" bullet
 * 6, applied to each sequence on its own; bounded-state streaming of mixed
 * lengths, review "Motivation and goals").  The sequences are packed along one
 * token axis per head: sequence s holds tokens cu_seqlens[s] ..
 * cu_seqlens[s+1] - 1 of every head.
 *   q, k : device [H][total_tokens][d];  v, o : device [H][total_tokens][dv];
 *          bf16 (must equal the draw dtype); fp32 accumulation.
 *   cu_seqlens : device int64 [n_seqs + 1], non-decreasing from 0 to
 *          total_tokens (read on the device; offsets that break this rule
 *          make the call compute nothing: o is left as it was and the final
 *          states equal the initial ones).
 *   S0, z0     : nullable device fp32 initial states [n_seqs][H][R*m][dv],
 *                [n_seqs][H][R*m] (NULL = zero);
 *   S_out, z_out: nullable device fp32 final states, same shapes (may alias
 *                S0, z0): a prefill's hand-off to slay_attn_recurrent_step.
 *   workspace  : device scratch of slay_attn_varlen_fwd_workspace_size() bytes.
 * Supported: bf16, d = dv = 64, R*m <= 256 with m a multiple of 32 (the
 * fused MFMA kernels; R*m below 256 on features zero-padded to 256, which
 * changes no result; other shapes return SLAY_E_UNSUPPORTED), total_tokens
 * below 2^31 - 64 (else SLAY_E_UNSUPPORTED).  One launch each of a
 * work-list kernel, the segment-state pass, the per-sequence scan and the
 * main pass, whatever the number of sequences; the tails of several short
 * sequences share one workgroup. */
slay_status_t slay_attn_varlen_fwd(const slay_params_t* params, const void* q, const void* k, const void* v,
                                   slay_dtype_t io_dtype, int32_t n_seqs, int32_t H, const int64_t* cu_seqlens,
                                   int64_t total_tokens, int32_t dv, const float* S0, const float* z0, void* o,
                                   float* S_out, float* z_out, void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes slay_attn_chunked_bwd needs for this shape (0 is possible). */
size_t slay_attn_chunked_bwd_workspace_size(const slay_params_t* params, int32_t B, int32_t H, int64_t L,
                                            int32_t dv, int32_t chunk, slay_dtype_t io_dtype);

/* Backward of slay_attn_chunked_fwd: the gradients of a scalar loss with
 * respect to q, k, v and the initial state, given its gradients with
 * respect to o and (optionally) the final state.  The pages define the
 * forward (review, "Proposed method" bullets 1-6); this is that forward
 * differentiated.  With g_i = dout_i / den_i and h_i = -(dout_i . o_i) / den_i
 * (den_i = phi(q_i)^T z_i):
 *   dphi(q_i) = S_i g_i + z_i h_i,
 *   dphi(k_j) = U_j v_j + u_j,  dv_j = U_j^T phi(k_j),
 *   U_j = dS_T + sum_{i>=j} phi(q_i) g_i^T,  u_j = dz_T + sum_{i>=j} phi(q_i) h_i,
 *   dS0 = U_0, dz0 = u_0,
 * and dq, dk through the feature map's Jacobian (including the projection
 * onto the sphere).  The draws are constants: no gradient is returned for them.
 *   q, k, dq, dk : device [B][H][L][d];  v, dout, dv : device [B][H][L][dv];
 *          dtype io_dtype (must equal the draw dtype); fp32 accumulation,
 *          gradients rounded to io_dtype (RNE).
 *   S0, z0     : nullable device fp32 initial state of the forward (as given to it);
 *   dS_T, dz_T : nullable device fp32 gradients of the final state [B*H][R*m][dv],
 *                [B*H][R*m] (NULL = zero);
 *   dS0, dz0   : nullable device fp32 outputs, gradients of the initial state
 *                (same shapes; may alias dS_T, dz_T);
 *   workspace  : device scratch of at least
 *                slay_attn_chunked_bwd_workspace_size(...) bytes (NULL if 0).
 * chunk in [1, 128] only changes the summation order; dv <= 256.  L = 0 sets
 * dS0 = dS_T and dz0 = dz_T (zero where those are NULL).
 * Kernel families, chosen from the shape:
 *   bf16, d = dv = 64, chunk = 64, m a multiple of 32, R*m <= 256: MFMA
 *     kernels (per-segment states, 16-token steps, phi recomputed on chip;
 *     every product that touches a state, phi or g runs on split hi + lo
 *     bf16 operands, because dq is a small difference of large terms);
 *     R*m below 256 runs them on features zero-padded to 256, which changes
 *     no result (the padded features and their gradients are exactly zero);
 *   every other accepted shape: general kernels (the feature map to the
 *     workspace, per-chunk states with a forward prefix and a reverse
 *     suffix, FMA contractions). */
slay_status_t slay_attn_chunked_bwd(const slay_params_t* params, const void* q, const void* k, const void* v,
                                    const void* dout, slay_dtype_t io_dtype, int32_t B, int32_t H, int64_t L,
                                    int32_t dv, int32_t chunk, const float* S0, const float* z0, const float* dS_T,
                                    const float* dz_T, void* dq, void* dk, void* dv_out, float* dS0, float* dz0,
                                    void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes slay_attn_noncausal_fwd needs for this shape (0 is possible). */
size_t slay_attn_noncausal_fwd_workspace_size(const slay_params_t* params, int32_t B, int32_t H, int64_t Lq,
                                              int64_t Lk, int32_t dv, slay_dtype_t io_dtype);

/* Non-causal SLAY forward: every query attends to every key, the standard
 * linear-attention contraction (review, "Proposed method" bullet 6) over all
 * keys, as used for the vision and extreme-classification settings (review,
 * "Motivation and goals" bullet 5, "Main results" bullet 4):
 *   o_i = phi(q_i)^T S / phi(q_i)^T z,  S = S0 + sum_j phi(k_j) v_j^T,
 *   z = z0 + sum_j phi(k_j).
 *   q, o : device [B][H][Lq][d], [B][H][Lq][dv];  k, v : device [B][H][Lk][d],
 *          [B][H][Lk][dv];  dtype io_dtype (must equal the draw dtype); bf16
 *          accumulates in fp32 and rounds the outputs to bf16 (RNE).
 *   S0, z0     : nullable device fp32 initial state [B*H][R*m][dv], [B*H][R*m];
 *   S_out, z_out: nullable device fp32 final state S, z (same shapes; may
 *                alias S0, z0).
 *   workspace  : device scratch of at least
 *                slay_attn_noncausal_fwd_workspace_size(...) bytes (NULL if 0).
 * Lq and Lk are independent (Lq = 0 only produces the state).  Lk = 0 needs
 * z0 when Lq > 0 (SLAY_E_INVALID otherwise: the denominators would be 0).
 * bf16 with d = dv = 64 and R*m <= 256 runs the fused MFMA kernels (segment
 * states of the keys, their sum, a readout pass over the queries; R*m not in
 * {64, 96, 128, 256} on zero-padded features, R*m above 128 with m a multiple
 * of 32); every other accepted shape runs the general kernels. */
slay_status_t slay_attn_noncausal_fwd(const slay_params_t* params, const void* q, const void* k, const void* v,
                                      slay_dtype_t io_dtype, int32_t B, int32_t H, int64_t Lq, int64_t Lk,
                                      int32_t dv, const float* S0, const float* z0, void* o, float* S_out,
                                      float* z_out, void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes slay_attn_recurrent_step needs (2 * n_heads * R*m * 4). */
size_t slay_attn_recurrent_step_workspace_size(const slay_params_t* params, int64_t n_heads, int32_t dv,
                                               slay_dtype_t io_dtype);

/* One O(1)-per-token decode step for n_heads independent heads (the
 * recurrent form of the same attention; review, "Proposed method" bullet 6):
 * phi(q), phi(k) of the new token, S += phi(k) v^T, z += phi(k), then
 * o = phi(q)^T S / phi(q)^T z.
 *   q, k : device [n_heads][d];  v, o : device [n_heads][dv];  dtype io_dtype
 *          (must equal params->draw_dtype); outputs in io_dtype
 *   S, z : device fp32 state [n_heads][R*m][dv], [n_heads][R*m], updated in place
 *   workspace: device scratch of slay_attn_recurrent_step_workspace_size()
 *          bytes (phi(q), phi(k) in fp32).
 * dv in {16, 32, 64, 128}; R*m a multiple of 16, at most 1024, and a multiple
 * of 1024/dv.  Two launches: the feature map of all heads, then one streaming
 * pass over the state. */
slay_status_t slay_attn_recurrent_step(const slay_params_t* params, const void* q, const void* k, const void* v,
                                       slay_dtype_t io_dtype, int64_t n_heads, int32_t dv, float* S, float* z,
                                       void* o, void* workspace, size_t workspace_bytes, void* stream);

/* Host-only: the R-point Gauss-Laguerre mixture parameters used by the
 * library, alpha[r] = w_r/(2+eps), beta[r] = 2 x_r/(2+eps) (fp64, R <= 16).
 * Returns SLAY_OK or SLAY_E_INVALID. */
slay_status_t slay_gl_table(int32_t R, double eps, double* alpha, double* beta);

/* Host-only: positive orthogonal random-feature draws (the linearized
 * 2-simplicial attention page's summary: positive orthogonal random features,
 * a variance-reduced alternative to i.i.d. PRF draws at the same F).  Rows
 * come in blocks of d: within a block they are mutually orthogonal, and each
 * row is marginally N(0, I_d) -- the block is the Haar-random orthogonal
 * factor of a Gaussian matrix (Householder QR with the signs fixed so that R
 * has a positive diagonal), row i scaled by the length of an independent
 * Gaussian vector.  The randomness is the caller's:
 *   gauss : [ceil(n_rows/d)][d][d] fp64, i.i.d. N(0, 1) (block b's matrix);
 *   chi   : [ceil(n_rows/d)][d][d] fp64, i.i.d. N(0, 1) (row i of block b has
 *           length |chi[b][i]|);
 *   out   : [n_rows][d] fp32, the first n_rows rows of the blocks in order.
 * For SLAY's PRF draws [R*m][d], call it once per node on that node's m rows
 * (orthogonal within the node), then copy to the device.  Returns SLAY_OK or
 * SLAY_E_INVALID (NULL pointer, d outside [1, 4096], non-finite input). */
slay_status_t slay_orthogonal_draws(int32_t n_rows, int32_t d, const double* gauss, const double* chi, float* out);

/* Static description of a status code. */
const char* slay_status_string(slay_status_t status);

/* Message of the last failed call on the calling thread ("" if none). */
const char* slay_last_error(void);

/* ABI version (major * 10000 + minor * 100 + patch). */
int32_t slay_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SLAY_H */
