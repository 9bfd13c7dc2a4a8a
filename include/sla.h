/*
 * sla.h -- C ABI of the sparse-linear attention forward library (libsla.so).
 *
 * What is computed (one attention head at a time, every head independent):
 *
 *   route          Q and K are mean-pooled over blocks of 64 consecutive
 *                  tokens; the block logits s_ij = qbar_i . kbar_j / sqrt(d)
 *                  are ranked per query block i (descending, equal logits by
 *                  ascending j); the first k_crit KV blocks are critical, the
 *                  next k_marg marginal, the rest negligible.
 *                  [SLA2 technical summary, section 2.B (router on pooled Q
 *                  and K, hard top-k at inference); SLA abstract (critical /
 *                  marginal / negligible classes)]
 *   linear states  per KV block j: H_j = phi(K_j)^T V_j (d x d) and
 *                  z_j = sum over the block's tokens of phi(k), phi = softmax
 *                  over the d features.
 *                  [PISA technical summary, "Algoritmo Central" (per-block
 *                  first-order matrices); SPLA technical summary, section 2.2
 *                  (compact linear-attention state of unselected blocks)]
 *   forward        O_s = softmax attention of each query over the tokens of
 *                  its query block's critical KV blocks only (renormalised
 *                  over those keys); O_l = phi(q) (sum_{j marginal} H_j) /
 *                  (phi(q) . sum_{j marginal} z_j); negligible blocks are
 *                  skipped; O = alpha_h O_s + (1 - alpha_h) O_l.
 *                  [SLA abstract (O(N^2) on critical, O(N) on marginal,
 *                  skip negligible, one fused kernel); SLA2 technical
 *                  summary, section 1 item 1 (renormalised sparse softmax)
 *                  and section 2.A (the alpha mixing equation)]
 *   fp8 variant    the sparse branch with Q, K, V quantised per 64-token
 *                  block to OCP E4M3 with a float32 scale, QK^T and PV on
 *                  fp8 matrix cores.
 *                  [SLA2 technical summary, section 2.C (low-bit sparse
 *                  branch)]
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Every function returns an int status: SLA_OK (0) or a negative
 *   sla_status.  On error a thread-local message is available from
 *   sla_last_error_message().  No function throws or aborts.
 * - Device pointers are HIP device addresses on the current device; host
 *   pointers are marked "host".  The caller owns and allocates every buffer
 *   (outputs and workspace included); the library allocates no device
 *   memory and keeps no per-call state.
 * - "stream" is a hipStream_t passed as void* (NULL = the null stream).
 *   All work is enqueued on it asynchronously; the library never
 *   synchronises.  A returned SLA_OK covers argument validation and kernel
 *   launch; faults inside a kernel surface at the caller's next sync.
 * - Q, K, V and O share the problem's element strides (stride_d == 1):
 *   element (b, h, n, c) is at b*stride_b + h*stride_h + n*stride_n + c.
 *   Their base pointers must be 16-byte aligned and stride_n * elem_size a
 *   multiple of 16.  O has the input dtype.
 * - Every other array is dense row-major in the shape given, owned by the
 *   caller: index lists int32, class map int8, states bf16 / float32.
 * - Functions are reentrant; concurrent calls on different streams with
 *   disjoint outputs and workspaces are safe.
 * - The library only runs on gfx950 (MI355X); on any other device, or with
 *   no device, compute entry points return SLA_ERR_NO_DEVICE after argument
 *   validation.
 */
#ifndef SLA_H_
#define SLA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SLA_VERSION_MAJOR 0
#define SLA_VERSION_MINOR 6
#define SLA_VERSION_PATCH 0

/* Status codes. */
typedef enum sla_status {
  SLA_OK = 0,
  SLA_ERR_INVALID_ARGUMENT = -1, /* null pointer, bad count, misalignment  */
  SLA_ERR_UNSUPPORTED = -2,      /* valid but not implemented: d, block, dtype, size */
  SLA_ERR_WORKSPACE = -3,        /* workspace pointer null or too small     */
  SLA_ERR_DEVICE = -4,           /* a HIP call or kernel launch failed      */
  SLA_ERR_NO_DEVICE = -5         /* no HIP device, or it is not gfx950      */
} sla_status;

/* Element type of Q, K, V and O. */
typedef enum sla_dtype { SLA_F32 = 0, SLA_BF16 = 1 } sla_dtype;

/* Operation selector for sla_workspace_size. */
typedef enum sla_op {
  SLA_OP_ROUTE = 0,
  SLA_OP_LINEAR_STATES = 1,
  SLA_OP_FORWARD = 2,
  SLA_OP_QUANTIZE_FP8 = 3,
  SLA_OP_FORWARD_FP8 = 4,
  SLA_OP_ROUTE_TAYLOR = 5,
  SLA_OP_FORWARD_PISA = 6,
  SLA_OP_BACKWARD = 7,
  SLA_OP_ROUTE_PISA = 8,
  SLA_OP_RESIDUAL_SUBTRACT = 9
} sla_op;

/* Problem description (host struct, read only during the call).
 * batch, heads, seq_len >= 1; head_dim in {64, 128}; block == 64;
 * k_crit >= 0, k_marg >= 0, 1 <= k_crit + k_marg <= nkb where
 * nkb = ceil(seq_len / 64); dtype is an sla_dtype; strides are in elements. */
typedef struct sla_problem {
  int32_t batch, heads, seq_len, head_dim;
  int32_t block;
  int32_t k_crit, k_marg;
  int32_t dtype;
  int64_t stride_b, stride_h, stride_n;
} sla_problem;

/* Host-only checks of a problem (no HIP call).  SLA_OK,
 * SLA_ERR_INVALID_ARGUMENT (null, sizes < 1, bad counts, strides that
 * overlap rows) or SLA_ERR_UNSUPPORTED (head_dim, block, dtype, more than
 * 4096 KV blocks, or one head spanning more than 4 GiB:
 * (seq_len - 1) * stride_n * elem_size + head_dim * elem_size > 2^32 - 1,
 * which only very wide row strides such as packed QKV of many heads reach,
 * or 2 * batch * heads * ceil(seq_len / 64) > 2^31 - 1, the launch grid). */
int sla_validate(const sla_problem* problem);

/* Host: number of query blocks and KV blocks (both ceil(seq_len / 64)). */
int sla_num_blocks(const sla_problem* problem, int32_t* nq, int32_t* nkb);

/* Host: bytes of device workspace the operation needs (0 if none).  The
 * workspace passed to a call must be at least this large and 256-byte
 * aligned.  SLA_OP_FORWARD (and SLA_OP_FORWARD_FP8) needs a bf16
 * [B,H,nq,d,d] marginal-state sum, a float32 [B,H,nq,d] normaliser sum,
 * B*H*2*ceil(nkb/64)*(nq rounded up to 512) 32-bit words of marginal-mask
 * bits and bf16 [B,H,nkb,2d] parts of z, each region 256-byte aligned;
 * SLA_OP_ROUTE
 * needs float64 pooled Q and K and the 64-bit selection keys of one pass
 * over heads (nq x nkb rounded up to 64 per head, as many heads as fit
 * 512 MiB, at least one), SLA_OP_ROUTE_TAYLOR those and float64 block
 * key variances; SLA_OP_FORWARD_PISA needs bf16 block means of K and V
 * [B,H,64*ceil(nkb/64),d], a bf16 Hbar [B,H,d,d] and float32 per-chunk
 * partial sums of the first-order matrices; SLA_OP_BACKWARD needs the
 * forward workspace, an O scratch in the problem layout, float O_s, O_l
 * [B,H,N,d], float row statistics [B,H,N] x 3, bf16 dS with dsigma
 * [B,H,nq,d*d+d], bf16 dH with dz [B,H,nkb,d*d+d], transposed mask bits and
 * float dalpha partials [B,H,nq]. */
int sla_workspace_size(const sla_problem* problem, int op, size_t* bytes);

/* Block routing.  [SLA2 summary 2.B; SLA abstract]
 * q, k         input [B,H,N,d] (problem strides, problem dtype)
 * crit_idx     out int32 [B,H,nq,k_crit], ascending KV block indices
 * marg_idx     out int32 [B,H,nq,k_marg], ascending
 * block_class  out int8  [B,H,nq,nkb] or NULL: 0 negligible, 1 marginal,
 *              2 critical
 * block_logits out float [B,H,nq,nkb] or NULL: s_ij rounded to float32
 * pooled_q,
 * pooled_k     out float [B,H,nb,d] or NULL: block means rounded to float32
 * ws           workspace of sla_workspace_size(SLA_OP_ROUTE) bytes.
 * Pooling and logits are evaluated in float64, so the ranking follows the
 * exact block means up to summation order.  The logits go as a tiled
 * product into the workspace's keys, then a second kernel selects; the keys,
 * and so the lists, are those of the one-kernel path sla_route_noalloc
 * takes. */
int sla_route(const sla_problem* problem, const void* q, const void* k,
              int32_t* crit_idx, int32_t* marg_idx, int8_t* block_class,
              float* block_logits, float* pooled_q, float* pooled_k, void* ws,
              size_t ws_bytes, void* stream);

/* Block routing that also quantises Q and K for the low-bit sparse branch.
 * [SLA2 summary 2.B, 2.C]  Exactly sla_route (same arguments, results and
 * errors) plus, from the tiles the pooling pass already reads, the E4M3
 * codes and scales of Q and K that sla_quantize_fp8 would write:
 * q8, k8         out uint8 [B,H,N,d] contiguous
 * q_scales,
 * k_scales       out float [B,H,nb]
 * so the fp8 forward needs no separate pass over Q and K. */
int sla_route_quantize(const sla_problem* problem, const void* q, const void* k,
                       int32_t* crit_idx, int32_t* marg_idx, int8_t* block_class,
                       float* block_logits, float* pooled_q, float* pooled_k, uint8_t* q8,
                       float* q_scales, uint8_t* k8, float* k_scales, void* ws,
                       size_t ws_bytes, void* stream);

/* Block routing and the per-block linear states in one call.  [SLA2
 * summary 2.B; SLA abstract; PISA summary]  Exactly sla_route followed by
 * sla_linear_states (same arguments, results and errors; h_states and
 * z_states as sla_linear_states writes them; ws of
 * sla_workspace_size(SLA_OP_ROUTE) bytes).  For bf16 inputs the states pass
 * also forms the pooled keys from the K tiles it reads anyway, in the
 * routing pass's summation order, so K crosses HBM once instead of twice;
 * float32 inputs take the two passes. */
int sla_route_states(const sla_problem* problem, const void* q, const void* k,
                     const void* v, int32_t* crit_idx, int32_t* marg_idx,
                     int8_t* block_class, float* block_logits, float* pooled_q,
                     float* pooled_k, void* h_states, float* z_states, void* ws,
                     size_t ws_bytes, void* stream);

/* Bytes of device scratch the library holds per GPU for the allocation-free
 * entry points. */
#define SLA_STATIC_SCRATCH_BYTES ((size_t)64 << 20)

/* Block routing without a workspace, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  Same arguments, results and errors as
 * sla_route, minus ws / ws_bytes: the float64 pooled sums live in a static
 * device array of SLA_STATIC_SCRATCH_BYTES that the library holds on every
 * GPU it runs on until the process ends (its device address is looked up
 * once per device on the first call there).  The call allocates nothing.
 * The selection runs as one fused kernel (keys in LDS), so only the pooled
 * sums need the scratch: returns SLA_ERR_WORKSPACE when those, 16 * B * H *
 * nkb * d bytes, exceed SLA_STATIC_SCRATCH_BYTES (at head_dim 128:
 * B * H * nkb > 32768).  Every
 * call on one GPU shares that GPU's array, whatever the stream: calls that
 * overlap in time on one GPU race on it and must be serialised by the
 * caller (one stream, or events). */
int sla_route_noalloc(const sla_problem* problem, const void* q, const void* k,
                      int32_t* crit_idx, int32_t* marg_idx, int8_t* block_class,
                      float* block_logits, float* pooled_q, float* pooled_k,
                      void* stream);

/* Check of caller-supplied index lists.  [SLA abstract: each KV block of a
 * row is critical, marginal or negligible, one class each]
 * crit_idx     in int32 [B,H,nq,k_crit] (NULL allowed when k_crit = 0)
 * marg_idx     in int32 [B,H,nq,k_marg] (NULL allowed when k_marg = 0)
 * Every entry must lie in [0, nkb), no list may repeat an index and no index
 * may be in both lists of a row (ascending order is not required).  The
 * compute entry points do not check lists: they clamp each entry into
 * [0, nkb) before forming an address, so no list makes them access memory
 * outside their arguments, but an invalid list gives meaningless results.
 * Returns SLA_OK, or SLA_ERR_INVALID_ARGUMENT naming the number of bad rows
 * and the first one.  The call waits for `stream` (the lists are read after
 * the work already queued on it).  It uses a small report array that the
 * library holds per GPU; calls on one GPU take turns on a host lock. */
int sla_validate_lists(const sla_problem* problem, const int32_t* crit_idx,
                       const int32_t* marg_idx, void* stream);

/* Block routing with the second-order score.  [SPLA summary 2.1]
 * The block score keeps the spread of the keys around their block mean,
 * to second order with a diagonal covariance:
 *   s_ij = qbar_i . kbar_j / sqrt(d) + log1p(sum_a qbar_ia^2 var_ja / (2 d)),
 * var_ja = population variance of feature a over block j's valid keys.
 * Outputs, ordering and tie rule are those of sla_route, with s_ij in
 * block_logits, plus
 * key_var      out float [B,H,nb,d] or NULL: var_ja rounded to float32
 * ws           workspace of sla_workspace_size(SLA_OP_ROUTE_TAYLOR) bytes.
 * Means, variances and logits are evaluated in float64. */
int sla_route_taylor(const sla_problem* problem, const void* q, const void* k,
                     int32_t* crit_idx, int32_t* marg_idx, int8_t* block_class,
                     float* block_logits, float* pooled_q, float* pooled_k,
                     float* key_var, void* ws, size_t ws_bytes, void* stream);

/* Per-block linear-attention states.  [PISA summary; SPLA summary 2.2]
 * k, v      input [B,H,N,d]
 * h_states  out bf16 [B,H,nkb,d,d], value-major: element [c][a] of block j
 *           is H_j[a][c] = sum_n phi(k_n)[a] v_n[c] (H_j^T row-major)
 * z_states  out float [B,H,nkb,d]: z_j[a] = sum_n phi(k_n)[a]
 * A short last block sums its valid tokens only.  phi is evaluated in
 * float32, H is accumulated in float32 from bf16 operands. */
int sla_linear_states(const sla_problem* problem, const void* k, const void* v,
                      void* h_states, float* z_states, void* stream);

/* Linear states that also quantise V for the low-bit sparse branch.
 * [PISA summary; SLA2 summary 2.C]  Exactly sla_linear_states plus the E4M3
 * codes (out uint8 [B,H,N,d] contiguous) and scales (out float [B,H,nb]) of
 * V that sla_quantize_fp8 would write, from the V tiles the states pass
 * already reads. */
int sla_linear_states_quantize(const sla_problem* problem, const void* k, const void* v,
                               void* h_states, float* z_states, uint8_t* v8,
                               float* v_scales, void* stream);

/* Fused sparse + linear forward.  [SLA abstract; SLA2 summary 1 and 2.A]
 * q, k, v    input [B,H,N,d]
 * crit_idx,
 * marg_idx   as written by sla_route (any ascending lists with valid,
 *            distinct indices are accepted)
 * h_states,
 * z_states   as written by sla_linear_states
 * alpha      float [H] mixing weight per head
 * o          out [B,H,N,d], problem dtype
 * o_sparse,
 * o_linear   out float [B,H,N,d] contiguous, or NULL (branch outputs)
 * ws         workspace of sla_workspace_size(SLA_OP_FORWARD) bytes.
 * A query block with k_crit == 0 has O_s = 0; with k_marg == 0, O_l = 0. */
int sla_forward(const sla_problem* problem, const void* q, const void* k,
                const void* v, const int32_t* crit_idx, const int32_t* marg_idx,
                const void* h_states, const float* z_states, const float* alpha,
                void* o, float* o_sparse, float* o_linear, void* ws,
                size_t ws_bytes, void* stream);

/* The two phases of sla_forward, for callers that schedule or time them
 * separately.  sla_marginal_sums writes, into the forward workspace, the
 * marginal-state sums S_i = sum_{j marginal} H_j (bf16 [B,H,nq,d,d],
 * value-major like h_states) and
 * sigma_i = sum_{j marginal} z_j (float [B,H,nq,d]; each z_j enters as the
 * sum of two bf16 parts hi + lo, within 2^-17 of z_j, and the sums are
 * float32, as for S_i); sla_forward_attend then
 * runs the fused sparse + linear attention reading them from the same
 * workspace.  Arguments mean what they mean for sla_forward; with
 * k_marg == 0 sla_marginal_sums does nothing.  sla_forward is exactly
 * sla_marginal_sums followed by sla_forward_attend on one stream.
 * [SLA abstract; PISA summary (per-block matrices); SLA2 summary 2.A] */
int sla_marginal_sums(const sla_problem* problem, const int32_t* marg_idx,
                      const void* h_states, const float* z_states, void* ws,
                      size_t ws_bytes, void* stream);
int sla_forward_attend(const sla_problem* problem, const void* q, const void* k,
                       const void* v, const int32_t* crit_idx,
                       const float* alpha, void* o, float* o_sparse,
                       float* o_linear, const void* ws, size_t ws_bytes,
                       void* stream);

/* Per-block E4M3 quantiser.  [SLA2 summary 2.C]
 * x        input [B,H,N,d] (problem strides and dtype)
 * x_e4m3   out uint8 [B,H,N,d] contiguous OCP E4M3 codes
 * scales   out float [B,H,nb]: scale_j = absmax_j / 448 (1 if absmax_j = 0)
 * code = e4m3_rne_saturate(fl32(x * fl32(448 / absmax_j))). */
int sla_quantize_fp8(const sla_problem* problem, const void* x, uint8_t* x_e4m3,
                     float* scales, void* stream);

/* Forward with the fp8 sparse branch.  [SLA2 summary 2.C]
 * q          bf16/f32 input [B,H,N,d] (phi(Q) of the linear branch)
 * q8,k8,v8   uint8 [B,H,N,d] contiguous codes from sla_quantize_fp8
 * q_s,k_s,v_s float [B,H,nb] their scales (positive and finite, as sla_quantize_fp8
 *            writes them)
 * the remaining arguments as for sla_forward.
 * The sparse branch computes S = (Q^ K^T) s_q s_k / sqrt(d) on fp8 matrix
 * cores, keeps the online-softmax statistics and the row sum in float32, and
 * quantises P per (query row, KV block): P s_v times a power of two 2^k that
 * puts the row's largest entry in (224, 448] is rounded to E4M3 (nearest
 * even) and the PV product is scaled back by 2^-k in the matrix core.  The
 * linear branch and the alpha mix are those of sla_forward (bf16 / float32).
 * Supported: bf16 Q and O, head_dim 128 (else SLA_ERR_UNSUPPORTED). */
int sla_forward_fp8(const sla_problem* problem, const void* q,
                    const uint8_t* q8, const float* q_s, const uint8_t* k8,
                    const float* k_s, const uint8_t* v8, const float* v_s,
                    const int32_t* crit_idx, const int32_t* marg_idx,
                    const void* h_states, const float* z_states,
                    const float* alpha, void* o, float* o_sparse,
                    float* o_linear, void* ws, size_t ws_bytes, void* stream);

/* Phase two of sla_forward_fp8, for callers that run sla_marginal_sums
 * themselves (as sla_forward_attend is for sla_forward); ws holds that
 * call's sums.  sla_forward_fp8 is exactly sla_marginal_sums followed by
 * sla_forward_attend_fp8 on one stream.  [SLA2 summary 2.C] */
int sla_forward_attend_fp8(const sla_problem* problem, const void* q,
                           const uint8_t* q8, const float* q_s,
                           const uint8_t* k8, const float* k_s,
                           const uint8_t* v8, const float* v_s,
                           const int32_t* crit_idx, const float* alpha, void* o,
                           float* o_sparse, float* o_linear, const void* ws,
                           size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Residual linear attention.  [SPLA technical summary, sections 2.2 and 2.3]
 * The blocks a query block does not select feed a linear-attention state
 * instead of being dropped, written as o_rla = o_bar - o_tilde (linear
 * attention over all blocks minus over the selected ones) with an
 * exponential feature map; the output is a gated sum of the exact sparse
 * branch and the RMS-normalised residual branch:
 *   O = alpha_h O_s + (1 - alpha_h) RMSNorm(phi(Q) S_i),
 *   S_i = sum over the KV blocks j not critical for query block i of H_j,
 *   H_j = exp(K_j)^T V_j,  phi(q) = exp(q - max q) (the RMS norm removes
 *   that per-row factor), RMSNorm(x) = x / sqrt(mean over the d features of
 *   x^2 + 1e-6) with unit scale.
 * The selected blocks are the critical ones; every other KV block is in the
 * residual state, so these calls need problem->k_marg == nkb - k_crit
 * (SLA_ERR_INVALID_ARGUMENT otherwise) and no marginal list.
 *
 * sla_linear_states_exp: as sla_linear_states with phi(k) = exp(k)
 *   elementwise (no per-token normalisation; float32, so keys must stay
 *   below about 88); h_states / z_states layouts as there.
 * sla_residual_sums: writes S_i (bf16 [B,H,nq,d,d], value-major) into the
 *   forward workspace (sla_workspace_size(SLA_OP_FORWARD) bytes) from the
 *   critical lists and the exponential-map states; the sigma region is not
 *   written.
 * sla_residual_sums_subtract: the same S_i in the page's subtraction form,
 *   S_i = (sum of every block's H_j) - (sum over the critical blocks of
 *   H_j): the global state of the head (float32, four partial sums over
 *   block ranges added in a fixed order) minus the product of the
 *   critical-block bits with the states (float32), rounded once to bf16.
 *   So phi(q) S_i = o_bar - o_tilde with o_bar from one global state and
 *   o_tilde from the selected blocks only; the unselected blocks are read
 *   only through the global state.  Its workspace is
 *   sla_workspace_size(SLA_OP_RESIDUAL_SUBTRACT) bytes, whose leading
 *   sla_workspace_size(SLA_OP_FORWARD) bytes are the forward workspace that
 *   sla_forward_attend_rla reads.  Same S_i as sla_residual_sums up to
 *   float32 summation order.
 * sla_forward_attend_rla: the fused forward reading S_i from that workspace;
 *   o_linear (when not NULL) receives RMSNorm(phi(Q) S_i).
 * sla_forward_rla: sla_residual_sums then sla_forward_attend_rla on one
 *   stream. */
int sla_linear_states_exp(const sla_problem* problem, const void* k, const void* v,
                          void* h_states, float* z_states, void* stream);
int sla_residual_sums_subtract(const sla_problem* problem, const int32_t* crit_idx,
                               const void* h_states, void* ws, size_t ws_bytes, void* stream);
int sla_residual_sums(const sla_problem* problem, const int32_t* crit_idx,
                      const void* h_states, void* ws, size_t ws_bytes, void* stream);
int sla_forward_attend_rla(const sla_problem* problem, const void* q, const void* k,
                           const void* v, const int32_t* crit_idx, const float* alpha,
                           void* o, float* o_sparse, float* o_linear, const void* ws,
                           size_t ws_bytes, void* stream);
int sla_forward_rla(const sla_problem* problem, const void* q, const void* k, const void* v,
                    const int32_t* crit_idx, const void* h_states, const float* alpha,
                    void* o, float* o_sparse, float* o_linear, void* ws, size_t ws_bytes,
                    void* stream);

/* Piecewise exact-or-approximate attention.  [PISA summary, section 2:
 * "Algoritmo Central", "Implementación de Hardware"]
 * The critical blocks of query block i (crit_idx, as written by sla_route)
 * are attended exactly (the problem's k_marg only has to pass validation;
 * the unselected set is every other block); every other KV block j enters
 * the same softmax through its centroid: alpha_tj = exp(q_t . kbar_j / sqrt(d))
 * adds alpha_tj * (sum of the block's values) to the numerator and
 * alpha_tj * n_j to the denominator; one global first-order correction
 * (q_t / sqrt(d)) Hbar sum_j alpha_tj joins the numerator, with
 * Hbar = mean over all KV blocks of H_j = sum_n (k_n - kbar_j)^T v_n.
 * o_t = numerator / denominator.
 *
 * sla_pisa_statistics writes kbar, the block means of V and Hbar into the
 * workspace (sla_workspace_size(SLA_OP_FORWARD_PISA) bytes); hbar, when not
 * NULL, receives Hbar as float [B,H,d,d] value-major (element [c][a] =
 * Hbar[a][c], a = key feature, c = value dim).  Block means are float32
 * sums of the valid tokens, rounded to bf16; H is accumulated in float32 on
 * the matrix cores from bf16 block-centred K and V.
 * sla_forward_attend_pisa runs the fused pass from that workspace:
 * o            out [B,H,N,d], problem dtype
 * o_softmax,
 * o_correction out float [B,H,N,d] contiguous, or NULL: the exact and
 *              zero-order part and the first-order part of the numerator,
 *              each divided by the denominator (o is their sum).
 * sla_forward_pisa is the two in order on one stream. */
int sla_pisa_statistics(const sla_problem* problem, const void* k, const void* v,
                        float* hbar, void* ws, size_t ws_bytes, void* stream);
int sla_forward_attend_pisa(const sla_problem* problem, const void* q, const void* k,
                            const void* v, const int32_t* crit_idx, void* o,
                            float* o_softmax, float* o_correction, const void* ws,
                            size_t ws_bytes, void* stream);
int sla_forward_pisa(const sla_problem* problem, const void* q, const void* k,
                     const void* v, const int32_t* crit_idx, void* o, float* o_softmax,
                     float* o_correction, void* ws, size_t ws_bytes, void* stream);

/* Covariance-aware block routing for piecewise attention.  [PISA summary,
 * section 2, "Enrutamiento Consciente de la Covarianza": the selection score
 * of a block takes in, beside its attention score, the norm
 * M_j = ||H_j - Hbar|| of its first-order matrix's deviation from the
 * shared Hbar]
 * An unselected block replaces its own first-order term by Hbar, so the
 * numerator misses alpha_tj (q_t / sqrt(d)) (H_j - Hbar), of norm at most
 * alpha_tj (|q_t| / sqrt(d)) M_j.  The logit weighs the block's zero-order
 * weight by one plus that discrepancy per token of a 64-token block, with
 * the pooled query:
 *   s_ij = qbar_i . kbar_j / sqrt(d) + log1p(|qbar_i| M_j / (sqrt(d) * 64)),
 * M_j the L2 norm of all d x d elements (Frobenius; it bounds the spectral
 * norm), H_j = sum_n (k_n - kbar_j)^T v_n, Hbar their mean over all KV
 * blocks.  The split, counts, tie rule and outputs are those of sla_route.
 * q, k, v      input [B,H,N,d] (problem strides and dtype)
 * crit_idx ... pooled_k   as for sla_route
 * block_dev    out float [B,H,nkb] or NULL: M_j rounded to float32
 * ws           workspace of sla_workspace_size(SLA_OP_ROUTE_PISA) bytes; its
 *              first sla_workspace_size(SLA_OP_FORWARD_PISA) bytes then hold
 *              the statistics of sla_pisa_statistics for the same k and v,
 *              so sla_forward_attend_pisa can run from it directly.
 * Pooled means, ||qbar_i||, M_j and the logits are float64 (H_j in float32:
 * matrix-core sums of the exact bf16 products, or float32 arithmetic for
 * float inputs). */
int sla_route_pisa(const sla_problem* problem, const void* q, const void* k, const void* v,
                   int32_t* crit_idx, int32_t* marg_idx, int8_t* block_class,
                   float* block_logits, float* pooled_q, float* pooled_k, float* block_dev,
                   void* ws, size_t ws_bytes, void* stream);

/* Backward pass of sla_forward for fixed block lists.  [SLA abstract
 * (forward and backward); SLA2 summary 2.A (the mix)]
 * The lists carry no gradient; alpha does.  With f = phi(q):
 *   dalpha_h = sum over the head's rows and dims of dO * (O_s - O_l);
 *   sparse branch (dO_s = alpha dO): the softmax backward over the critical
 *     keys, dq += dS K / sqrt(d), dk += dS^T q / sqrt(d), dv += P^T dO_s;
 *   linear branch (dO_l = (1 - alpha) dO): through O_l = f S_i / (f . sigma_i),
 *     S_i = sum_{j in M_i} H_j, sigma_i = sum z_j, H_j = phi(K_j)^T V_j,
 *     z_j = colsum phi(K_j), and the feature softmax phi.
 * q, k, v, dout bf16 [B,H,N,d] (problem strides; float inputs are
 *              SLA_ERR_UNSUPPORTED)
 * crit_idx,
 * marg_idx     as for sla_forward
 * h_states,
 * z_states     as written by sla_linear_states (read when k_marg > 0)
 * alpha        float [H]
 * dq, dk, dv   out float [B,H,N,d] contiguous
 * dalpha       out float [H] (summed over the batch)
 * ws           workspace of sla_workspace_size(SLA_OP_BACKWARD) bytes.
 * The call recomputes the forward (marginal sums, then the fused kernel
 * writing O_s, O_l and each row's log2 softmax normaliser into ws) before
 * the gradient kernels.  P, dS and the linear-branch operands enter the
 * matrix cores as bf16; accumulation is float32. */
int sla_backward(const sla_problem* problem, const void* q, const void* k,
                 const void* v, const void* dout, const int32_t* crit_idx,
                 const int32_t* marg_idx, const void* h_states, const float* z_states,
                 const float* alpha, float* dq, float* dk, float* dv, float* dalpha,
                 void* ws, size_t ws_bytes, void* stream);

/* The backward pass split at its forward part, for a training step that
 * runs the forward once.  [SLA abstract (forward and backward)]
 * sla_forward_save is sla_forward (same arguments, bf16 only) that also
 * keeps what the gradient kernels read: it writes O to o and, into ws (a
 * workspace of sla_workspace_size(SLA_OP_BACKWARD) bytes), the marginal
 * sums S_i and sigma_i, O_s and O_l (float) and each row's log2 softmax
 * normaliser.  sla_backward_saved then runs only the gradient kernels of
 * sla_backward, reading those from ws: the caller passes the ws that
 * sla_forward_save filled for the same problem, inputs, lists and alpha,
 * unmodified in between (nothing checks this; other contents give wrong
 * gradients, never an out-of-range access).  Arguments mean what they mean
 * for sla_backward; the states are not read again.  sla_backward is exactly
 * sla_forward_save (O into ws) followed by sla_backward_saved on one stream,
 * and both calls' results equal it bit for bit. */
int sla_forward_save(const sla_problem* problem, const void* q, const void* k,
                     const void* v, const int32_t* crit_idx, const int32_t* marg_idx,
                     const void* h_states, const float* z_states, const float* alpha,
                     void* o, void* ws, size_t ws_bytes, void* stream);
int sla_backward_saved(const sla_problem* problem, const void* q, const void* k,
                       const void* v, const void* dout, const int32_t* crit_idx,
                       const int32_t* marg_idx, const float* alpha, float* dq, float* dk,
                       float* dv, float* dalpha, void* ws, size_t ws_bytes, void* stream);

/* Low-bit forward paired with the bf16 backward, for quantisation-aware
 * training.  [SLA2 summary 2.C: the forward runs the sparse branch in a
 * low-bit format while the backward stays in 16-bit]
 * sla_forward_save_fp8 is sla_forward_fp8 (same q8 / k8 / v8 codes and
 * scales as sla_quantize_fp8 writes, head_dim 128) that keeps, like
 * sla_forward_save, what sla_backward_saved reads: the marginal sums, O_s
 * and O_l of the fp8 forward (float) and each row's log2 normaliser of the
 * fp8 sparse softmax, in ws of sla_workspace_size(SLA_OP_BACKWARD) bytes;
 * O (bf16) goes to o.  q, k, v are the bf16 inputs the codes were made
 * from.  sla_backward_saved on that ws then gives the bf16 gradients: they
 * rebuild P from the bf16 scores q k^T and the fp8 forward's normaliser and
 * take rowsum(dO_s * O_s) from the fp8 O_s, i.e. the quantisation is passed
 * through unchanged in the backward (straight-through), and the gradients
 * differ from those of the unquantised forward by the fp8 forward's error. */
int sla_forward_save_fp8(const sla_problem* problem, const void* q, const void* k,
                         const void* v, const uint8_t* q8, const float* q_scales,
                         const uint8_t* k8, const float* k_scales, const uint8_t* v8,
                         const float* v_scales, const int32_t* crit_idx,
                         const int32_t* marg_idx, const void* h_states, const float* z_states,
                         const float* alpha, void* o, void* ws, size_t ws_bytes, void* stream);

/* Host: static text of a status code. */
const char* sla_status_string(int status);

/* Host: thread-local detail of the last error raised on this thread
 * ("" if none). */
const char* sla_last_error_message(void);

/* Host: library version (host pointers). */
int sla_version(int* major, int* minor, int* patch);

#ifdef __cplusplus
}
#endif

#endif /* SLA_H_ */
