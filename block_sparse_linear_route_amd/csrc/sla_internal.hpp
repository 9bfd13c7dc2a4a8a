// Internal interface between the C-ABI layer (api.cpp) and the kernel
// translation units.  Not installed; not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>


namespace sla {

// Validated problem geometry (all sizes checked by the API layer).
struct Geometry {
  int B, H, N, D;        // batch, heads, tokens, head dim
  int nq, nkb;           // query blocks, KV blocks (both ceil(N / 64))
  int k_crit, k_marg;    // critical / marginal blocks per query block
  int dtype;             // 0 = float32, 1 = bfloat16 (Q, K, V, O)
  int64_t sb, sh, sn;    // element strides of Q, K, V, O
};

// Static device scratch of the allocation-free entry points (scratch.hip):
// kStaticScratchBytes per GPU, 256-byte aligned.  static_scratch() returns
// the current device's copy (looked up once per device); calls that use it
// concurrently on one GPU share it.
constexpr size_t kStaticScratchBytes = size_t(64) << 20;
hipError_t static_scratch(void** ptr);

// ws_kvar non-null: second-order routing score (block key variances pooled
// into it, and into key_var as float32 when that is non-null).  block_dev
// non-null (and ws_kvar null): covariance-aware score, block_dev holding
// the float64 deviation norms M_j [B*H][nkb].
// f8 non-null (plain score only): the pooling pass also writes the E4M3
// codes and scales of Q and K ([B,H,N,d] u8, [B,H,nb] float).
struct Fp8Out {
  uint8_t* q8;
  float* q_scale;
  uint8_t* k8;
  float* k_scale;
};
// ws_keys non-null: the logits go through memory (route_key_bytes(g) of
// workspace) and the selection runs as a kernel of its own; null: one fused
// kernel keeps them in LDS.  ws_kpool (and ws_kvar) hold pooled K (and the
// key variances) as rows [B*H][nkb][d] on the split path, transposed
// [B*H][d][nkb] for the fused kernel.  k_pooled (plain score, no f8, split
// path): ws_kpool already holds the pooled keys (launch_states with kpool),
// so only Q is pooled.
constexpr size_t kRouteKeyBytes = size_t(512) << 20;   // keys of one pass over heads, at most
inline int route_key_nkbp(const Geometry& g) { return (g.nkb + 63) / 64 * 64; }
// heads whose keys one pass holds (all, or as many as fit kRouteKeyBytes)
inline int route_key_heads(const Geometry& g) {
  const size_t per = static_cast<size_t>(g.nq) * route_key_nkbp(g) * 8;
  const size_t fit = kRouteKeyBytes / per;
  const size_t bh = static_cast<size_t>(g.B) * g.H;
  return static_cast<int>(fit < 1 ? 1 : (fit < bh ? fit : bh));
}
inline size_t route_key_bytes(const Geometry& g) {
  return static_cast<size_t>(route_key_heads(g)) * g.nq * route_key_nkbp(g) * 8;
}
hipError_t launch_route(const Geometry& g, const void* q, const void* k, int32_t* crit,
                        int32_t* marg, int8_t* cls, float* logits, float* pooled_q,
                        float* pooled_k, double* ws_qpool, double* ws_kpool,
                        double* ws_kvar, float* key_var, hipStream_t stream,
                        const double* block_dev = nullptr, const Fp8Out* f8 = nullptr,
                        uint64_t* ws_keys = nullptr, bool k_pooled = false);

// exp_map: phi(k) = exp(k) elementwise instead of the softmax over features.
// v8 non-null (softmax map only): also the E4M3 codes and scales of V.
// kpool non-null (bf16, softmax map, no v8): also the pooled key rows of
// the router, float64 [B*H][nkb][d] as the pooling pass writes them for the
// split selection (and float32 [B,H,nkb,d] into kout when non-null).
hipError_t launch_states(const Geometry& g, const void* k, const void* v, uint16_t* h_states,
                         float* z_states, bool exp_map, hipStream_t stream,
                         uint8_t* v8 = nullptr, float* v_scale = nullptr,
                         double* kpool = nullptr, float* kout = nullptr);

// Marginal-state sums S_i = sum_{j in M_i} H_j (bf16, [B,H,nq,d,d], value-major
// like the states) and sigma_i = sum_{j in M_i} z_j (float, [B,H,nq,d]); bits
// is scratch of B*H*marginal_chunks(g)*marginal_rows_pad(g)*2 32-bit words for
// the mask rows (two words per query block and chunk of 64 KV blocks).
inline int marginal_chunks(const Geometry& g) { return (g.nkb + 63) / 64; }
inline int marginal_rows_pad(const Geometry& g) { return (g.nq + 511) / 512 * 512; }
// zhl: scratch of B*H*nkb*2*d bf16 for the hi / lo parts of z (sigma comes
// out of the same product as S).
// complement: marg is the critical list (k_crit entries per query block) and
// S_i sums every KV block outside it (the residual state of residual linear
// attention); sigma_sum, z_states and zhl are not used.
hipError_t launch_marginal_sums(const Geometry& g, const int32_t* marg, const uint16_t* h_states,
                                const float* z_states, uint16_t* s_sum, float* sigma_sum,
                                uint32_t* bits, uint16_t* zhl, bool complement, hipStream_t stream);

// The product S = M H alone, from mask bits already in the layout the
// marginal sums write (chunk-major, rows padded to the 512-row tile); with
// nq = nkb the roles of query and KV blocks can be swapped (a transposed mask).
// with_vector: rows of d*d + d elements (a d-vector after each matrix, summed
// the same way).  zhl (with_vector false): also the float32 sums
// sigma = M (hi + lo) of the bf16 parts of z, rows of 2 d.
hipError_t launch_mask_gemm(const Geometry& g, const uint32_t* bits, const uint16_t* h_states,
                            uint16_t* s_sum, hipStream_t stream, bool with_vector = false,
                            const uint16_t* zhl = nullptr, float* sigma = nullptr,
                            const float* tot = nullptr);

// Residual sums in the subtraction form: the global state of each head (as
// float32 partial sums in tot, residual_total_bytes) minus the product of
// the critical-block bits with the states, rounded to bf16 into s_sum.
hipError_t launch_residual_subtract(const Geometry& g, const int32_t* crit, const uint16_t* h_states,
                                    uint16_t* s_sum, uint32_t* bits, float* tot,
                                    hipStream_t stream);
size_t residual_total_bytes(const Geometry& g);

// rla: residual linear attention epilogue (s_sum holds every non-critical
// block's exponential-map state; RMS norm in place of the sigma denominator).
// lse (optional, float [B,H,N]): log2 of each row's sparse softmax normaliser.
hipError_t launch_attention(const Geometry& g, const void* q, const void* k, const void* v,
                            const int32_t* crit, const uint16_t* s_sum, const float* sigma_sum,
                            const float* alpha, void* o, float* o_sparse, float* o_linear,
                            bool rla, hipStream_t stream, float* lse = nullptr);

// Piecewise exact-or-approximate attention.  Pseudo-blocks: the centroid
// rows are grouped 64 to a tile; the block statistics are reduced in chunks
// of G consecutive KV blocks (fewer blocks per chunk when that leaves fewer
// than 512 workgroups), each chunk leaving a float32 d x d partial sum.
inline int pisa_pseudo_blocks(const Geometry& g) { return (g.nkb + 63) / 64; }
inline int pisa_chunk_blocks(const Geometry& g) {
  int G = 16;
  while (G > 1 && static_cast<int64_t>(g.B) * g.H * ((g.nkb + G - 1) / G) < 512) G /= 2;
  return G;
}
inline int pisa_chunks(const Geometry& g) {
  const int G = pisa_chunk_blocks(g);
  return (g.nkb + G - 1) / G;
}
// kbar / vbar: bf16 [B*H][pisa_pseudo_blocks*64][d] block means of K / V;
// hbar: bf16 [B*H][d][d] value-major mean first-order matrix; part: float32
// [B*H][pisa_chunks][d][d] scratch; hbar_f32: optional float32 copy of hbar.
hipError_t launch_pisa_stats(const Geometry& g, const void* k, const void* v, uint16_t* kbar,
                             uint16_t* vbar, uint16_t* hbar, float* part, float* hbar_f32,
                             hipStream_t stream);
// Covariance-aware routing statistics, after launch_pisa_stats wrote
// hbar_f32: mdev [B*H][nkb] float64 (and mdev_out float32, optional)
// receives M_j = || H_j - Hbar || (all d x d elements).  For float32 inputs
// Hbar (hbar, hbar_f32) is first recomputed from float32 operands through
// part.
hipError_t launch_pisa_deviation(const Geometry& g, const void* k, const void* v, uint16_t* hbar,
                                 float* part, float* hbar_f32, double* mdev, float* mdev_out,
                                 hipStream_t stream);
// The fused pass: exact online softmax over the critical blocks, then the
// centroid pseudo-blocks in the same softmax, then the first-order
// correction; o_softmax / o_correction (float, optional) are the two parts
// of O divided by the shared denominator.
hipError_t launch_attention_pisa(const Geometry& g, const void* q, const void* k, const void* v,
                                 const int32_t* crit, const uint16_t* kbar, const uint16_t* vbar,
                                 const uint16_t* hbar, void* o, float* o_softmax,
                                 float* o_correction, hipStream_t stream);

// Backward pass.  Buffers (all in the backward workspace): the forward's
// float O_s, O_l [B*H][N][d] and log2 softmax normaliser [B*H][N]; the
// forward workspace's marginal sums (s_sum, sigma); D_t [B*H][N]; dS_i bf16
// [B*H][nq][d*d + d] (the d x d matrix value-major, then dsigma_i); dH bf16
// [B*H][nkb][d*d + d] (likewise, dz_j after the matrix); the
// transposed critical bit rows [B*H][nkb][backward_crit_words] and the
// transposed marginal mask in the mask-product layout; dalpha partials
// [B*H][nq].  Inputs bf16 only.
struct BackwardBuffers {
  const float* o_s;
  const float* o_l;
  const float* lse;
  float* dd;
  float* dol;
  const uint16_t* s_sum;
  const float* sigma;
  uint16_t* ds;
  uint16_t* dh;
  uint32_t* crit_t;
  uint32_t* marg_t;
  float* dalpha_part;
};
inline int backward_crit_words(const Geometry& g) { return (g.nq + 31) / 32; }
hipError_t launch_backward(const Geometry& g, const BackwardBuffers& w, const void* q,
                           const void* k, const void* v, const void* dout, const int32_t* crit,
                           const int32_t* marg, const float* alpha, float* dq, float* dk,
                           float* dv, float* dalpha, hipStream_t stream);

// Largest KV block count the library accepts (validated on the host).
constexpr int kMaxKvBlocks = 4096;

// Checks the index lists of every row (range, repeats, overlap); waits on
// the stream and returns the number of bad rows and the smallest bad row
// index (0xffffffff when none).
hipError_t validate_lists(const Geometry& g, const int32_t* crit, const int32_t* marg,
                          hipStream_t stream, unsigned int* bad_rows, unsigned int* first_bad);

hipError_t launch_quantize_fp8(const Geometry& g, const void* x, uint8_t* codes, float* scales,
                               hipStream_t stream);

hipError_t launch_attention_fp8(const Geometry& g, const void* q, const uint8_t* q8,
                                const float* q_s, const uint8_t* k8, const float* k_s,
                                const uint8_t* v8, const float* v_s, const int32_t* crit,
                                const uint16_t* s_sum, const float* sigma_sum,
                                const float* alpha, void* o, float* o_sparse, float* o_linear,
                                hipStream_t stream, float* lse = nullptr);

}  // namespace sla
