// Epilogue shared by the fused attention kernels (bf16 and fp8 sparse branch).
//
// Both kernels run 4 waves per (b, h, query block i), wave = qh + 2*kh: qh
// picks 32 of the 64 query rows and kh one of two disjoint key subsets whose
// online softmaxes ran separately.  Each wave arrives with the O^T tiles it
// accumulated (lane = query, 32 dims per tile), its running reference max
// m_run and its partial row sum l_run (this lane's keys only; the partner lane
// l ^ 32 holds the rest of the row).  The epilogue
//   * merges the two key subsets through LDS ([SLA2 technical summary,
//     section 1 item 1]: the sparse softmax is renormalised over the kept keys
//     only), each wave finalising half of the output dims;
//   * computes the linear branch O_l = phi(Q) S_i / (phi(Q) . sigma_i) from
//     the marginal-state sum S_i and sigma_i ([SLA2 summary, section 2.A];
//     phi = softmax over the features, evaluated as exp(q - max q) because the
//     row normaliser cancels between numerator and denominator);
//   * mixes O = alpha_h O_s + (1 - alpha_h) O_l ([SLA2 summary, section 2.A
//     equation]) and stores O, plus O_s / O_l when requested.
// With kRla (residual linear attention, [SPLA technical summary, sections 2.2
// and 2.3]) S_i sums every non-critical block's exponential-map state, the
// linear output phi(Q) S_i is not divided by phi(Q) . sigma_i but RMS-
// normalised over the d value features of each row (x / sqrt(mean x^2 +
// 1e-6); the factor exp(-max q) of phi(Q) cancels there), and O_l is that
// normalised output.
// With kPisa (piecewise exact-or-approximate attention, [PISA technical
// summary, "Algoritmo Central"]) the merged softmax already holds the exact
// and zero-order terms; the epilogue adds the global first-order term
// (q_t / sqrt(d)) Hbar A_t to the numerator, A_t = sum of alpha_{t,j} over
// the unselected blocks (a_run, merged like l_run), before the one division:
// O_s is the softmax part, O_l the correction part, O = O_s + O_l.
// kLse: lse (float [B,H,N]) receives log2 of each row's sparse softmax
// normaliser in the scaled log2 units of the scores.
// m_run is in the units of S; cl converts them to log2 units.
#pragma once

#include "device_common.hpp"
#include "sla_internal.hpp"

namespace sla {

__device__ __forceinline__ void store4(uint16_t* p, const float* x) {
  u32x2 w;
  w[0] = static_cast<uint32_t>(f32_to_bf16_bits(x[0])) | (static_cast<uint32_t>(f32_to_bf16_bits(x[1])) << 16);
  w[1] = static_cast<uint32_t>(f32_to_bf16_bits(x[2])) | (static_cast<uint32_t>(f32_to_bf16_bits(x[3])) << 16);
  *reinterpret_cast<u32x2*>(p) = w;
}
__device__ __forceinline__ void store4(float* p, const float* x) {
  f32x4 w = {x[0], x[1], x[2], x[3]};
  *reinterpret_cast<f32x4*>(p) = w;
}

// LDS bytes the epilogue needs at the start of the shared buffer: merge
// buffers, sigma_i, and the per-row sums of squares of the residual branch.
template <int D>
constexpr int epilogue_smem_bytes() {
  return 4 * (256 + 4 * (D / 64) * 16 * 64) + D * 4 + 4 * 128;
}

constexpr float kRmsEps = 1e-6f;

// XOR swizzle of the 16-byte chunks of a bf16 tile row (64 rows x D): the
// operand reads of 16 consecutive rows at one chunk, and the transposing V
// reads (4 consecutive keys x 4 chunks), hit distinct LDS banks.
template <int D>
__device__ __forceinline__ int swz(int r) {
  if constexpr (D == 128) return 4 * (r & 3) + ((r >> 2) & 3);
  else return (r >> 1) & 7;
}

// merge_lds: epilogue_smem_bytes<D>() bytes of LDS for the merge buffers.
// sg_lds: sigma_i already in LDS (visible to all waves) when sg_ok, else it
// is loaded from sigma_sum here.  (Both LDS pointers are always valid, so
// the compiler keeps them in the LDS address space.)
// st_half (read when kStLds; D = 128 only): the 64 rows c = 64*kh .. +63 of
// the value-major sum S_i^T that this wave's key half finalises, already in
// LDS as a swizzled 64 x D tile; otherwise S_i^T is read from s_sum in HBM.
// qf: bf16 Q fragments of query 32*qh + l32, features 16*s + 8*(lane/32) .. +7.
// With kHooks, hook(1) runs once the LDS below merge_lds is no longer read
// and hook(2) once the merge buffers are no longer read (all waves, after a
// barrier): a caller can start loads for its next block there.
template <typename T, int D, bool kStLds, bool kHooks, bool kRla = false, bool kPisa = false,
          bool kLse = false, typename Hook>
__device__ __forceinline__ void attention_finish(
    unsigned char* merge_lds, const uint16_t* st_half, const float* sg_lds, bool sg_ok,
    const Geometry& g, int bh, int h, int i,
    int n_i, int qrow, int64_t hoff, const uint16_t* __restrict__ s_sum,
    const float* __restrict__ sigma_sum, const float* __restrict__ alpha, void* o,
    float* o_sparse, float* o_linear, const f32x16 (&oacc)[D / 32], float m_run, float l_run,
    float cl, const bf16x8 (&qf)[D / 16], Hook&& hook, float a_run = 0.0f,
    float* __restrict__ lse = nullptr) {
  constexpr int NS = D / 16;
  constexpr int DT = D / 32;
  constexpr int DTH = DT / 2;
  constexpr int MERGE_BYTES = 4 * (256 + 4 * DTH * 16 * 64);
  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int kh = wave >> 1;
  const int l32 = lane & 31, hh = lane >> 5;

  // ---- merge the two key halves; stage the linear-branch operands ----
  float* mbuf = reinterpret_cast<float*>(merge_lds);  // [4][32]
  float* lbuf = mbuf + 128;                            // [4][32]
  float* obuf = mbuf + 256;                            // [4][DTH][16][64]
  float* sg = reinterpret_cast<float*>(merge_lds + MERGE_BYTES);  // sigma_i [D]
  float* rbuf = sg + D;                                            // [4][32] row sums of squares
  const int own0 = kh * DTH;

  const float l_full = l_run + xor_lane(l_run, 32);
  [[maybe_unused]] float a_full = 0.0f;
  if constexpr (kPisa) a_full = a_run + xor_lane(a_run, 32);
  if (hh == 0) {
    mbuf[wave * 32 + l32] = m_run;
    lbuf[wave * 32 + l32] = l_full;
    if constexpr (kPisa) rbuf[wave * 32 + l32] = a_full;
  }
  // the wave keeps dims [32*own0, +32*DTH) and hands the other half to its
  // partner; select with static indices so the accumulators stay in registers
  f32x16 o_own[DTH];
#pragma unroll
  for (int u = 0; u < DTH; ++u) {
    o_own[u] = kh ? oacc[DTH + u] : oacc[u];
    const f32x16 oth = kh ? oacc[u] : oacc[DTH + u];
#pragma unroll
    for (int r = 0; r < 16; ++r) obuf[((wave * DTH + u) * 16 + r) * 64 + lane] = oth[r];
  }

  // phi(Q) as the B operand of O_l^T = S_i^T phi(Q)^T (exp(q - max q) per
  // query row; the row normaliser cancels against the denominator)
  const bool has_lin = kPisa || g.k_marg > 0;
  bf16x8 pf[NS];
  if (!kPisa && has_lin) {
    float qmax = -INFINITY;
#pragma unroll
    for (int s = 0; s < NS; ++s)
#pragma unroll
      for (int e = 0; e < 8; ++e) qmax = fmaxf(qmax, bf16v_to_f32(qf[s][e]));
    qmax = fmaxf(qmax, xor_lane(qmax, 32));
#pragma unroll
    for (int s = 0; s < NS; ++s)
#pragma unroll
      for (int e = 0; e < 8; ++e)
        pf[s][e] = f32_to_bf16(__builtin_amdgcn_exp2f((bf16v_to_f32(qf[s][e]) - qmax) * kLog2e));
  }

  // S_i^T rows (value dim c = 32*(own0+u) + l32, features 16*s + 8*hh .. +7)
  // of the value-major sum: from the LDS copy, or straight from HBM (their
  // latency then overlaps the merge)
  const int64_t row = static_cast<int64_t>(bh) * g.nq + i;
  const int64_t srow = kPisa ? static_cast<int64_t>(bh) : row;   // Hbar is per head
  bf16x8 sf[DTH][NS];
  if (has_lin) {
    if constexpr (kStLds) {
#pragma unroll
      for (int u = 0; u < DTH; ++u) {
        const int r = 32 * u + l32;
#pragma unroll
        for (int s = 0; s < NS; ++s)
          sf[u][s] = *reinterpret_cast<const bf16x8*>(st_half + r * D + 8 * ((2 * s + hh) ^ swz<D>(r)));
      }
    } else {
      const uint16_t* sgl = s_sum + srow * D * D;   // uniform base, 32-bit lane offsets
#pragma unroll
      for (int u = 0; u < DTH; ++u)
#pragma unroll
        for (int s = 0; s < NS; ++s)
          sf[u][s] = load8_at(sgl, static_cast<uint32_t>(((32 * (own0 + u) + l32) * D + 16 * s + 8 * hh) * 2));
    }
    if (!kRla && !kPisa && !sg_ok && t < D) sg[t] = sigma_sum[row * D + t];
  }
  __syncthreads();
  if constexpr (kHooks) hook(1);   // every wave has read S_i^T: the LDS below merge_lds is free

  const int partner = wave ^ 2;
  const float m_p = mbuf[partner * 32 + l32];
  const float l_p = lbuf[partner * 32 + l32];
  const float m_tot = fmaxf(m_run, m_p);
  const float w_me = (m_run == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f((m_run - m_tot) * cl);
  const float w_p = (m_p == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f((m_p - m_tot) * cl);
  const float den = l_full * w_me + l_p * w_p;
  const float inv = den > 0.0f ? 1.0f / den : 0.0f;
  // log2 of the sparse softmax normaliser, sum over kept keys of
  // exp2(s * cl), for a backward pass to rebuild P (-inf when no key)
  if (kLse && kh == 0 && hh == 0 && qrow < n_i)
    lse[static_cast<int64_t>(bh) * g.N + kBlock * i + qrow] =
        den > 0.0f ? m_tot * cl + log2f(den) : -INFINITY;
  // merged O_s, in place of the wave's own partial output
#pragma unroll
  for (int u = 0; u < DTH; ++u)
#pragma unroll
    for (int r = 0; r < 16; ++r)
      o_own[u][r] = (o_own[u][r] * w_me + obuf[((partner * DTH + u) * 16 + r) * 64 + lane] * w_p) * inv;
  if constexpr (kHooks) {
    __syncthreads();
    hook(2);   // the merge buffers are free (sigma stays in use when it lives there)
  }

  f32x16 ol[DTH];
#pragma unroll
  for (int u = 0; u < DTH; ++u) ol[u] = zero16();
  if constexpr (kPisa) {
    // Hbar^T Q^T on the matrix cores (raw Q: the 1/sqrt(d) goes into the
    // row factor with A_t and the denominator)
#pragma unroll
    for (int s = 0; s < NS; ++s)
#pragma unroll
      for (int u = 0; u < DTH; ++u) ol[u] = mfma32(sf[u][s], qf[s], ol[u]);
    const float a_p = rbuf[partner * 32 + l32];
    const float fac = (a_full * w_me + a_p * w_p) * inv * (cl * (1.0f / kLog2e));
#pragma unroll
    for (int u = 0; u < DTH; ++u)
#pragma unroll
      for (int r = 0; r < 16; ++r) ol[u][r] *= fac;
  } else if constexpr (kRla) {
    // RMS norm of phi(Q) S_i over the row's D dims: this lane's 16 * DTH, the
    // partner lane's (l ^ 32) and the other key-half wave's (wave ^ 2) half
    float ss = 0.0f;
    if (has_lin) {
#pragma unroll
      for (int s = 0; s < NS; ++s)
#pragma unroll
        for (int u = 0; u < DTH; ++u) ol[u] = mfma32(sf[u][s], pf[s], ol[u]);
#pragma unroll
      for (int u = 0; u < DTH; ++u)
#pragma unroll
        for (int r = 0; r < 16; ++r) ss = fmaf(ol[u][r], ol[u][r], ss);
      ss = swap_sum32(ss);
      if (hh == 0) rbuf[wave * 32 + l32] = ss;
    }
    __syncthreads();
    if (has_lin) {
      const float rinv =
          1.0f / __builtin_sqrtf((ss + rbuf[partner * 32 + l32]) * (1.0f / D) + kRmsEps);
#pragma unroll
      for (int u = 0; u < DTH; ++u)
#pragma unroll
        for (int r = 0; r < 16; ++r) ol[u][r] *= rinv;
    }
  } else if (has_lin) {
    float dpart = 0.0f;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
#pragma unroll
      for (int e = 0; e < 8; ++e)
        dpart += bf16v_to_f32(pf[s][e]) * (sg_ok ? sg_lds[16 * s + 8 * hh + e] : sg[16 * s + 8 * hh + e]);
#pragma unroll
      for (int u = 0; u < DTH; ++u) ol[u] = mfma32(sf[u][s], pf[s], ol[u]);
    }
    const float dsum = dpart + xor_lane(dpart, 32);
    const float dinv = 1.0f / dsum;
#pragma unroll
    for (int u = 0; u < DTH; ++u)
#pragma unroll
      for (int r = 0; r < 16; ++r) ol[u][r] *= dinv;
  }

  // ---- alpha mix and store ----
  const float al = kPisa ? 1.0f : alpha[h];
  if (qrow < n_i) {
    // uniform bases of the query block, 32-bit offsets of this lane's row
    char* obase = reinterpret_cast<char*>(static_cast<T*>(o) + hoff + static_cast<int64_t>(kBlock * i) * g.sn);
    const uint32_t orow = static_cast<uint32_t>(qrow * g.sn * sizeof(T));
    const int64_t dbg0 = (static_cast<int64_t>(bh) * g.N + kBlock * i) * D;
    const uint32_t drow = static_cast<uint32_t>(qrow * D * 4);
#pragma unroll
    for (int u = 0; u < DTH; ++u)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int dim0 = 32 * (own0 + u) + 8 * r4 + 4 * hh;
        float ov[4], sv[4], lv[4];
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          sv[x] = o_own[u][4 * r4 + x];
          lv[x] = ol[u][4 * r4 + x];
          ov[x] = kPisa ? sv[x] + lv[x] : al * sv[x] + (1.0f - al) * lv[x];
        }
        store4(reinterpret_cast<T*>(obase + orow + dim0 * sizeof(T)), ov);
        if (o_sparse) store4(reinterpret_cast<float*>(reinterpret_cast<char*>(o_sparse + dbg0) + drow + dim0 * 4), sv);
        if (o_linear) store4(reinterpret_cast<float*>(reinterpret_cast<char*>(o_linear + dbg0) + drow + dim0 * 4), lv);
      }
  }
}


}  // namespace sla
