// Fused sparse + linear attention forward (bf16 matrix cores).
//
// [SLA abstract] exact O(N^2) attention on the critical KV blocks, O(N)
// linear attention on the marginal blocks, negligible blocks skipped, all in
// one kernel; [SLA2 technical summary, section 1 item 1] the sparse softmax
// is renormalised over the kept keys; [SLA2 summary, section 2.A equation]
// O = alpha O_s + (1 - alpha) O_l with alpha per head.
//
// One workgroup per (b, h, query block i), 4 waves: wave = qh + 2*kh, where
// qh picks 32 of the 64 query rows and kh picks 32 of the 64 keys of every
// gathered KV block.  Per critical block (one loop iteration):
//   * the block's K tile [64 keys][d] and V^T tile [d][64 keys] sit in LDS
//     (double-buffered: block t+1 is written while block t is consumed, and
//     the global loads for block t+2 are in flight meanwhile);
//   * each wave computes S^T = K Q^T for its 32 keys x 32 queries on
//     v_mfma_f32_32x32x16_bf16, runs the online-softmax update on the S^T
//     registers (query = lane % 32, so a row max is a reduction over the
//     lane's own registers plus the partner lane l ^ 32), and accumulates
//     O^T += V^T P^T with P^T taken straight from the S^T registers;
//   * the V^T tile stores keys in a permuted order (bits 2 and 3 of the key
//     index swapped inside every 16-key group) so that the 8 keys a lane
//     holds in P^T at each 16-key step are 8 consecutive LDS slots.
// The two key halves keep separate running max / sum / output (no per-block
// cross-wave reduction) and are merged once through LDS at the end, each
// wave finalising half of the d output dims.  The linear branch then
// computes O_l^T = S_i^T phi(Q)^T / (phi(Q) . sigma_i) from the
// marginal-state sum S_i precomputed by the marginal-sum kernel (phi(Q)
// uses exp(q - max q); the row normaliser cancels), and the alpha mix is
// stored.
#include "device_common.hpp"
#include "sla_internal.hpp"

namespace sla {
namespace {

struct AttnArgs {
  const void* q;
  const void* k;
  const void* v;
  const int32_t* crit;
  const uint16_t* s_sum;
  const float* sigma_sum;
  const float* alpha;
  void* o;
  float* o_sparse;
  float* o_linear;
  Geometry g;
  float c_log2;      // log2(e) / sqrt(d)
};

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

// LDS slot of key 4*grp .. 4*grp+3 in a V^T row (bits 2 and 3 of the key
// index swapped within each group of 16 keys).
__device__ __forceinline__ int vt_slot(int grp) {
  return 16 * (grp >> 2) + 8 * (grp & 1) + 4 * ((grp >> 1) & 1);
}

template <typename T, int D>
struct Tile {
  static constexpr int CH = D / 8;                 // 8-element chunks per row
  static constexpr int KS = D + 8;                 // K row stride (elements)
  static constexpr int VS = kBlock + 8;            // V^T row stride
  static constexpr int KT = kBlock * KS;           // K tile elements
  static constexpr int VT = D * VS;                // V^T tile elements
  static constexpr int BUF = KT + VT;              // one buffer
  static constexpr int KPT = kBlock * CH / kThreads;       // K chunks per thread
  static constexpr int VSUB = 16 * CH;                      // V 4x8 sub-tiles per block
  static constexpr int VPT = (VSUB + kThreads - 1) / kThreads;
};

template <typename T, int D>
__global__ void __launch_bounds__(kThreads, 2)
attention_kernel(AttnArgs A) {
  using TL = Tile<T, D>;
  constexpr int CH = TL::CH, KS = TL::KS, VS = TL::VS, KT = TL::KT, BUF = TL::BUF;
  constexpr int KPT = TL::KPT, VSUB = TL::VSUB, VPT = TL::VPT;
  constexpr int NS = D / 16;           // 16-wide k-steps over the features
  constexpr int DT = D / 32;           // 32-row tiles over the value dims
  constexpr int DTH = DT / 2;          // tiles each wave finalises
  constexpr int SS = D + 8;            // S^T row stride
  static_assert(KPT >= 1, "tile split");
  static_assert(BUF >= D * SS + 2 * D, "S^T and sigma fit in the second buffer");
  static_assert(BUF * 2 >= 4 * (256 + 4 * DTH * 16 * 64), "merge data fits in the first buffer");
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * BUF];

  const Geometry& g = A.g;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int qh = wave & 1, kh = wave >> 1;
  const int l32 = lane & 31, hh = lane >> 5;

  const int total = g.B * g.H * g.nq;
  const int logical = xcd_remap(blockIdx.x, total);
  const int i = logical % g.nq;
  const int bh = logical / g.nq;
  const int b = bh / g.H, h = bh % g.H;
  const int64_t hoff = b * g.sb + h * g.sh;
  const T* __restrict__ qp = static_cast<const T*>(A.q) + hoff;
  const T* __restrict__ kp = static_cast<const T*>(A.k) + hoff;
  const T* __restrict__ vp = static_cast<const T*>(A.v) + hoff;
  const int n_i = min(kBlock, g.N - kBlock * i);
  const float cl = A.c_log2;
  const int64_t sn = g.sn;

  // Q fragments (B operand of S^T = K Q^T): query 32*qh + l32, features
  // 16*s + 8*hh .. +7.
  bf16x8 qf[NS];
  const int qrow = 32 * qh + l32;
#pragma unroll
  for (int s = 0; s < NS; ++s)
    qf[s] = (qrow < n_i) ? load8(qp + static_cast<int64_t>(kBlock * i + qrow) * sn + 16 * s + 8 * hh)
                         : zero_bf16x8();

  const int32_t* __restrict__ crow = A.crit + (static_cast<int64_t>(bh) * g.nq + i) * g.k_crit;
  const int kc = g.k_crit;

  // staging registers for one block: K chunks and one V 4x8 sub-tile
  bf16x8 kr[KPT];
  bf16x8 vr[VPT][4];

#define SLA_LOAD_BLOCK(c_)                                                              \
  do {                                                                                  \
    const int jb_ = crow[(c_)];                                                         \
    const int nj_ = min(kBlock, g.N - kBlock * jb_);                                    \
    const T* kb_ = kp + static_cast<int64_t>(kBlock * jb_) * sn;                        \
    const T* vb_ = vp + static_cast<int64_t>(kBlock * jb_) * sn;                        \
    _Pragma("unroll") for (int u = 0; u < KPT; ++u) {                                   \
      const int id = t + kThreads * u;                                                  \
      const int row = id / CH, chk = id % CH;                                           \
      kr[u] = (row < nj_) ? load8(kb_ + row * sn + 8 * chk) : zero_bf16x8();            \
    }                                                                                   \
    _Pragma("unroll") for (int u = 0; u < VPT; ++u) {                                   \
      const int id = t + kThreads * u;                                                  \
      const int grp = id % 16, chk = id / 16;                                           \
      _Pragma("unroll") for (int x = 0; x < 4; ++x) {                                   \
        const int row = 4 * grp + x;                                                    \
        vr[u][x] = (id < VSUB && row < nj_) ? load8(vb_ + row * sn + 8 * chk)           \
                                            : zero_bf16x8();                            \
      }                                                                                 \
    }                                                                                   \
  } while (0)

#define SLA_STORE_BLOCK(buf_)                                                           \
  do {                                                                                  \
    uint16_t* kd_ = smem + (buf_) * BUF;                                                \
    uint16_t* vd_ = kd_ + KT;                                                           \
    _Pragma("unroll") for (int u = 0; u < KPT; ++u) {                                   \
      const int id = t + kThreads * u;                                                  \
      const int row = id / CH, chk = id % CH;                                           \
      *reinterpret_cast<bf16x8*>(&kd_[row * KS + 8 * chk]) = kr[u];                     \
    }                                                                                   \
    _Pragma("unroll") for (int u = 0; u < VPT; ++u) {                                   \
      const int id = t + kThreads * u;                                                  \
      if (id < VSUB) {                                                                  \
        const int grp = id % 16, chk = id / 16;                                         \
        const int slot = vt_slot(grp);                                                  \
        _Pragma("unroll") for (int e = 0; e < 8; ++e) {                                 \
          bf16x4 w4;                                                                    \
          w4[0] = vr[u][0][e]; w4[1] = vr[u][1][e];                                     \
          w4[2] = vr[u][2][e]; w4[3] = vr[u][3][e];                                     \
          *reinterpret_cast<bf16x4*>(&vd_[(8 * chk + e) * VS + slot]) = w4;             \
        }                                                                               \
      }                                                                                 \
    }                                                                                   \
  } while (0)

  float m_run = -INFINITY, l_run = 0.0f;
  f32x16 oacc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) oacc[dt] = zero16();

  if (kc > 0) {
    SLA_LOAD_BLOCK(0);
    SLA_STORE_BLOCK(0);
    if (kc > 1) SLA_LOAD_BLOCK(1);
    __syncthreads();
  }
  for (int it = 0; it < kc; ++it) {
    const int buf = it & 1;
    const int jb = crow[it];
    const int nj = min(kBlock, g.N - kBlock * jb);
    const uint16_t* kt = smem + buf * BUF;
    const uint16_t* vt = kt + KT;

    // S^T for keys 32*kh .. +31 and queries 32*qh .. +31
    f32x16 sacc = zero16();
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(&kt[(32 * kh + l32) * KS + 16 * s + 8 * hh]);
      sacc = mfma32(a, qf[s], sacc);
    }
    if (nj < kBlock) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = 32 * kh + 8 * (r >> 2) + 4 * hh + (r & 3);
        if (key >= nj) sacc[r] = -INFINITY;
      }
    }
    float mx = sacc[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, sacc[r]);
    mx = fmaxf(mx, xor_lane(mx, 32));
    const float m_new = fmaxf(m_run, mx);
    const float m_use = (m_new == -INFINITY) ? 0.0f : m_new;   // all keys masked so far
    const float corr = __builtin_amdgcn_exp2f((m_run - m_use) * cl);
    const float mb = m_use * cl;
    float ps = 0.0f;
    bf16x8 pb[2];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float p = __builtin_amdgcn_exp2f(fmaf(sacc[r], cl, -mb));
      ps += p;
      pb[r >> 3][r & 7] = f32_to_bf16(p);
    }
    l_run = l_run * corr + ps;
    m_run = m_new;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[dt][r] *= corr;
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(&vt[(32 * dt + l32) * VS + 32 * kh + 16 * s + 8 * hh]);
        oacc[dt] = mfma32(a, pb[s], oacc[dt]);
      }
    }

    if (it + 1 < kc) {
      SLA_STORE_BLOCK(buf ^ 1);          // block it+1 (its loads were issued last iteration)
      if (it + 2 < kc) SLA_LOAD_BLOCK(it + 2);
    }
    __syncthreads();
  }
#undef SLA_LOAD_BLOCK
#undef SLA_STORE_BLOCK

  // ---- merge the two key halves; stage the linear-branch operands ----
  float* mbuf = reinterpret_cast<float*>(smem);   // [4][32]
  float* lbuf = mbuf + 128;                        // [4][32]
  float* obuf = mbuf + 256;                        // [4][DTH][16][64]
  const float l_full = l_run + xor_lane(l_run, 32);
  if (hh == 0) {
    mbuf[wave * 32 + l32] = m_run;
    lbuf[wave * 32 + l32] = l_full;
  }
  const int own0 = kh * DTH;
  // the wave keeps dims [32*own0, +32*DTH); select with static indices so the
  // accumulators stay in registers
  f32x16 o_own[DTH], o_oth[DTH];
#pragma unroll
  for (int u = 0; u < DTH; ++u) {
    o_own[u] = kh ? oacc[DTH + u] : oacc[u];
    o_oth[u] = kh ? oacc[u] : oacc[DTH + u];
  }
#pragma unroll
  for (int u = 0; u < DTH; ++u)
#pragma unroll
    for (int r = 0; r < 16; ++r) obuf[((wave * DTH + u) * 16 + r) * 64 + lane] = o_oth[u][r];

  const bool has_lin = g.k_marg > 0;
  uint16_t* st = smem + BUF;                                   // S_i^T [D][SS] (second buffer)
  float* sg = reinterpret_cast<float*>(st + D * SS);           // sigma_i [D]
  if (has_lin) {
    const int64_t row = static_cast<int64_t>(bh) * g.nq + i;
    const uint16_t* sgl = A.s_sum + row * D * D;
    for (int e = t; e < (D / 4) * CH; e += kThreads) {
      const int ag = e % (D / 4), bc = e / (D / 4);
      bf16x8 w[4];
#pragma unroll
      for (int x = 0; x < 4; ++x) w[x] = load8(sgl + (4 * ag + x) * D + 8 * bc);
#pragma unroll
      for (int x = 0; x < 8; ++x) {
        bf16x4 p4;
        p4[0] = w[0][x]; p4[1] = w[1][x]; p4[2] = w[2][x]; p4[3] = w[3][x];
        *reinterpret_cast<bf16x4*>(&st[(8 * bc + x) * SS + 4 * ag]) = p4;
      }
    }
    if (t < D) sg[t] = A.sigma_sum[row * D + t];
  }
  __syncthreads();

  const int partner = wave ^ 2;
  const float m_p = mbuf[partner * 32 + l32];
  const float l_p = lbuf[partner * 32 + l32];
  const float m_tot = fmaxf(m_run, m_p);
  const float w_me = (m_run == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f((m_run - m_tot) * cl);
  const float w_p = (m_p == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f((m_p - m_tot) * cl);
  const float den = l_full * w_me + l_p * w_p;
  const float inv = den > 0.0f ? 1.0f / den : 0.0f;
  f32x16 os[DTH];
#pragma unroll
  for (int u = 0; u < DTH; ++u)
#pragma unroll
    for (int r = 0; r < 16; ++r)
      os[u][r] = (o_own[u][r] * w_me + obuf[((partner * DTH + u) * 16 + r) * 64 + lane] * w_p) * inv;

  f32x16 ol[DTH];
#pragma unroll
  for (int u = 0; u < DTH; ++u) ol[u] = zero16();
  if (has_lin) {
    float qmax = -INFINITY;
#pragma unroll
    for (int s = 0; s < NS; ++s)
#pragma unroll
      for (int e = 0; e < 8; ++e) qmax = fmaxf(qmax, bf16v_to_f32(qf[s][e]));
    qmax = fmaxf(qmax, xor_lane(qmax, 32));
    float dpart = 0.0f;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      bf16x8 pf;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const __bf16 pv = f32_to_bf16(__builtin_amdgcn_exp2f((bf16v_to_f32(qf[s][e]) - qmax) * kLog2e));
        pf[e] = pv;
        dpart += bf16v_to_f32(pv) * sg[16 * s + 8 * hh + e];
      }
#pragma unroll
      for (int u = 0; u < DTH; ++u) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(&st[(32 * (own0 + u) + l32) * SS + 16 * s + 8 * hh]);
        ol[u] = mfma32(a, pf, ol[u]);
      }
    }
    const float dsum = dpart + xor_lane(dpart, 32);
    const float dinv = 1.0f / dsum;
#pragma unroll
    for (int u = 0; u < DTH; ++u)
#pragma unroll
      for (int r = 0; r < 16; ++r) ol[u][r] *= dinv;
  }

  // ---- alpha mix and store ----
  const float al = A.alpha[h];
  if (qrow < n_i) {
    const int tok = kBlock * i + qrow;
    T* orow = static_cast<T*>(A.o) + hoff + static_cast<int64_t>(tok) * sn;
    const int64_t dbg = (static_cast<int64_t>(bh) * g.N + tok) * D;
#pragma unroll
    for (int u = 0; u < DTH; ++u)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int dim0 = 32 * (own0 + u) + 8 * r4 + 4 * hh;
        float ov[4], sv[4], lv[4];
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          sv[x] = os[u][4 * r4 + x];
          lv[x] = ol[u][4 * r4 + x];
          ov[x] = al * sv[x] + (1.0f - al) * lv[x];
        }
        store4(orow + dim0, ov);
        if (A.o_sparse) store4(A.o_sparse + dbg + dim0, sv);
        if (A.o_linear) store4(A.o_linear + dbg + dim0, lv);
      }
  }
}

template <typename T, int D>
void launch_attn_t(const AttnArgs& a, hipStream_t stream) {
  const int total = a.g.B * a.g.H * a.g.nq;
  hipLaunchKernelGGL((attention_kernel<T, D>), dim3(total), dim3(kThreads), 0, stream, a);
}

}  // namespace

hipError_t launch_attention(const Geometry& g, const void* q, const void* k, const void* v,
                            const int32_t* crit, const uint16_t* s_sum, const float* sigma_sum,
                            const float* alpha, void* o, float* o_sparse, float* o_linear,
                            hipStream_t stream) {
  AttnArgs a{q, k, v, crit, s_sum, sigma_sum, alpha, o, o_sparse, o_linear, g,
             static_cast<float>(1.4426950408889634 / __builtin_sqrt(static_cast<double>(g.D)))};
  if (g.dtype == 1) {
    if (g.D == 128) launch_attn_t<uint16_t, 128>(a, stream);
    else launch_attn_t<uint16_t, 64>(a, stream);
  } else {
    if (g.D == 128) launch_attn_t<float, 128>(a, stream);
    else launch_attn_t<float, 64>(a, stream);
  }
  return hipGetLastError();
}

}  // namespace sla
