// Fused sparse + linear attention forward (bf16 matrix cores).
//
// [SLA abstract] exact O(N^2) attention on the critical KV blocks, O(N)
// linear attention on the marginal blocks, negligible blocks skipped, all in
// one kernel; [SLA2 technical summary, section 1 item 1] the sparse softmax
// is renormalised over the kept keys; [SLA2 summary, section 2.A equation]
// O = alpha O_s + (1 - alpha) O_l with alpha per head.
//
// One workgroup per (b, h, query block i), 4 waves:
//   wave = qh + 2*kh; qh picks 32 of the 64 query rows, kh picks the stream
//   of critical blocks c = kh, kh+2, kh+4, ... of the query block's list.
// Each iteration stages two gathered KV blocks (one per stream) in LDS:
//   K tile [64 keys][d] row-major (row padded by 16 bytes), and
//   V^T tile [d][64 keys] with the key order permuted to match the P
//   operand that comes straight out of the S^T accumulator registers.
// Per wave and block: S^T = K Q^T (keys x queries, 32x32x16 bf16 MFMA),
// online softmax on the S^T registers (row max across the lane pair l,
// l^32), then O^T += V^T P^T.  The two streams are merged through LDS at
// the end (each wave finalises half of the d output dims), then the linear
// branch O_l^T = S_i^T phi(Q)^T / (phi(Q) . sigma_i) uses the marginal-state
// sum S_i precomputed by the marginal-sum kernel, and the mixed output is
// written.  phi(Q) uses exp(q - max q) without its row normaliser, which
// cancels between the linear branch's numerator and denominator.
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

// Key slot of the V^T tile for key 4*grp + x: within each group of 16 keys,
// bits 2 and 3 of the key index are swapped, so that the 8 keys a lane's
// P^T operand covers at each 16-key step are 8 consecutive slots.
__device__ __forceinline__ int vt_slot(int grp) {
  return 16 * (grp >> 2) + 8 * (grp & 1) + 4 * ((grp >> 1) & 1);
}

template <typename T, int D>
__global__ void __launch_bounds__(kThreads, 2)
attention_kernel(AttnArgs A) {
  constexpr int KS = D + 8;            // K tile row stride (elements)
  constexpr int VS = kBlock + 8;       // V^T tile row stride
  constexpr int KT = kBlock * KS;      // elements per K tile
  constexpr int VT = D * VS;           // elements per V^T tile
  constexpr int NS = D / 16;           // 16-wide k-steps over the features
  constexpr int DT = D / 32;           // 32-row tiles over the value dims
  constexpr int DTH = DT / 2;          // tiles each wave finalises
  constexpr int CH = D / 8;            // 8-element chunks per row
  constexpr int KPT = 2 * kBlock * CH / kThreads;   // K chunks per thread
  constexpr int VPT = 2 * 16 * CH / kThreads;       // V 4x8 sub-tiles per thread
  constexpr int SS = D + 8;            // S^T row stride
  static_assert(KPT >= 1 && VPT >= 1, "tile split");
  static_assert(2 * VT >= D * SS + D * 2, "S^T and sigma fit in the V region");
  static_assert(2 * KT * 2 >= 4 * (256 + 4 * DTH * 16 * 64), "merge buffer fits in the K region");
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * KT + 2 * VT];

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
  const T* qp = static_cast<const T*>(A.q) + hoff;
  const T* kp = static_cast<const T*>(A.k) + hoff;
  const T* vp = static_cast<const T*>(A.v) + hoff;
  const int n_i = min(kBlock, g.N - kBlock * i);
  const float cl = A.c_log2;

  // Q fragments (B operand of S^T = K Q^T): query 32*qh + l32, features
  // 16*s + 8*hh .. +7.
  bf16x8 qf[NS];
  const int qrow = 32 * qh + l32;
  if (qrow < n_i) {
#pragma unroll
    for (int s = 0; s < NS; ++s)
      qf[s] = load8(qp + static_cast<int64_t>(kBlock * i + qrow) * g.sn + 16 * s + 8 * hh);
  } else {
#pragma unroll
    for (int s = 0; s < NS; ++s) qf[s] = zero_bf16x8();
  }

  uint16_t* kbuf = smem;
  uint16_t* vbuf = smem + 2 * KT;
  const int32_t* crow = A.crit + (static_cast<int64_t>(bh) * g.nq + i) * g.k_crit;
  const int kc = g.k_crit;
  const int iters = (kc + 1) / 2;

  bf16x8 kreg[KPT];
  bf16x8 vreg[VPT][4];
  auto load_regs = [&](int it) {
#pragma unroll
    for (int u = 0; u < KPT; ++u) {
      const int id = t + kThreads * u;
      const int kb = id / (kBlock * CH);
      const int rem = id % (kBlock * CH);
      const int row = rem / CH, chk = rem % CH;
      const int c = 2 * it + kb;
      kreg[u] = zero_bf16x8();
      if (c < kc) {
        const int j = crow[c];
        if (row < g.N - kBlock * j)
          kreg[u] = load8(kp + static_cast<int64_t>(kBlock * j + row) * g.sn + 8 * chk);
      }
    }
#pragma unroll
    for (int u = 0; u < VPT; ++u) {
      const int id = t + kThreads * u;
      const int kb = id / (16 * CH);
      const int rem = id % (16 * CH);
      const int grp = rem / CH, chk = rem % CH;
      const int c = 2 * it + kb;
      const int j = (c < kc) ? crow[c] : 0;
      const int nj = (c < kc) ? min(kBlock, g.N - kBlock * j) : 0;
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        const int row = 4 * grp + x;
        vreg[u][x] = (row < nj)
                         ? load8(vp + static_cast<int64_t>(kBlock * j + row) * g.sn + 8 * chk)
                         : zero_bf16x8();
      }
    }
  };
  auto store_lds = [&]() {
#pragma unroll
    for (int u = 0; u < KPT; ++u) {
      const int id = t + kThreads * u;
      const int kb = id / (kBlock * CH);
      const int rem = id % (kBlock * CH);
      const int row = rem / CH, chk = rem % CH;
      *reinterpret_cast<bf16x8*>(&kbuf[kb * KT + row * KS + 8 * chk]) = kreg[u];
    }
#pragma unroll
    for (int u = 0; u < VPT; ++u) {
      const int id = t + kThreads * u;
      const int kb = id / (16 * CH);
      const int rem = id % (16 * CH);
      const int grp = rem / CH, chk = rem % CH;
      const int slot = vt_slot(grp);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        bf16x4 w;
        w[0] = vreg[u][0][e]; w[1] = vreg[u][1][e]; w[2] = vreg[u][2][e]; w[3] = vreg[u][3][e];
        *reinterpret_cast<bf16x4*>(&vbuf[kb * VT + (8 * chk + e) * VS + slot]) = w;
      }
    }
  };

  float m_run = -INFINITY, l_run = 0.0f;
  f32x16 oacc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) oacc[dt] = zero16();

  if (iters > 0) load_regs(0);
  for (int it = 0; it < iters; ++it) {
    __syncthreads();
    store_lds();
    __syncthreads();
    if (it + 1 < iters) load_regs(it + 1);
    const int c = 2 * it + kh;
    if (c < kc) {
      const int j = crow[c];
      const int nj = min(kBlock, g.N - kBlock * j);
      const uint16_t* kt = kbuf + kh * KT;
      const uint16_t* vt = vbuf + kh * VT;
      f32x16 sacc[2];
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        sacc[mt] = zero16();
#pragma unroll
        for (int s = 0; s < NS; ++s) {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(&kt[(32 * mt + l32) * KS + 16 * s + 8 * hh]);
          sacc[mt] = mfma32(a, qf[s], sacc[mt]);
        }
      }
      if (nj < kBlock) {
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = 32 * mt + 8 * (r >> 2) + 4 * hh + (r & 3);
            if (key >= nj) sacc[mt][r] = -INFINITY;
          }
      }
      float mx = -INFINITY;
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[mt][r]);
      mx = fmaxf(mx, xor_lane(mx, 32));
      const float m_new = fmaxf(m_run, mx);
      const float corr = exp2f((m_run - m_new) * cl);
      const float mb = m_new * cl;
      float ps = 0.0f;
      bf16x8 pb[4];
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = exp2f(fmaf(sacc[mt][r], cl, -mb));
          ps += p;
          pb[2 * mt + (r >> 3)][r & 7] = f32_to_bf16(p);
        }
      l_run = l_run * corr + ps;
      m_run = m_new;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[dt][r] *= corr;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(&vt[(32 * dt + l32) * VS + 16 * s + 8 * hh]);
          oacc[dt] = mfma32(a, pb[s], oacc[dt]);
        }
      }
    }
  }

  // ---- merge the two block streams; stage the linear-branch operands ----
  __syncthreads();
  float* mbuf = reinterpret_cast<float*>(smem);   // [4][32]
  float* lbuf = mbuf + 128;                        // [4][32]
  float* obuf = mbuf + 256;                        // [4][DTH][16][64]
  const float l_full = l_run + xor_lane(l_run, 32);
  if (hh == 0) {
    mbuf[wave * 32 + l32] = m_run;
    lbuf[wave * 32 + l32] = l_full;
  }
  const int own0 = kh * DTH, oth0 = (1 - kh) * DTH;
#pragma unroll
  for (int u = 0; u < DTH; ++u)
#pragma unroll
    for (int r = 0; r < 16; ++r) obuf[((wave * DTH + u) * 16 + r) * 64 + lane] = oacc[oth0 + u][r];

  const bool has_lin = g.k_marg > 0;
  uint16_t* st = vbuf;                                         // S_i^T [D][SS]
  float* sg = reinterpret_cast<float*>(vbuf + D * SS);         // sigma_i [D]
  if (has_lin) {
    const int64_t row = static_cast<int64_t>(bh) * g.nq + i;
    const uint16_t* sgl = A.s_sum + row * D * D;
    for (int e = t; e < (D / 4) * CH; e += kThreads) {
      const int ag = e / CH, bc = e % CH;
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
  const float w_me = (m_run == -INFINITY) ? 0.0f : exp2f((m_run - m_tot) * cl);
  const float w_p = (m_p == -INFINITY) ? 0.0f : exp2f((m_p - m_tot) * cl);
  const float den = l_full * w_me + l_p * w_p;
  const float inv = den > 0.0f ? 1.0f / den : 0.0f;
  f32x16 os[DTH];
#pragma unroll
  for (int u = 0; u < DTH; ++u)
#pragma unroll
    for (int r = 0; r < 16; ++r)
      os[u][r] = (oacc[own0 + u][r] * w_me + obuf[((partner * DTH + u) * 16 + r) * 64 + lane] * w_p) * inv;

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
    bf16x8 pf[NS];
    float dpart = 0.0f;
#pragma unroll
    for (int s = 0; s < NS; ++s)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const __bf16 pv = f32_to_bf16(exp2f((bf16v_to_f32(qf[s][e]) - qmax) * kLog2e));
        pf[s][e] = pv;
        dpart += bf16v_to_f32(pv) * sg[16 * s + 8 * hh + e];
      }
    const float dsum = dpart + xor_lane(dpart, 32);
#pragma unroll
    for (int u = 0; u < DTH; ++u) {
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(&st[(32 * (own0 + u) + l32) * SS + 16 * s + 8 * hh]);
        ol[u] = mfma32(a, pf[s], ol[u]);
      }
    }
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
    T* orow = static_cast<T*>(A.o) + hoff + static_cast<int64_t>(tok) * g.sn;
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
