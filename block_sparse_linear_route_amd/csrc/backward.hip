// Backward pass of the sparse-linear attention forward.
//
// [SLA abstract] the fused kernel serves both the forward and the backward
// pass (the method is fine-tuned).  With the block index lists fixed (the
// router's hard top-k has no gradient), the forward is
//   O = alpha O_s + (1 - alpha) O_l          [SLA2 summary, section 2.A]
//   O_s = softmax over the critical keys of q k^T / sqrt(d), times V
//   O_l = phi(q) S_i / (phi(q) . sigma_i), S_i = sum_{j in M_i} H_j,
//   H_j = phi(K_j)^T V_j, z_j = colsum phi(K_j), phi = softmax over features,
// and its gradients follow by the chain rule (the same steps the CPU
// reference writes out):
//   dalpha = sum dO * (O_s - O_l); dO_s = alpha dO; dO_l = (1 - alpha) dO;
//   sparse: D_t = dO_s . O_s, P from the saved log2 normaliser,
//           dS = P * (dP - D_t), dQ = dS K / sqrt(d), dK = dS^T Q / sqrt(d),
//           dV = P^T dO_s;
//   linear: dnum = dO_l / den, dden = -(dO_l . O_l) / den,
//           df = dnum S_i^T + dden sigma_i, dq = phi-backward(df);
//           dS_i = f^T dnum, dsigma_i = f^T dden; dH_j = sum over the query
//           blocks that hold j of dS_i (the mask product, transposed),
//           dz_j likewise; dphi(k_n) = dH_j v_n + dz_j, dv_n += phi(k_n) dH_j,
//           dk = phi-backward(dphi).
//
// Kernels (one launch each, in this order, after the forward has written
// O_s, O_l and the log2 normaliser into the workspace):
//   bwd_rowdot_kernel   D_t = alpha dO . O_s and dO . O_l per row (the
//                       linear query side reads the latter); per-block
//                       partial sums of dO . (O_s - O_l) for dalpha;
//   bwd_dq_kernel       query-major: the critical blocks of query block i
//                       through the same LDS ring as the forward; S^T, dP^T
//                       and dQ^T += K^T dS^T on the matrix cores (K^T by
//                       transposing LDS reads, dS^T fed from registers);
//   bwd_lin_q_kernel    the linear branch on the query side: dq (added),
//                       dS_i (bf16, value-major like H) with dsigma_i after
//                       it in the same row;
//   bwd_bits_kernel     the transposed critical relation as bit rows per KV
//                       block, and the transposed marginal relation in the
//                       mask-product layout (then dH = M^T dS by that product,
//                       dz riding along as d more columns of each row);
//   bwd_kv_kernel       KV-major (one instance for dV, one for dK): for KV
//                       block j, the query blocks holding j critical (from
//                       its bit row) stream Q and dO tiles through an LDS
//                       ring; dV^T or dK^T accumulates on the matrix cores;
//   bwd_lin_kv_kernel   the linear branch on the KV side (added to dk, dv);
//   bwd_dalpha_kernel   dalpha per head, summed in a fixed order.
// Gradients are float32; every kernel is deterministic (no atomics on
// floating-point data).
#include <algorithm>
#include <type_traits>

#include "attention_epilogue.hpp"

namespace sla {
namespace {

struct BwdArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* dout;
  const int32_t* crit;
  const int32_t* marg;
  const float* alpha;
  const float* o_s;        // float [BH][N][D]
  const float* o_l;        // float [BH][N][D]
  const float* lse;        // float [BH][N], log2 normaliser of the sparse softmax
  float* dd;               // float [BH][N], D_t
  float* dol;              // float [BH][N], dO . O_l per row
  const uint16_t* s_sum;   // bf16 [BH][nq][D][D] value-major (forward workspace)
  const float* sigma;      // float [BH][nq][D]
  uint16_t* ds;            // bf16 [BH][nq][D*D + D]: dS_i value-major, then dsigma_i
  const uint16_t* dh;      // bf16 [BH][nkb][D*D + D]: dH_j value-major, then dz_j
  uint32_t* crit_t;        // [BH][nkb][crit_words]
  int crit_words;
  uint32_t* marg_t;        // mask-product bit layout, rows = KV blocks
  float* dq;               // float [BH][N][D]
  float* dk;
  float* dv;
  float* dalpha_part;      // float [BH][nq]
  float* dalpha;           // float [H]
  Geometry g;
  float c_log2;            // log2(e) / sqrt(d)
};

// 4 bf16 (8 bytes) -> float
__device__ __forceinline__ void load4_f32(const uint16_t* p, float* out) {
  const u32x2 w = *reinterpret_cast<const u32x2*>(p);
  out[0] = __uint_as_float(w[0] << 16);
  out[1] = __uint_as_float(w[0] & 0xffff0000u);
  out[2] = __uint_as_float(w[1] << 16);
  out[3] = __uint_as_float(w[1] & 0xffff0000u);
}

// element offset of (row, col) in a 64- or D-row bf16 tile of D columns
// stored with the 16-byte chunk swizzle swz<D>(row)
template <int D>
__device__ __forceinline__ int tile_off(int row, int col) {
  return row * D + 8 * ((col >> 3) ^ swz<D>(row)) + (col & 7);
}

// Transposing-read offsets (elements, relative to a tile) for the operand
// "feature column 32*ft + lane%32 at rows r0 + 16 s + {4 hh + e, 8 + 4 hh + e}":
// o1 covers the first four rows, o2 the next four; + 16*s*D per k-step.
template <int D>
__device__ __forceinline__ void tr_offsets(int lane, int r0, int ft, int& o1, int& o2) {
  const int hh = lane >> 5, li = lane & 15, ep = li >> 2, q4 = li & 3, gm = (lane >> 4) & 1;
  const int key1 = r0 + 4 * hh + ep;
  const int c = 4 * ft + 2 * gm + (q4 >> 1);
  o1 = key1 * D + 8 * (c ^ swz<D>(key1)) + 4 * (q4 & 1);
  o2 = (key1 + 8) * D + 8 * (c ^ swz<D>(key1 + 8)) + 4 * (q4 & 1);
}

__device__ __forceinline__ bf16x8 tr_operand(const uint16_t* tile, int o1, int o2) {
  const u32x2 x0 = lds_read_tr16(tile + o1);
  const u32x2 x1 = lds_read_tr16(tile + o2);
  u32x4 w;
  w[0] = x0[0]; w[1] = x0[1]; w[2] = x1[0]; w[3] = x1[1];
  return __builtin_bit_cast(bf16x8, w);
}

// ------------------------------------------------------------ row dots
// grid (nq, B*H).  The block's float O_s and O_l rows are read as contiguous
// 1 KB pieces: in pass k thread t takes the 4 values 4 (256 k + t) .. +3 of
// the block, so a row spans D / 4 consecutive lanes and its sums reduce
// across them (rows past the last token are clamped and not written).
template <int D>
__global__ void __launch_bounds__(kThreads)
bwd_rowdot_kernel(BwdArgs A) {
  constexpr int LPR = D / 4;                               // lanes per row
  constexpr int PASSES = kBlock * D / (4 * kThreads);      // rows per thread
  __shared__ float red[4];
  const Geometry& g = A.g;
  const int i = blockIdx.x, bh = blockIdx.y;
  const int b = bh / g.H, h = bh % g.H;
  const int t = threadIdx.x, lane = t & 63;
  const int col = (4 * t) % D;
  const uint16_t* gbase = A.dout + b * g.sb + h * g.sh + col;
  f32x4 sv[PASSES], lv[PASSES];
  float gv[PASSES][4];
  int nrow[PASSES];
#pragma unroll
  for (int k = 0; k < PASSES; ++k) {
    nrow[k] = kBlock * i + (kThreads * k + t) / LPR;
    const int nn = min(nrow[k], g.N - 1);
    const int64_t o = (static_cast<int64_t>(bh) * g.N + nn) * D + col;
    sv[k] = *reinterpret_cast<const f32x4*>(A.o_s + o);
    lv[k] = *reinterpret_cast<const f32x4*>(A.o_l + o);
    load4_f32(gbase + static_cast<int64_t>(nn) * g.sn, gv[k]);
  }
  float da = 0.0f;
  const float al = A.alpha[h];
#pragma unroll
  for (int k = 0; k < PASSES; ++k) {
    float ds = 0.0f, dl = 0.0f, dak = 0.0f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      ds = fmaf(gv[k][e], sv[k][e], ds);
      dl = fmaf(gv[k][e], lv[k][e], dl);
      dak = fmaf(gv[k][e], sv[k][e] - lv[k][e], dak);
    }
    if (nrow[k] < g.N) da += dak;
#pragma unroll
    for (int m = 1; m < LPR; m <<= 1) {
      ds += xor_lane(ds, m);
      dl += xor_lane(dl, m);
    }
    if ((t % LPR) == 0 && nrow[k] < g.N) {
      A.dd[static_cast<int64_t>(bh) * g.N + nrow[k]] = al * ds;
      A.dol[static_cast<int64_t>(bh) * g.N + nrow[k]] = dl;
    }
  }
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) da += xor_lane(da, m);
  if (lane == 0) red[t >> 6] = da;
  __syncthreads();
  if (t == 0) A.dalpha_part[static_cast<int64_t>(bh) * g.nq + i] = (red[0] + red[1]) + (red[2] + red[3]);
}

// ------------------------------------------------------------ sparse dQ
// One workgroup per (b, h, query block i); wave = qh + 2 kh as in the
// forward (qh: 32 of the 64 query rows, kh: 32 of the 64 keys of every
// critical block).  Step it finds K(it), V(it) in stage X = it & 1 of a
// two-stage ring (one __shared__ array per stage and tensor, so reads of one
// stage wait on nothing filling the other) and first sends K(it+1), V(it+1)
// into the other stage.  One operand buffer serves K, then V, then K^T:
// S^T = K Q^T, dP^T = V dO^T, dS^T = P^T (alpha dP^T - D_t), dQ^T += K^T dS^T.
template <int D>
__global__ void __launch_bounds__(kThreads, 2)
bwd_dq_kernel(BwdArgs A) {
  constexpr int CH = D / 8;
  constexpr int TILE = kBlock * D;
  constexpr int RPI = 64 / CH;
  constexpr int IPW = (kBlock / 4) / RPI;
  constexpr int NS = D / 16;
  constexpr int DT = D / 32;
  constexpr int DTH = DT / 2;
  __shared__ __attribute__((aligned(16))) uint16_t k0[TILE], k1[TILE], v0[TILE], v1[TILE];

  const Geometry& g = A.g;
  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int qh = wave & 1, kh = wave >> 1;
  const int l32 = lane & 31, hh = lane >> 5;
  const int total = g.B * g.H * g.nq;
  const int logical = xcd_remap(blockIdx.x, total);
  const int i = logical % g.nq;
  const int bh = logical / g.nq;
  const int b = bh / g.H, h = bh % g.H;
  const int64_t hoff = b * g.sb + h * g.sh;
  const int n_i = min(kBlock, g.N - kBlock * i);
  const float cl = A.c_log2;
  const int64_t sn = g.sn;

  const int32_t* __restrict__ crow = A.crit + (static_cast<int64_t>(bh) * g.nq + i) * g.k_crit;
  const int kc = g.k_crit;
  int cl0 = lane < kc ? list_block(crow[lane], g.nkb) : 0;
  int cl1 = 64 + lane < kc ? list_block(crow[64 + lane], g.nkb) : 0;
  int cbase = 0;
  auto crit_at = [&](int c) -> int {
    const int o = c - cbase;
    return o < 64 ? __builtin_amdgcn_readlane(cl0, o) : __builtin_amdgcn_readlane(cl1, o - 64);
  };

  const int lrow = lane / CH, lslot = lane % CH;
  const uint32_t rowb = static_cast<uint32_t>(sn * 2);
  const uint32_t head_bytes = static_cast<uint32_t>((g.N - 1) * sn * 2 + D * 2);
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(A.k + hoff, head_bytes);
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc(A.v + hoff, head_bytes);
  uint32_t toff[IPW];
#pragma unroll
  for (int u = 0; u < IPW; ++u) {
    const int r = 16 * wave + RPI * u + lrow;
    toff[u] = static_cast<uint32_t>(r) * rowb + static_cast<uint32_t>(16 * (lslot ^ swz<D>(r)));
  }
  auto issue = [&](auto xc, int c) {
    constexpr int X = decltype(xc)::value;
    const uint32_t soff = static_cast<uint32_t>(kBlock * crit_at(c)) * rowb;
    uint16_t* kd = (X ? k1 : k0) + 16 * wave * D;
    uint16_t* vd = (X ? v1 : v0) + 16 * wave * D;
#pragma unroll
    for (int u = 0; u < IPW; ++u) {
      buffer_load_lds16(krs, kd + RPI * u * D, toff[u], soff);
      buffer_load_lds16(vrs, vd + RPI * u * D, toff[u], soff);
    }
  };

  const int krow = 32 * kh + l32;
  int kofs[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) kofs[s] = krow * D + 8 * ((2 * s + hh) ^ swz<D>(krow));
  int to1[DT], to2[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) tr_offsets<D>(lane, 32 * kh, dt, to1[dt], to2[dt]);

  const int qrow = 32 * qh + l32;
  const int qr = min(qrow, n_i - 1);
  bf16x8 qf[NS], gf[NS];
  f32x16 dqacc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) dqacc[dt] = zero16();
  const float al = A.alpha[h];

  wait_vmem();
  if (kc > 0) issue(std::integral_constant<int, 0>(), 0);
  const int64_t rowg = hoff + static_cast<int64_t>(kBlock * i + qr) * sn;
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    qf[s] = load8(A.q + rowg + 16 * s + 8 * hh);
    gf[s] = load8(A.dout + rowg + 16 * s + 8 * hh);
  }
  const int64_t rowt = static_cast<int64_t>(bh) * g.N + kBlock * i + qr;
  const float lse_t = A.lse[rowt];
  const float d_t = A.dd[rowt];

  auto step = [&](auto xc, int it) {
    constexpr int X = decltype(xc)::value;
    wait_vmem();
    __syncthreads();   // K(it), V(it) landed; the other stage's reads are done
    if (it + 1 < kc) issue(std::integral_constant<int, X ^ 1>(), it + 1);
    const uint16_t* kb = X ? k1 : k0;
    const uint16_t* vb = X ? v1 : v0;
    bf16x8 op[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) op[s] = *reinterpret_cast<const bf16x8*>(kb + kofs[s]);
    f32x16 sc = zero16(), dp = zero16();
#pragma unroll
    for (int s = 0; s < NS; ++s) sc = mfma32(op[s], qf[s], sc);
#pragma unroll
    for (int s = 0; s < NS; ++s) op[s] = *reinterpret_cast<const bf16x8*>(vb + kofs[s]);
#pragma unroll
    for (int s = 0; s < NS; ++s) dp = mfma32(op[s], gf[s], dp);
    const int nj = min(kBlock, g.N - kBlock * crit_at(it));
    bf16x8 pb[2];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = 32 * kh + 8 * (r >> 2) + 4 * hh + (r & 3);
      const float p = key < nj ? __builtin_amdgcn_exp2f(fmaf(sc[r], cl, -lse_t)) : 0.0f;
      pb[r >> 3][r & 7] = f32_to_bf16(p * fmaf(al, dp[r], -d_t));
    }
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      dqacc[dt] = mfma32(tr_operand(kb, to1[dt], to2[dt]), pb[0], dqacc[dt]);
      dqacc[dt] = mfma32(tr_operand(kb + 16 * D, to1[dt], to2[dt]), pb[1], dqacc[dt]);
    }
    if (it + 1 - cbase == 64) {
      cbase += 64;
      cl0 = cl1;
      cl1 = cbase + 64 + lane < kc ? list_block(crow[cbase + 64 + lane], g.nkb) : 0;
    }
  };
  for (int it = 0; it < kc; it += 2) {
    step(std::integral_constant<int, 0>(), it);
    if (it + 1 < kc) step(std::integral_constant<int, 1>(), it + 1);
  }
  wait_vmem();
  __syncthreads();

  // merge the key halves: the wave keeps dims [32*own0, +32*DTH) and hands
  // the rest to the wave of the same query half
  // each wave's outgoing half: [DTH][16][64] floats, waves 0-1 in k0, 2-3 in k1
  auto wbuf = [&](int w) -> float* {
    return reinterpret_cast<float*>(w < 2 ? k0 : k1) + (w & 1) * DTH * 16 * 64;
  };
  const int own0 = kh * DTH;
  f32x16 own[DTH];
  float* obuf_out = wbuf(wave);
#pragma unroll
  for (int u = 0; u < DTH; ++u) {
    own[u] = kh ? dqacc[DTH + u] : dqacc[u];
    const f32x16 oth = kh ? dqacc[u] : dqacc[DTH + u];
#pragma unroll
    for (int r = 0; r < 16; ++r) obuf_out[(u * 16 + r) * 64 + lane] = oth[r];
  }
  __syncthreads();
  const int partner = wave ^ 2;
  const float* obuf_in = wbuf(partner);
  const float rs = cl * (1.0f / kLog2e);   // 1 / sqrt(d)
  if (qrow < n_i) {
    float* dst = A.dq + (static_cast<int64_t>(bh) * g.N + kBlock * i + qrow) * D;
#pragma unroll
    for (int u = 0; u < DTH; ++u)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        f32x4 w;
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          const int r = 4 * r4 + x;
          w[x] = (own[u][r] + obuf_in[(u * 16 + r) * 64 + lane]) * rs;
        }
        *reinterpret_cast<f32x4*>(dst + 32 * (own0 + u) + 8 * r4 + 4 * hh) = w;
      }
  }
}

// ------------------------------------------------------------ linear, query side
// One workgroup per (b, h, query block i); wave = qh + 2 ah: qh picks 32
// query rows, ah half of the key features for df and dq.
template <int D>
__global__ void __launch_bounds__(kThreads, 2)
bwd_lin_q_kernel(BwdArgs A) {
  constexpr int CH = D / 8;
  constexpr int RPI = 64 / CH;
  constexpr int NS = D / 16;
  constexpr int DT = D / 32;
  constexpr int DTH = DT / 2;
  constexpr int NTW = DT * DT / 4;                   // dS tiles per wave
  __shared__ __attribute__((aligned(16))) uint16_t stile[D * D];        // S_i^T, rows c
  __shared__ __attribute__((aligned(16))) uint16_t ntile[kBlock * D];   // dnum [t][c]
  __shared__ __attribute__((aligned(16))) uint16_t ftile[kBlock * D];   // f [t][a]
  __shared__ __attribute__((aligned(16))) float sig[D];
  __shared__ float dden_s[kBlock];
  __shared__ float red[4][32];

  const Geometry& g = A.g;
  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int qh = wave & 1, ah = wave >> 1;
  const int l32 = lane & 31, hh = lane >> 5;
  const int i = blockIdx.x, bh = blockIdx.y;
  const int b = bh / g.H, h = bh % g.H;
  const int64_t hoff = b * g.sb + h * g.sh;
  const int n_i = min(kBlock, g.N - kBlock * i);
  const int64_t sn = g.sn;
  const int64_t irow = static_cast<int64_t>(bh) * g.nq + i;

  // S_i^T (D rows of D) and sigma_i into LDS
  {
    const __amdgpu_buffer_rsrc_t srs = make_rsrc(A.s_sum + irow * D * D, D * D * 2);
    const int lrow = lane / CH, lslot = lane % CH;
    constexpr int RPW = D / 4;
#pragma unroll
    for (int u = 0; u < RPW / RPI; ++u) {
      const int r = RPW * wave + RPI * u + lrow;
      buffer_load_lds16(srs, stile + (RPW * wave + RPI * u) * D,
                        static_cast<uint32_t>(r * D * 2 + 16 * (lslot ^ swz<D>(r))), 0u);
    }
    if (wave == 0 && lane < D / 4) {
      const __amdgpu_buffer_rsrc_t sgr = make_rsrc(A.sigma + irow * D, D * 4);
      buffer_load_lds16(sgr, sig, 16u * lane, 0u);
    }
  }

  const int qrow = 32 * qh + l32;
  const bool vrow = qrow < n_i;
  const int qr = min(qrow, n_i - 1);
  const int64_t rowg = hoff + static_cast<int64_t>(kBlock * i + qr) * sn;
  const int64_t rowt = static_cast<int64_t>(bh) * g.N + kBlock * i + qr;
  const float al = A.alpha[h];

  // phi(q): row max and normaliser from the lane's half of the features and
  // its partner's
  float qv[NS][8];
  float qmax = -INFINITY;
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    load8_f32(A.q + rowg + 16 * s + 8 * hh, qv[s]);
#pragma unroll
    for (int e = 0; e < 8; ++e) qmax = fmaxf(qmax, qv[s][e]);
  }
  qmax = fmaxf(qmax, xor_lane(qmax, 32));
  float zp = 0.0f;
#pragma unroll
  for (int s = 0; s < NS; ++s)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      qv[s][e] = __builtin_amdgcn_exp2f((qv[s][e] - qmax) * kLog2e);
      zp += qv[s][e];
    }
  const float zinv = 1.0f / (zp + xor_lane(zp, 32));
  // dO (kept packed, in the k-slot order of the transposing reads: c = 16 s
  // + {4 hh + e, 8 + 4 hh + e}) and the row's dO . O_l (from the row-dot
  // pass), before the barrier so that these loads overlap the S_i^T and
  // sigma_i transfers
  u32x2 graw[NS][2];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const int c0 = 16 * s + 4 * hh;
    graw[s][0] = *reinterpret_cast<const u32x2*>(A.dout + rowg + c0);
    graw[s][1] = *reinterpret_cast<const u32x2*>(A.dout + rowg + c0 + 8);
  }
  const float gdot = A.dol[rowt];
  // q at the df positions (a = 32 at + 8 r4 + 4 hh + x), packed
  u32x2 qraw[DTH][4];
#pragma unroll
  for (int u = 0; u < DTH; ++u)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4)
      qraw[u][r4] = *reinterpret_cast<const u32x2*>(A.q + rowg + 32 * (ah * DTH + u) + 8 * r4 + 4 * hh);
  wait_vmem();
  __syncthreads();
  float dpart = 0.0f;
#pragma unroll
  for (int s = 0; s < NS; ++s)
#pragma unroll
    for (int e = 0; e < 8; ++e) dpart = fmaf(qv[s][e], sig[16 * s + 8 * hh + e], dpart);
  const float den = (dpart + xor_lane(dpart, 32)) * zinv;

  // dO_l / den as the B operand of df^T
  const float cdo = (1.0f - al) / den;
  bf16x8 dn[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    float g0[4], g1[4];
    load4_f32(reinterpret_cast<const uint16_t*>(&graw[s][0]), g0);
    load4_f32(reinterpret_cast<const uint16_t*>(&graw[s][1]), g1);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      dn[s][e] = f32_to_bf16(vrow ? g0[e] * cdo : 0.0f);
      dn[s][4 + e] = f32_to_bf16(vrow ? g1[e] * cdo : 0.0f);
    }
  }
  const float dden = vrow ? -(1.0f - al) * gdot / den : 0.0f;

  // df^T for the key-feature tiles at = ah*DTH + u: S_i rows a (transposing
  // reads of S_i^T) times dn, plus sigma_i[a] dden
  f32x16 df[DTH];
#pragma unroll
  for (int u = 0; u < DTH; ++u) {
    int o1, o2;
    tr_offsets<D>(lane, 0, ah * DTH + u, o1, o2);
    df[u] = zero16();
#pragma unroll
    for (int s = 0; s < NS; ++s) df[u] = mfma32(tr_operand(stile + 16 * s * D, o1, o2), dn[s], df[u]);
  }
  // f at the df positions (a = 32 at + 8 r4 + 4 hh + x), rows sums of df f
  float fv[DTH][16];
  float rsum = 0.0f;
#pragma unroll
  for (int u = 0; u < DTH; ++u)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const int a0 = 32 * (ah * DTH + u) + 8 * r4 + 4 * hh;
      float qa[4];
      load4_f32(reinterpret_cast<const uint16_t*>(&qraw[u][r4]), qa);
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        const int r = 4 * r4 + x;
        fv[u][r] = vrow ? __builtin_amdgcn_exp2f((qa[x] - qmax) * kLog2e) * zinv : 0.0f;
        df[u][r] = fmaf(sig[a0 + x], dden, df[u][r]);
        rsum = fmaf(df[u][r], fv[u][r], rsum);
      }
    }
  rsum += xor_lane(rsum, 32);
  if (hh == 0) red[wave][l32] = rsum;
  // dnum and f rows into LDS for dS_i^T = dnum^T f (rows t = query rows)
  if (ah == 0) {
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int c0 = 16 * s + 4 * hh;
      u32x2 w0, w1;
      const u32x4 w = __builtin_bit_cast(u32x4, dn[s]);
      w0[0] = w[0]; w0[1] = w[1]; w1[0] = w[2]; w1[1] = w[3];
      *reinterpret_cast<u32x2*>(ntile + tile_off<D>(qrow, c0)) = w0;
      *reinterpret_cast<u32x2*>(ntile + tile_off<D>(qrow, c0 + 8)) = w1;
    }
    if (hh == 0) dden_s[qrow] = dden;
  }
#pragma unroll
  for (int u = 0; u < DTH; ++u)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const int a0 = 32 * (ah * DTH + u) + 8 * r4 + 4 * hh;
      float x4[4] = {fv[u][4 * r4], fv[u][4 * r4 + 1], fv[u][4 * r4 + 2], fv[u][4 * r4 + 3]};
      store4(ftile + tile_off<D>(qrow, a0), x4);
    }
  __syncthreads();

  // dq += f (df - rowsum(df f))
  const float tot = rsum + red[wave ^ 2][l32];
  if (vrow) {
    float* dst = A.dq + (static_cast<int64_t>(bh) * g.N + kBlock * i + qrow) * D;
#pragma unroll
    for (int u = 0; u < DTH; ++u)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int a0 = 32 * (ah * DTH + u) + 8 * r4 + 4 * hh;
        f32x4 w = *reinterpret_cast<const f32x4*>(dst + a0);
#pragma unroll
        for (int x = 0; x < 4; ++x) w[x] += fv[u][4 * r4 + x] * (df[u][4 * r4 + x] - tot);
        *reinterpret_cast<f32x4*>(dst + a0) = w;
      }
  }

  // dS_i^T[c][a] = sum_t dnum[t][c] f[t][a]: tiles (ct, at), k = the 64 rows
  uint16_t* dso = A.ds + irow * (D * D + D);
#pragma unroll
  for (int u = 0; u < NTW; ++u) {
    const int ti = wave * NTW + u;
    const int ct = ti / DT, at = ti % DT;
    f32x16 acc = zero16();
#pragma unroll
    for (int s = 0; s < kBlock / 16; ++s) {
      int a1, a2, b1, b2;
      tr_offsets<D>(lane, 0, ct, a1, a2);
      tr_offsets<D>(lane, 0, at, b1, b2);
      acc = mfma32(tr_operand(ntile + 16 * s * D, a1, a2), tr_operand(ftile + 16 * s * D, b1, b2), acc);
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int c = 32 * ct + 8 * (r >> 2) + 4 * hh + (r & 3);
      dso[c * D + 32 * at + l32] = f32_to_bf16_bits(acc[r]);
    }
  }
  // dsigma_i[a] = sum_t f[t][a] dden_t, after dS_i in the same row (the
  // mask product then sums both)
  if (t < D) {
    float acc = 0.0f;
    for (int r = 0; r < kBlock; ++r) acc = fmaf(bf16_to_f32(ftile[tile_off<D>(r, t)]), dden_s[r], acc);
    dso[D * D + t] = f32_to_bf16_bits(acc);
  }
}

// ------------------------------------------------------------ transposed masks
// grid (nq, B*H): query block i sets bit i in the rows of its critical and
// marginal KV blocks (rows zeroed beforehand by bwd_fill_kernel).
__global__ void __launch_bounds__(kThreads)
bwd_bits_kernel(BwdArgs A, int nchunks, int rows_pad) {
  const Geometry& g = A.g;
  const int i = blockIdx.x, bh = blockIdx.y;
  const int64_t irow = static_cast<int64_t>(bh) * g.nq + i;
  const uint32_t bit = 1u << (i & 31);
  for (int u = threadIdx.x; u < g.k_crit; u += kThreads) {
    const int j = list_block(A.crit[irow * g.k_crit + u], g.nkb);
    atomicOr(A.crit_t + (static_cast<int64_t>(bh) * g.nkb + j) * A.crit_words + (i >> 5), bit);
  }
  const int w = i >> 5;
  for (int u = threadIdx.x; u < g.k_marg; u += kThreads) {
    const int j = list_block(A.marg[irow * g.k_marg + u], g.nkb);
    atomicOr(A.marg_t + ((static_cast<int64_t>(bh) * nchunks + (w >> 1)) * rows_pad + j) * 2 + (w & 1), bit);
  }
}

__global__ void __launch_bounds__(kThreads)
bwd_fill_kernel(uint32_t* __restrict__ p, int64_t n) {
  for (int64_t e = blockIdx.x * static_cast<int64_t>(kThreads) + threadIdx.x; e < n;
       e += static_cast<int64_t>(gridDim.x) * kThreads)
    p[e] = 0u;
}

// ------------------------------------------------------------ sparse dK, dV
// The query blocks holding KV block j critical, ascending, from j's bit row
// (returns the count; the list is complete after the caller's next barrier).
__device__ __forceinline__ int bit_row_list(const uint32_t* __restrict__ brow, int W,
                                            uint16_t* qlist, int* wcount) {
  const int t = threadIdx.x;
  uint32_t myword = 0;
  if (t < W) {
    myword = brow[t];
    wcount[t + 1] = __builtin_popcount(myword);
  }
  if (t == 0) wcount[0] = 0;
  __syncthreads();
  if (t == 0)
    for (int w = 1; w <= W; ++w) wcount[w] += wcount[w - 1];
  __syncthreads();
  if (t < W) {
    int pos = wcount[t];
    uint32_t word = myword;
    while (word) {
      qlist[pos++] = static_cast<uint16_t>(32 * t + __builtin_ctz(word));
      word &= word - 1;
    }
  }
  return wcount[W];
}

// One workgroup per (b, h, KV block j); wave = qh + 2 kh: kh picks 32 of the
// block's 64 keys (their K rows, and V rows for dK, stay in registers as B
// operands), qh 32 of the 64 rows of each streamed query block.  The query
// blocks holding j critical stream their Q and dO tiles and the rows' log2
// normaliser and D_t through a two-stage ring (one __shared__ array per
// stage and tensor).  Per block, S = Q K^T on the matrix cores gives P (lane
// = key), which feeds the B operand directly:
//   GRAD_K = false: dV^T += dO^T (alpha P)          (dO^T by transposing reads)
//   GRAD_K = true:  dP = dO V^T, dS = P (alpha dP - D_t), dK^T += Q^T dS
// Two kernels instead of one keep each within 256 registers (two waves per
// SIMD) at the price of computing S twice.
template <int D, bool GRAD_K>
__global__ void __launch_bounds__(kThreads, 2)
bwd_kv_kernel(BwdArgs A) {
  constexpr int CH = D / 8;
  constexpr int TILE = kBlock * D;
  constexpr int RPI = 64 / CH;
  constexpr int IPW = (kBlock / 4) / RPI;
  constexpr int NS = D / 16;
  constexpr int DT = D / 32;
  constexpr int DTH = DT / 2;
  __shared__ __attribute__((aligned(16))) uint16_t q0[TILE], q1[TILE], g0[TILE], g1[TILE];
  __shared__ __attribute__((aligned(16))) float st0[2][kBlock], st1[2][kBlock];   // [lse, D]
  __shared__ uint16_t qlist[4096];
  __shared__ int wcount[129];

  const Geometry& g = A.g;
  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int qh = wave & 1, kh = wave >> 1;
  const int l32 = lane & 31, hh = lane >> 5;
  const int total = g.B * g.H * g.nkb;
  const int logical = xcd_remap(blockIdx.x, total);
  const int j = logical % g.nkb;
  const int bh = logical / g.nkb;
  const int b = bh / g.H, h = bh % g.H;
  const int64_t hoff = b * g.sb + h * g.sh;
  const int nj = min(kBlock, g.N - kBlock * j);
  const float cl = A.c_log2;
  const int64_t sn = g.sn;
  const float al = A.alpha[h];

  const int cnt = bit_row_list(A.crit_t + (static_cast<int64_t>(bh) * g.nkb + j) * A.crit_words,
                               A.crit_words, qlist, wcount);

  const int lrow = lane / CH, lslot = lane % CH;
  const uint32_t rowb = static_cast<uint32_t>(sn * 2);
  const uint32_t head_bytes = static_cast<uint32_t>((g.N - 1) * sn * 2 + D * 2);
  const __amdgpu_buffer_rsrc_t qrs = make_rsrc(A.q + hoff, head_bytes);
  const __amdgpu_buffer_rsrc_t grs = make_rsrc(A.dout + hoff, head_bytes);
  const __amdgpu_buffer_rsrc_t lrs = make_rsrc(A.lse + static_cast<int64_t>(bh) * g.N, g.N * 4);
  const __amdgpu_buffer_rsrc_t drs = make_rsrc(A.dd + static_cast<int64_t>(bh) * g.N, g.N * 4);
  uint32_t toff[IPW];
#pragma unroll
  for (int u = 0; u < IPW; ++u) {
    const int r = 16 * wave + RPI * u + lrow;
    toff[u] = static_cast<uint32_t>(r) * rowb + static_cast<uint32_t>(16 * (lslot ^ swz<D>(r)));
  }
  auto issue = [&](auto xc, int it) {
    constexpr int X = decltype(xc)::value;
    // the list entry is the same in every lane: in a scalar register the
    // buffer loads take it as their scalar offset directly
    const int qi = __builtin_amdgcn_readfirstlane(qlist[it]);
    const uint32_t soff = static_cast<uint32_t>(kBlock * qi) * rowb;
    uint16_t* qd = (X ? q1 : q0) + 16 * wave * D;
    uint16_t* gd = (X ? g1 : g0) + 16 * wave * D;
#pragma unroll
    for (int u = 0; u < IPW; ++u) {
      buffer_load_lds16(qrs, qd + RPI * u * D, toff[u], soff);
      buffer_load_lds16(grs, gd + RPI * u * D, toff[u], soff);
    }
    float* stx = X ? &st1[0][0] : &st0[0][0];
    if (wave == 0 && lane < 16)
      buffer_load_lds16(lrs, stx, 16u * lane, static_cast<uint32_t>(kBlock * qi * 4));
    if (wave == 1 && lane < 16)
      buffer_load_lds16(drs, stx + kBlock, 16u * lane, static_cast<uint32_t>(kBlock * qi * 4));
  };

  // B operands: this wave's keys (rows past the block's end clamped; their
  // columns are masked)
  const int key = 32 * kh + l32;
  const int64_t krowg = hoff + static_cast<int64_t>(kBlock * j + min(key, nj - 1)) * sn;
  bf16x8 kf[NS];
  [[maybe_unused]] bf16x8 vf[GRAD_K ? NS : 1];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    kf[s] = load8(A.k + krowg + 16 * s + 8 * hh);
    if constexpr (GRAD_K) vf[s] = load8(A.v + krowg + 16 * s + 8 * hh);
  }
  const int arow = 32 * qh + l32;
  int aofs[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) aofs[s] = arow * D + 8 * ((2 * s + hh) ^ swz<D>(arow));
  int to1[DT], to2[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) tr_offsets<D>(lane, 32 * qh, dt, to1[dt], to2[dt]);

  f32x16 acc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) acc[dt] = zero16();

  wait_vmem();
  __syncthreads();   // list complete
  if (cnt > 0) issue(std::integral_constant<int, 0>(), 0);

  auto step = [&](auto xc, int it) {
    constexpr int X = decltype(xc)::value;
    wait_vmem();
    __syncthreads();   // block it in LDS; the other stage's reads are done
    if (it + 1 < cnt) issue(std::integral_constant<int, X ^ 1>(), it + 1);
    const uint16_t* qt = X ? q1 : q0;
    const uint16_t* gt = X ? g1 : g0;
    const float* stx = X ? &st1[0][0] : &st0[0][0];
    const int n_q = min(kBlock, g.N - kBlock * __builtin_amdgcn_readfirstlane(qlist[it]));
    // row statistics of the 16 query rows in this lane's registers
    float lse_r[16], d_r[16];
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const int tq = 32 * qh + 8 * r4 + 4 * hh;
      const f32x4 a = *reinterpret_cast<const f32x4*>(stx + tq);
#pragma unroll
      for (int x = 0; x < 4; ++x) lse_r[4 * r4 + x] = a[x];
      if constexpr (GRAD_K) {
        const f32x4 dq4 = *reinterpret_cast<const f32x4*>(stx + kBlock + tq);
#pragma unroll
        for (int x = 0; x < 4; ++x) d_r[4 * r4 + x] = dq4[x];
      }
    }
    bf16x8 op[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) op[s] = *reinterpret_cast<const bf16x8*>(qt + aofs[s]);
    f32x16 sc = zero16();
#pragma unroll
    for (int s = 0; s < NS; ++s) sc = mfma32(op[s], kf[s], sc);
    bf16x8 pb[2];
    if constexpr (GRAD_K) {
#pragma unroll
      for (int s = 0; s < NS; ++s) op[s] = *reinterpret_cast<const bf16x8*>(gt + aofs[s]);
      f32x16 dp = zero16();
#pragma unroll
      for (int s = 0; s < NS; ++s) dp = mfma32(op[s], vf[s], dp);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int tq = 32 * qh + 8 * (r >> 2) + 4 * hh + (r & 3);
        const float p = (tq < n_q && key < nj) ? __builtin_amdgcn_exp2f(fmaf(sc[r], cl, -lse_r[r])) : 0.0f;
        pb[r >> 3][r & 7] = f32_to_bf16(p * fmaf(al, dp[r], -d_r[r]));
      }
    } else {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int tq = 32 * qh + 8 * (r >> 2) + 4 * hh + (r & 3);
        const float p = (tq < n_q && key < nj) ? __builtin_amdgcn_exp2f(fmaf(sc[r], cl, -lse_r[r])) : 0.0f;
        pb[r >> 3][r & 7] = f32_to_bf16(al * p);
      }
    }
    const uint16_t* at = GRAD_K ? qt : gt;     // Q^T for dK, dO^T for dV
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      acc[dt] = mfma32(tr_operand(at, to1[dt], to2[dt]), pb[0], acc[dt]);
      acc[dt] = mfma32(tr_operand(at + 16 * D, to1[dt], to2[dt]), pb[1], acc[dt]);
    }
  };
  for (int it = 0; it < cnt; it += 2) {
    step(std::integral_constant<int, 0>(), it);
    if (it + 1 < cnt) step(std::integral_constant<int, 1>(), it + 1);
  }
  wait_vmem();
  __syncthreads();

  // merge the two query halves: the wave keeps dims [32*own0, +32*DTH) and
  // hands the rest to the wave of the same key half (partner = wave ^ 1;
  // waves 0-1 exchange through q0, waves 2-3 through q1)
  auto wbuf = [&](int w) -> float* {
    return reinterpret_cast<float*>(w < 2 ? q0 : q1) + (w & 1) * DTH * 16 * 64;
  };
  const int own0 = qh * DTH;
  f32x16 own[DTH];
  float* obuf_out = wbuf(wave);
#pragma unroll
  for (int u = 0; u < DTH; ++u) {
    own[u] = qh ? acc[DTH + u] : acc[u];
    const f32x16 oth = qh ? acc[u] : acc[DTH + u];
#pragma unroll
    for (int r = 0; r < 16; ++r) obuf_out[(u * 16 + r) * 64 + lane] = oth[r];
  }
  __syncthreads();
  const float* obuf_in = wbuf(wave ^ 1);
  const float scale = GRAD_K ? cl * (1.0f / kLog2e) : 1.0f;   // dK carries 1 / sqrt(d)
  float* out = GRAD_K ? A.dk : A.dv;
  if (key < nj) {
    const int64_t ro = (static_cast<int64_t>(bh) * g.N + kBlock * j + key) * D;
#pragma unroll
    for (int u = 0; u < DTH; ++u)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        f32x4 w;
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          const int r = 4 * r4 + x;
          w[x] = (own[u][r] + obuf_in[(u * 16 + r) * 64 + lane]) * scale;
        }
        *reinterpret_cast<f32x4*>(out + ro + 32 * (own0 + u) + 8 * r4 + 4 * hh) = w;
      }
  }
}

// ------------------------------------------------------------ linear, KV side
// One workgroup per (b, h, KV block j); wave = nt + 2 fh: nt picks 32 of the
// block's 64 tokens, fh half of the feature (or value) tiles.
template <int D>
__global__ void __launch_bounds__(kThreads, 2)
bwd_lin_kv_kernel(BwdArgs A, int nchunks, int rows_pad) {
  constexpr int CH = D / 8;
  constexpr int RPI = 64 / CH;
  constexpr int NS = D / 16;
  constexpr int DT = D / 32;
  constexpr int DTH = DT / 2;
  constexpr int CW = D / 4;
  __shared__ __attribute__((aligned(16))) uint16_t htile[D * D];       // dH_j^T, rows c
  __shared__ __attribute__((aligned(16))) uint16_t vtile[kBlock * D];  // V_j [n][c]
  __shared__ __attribute__((aligned(16))) uint16_t ptile[kBlock * D];  // phi(K_j) [n][a]
  __shared__ float dz[D];
  __shared__ float kstat[2][kBlock];                                  // row max, 1 / normaliser
  __shared__ float red[4][32];

  const Geometry& g = A.g;
  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int nt = wave & 1, fh = wave >> 1;
  const int l32 = lane & 31, hh = lane >> 5;
  const int j = blockIdx.x, bh = blockIdx.y;
  const int b = bh / g.H, h = bh % g.H;
  const int64_t hoff = b * g.sb + h * g.sh;
  const int nj = min(kBlock, g.N - kBlock * j);
  const int64_t sn = g.sn;

  // dH_j^T into LDS
  {
    const __amdgpu_buffer_rsrc_t hrs =
        make_rsrc(A.dh + (static_cast<int64_t>(bh) * g.nkb + j) * (D * D + D), D * D * 2);
    const int lrow = lane / CH, lslot = lane % CH;
    constexpr int RPW = D / 4;
#pragma unroll
    for (int u = 0; u < RPW / RPI; ++u) {
      const int r = RPW * wave + RPI * u + lrow;
      buffer_load_lds16(hrs, htile + (RPW * wave + RPI * u) * D,
                        static_cast<uint32_t>(r * D * 2 + 16 * (lslot ^ swz<D>(r))), 0u);
    }
  }
  if (t < D) dz[t] = bf16_to_f32(A.dh[(static_cast<int64_t>(bh) * g.nkb + j) * (D * D + D) + D * D + t]);
  // phi(K_j) and V_j as bf16 tiles: 4 threads per token (row = t/4)
  {
    const int row = t >> 2, prt = t & 3;
    const bool valid = row < nj;
    const int64_t off = hoff + static_cast<int64_t>(kBlock * j + min(row, nj - 1)) * sn + prt * CW;
    float kv[CW], vv[CW];
#pragma unroll
    for (int c = 0; c < CW; c += 8) {
      load8_f32(A.k + off + c, kv + c);
      load8_f32(A.v + off + c, vv + c);
    }
    float mx = kv[0];
#pragma unroll
    for (int c = 1; c < CW; ++c) mx = fmaxf(mx, kv[c]);
    mx = fmaxf(mx, dpp_f<0xB1>(mx));
    mx = fmaxf(mx, dpp_f<0x4E>(mx));
    float sum = 0.0f;
#pragma unroll
    for (int c = 0; c < CW; ++c) {
      kv[c] = __builtin_amdgcn_exp2f((kv[c] - mx) * kLog2e);
      sum += kv[c];
    }
    sum += dpp_f<0xB1>(sum);
    sum += dpp_f<0x4E>(sum);
    const float inv = valid ? 1.0f / sum : 0.0f;
#pragma unroll
    for (int c = 0; c < CW; c += 4) {
      float p4[4] = {kv[c] * inv, kv[c + 1] * inv, kv[c + 2] * inv, kv[c + 3] * inv};
      float v4[4] = {valid ? vv[c] : 0.0f, valid ? vv[c + 1] : 0.0f, valid ? vv[c + 2] : 0.0f,
                     valid ? vv[c + 3] : 0.0f};
      store4(ptile + tile_off<D>(row, prt * CW + c), p4);
      store4(vtile + tile_off<D>(row, prt * CW + c), v4);
    }
    if (prt == 0) {
      kstat[0][row] = mx;
      kstat[1][row] = inv;
    }
  }
  wait_vmem();
  __syncthreads();

  // dphi^T[a][n] = sum_c dH_j[a][c] V[n][c] + dz[a]: A = dH rows a
  // (transposing reads of dH_j^T), B = V rows n read in the same k-slot order
  const int nrow = 32 * nt + l32;
  const bool nvalid = nrow < nj;
  f32x16 dphi[DTH];
#pragma unroll
  for (int u = 0; u < DTH; ++u) {
    int o1, o2;
    tr_offsets<D>(lane, 0, fh * DTH + u, o1, o2);
    dphi[u] = zero16();
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int c0 = 16 * s + 4 * hh;
      u32x4 w;
      const u32x2 x0 = *reinterpret_cast<const u32x2*>(vtile + tile_off<D>(nrow, c0));
      const u32x2 x1 = *reinterpret_cast<const u32x2*>(vtile + tile_off<D>(nrow, c0 + 8));
      w[0] = x0[0]; w[1] = x0[1]; w[2] = x1[0]; w[3] = x1[1];
      dphi[u] = mfma32(tr_operand(htile + 16 * s * D, o1, o2), __builtin_bit_cast(bf16x8, w), dphi[u]);
    }
  }
  // phi (float) at the dphi positions, the row sum of dphi * phi
  const int64_t krowg = hoff + static_cast<int64_t>(kBlock * j + min(nrow, nj - 1)) * sn;
  const float kmx = kstat[0][nrow], kinv = kstat[1][nrow];
  float pv[DTH][16];
  float rsum = 0.0f;
#pragma unroll
  for (int u = 0; u < DTH; ++u)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const int a0 = 32 * (fh * DTH + u) + 8 * r4 + 4 * hh;
      float ka[4];
      load4_f32(A.k + krowg + a0, ka);
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        const int r = 4 * r4 + x;
        pv[u][r] = __builtin_amdgcn_exp2f((ka[x] - kmx) * kLog2e) * kinv;
        dphi[u][r] += dz[a0 + x];
        rsum = fmaf(dphi[u][r], pv[u][r], rsum);
      }
    }
  rsum += xor_lane(rsum, 32);
  if (hh == 0) red[wave][l32] = rsum;
  // dv^T[c][n] = sum_a dH_j^T[c][a] phi[n][a]: A = dH^T rows c, B = phi rows n
  f32x16 dvl[DTH];
#pragma unroll
  for (int u = 0; u < DTH; ++u) {
    const int crow = 32 * (fh * DTH + u) + l32;
    dvl[u] = zero16();
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(htile + tile_off<D>(crow, 16 * s + 8 * hh));
      const bf16x8 bq = *reinterpret_cast<const bf16x8*>(ptile + tile_off<D>(nrow, 16 * s + 8 * hh));
      dvl[u] = mfma32(a, bq, dvl[u]);
    }
  }
  __syncthreads();
  const float tot = rsum + red[wave ^ 2][l32];
  if constexpr (D != 128) {
    // (d = 64: the tiles are too small to stage the block; add in place)
    if (nvalid) {
      const int64_t ro = (static_cast<int64_t>(bh) * g.N + kBlock * j + nrow) * D;
#pragma unroll
      for (int u = 0; u < DTH; ++u)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const int a0 = 32 * (fh * DTH + u) + 8 * r4 + 4 * hh;
          f32x4 wk = *reinterpret_cast<const f32x4*>(A.dk + ro + a0);
          f32x4 wv = *reinterpret_cast<const f32x4*>(A.dv + ro + a0);
#pragma unroll
          for (int x = 0; x < 4; ++x) {
            const int r = 4 * r4 + x;
            wk[x] += pv[u][r] * (dphi[u][r] - tot);
            wv[x] += dvl[u][r];
          }
          *reinterpret_cast<f32x4*>(A.dk + ro + a0) = wk;
          *reinterpret_cast<f32x4*>(A.dv + ro + a0) = wv;
        }
    }
    return;
  }
  // d = 128: the contributions to dk and dv go through LDS (the tiles are no
  // longer read): dk's 64 token rows in htile (32 KB), dv's rows 0-31 in
  // vtile and 32-63 in ptile (16 KB each), each row's 16-byte chunks
  // XOR-swizzled by the row.  All threads then add them into dk and dv with
  // contiguous 1 KB reads and writes per instruction, where the register
  // layout would touch 32 B of 32 rows.
  constexpr int CPR = D / 4;                           // 16-byte chunks per row
  float* sk = reinterpret_cast<float*>(htile);
  auto sv_row = [&](int r) -> float* {
    return reinterpret_cast<float*>(r < 32 ? vtile : ptile) + (r & 31) * D;
  };
#pragma unroll
  for (int u = 0; u < DTH; ++u)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const int a0 = 32 * (fh * DTH + u) + 8 * r4 + 4 * hh;
      const int pc = ((a0 >> 2) ^ (nrow & (CPR - 1))) * 4;
      f32x4 wk, wv;
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        const int r = 4 * r4 + x;
        wk[x] = pv[u][r] * (dphi[u][r] - tot);
        wv[x] = dvl[u][r];
      }
      *reinterpret_cast<f32x4*>(sk + nrow * D + pc) = wk;
      *reinterpret_cast<f32x4*>(sv_row(nrow) + pc) = wv;
    }
  __syncthreads();
  const int64_t rb = (static_cast<int64_t>(bh) * g.N + kBlock * j) * D;
#pragma unroll
  for (int k = 0; k < kBlock * CPR / kThreads; ++k) {
    const int e4 = k * kThreads + t;
    const int row = e4 / CPR, c = e4 % CPR;
    if (row < nj) {
      const int pc = (c ^ (row & (CPR - 1))) * 4;
      const f32x4 ak = *reinterpret_cast<const f32x4*>(sk + row * D + pc);
      const f32x4 av = *reinterpret_cast<const f32x4*>(sv_row(row) + pc);
      f32x4* gk = reinterpret_cast<f32x4*>(A.dk + rb + row * D + 4 * c);
      f32x4* gv = reinterpret_cast<f32x4*>(A.dv + rb + row * D + 4 * c);
      f32x4 wk = *gk, wv = *gv;
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        wk[x] += ak[x];
        wv[x] += av[x];
      }
      *gk = wk;
      *gv = wv;
    }
  }
}

// ------------------------------------------------------------ dalpha
// grid (H): sum over batches and query blocks of the per-block partials, in
// a fixed order.
__global__ void __launch_bounds__(kThreads)
bwd_dalpha_kernel(BwdArgs A) {
  __shared__ float red[kThreads];
  const Geometry& g = A.g;
  const int h = blockIdx.x;
  float acc = 0.0f;
  for (int b = 0; b < g.B; ++b)
    for (int i = threadIdx.x; i < g.nq; i += kThreads)
      acc += A.dalpha_part[(static_cast<int64_t>(b) * g.H + h) * g.nq + i];
  red[threadIdx.x] = acc;
  __syncthreads();
  for (int s = kThreads / 2; s > 0; s >>= 1) {
    if (static_cast<int>(threadIdx.x) < s) red[threadIdx.x] += red[threadIdx.x + s];
    __syncthreads();
  }
  if (threadIdx.x == 0) A.dalpha[h] = red[0];
}

template <int D>
hipError_t launch_backward_t(const BwdArgs& a, hipStream_t stream) {
  const Geometry& g = a.g;
  const int bh = g.B * g.H;
  const int nchunks = marginal_chunks(g);
  const int rows_pad = marginal_rows_pad(g);
  hipLaunchKernelGGL((bwd_rowdot_kernel<D>), dim3(g.nq, bh), dim3(kThreads), 0, stream, a);
  hipLaunchKernelGGL((bwd_dq_kernel<D>), dim3(bh * g.nq), dim3(kThreads), 0, stream, a);
  if (g.k_marg > 0)
    hipLaunchKernelGGL((bwd_lin_q_kernel<D>), dim3(g.nq, bh), dim3(kThreads), 0, stream, a);
  const int64_t nct = static_cast<int64_t>(bh) * g.nkb * a.crit_words;
  const int64_t nmt = static_cast<int64_t>(bh) * nchunks * rows_pad * 2;
  hipLaunchKernelGGL(bwd_fill_kernel, dim3(static_cast<unsigned>(std::min<int64_t>((nct + kThreads - 1) / kThreads, 4096))),
                     dim3(kThreads), 0, stream, a.crit_t, nct);
  hipLaunchKernelGGL(bwd_fill_kernel, dim3(static_cast<unsigned>(std::min<int64_t>((nmt + kThreads - 1) / kThreads, 4096))),
                     dim3(kThreads), 0, stream, a.marg_t, nmt);
  hipLaunchKernelGGL(bwd_bits_kernel, dim3(g.nq, bh), dim3(kThreads), 0, stream, a, nchunks, rows_pad);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (g.k_marg > 0) {
    e = launch_mask_gemm(g, a.marg_t, a.ds, const_cast<uint16_t*>(a.dh), stream, true);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((bwd_kv_kernel<D, false>), dim3(bh * g.nkb), dim3(kThreads), 0, stream, a);
  hipLaunchKernelGGL((bwd_kv_kernel<D, true>), dim3(bh * g.nkb), dim3(kThreads), 0, stream, a);
  if (g.k_marg > 0)
    hipLaunchKernelGGL((bwd_lin_kv_kernel<D>), dim3(g.nkb, bh), dim3(kThreads), 0, stream, a,
                       nchunks, rows_pad);
  hipLaunchKernelGGL(bwd_dalpha_kernel, dim3(g.H), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_backward(const Geometry& g, const BackwardBuffers& w, const void* q,
                           const void* k, const void* v, const void* dout, const int32_t* crit,
                           const int32_t* marg, const float* alpha, float* dq, float* dk,
                           float* dv, float* dalpha, hipStream_t stream) {
  BwdArgs a{static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
            static_cast<const uint16_t*>(v), static_cast<const uint16_t*>(dout), crit, marg, alpha,
            w.o_s, w.o_l, w.lse, w.dd, w.dol, w.s_sum, w.sigma, w.ds, w.dh, w.crit_t,
            backward_crit_words(g), w.marg_t, dq, dk, dv, w.dalpha_part, dalpha, g,
            static_cast<float>(1.4426950408889634 / __builtin_sqrt(static_cast<double>(g.D)))};
  if (g.D == 128) return launch_backward_t<128>(a, stream);
  return launch_backward_t<64>(a, stream);
}

}  // namespace sla
