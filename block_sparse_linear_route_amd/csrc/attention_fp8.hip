// Fused sparse + linear attention forward with the sparse branch on fp8
// matrix cores.
//
// [SLA2 technical summary, section 2.C] the sparse branch runs in a low-bit
// format.  Q, K and V arrive as OCP E4M3 codes with one float32 scale per
// (b, h, 64-token block) (the per-block quantiser); the linear branch and the
// alpha mix stay in bf16 / float32 and share the epilogue of the bf16 kernel.
//
// One workgroup per (b, h, query block i), 4 waves: wave = qh + 2*lh.  qh
// picks 32 of the 64 query rows; lh picks one half of the critical list
// (list positions lh, lh + 2, lh + 4, ...), so every wave covers all 64 keys
// of its blocks and the PV product contracts over 64 keys, the depth of
// v_mfma_scale_f32_32x32x64_f8f6f4.  Per block of a half:
//   * S^T = K^ Q^T on the fp8 matrix cores (2 key tiles x 2 feature chunks),
//     scaled to log2 units by s_q * s_k * log2(e) / sqrt(d) on the VALU;
//   * online softmax on the S^T registers (query = lane % 32);
//   * P is quantised per (query row, block): its entries times s_v are scaled
//     by a power of two 2^k that puts the row's largest one in (224, 448],
//     converted to E4M3 (round to nearest even), and O^T += V^T P^T runs with
//     the matrix core's per-column E8M0 scale 2^-k, so the accumulator holds
//     sum_j P_true v_j in float32 with no extra VALU pass;
//   * the running row sum is taken from the float32 values before
//     quantisation.
// K^ and V^ tiles (64 rows x 128 bytes) reach LDS by direct global->LDS
// loads, double-buffered per half; the V^T operand is read from the
// row-major V^ tile with ds_read_b64_tr_b8.
#include "attention_epilogue.hpp"

namespace sla {
namespace {

struct AttnFp8Args {
  const uint16_t* q;
  const uint8_t* q8;
  const float* q_s;
  const uint8_t* k8;
  const float* k_s;
  const uint8_t* v8;
  const float* v_s;
  const int32_t* crit;
  const uint16_t* s_sum;
  const float* sigma_sum;
  const float* alpha;
  void* o;
  float* o_sparse;
  float* o_linear;
  Geometry g;
  float c_log2;      // log2(e) / sqrt(d)
  float* lse;        // LSE: log2 normaliser of the sparse softmax per row
};

// XOR swizzle of the 16-byte chunks of a 128-byte fp8 tile row.  With
// m = (r >> 1) & 7 and its bits 0 and 1 swapped, both the K^ operand reads
// (16 consecutive rows, one chunk, ds_read_b128) and the transposing V^ reads
// (rows {0..3, 8..11} + 4g, two chunks, ds_read_b64_tr_b8) hit distinct banks.
__device__ __forceinline__ int swz8(int r) {
  const int m = (r >> 1) & 7;
  return ((m >> 1) & 1) | ((m & 1) << 1) | (m & 4);
}

__device__ __forceinline__ f32x16 mfma_fp8(i32x8 a, i32x8 b, f32x16 c, int scale_b) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, scale_b);
}

__device__ __forceinline__ float readlane_f(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}

__device__ __forceinline__ i32x8 load32b(const uint8_t* p) {
  const u32x4 a = *reinterpret_cast<const u32x4*>(p);
  const u32x4 b = *reinterpret_cast<const u32x4*>(p + 16);
  i32x8 r;
#pragma unroll
  for (int x = 0; x < 4; ++x) { r[x] = static_cast<int>(a[x]); r[4 + x] = static_cast<int>(b[x]); }
  return r;
}

// LSE: also write each row's log2 sparse-softmax normaliser (for a bf16
// backward pass that rebuilds P from the unquantised scores).
template <bool LSE>
__global__ void __launch_bounds__(kThreads, 2)
attention_fp8_kernel(AttnFp8Args A) {
  constexpr int D = 128;
  constexpr int NS = D / 16;
  constexpr int DT = D / 32;
  constexpr int TB = kBlock * D;               // bytes per fp8 tile
  // LDS: the K buffers of both list halves [0, 4 TB), then their V buffers
  // [4 TB, 8 TB); the epilogue's merge buffers start at the V buffers and
  // sigma_i sits past them.
  constexpr int VREG = 4 * TB;
  constexpr int EPI_BYTES = epilogue_smem_bytes<D>();
  constexpr int SIG_OFF = VREG + EPI_BYTES;
  constexpr int SMEM_BYTES = SIG_OFF + D * 4;
  static_assert(SIG_OFF >= 8 * TB, "sigma_i must lie past the ring");
  constexpr float kLazy = 8.0f;
  constexpr float kLog2Max = 8.807354922057604f;   // log2(448)
  __shared__ __attribute__((aligned(16))) unsigned char smem_raw[SMEM_BYTES];
  const uint16_t* smem_u16 = reinterpret_cast<const uint16_t*>(smem_raw);
  float* sig_lds = reinterpret_cast<float*>(smem_raw + SIG_OFF);

  const Geometry& g = A.g;
  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);   // wave-uniform (scalar)
  const int qh = wave & 1, lh = wave >> 1;
  const int l32 = lane & 31, hh = lane >> 5;

  const int total = g.B * g.H * g.nq;
  const int logical = xcd_remap(blockIdx.x, total);
  const int i = logical % g.nq;
  const int bh = logical / g.nq;
  const int b = bh / g.H, h = bh % g.H;
  const int64_t hoff = b * g.sb + h * g.sh;
  const int n_i = min(kBlock, g.N - kBlock * i);
  const int64_t code_base = static_cast<int64_t>(bh) * g.N * D;
  const uint8_t* __restrict__ k8p = A.k8 + code_base;
  const uint8_t* __restrict__ v8p = A.v8 + code_base;

  // Q^ fragments (B operand of S^T): query 32*qh + l32, feature bytes
  // 64*cc + 32*hh .. +31.  Rows past the last query are clamped (not stored).
  const int qrow = 32 * qh + l32;
  const int qr = qrow < n_i ? qrow : n_i - 1;
  i32x8 qf8[2];
#pragma unroll
  for (int cc = 0; cc < 2; ++cc)
    qf8[cc] = load32b(A.q8 + code_base + static_cast<int64_t>(kBlock * i + qr) * D + 64 * cc + 32 * hh);
  const float sqc = A.q_s[static_cast<int64_t>(bh) * g.nq + i] * A.c_log2;

  // This half's critical blocks and their scales, 64 list entries per
  // register (lane l holds half-list entry base + l); entries are taken with
  // v_readlane so the loop issues no index loads.
  const int32_t* __restrict__ crow = A.crit + (static_cast<int64_t>(bh) * g.nq + i) * g.k_crit;
  const int kc = g.k_crit;
  const int nh = (kc - lh + 1) / 2;            // blocks of this half
  const int nit = (kc + 1) / 2;                // loop trips (all waves)
  const float* __restrict__ ksb = A.k_s + static_cast<int64_t>(bh) * g.nkb;
  const float* __restrict__ vsb = A.v_s + static_cast<int64_t>(bh) * g.nkb;
  int ebase = 0;
  int ej0 = lane < nh ? list_block(crow[lh + 2 * lane], g.nkb) : 0;
  int ej1 = 64 + lane < nh ? list_block(crow[lh + 2 * (64 + lane)], g.nkb) : 0;
  float efb = 0.0f, elv = 0.0f, eiv = 1.0f;    // s_q s_k c, log2 s_v, 1 / s_v
  auto load_scales = [&]() {
    if (ebase + lane < nh) {
      const int jb = ej0;
      const float vs = vsb[jb];
      efb = sqc * ksb[jb];
      elv = __log2f(vs);
      eiv = 1.0f / vs;
    }
  };
  load_scales();
  auto crit_at = [&](int c) -> int {
    const int o = c - ebase;
    return o < 64 ? __builtin_amdgcn_readlane(ej0, o) : __builtin_amdgcn_readlane(ej1, o - 64);
  };

  // LDS ring of a half: K buffers K0, K1 at kbase, V buffers V0, V1 at
  // vbase, 8 KB each.  Wave qh of half lh loads rows 32*qh + 8*u + lane/8 of
  // the half's tiles; lane l writes chunk slot l%8 of its row, which holds
  // global chunk (l%8) ^ swz8(row).
  unsigned char* kbase = smem_raw + lh * 2 * TB;
  unsigned char* vbase = smem_raw + VREG + lh * 2 * TB;
  uint32_t toff[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int r = 32 * qh + 8 * u + (lane >> 3);
    toff[u] = static_cast<uint32_t>(r * D + 16 * ((lane & 7) ^ swz8(r)));
  }
  // Tiles come through a range-checked buffer resource ending at the head's
  // last token, so rows past the end of a short last block read as zeros
  // (their keys are masked to -inf in S, so their P is 0).
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(k8p, static_cast<uint32_t>(g.N) * D);
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc(v8p, static_cast<uint32_t>(g.N) * D);
  auto issue_tile = [&](bool is_k, int c, unsigned char* dst) {
    const int jb = crit_at(c);
    const uint32_t soff = static_cast<uint32_t>(kBlock * jb) * D;
#pragma unroll
    for (int u = 0; u < 4; ++u)
      buffer_load_lds16(is_k ? krs : vrs, dst + (32 * qh + 8 * u) * D, toff[u], soff);
  };

  // K^ operand reads: row 32*tt + l32, chunks 4*cc + 2*hh + {0, 1}
  const int ksw = swz8(l32);
  uint32_t kofs[2][2];
#pragma unroll
  for (int cc = 0; cc < 2; ++cc)
#pragma unroll
    for (int x = 0; x < 2; ++x)
      kofs[cc][x] = static_cast<uint32_t>(l32 * D + 16 * ((4 * cc + 2 * hh + x) ^ ksw));
  auto qk = [&](const unsigned char* kt, f32x16 (&s)[2]) {
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      i32x8 kf[2];
#pragma unroll
      for (int cc = 0; cc < 2; ++cc) {
        const u32x4 a = *reinterpret_cast<const u32x4*>(kt + tt * 32 * D + kofs[cc][0]);
        const u32x4 c2 = *reinterpret_cast<const u32x4*>(kt + tt * 32 * D + kofs[cc][1]);
#pragma unroll
        for (int x = 0; x < 4; ++x) { kf[cc][x] = static_cast<int>(a[x]); kf[cc][4 + x] = static_cast<int>(c2[x]); }
      }
      f32x16 acc = zero16();
      acc = mfma_fp8(kf[0], qf8[0], acc, 127);
      acc = mfma_fp8(kf[1], qf8[1], acc, 127);
      s[tt] = acc;
    }
  };

  // Transposing V^ reads (ds_read_b64_tr_b8): within each 16-lane group
  // (G = lane / 16, g = G / 2 = hh, h = G % 2), output lane i receives byte
  // i % 8 of the 8-byte segments addressed by lanes 2e + i / 8, e = 0..7.
  // Source lane j addresses key 16*rho + 8*(e/4) + 4*g + e%4 (e = j / 2) at
  // feature bytes 32*dt + 16*h + 8*(j%2), so output lane l gets feature
  // 32*dt + l%32 at the keys whose P^T bytes it pairs with: byte 8*rho + e
  // <-> key 16*rho + 8*(e/4) + 4*g + e%4, the S^T register order below.
  uint32_t vofs[DT];
  {
    const int hgrp = (lane >> 4) & 1, j = lane & 15, e = j >> 1;
    const int row0 = 8 * (e >> 2) + 4 * hh + (e & 3);
    const int vsw = swz8(row0);                  // rows row0 + 16*rho share it
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
      vofs[dt] = static_cast<uint32_t>(row0 * D + 16 * ((2 * dt + hgrp) ^ vsw) + 8 * (j & 1));
  }

  float m_run = -INFINITY, l_run = 0.0f;       // log2 units
  i32x8 ones8;                                   // e4m3 1.0 in every byte
#pragma unroll
  for (int w = 0; w < 8; ++w) ones8[w] = 0x38383838;
  f32x16 oacc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) oacc[dt] = zero16();

  // Epilogue operands prefetched into LDS while the last blocks compute, so
  // the epilogue waits on no HBM load: sigma_i at the start; the value-major
  // S_i^T half this list half finalises (rows 64*lh .. +63, a swizzled
  // 64 x D bf16 tile) into the half's two K buffers as each falls free
  // (K[c] takes rows 32c .. +31; K[(nh-2)&1] is free from step nh-2 on and
  // K[(nh-1)&1] from step nh-1); bf16 Q rows 32*lh .. +31 into the half's
  // V buffer that is free in its last step (V[(nh-2)&1]), with a 16-byte
  // chunk swizzle row & 15.
  const bool has_lin = g.k_marg > 0;
  const __amdgpu_buffer_rsrc_t srs =
      make_rsrc(A.s_sum + (static_cast<int64_t>(bh) * g.nq + i) * D * D, D * D * 2);
  const uint16_t* __restrict__ qblk = A.q + hoff + static_cast<int64_t>(kBlock * i) * g.sn;
  const __amdgpu_buffer_rsrc_t qrs =
      make_rsrc(qblk, static_cast<uint32_t>(((n_i - 1) * g.sn + D) * 2));
  if (has_lin && wave == 0 && lane < D / 4) {
    const __amdgpu_buffer_rsrc_t sgr =
        make_rsrc(A.sigma_sum + (static_cast<int64_t>(bh) * g.nq + i) * D, D * 4);
    buffer_load_lds16(sgr, sig_lds, 16u * lane, 0u);
  }
  // Lane l of a 1 KB load covers row l/16 (of 4) at chunk slot l%16.  For
  // S_i^T row r = 4m + l/16 the swizzle swz(r) is 4(l/16) + m%4, so the slot
  // holds global chunk (l%16) ^ 4(l/16) ^ (m%4): one lane constant, and the
  // row base goes into the scalar offset.  Q rows use the swizzle row & 15,
  // i.e. chunk (l%16) ^ (l/16) ^ 4(m%4).
  const int lr16 = lane >> 4;
  const uint32_t s_lane = static_cast<uint32_t>(lr16 * D * 2 + 16 * ((lane & 15) ^ (4 * lr16)));
  const uint32_t q_row = static_cast<uint32_t>(lr16 * g.sn * 2);
  const int q_chunk = (lane & 15) ^ lr16;
  auto issue_s_rows = [&](int piece) {
    unsigned char* dst = kbase + piece * TB;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int r0 = 32 * piece + 16 * qh + 4 * u;              // first row of this load
      buffer_load_lds16(srs, dst + (16 * qh + 4 * u) * D * 2, s_lane ^ (16u * u),
                        static_cast<uint32_t>((64 * lh + r0) * D * 2));
    }
  };
  // the V buffer of half h that holds Q rows 32h .. +31 (free in its last step)
  auto q_buf = [&](int nhh) { return nhh >= 1 ? (((nhh - 1) & 1) ^ 1) : 1; };
  auto issue_q_rows = [&]() {
    unsigned char* dst = vbase + q_buf(nh) * TB;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int rb0 = 16 * qh + 4 * u;                           // first buffer row of this load
      buffer_load_lds16(qrs, dst + rb0 * D * 2, q_row + 16u * static_cast<uint32_t>(q_chunk ^ (4 * u)),
                        static_cast<uint32_t>((32 * lh + rb0) * g.sn * 2));
    }
  };
  auto issue_tail = [&](int it) {
    if (nh == 0) {
      if (it == 0) { issue_s_rows(0); issue_s_rows(1); issue_q_rows(); }
      return;
    }
    if (it == nh - 2) issue_s_rows(it & 1);
    if (it == nh - 1) {
      issue_s_rows(it & 1);
      if (nh == 1) issue_s_rows(1);
      issue_q_rows();
    }
  };

  f32x16 s_cur[2];
  s_cur[0] = zero16();
  s_cur[1] = zero16();
  if (nh > 0) {
    issue_tile(true, 0, kbase);
    issue_tile(false, 0, vbase);
    if (nh > 1) issue_tile(true, 1, kbase + TB);
  }
  wait_vmem();
  __syncthreads();
  if (nh > 0) qk(kbase, s_cur);
  __syncthreads();   // every wave has read K0 before the first step refills it

  for (int it = 0; it < nit; ++it) {
    const int cur = it & 1;
    if (has_lin) issue_tail(it);   // into buffers that fell free at the last barrier
    // V^T fragments of this step's block (in LDS since the last barrier):
    // all 16 transposing reads in flight together, one wait, before the
    // tile loads for the next blocks are issued
    u32x2 vr[4 * DT];
    {
      const uint32_t vt_addr = lds_addr(vbase + cur * TB);
      asm volatile(
          "ds_read_b64_tr_b8 %0, %16\n\t"
          "ds_read_b64_tr_b8 %1, %16 offset:2048\n\t"
          "ds_read_b64_tr_b8 %2, %16 offset:4096\n\t"
          "ds_read_b64_tr_b8 %3, %16 offset:6144\n\t"
          "ds_read_b64_tr_b8 %4, %17\n\t"
          "ds_read_b64_tr_b8 %5, %17 offset:2048\n\t"
          "ds_read_b64_tr_b8 %6, %17 offset:4096\n\t"
          "ds_read_b64_tr_b8 %7, %17 offset:6144\n\t"
          "ds_read_b64_tr_b8 %8, %18\n\t"
          "ds_read_b64_tr_b8 %9, %18 offset:2048\n\t"
          "ds_read_b64_tr_b8 %10, %18 offset:4096\n\t"
          "ds_read_b64_tr_b8 %11, %18 offset:6144\n\t"
          "ds_read_b64_tr_b8 %12, %19\n\t"
          "ds_read_b64_tr_b8 %13, %19 offset:2048\n\t"
          "ds_read_b64_tr_b8 %14, %19 offset:4096\n\t"
          "ds_read_b64_tr_b8 %15, %19 offset:6144\n\t"
          "s_waitcnt lgkmcnt(0)"
          : "=&v"(vr[0]), "=&v"(vr[1]), "=&v"(vr[2]), "=&v"(vr[3]), "=&v"(vr[4]), "=&v"(vr[5]),
            "=&v"(vr[6]), "=&v"(vr[7]), "=&v"(vr[8]), "=&v"(vr[9]), "=&v"(vr[10]), "=&v"(vr[11]),
            "=&v"(vr[12]), "=&v"(vr[13]), "=&v"(vr[14]), "=&v"(vr[15])
          : "v"(vt_addr + vofs[0]), "v"(vt_addr + vofs[1]), "v"(vt_addr + vofs[2]),
            "v"(vt_addr + vofs[3])
          : "memory");
    }
    if (it + 2 < nh) issue_tile(true, it + 2, kbase + cur * TB);
    if (it + 1 < nh) issue_tile(false, it + 1, vbase + (cur ^ 1) * TB);
    // S of the next block (from a stale but in-bounds buffer when this half
    // has no next block; the result is then dropped)
    f32x16 s_next[2];
    qk(kbase + (cur ^ 1) * TB, s_next);

    if (it < nh) {
      const int o = it - ebase;
      const int jb = crit_at(it);
      const int nj = min(kBlock, g.N - kBlock * jb);
      const float fb = readlane_f(efb, o);
      const float lv = readlane_f(elv, o);
      const float iv = readlane_f(eiv, o);
      if (nj < kBlock) {
        // short last block: keys past the end score -inf (p = 0)
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = 32 * tt + 8 * (r >> 2) + 4 * hh + (r & 3);
            if (key >= nj) s_cur[tt][r] = -INFINITY;
          }
      }
      // the scores in log2 units are fb * s with fb > 0, so their maximum is
      // fb times the largest raw score
      const float m0 = max16(s_cur[0]), m1 = max16(s_cur[1]);
      float mx = fb * vmax3(m0, m1, m1);
      {
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx),
                                                         false, false);
        mx = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));   // with lane l ^ 32
      }
      // lazy reference max, as in the bf16 kernel: P_true <= 2^kLazy
      const bool grow = __ballot(mx - m_run > kLazy) != 0ull;
      if (grow) {
        const float m_new = fmaxf(m_run, mx);
        const float corr = __builtin_amdgcn_exp2f(m_run - m_new);
        l_run *= corr;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[dt][r] *= corr;
        m_run = m_new;
      }
      // 2^kq * s_v * max_j P_true lies in (224, 448]
      const float kq = fminf(fmaxf(floorf(kLog2Max - (mx - m_run) - lv), -126.0f), 126.0f);
      const float bias = lv + kq - m_run;
      i32x8 pk;
#pragma unroll
      for (int w = 0; w < 8; ++w) pk[w] = 0;
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int r = 0; r < 16; r += 4) {
          float e[4];
#pragma unroll
          for (int x4 = 0; x4 < 4; ++x4) {
            e[x4] = __builtin_amdgcn_exp2f(fmaf(s_cur[tt][r + x4], fb, bias));
          }
          const int w = 4 * tt + (r >> 2);
          pk[w] = __builtin_amdgcn_cvt_pk_fp8_f32(e[0], e[1], pk[w], false);
          pk[w] = __builtin_amdgcn_cvt_pk_fp8_f32(e[2], e[3], pk[w], true);
        }
      const int scale_b = 127 - static_cast<int>(kq);
      // Row sums of the quantized weights on the matrix core: a ones operand
      // times P^T puts sum_k e_k 2^-kq (this block's 64 keys) in every row
      // of the lane's query column, so both lanes of a query hold the whole
      // sum and each adds half (the epilogue adds the partner lane's l).
      // The normaliser then sums exactly the weights P V uses.
      const f32x16 lsum = mfma_fp8(ones8, pk, zero16(), scale_b);
      l_run = fmaf(lsum[0], 0.5f * iv, l_run);

#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const u32x2 a0 = vr[4 * dt], a1 = vr[4 * dt + 1], a2 = vr[4 * dt + 2], a3 = vr[4 * dt + 3];
        i32x8 vf;
        vf[0] = static_cast<int>(a0[0]); vf[1] = static_cast<int>(a0[1]);
        vf[2] = static_cast<int>(a1[0]); vf[3] = static_cast<int>(a1[1]);
        vf[4] = static_cast<int>(a2[0]); vf[5] = static_cast<int>(a2[1]);
        vf[6] = static_cast<int>(a3[0]); vf[7] = static_cast<int>(a3[1]);
        oacc[dt] = mfma_fp8(vf, pk, oacc[dt], scale_b);
      }
    }
    s_cur[0] = s_next[0];
    s_cur[1] = s_next[1];
    if (it + 1 - ebase == 64) {          // half-list entries it+1 .. now start at register 1
      ebase += 64;
      ej0 = ej1;
      ej1 = ebase + 64 + lane < nh ? list_block(crow[lh + 2 * (ebase + 64 + lane)], g.nkb) : 0;
      load_scales();
    }
    wait_vmem();
    __syncthreads();
  }

  // no critical block (no loop): the epilogue operands go in now
  if (nit == 0) {
    if (has_lin) issue_tail(0);
    wait_vmem();
    __syncthreads();
  }
  // bf16 Q fragments for phi(Q) in the linear branch: query 32*qh + l32 from
  // the V buffer of half qh that took Q rows 32*qh .. +31
  bf16x8 qf[NS];
  if (has_lin) {
    const int nhq = (kc - qh + 1) / 2;
    const uint16_t* qsrc = reinterpret_cast<const uint16_t*>(smem_raw + VREG + qh * 2 * TB + q_buf(nhq) * TB);
#pragma unroll
    for (int s = 0; s < NS; ++s)
      qf[s] = *reinterpret_cast<const bf16x8*>(qsrc + l32 * D + 8 * ((2 * s + hh) ^ (l32 & 15)));
  } else {
#pragma unroll
    for (int s = 0; s < NS; ++s) qf[s] = bf16x8{};
  }
  __syncthreads();   // every wave holds its Q before the merge buffers overwrite the V buffers
  attention_finish<uint16_t, D, true, false, false, false, LSE>(
      smem_raw + VREG, smem_u16 + lh * (2 * TB / 2), sig_lds, true, g, bh, h, i, n_i, qrow, hoff,
      A.s_sum, A.sigma_sum, A.alpha, A.o, A.o_sparse, A.o_linear, oacc, m_run, l_run, 1.0f, qf,
      [](int) {}, 0.0f, A.lse);
}

}  // namespace

hipError_t launch_attention_fp8(const Geometry& g, const void* q, const uint8_t* q8,
                                const float* q_s, const uint8_t* k8, const float* k_s,
                                const uint8_t* v8, const float* v_s, const int32_t* crit,
                                const uint16_t* s_sum, const float* sigma_sum,
                                const float* alpha, void* o, float* o_sparse, float* o_linear,
                                hipStream_t stream, float* lse) {
  if (g.D != 128 || g.dtype != 1) return hipErrorNotSupported;
  AttnFp8Args a{static_cast<const uint16_t*>(q), q8, q_s, k8, k_s, v8, v_s, crit, s_sum, sigma_sum,
                alpha, o, o_sparse, o_linear, g,
                static_cast<float>(1.4426950408889634 / __builtin_sqrt(static_cast<double>(g.D))),
                lse};
  const int total = g.B * g.H * g.nq;
  if (lse)
    hipLaunchKernelGGL(attention_fp8_kernel<true>, dim3(total), dim3(kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL(attention_fp8_kernel<false>, dim3(total), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace sla
