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
//   * the block's K and V tiles [64 keys][d] sit in LDS, row-major with a
//     16-byte-chunk XOR swizzle; two K and two V buffers form a ring that the
//     direct global->LDS loads for the next blocks fill while this one
//     computes;
//   * each wave computes S^T = K Q^T for its 32 keys x 32 queries on
//     v_mfma_f32_32x32x16_bf16, runs the online-softmax update on the S^T
//     registers (query = lane % 32, so a row max is a reduction over the
//     lane's own registers plus the partner lane l ^ 32), and accumulates
//     O^T += V^T P^T with P^T taken straight from the S^T registers and the
//     V^T operand read from the row-major V tile by transposing LDS reads
//     (ds_read_b64_tr_b16).
// The two key halves keep separate running max / sum / output (no per-block
// cross-wave reduction); the shared epilogue merges them, adds the linear
// branch from the precomputed marginal-state sums and stores the alpha mix.
//
// PISA instance ([PISA technical summary, "Algoritmo Central" and
// "Implementación de Hardware"]): after the critical blocks the same loop
// runs over pseudo-blocks of 64 block centroids (kbar rows as keys, block
// value means as values), so the zero-order terms of every unselected block
// enter the one online softmax: a centroid key carries log(n_j) in its score
// (its block's n_j tokens) and selected or padding centroids are masked out.
// A third running sum collects sum_j alpha_{t,j} over the unselected blocks,
// and the epilogue adds the global first-order correction
// (q_t / sqrt(d)) Hbar sum_j alpha_{t,j} to the numerator before the one
// division.
#include <type_traits>

#include "attention_epilogue.hpp"

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
  // PISA only: centroid tiles, pseudo-block count, the log2(n_j) score
  // offsets in units of the raw dot product, 1 / n_j of the last block
  const uint16_t* kbar;
  const uint16_t* vbar;
  int npb;
  float bias_full;
  float bias_last;
  float inv_last;
  float* lse;        // optional log2 normaliser of the sparse softmax per row
};

// RLA: residual linear attention epilogue (the marginal sum holds every
// non-critical block's exponential-map state; RMS norm instead of the
// phi(Q) . sigma_i denominator, so sigma_i is not loaded).  PISA: piecewise
// exact-or-approximate attention (s_sum holds Hbar per head).
template <typename T, int D, bool RLA, bool PISA = false, bool LSE = false>
__global__ void __launch_bounds__(kThreads, 2)
attention_kernel(AttnArgs A) {
  constexpr int CH = D / 8;                    // 16-byte chunks per row
  constexpr int TILE = kBlock * D;             // elements per K or V tile
  constexpr int NSTAGE = 4;                    // two K buffers, two V buffers
  constexpr int RPI = 64 / CH;                 // rows per 64-lane load instruction
  constexpr int IPW = (kBlock / 4) / RPI;      // load instructions per wave per tile
  constexpr int NS = D / 16;                   // 16-wide k-steps over the features
  constexpr int DT = D / 32;                   // 32-row tiles over the value dims
  constexpr int LOOP_BYTES = NSTAGE * TILE * 2;
  constexpr int EPI_BYTES = epilogue_smem_bytes<D>();
  // The merge buffers of the epilogue start at the V buffers; at d = 128 the
  // last two steps prefetch S_i^T into the two K buffers (d = 64 reads S_i^T
  // from HBM).
  constexpr bool ST_LDS = (D == 128);
  constexpr int EPI_OFF = 2 * TILE * 2;
  constexpr int SMEM_BYTES = (LOOP_BYTES > EPI_OFF + EPI_BYTES ? LOOP_BYTES : EPI_OFF + EPI_BYTES);
  __shared__ __attribute__((aligned(16))) unsigned char smem_raw[SMEM_BYTES];
  __shared__ __attribute__((aligned(16))) float sig_lds[D];     // sigma_i, loaded at the start
  // PISA: excluded centroids (selected blocks and padding), one bit each
  __shared__ uint64_t excl[PISA ? 64 : 1];
  uint16_t* smem = reinterpret_cast<uint16_t*>(smem_raw);

  const Geometry& g = A.g;
  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);   // wave-uniform (scalar)
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
  constexpr float kLazy = 8.0f;
  const int64_t sn = g.sn;

  // Q fragments (B operand of S^T = K Q^T): query 32*qh + l32, features
  // 16*s + 8*hh .. +7, loaded once the first tiles are on their way.
  bf16x8 qf[NS];
  const int qrow = 32 * qh + l32;

  const int32_t* __restrict__ crow = A.crit + (static_cast<int64_t>(bh) * g.nq + i) * g.k_crit;
  const int kc = g.k_crit;
  // steps of the loop: the critical blocks, then (PISA) the pseudo-blocks
  const int nst = PISA ? kc + A.npb : kc;
  if constexpr (PISA) {
    for (int w = t; w < A.npb; w += kThreads)
      excl[w] = (w == A.npb - 1 && (g.nkb & 63)) ? (~0ull << (g.nkb & 63)) : 0ull;
    __syncthreads();
    for (int c = t; c < kc; c += kThreads) {
      const int jb = list_block(crow[c], g.nkb);
      atomicOr(reinterpret_cast<unsigned long long*>(excl + (jb >> 6)), 1ull << (jb & 63));
    }
  }
  // The critical list is read once into registers, 64 entries per register
  // (lane l holds entry base + l), and entries are taken with v_readlane, so
  // the loop issues no index loads: a vector load there would make the
  // compiler's vmcnt wait cover the in-flight K/V tile loads as well.
  int cl0 = lane < kc ? list_block(crow[lane], g.nkb) : 0;
  int cl1 = 64 + lane < kc ? list_block(crow[64 + lane], g.nkb) : 0;
  int cbase = 0;
  auto crit_at = [&](int c) -> int {
    const int o = c - cbase;
    return o < 64 ? __builtin_amdgcn_readlane(cl0, o) : __builtin_amdgcn_readlane(cl1, o - 64);
  };

  // LDS ring: K buffers kbuf[2] and V buffers vbuf[2] (16 KB each at d=128).
  // Iteration it reads K of block it+1 (for the next S) and V of block it;
  // right after its barrier it issues K of block it+2 and V of block it+1
  // straight into LDS (no staging registers), which land while it computes.
  //
  // Wave w fills rows 16w .. 16w+15 of a tile; lane l of instruction u writes
  // row 16w + RPI*u + l/CH at chunk slot l%CH, which holds global chunk
  // (l%CH) ^ swz(row).  bf16 tiles come through a range-checked buffer
  // resource ending at the last token's row, so rows past the end of a short
  // last block read as zeros (their keys are masked to -inf in S); float
  // tiles are converted in registers with the row index clamped instead.
  const int lrow = lane / CH, lslot = lane % CH;
  const uint32_t rowb = static_cast<uint32_t>(sn * sizeof(T));
  const uint32_t head_bytes = static_cast<uint32_t>((g.N - 1) * sn * sizeof(T) + D * sizeof(T));
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(kp, head_bytes);
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc(vp, head_bytes);
  uint32_t toff[IPW], tcol[IPW];
#pragma unroll
  for (int u = 0; u < IPW; ++u) {
    const int r = 16 * wave + RPI * u + lrow;
    tcol[u] = static_cast<uint32_t>(8 * (lslot ^ swz<D>(r)) * sizeof(T));
    toff[u] = static_cast<uint32_t>(r) * rowb + tcol[u];
  }
  [[maybe_unused]] __amdgpu_buffer_rsrc_t kbrs, vbrs;
  if constexpr (PISA) {
    const int64_t cb = static_cast<int64_t>(bh) * A.npb * kBlock * D;
    kbrs = make_rsrc(A.kbar + cb, static_cast<uint32_t>(g.nkb * D * 2));
    vbrs = make_rsrc(A.vbar + cb, static_cast<uint32_t>(g.nkb * D * 2));
  }
  auto issue_tile = [&](bool is_k, int c, uint16_t* dst) {
    if constexpr (PISA) {
      if (c >= kc) {
        // centroid tile: bf16 rows of D, rows past nkb read as zeros
        const uint32_t soff = static_cast<uint32_t>((c - kc) * kBlock * D * 2);
#pragma unroll
        for (int u = 0; u < IPW; ++u) {
          const int r = 16 * wave + RPI * u + lrow;
          const uint32_t off = static_cast<uint32_t>(r * D * 2 + 16 * (lslot ^ swz<D>(r)));
          buffer_load_lds16(is_k ? kbrs : vbrs, dst + (16 * wave + RPI * u) * D, off, soff);
        }
        return;
      }
    }
    const int jb = crit_at(c);
    if constexpr (sizeof(T) == 2) {
      const uint32_t soff = static_cast<uint32_t>(kBlock * jb) * rowb;
#pragma unroll
      for (int u = 0; u < IPW; ++u)
        buffer_load_lds16(is_k ? krs : vrs, dst + (16 * wave + RPI * u) * D, toff[u], soff);
    } else {
      const int nj = min(kBlock, g.N - kBlock * jb);
      const T* tb = (is_k ? kp : vp) + static_cast<int64_t>(kBlock * jb) * sn;
#pragma unroll
      for (int u = 0; u < IPW; ++u) {
        const int r0 = 16 * wave + RPI * u;
        const int r = r0 + lrow;
        const uint32_t off = static_cast<uint32_t>(r < nj ? r : nj - 1) * rowb + tcol[u];
        const T* src = reinterpret_cast<const T*>(reinterpret_cast<const char*>(tb) + off);
        *reinterpret_cast<bf16x8*>(dst + r0 * D + 8 * lane) = load8(src);
      }
    }
  };

  // S_i^T (value-major, D rows x D) halves: rows 64*half .. +63 as a
  // swizzled tile, same pattern as a K tile (contiguous rows of D bf16)
  const bool has_lin = PISA || g.k_marg > 0;
  const __amdgpu_buffer_rsrc_t srs =
      make_rsrc(A.s_sum + (PISA ? static_cast<int64_t>(bh) : static_cast<int64_t>(bh) * g.nq + i) * D * D,
                D * D * 2);
  if (!RLA && !PISA && has_lin && wave == 0 && lane < D / 4) {
    const __amdgpu_buffer_rsrc_t sgr =
        make_rsrc(A.sigma_sum + (static_cast<int64_t>(bh) * g.nq + i) * D, D * 4);
    buffer_load_lds16(sgr, sig_lds, 16u * lane, 0u);
  }
  auto issue_st = [&](int half, uint16_t* dst) {
#pragma unroll
    for (int u = 0; u < IPW; ++u) {
      const int r = 16 * wave + RPI * u + lrow;
      const uint32_t off = static_cast<uint32_t>(r * D * 2 + 16 * (lslot ^ swz<D>(r)));
      buffer_load_lds16(srs, dst + (16 * wave + RPI * u) * D, off,
                        static_cast<uint32_t>(half * kBlock * D * 2));
    }
  };

  // K operand rows: S^T of keys 32*kh .. +31 (of a K tile) and queries
  // 32*qh .. +31; element offsets of the 8 feature chunks (loop-invariant).
  const int krow = 32 * kh + l32;
  const int ksw = swz<D>(krow);
  int kofs[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) kofs[s] = krow * D + 8 * ((2 * s + hh) ^ ksw);

  // Transposing V reads (ds_read_b64_tr_b16): within each 16-lane group,
  // output lane i receives element i % 4 of the 8-byte rows addressed by
  // lanes 4e + i / 4 (e = 0..3).  This lane addresses key
  // 32*kh + 16*s + 8*x + 4*hh + ep (x = 0, 1 for the two reads of a k-step)
  // at the 4 dims from 32*dt + 16*gm + 4*q4, so that output lane l gets dim
  // 32*dt + l % 32 at the keys its P^T k-slots hold.
  const int g16 = lane >> 4, li = lane & 15;
  const int ep = li >> 2, q4 = li & 3, gm = g16 & 1;
  const int key1 = 32 * kh + 4 * hh + ep;                 // + 16 s, and + 8 for the second read
  const int sw1 = swz<D>(key1), sw2 = swz<D>(key1 + 8);   // independent of s (16 s keeps bits 0..3)
  // LDS byte addresses of the (s = 0) reads for each 32-dim tile, relative
  // to the start of the tile area; the V buffer and s = 1 (+16 rows) are
  // immediate offsets
  uint32_t va1[DT], va2[DT];
  {
    const uint32_t base = lds_addr(smem);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const int c = 4 * dt + 2 * gm + (q4 >> 1);
      va1[dt] = base + static_cast<uint32_t>((key1 * D + 8 * (c ^ sw1) + 4 * (q4 & 1)) * 2);
      va2[dt] = base + static_cast<uint32_t>(((key1 + 8) * D + 8 * (c ^ sw2) + 4 * (q4 & 1)) * 2);
    }
  }

  float m_run = -INFINITY, l_run = 0.0f;
  float a_run = 0.0f;   // PISA: sum of alpha_{t,j} over this lane's unselected centroids
  // PISA: the exclusion words, lane w holding pseudo-block w (set below,
  // once the bits are complete), read in the loop with v_readlane
  uint32_t exw_lo = 0, exw_hi = 0;
  f32x16 oacc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) oacc[dt] = zero16();

  // One critical block per step.  Step it (buffer parity X = it & 1) finds
  // K(it+1) in kbuf[X^1] and V(it) in vbuf[X], sends K(it+2) into kbuf[X]
  // and V(it+1) into vbuf[X^1], computes S(it+1) (from a stale but
  // in-bounds buffer when there is no block it+1; the result is dropped)
  // while the softmax of S(it) runs, then adds P V(it).
  auto step = [&](auto xc, int it, f32x16& s_cur, f32x16& s_next) {
    constexpr int X = decltype(xc)::value;
    const uint16_t* kb_next = smem + (X ^ 1) * TILE;
    // K and V fragments first: no direct-to-LDS load of this wave is in
    // flight yet (the previous step ended with vmcnt(0)), so these reads need
    // no wait on the loads issued right after them.
    bf16x8 kf[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) kf[s] = *reinterpret_cast<const bf16x8*>(kb_next + kofs[s]);
    // V^T fragments for O^T += V^T P^T, read now (V(it) has been in LDS
    // since the last barrier) so that one wait covers them and the K
    // fragments: lane l gets dim 32*dt + l%32 at keys 32*kh + 16*s +
    // 8*(e/4) + 4*hh + e%4, matching P^T's k-slots.  All 16 transposing reads
    // and the wait sit in one asm block.
    constexpr int VOFF0 = (2 + X) * TILE * 2;
    constexpr int VOFF1 = VOFF0 + 16 * D * 2;
    u32x2 rd[4 * DT];
    if constexpr (DT == 4) {
      asm volatile(
          "ds_read_b64_tr_b16 %0, %16 offset:%24\n\t"
          "ds_read_b64_tr_b16 %1, %17 offset:%24\n\t"
          "ds_read_b64_tr_b16 %2, %16 offset:%25\n\t"
          "ds_read_b64_tr_b16 %3, %17 offset:%25\n\t"
          "ds_read_b64_tr_b16 %4, %18 offset:%24\n\t"
          "ds_read_b64_tr_b16 %5, %19 offset:%24\n\t"
          "ds_read_b64_tr_b16 %6, %18 offset:%25\n\t"
          "ds_read_b64_tr_b16 %7, %19 offset:%25\n\t"
          "ds_read_b64_tr_b16 %8, %20 offset:%24\n\t"
          "ds_read_b64_tr_b16 %9, %21 offset:%24\n\t"
          "ds_read_b64_tr_b16 %10, %20 offset:%25\n\t"
          "ds_read_b64_tr_b16 %11, %21 offset:%25\n\t"
          "ds_read_b64_tr_b16 %12, %22 offset:%24\n\t"
          "ds_read_b64_tr_b16 %13, %23 offset:%24\n\t"
          "ds_read_b64_tr_b16 %14, %22 offset:%25\n\t"
          "ds_read_b64_tr_b16 %15, %23 offset:%25\n\t"
          "s_waitcnt lgkmcnt(0)"
          : "=&v"(rd[0]), "=&v"(rd[1]), "=&v"(rd[2]), "=&v"(rd[3]), "=&v"(rd[4]), "=&v"(rd[5]),
            "=&v"(rd[6]), "=&v"(rd[7]), "=&v"(rd[8]), "=&v"(rd[9]), "=&v"(rd[10]), "=&v"(rd[11]),
            "=&v"(rd[12]), "=&v"(rd[13]), "=&v"(rd[14]), "=&v"(rd[15])
          : "v"(va1[0]), "v"(va2[0]), "v"(va1[1]), "v"(va2[1]), "v"(va1[2]), "v"(va2[2]),
            "v"(va1[3]), "v"(va2[3]), "i"(VOFF0), "i"(VOFF1)
          : "memory");
    } else {
      asm volatile(
          "ds_read_b64_tr_b16 %0, %8 offset:%12\n\t"
          "ds_read_b64_tr_b16 %1, %9 offset:%12\n\t"
          "ds_read_b64_tr_b16 %2, %8 offset:%13\n\t"
          "ds_read_b64_tr_b16 %3, %9 offset:%13\n\t"
          "ds_read_b64_tr_b16 %4, %10 offset:%12\n\t"
          "ds_read_b64_tr_b16 %5, %11 offset:%12\n\t"
          "ds_read_b64_tr_b16 %6, %10 offset:%13\n\t"
          "ds_read_b64_tr_b16 %7, %11 offset:%13\n\t"
          "s_waitcnt lgkmcnt(0)"
          : "=&v"(rd[0]), "=&v"(rd[1]), "=&v"(rd[2]), "=&v"(rd[3]), "=&v"(rd[4]), "=&v"(rd[5]),
            "=&v"(rd[6]), "=&v"(rd[7])
          : "v"(va1[0]), "v"(va2[0]), "v"(va1[1]), "v"(va2[1]), "i"(VOFF0), "i"(VOFF1)
          : "memory");
    }
    if (it + 2 < nst) {
      issue_tile(true, it + 2, smem + X * TILE);
    } else if constexpr (ST_LDS) {
      // kbuf[X] (K(it), consumed last step) stays free: S_i^T half 0 goes in
      // at step kc-2, half 1 at step kc-1 (both at step 0 when kc = 1), so
      // half 0 ends in kbuf[kc & 1] and half 1 in kbuf[(kc & 1) ^ 1]
      if (has_lin) {
        if (it == nst - 2) {
          issue_st(0, smem + X * TILE);
        } else {
          issue_st(1, smem + X * TILE);
          if (nst == 1) issue_st(0, smem + (X ^ 1) * TILE);
        }
      }
    }
    if (it + 1 < nst) issue_tile(false, it + 1, smem + (2 + (X ^ 1)) * TILE);
    f32x16 acc = zero16();
    acc = mfma32(kf[0], qf[0], acc);
    acc = mfma32(kf[1], qf[1], acc);

    const bool pseudo = PISA && it >= kc;
    [[maybe_unused]] int key0 = 0;
    if (pseudo) {
      // centroid 64*(it-kc) + key of this lane's registers: excluded ones
      // drop out, the others carry log(n_j) (in units of the raw score)
      const int pbk = it - kc;
      const uint32_t w32 = kh ? __builtin_amdgcn_readlane(exw_hi, pbk) : __builtin_amdgcn_readlane(exw_lo, pbk);
      const uint32_t wl = w32 >> (4 * hh);
      key0 = kBlock * pbk + 32 * kh + 4 * hh;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int kk = 8 * (r >> 2) + (r & 3);
        const float bias = key0 + kk == g.nkb - 1 ? A.bias_last : A.bias_full;
        s_cur[r] = ((wl >> kk) & 1u) ? -INFINITY : s_cur[r] + bias;
      }
    } else {
      const int jb = crit_at(it);
      const int nj = min(kBlock, g.N - kBlock * jb);
      if (nj < kBlock) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = 32 * kh + 8 * (r >> 2) + 4 * hh + (r & 3);
          if (key >= nj) s_cur[r] = -INFINITY;
        }
      }
    }
    float mx = max16(s_cur);
    {
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx),
                                                       false, false);
      mx = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));   // with lane l ^ 32
    }
    // The running reference max m_run only moves when some query's tile max
    // exceeds it by more than kLazy (in log2 units), so p <= 2^kLazy and the
    // output / sum rescale is skipped on most blocks; O and l always share
    // the same reference, so the final O / l is unchanged.
    const bool grow = __ballot((mx - m_run) * cl > kLazy) != 0ull;
    if (grow) {
      const float m_new = fmaxf(m_run, mx);
      const float corr = __builtin_amdgcn_exp2f((m_run - m_new) * cl);
      l_run *= corr;
      if constexpr (PISA) a_run *= corr;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[dt][r] *= corr;
      m_run = m_new;
    }
#pragma unroll
    for (int s = 2; s < NS; ++s) acc = mfma32(kf[s], qf[s], acc);

    const float mb = (m_run == -INFINITY ? 0.0f : m_run) * cl;
    bf16x8 pb[2];
    float ps = 0.0f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float p = __builtin_amdgcn_exp2f(fmaf(s_cur[r], cl, -mb));
      ps += p;
      pb[r >> 3][r & 7] = f32_to_bf16(p);
    }
    l_run += ps;
    if (pseudo) {
      // alpha_{t,j} = p / n_j: 1/64 for full blocks, 1/n_last for the last
      float plast = 0.0f;
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (key0 + 8 * (r >> 2) + (r & 3) == g.nkb - 1) plast = __builtin_amdgcn_exp2f(fmaf(s_cur[r], cl, -mb));
      a_run += ps * (1.0f / kBlock) + plast * (A.inv_last - 1.0f / kBlock);
    }
    s_next = acc;

#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      u32x4 w0, w1;
      w0[0] = rd[4 * dt][0]; w0[1] = rd[4 * dt][1]; w0[2] = rd[4 * dt + 1][0]; w0[3] = rd[4 * dt + 1][1];
      w1[0] = rd[4 * dt + 2][0]; w1[1] = rd[4 * dt + 2][1]; w1[2] = rd[4 * dt + 3][0]; w1[3] = rd[4 * dt + 3][1];
      oacc[dt] = mfma32(__builtin_bit_cast(bf16x8, w0), pb[0], oacc[dt]);
      oacc[dt] = mfma32(__builtin_bit_cast(bf16x8, w1), pb[1], oacc[dt]);
    }
    if ((!PISA || it + 1 < kc) && it + 1 - cbase == 64) {   // entries it+1 .. it+64 now start at register 1
      cbase += 64;
      cl0 = cl1;
      cl1 = cbase + 64 + lane < kc ? list_block(crow[cbase + 64 + lane], g.nkb) : 0;
    }
    wait_vmem();   // this wave's loads for the next step
    __syncthreads();
  };

  // The critical list is needed for the first tile addresses; the Q loads
  // go out after those tiles so that both are in flight together.  Q and
  // the list are in registers before the loop; a wait the compiler can see
  // keeps it from guarding their first uses inside the loop with waits that
  // would then also stall on the tile prefetches.  Q rows past the last
  // query are clamped (not stored).
  wait_vmem();
  f32x16 sa = zero16(), sb = zero16();
  if (nst > 0) {
    issue_tile(true, 0, smem);
    issue_tile(false, 0, smem + 2 * TILE);
    if (nst > 1) issue_tile(true, 1, smem + TILE);
  }
  {
    const int qr = qrow < n_i ? qrow : n_i - 1;
#pragma unroll
    for (int s = 0; s < NS; ++s)
      qf[s] = load8(qp + static_cast<int64_t>(kBlock * i + qr) * sn + 16 * s + 8 * hh);
  }
  wait_vmem();
  if (nst > 0) {
    __syncthreads();
    bf16x8 kf[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) kf[s] = *reinterpret_cast<const bf16x8*>(smem + kofs[s]);
#pragma unroll
    for (int s = 0; s < NS; ++s) sa = mfma32(kf[s], qf[s], sa);
  }
  // every wave has read kbuf[0] before step 0 refills it
  __syncthreads();
  if constexpr (PISA) {
    if (lane < A.npb) {
      const uint64_t w = excl[lane];
      exw_lo = static_cast<uint32_t>(w);
      exw_hi = static_cast<uint32_t>(w >> 32);
    }
  }
  // no critical block: the idle K buffers take S_i^T right away (the
  // epilogue then always finds it in LDS)
  if (ST_LDS && nst == 0 && has_lin) {
    issue_st(0, smem);
    issue_st(1, smem + TILE);
  }
  for (int it = 0; it < nst; it += 2) {
    step(std::integral_constant<int, 0>(), it, sa, sb);
    if (it + 1 < nst) step(std::integral_constant<int, 1>(), it + 1, sb, sa);
  }
  wait_vmem();       // (no step: the S_i^T loads above)
  __syncthreads();

  const uint16_t* st_half = smem + ((nst & 1) ^ kh) * TILE;
  attention_finish<T, D, ST_LDS, false, RLA, PISA, LSE>(smem_raw + EPI_OFF, st_half, sig_lds,
                                                   !RLA && !PISA && has_lin, g, bh, h, i, n_i, qrow,
                                                   hoff, A.s_sum, A.sigma_sum, A.alpha, A.o,
                                                   A.o_sparse, A.o_linear, oacc, m_run, l_run, cl,
                                                   qf, [](int) {}, a_run, A.lse);
}

template <typename T, int D>
void launch_attn_t(const AttnArgs& a, bool rla, hipStream_t stream) {
  const int total = a.g.B * a.g.H * a.g.nq;
  if (a.lse)
    hipLaunchKernelGGL((attention_kernel<T, D, false, false, true>), dim3(total), dim3(kThreads), 0,
                       stream, a);
  else if (rla)
    hipLaunchKernelGGL((attention_kernel<T, D, true>), dim3(total), dim3(kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL((attention_kernel<T, D, false>), dim3(total), dim3(kThreads), 0, stream, a);
}

template <typename T, int D>
void launch_attn_pisa_t(const AttnArgs& a, hipStream_t stream) {
  const int total = a.g.B * a.g.H * a.g.nq;
  hipLaunchKernelGGL((attention_kernel<T, D, false, true>), dim3(total), dim3(kThreads), 0, stream, a);
}

}  // namespace

hipError_t launch_attention_pisa(const Geometry& g, const void* q, const void* k, const void* v,
                                 const int32_t* crit, const uint16_t* kbar, const uint16_t* vbar,
                                 const uint16_t* hbar, void* o, float* o_softmax,
                                 float* o_correction, hipStream_t stream) {
  const double cl = 1.4426950408889634 / __builtin_sqrt(static_cast<double>(g.D));
  const int n_last = g.N - kBlock * (g.nkb - 1);
  AttnArgs a{q, k, v, crit, hbar, nullptr, nullptr, o, o_softmax, o_correction, g,
             static_cast<float>(cl), kbar, vbar, pisa_pseudo_blocks(g),
             static_cast<float>(6.0 / cl),
             static_cast<float>(__builtin_log2(static_cast<double>(n_last)) / cl),
             1.0f / static_cast<float>(n_last), nullptr};
  if (g.dtype == 1) {
    if (g.D == 128) launch_attn_pisa_t<uint16_t, 128>(a, stream);
    else launch_attn_pisa_t<uint16_t, 64>(a, stream);
  } else {
    if (g.D == 128) launch_attn_pisa_t<float, 128>(a, stream);
    else launch_attn_pisa_t<float, 64>(a, stream);
  }
  return hipGetLastError();
}

hipError_t launch_attention(const Geometry& g, const void* q, const void* k, const void* v,
                            const int32_t* crit, const uint16_t* s_sum, const float* sigma_sum,
                            const float* alpha, void* o, float* o_sparse, float* o_linear,
                            bool rla, hipStream_t stream, float* lse) {
  AttnArgs a{q, k, v, crit, s_sum, sigma_sum, alpha, o, o_sparse, o_linear, g,
             static_cast<float>(1.4426950408889634 / __builtin_sqrt(static_cast<double>(g.D))),
             nullptr, nullptr, 0, 0.0f, 0.0f, 0.0f, lse};
  if (g.dtype == 1) {
    if (g.D == 128) launch_attn_t<uint16_t, 128>(a, rla, stream);
    else launch_attn_t<uint16_t, 64>(a, rla, stream);
  } else {
    if (g.D == 128) launch_attn_t<float, 128>(a, rla, stream);
    else launch_attn_t<float, 64>(a, rla, stream);
  }
  return hipGetLastError();
}

}  // namespace sla
