// Block routing: pooled Q/K, block logits and the three-way top-k split.
//
// [SLA2 technical summary, section 2.B] the router sees only Q and K, pools
// adjacent tokens so its cost stays far below O(N^2), and keeps a hard top-k
// at inference.  [SLA abstract] KV blocks of each query block fall into
// critical, marginal and negligible classes.
//
// Pooling sums bf16/f32 rows in float64 (exact for bf16 blocks) and divides
// by the valid token count; logits are float64 dot products divided by
// sqrt(d).  The second-order score of [SPLA technical summary, section 2.1]
// adds log1p(sum_a qbar_a^2 var_a / (2 d)), var_a the population variance of
// feature a over the KV block's valid keys (two passes in float64 over the
// block held in registers).  The selection is an exact radix select over a 64-bit key that
// orders logits descending, so the split is the one the float64 logits
// define; equal logits are ordered by ascending KV block index.  Compaction
// writes each class's KV block indices in ascending order.
#include "device_common.hpp"
#include "sla_internal.hpp"

namespace sla {
namespace {

// ---------------------------------------------------------------- pooling
// grid (nb, B*H, 2): z = 0 pools Q, z = 1 pools K.  One workgroup per block:
// thread t reads the 16-byte chunk t % CH of rows t / CH + RG m (rows past
// a ragged end load the block's last row and are zeroed, so every load is in
// flight at once), then LDS sums the row groups in float64.  VAR adds, for
// K blocks, a second pass: squared deviations from the block mean, summed
// the same way.
template <typename T, int D, bool VAR>
__global__ void __launch_bounds__(kThreads)
pool_kernel(const T* __restrict__ q, const T* __restrict__ k, Geometry g,
            double* __restrict__ qpool, double* __restrict__ kpool_t,
            float* __restrict__ qout, float* __restrict__ kout,
            double* __restrict__ kvar_t, float* __restrict__ vout) {
  constexpr int CH = D / 8;           // 8-element chunks per row
  constexpr int RG = kThreads / CH;   // row groups
  constexpr int RPG = kBlock / RG;    // rows per group
  __shared__ double red[RG][D];
  __shared__ double mean_s[VAR ? D : 1];

  const int j = blockIdx.x;
  const int bh = blockIdx.y;
  const int which = blockIdx.z;
  const int b = bh / g.H, h = bh % g.H;
  const T* x = (which == 0 ? q : k) + b * g.sb + h * g.sh;
  const int t = threadIdx.x;
  const int ch = t % CH, rg = t / CH;
  const int row0 = j * kBlock;
  const int nj = min(kBlock, g.N - row0);

  float f[RPG][8];
#pragma unroll
  for (int rr = 0; rr < RPG; ++rr)
    load8_f32(x + static_cast<int64_t>(row0 + min(rg + rr * RG, nj - 1)) * g.sn + ch * 8, f[rr]);
  double acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    acc[e] = 0.0;
#pragma unroll
    for (int rr = 0; rr < RPG; ++rr)
      acc[e] += rg + rr * RG < nj ? static_cast<double>(f[rr][e]) : 0.0;
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) red[rg][ch * 8 + e] = acc[e];
  __syncthreads();
  if (t < D) {
    double s = 0.0;
    for (int r = 0; r < RG; ++r) s += red[r][t];
    const double m = s / static_cast<double>(nj);
    if (which == 0) {
      const int64_t o = (static_cast<int64_t>(bh) * g.nq + j) * D + t;
      qpool[o] = m;
      if (qout) qout[o] = static_cast<float>(m);
    } else {
      kpool_t[(static_cast<int64_t>(bh) * D + t) * g.nkb + j] = m;
      if (kout) kout[(static_cast<int64_t>(bh) * g.nkb + j) * D + t] = static_cast<float>(m);
      if constexpr (VAR) mean_s[t] = m;
    }
  }
  if constexpr (VAR) {
    if (which == 1) {          // uniform over the workgroup
      __syncthreads();         // means visible, first-pass reads of red done
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const double me = mean_s[ch * 8 + e];
        acc[e] = 0.0;
#pragma unroll
        for (int rr = 0; rr < RPG; ++rr) {
          const double dv = static_cast<double>(f[rr][e]) - me;
          acc[e] += rg + rr * RG < nj ? dv * dv : 0.0;
        }
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) red[rg][ch * 8 + e] = acc[e];
      __syncthreads();
      if (t < D) {
        double s = 0.0;
        for (int r = 0; r < RG; ++r) s += red[r][t];
        const double var = s / static_cast<double>(nj);
        kvar_t[(static_cast<int64_t>(bh) * D + t) * g.nkb + j] = var;
        if (vout) vout[(static_cast<int64_t>(bh) * g.nkb + j) * D + t] = static_cast<float>(var);
      }
    }
  }
}

// 64-bit key whose unsigned order is the descending order of the logit
// (-0.0 and +0.0 map to the same key).
__device__ __forceinline__ uint64_t desc_key(double s) {
  if (s == 0.0) s = 0.0;
  uint64_t u = static_cast<uint64_t>(__double_as_longlong(s));
  u = (u >> 63) ? ~u : (u | 0x8000000000000000ull);
  return ~u;
}

// DPP lane move within rows of 16 lanes; lanes whose source falls outside
// the row read 0.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_mov(uint32_t v) {
  return static_cast<uint32_t>(
      __builtin_amdgcn_update_dpp(0, static_cast<int>(v), CTRL, 0xF, 0xF, true));
}

// Inclusive prefix sum over the 64 lanes: Hillis-Steele inside each row of 16
// lanes (row_shr 1, 2, 4, 8), then the totals of the lower rows.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v, int lane) {
  v += dpp_mov<0x111>(v);
  v += dpp_mov<0x112>(v);
  v += dpp_mov<0x114>(v);
  v += dpp_mov<0x118>(v);
  const uint32_t r0 = __builtin_amdgcn_readlane(v, 15);
  const uint32_t r1 = __builtin_amdgcn_readlane(v, 31);
  const uint32_t r2 = __builtin_amdgcn_readlane(v, 47);
  const int row = lane >> 4;
  return v + (row >= 1 ? r0 : 0u) + (row >= 2 ? r1 : 0u) + (row >= 3 ? r2 : 0u);
}

// Bitwise OR over the 64 lanes (quad swaps, half-row and row mirrors, then
// the four row results).
__device__ __forceinline__ uint32_t wave_or(uint32_t v) {
  v |= dpp_mov<0xB1>(v);
  v |= dpp_mov<0x4E>(v);
  v |= dpp_mov<0x141>(v);
  v |= dpp_mov<0x140>(v);
  return __builtin_amdgcn_readlane(v, 0) | __builtin_amdgcn_readlane(v, 16) |
         __builtin_amdgcn_readlane(v, 32) | __builtin_amdgcn_readlane(v, 48);
}

__device__ __forceinline__ uint64_t readlane64(uint64_t v, int l) {
  const uint32_t lo = __builtin_amdgcn_readlane(static_cast<uint32_t>(v), l);
  const uint32_t hi = __builtin_amdgcn_readlane(static_cast<uint32_t>(v >> 32), l);
  return (static_cast<uint64_t>(hi) << 32) | lo;
}

__device__ __forceinline__ void lds_wait() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// ---------------------------------------------------------------- selection
// One wave splits one query block's row of nkb keys (key order = descending
// logit).  Lane l holds the keys of KV blocks l + 64u in registers.
//
// The two cuts sit at ranks k_crit - 1 and k_crit + k_marg - 1.  Each is
// found by a radix select that starts at the highest bit where the row's
// keys differ (the bits above are common to all keys) and takes 8 bits per
// pass.  A pass histograms the digit of the keys that share the cut's prefix,
// a prefix scan of the bins finds the bin holding the cut's rank, and the
// search ends as soon as that bin holds a single key: that key is the cut.
// If all 64 bits are consumed, the remaining rank counts equal keys, which
// are taken in ascending KV block order.
template <int KPL>
__device__ __forceinline__ void select_row(const uint64_t* rk, int nkb, int lane, uint32_t* wh,
                                           int k_crit, int k_marg, int64_t row, int32_t* crit,
                                           int32_t* marg, int8_t* cls) {
  uint64_t kk[KPL];
#pragma unroll
  for (int u = 0; u < KPL; ++u) {
    const int j = lane + 64 * u;
    kk[u] = j < nkb ? rk[j] : ~0ull;
  }
  const uint64_t k0 = rk[0];
  uint64_t dx = 0;
#pragma unroll
  for (int u = 0; u < KPL; ++u)
    if (lane + 64 * u < nkb) dx |= kk[u] ^ k0;
  const uint64_t diff = (static_cast<uint64_t>(wave_or(static_cast<uint32_t>(dx >> 32))) << 32) |
                        wave_or(static_cast<uint32_t>(dx));
  int hi = diff ? 63 - __builtin_clzll(diff) : -1;
  // bits above the highest differing bit (for hi = 63: none)
  const uint64_t common = diff ? (k0 & ~((2ull << hi) - 1ull)) : k0;

  const int target[2] = {k_crit, k_crit + k_marg};
  uint64_t pref[2] = {common, common};
  uint32_t rem[2];
  bool done[2];
#pragma unroll
  for (int w = 0; w < 2; ++w) {
    rem[w] = target[w] > 0 ? static_cast<uint32_t>(target[w] - 1) : 0u;
    done[w] = target[w] <= 0;
  }

  while (hi >= 0 && !(done[0] && done[1])) {
    const int lo = hi >= 7 ? hi - 7 : 0;
    const uint32_t dmask = (2u << (hi - lo)) - 1u;
    const uint64_t above = ~((2ull << hi) - 1ull);
    const uint64_t from_lo = ~((1ull << lo) - 1ull);
    const bool shared = !done[0] && !done[1] && pref[0] == pref[1];
#pragma unroll
    for (int w = 0; w < 2; ++w) {
      if (done[w] || (shared && w == 1)) continue;
      *reinterpret_cast<u32x2*>(wh + 2 * lane) = u32x2{0u, 0u};
      const uint64_t pw = pref[w];
#pragma unroll
      for (int u = 0; u < KPL; ++u) {
        if (64 * u >= nkb) break;
        if (lane + 64 * u < nkb && ((kk[u] ^ pw) & above) == 0ull) {
          const uint32_t bin = static_cast<uint32_t>(kk[u] >> lo) & dmask;
          atomicAdd(&wh[bin >> 1], 1u << (16 * (bin & 1)));
        }
      }
      lds_wait();
      const u32x2 cw = *reinterpret_cast<const u32x2*>(wh + 2 * lane);
      const u32x4 c = u32x4{cw[0] & 0xffffu, cw[0] >> 16, cw[1] & 0xffffu, cw[1] >> 16};
      const uint32_t tot = c[0] + c[1] + c[2] + c[3];
      const uint32_t incl = wave_incl_scan(tot, lane);
      const uint32_t excl = incl - tot;
#pragma unroll
      for (int ww = 0; ww < 2; ++ww) {
        if (ww != w && !shared) continue;
        const uint32_t rr = rem[ww];
        const bool mine = rr >= excl && rr < incl;
        uint32_t bin = 4u * lane, cum = excl, cnt = c[0];
        if (mine && rr >= cum + c[0]) {
          cum += c[0]; ++bin; cnt = c[1];
          if (rr >= cum + c[1]) {
            cum += c[1]; ++bin; cnt = c[2];
            if (rr >= cum + c[2]) { cum += c[2]; ++bin; cnt = c[3]; }
          }
        }
        const int src = __builtin_ctzll(__ballot(mine));
        const uint32_t b_bin = __builtin_amdgcn_readlane(bin, src);
        const uint32_t b_cum = __builtin_amdgcn_readlane(cum, src);
        const uint32_t b_cnt = __builtin_amdgcn_readlane(cnt, src);
        pref[ww] |= static_cast<uint64_t>(b_bin) << lo;
        rem[ww] -= b_cum;
        if (b_cnt == 1u) {
          // the bin holds one key: it is the cut
          const uint64_t pv = pref[ww];
          uint64_t key = pv;
#pragma unroll
          for (int u = 0; u < KPL; ++u) {
            if (64 * u >= nkb) break;
            const uint64_t bm = __ballot(lane + 64 * u < nkb && ((kk[u] ^ pv) & from_lo) == 0ull);
            if (bm) key = readlane64(kk[u], __builtin_ctzll(bm));
          }
          pref[ww] = key;
          rem[ww] = 0u;
          done[ww] = true;
        }
      }
      lds_wait();
    }
    hi = lo - 1;
  }

  // classes (equal keys ranked by ascending j) and compaction
  const uint64_t lt_mask = (1ull << lane) - 1ull;
  uint32_t eq_base[2] = {0u, 0u};
  uint32_t out_base[2] = {0u, 0u};
#pragma unroll
  for (int u = 0; u < KPL; ++u) {
    if (64 * u >= nkb) break;
    const int j = lane + 64 * u;
    const uint64_t kv = kk[u];
    bool in_w[2];
#pragma unroll
    for (int w = 0; w < 2; ++w) {
      const uint64_t eqb = __ballot(kv == pref[w] && j < nkb);
      const uint32_t tie_rank = eq_base[w] + static_cast<uint32_t>(__popcll(eqb & lt_mask));
      in_w[w] = target[w] > 0 && (kv < pref[w] || (kv == pref[w] && tie_rank <= rem[w]));
      eq_base[w] += static_cast<uint32_t>(__popcll(eqb));
    }
    const bool ok = j < nkb;
    const int c = !ok ? 0 : (in_w[0] ? 2 : (in_w[1] ? 1 : 0));
    const uint64_t b2 = __ballot(c == 2);
    const uint64_t b1 = __ballot(c == 1);
    const uint32_t p2 = out_base[0] + static_cast<uint32_t>(__popcll(b2 & lt_mask));
    const uint32_t p1 = out_base[1] + static_cast<uint32_t>(__popcll(b1 & lt_mask));
    out_base[0] += static_cast<uint32_t>(__popcll(b2));
    out_base[1] += static_cast<uint32_t>(__popcll(b1));
    if (ok) {
      if (cls) cls[row * nkb + j] = static_cast<int8_t>(c);
      if (c == 2 && p2 < static_cast<uint32_t>(k_crit)) crit[row * k_crit + p2] = j;
      else if (c == 1 && p1 < static_cast<uint32_t>(k_marg)) marg[row * k_marg + p1] = j;
    }
  }
}

// grid (ceil(nq / R), B*H), dynamic LDS: keys [R][nkbp] u64, per-wave
// histograms of 256 16-bit bins packed two to a word ([4][128] u32; a bin
// never counts more than nkb <= 4096 keys).
//
// Phase 1 (whole workgroup): thread t owns KV blocks j = t + 512 m and
// t + 256 + 512 m and computes the float64 logits of the R query blocks
// against them, so each pooled-K value read serves R logits; the pooled-Q
// rows are uniform across the workgroup and are read as scalar operands,
// each serving two logits.  Results go to LDS as keys.
// TAYLOR accumulates the second-order term beside the dot product, from the
// same scalar pooled-Q values squared and the block variances laid out like
// the pooled K.
// Phase 2: one wave per query block (select_row).
constexpr int kFC = 4;

template <int R, int KPL, bool TAYLOR>
__global__ void __launch_bounds__(kThreads)
select_kernel(Geometry g, int nkbp, const double* __restrict__ qpool,
              const double* __restrict__ kpool_t, const double* __restrict__ kvar_t,
              double sqrt_d, double inv_2d, int32_t* __restrict__ crit,
              int32_t* __restrict__ marg, int8_t* __restrict__ cls,
              float* __restrict__ logits_out) {
  extern __shared__ __attribute__((aligned(16))) unsigned char dyn[];
  uint64_t* keys = reinterpret_cast<uint64_t*>(dyn);                 // [R][nkbp]
  uint32_t* hist = reinterpret_cast<uint32_t*>(keys + R * nkbp);      // [4][128]

  // One-dimensional grid of row groups x B*H, the row group fastest in the
  // logical order and each XCD given a contiguous range of it: an XCD then
  // works through its heads one at a time, and the head's pooled keys,
  // which every row group reads in full, stay in its L2.
  const int nq = g.nq, nkb = g.nkb, D = g.D;
  const int ngroups = (nq + R - 1) / R;
  const int logical = xcd_remap(blockIdx.x, ngroups * g.B * g.H);
  const int bh = logical / ngroups;
  const int i0 = (logical % ngroups) * R;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;

  const double* qrow[R];
#pragma unroll
  for (int r = 0; r < R; ++r)
    qrow[r] = qpool + (static_cast<int64_t>(bh) * nq + min(i0 + r, nq - 1)) * D;
  const double* kt = kpool_t + static_cast<int64_t>(bh) * D * nkb;
  const double* vt = TAYLOR ? kvar_t + static_cast<int64_t>(bh) * D * nkb : nullptr;

  // Two KV blocks per thread (j and j + 256); kFC features per step, the next
  // step's pooled-K values loaded before this step's FMAs.
  for (int j0 = t; j0 < nkbp; j0 += 2 * kThreads) {
    const int jj[2] = {j0, j0 + kThreads};
    const int64_t jl[2] = {jj[0] < nkb ? jj[0] : 0, jj[1] < nkb ? jj[1] : 0};
    double acc[2][R], acc2[TAYLOR ? 2 : 1][TAYLOR ? R : 1];
#pragma unroll
    for (int x = 0; x < 2; ++x)
#pragma unroll
      for (int r = 0; r < R; ++r) {
        acc[x][r] = 0.0;
        if constexpr (TAYLOR) acc2[x][r] = 0.0;
      }
    const int qz = 0;
    double kv[2][kFC], qv[R][kFC];
    double vv[TAYLOR ? 2 : 1][kFC], vn[TAYLOR ? 2 : 1][kFC];
#pragma unroll
    for (int e = 0; e < kFC; ++e) {
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        kv[x][e] = kt[static_cast<int64_t>(e) * nkb + jl[x]];
        if constexpr (TAYLOR) vv[x][e] = vt[static_cast<int64_t>(e) * nkb + jl[x]];
      }
#pragma unroll
      for (int r = 0; r < R; ++r) qv[r][e] = qrow[r][e + qz];
    }
#pragma unroll 2
    for (int a0 = 0; a0 < D; a0 += kFC) {
      const int an = a0 + kFC < D ? a0 + kFC : a0;
      double kn[2][kFC], qn[R][kFC];
#pragma unroll
      for (int e = 0; e < kFC; ++e) {
#pragma unroll
        for (int x = 0; x < 2; ++x) {
          kn[x][e] = kt[static_cast<int64_t>(an + e) * nkb + jl[x]];
          if constexpr (TAYLOR) vn[x][e] = vt[static_cast<int64_t>(an + e) * nkb + jl[x]];
        }
#pragma unroll
        for (int r = 0; r < R; ++r) qn[r][e] = qrow[r][an + e + qz];
      }
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int e = 0; e < kFC; ++e) {
          acc[0][r] = fma(qv[r][e], kv[0][e], acc[0][r]);
          acc[1][r] = fma(qv[r][e], kv[1][e], acc[1][r]);
          if constexpr (TAYLOR) {
            const double q2 = qv[r][e] * qv[r][e];
            acc2[0][r] = fma(q2, vv[0][e], acc2[0][r]);
            acc2[1][r] = fma(q2, vv[1][e], acc2[1][r]);
          }
        }
#pragma unroll
      for (int e = 0; e < kFC; ++e) {
#pragma unroll
        for (int x = 0; x < 2; ++x) {
          kv[x][e] = kn[x][e];
          if constexpr (TAYLOR) vv[x][e] = vn[x][e];
        }
#pragma unroll
        for (int r = 0; r < R; ++r) qv[r][e] = qn[r][e];
      }
    }
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      const int j = jj[x];
      if (j >= nkbp) continue;
#pragma unroll
      for (int r = 0; r < R; ++r) {
        double sv = acc[x][r] / sqrt_d;
        if constexpr (TAYLOR) sv += log1p(acc2[x][r] * inv_2d);
        const bool ok = i0 + r < nq && j < nkb;
        keys[r * nkbp + j] = ok ? desc_key(sv) : ~0ull;
        if (ok && logits_out)
          logits_out[(static_cast<int64_t>(bh) * nq + i0 + r) * nkb + j] = static_cast<float>(sv);
      }
    }
  }
  __syncthreads();

  for (int r = wave; r < R; r += 4) {
    const int i = i0 + r;
    if (i >= nq) break;
    select_row<KPL>(keys + r * nkbp, nkb, lane, hist + wave * 128, g.k_crit, g.k_marg,
                    static_cast<int64_t>(bh) * nq + i, crit, marg, cls);
  }
}

template <int R, int KPL, bool TAYLOR>
hipError_t launch_select_rk(const Geometry& g, int nkbp, const double* qpool,
                            const double* kpool_t, const double* kvar_t, int32_t* crit,
                            int32_t* marg, int8_t* cls, float* logits, hipStream_t stream) {
  const size_t lds = static_cast<size_t>(R) * nkbp * 8 + 4 * 128 * 4;
  if (lds > 65536) {
    // more than 64 KB of dynamic LDS has to be allowed for the kernel (on
    // the current device)
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&select_kernel<R, KPL, TAYLOR>),
                                             hipFuncAttributeMaxDynamicSharedMemorySize,
                                             static_cast<int>(lds));
    if (e != hipSuccess) return e;
  }
  dim3 grid(((g.nq + R - 1) / R) * g.B * g.H);
  const double sqrt_d = __builtin_sqrt(static_cast<double>(g.D));
  const double inv_2d = 1.0 / (2.0 * g.D);
  hipLaunchKernelGGL((select_kernel<R, KPL, TAYLOR>), grid, dim3(kThreads), lds, stream, g, nkbp,
                     qpool, kpool_t, kvar_t, sqrt_d, inv_2d, crit, marg, cls, logits);
  return hipGetLastError();
}

// Eight query rows per workgroup (every pooled-K value read serves eight
// logits) up to nkb = 1024, then four and two, so that the key rows stay
// within 64 KB of LDS and several workgroups share a CU (the kernel is
// latency-bound; at nkb = 1182 four rows measured faster than eight).  Keys
// per lane cover the row (nkb <= 4096).
template <bool TAYLOR>
hipError_t launch_select(const Geometry& g, const double* qpool, const double* kpool_t,
                         const double* kvar_t, int32_t* crit, int32_t* marg, int8_t* cls,
                         float* logits, hipStream_t stream) {
  const int nkbp = (g.nkb + 63) / 64 * 64;
  if (nkbp <= 128)
    return launch_select_rk<8, 2, TAYLOR>(g, nkbp, qpool, kpool_t, kvar_t, crit, marg, cls, logits, stream);
  if (nkbp <= 512)
    return launch_select_rk<8, 8, TAYLOR>(g, nkbp, qpool, kpool_t, kvar_t, crit, marg, cls, logits, stream);
  if (nkbp <= 1024)
    return launch_select_rk<8, 16, TAYLOR>(g, nkbp, qpool, kpool_t, kvar_t, crit, marg, cls, logits, stream);
  if (nkbp <= 2048)
    return launch_select_rk<4, 32, TAYLOR>(g, nkbp, qpool, kpool_t, kvar_t, crit, marg, cls, logits, stream);
  return launch_select_rk<2, 64, TAYLOR>(g, nkbp, qpool, kpool_t, kvar_t, crit, marg, cls, logits, stream);
}

template <typename T, int D>
void launch_pool_t(const Geometry& g, const void* q, const void* k, double* qpool, double* kpool_t,
                   float* qo, float* ko, double* kvar_t, float* vo, hipStream_t stream) {
  dim3 grid(g.nq, g.B * g.H, 2);
  if (kvar_t)
    hipLaunchKernelGGL((pool_kernel<T, D, true>), grid, dim3(kThreads), 0, stream,
                       static_cast<const T*>(q), static_cast<const T*>(k), g, qpool, kpool_t, qo,
                       ko, kvar_t, vo);
  else
    hipLaunchKernelGGL((pool_kernel<T, D, false>), grid, dim3(kThreads), 0, stream,
                       static_cast<const T*>(q), static_cast<const T*>(k), g, qpool, kpool_t, qo,
                       ko, nullptr, nullptr);
}

}  // namespace

hipError_t launch_route(const Geometry& g, const void* q, const void* k, int32_t* crit,
                        int32_t* marg, int8_t* cls, float* logits, float* pooled_q,
                        float* pooled_k, double* ws_qpool, double* ws_kpool_t,
                        double* ws_kvar_t, float* key_var, hipStream_t stream) {
  if (g.dtype == 1) {
    if (g.D == 128)
      launch_pool_t<uint16_t, 128>(g, q, k, ws_qpool, ws_kpool_t, pooled_q, pooled_k, ws_kvar_t, key_var, stream);
    else
      launch_pool_t<uint16_t, 64>(g, q, k, ws_qpool, ws_kpool_t, pooled_q, pooled_k, ws_kvar_t, key_var, stream);
  } else {
    if (g.D == 128)
      launch_pool_t<float, 128>(g, q, k, ws_qpool, ws_kpool_t, pooled_q, pooled_k, ws_kvar_t, key_var, stream);
    else
      launch_pool_t<float, 64>(g, q, k, ws_qpool, ws_kpool_t, pooled_q, pooled_k, ws_kvar_t, key_var, stream);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (ws_kvar_t)
    return launch_select<true>(g, ws_qpool, ws_kpool_t, ws_kvar_t, crit, marg, cls, logits, stream);
  return launch_select<false>(g, ws_qpool, ws_kpool_t, nullptr, crit, marg, cls, logits, stream);
}

}  // namespace sla
