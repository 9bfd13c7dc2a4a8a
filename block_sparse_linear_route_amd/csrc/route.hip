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
#include "fp8_encode.hpp"
#include "sla_internal.hpp"

namespace sla {
namespace {

// ---------------------------------------------------------------- pooling
// One-dimensional grid of nb x B*H x nwhich (Q, then K when nwhich = 2;
// Q alone when the states pass pooled K) blocks, the block index
// fastest in the logical order and each XCD given a contiguous range of it.
// Pooled K (and the key variances) go out as rows [B*H][nkb][d] when k_rows
// is set (the split selection, whose logits kernel stages them like pooled
// Q: one 1 KB row per block), else transposed [B*H][d][nkb] for the fused
// selection kernel, each of whose threads walks one block's column; there
// the 8-byte entries of neighbouring blocks, which run on one XCD, meet in
// the same L2 lines before those are written back.  One workgroup per block:
// thread t reads the 16-byte chunk t % CH of rows t / CH + RG m (rows past
// a ragged end load the block's last row and are zeroed, so every load is in
// flight at once), then LDS sums the row groups in float64.  VAR adds, for
// K blocks, a second pass: squared deviations from the block mean, summed
// the same way.  QNT (low-bit sparse branch) also writes the block's E4M3
// codes and float32 scale ([SLA2 technical summary, section 2.C]; the bytes
// of the stand-alone quantiser) from the tile already in registers.
template <typename T, int D, bool VAR, bool QNT = false>
__global__ void __launch_bounds__(kThreads)
pool_kernel(const T* __restrict__ q, const T* __restrict__ k, Geometry g, int nwhich, int k_rows,
            double* __restrict__ qpool, double* __restrict__ kpool,
            float* __restrict__ qout, float* __restrict__ kout,
            double* __restrict__ kvar, float* __restrict__ vout,
            uint8_t* __restrict__ q8 = nullptr, float* __restrict__ q_scale = nullptr,
            uint8_t* __restrict__ k8 = nullptr, float* __restrict__ k_scale = nullptr) {
  constexpr int CH = D / 8;           // 8-element chunks per row
  constexpr int RG = kThreads / CH;   // row groups
  constexpr int RPG = kBlock / RG;    // rows per group
  __shared__ double red[RG][D];
  __shared__ double mean_s[VAR ? D : 1];

  const int bhn = g.B * g.H;
  const int logical = xcd_remap(blockIdx.x, g.nq * bhn * nwhich);
  const int j = logical % g.nq;
  const int bh = (logical / g.nq) % bhn;
  const int which = logical / (g.nq * bhn);
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
  if constexpr (QNT) {
    __shared__ float wmax[4];
    float amax = 0.0f;
#pragma unroll
    for (int rr = 0; rr < RPG; ++rr)
#pragma unroll
      for (int e = 0; e < 8; ++e) amax = fmaxf(amax, rg + rr * RG < nj ? fabsf(f[rr][e]) : 0.0f);
    amax = workgroup_max4(amax, wmax);     // (its barrier also publishes red)
    const float r = e4m3_block_factor(amax);
    uint8_t* codes = (which == 0 ? q8 : k8) + (static_cast<int64_t>(bh) * g.N + row0) * D + ch * 8;
    if (t == 0) (which == 0 ? q_scale : k_scale)[static_cast<int64_t>(bh) * g.nq + j] = e4m3_block_scale(amax);
#pragma unroll
    for (int rr = 0; rr < RPG; ++rr)
      if (rg + rr * RG < nj)
        *reinterpret_cast<u32x2*>(codes + static_cast<int64_t>(rg + rr * RG) * D) = e4m3_pack8(f[rr], r);
  }
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
      kpool[k_rows ? (static_cast<int64_t>(bh) * g.nkb + j) * D + t
                   : (static_cast<int64_t>(bh) * D + t) * g.nkb + j] = m;
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
        kvar[k_rows ? (static_cast<int64_t>(bh) * g.nkb + j) * D + t
                    : (static_cast<int64_t>(bh) * D + t) * g.nkb + j] = var;
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
// search ends as soon as that bin holds a single key: that key is the cut,
// and as no other key shares its bits from the window's low end up, the cut
// is recorded as that prefix with every lower bit set (the largest key with
// the prefix), which ranks every key exactly as the cut itself would.
// If all 64 bits are consumed, the remaining rank counts equal keys, which
// are taken in ascending KV block order.
//
// Histogram (wh, kHistWords u32 per wave): kHistCopies copies of 256 bins,
// lane l counting into copy l / 16.  In the first passes most keys share one
// or two digits (the window holds the sign and the exponent), and LDS atomics
// on one word from many lanes are serialised; successive copies start
// kHistStride = 264 words apart, i.e. 8 banks further on, so the four copies
// of a bin sit in different banks and the lanes of one instruction split
// four ways.
constexpr int kHistBins = 256;
constexpr int kHistCopies = 4;
constexpr int kHistStride = kHistBins + 8;
constexpr int kHistWords = kHistCopies * kHistStride;
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
    // keys sharing a prefix p (bits above hi; p is zero from hi down) are
    // those with key - p <= lim, and their digit is (key - p) >> lo < 256
    const uint64_t lim = (2ull << hi) - 1ull;
    const bool shared = !done[0] && !done[1] && pref[0] == pref[1];
#pragma unroll
    for (int w = 0; w < 2; ++w) {
      if (done[w] || (shared && w == 1)) continue;
#pragma unroll
      for (int h = 0; h < kHistCopies; ++h)
        *reinterpret_cast<u32x4*>(wh + h * kHistStride + 4 * lane) = u32x4{0u, 0u, 0u, 0u};
      const uint64_t pw = pref[w];
      uint32_t* whl = wh + (lane >> 4) * kHistStride;
#pragma unroll
      for (int u = 0; u < KPL; ++u) {
        if (64 * u >= nkb) break;
        const uint64_t dk = kk[u] - pw;
        if (lane + 64 * u < nkb && dk <= lim) atomicAdd(&whl[static_cast<uint32_t>(dk >> lo)], 1u);
      }
      lds_wait();
      u32x4 c = *reinterpret_cast<const u32x4*>(wh + 4 * lane);
#pragma unroll
      for (int h = 1; h < kHistCopies; ++h)
        c += *reinterpret_cast<const u32x4*>(wh + h * kHistStride + 4 * lane);
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
          // the bin holds one key, the cut: no other key shares its bits
          // from lo up, so the largest key with that prefix stands in for it
          pref[ww] |= (1ull << lo) - 1ull;
          rem[ww] = 0u;
          done[ww] = true;
        }
      }
      lds_wait();
    }
    hi = lo - 1;
  }

  // classes (equal keys ranked by ascending j) and compaction.  A cut left
  // open when the bits ran out sits among equal keys, which need their tie
  // ranks; a cut found as a single key (or an empty target) does not.
  const uint64_t lt_mask = (1ull << lane) - 1ull;
  auto compact = [&](auto ties_c) {
    constexpr bool TIES = decltype(ties_c)::value;
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
        if constexpr (TIES) {
          const uint64_t eqb = __ballot(kv == pref[w] && j < nkb);
          const uint32_t tie_rank = eq_base[w] + static_cast<uint32_t>(__popcll(eqb & lt_mask));
          in_w[w] = target[w] > 0 && (kv < pref[w] || (kv == pref[w] && tie_rank <= rem[w]));
          eq_base[w] += static_cast<uint32_t>(__popcll(eqb));
        } else {
          in_w[w] = target[w] > 0 && kv <= pref[w];
        }
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
  };
  if (done[0] && done[1]) compact(std::false_type{});
  else compact(std::true_type{});
}

// The fused routing kernel (plain score; the routing path of
// sla_route_noalloc, whose static scratch holds no key buffer).
// One-dimensional grid of ceil(nq / R) row groups x B*H, dynamic LDS: keys
// [R][nkbp] u64, then the four waves' histograms ([4][kHistWords] u32).
//
// Phase 1 (whole workgroup): thread t owns KV blocks j = t + 512 m and
// t + 256 + 512 m and computes the float64 logits of the R query blocks
// against them, so each pooled-K value read serves R logits; the pooled-Q
// rows are uniform across the workgroup and are read as scalar operands,
// each serving two logits.  Each logit is one FMA chain over the features in
// ascending order, divided by sqrt(d).  Results go to LDS as keys.
// Phase 2: one wave per query block (select_row).
constexpr int kFC = 4;

template <int R, int KPL>
__global__ void __launch_bounds__(kThreads)
select_kernel(Geometry g, int nkbp, const double* __restrict__ qpool,
              const double* __restrict__ kpool_t, double sqrt_d, int32_t* __restrict__ crit,
              int32_t* __restrict__ marg, int8_t* __restrict__ cls,
              float* __restrict__ logits_out) {
  extern __shared__ __attribute__((aligned(16))) unsigned char dyn[];
  uint64_t* keys = reinterpret_cast<uint64_t*>(dyn);                 // [R][nkbp]
  uint32_t* hist = reinterpret_cast<uint32_t*>(keys + R * nkbp);      // [4][kHistWords]

  // The row group fastest in the logical order and each XCD given a
  // contiguous range of it: an XCD then works through its heads one at a
  // time, and the head's pooled keys, which every row group reads in full,
  // stay in its L2.
  const int nq = g.nq, nkb = g.nkb, D = g.D;
  const int ngroups = (nq + R - 1) / R;
  const int logical = xcd_remap(blockIdx.x, ngroups * g.B * g.H);
  const int bh = logical / ngroups;
  const int i0 = (logical % ngroups) * R;
  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);   // wave-uniform (scalar)

  const double* qrow[R];
#pragma unroll
  for (int r = 0; r < R; ++r)
    qrow[r] = qpool + (static_cast<int64_t>(bh) * nq + min(i0 + r, nq - 1)) * D;
  const double* kt = kpool_t + static_cast<int64_t>(bh) * D * nkb;

  // Two KV blocks per thread (j and j + 256); kFC features per step, the next
  // step's pooled-K values loaded before this step's FMAs.
  for (int j0 = t; j0 < nkbp; j0 += 2 * kThreads) {
    const int jj[2] = {j0, j0 + kThreads};
    const int64_t jl[2] = {jj[0] < nkb ? jj[0] : 0, jj[1] < nkb ? jj[1] : 0};
    double acc[2][R];
#pragma unroll
    for (int x = 0; x < 2; ++x)
#pragma unroll
      for (int r = 0; r < R; ++r) acc[x][r] = 0.0;
    double kv[2][kFC], qv[R][kFC];
#pragma unroll
    for (int e = 0; e < kFC; ++e) {
#pragma unroll
      for (int x = 0; x < 2; ++x) kv[x][e] = kt[static_cast<int64_t>(e) * nkb + jl[x]];
#pragma unroll
      for (int r = 0; r < R; ++r) qv[r][e] = qrow[r][e];
    }
#pragma unroll 2
    for (int a0 = 0; a0 < D; a0 += kFC) {
      const int an = a0 + kFC < D ? a0 + kFC : a0;
      double kn[2][kFC], qn[R][kFC];
#pragma unroll
      for (int e = 0; e < kFC; ++e) {
#pragma unroll
        for (int x = 0; x < 2; ++x) kn[x][e] = kt[static_cast<int64_t>(an + e) * nkb + jl[x]];
#pragma unroll
        for (int r = 0; r < R; ++r) qn[r][e] = qrow[r][an + e];
      }
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int e = 0; e < kFC; ++e) {
          acc[0][r] = fma(qv[r][e], kv[0][e], acc[0][r]);
          acc[1][r] = fma(qv[r][e], kv[1][e], acc[1][r]);
        }
#pragma unroll
      for (int e = 0; e < kFC; ++e) {
#pragma unroll
        for (int x = 0; x < 2; ++x) kv[x][e] = kn[x][e];
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
        const double sv = acc[x][r] / sqrt_d;
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
    select_row<KPL>(keys + r * nkbp, nkb, lane, hist + wave * kHistWords, g.k_crit, g.k_marg,
                    static_cast<int64_t>(bh) * nq + i, crit, marg, cls);
  }
}

template <int R, int KPL>
hipError_t launch_select_rk(const Geometry& g, int nkbp, const double* qpool,
                            const double* kpool_t, int32_t* crit, int32_t* marg, int8_t* cls,
                            float* logits, hipStream_t stream) {
  const size_t lds = static_cast<size_t>(R) * nkbp * 8 + 4 * kHistWords * 4;
  if (lds > 65536) {
    // more than 64 KB of dynamic LDS has to be allowed for the kernel (on
    // the current device)
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&select_kernel<R, KPL>),
                                             hipFuncAttributeMaxDynamicSharedMemorySize,
                                             static_cast<int>(lds));
    if (e != hipSuccess) return e;
  }
  dim3 grid(((g.nq + R - 1) / R) * g.B * g.H);
  const double sqrt_d = __builtin_sqrt(static_cast<double>(g.D));
  hipLaunchKernelGGL((select_kernel<R, KPL>), grid, dim3(kThreads), lds, stream, g, nkbp, qpool,
                     kpool_t, sqrt_d, crit, marg, cls, logits);
  return hipGetLastError();
}

// ------------------------------------------------- split selection
// Given workspace for them, the logits and the selection run as two kernels
// with the keys in between in memory ([heads][nq][nkbp] u64, ~0 past nkb).
//
// logits_kernel: one workgroup per 64 x 64 tile of (query block, KV block)
// pairs of one head, each wave a 32 x 32 quarter of it as 2 x 2 products
// on the float64 matrix cores (v_mfma_f64_16x16x4_f64).  The pooled rows go
// through LDS 16 features at a time (the next chunk loaded into registers
// while the current one is used), so each pooled value read from L2 serves
// 64 logits; in the fused kernel a row group reads the head's whole pooled
// K for R rows.  The matrix core accumulates each output as a chain of
// fused multiply-adds over its four k-slots in ascending order (checked on
// the device against the plain FMA chain: bit-equal on random operands
// spanning 2^40 in magnitude, where a single-rounding four-term dot or a
// tree of rounded products differs in ~80% of outputs), and the k-slots of
// successive products take features in ascending order, so each plain
// logit (then divided by sqrt(d)) is the fused kernel's FMA chain bit for
// bit.  SCORE 1 adds log1p(t / 2d), t a second such chain over the squared
// pooled queries (rounded once) and the key variances; SCORE 2 adds
// log1p(c_i M_j) with c_i = |qbar_i| / (sqrt(d) 64), the squares of qbar_i
// summed in ascending feature order.
//
// Operand layouts (16 x 16 x 4): A lane l holds row l % 16 at k-slot l / 16,
// B lane l holds k-slot l / 16 at column l % 16; the result's lane l holds
// rows l / 16 + 4 x (x = 0..3) at column l % 16.
constexpr int kLT = 64;   // tile rows and columns
constexpr int kLA = 16;   // features per LDS chunk
constexpr int kKS = kLA + 2;   // LDS row of a pooled-K chunk
typedef double f64x4 __attribute__((ext_vector_type(4)));

template <int SCORE>
__global__ void __launch_bounds__(kThreads)
logits_kernel(Geometry g, int nkbp, int bh0, int nbh, const double* __restrict__ qpool,
              const double* __restrict__ kpool, const double* __restrict__ kvar,
              const double* __restrict__ mdev, double sqrt_d, double inv_2d,
              uint64_t* __restrict__ keys, float* __restrict__ logits_out) {
  constexpr bool TAYLOR = SCORE == 1;
  constexpr bool COV = SCORE == 2;
  // pooled Q, K (and variances) row-major with rows of kKS = kLA + 2
  // values, so a thread's four features go in as two 16-byte stores and the
  // operand reads below spread over the banks
  __shared__ __attribute__((aligned(16))) double qs[kLT][kKS];
  __shared__ __attribute__((aligned(16))) double ks[kLT][kKS];
  __shared__ __attribute__((aligned(16))) double vs[TAYLOR ? kLT : 1][kKS];
  __shared__ double cq[COV ? kLT : 1];
  const int nq = g.nq, nkb = g.nkb, D = g.D;
  const int tr_n = (nq + kLT - 1) / kLT, tc_n = nkbp / kLT;
  const int logical = xcd_remap(blockIdx.x, tr_n * tc_n * nbh);
  const int ct = logical % tc_n;
  const int rt = (logical / tc_n) % tr_n;
  const int bhl = logical / (tc_n * tr_n);
  const int bh = bh0 + bhl;
  const int i0 = rt * kLT, j0 = ct * kLT;
  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);   // wave-uniform (scalar)
  const int wr = (wave >> 1) * 32, wc = (wave & 1) * 32;   // this wave's quarter
  const int l16 = lane & 15, kslot = lane >> 4;

  // staging, kSV values per thread: pooled-Q row i0 + t / 4 and pooled-K
  // (and variance) row j0 + t / 4, features kSV (t % 4) .. of the chunk;
  // rows past the end repeat the last
  constexpr int kSV = kLA / 4;
  const int sq_row = t >> 2, sq_a = (t & 3) * kSV;
  const double* gq = qpool + (static_cast<int64_t>(bh) * nq + min(i0 + sq_row, nq - 1)) * D + sq_a;
  const int64_t krow = (static_cast<int64_t>(bh) * nkb + min(j0 + sq_row, nkb - 1)) * D + sq_a;
  const double* gk = kpool + krow;
  const double* gv = TAYLOR ? kvar + krow : nullptr;
  double rq[kSV], rk[kSV], rv[TAYLOR ? kSV : 1];
  auto fetch = [&](int a0) {
#pragma unroll
    for (int n = 0; n < kSV; ++n) {
      rq[n] = gq[a0 + n];
      rk[n] = gk[a0 + n];
      if constexpr (TAYLOR) rv[n] = gv[a0 + n];
    }
  };

  f64x4 acc[2][2], acc2[TAYLOR ? 2 : 1][TAYLOR ? 2 : 1];
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int n = 0; n < 2; ++n) {
      acc[m][n] = f64x4{0.0, 0.0, 0.0, 0.0};
      if constexpr (TAYLOR) acc2[m][n] = f64x4{0.0, 0.0, 0.0, 0.0};
    }
  double ss = 0.0;   // COV: sum of squares of row t (t < 64)

  fetch(0);
  for (int a0 = 0; a0 < D; a0 += kLA) {
    __syncthreads();
#pragma unroll
    for (int n = 0; n < kSV; ++n) {
      qs[sq_row][sq_a + n] = rq[n];
      ks[sq_row][sq_a + n] = rk[n];
      if constexpr (TAYLOR) vs[sq_row][sq_a + n] = rv[n];
    }
    __syncthreads();
    if (a0 + kLA < D) fetch(a0 + kLA);
    if constexpr (COV) {
      if (t < kLT) {
#pragma unroll
        for (int a = 0; a < kLA; ++a) ss = fma(qs[t][a], qs[t][a], ss);
      }
    }
#pragma unroll
    for (int kk = 0; kk < kLA / 4; ++kk) {
      const int a = 4 * kk + kslot;
      double af[2], bf[2];
#pragma unroll
      for (int m = 0; m < 2; ++m) af[m] = qs[wr + 16 * m + l16][a];
#pragma unroll
      for (int n = 0; n < 2; ++n) bf[n] = ks[wc + 16 * n + l16][a];
#pragma unroll
      for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int n = 0; n < 2; ++n)
          acc[m][n] = __builtin_amdgcn_mfma_f64_16x16x4f64(af[m], bf[n], acc[m][n], 0, 0, 0);
      if constexpr (TAYLOR) {
        double vf[2];
#pragma unroll
        for (int n = 0; n < 2; ++n) vf[n] = vs[wc + 16 * n + l16][a];
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          const double q2 = af[m] * af[m];
#pragma unroll
          for (int n = 0; n < 2; ++n)
            acc2[m][n] = __builtin_amdgcn_mfma_f64_16x16x4f64(q2, vf[n], acc2[m][n], 0, 0, 0);
        }
      }
    }
  }
  if constexpr (COV) {
    if (t < kLT) cq[t] = sqrt(ss) * inv_2d;
    __syncthreads();
  }

#pragma unroll
  for (int n = 0; n < 2; ++n) {
    const int jl = wc + 16 * n + l16;
    const int j = j0 + jl;
    const double md = COV && j < nkb ? mdev[static_cast<int64_t>(bh) * nkb + j] : 0.0;
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        const int il = wr + 16 * m + kslot + 4 * x;
        const int i = i0 + il;
        if (i >= nq) continue;
        double sv = acc[m][n][x] / sqrt_d;
        if constexpr (TAYLOR) sv += log1p(acc2[m][n][x] * inv_2d);
        if constexpr (COV) sv += log1p(cq[il] * md);
        keys[(static_cast<int64_t>(bhl) * nq + i) * nkbp + j] = j < nkb ? desc_key(sv) : ~0ull;
        if (j < nkb && logits_out)
          logits_out[(static_cast<int64_t>(bh) * nq + i) * nkb + j] = static_cast<float>(sv);
      }
  }
}

// select_rows_kernel: one wave per row of keys written by logits_kernel
// (select_row reading the row from memory); four rows per workgroup.
template <int KPL>
__global__ void __launch_bounds__(kThreads)
select_rows_kernel(Geometry g, int nkbp, int bh0, int nbh, const uint64_t* __restrict__ keys,
                   int32_t* __restrict__ crit, int32_t* __restrict__ marg,
                   int8_t* __restrict__ cls) {
  __shared__ __attribute__((aligned(16))) uint32_t hist[4][kHistWords];
  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);   // wave-uniform (scalar)
  const int r = blockIdx.x * 4 + wave;
  if (r >= nbh * g.nq) return;
  const int bhl = r / g.nq, i = r % g.nq;
  select_row<KPL>(keys + static_cast<int64_t>(r) * nkbp, g.nkb, lane, hist[wave], g.k_crit,
                  g.k_marg, static_cast<int64_t>(bh0 + bhl) * g.nq + i, crit, marg, cls);
}

template <int SCORE>
hipError_t launch_select_split(const Geometry& g, const double* qpool, const double* kpool,
                               const double* kvar, const double* mdev, uint64_t* keys,
                               int32_t* crit, int32_t* marg, int8_t* cls, float* logits,
                               hipStream_t stream) {
  const int nkbp = (g.nkb + 63) / 64 * 64;
  const int bh_all = g.B * g.H;
  const int chunk = route_key_heads(g);
  const double sqrt_d = __builtin_sqrt(static_cast<double>(g.D));
  const double inv_2d = SCORE == 2 ? 1.0 / (sqrt_d * kBlock) : 1.0 / (2.0 * g.D);
  const int tiles = ((g.nq + kLT - 1) / kLT) * (nkbp / kLT);
  for (int bh0 = 0; bh0 < bh_all; bh0 += chunk) {
    const int nbh = bh_all - bh0 < chunk ? bh_all - bh0 : chunk;
    hipLaunchKernelGGL((logits_kernel<SCORE>), dim3(tiles * nbh), dim3(kThreads), 0, stream, g,
                       nkbp, bh0, nbh, qpool, kpool, kvar, mdev, sqrt_d, inv_2d, keys, logits);
    const dim3 sg((nbh * g.nq + 3) / 4);
    if (nkbp <= 128)
      hipLaunchKernelGGL((select_rows_kernel<2>), sg, dim3(kThreads), 0, stream, g, nkbp, bh0, nbh, keys, crit, marg, cls);
    else if (nkbp <= 512)
      hipLaunchKernelGGL((select_rows_kernel<8>), sg, dim3(kThreads), 0, stream, g, nkbp, bh0, nbh, keys, crit, marg, cls);
    else if (nkbp <= 1024)
      hipLaunchKernelGGL((select_rows_kernel<16>), sg, dim3(kThreads), 0, stream, g, nkbp, bh0, nbh, keys, crit, marg, cls);
    else if (nkbp <= 1536)
      hipLaunchKernelGGL((select_rows_kernel<24>), sg, dim3(kThreads), 0, stream, g, nkbp, bh0, nbh, keys, crit, marg, cls);
    else if (nkbp <= 2048)
      hipLaunchKernelGGL((select_rows_kernel<32>), sg, dim3(kThreads), 0, stream, g, nkbp, bh0, nbh, keys, crit, marg, cls);
    else
      hipLaunchKernelGGL((select_rows_kernel<64>), sg, dim3(kThreads), 0, stream, g, nkbp, bh0, nbh, keys, crit, marg, cls);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// With key workspace (every score mode): the split path.  Without it (the
// plain score of sla_route_noalloc): the fused kernel, eight query rows per
// workgroup (every pooled-K value read serves eight logits) up to
// nkb = 1024, then four and two, so that the key rows stay within 64 KB of
// LDS and several workgroups share a CU (at nkb = 1182 four rows measured
// faster than eight).  Keys per lane cover the row (nkb <= 4096).
template <int SCORE>
// kpool (and kvar): rows [B*H][nkb][d] for the split path (keys non-null),
// transposed [B*H][d][nkb] for the fused kernel
hipError_t launch_select(const Geometry& g, const double* qpool, const double* kpool,
                         const double* kvar, const double* mdev, int32_t* crit, int32_t* marg,
                         int8_t* cls, float* logits, hipStream_t stream, uint64_t* keys) {
  if (keys)
    return launch_select_split<SCORE>(g, qpool, kpool, kvar, mdev, keys, crit, marg, cls,
                                      logits, stream);
  if (SCORE != 0) return hipErrorInvalidValue;   // the score modes always carry key workspace
  const int nkbp = (g.nkb + 63) / 64 * 64;
  if (nkbp <= 128) return launch_select_rk<8, 2>(g, nkbp, qpool, kpool, crit, marg, cls, logits, stream);
  if (nkbp <= 512) return launch_select_rk<8, 8>(g, nkbp, qpool, kpool, crit, marg, cls, logits, stream);
  if (nkbp <= 1024) return launch_select_rk<8, 16>(g, nkbp, qpool, kpool, crit, marg, cls, logits, stream);
  if (nkbp <= 2048) return launch_select_rk<4, 32>(g, nkbp, qpool, kpool, crit, marg, cls, logits, stream);
  return launch_select_rk<2, 64>(g, nkbp, qpool, kpool, crit, marg, cls, logits, stream);
}

template <typename T, int D>
void launch_pool_t(const Geometry& g, const void* q, const void* k, double* qpool, double* kpool,
                   float* qo, float* ko, double* kvar, float* vo, hipStream_t stream,
                   const Fp8Out* f8, int nwhich, int k_rows) {
  dim3 grid(g.nq * g.B * g.H * nwhich);
  if (f8)
    hipLaunchKernelGGL((pool_kernel<T, D, false, true>), grid, dim3(kThreads), 0, stream,
                       static_cast<const T*>(q), static_cast<const T*>(k), g, nwhich, k_rows, qpool,
                       kpool, qo, ko, nullptr, nullptr, f8->q8, f8->q_scale, f8->k8, f8->k_scale);
  else if (kvar)
    hipLaunchKernelGGL((pool_kernel<T, D, true>), grid, dim3(kThreads), 0, stream,
                       static_cast<const T*>(q), static_cast<const T*>(k), g, nwhich, k_rows, qpool,
                       kpool, qo, ko, kvar, vo);
  else
    hipLaunchKernelGGL((pool_kernel<T, D, false>), grid, dim3(kThreads), 0, stream,
                       static_cast<const T*>(q), static_cast<const T*>(k), g, nwhich, k_rows, qpool,
                       kpool, qo, ko, nullptr, nullptr);
}

}  // namespace

hipError_t launch_route(const Geometry& g, const void* q, const void* k, int32_t* crit,
                        int32_t* marg, int8_t* cls, float* logits, float* pooled_q,
                        float* pooled_k, double* ws_qpool, double* ws_kpool,
                        double* ws_kvar, float* key_var, hipStream_t stream,
                        const double* block_dev, const Fp8Out* f8, uint64_t* ws_keys,
                        bool k_pooled) {
  // the states pass writes pooled K in the split selection's row layout
  if (k_pooled && (f8 || ws_kvar || block_dev || !ws_keys)) return hipErrorInvalidValue;
  const int nwhich = k_pooled ? 1 : 2;
  const int k_rows = ws_keys != nullptr;
  if (g.dtype == 1) {
    if (g.D == 128)
      launch_pool_t<uint16_t, 128>(g, q, k, ws_qpool, ws_kpool, pooled_q, pooled_k, ws_kvar, key_var, stream, f8, nwhich, k_rows);
    else
      launch_pool_t<uint16_t, 64>(g, q, k, ws_qpool, ws_kpool, pooled_q, pooled_k, ws_kvar, key_var, stream, f8, nwhich, k_rows);
  } else {
    if (g.D == 128)
      launch_pool_t<float, 128>(g, q, k, ws_qpool, ws_kpool, pooled_q, pooled_k, ws_kvar, key_var, stream, f8, nwhich, k_rows);
    else
      launch_pool_t<float, 64>(g, q, k, ws_qpool, ws_kpool, pooled_q, pooled_k, ws_kvar, key_var, stream, f8, nwhich, k_rows);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (ws_kvar)
    return launch_select<1>(g, ws_qpool, ws_kpool, ws_kvar, nullptr, crit, marg, cls, logits, stream,
                             ws_keys);
  if (block_dev)
    return launch_select<2>(g, ws_qpool, ws_kpool, nullptr, block_dev, crit, marg, cls, logits, stream,
                             ws_keys);
  return launch_select<0>(g, ws_qpool, ws_kpool, nullptr, nullptr, crit, marg, cls, logits, stream,
                             ws_keys);
}

}  // namespace sla
