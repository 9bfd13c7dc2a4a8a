// Block routing: pooled Q/K, block logits and the three-way top-k split.
//
// [SLA2 technical summary, section 2.B] the router sees only Q and K, pools
// adjacent tokens so its cost stays far below O(N^2), and keeps a hard top-k
// at inference.  [SLA abstract] KV blocks of each query block fall into
// critical, marginal and negligible classes.
//
// Pooling sums bf16/f32 rows in float64 (exact for bf16 blocks) and divides
// by the valid token count; logits are float64 dot products divided by
// sqrt(d).  The selection is an exact 8-pass radix select over a 64-bit key
// that orders logits descending, so the split is the one the float64 logits
// define; equal logits are ordered by ascending KV block index.  Compaction
// writes each class's KV block indices in ascending order.
#include "device_common.hpp"
#include "sla_internal.hpp"

namespace sla {
namespace {

// ---------------------------------------------------------------- pooling
// grid (nb, B*H, 2): z = 0 pools Q, z = 1 pools K.  One workgroup per block.
template <typename T, int D>
__global__ void __launch_bounds__(kThreads)
pool_kernel(const T* __restrict__ q, const T* __restrict__ k, Geometry g,
            double* __restrict__ qpool, double* __restrict__ kpool_t,
            float* __restrict__ qout, float* __restrict__ kout) {
  constexpr int CH = D / 8;           // 8-element chunks per row
  constexpr int RG = kThreads / CH;   // row groups
  constexpr int RPG = kBlock / RG;    // rows per group
  __shared__ double red[RG][D];

  const int j = blockIdx.x;
  const int bh = blockIdx.y;
  const int which = blockIdx.z;
  const int b = bh / g.H, h = bh % g.H;
  const T* x = (which == 0 ? q : k) + b * g.sb + h * g.sh;
  const int t = threadIdx.x;
  const int ch = t % CH, rg = t / CH;
  const int row0 = j * kBlock;
  const int nj = min(kBlock, g.N - row0);

  double acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.0;
#pragma unroll
  for (int rr = 0; rr < RPG; ++rr) {
    const int r = rg + rr * RG;
    if (r < nj) {
      float f[8];
      load8_f32(x + static_cast<int64_t>(row0 + r) * g.sn + ch * 8, f);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] += static_cast<double>(f[e]);
    }
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

__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = __shfl_up(v, o, 64);
    if (lane >= o) v += y;
  }
  return v;
}

// ---------------------------------------------------------------- selection
// grid (ceil(nq / R), B*H), dynamic LDS: q rows [R][D] f64, keys [R][nkbp]
// u64, per-wave histograms [4][256] u32.
//
// Phase 1 (whole workgroup): float64 logits of the R query blocks against
// every KV block, thread t owning KV blocks j = t, t + 256, ... so each
// pooled-K column read serves all R rows; stored as 64-bit descending keys.
// Phase 2 (one wave per row, no further workgroup barriers): an 8-pass radix
// select finds, for each of the two cut counts k_crit and k_crit + k_marg,
// the key of the element at that rank and how many elements equal to it
// fall inside the cut (equal keys are taken in ascending j); classes follow,
// then ballot prefix counts compact each class in ascending j.

__device__ __forceinline__ void lds_wait() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

template <int D>
__global__ void __launch_bounds__(kThreads)
select_kernel(Geometry g, int R, int nkbp, const double* __restrict__ qpool,
              const double* __restrict__ kpool_t, double sqrt_d, int32_t* __restrict__ crit,
              int32_t* __restrict__ marg, int8_t* __restrict__ cls,
              float* __restrict__ logits_out) {
  extern __shared__ __attribute__((aligned(16))) unsigned char dyn[];
  double* qs = reinterpret_cast<double*>(dyn);                       // [R][D]
  uint64_t* keys = reinterpret_cast<uint64_t*>(qs + R * D);           // [R][nkbp]
  uint32_t* hist = reinterpret_cast<uint32_t*>(keys + R * nkbp);      // [4][256]

  const int bh = blockIdx.y;
  const int i0 = blockIdx.x * R;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int nq = g.nq, nkb = g.nkb;

  for (int e = t; e < R * D; e += kThreads) {
    const int r = e / D, a = e % D;
    const int i = i0 + r;
    qs[e] = (i < nq) ? qpool[(static_cast<int64_t>(bh) * nq + i) * D + a] : 0.0;
  }
  __syncthreads();

  // ---- phase 1: logits -> keys
  const double* kt = kpool_t + static_cast<int64_t>(bh) * D * nkb;
  for (int j = t; j < nkbp; j += kThreads) {
    if (j >= nkb) {
      for (int r = 0; r < R; ++r) keys[r * nkbp + j] = ~0ull;
      continue;
    }
    double acc[8];
#pragma unroll
    for (int r = 0; r < 8; ++r) acc[r] = 0.0;
#pragma unroll 1
    for (int a0 = 0; a0 < D; a0 += 16) {
      double kv[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) kv[u] = kt[static_cast<int64_t>(a0 + u) * nkb + j];
#pragma unroll
      for (int u = 0; u < 16; ++u)
#pragma unroll
        for (int r = 0; r < 8; ++r)
          if (r < R) acc[r] = fma(qs[r * D + a0 + u], kv[u], acc[r]);
    }
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      if (r >= R) break;
      const double sv = acc[r] / sqrt_d;
      const bool ok = i0 + r < nq;
      keys[r * nkbp + j] = ok ? desc_key(sv) : ~0ull;
      if (ok && logits_out)
        logits_out[(static_cast<int64_t>(bh) * nq + i0 + r) * nkb + j] = static_cast<float>(sv);
    }
  }
  __syncthreads();

  // ---- phase 2: one wave per query block
  uint32_t* wh = hist + wave * 256;
  const uint64_t lt_mask = (1ull << lane) - 1ull;
  const int nu = nkbp / 64;
  const int target[2] = {g.k_crit, g.k_crit + g.k_marg};
  for (int r = wave; r < R; r += 4) {
    const int i = i0 + r;
    if (i >= nq) break;
    const uint64_t* rk = keys + r * nkbp;
    uint64_t pref[2] = {0ull, 0ull};
    uint32_t rem[2] = {target[0] > 0 ? static_cast<uint32_t>(target[0] - 1) : 0u,
                       target[1] > 0 ? static_cast<uint32_t>(target[1] - 1) : 0u};
    for (int pass = 0; pass < 8; ++pass) {
      const int shift = 56 - 8 * pass;
      // while both cuts share their prefix they share the histogram
      const bool shared = pref[0] == pref[1];
      for (int w = 0; w < (shared ? 1 : 2); ++w) {
#pragma unroll
        for (int x = 0; x < 4; ++x) wh[4 * lane + x] = 0u;
        lds_wait();
        for (int u = 0; u < nu; ++u) {
          const uint64_t kk = rk[lane + 64 * u];
          const bool match = (pass == 0) || (((kk ^ pref[w]) >> (shift + 8)) == 0ull);
          const uint32_t digit = static_cast<uint32_t>(kk >> shift) & 255u;
          if (pass == 0) {
            // the leading byte takes few values: one atomic per distinct digit
            uint64_t active = __ballot(true);
            while (active) {
              const int leader = __builtin_ctzll(active);
              const uint32_t dd = __builtin_amdgcn_readlane(digit, leader);
              const uint64_t same = __ballot(digit == dd);
              if (lane == leader) atomicAdd(&wh[dd], static_cast<uint32_t>(__popcll(same)));
              active &= ~same;
            }
          } else if (match) {
            atomicAdd(&wh[digit], 1u);
          }
        }
        lds_wait();
        const uint32_t c0 = wh[4 * lane], c1 = wh[4 * lane + 1], c2 = wh[4 * lane + 2],
                       c3 = wh[4 * lane + 3];
        const uint32_t tot = c0 + c1 + c2 + c3;
        const uint32_t incl = wave_incl_scan(tot, lane);
        const uint32_t excl = incl - tot;
#pragma unroll
        for (int ww = 0; ww < 2; ++ww) {
          if (!shared && ww != w) continue;
          const bool mine = rem[ww] >= excl && rem[ww] < incl;
          uint32_t bin = 4u * lane, cum = excl;
          if (mine) {
            if (rem[ww] >= cum + c0) { cum += c0; ++bin;
              if (rem[ww] >= cum + c1) { cum += c1; ++bin;
                if (rem[ww] >= cum + c2) { cum += c2; ++bin; } } }
          }
          const uint64_t who = __ballot(mine);
          const int src = __builtin_ctzll(who);
          const uint32_t b_bin = __builtin_amdgcn_readlane(bin, src);
          const uint32_t b_cum = __builtin_amdgcn_readlane(cum, src);
          pref[ww] |= static_cast<uint64_t>(b_bin) << shift;
          rem[ww] -= b_cum;
        }
        lds_wait();
      }
    }

    // classes (equal keys ranked by ascending j) and compaction
    const int64_t row = static_cast<int64_t>(bh) * nq + i;
    uint32_t eq_base[2] = {0u, 0u};
    uint32_t out_base[2] = {0u, 0u};
    for (int u = 0; u < nu; ++u) {
      const int j = lane + 64 * u;
      const uint64_t kk = rk[j];
      bool in_w[2];
#pragma unroll
      for (int w = 0; w < 2; ++w) {
        const uint64_t eqb = __ballot(kk == pref[w]);
        const uint32_t tie_rank = eq_base[w] + static_cast<uint32_t>(__popcll(eqb & lt_mask));
        in_w[w] = target[w] > 0 && (kk < pref[w] || (kk == pref[w] && tie_rank <= rem[w]));
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
        if (c == 2 && p2 < static_cast<uint32_t>(g.k_crit)) crit[row * g.k_crit + p2] = j;
        else if (c == 1 && p1 < static_cast<uint32_t>(g.k_marg)) marg[row * g.k_marg + p1] = j;
      }
    }
  }
}

hipError_t launch_select(const Geometry& g, const double* qpool, const double* kpool_t,
                         int32_t* crit, int32_t* marg, int8_t* cls, float* logits,
                         hipStream_t stream) {
  const int nkbp = (g.nkb + 63) / 64 * 64;
  int R = static_cast<int>(40960 / (static_cast<size_t>(nkbp) * 8));
  R = R < 1 ? 1 : (R > 8 ? 8 : R);
  const size_t lds = static_cast<size_t>(R) * g.D * 8 + static_cast<size_t>(R) * nkbp * 8 + 4 * 256 * 4;
  dim3 grid((g.nq + R - 1) / R, g.B * g.H);
  const double sqrt_d = __builtin_sqrt(static_cast<double>(g.D));
  if (g.D == 128)
    hipLaunchKernelGGL((select_kernel<128>), grid, dim3(kThreads), lds, stream, g, R, nkbp, qpool,
                       kpool_t, sqrt_d, crit, marg, cls, logits);
  else
    hipLaunchKernelGGL((select_kernel<64>), grid, dim3(kThreads), lds, stream, g, R, nkbp, qpool,
                       kpool_t, sqrt_d, crit, marg, cls, logits);
  return hipGetLastError();
}

template <typename T, int D>
void launch_pool_t(const Geometry& g, const void* q, const void* k, double* qpool, double* kpool_t,
                   float* qo, float* ko, hipStream_t stream) {
  dim3 grid(g.nq, g.B * g.H, 2);
  hipLaunchKernelGGL((pool_kernel<T, D>), grid, dim3(kThreads), 0, stream,
                     static_cast<const T*>(q), static_cast<const T*>(k), g, qpool, kpool_t, qo, ko);
}

}  // namespace

hipError_t launch_route(const Geometry& g, const void* q, const void* k, int32_t* crit,
                        int32_t* marg, int8_t* cls, float* logits, float* pooled_q,
                        float* pooled_k, double* ws_qpool, double* ws_kpool_t,
                        hipStream_t stream) {
  if (g.dtype == 1) {
    if (g.D == 128) launch_pool_t<uint16_t, 128>(g, q, k, ws_qpool, ws_kpool_t, pooled_q, pooled_k, stream);
    else launch_pool_t<uint16_t, 64>(g, q, k, ws_qpool, ws_kpool_t, pooled_q, pooled_k, stream);
  } else {
    if (g.D == 128) launch_pool_t<float, 128>(g, q, k, ws_qpool, ws_kpool_t, pooled_q, pooled_k, stream);
    else launch_pool_t<float, 64>(g, q, k, ws_qpool, ws_kpool_t, pooled_q, pooled_k, stream);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_select(g, ws_qpool, ws_kpool_t, crit, marg, cls, logits, stream);
}

}  // namespace sla
