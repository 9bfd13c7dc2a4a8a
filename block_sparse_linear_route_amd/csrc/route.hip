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
// grid (ceil(nq / R), B*H).  Thread t owns KV blocks j = jj*256 + t for
// jj < J, for each of the workgroup's R query blocks.
template <int J, int R>
__global__ void __launch_bounds__(kThreads)
select_kernel(Geometry g, const double* __restrict__ qpool, const double* __restrict__ kpool_t,
              double sqrt_d, int32_t* __restrict__ crit, int32_t* __restrict__ marg,
              int8_t* __restrict__ cls, float* __restrict__ logits_out) {
  __shared__ double qs[R][128];
  __shared__ uint32_t hist[R][2][256];
  __shared__ uint64_t pref[R][2];
  __shared__ uint32_t remk[R][2];
  __shared__ uint32_t cnt[R][2][J][4];

  const int bh = blockIdx.y;
  const int i0 = blockIdx.x * R;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int D = g.D, nq = g.nq, nkb = g.nkb;
  const int target[2] = {g.k_crit, g.k_crit + g.k_marg};

  for (int e = t; e < R * D; e += kThreads) {
    const int r = e / D, a = e % D;
    const int i = i0 + r;
    qs[r][a] = (i < nq) ? qpool[(static_cast<int64_t>(bh) * nq + i) * D + a] : 0.0;
  }
  if (t < 2 * R) {
    pref[t >> 1][t & 1] = 0ull;
    remk[t >> 1][t & 1] = target[t & 1] > 0 ? static_cast<uint32_t>(target[t & 1] - 1) : 0u;
  }
  __syncthreads();

  uint64_t key[R][J];
  const double* kt = kpool_t + static_cast<int64_t>(bh) * D * nkb;
#pragma unroll
  for (int jj = 0; jj < J; ++jj) {
    const int j = jj * kThreads + t;
    double acc[R];
#pragma unroll
    for (int r = 0; r < R; ++r) acc[r] = 0.0;
    if (j < nkb) {
      for (int a = 0; a < D; ++a) {
        const double kv = kt[static_cast<int64_t>(a) * nkb + j];
#pragma unroll
        for (int r = 0; r < R; ++r) acc[r] = fma(qs[r][a], kv, acc[r]);
      }
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const double s = acc[r] / sqrt_d;
      const bool ok = (j < nkb) && (i0 + r < nq);
      key[r][jj] = ok ? desc_key(s) : ~0ull;
      if (ok && logits_out)
        logits_out[(static_cast<int64_t>(bh) * nq + i0 + r) * nkb + j] = static_cast<float>(s);
    }
  }

  // 8 radix passes of 8 bits, most significant first, for both targets.
  // Lanes whose key matches the prefix so far are counted with one LDS
  // atomic per distinct digit in the wave (early passes put most keys of a
  // row in the same bin).
  for (int pass = 0; pass < 8; ++pass) {
    const int shift = 56 - 8 * pass;
    for (int e = t; e < R * 2 * 256; e += kThreads) (&hist[0][0][0])[e] = 0u;
    __syncthreads();
#pragma unroll
    for (int r = 0; r < R; ++r) {
#pragma unroll
      for (int w = 0; w < 2; ++w) {
        const uint64_t p = pref[r][w];
#pragma unroll
        for (int jj = 0; jj < J; ++jj) {
          const uint64_t kk = key[r][jj];
          const bool match = (pass == 0) || (((kk ^ p) >> (shift + 8)) == 0ull);
          const uint32_t digit = static_cast<uint32_t>(kk >> shift) & 255u;
          uint64_t active = __ballot(match);
          while (active) {
            const int leader = __builtin_ctzll(active);
            const uint32_t d = __builtin_amdgcn_readlane(digit, leader);
            const uint64_t same = __ballot(match && digit == d);
            if (lane == leader) atomicAdd(&hist[r][w][d], static_cast<uint32_t>(__popcll(same)));
            active &= ~same;
          }
        }
      }
    }
    __syncthreads();
    for (int pr = wave; pr < 2 * R; pr += 4) {
      const int r = pr >> 1, w = pr & 1;
      const uint32_t* hs = hist[r][w];
      const uint32_t c0 = hs[4 * lane], c1 = hs[4 * lane + 1], c2 = hs[4 * lane + 2],
                     c3 = hs[4 * lane + 3];
      const uint32_t tot = c0 + c1 + c2 + c3;
      const uint32_t incl = wave_incl_scan(tot, lane);
      const uint32_t excl = incl - tot;
      const uint32_t rem = remk[r][w];
      if (rem >= excl && rem < incl) {
        uint32_t cum = excl;
        int bin = 4 * lane;
        const uint32_t cs[4] = {c0, c1, c2, c3};
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          if (rem < cum + cs[u]) { bin = 4 * lane + u; break; }
          cum += cs[u];
        }
        pref[r][w] = pref[r][w] | (static_cast<uint64_t>(bin) << shift);
        remk[r][w] = rem - cum;
      }
    }
    __syncthreads();
  }

  // Ties at a threshold: an element whose key equals the threshold key is in
  // iff its rank among the equal keys (ascending j) is <= remk.  Ballots are
  // recomputed after the barrier rather than kept live across it.
  const uint64_t lt_mask = (1ull << lane) - 1ull;
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int w = 0; w < 2; ++w)
#pragma unroll
      for (int jj = 0; jj < J; ++jj) {
        const uint64_t bal = __ballot(key[r][jj] == pref[r][w]);
        if (lane == 0) cnt[r][w][jj][wave] = static_cast<uint32_t>(__popcll(bal));
      }
  __syncthreads();
  uint8_t cls_v[R][J];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    bool in_w[2][J];
#pragma unroll
    for (int w = 0; w < 2; ++w) {
      const uint64_t v = pref[r][w];
      const uint32_t rk = remk[r][w];
      uint32_t base = 0;
#pragma unroll
      for (int jj = 0; jj < J; ++jj) {
        const uint64_t kk = key[r][jj];
        const uint64_t bal = __ballot(kk == v);
        uint32_t before = base;
        for (int ww = 0; ww < wave; ++ww) before += cnt[r][w][jj][ww];
        const uint32_t tie_rank = before + static_cast<uint32_t>(__popcll(bal & lt_mask));
        in_w[w][jj] = target[w] > 0 && (kk < v || (kk == v && tie_rank <= rk));
        base += cnt[r][w][jj][0] + cnt[r][w][jj][1] + cnt[r][w][jj][2] + cnt[r][w][jj][3];
      }
    }
#pragma unroll
    for (int jj = 0; jj < J; ++jj)
      cls_v[r][jj] = in_w[0][jj] ? 2 : (in_w[1][jj] ? 1 : 0);
  }
  __syncthreads();   // cnt is reused below

  // Compaction in ascending j: counts of critical / marginal per chunk and wave.
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int jj = 0; jj < J; ++jj) {
      const bool ok = jj * kThreads + t < nkb;
      const uint64_t b2 = __ballot(ok && cls_v[r][jj] == 2);
      const uint64_t b1 = __ballot(ok && cls_v[r][jj] == 1);
      if (lane == 0) {
        cnt[r][0][jj][wave] = static_cast<uint32_t>(__popcll(b2));
        cnt[r][1][jj][wave] = static_cast<uint32_t>(__popcll(b1));
      }
    }
  __syncthreads();
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int i = i0 + r;
    if (i >= nq) continue;
    const int64_t row = static_cast<int64_t>(bh) * nq + i;
    uint32_t base[2] = {0u, 0u};
#pragma unroll
    for (int jj = 0; jj < J; ++jj) {
      const int j = jj * kThreads + t;
      const bool ok = j < nkb;
      const int c = cls_v[r][jj];
      const uint64_t bal[2] = {__ballot(ok && c == 2), __ballot(ok && c == 1)};
      uint32_t pos[2];
#pragma unroll
      for (int w = 0; w < 2; ++w) {
        uint32_t before = base[w];
        for (int ww = 0; ww < wave; ++ww) before += cnt[r][w][jj][ww];
        pos[w] = before + static_cast<uint32_t>(__popcll(bal[w] & lt_mask));
        base[w] += cnt[r][w][jj][0] + cnt[r][w][jj][1] + cnt[r][w][jj][2] + cnt[r][w][jj][3];
      }
      if (ok) {
        if (cls) cls[row * nkb + j] = static_cast<int8_t>(c);
        if (c == 2 && pos[0] < static_cast<uint32_t>(g.k_crit)) crit[row * g.k_crit + pos[0]] = j;
        else if (c == 1 && pos[1] < static_cast<uint32_t>(g.k_marg)) marg[row * g.k_marg + pos[1]] = j;
      }
    }
  }
}

constexpr int rows_for(int J) { return (32 / J) > 16 ? 16 : ((32 / J) < 1 ? 1 : 32 / J); }

template <int J>
hipError_t launch_select_j(const Geometry& g, const double* qpool, const double* kpool_t,
                           int32_t* crit, int32_t* marg, int8_t* cls, float* logits,
                           hipStream_t stream) {
  constexpr int R = rows_for(J);
  dim3 grid((g.nq + R - 1) / R, g.B * g.H);
  hipLaunchKernelGGL((select_kernel<J, R>), grid, dim3(kThreads), 0, stream, g, qpool, kpool_t,
                     __builtin_sqrt(static_cast<double>(g.D)), crit, marg, cls, logits);
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
  const int J = (g.nkb + kThreads - 1) / kThreads;
  if (J <= 1) return launch_select_j<1>(g, ws_qpool, ws_kpool_t, crit, marg, cls, logits, stream);
  if (J <= 2) return launch_select_j<2>(g, ws_qpool, ws_kpool_t, crit, marg, cls, logits, stream);
  if (J <= 4) return launch_select_j<4>(g, ws_qpool, ws_kpool_t, crit, marg, cls, logits, stream);
  if (J <= 8) return launch_select_j<8>(g, ws_qpool, ws_kpool_t, crit, marg, cls, logits, stream);
  if (J <= 16) return launch_select_j<16>(g, ws_qpool, ws_kpool_t, crit, marg, cls, logits, stream);
  return hipErrorInvalidValue;
}

}  // namespace sla
