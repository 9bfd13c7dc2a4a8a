// Block statistics of piecewise exact-or-approximate attention.
//
// [PISA technical summary, "Algoritmo Central" and "Implementación de
// Hardware" step 1] before the fused pass, each KV block j is reduced to its
// key centroid kbar_j and value sum, and one global first-order matrix
// Hbar = mean_j H_j, H_j = sum_n (k_n - kbar_j)^T v_n, serves every
// unselected block.  Here:
//   kbar  bf16 [B*H][npb*64][d]  block means of K (rows >= nkb unwritten)
//   vbar  bf16 [B*H][npb*64][d]  block means of V (sum = n_j * mean)
//   hbar  bf16 [B*H][d][d]       Hbar value-major: element [c][a] = Hbar[a][c]
// The sum over blocks of H_j is one contraction over all N tokens of the
// block-centred keys and values (centring V too leaves H_j unchanged, since
// the centred keys of a block sum to 0, and keeps the bf16 operands small).
//
// pisa_stats_kernel: one workgroup per (chunk of G consecutive KV blocks,
// b*h).  Per block the 64 x d tiles of K and V are read once (coalesced
// 16-byte loads, 4 threads per token; the next block's loads are issued as
// soon as this block's tiles are staged), their column sums come from DPP row
// rotations and permlane swaps plus a 4-wave LDS sum, the means are written
// out, and the centred tiles go to LDS transposed (token-contiguous) as bf16
// operands of v_mfma_f32_32x32x16_bf16, accumulating the d x d partial sum
// of the chunk in registers.  The partial (float32, value-major) goes to a
// scratch buffer; pisa_reduce_kernel sums the chunks in a fixed order (so
// the result does not depend on scheduling) and divides by nkb.
#include <type_traits>

#include "attention_epilogue.hpp"   // swz: the tile swizzle shared with the attention kernels
#include "device_common.hpp"
#include "sla_internal.hpp"

namespace sla {
namespace {

template <typename T, int D>
__global__ void __launch_bounds__(kThreads)
pisa_stats_kernel(const T* __restrict__ k, const T* __restrict__ v, Geometry g, int G, int npb,
                  uint16_t* __restrict__ kbar, uint16_t* __restrict__ vbar,
                  float* __restrict__ part) {
  constexpr int TS = kBlock + 8;        // token stride of the transposed tiles
  constexpr int CW = D / 4;             // features per thread (4 threads per token)
  constexpr int TA = D / 32;            // 32-row tiles per dimension
  constexpr int NT = TA * TA / 4;       // output tiles per wave
  __shared__ __attribute__((aligned(16))) uint16_t k_t[D * TS];   // centred K^T
  __shared__ __attribute__((aligned(16))) uint16_t v_t[D * TS];   // centred V^T
  __shared__ float zk[4][D], zv[4][D];
  __shared__ float mk[D], mv[D];

  const int chunk = blockIdx.x, bh = blockIdx.y;
  const int nch = gridDim.x;
  const int b = bh / g.H, h = bh % g.H;
  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);   // wave-uniform (scalar)
  const int row = t >> 2, prt = t & 3;
  const int l32 = lane & 31, hh = lane >> 5;
  const int j0 = chunk * G, j1 = min(j0 + G, g.nkb);

  f32x16 acc[NT];
#pragma unroll
  for (int u = 0; u < NT; ++u) acc[u] = zero16();

  // rows past a short last block load its last row and are zeroed
  float kv[CW], vv[CW];
  auto load_block = [&](int j) {
    const int nj = min(kBlock, g.N - j * kBlock);
    const int64_t off = b * g.sb + h * g.sh + static_cast<int64_t>(j * kBlock + min(row, nj - 1)) * g.sn +
                        prt * CW;
#pragma unroll
    for (int c = 0; c < CW / 8; ++c) {
      load8_f32(k + off + 8 * c, kv + 8 * c);
      load8_f32(v + off + 8 * c, vv + 8 * c);
    }
  };
  if (j0 < j1) load_block(j0);

  for (int j = j0; j < j1; ++j) {
    const int nj = min(kBlock, g.N - j * kBlock);
    const bool valid = row < nj;
#pragma unroll
    for (int c = 0; c < CW; ++c) {
      kv[c] = valid ? kv[c] : 0.0f;
      vv[c] = valid ? vv[c] : 0.0f;
    }
    // column sums over the wave's 16 tokens (lanes prt + 4m), then 4 waves
#pragma unroll
    for (int c = 0; c < CW; ++c) {
      float a = kv[c], s = vv[c];
      a += dpp_f<0x124>(a);
      s += dpp_f<0x124>(s);
      a += dpp_f<0x128>(a);
      s += dpp_f<0x128>(s);
      a = swap_sum32(swap_sum16(a));
      s = swap_sum32(swap_sum16(s));
      if (lane < 4) {
        zk[wave][prt * CW + c] = a;
        zv[wave][prt * CW + c] = s;
      }
    }
    __syncthreads();   // also: every wave is past the previous block's operand reads
    const int64_t orow = (static_cast<int64_t>(bh) * npb * kBlock + j) * D;
    const float inv_n = 1.0f / static_cast<float>(nj);
    if (t < D) {
      const float m = (zk[0][t] + zk[1][t] + zk[2][t] + zk[3][t]) * inv_n;
      mk[t] = m;
      kbar[orow + t] = f32_to_bf16_bits(m);
    } else if (t < 2 * D) {
      const int e = t - D;
      const float m = (zv[0][e] + zv[1][e] + zv[2][e] + zv[3][e]) * inv_n;
      mv[e] = m;
      vbar[orow + e] = f32_to_bf16_bits(m);
    }
    __syncthreads();
    // centred, token-contiguous bf16 operands (invalid rows stay 0)
#pragma unroll
    for (int c = 0; c < CW; ++c) {
      const int f = prt * CW + c;
      k_t[f * TS + row] = f32_to_bf16_bits(valid ? kv[c] - mk[f] : 0.0f);
      v_t[f * TS + row] = f32_to_bf16_bits(valid ? vv[c] - mv[f] : 0.0f);
    }
    // the tiles are in LDS: the next block's loads fly during the products
    if (j + 1 < j1) load_block(j + 1);
    __syncthreads();
    // acc tile (ct, at) = sum over tokens of Vc[token][c] Kc[token][a]: the
    // value dims are the A rows (registers), the key features the B rows
    // (lanes), so the tile is value-major
#pragma unroll
    for (int u = 0; u < NT; ++u) {
      const int ti = wave * NT + u;
      const int ct = ti / TA, at = ti % TA;
#pragma unroll
      for (int s = 0; s < kBlock / 16; ++s) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(&v_t[(ct * 32 + l32) * TS + 16 * s + 8 * hh]);
        const bf16x8 bb = *reinterpret_cast<const bf16x8*>(&k_t[(at * 32 + l32) * TS + 16 * s + 8 * hh]);
        acc[u] = mfma32(a, bb, acc[u]);
      }
    }
  }

  // partial [c][a]: for each register, the 32 lanes of a half write 32
  // consecutive a (128-byte rows)
  float* dst = part + (static_cast<int64_t>(bh) * nch + chunk) * D * D;
#pragma unroll
  for (int u = 0; u < NT; ++u) {
    const int ti = wave * NT + u;
    const int ct = ti / TA, at = ti % TA;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int c = ct * 32 + 8 * (r >> 2) + 4 * hh + (r & 3);
      dst[c * D + at * 32 + l32] = acc[u][r];
    }
  }
}

// bf16 inputs: the same statistics without staging through registers.  The
// K and V tiles of each block go from HBM straight into a two-stage LDS ring
// (global -> LDS buffer loads, 16-byte chunks XOR-swizzled per row, rows past
// the last token read as zeros), and the matrix-core operands (8 tokens of
// one feature per lane) come from transposing LDS reads.  With exact bf16
// inputs the products need no centring: per block the matrix cores
// accumulate sum_n v_n[c] k_n[a] and the column sums of K and V (a ones
// operand), and the rank-one term (sum v)(sum k)^T / n_j is subtracted in
// float32, which equals sum_n (v_n - vbar)[c] (k_n - kbar)[a] up to float32
// rounding.  Wave w owns value tile ct = w*NT/TA and key tiles at, and
// computes the key-sum tile its first B operand covers and the value-sum
// tile of ct; the key sums reach the other waves through LDS one block later
// (after the next barrier), so each block costs one barrier.
//
// DEV (covariance-aware routing): the same per-block products, but each
// block's H_j is finished on its own (the accumulators restart at every
// block) and reduced to M_j = sqrt(sum (H_j - Hbar)^2) against the float32
// Hbar of an earlier pass; nothing else is written.
template <int D, bool DEV = false>
__global__ void __launch_bounds__(kThreads, 2)
pisa_stats_bf16_kernel(const uint16_t* __restrict__ k, const uint16_t* __restrict__ v, Geometry g,
                       int G, int npb, uint16_t* __restrict__ kbar, uint16_t* __restrict__ vbar,
                       float* __restrict__ part, const float* __restrict__ hbar_f32 = nullptr,
                       double* __restrict__ mdev = nullptr, float* __restrict__ mdev_out = nullptr) {
  constexpr int CH = D / 8;                 // 16-byte chunks per row
  constexpr int RPI = 64 / CH;              // rows per 64-lane load instruction
  constexpr int IPW = (kBlock / 4) / RPI;   // load instructions per wave per tile
  constexpr int TILE = kBlock * D;          // elements per tile
  constexpr int TA = D / 32;
  constexpr int NT = TA * TA / 4;           // output tiles per wave
  // the ring: one array per stage and tensor, so that reads of one stage
  // carry no false dependence on the loads filling the other
  __shared__ __attribute__((aligned(16))) uint16_t k0[TILE], v0[TILE], k1[TILE], v1[TILE];
  __shared__ float ksum[2][D], vsum[2][D];
  __shared__ float devp[4];

  const int chunk = blockIdx.x, bh = blockIdx.y;
  const int nch = gridDim.x;
  const int b = bh / g.H, h = bh % g.H;
  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int l32 = lane & 31, hh = lane >> 5;
  const int j0 = chunk * G, j1 = min(j0 + G, g.nkb);
  const int nblk = j1 - j0;
  const int ct = wave * NT / TA;            // value tile of this wave
  const int at0 = wave * NT % TA;           // first key tile of this wave
  // key-sum tile of this wave: its own index at d = 128 (each wave holds all
  // four key tiles), its single key tile at d = 64 (waves 0 and 1 publish)
  const int ksu = (NT == TA) ? wave : 0;
  const bool ks_pub = (NT == TA) || ct == 0;

  // global -> LDS loads: lane l of instruction u fills row 16w + RPI u + l/CH
  // at chunk slot l%CH with global chunk (l%CH) ^ swz(row)
  const int64_t hoff = b * g.sb + h * g.sh;
  const uint32_t rowb = static_cast<uint32_t>(g.sn * 2);
  const uint32_t head_bytes = static_cast<uint32_t>(((g.N - 1) * g.sn + D) * 2);
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(k + hoff, head_bytes);
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc(v + hoff, head_bytes);
  const int lrow = lane / CH, lslot = lane % CH;
  uint32_t toff[IPW];
#pragma unroll
  for (int u = 0; u < IPW; ++u) {
    const int r = 16 * wave + RPI * u + lrow;
    toff[u] = static_cast<uint32_t>(r) * rowb + static_cast<uint32_t>(16 * (lslot ^ swz<D>(r)));
  }
  auto issue = [&](auto xc, int it) {
    constexpr int X = decltype(xc)::value;
    const uint32_t soff = static_cast<uint32_t>((j0 + it) * kBlock) * rowb;
    uint16_t* kd = (X ? k1 : k0) + 16 * wave * D;
    uint16_t* vd = (X ? v1 : v0) + 16 * wave * D;
#pragma unroll
    for (int u = 0; u < IPW; ++u) {
      buffer_load_lds16(krs, kd + RPI * u * D, toff[u], soff);
      buffer_load_lds16(vrs, vd + RPI * u * D, toff[u], soff);
    }
  };

  // transposing reads: lane l receives feature 32*ft + l%32 at tokens
  // 16 s + {4 hh + e, 8 + 4 hh + e} (e = 0..3), the same token order in
  // every operand, so the k-slots of A and B match
  const int li = lane & 15, ep = li >> 2, q4 = li & 3, gm = (lane >> 4) & 1;
  const int key1 = 4 * hh + ep;
  const int sw1 = swz<D>(key1), sw2 = swz<D>(key1 + 8);
  int ro1[TA], ro2[TA];
#pragma unroll
  for (int ft = 0; ft < TA; ++ft) {
    const int c = 4 * ft + 2 * gm + (q4 >> 1);
    ro1[ft] = key1 * D + 8 * (c ^ sw1) + 4 * (q4 & 1);
    ro2[ft] = (key1 + 8) * D + 8 * (c ^ sw2) + 4 * (q4 & 1);
  }
  auto operand = [&](const uint16_t* tile, int ft, int s) -> bf16x8 {
    const u32x2 x0 = lds_read_tr16(tile + ro1[ft] + 16 * s * D);
    const u32x2 x1 = lds_read_tr16(tile + ro2[ft] + 16 * s * D);
    u32x4 w;
    w[0] = x0[0]; w[1] = x0[1]; w[2] = x1[0]; w[3] = x1[1];
    return __builtin_bit_cast(bf16x8, w);
  };
  bf16x8 ones;
#pragma unroll
  for (int e = 0; e < 8; ++e) ones[e] = static_cast<__bf16>(1.0f);

  f32x16 acc[NT];
#pragma unroll
  for (int u = 0; u < NT; ++u) acc[u] = zero16();
  f32x16 vs_prev = zero16();
  // DEV: this lane's elements of Hbar, in the accumulator layout
  [[maybe_unused]] f32x16 hb[DEV ? NT : 1];
  if constexpr (DEV) {
    const float* hsrc = hbar_f32 + static_cast<int64_t>(bh) * D * D;
#pragma unroll
    for (int u = 0; u < NT; ++u)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int c = ct * 32 + 8 * (r >> 2) + 4 * hh + (r & 3);
        hb[u][r] = hsrc[c * D + (at0 + u) * 32 + l32];
      }
  }

  // rank-one term and means of block it (sums in LDS buffer it & 1, value
  // sums of this wave's rows in vs_prev)
  auto finish_block = [&](int it) __attribute__((always_inline)) {
    const int j = j0 + it;
    const float inv_n = 1.0f / static_cast<float>(min(kBlock, g.N - j * kBlock));
    const float* ks = ksum[it & 1];
#pragma unroll
    for (int u = 0; u < NT; ++u) {
      const float ka = ks[(at0 + u) * 32 + l32] * inv_n;
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[u][r] = fmaf(-vs_prev[r], ka, acc[u][r]);
    }
    if constexpr (DEV) {
      // acc holds H_j of this block alone: sum of squared deviations from
      // Hbar over the wave's tiles, then over the lanes and the four waves
      float ss = 0.0f;
#pragma unroll
      for (int u = 0; u < NT; ++u)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float dl = acc[u][r] - hb[u][r];
          ss = fmaf(dl, dl, ss);
          acc[u][r] = 0.0f;
        }
#pragma unroll
      for (int m = 32; m >= 1; m >>= 1) ss += __shfl_xor(ss, m, 64);
      if (lane == 0) devp[wave] = ss;
      __syncthreads();
      if (t == 0) {
        const double tot = (static_cast<double>(devp[0]) + devp[1]) + (static_cast<double>(devp[2]) + devp[3]);
        const double m = sqrt(tot);
        mdev[static_cast<int64_t>(bh) * g.nkb + j] = m;
        if (mdev_out) mdev_out[static_cast<int64_t>(bh) * g.nkb + j] = static_cast<float>(m);
      }
    } else {
      const int64_t orow = (static_cast<int64_t>(bh) * npb * kBlock + j) * D;
      if (t < D) kbar[orow + t] = f32_to_bf16_bits(ks[t] * inv_n);
      else if (t < 2 * D) vbar[orow + t - D] = f32_to_bf16_bits(vsum[it & 1][t - D] * inv_n);
    }
  };

  auto body = [&](auto xc, int it) {
    constexpr int X = decltype(xc)::value;
    wait_vmem();       // this wave's part of block it
    __syncthreads();   // all parts landed; block it-1's reads and sums done
    if (it + 1 < nblk) issue(std::integral_constant<int, 1 - X>(), it + 1);
    if (it > 0) finish_block(it - 1);
    const uint16_t* kt = X ? k1 : k0;
    const uint16_t* vt = X ? v1 : v0;
    f32x16 ksm = zero16(), vsm = zero16();
#pragma unroll
    for (int s = 0; s < kBlock / 16; ++s) {
      const bf16x8 a = operand(vt, ct, s);
      bf16x8 bq[NT];
#pragma unroll
      for (int u = 0; u < NT; ++u) bq[u] = operand(kt, at0 + u, s);
#pragma unroll
      for (int u = 0; u < NT; ++u) acc[u] = mfma32(a, bq[u], acc[u]);
      vsm = mfma32(a, ones, vsm);
      bf16x8 kop = bq[0];
#pragma unroll
      for (int u = 1; u < NT; ++u)
        if (ksu == u) kop = bq[u];
      ksm = mfma32(kop, ones, ksm);
    }
    // sums: every lane holds the tile's 16 row sums of its half; lanes 0
    // and 32 publish them (key sums of tile at0 + ksu, value sums of tile ct)
    if (l32 == 0) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = 8 * (r >> 2) + 4 * hh + (r & 3);
        if (ks_pub) ksum[it & 1][(at0 + ksu) * 32 + row] = ksm[r];
        if (at0 == 0) vsum[it & 1][ct * 32 + row] = vsm[r];
      }
    }
    vs_prev = vsm;
  };
  if (nblk > 0) issue(std::integral_constant<int, 0>(), 0);
  for (int it = 0; it < nblk; it += 2) {
    body(std::integral_constant<int, 0>(), it);
    if (it + 1 < nblk) body(std::integral_constant<int, 1>(), it + 1);
  }
  __syncthreads();
  if (nblk > 0) finish_block(nblk - 1);
  if constexpr (DEV) return;

  float* dst = part + (static_cast<int64_t>(bh) * nch + chunk) * D * D;
#pragma unroll
  for (int u = 0; u < NT; ++u) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int c = ct * 32 + 8 * (r >> 2) + 4 * hh + (r & 3);
      dst[c * D + (at0 + u) * 32 + l32] = acc[u][r];
    }
  }
}

// Float32 first-order matrices for covariance-aware routing (any input
// type, float32 arithmetic throughout, no bf16 rounding of the operands).
// grid (chunks of G blocks, B*H); per block the K and V tiles go to LDS as
// float32 with the keys centred on their block mean (rows past a short last
// block are 0), and thread t accumulates the (D/16) x (D/16) elements
// a in [a0, a0 + D/16), c in [c0, c0 + D/16) of sum_n (k_n - kbar)[a] v_n[c].
// SUM: the chunk's sum of H_j goes to part (value-major, as the statistics
// kernels write it) for pisa_reduce_kernel.  DEV: each block's
// M_j = sqrt(sum (H_j - Hbar)^2) against hbar_f32 goes to mdev (float64) and
// mdev_out (float32, optional).
template <typename T, int D, bool DEV>
__global__ void __launch_bounds__(kThreads)
pisa_first_order_f32_kernel(const T* __restrict__ k, const T* __restrict__ v, Geometry g, int G,
                            float* __restrict__ part, const float* __restrict__ hbar_f32,
                            double* __restrict__ mdev, float* __restrict__ mdev_out) {
  constexpr int AW = D / 16;
  __shared__ float kc[kBlock][D];
  __shared__ float vv[kBlock][D];
  __shared__ float mk[D];
  __shared__ double red[4];
  const int chunk = blockIdx.x, bh = blockIdx.y;
  const int nch = gridDim.x;
  const int b = bh / g.H, h = bh % g.H;
  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);   // wave-uniform (scalar)
  const int a0 = (t / 16) * AW, c0 = (t % 16) * AW;
  const int j0 = chunk * G, j1 = min(j0 + G, g.nkb);
  const T* kh = k + b * g.sb + h * g.sh;
  const T* vh = v + b * g.sb + h * g.sh;
  float acc[AW][AW];
#pragma unroll
  for (int x = 0; x < AW; ++x)
#pragma unroll
    for (int y = 0; y < AW; ++y) acc[x][y] = 0.0f;
  [[maybe_unused]] float hb[DEV ? AW : 1][DEV ? AW : 1];
  if constexpr (DEV) {
    const float* hs = hbar_f32 + static_cast<int64_t>(bh) * D * D;
#pragma unroll
    for (int x = 0; x < AW; ++x)
#pragma unroll
      for (int y = 0; y < AW; ++y) hb[x][y] = hs[(c0 + y) * D + a0 + x];
  }
  for (int j = j0; j < j1; ++j) {
    const int nj = min(kBlock, g.N - j * kBlock);
    for (int e = t; e < kBlock * D; e += kThreads) {
      const int n = e / D, f = e % D;
      const int64_t off = static_cast<int64_t>(j * kBlock + n) * g.sn + f;
      float kx = 0.0f, vx = 0.0f;
      if (n < nj) {
        if constexpr (sizeof(T) == 2) {
          kx = bf16_to_f32(reinterpret_cast<const uint16_t*>(kh)[off]);
          vx = bf16_to_f32(reinterpret_cast<const uint16_t*>(vh)[off]);
        } else {
          kx = kh[off];
          vx = vh[off];
        }
      }
      kc[n][f] = kx;
      vv[n][f] = vx;
    }
    __syncthreads();
    if (t < D) {
      float sm = 0.0f;
      for (int n = 0; n < nj; ++n) sm += kc[n][t];
      mk[t] = sm / static_cast<float>(nj);
    }
    __syncthreads();
    for (int e = t; e < nj * D; e += kThreads) kc[e / D][e % D] -= mk[e % D];
    __syncthreads();
    for (int n = 0; n < nj; ++n) {
      float ka[AW], vc[AW];
#pragma unroll
      for (int x = 0; x < AW; ++x) ka[x] = kc[n][a0 + x];
#pragma unroll
      for (int y = 0; y < AW; ++y) vc[y] = vv[n][c0 + y];
#pragma unroll
      for (int x = 0; x < AW; ++x)
#pragma unroll
        for (int y = 0; y < AW; ++y) acc[x][y] = fmaf(ka[x], vc[y], acc[x][y]);
    }
    if constexpr (DEV) {
      double ss = 0.0;
#pragma unroll
      for (int x = 0; x < AW; ++x)
#pragma unroll
        for (int y = 0; y < AW; ++y) {
          const double dl = static_cast<double>(acc[x][y]) - hb[x][y];
          ss = fma(dl, dl, ss);
          acc[x][y] = 0.0f;
        }
#pragma unroll
      for (int m = 32; m >= 1; m >>= 1) ss += __shfl_xor(ss, m, 64);
      if (lane == 0) red[wave] = ss;
      __syncthreads();
      if (t == 0) {
        const double m = sqrt((red[0] + red[1]) + (red[2] + red[3]));
        mdev[static_cast<int64_t>(bh) * g.nkb + j] = m;
        if (mdev_out) mdev_out[static_cast<int64_t>(bh) * g.nkb + j] = static_cast<float>(m);
      }
    }
    __syncthreads();   // every thread is past this block's LDS reads
  }
  if constexpr (!DEV) {
    float* dst = part + (static_cast<int64_t>(bh) * nch + chunk) * D * D;
#pragma unroll
    for (int x = 0; x < AW; ++x)
#pragma unroll
      for (int y = 0; y < AW; ++y) dst[(c0 + y) * D + a0 + x] = acc[x][y];
  }
}

// grid (D*D / 256, B*H): a workgroup owns 256 consecutive elements (64
// lanes x 4); wave w sums chunks w, w + 4, ... (four loads in flight per
// lane), then the four waves' sums are added in a fixed order through LDS,
// divided by nkb and written as bf16 (and float32 when requested).
template <int D>
__global__ void __launch_bounds__(kThreads)
pisa_reduce_kernel(const float* __restrict__ part, int nch, int nkb, uint16_t* __restrict__ hbar,
                   float* __restrict__ hbar_f32) {
  __shared__ f32x4 red[4][64];
  const int bh = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform (scalar)
  const int e = 256 * blockIdx.x + 4 * lane;
  const float* src = part + static_cast<int64_t>(bh) * nch * D * D + e;
  f32x4 s = {0.0f, 0.0f, 0.0f, 0.0f};
  int c = wave;
  for (; c + 12 < nch; c += 16) {
    const f32x4 a0 = *reinterpret_cast<const f32x4*>(src + static_cast<int64_t>(c) * D * D);
    const f32x4 a1 = *reinterpret_cast<const f32x4*>(src + static_cast<int64_t>(c + 4) * D * D);
    const f32x4 a2 = *reinterpret_cast<const f32x4*>(src + static_cast<int64_t>(c + 8) * D * D);
    const f32x4 a3 = *reinterpret_cast<const f32x4*>(src + static_cast<int64_t>(c + 12) * D * D);
    s += (a0 + a1) + (a2 + a3);
  }
  for (; c < nch; c += 4) s += *reinterpret_cast<const f32x4*>(src + static_cast<int64_t>(c) * D * D);
  red[wave][lane] = s;
  __syncthreads();
  if (wave != 0) return;
  s = ((red[0][lane] + red[1][lane]) + (red[2][lane] + red[3][lane])) * (1.0f / static_cast<float>(nkb));
  const int64_t o = static_cast<int64_t>(bh) * D * D + e;
  u32x2 w;
  w[0] = static_cast<uint32_t>(f32_to_bf16_bits(s[0])) | (static_cast<uint32_t>(f32_to_bf16_bits(s[1])) << 16);
  w[1] = static_cast<uint32_t>(f32_to_bf16_bits(s[2])) | (static_cast<uint32_t>(f32_to_bf16_bits(s[3])) << 16);
  *reinterpret_cast<u32x2*>(hbar + o) = w;
  if (hbar_f32) *reinterpret_cast<f32x4*>(hbar_f32 + o) = s;
}

template <typename T, int D>
void launch_pisa_stats_t(const Geometry& g, const void* k, const void* v, int G, int nch,
                         uint16_t* kbar, uint16_t* vbar, uint16_t* hbar, float* part,
                         float* hbar_f32, hipStream_t stream) {
  const int npb = pisa_pseudo_blocks(g);
  if constexpr (sizeof(T) == 2)
    hipLaunchKernelGGL((pisa_stats_bf16_kernel<D>), dim3(nch, g.B * g.H), dim3(kThreads), 0, stream,
                       static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v), g, G, npb,
                       kbar, vbar, part);
  else
    hipLaunchKernelGGL((pisa_stats_kernel<T, D>), dim3(nch, g.B * g.H), dim3(kThreads), 0, stream,
                       static_cast<const T*>(k), static_cast<const T*>(v), g, G, npb, kbar, vbar, part);
  hipLaunchKernelGGL((pisa_reduce_kernel<D>), dim3(D * D / 256, g.B * g.H), dim3(kThreads), 0, stream,
                     part, nch, g.nkb, hbar, hbar_f32);
}

template <typename T, int D>
void launch_pisa_dev_t(const Geometry& g, const void* k, const void* v, int G, int nch,
                       uint16_t* hbar, float* part, float* hbar_f32, double* mdev,
                       float* mdev_out, hipStream_t stream) {
  if constexpr (sizeof(T) == 2) {
    hipLaunchKernelGGL((pisa_stats_bf16_kernel<D, true>), dim3(nch, g.B * g.H), dim3(kThreads), 0,
                       stream, static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v), g, G,
                       pisa_pseudo_blocks(g), nullptr, nullptr, nullptr, hbar_f32, mdev, mdev_out);
  } else {
    // float32 inputs: Hbar again from float32 operands (the statistics
    // kernel rounds its centred operands to bf16), then the deviations
    hipLaunchKernelGGL((pisa_first_order_f32_kernel<T, D, false>), dim3(nch, g.B * g.H), dim3(kThreads),
                       0, stream, static_cast<const T*>(k), static_cast<const T*>(v), g, G, part,
                       nullptr, nullptr, nullptr);
    hipLaunchKernelGGL((pisa_reduce_kernel<D>), dim3(D * D / 256, g.B * g.H), dim3(kThreads), 0, stream,
                       part, nch, g.nkb, hbar, hbar_f32);
    hipLaunchKernelGGL((pisa_first_order_f32_kernel<T, D, true>), dim3(nch, g.B * g.H), dim3(kThreads),
                       0, stream, static_cast<const T*>(k), static_cast<const T*>(v), g, G, nullptr,
                       hbar_f32, mdev, mdev_out);
  }
}

}  // namespace

hipError_t launch_pisa_deviation(const Geometry& g, const void* k, const void* v, uint16_t* hbar,
                                 float* part, float* hbar_f32, double* mdev, float* mdev_out,
                                 hipStream_t stream) {
  const int G = pisa_chunk_blocks(g);
  const int nch = (g.nkb + G - 1) / G;
  if (g.dtype == 1) {
    if (g.D == 128) launch_pisa_dev_t<uint16_t, 128>(g, k, v, G, nch, hbar, part, hbar_f32, mdev, mdev_out, stream);
    else launch_pisa_dev_t<uint16_t, 64>(g, k, v, G, nch, hbar, part, hbar_f32, mdev, mdev_out, stream);
  } else {
    if (g.D == 128) launch_pisa_dev_t<float, 128>(g, k, v, G, nch, hbar, part, hbar_f32, mdev, mdev_out, stream);
    else launch_pisa_dev_t<float, 64>(g, k, v, G, nch, hbar, part, hbar_f32, mdev, mdev_out, stream);
  }
  return hipGetLastError();
}

hipError_t launch_pisa_stats(const Geometry& g, const void* k, const void* v, uint16_t* kbar,
                             uint16_t* vbar, uint16_t* hbar, float* part, float* hbar_f32,
                             hipStream_t stream) {
  const int G = pisa_chunk_blocks(g);
  const int nch = (g.nkb + G - 1) / G;
  if (g.dtype == 1) {
    if (g.D == 128) launch_pisa_stats_t<uint16_t, 128>(g, k, v, G, nch, kbar, vbar, hbar, part, hbar_f32, stream);
    else launch_pisa_stats_t<uint16_t, 64>(g, k, v, G, nch, kbar, vbar, hbar, part, hbar_f32, stream);
  } else {
    if (g.D == 128) launch_pisa_stats_t<float, 128>(g, k, v, G, nch, kbar, vbar, hbar, part, hbar_f32, stream);
    else launch_pisa_stats_t<float, 64>(g, k, v, G, nch, kbar, vbar, hbar, part, hbar_f32, stream);
  }
  return hipGetLastError();
}

}  // namespace sla
