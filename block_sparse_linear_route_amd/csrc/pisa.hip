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
// 16-byte loads, 4 threads per token), their column sums come from DPP row
// rotations and permlane swaps plus a 4-wave LDS sum, the means are written
// out, and the centred tiles go to LDS transposed (token-contiguous) as bf16
// operands of v_mfma_f32_32x32x16_bf16, accumulating the d x d partial sum
// of the chunk in registers.  The partial (float32, value-major) goes to a
// scratch buffer; pisa_reduce_kernel sums the chunks in a fixed order (so
// the result does not depend on scheduling) and divides by nkb.
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
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int row = t >> 2, prt = t & 3;
  const int l32 = lane & 31, hh = lane >> 5;
  const int j0 = chunk * G, j1 = min(j0 + G, g.nkb);

  f32x16 acc[NT];
#pragma unroll
  for (int u = 0; u < NT; ++u) acc[u] = zero16();

  for (int j = j0; j < j1; ++j) {
    const int nj = min(kBlock, g.N - j * kBlock);
    const bool valid = row < nj;
    // rows past a short last block load its last row and are zeroed
    const int64_t off = b * g.sb + h * g.sh + static_cast<int64_t>(j * kBlock + min(row, nj - 1)) * g.sn +
                        prt * CW;
    float kv[CW], vv[CW];
#pragma unroll
    for (int c = 0; c < CW / 8; ++c) {
      load8_f32(k + off + 8 * c, kv + 8 * c);
      load8_f32(v + off + 8 * c, vv + 8 * c);
    }
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

// grid (D*D / (4*kThreads), B*H): each thread sums 4 consecutive elements
// over the chunks in order, divides by nkb and writes bf16 (and float32 when
// requested).
template <int D>
__global__ void __launch_bounds__(kThreads)
pisa_reduce_kernel(const float* __restrict__ part, int nch, int nkb, uint16_t* __restrict__ hbar,
                   float* __restrict__ hbar_f32) {
  const int bh = blockIdx.y;
  const int e = 4 * (blockIdx.x * kThreads + threadIdx.x);
  const float* src = part + static_cast<int64_t>(bh) * nch * D * D + e;
  f32x4 s = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int c = 0; c < nch; ++c) s += *reinterpret_cast<const f32x4*>(src + static_cast<int64_t>(c) * D * D);
  const float inv = 1.0f / static_cast<float>(nkb);
  s *= inv;
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
  hipLaunchKernelGGL((pisa_stats_kernel<T, D>), dim3(nch, g.B * g.H), dim3(kThreads), 0, stream,
                     static_cast<const T*>(k), static_cast<const T*>(v), g, G, npb, kbar, vbar, part);
  hipLaunchKernelGGL((pisa_reduce_kernel<D>), dim3(D * D / (4 * kThreads), g.B * g.H), dim3(kThreads),
                     0, stream, part, nch, g.nkb, hbar, hbar_f32);
}

}  // namespace

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
