// Marginal-state sums of the linear branch on the matrix cores.
//
// [SLA abstract] marginal KV blocks get O(N) linear attention; [PISA
// technical summary] per-block first-order matrices H_j; the linear branch of
// query block i needs S_i = sum_{j in M_i} H_j and sigma_i = sum_{j in M_i}
// z_j.  Per head this is a product with the 0/1 marginal mask M
// ([nq x nkb], exact in bf16):
//     S[i, e] = sum_j M[i, j] H[j, e]        (e runs over the d*d entries)
//     sigma[i, a] = sum_j M[i, j] z[j, a]
// which runs as a dense bf16 GEMM on v_mfma_f32_32x32x16_bf16 with float32
// accumulation, so every product is exact and S is the float32 sum of the
// bf16 states (rounded once to bf16 on store).  z is float32: it enters the
// same GEMM as two bf16 columns per feature (hi = bf16(z), lo = bf16(z - hi))
// whose products are added in float32, giving sigma to ~2^-17 relative.
//
// Kernel 1 turns the ascending marginal index lists into bit rows
// (nkb bits per query block).  Kernel 2 tiles the GEMM: 256 query blocks x
// 128 columns per workgroup, K-loop over chunks of 32 KV blocks; the H chunk
// is staged in LDS transposed (column-major in j) so both MFMA operands are
// contiguous in the contraction index, and the mask operand is expanded from
// the bit rows in registers.
#include "device_common.hpp"
#include "sla_internal.hpp"

namespace sla {
namespace {

constexpr int kTM = 256;        // query blocks per workgroup
constexpr int kTN = 128;        // GEMM columns per workgroup
constexpr int kTK = 32;         // KV blocks per K chunk
constexpr int kHS = kTK + 8;    // LDS row stride of the transposed chunk (elements)

// grid (ceil(nq / 64), B*H): bit rows of the marginal sets.
__global__ void __launch_bounds__(kThreads)
marg_bits_kernel(Geometry g, const int32_t* __restrict__ marg, uint32_t* __restrict__ bits, int nw) {
  extern __shared__ uint32_t sbits[];        // [64][nw]
  const int bh = blockIdx.y;
  const int i0 = blockIdx.x * 64;
  const int t = threadIdx.x;
  for (int e = t; e < 64 * nw; e += kThreads) sbits[e] = 0u;
  __syncthreads();
  const int km = g.k_marg;
  for (int e = t; e < 64 * km; e += kThreads) {
    const int r = e / km, u = e % km;
    const int i = i0 + r;
    if (i < g.nq) {
      const int j = marg[(static_cast<int64_t>(bh) * g.nq + i) * km + u];
      atomicOr(&sbits[r * nw + (j >> 5)], 1u << (j & 31));
    }
  }
  __syncthreads();
  for (int e = t; e < 64 * nw; e += kThreads) {
    const int r = e / nw, w = e % nw;
    const int i = i0 + r;
    if (i < g.nq) bits[(static_cast<int64_t>(bh) * g.nq + i) * nw + w] = sbits[e];
  }
}

// Eight mask bits -> eight bf16 values 0.0 / 1.0.
__device__ __forceinline__ bf16x8 bits_to_bf16x8(uint32_t byte) {
  u32x4 w;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const uint32_t lo = (byte >> (2 * p)) & 1u ? 0x3f80u : 0u;
    const uint32_t hi = (byte >> (2 * p + 1)) & 1u ? 0x3f800000u : 0u;
    w[p] = lo | hi;
  }
  return __builtin_bit_cast(bf16x8, w);
}

// grid (ceil(nq / 256), D*D/128 + D/64, B*H).  Column tiles ct < D*D/128
// take entries e in [128 ct, 128 ct + 128) of H; the last D/64 take z
// features [64 zt, 64 zt + 64) as (hi, lo) column pairs.
template <int D>
__global__ void __launch_bounds__(kThreads, 2)
marg_gemm_kernel(Geometry g, const uint32_t* __restrict__ bits, int nw,
                 const uint16_t* __restrict__ hs, const float* __restrict__ zs,
                 uint16_t* __restrict__ s_out, float* __restrict__ sigma_out) {
  constexpr int HT = D * D / kTN;                  // H column tiles
  __shared__ __attribute__((aligned(16))) uint16_t ht[2][kTN * kHS];

  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int l32 = lane & 31, hh = lane >> 5;
  const int bh = blockIdx.z;
  const int ct = blockIdx.y;
  const bool ztile = ct >= HT;
  const int i0 = blockIdx.x * kTM;
  const int nq = g.nq, nkb = g.nkb;
  const int nchunks = (nkb + kTK - 1) / kTK;
  const uint16_t* hb = hs + static_cast<int64_t>(bh) * nkb * D * D + (ztile ? 0 : ct * kTN);
  const float* zb = zs + static_cast<int64_t>(bh) * nkb * D + (ztile ? (ct - HT) * 64 : 0);

  // staging: thread loads KV blocks 2*jp, 2*jp+1 of the chunk, columns 8*ec .. +7
  const int jp = t % 16, ec = t / 16;
  bf16x8 st0, st1;
#define SLA_LOAD_CHUNK(c_)                                                                   \
  do {                                                                                       \
    const int j = kTK * (c_) + 2 * jp;                                                       \
    if (!ztile) {                                                                            \
      st0 = (j < nkb) ? load8(hb + static_cast<int64_t>(j) * D * D + 8 * ec) : zero_bf16x8(); \
      st1 = (j + 1 < nkb) ? load8(hb + static_cast<int64_t>(j + 1) * D * D + 8 * ec)         \
                          : zero_bf16x8();                                                   \
    } else {                                                                                 \
      f32x4 z0 = {0.f, 0.f, 0.f, 0.f}, z1 = z0;                                              \
      if (j < nkb) z0 = *reinterpret_cast<const f32x4*>(zb + static_cast<int64_t>(j) * D + 4 * ec); \
      if (j + 1 < nkb)                                                                       \
        z1 = *reinterpret_cast<const f32x4*>(zb + static_cast<int64_t>(j + 1) * D + 4 * ec); \
      _Pragma("unroll") for (int x = 0; x < 4; ++x) {                                        \
        const __bf16 h0 = f32_to_bf16(z0[x]);                                                \
        const __bf16 h1 = f32_to_bf16(z1[x]);                                                \
        st0[2 * x] = h0;                                                                     \
        st0[2 * x + 1] = f32_to_bf16(z0[x] - bf16v_to_f32(h0));                              \
        st1[2 * x] = h1;                                                                     \
        st1[2 * x + 1] = f32_to_bf16(z1[x] - bf16v_to_f32(h1));                              \
      }                                                                                      \
    }                                                                                        \
  } while (0)

#define SLA_STORE_CHUNK(buf_)                                                                \
  do {                                                                                       \
    const u32x4 a_ = __builtin_bit_cast(u32x4, st0);                                         \
    const u32x4 b_ = __builtin_bit_cast(u32x4, st1);                                         \
    _Pragma("unroll") for (int x = 0; x < 8; ++x) {                                          \
      const uint32_t w = (x & 1) ? ((a_[x >> 1] >> 16) | (b_[x >> 1] & 0xffff0000u))         \
                                 : ((a_[x >> 1] & 0xffffu) | (b_[x >> 1] << 16));            \
      *reinterpret_cast<uint32_t*>(&ht[(buf_)][(8 * ec + x) * kHS + 2 * jp]) = w;            \
    }                                                                                        \
  } while (0)

  // rows of this wave: i0 + 64*wave + 32*nt + l32
  const uint32_t* brow[2];
  bool rok[2];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const int i = i0 + 64 * wave + 32 * nt + l32;
    rok[nt] = i < nq;
    brow[nt] = bits + (static_cast<int64_t>(bh) * nq + (rok[nt] ? i : 0)) * nw;
  }

  f32x16 acc[4][2];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) acc[mt][nt] = zero16();

  SLA_LOAD_CHUNK(0);
  SLA_STORE_CHUNK(0);
  if (nchunks > 1) SLA_LOAD_CHUNK(1);
  __syncthreads();
  for (int c = 0; c < nchunks; ++c) {
    const int buf = c & 1;
    uint32_t word[2];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) word[nt] = rok[nt] ? brow[nt][c] : 0u;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      bf16x8 bm[2];
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) bm[nt] = bits_to_bf16x8((word[nt] >> (16 * s + 8 * hh)) & 0xffu);
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(&ht[buf][(32 * mt + l32) * kHS + 16 * s + 8 * hh]);
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) acc[mt][nt] = mfma32(a, bm[nt], acc[mt][nt]);
      }
    }
    if (c + 1 < nchunks) {
      SLA_STORE_CHUNK(buf ^ 1);
      if (c + 2 < nchunks) SLA_LOAD_CHUNK(c + 2);
    }
    __syncthreads();
  }

#undef SLA_LOAD_CHUNK
#undef SLA_STORE_CHUNK

  // epilogue: acc[mt][nt][r] = C[i = i0 + 64*wave + 32*nt + l32][col = 32*mt + 8*(r/4) + 4*hh + r%4]
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    if (!rok[nt]) continue;
    const int64_t i = static_cast<int64_t>(i0 + 64 * wave + 32 * nt + l32);
    const int64_t row = static_cast<int64_t>(bh) * nq + i;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int col = 32 * mt + 8 * r4 + 4 * hh;
        if (!ztile) {
          u32x2 w;
          w[0] = static_cast<uint32_t>(f32_to_bf16_bits(acc[mt][nt][4 * r4])) |
                 (static_cast<uint32_t>(f32_to_bf16_bits(acc[mt][nt][4 * r4 + 1])) << 16);
          w[1] = static_cast<uint32_t>(f32_to_bf16_bits(acc[mt][nt][4 * r4 + 2])) |
                 (static_cast<uint32_t>(f32_to_bf16_bits(acc[mt][nt][4 * r4 + 3])) << 16);
          *reinterpret_cast<u32x2*>(s_out + row * D * D + ct * kTN + col) = w;
        } else {
          float2 sg;
          sg.x = acc[mt][nt][4 * r4] + acc[mt][nt][4 * r4 + 1];
          sg.y = acc[mt][nt][4 * r4 + 2] + acc[mt][nt][4 * r4 + 3];
          *reinterpret_cast<float2*>(sigma_out + row * D + (ct - HT) * 64 + col / 2) = sg;
        }
      }
  }
}

}  // namespace

hipError_t launch_marginal_sums(const Geometry& g, const int32_t* marg, const uint16_t* h_states,
                                const float* z_states, uint16_t* s_sum, float* sigma_sum,
                                uint32_t* bits, hipStream_t stream) {
  const int nw = marginal_bit_words(g);     // one 32-bit word per chunk of 32 KV blocks
  dim3 g1((g.nq + 63) / 64, g.B * g.H);
  hipLaunchKernelGGL(marg_bits_kernel, g1, dim3(kThreads), 64 * nw * sizeof(uint32_t), stream,
                     g, marg, bits, nw);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (g.D == 128) {
    dim3 g2((g.nq + kTM - 1) / kTM, 128 * 128 / kTN + 2, g.B * g.H);
    hipLaunchKernelGGL((marg_gemm_kernel<128>), g2, dim3(kThreads), 0, stream, g, bits, nw,
                       h_states, z_states, s_sum, sigma_sum);
  } else {
    dim3 g2((g.nq + kTM - 1) / kTM, 64 * 64 / kTN + 1, g.B * g.H);
    hipLaunchKernelGGL((marg_gemm_kernel<64>), g2, dim3(kThreads), 0, stream, g, bits, nw,
                       h_states, z_states, s_sum, sigma_sum);
  }
  return hipGetLastError();
}

}  // namespace sla
