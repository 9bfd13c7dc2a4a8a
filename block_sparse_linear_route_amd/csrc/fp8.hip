// Low-bit sparse branch: per-block OCP E4M3 quantiser.
//
// [SLA2 technical summary, section 2.C] the sparse branch runs in a low-bit
// format.  Each (b, h, 64-token block) of a tensor gets one float32 scale:
//   r = fl32(448 / absmax), scale = fl32(absmax / 448), code = e4m3(fl32(x * r))
// (scale 1 and all-zero codes for an all-zero block).  The float -> E4M3
// conversion is done in integer/float steps below (round to nearest even,
// saturate to +-448, -0 kept as 0x80) so that the bytes are
// fully specified by the OCP 8-bit floating-point format rather than by a
// conversion instruction's modes.
#include "device_common.hpp"
#include "sla_internal.hpp"

namespace sla {

// E4M3 code of x, branch-free.  |x| >= 2^-6: adding 2^19 - 1 plus the kept
// lowest bit to the float's bits and dropping 20 mantissa bits rounds to 3
// mantissa bits, nearest even, with any carry moving into the exponent; the
// result minus (127 - 7) << 3 is the code (exponent bias 7), and everything
// above 448 (0x7e), infinities and NaN included, saturates to 0x7e.  Below
// 2^-6 the codes are the multiples of 2^-9 (code 8 being 2^-6 itself).
__device__ __forceinline__ uint32_t e4m3_encode(float x) {
  const uint32_t bits = __float_as_uint(x);
  const uint32_t sign = (bits >> 24) & 0x80u;
  const uint32_t ab = bits & 0x7fffffffu;
  const uint32_t rn = (ab + 0x7ffffu + ((ab >> 20) & 1u)) >> 20;
  const uint32_t nc = min(rn - (120u << 3), 0x7eu);
  const uint32_t sc = static_cast<uint32_t>(rintf(__uint_as_float(ab) * 512.0f));
  return sign | (ab < 0x3c800000u ? sc : nc);
}

namespace {

template <typename T, int D>
__global__ void __launch_bounds__(kThreads)
quantize_kernel(const T* __restrict__ x, Geometry g, uint8_t* __restrict__ codes,
                float* __restrict__ scales) {
  constexpr int CH = D / 8;
  constexpr int NCH = kBlock * CH / kThreads;   // 8-element chunks per thread
  __shared__ float wmax[4];
  const int j = blockIdx.x, bh = blockIdx.y;
  const int b = bh / g.H, h = bh % g.H;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int nj = min(kBlock, g.N - j * kBlock);
  const T* src = x + b * g.sb + h * g.sh;

  float v[NCH][8];
  float amax = 0.0f;
#pragma unroll
  for (int u = 0; u < NCH; ++u) {
    // rows past a short last block load its last row and are zeroed after
    // the load, so all loads are in flight together
    const int id = t + kThreads * u;
    const int row = id / CH, c8 = id % CH;
    load8_f32(src + static_cast<int64_t>(j * kBlock + min(row, nj - 1)) * g.sn + 8 * c8, v[u]);
  }
#pragma unroll
  for (int u = 0; u < NCH; ++u) {
    const bool in = (t + kThreads * u) / CH < nj;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      v[u][e] = in ? v[u][e] : 0.0f;
      amax = fmaxf(amax, fabsf(v[u][e]));
    }
  }
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) amax = fmaxf(amax, xor_lane(amax, o));
  if (lane == 0) wmax[wave] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
  const bool zero = !(amax > 0.0f);
  const float r = zero ? 1.0f : __fdiv_rn(448.0f, amax);
  if (t == 0) scales[static_cast<int64_t>(bh) * g.nq + j] = zero ? 1.0f : __fdiv_rn(amax, 448.0f);

  uint8_t* dst = codes + (static_cast<int64_t>(bh) * g.N + j * kBlock) * D;
#pragma unroll
  for (int u = 0; u < NCH; ++u) {
    const int id = t + kThreads * u;
    const int row = id / CH, c8 = id % CH;
    if (row < nj) {
      u32x2 w;
      w[0] = w[1] = 0u;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float y = __fmul_rn(v[u][e], r);
        w[e >> 2] |= e4m3_encode(y) << (8 * (e & 3));
      }
      *reinterpret_cast<u32x2*>(dst + row * D + 8 * c8) = w;
    }
  }
}

template <typename T, int D>
void launch_q_t(const Geometry& g, const void* x, uint8_t* codes, float* scales, hipStream_t s) {
  dim3 grid(g.nq, g.B * g.H);
  hipLaunchKernelGGL((quantize_kernel<T, D>), grid, dim3(kThreads), 0, s,
                     static_cast<const T*>(x), g, codes, scales);
}

}  // namespace

hipError_t launch_quantize_fp8(const Geometry& g, const void* x, uint8_t* codes, float* scales,
                               hipStream_t stream) {
  if (g.dtype == 1) {
    if (g.D == 128) launch_q_t<uint16_t, 128>(g, x, codes, scales, stream);
    else launch_q_t<uint16_t, 64>(g, x, codes, scales, stream);
  } else {
    if (g.D == 128) launch_q_t<float, 128>(g, x, codes, scales, stream);
    else launch_q_t<float, 64>(g, x, codes, scales, stream);
  }
  return hipGetLastError();
}

}  // namespace sla
