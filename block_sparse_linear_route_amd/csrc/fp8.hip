// Low-bit sparse branch: per-block OCP E4M3 quantiser.
//
// [SLA2 technical summary, section 2.C] the sparse branch runs in a low-bit
// format.  Each (b, h, 64-token block) of a tensor gets one float32 scale:
//   r = fl32(448 / absmax), scale = fl32(absmax / 448), code = e4m3(fl32(x * r))
// (scale 1 and all-zero codes for an all-zero block).  The float -> E4M3
// conversion is done in integer/float steps below (round to nearest even,
// saturate finite values to +-448, -0 kept as 0x80) so that the bytes are
// fully specified by the OCP 8-bit floating-point format rather than by a
// conversion instruction's modes.
#include "device_common.hpp"
#include "sla_internal.hpp"

namespace sla {

__device__ __forceinline__ uint32_t e4m3_encode(float x) {
  const uint32_t bits = __float_as_uint(x);
  const uint32_t sign = (bits >> 24) & 0x80u;
  const float a = fabsf(x);
  if (a < 0.015625f) {                       // below 2^-6: grid of 2^-9
    const uint32_t m = static_cast<uint32_t>(rintf(a * 512.0f));   // 0..8, 8 = 2^-6
    return sign | m;
  }
  int e = static_cast<int>((bits >> 23) & 0xffu) - 127;     // a is a normal float
  if (e > 8) return sign | 0x7eu;
  uint32_t m = static_cast<uint32_t>(rintf(ldexpf(a, 3 - e)));   // 8..16
  if (m == 16u) { m = 8u; ++e; }
  if (e > 8 || (e == 8 && m > 14u)) return sign | 0x7eu;
  return sign | (static_cast<uint32_t>(e + 7) << 3) | (m - 8u);
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
    const int id = t + kThreads * u;
    const int row = id / CH, c8 = id % CH;
    if (row < nj) {
      load8_f32(src + static_cast<int64_t>(j * kBlock + row) * g.sn + 8 * c8, v[u]);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) v[u][e] = 0.0f;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(v[u][e]));
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
