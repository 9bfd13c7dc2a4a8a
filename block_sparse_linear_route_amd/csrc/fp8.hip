// Low-bit sparse branch: per-block OCP E4M3 quantiser.
//
// [SLA2 technical summary, section 2.C] the sparse branch runs in a low-bit
// format; the per-block scale and the encoding (fp8_encode.hpp: round to
// nearest even, saturating at +-448 by construction of the scale, -0 kept
// as 0x80) make the bytes those the OCP 8-bit floating-point format fixes
// for the scaled values.
#include "fp8_encode.hpp"
#include "sla_internal.hpp"

namespace sla {

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
  const int t = threadIdx.x;
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
  amax = workgroup_max4(amax, wmax);
  const float r = e4m3_block_factor(amax);
  if (t == 0) scales[static_cast<int64_t>(bh) * g.nq + j] = e4m3_block_scale(amax);

  uint8_t* dst = codes + (static_cast<int64_t>(bh) * g.N + j * kBlock) * D;
#pragma unroll
  for (int u = 0; u < NCH; ++u) {
    const int id = t + kThreads * u;
    const int row = id / CH, c8 = id % CH;
    if (row < nj) *reinterpret_cast<u32x2*>(dst + row * D + 8 * c8) = e4m3_pack8(v[u], r);
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
