// OCP E4M3 encoding and the per-block scale of the low-bit sparse branch,
// shared by the stand-alone quantiser and the passes that quantise the
// tiles they already hold (the pooling pass for Q and K, the states pass
// for V).
//
// [SLA2 technical summary, section 2.C] the sparse branch runs in a low-bit
// format.  Each (b, h, 64-token block) of a tensor gets one float32 scale:
//   r = fl32(448 / absmax), scale = fl32(absmax / 448), code = e4m3(fl32(x * r))
// (scale 1 and all-zero codes for an all-zero block).
#pragma once

#include "device_common.hpp"

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

// Largest of the 256 threads' values (4 waves; wmax: 4 floats of LDS).
// Every thread returns it; contains one barrier.
__device__ __forceinline__ float workgroup_max4(float a, float* wmax) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) a = fmaxf(a, __shfl_xor(a, o, 64));
  if (lane == 0) wmax[wave] = a;
  __syncthreads();
  return fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
}

// Scale factor r applied before encoding, and the stored scale, of a block
// whose largest magnitude is amax.
__device__ __forceinline__ float e4m3_block_factor(float amax) {
  return amax > 0.0f ? __fdiv_rn(448.0f, amax) : 1.0f;
}
__device__ __forceinline__ float e4m3_block_scale(float amax) {
  return amax > 0.0f ? __fdiv_rn(amax, 448.0f) : 1.0f;
}

// Codes of 8 consecutive values, packed little-endian.
__device__ __forceinline__ u32x2 e4m3_pack8(const float* v, float r) {
  u32x2 w;
  w[0] = w[1] = 0u;
#pragma unroll
  for (int e = 0; e < 8; ++e) w[e >> 2] |= e4m3_encode(__fmul_rn(v[e], r)) << (8 * (e & 3));
  return w;
}

}  // namespace sla
