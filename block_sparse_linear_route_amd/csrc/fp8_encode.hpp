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

// Codes of 8 consecutive values, packed little-endian, by the matrix-core
// format's own conversion (v_cvt_pk_fp8_f32: OCP E4M3, round to nearest
// even, subnormals kept, -0 as 0x80).  The scaled values lie within
// 448 (1 + 2^-22) in magnitude (x is at most the block's absolute maximum
// and r = fl32(448 / absmax)), below 464, the midpoint to the next
// magnitude, so they round to at most 448 and the conversion never
// overflows; the codes are those of rounding to nearest even with
// saturation.  A non-finite input makes the block's scale non-finite and
// its codes unspecified.
__device__ __forceinline__ u32x2 e4m3_pack8(const float* v, float r) {
  int w0 = 0, w1 = 0;
  w0 = __builtin_amdgcn_cvt_pk_fp8_f32(__fmul_rn(v[0], r), __fmul_rn(v[1], r), w0, false);
  w0 = __builtin_amdgcn_cvt_pk_fp8_f32(__fmul_rn(v[2], r), __fmul_rn(v[3], r), w0, true);
  w1 = __builtin_amdgcn_cvt_pk_fp8_f32(__fmul_rn(v[4], r), __fmul_rn(v[5], r), w1, false);
  w1 = __builtin_amdgcn_cvt_pk_fp8_f32(__fmul_rn(v[6], r), __fmul_rn(v[7], r), w1, true);
  u32x2 w;
  w[0] = static_cast<uint32_t>(w0);
  w[1] = static_cast<uint32_t>(w1);
  return w;
}

}  // namespace sla
