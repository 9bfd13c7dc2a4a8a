// Device-side helpers shared by the gfx950 kernels of libsla.
//
// Conventions used by every kernel:
//  * 256-thread workgroups = 4 waves of 64 lanes (CDNA wavefront).
//  * bf16 tensors are carried as raw uint16_t bit patterns in memory and as
//    __bf16 vectors in registers for the matrix-core builtins.
//  * Matrix-core tiles use v_mfma_f32_32x32x16_bf16: lane l holds row/column
//    (l % 32) of an A/B operand and 8 consecutive k-slots chosen by (l / 32);
//    the 32x32 float accumulator gives lane l column (l % 32) and rows
//    8*(r/4) + 4*(l/32) + (r%4) for its 16 registers r.  A and B operands use
//    the same k-slot mapping, so any assignment of k indices to slots that is
//    applied identically to both operands yields the full dot product.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sla {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef int32_t i32x8 __attribute__((ext_vector_type(8)));

constexpr int kBlock = 64;
constexpr int kThreads = 256;
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round-to-nearest-even float -> bf16 (the gfx950 conversion instruction).
__device__ __forceinline__ __bf16 f32_to_bf16(float f) { return static_cast<__bf16>(f); }

__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  __bf16 h = static_cast<__bf16>(f);
  return __builtin_bit_cast(uint16_t, h);
}

__device__ __forceinline__ float bf16v_to_f32(__bf16 h) {
  return __uint_as_float(static_cast<uint32_t>(__builtin_bit_cast(uint16_t, h)) << 16);
}

// 8 consecutive elements as a bf16 vector (pointer 16-byte aligned for bf16,
// 32-byte aligned for float).
__device__ __forceinline__ bf16x8 load8(const uint16_t* p) {
  return *reinterpret_cast<const bf16x8*>(p);
}
__device__ __forceinline__ bf16x8 load8(const float* p) {
  const f32x4 a = *reinterpret_cast<const f32x4*>(p);
  const f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
  bf16x8 r;
  r[0] = f32_to_bf16(a[0]); r[1] = f32_to_bf16(a[1]);
  r[2] = f32_to_bf16(a[2]); r[3] = f32_to_bf16(a[3]);
  r[4] = f32_to_bf16(b[0]); r[5] = f32_to_bf16(b[1]);
  r[6] = f32_to_bf16(b[2]); r[7] = f32_to_bf16(b[3]);
  return r;
}

// 8 consecutive elements at a 32-bit byte offset from a uniform base, so the
// load can use the scalar-base + vector-offset addressing form.
template <typename T>
__device__ __forceinline__ bf16x8 load8_at(const T* base, uint32_t byte_off) {
  return load8(reinterpret_cast<const T*>(reinterpret_cast<const char*>(base) + byte_off));
}

// 8 consecutive elements widened to float.
__device__ __forceinline__ void load8_f32(const uint16_t* p, float* out) {
  const u32x4 w = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    out[2 * i] = __uint_as_float(w[i] << 16);
    out[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}
__device__ __forceinline__ void load8_f32(const float* p, float* out) {
  const f32x4 a = *reinterpret_cast<const f32x4*>(p);
  const f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
  for (int i = 0; i < 4; ++i) { out[i] = a[i]; out[4 + i] = b[i]; }
}

__device__ __forceinline__ bf16x8 zero_bf16x8() {
  bf16x8 r;
#pragma unroll
  for (int i = 0; i < 8; ++i) r[i] = f32_to_bf16(0.0f);
  return r;
}

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 zero16() {
  f32x16 r;
#pragma unroll
  for (int i = 0; i < 16; ++i) r[i] = 0.0f;
  return r;
}

// Direct global -> LDS load of 16 bytes per lane: lane l's bytes land at
// lds_base + 16 * l (lds_base must be uniform across the wave).
__device__ __forceinline__ void load_lds16(const void* gsrc, void* lds_base) {
  __builtin_amdgcn_global_load_lds(gsrc, (__attribute__((address_space(3))) void*)lds_base, 16, 0, 0);
}

// Wait until all of this wave's vector-memory loads (including direct-to-LDS
// loads) have completed.  Issued through the builtin, not inline asm, so the
// compiler's own wait-count tracking knows that nothing is outstanding after
// it (s_waitcnt vmcnt(0) with the other counters left at their maximum).
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Buffer resource over [base, base + bytes): raw (unstructured) loads through
// it are range-checked per dword, and dwords past the end read as zero.  The
// check covers the whole offset, the scalar (soffset) part included, for
// loads into registers and direct loads into LDS alike (verified on gfx950
// with offsets past the end inside a larger allocation: all zeros), so a
// tile base passed as soffset still gets zeros past the tensor's end.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(bytes),
                                           0x00020000);
}

// Range-checked direct buffer -> LDS load of 16 bytes per lane from byte
// offset voff + soff: lane l's bytes land at lds_base + 16 * l (lds_base
// uniform across the wave).
__device__ __forceinline__ void buffer_load_lds16(__amdgpu_buffer_rsrc_t r, void* lds_base,
                                                  uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds_base, 16,
                                           voff, soff, 0, 0);
}

// Transposing LDS read of 4 bf16 (gfx950 ds_read_b64_tr_b16): within each
// group of 16 lanes, lane i receives element (i % 4) of the 8-byte rows
// addressed by lanes 4e + i/4 of the group, for e = 0..3.
typedef short s16x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ u32x2 lds_read_tr16(const uint16_t* p) {
  const s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)(const_cast<uint16_t*>(p)));
  return __builtin_bit_cast(u32x2, r);
}

// 32-bit LDS byte address of a pointer into a __shared__ array.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
      (const __attribute__((address_space(3))) void*)(p)));
}

// Lane-crossing helpers (wave64).
__device__ __forceinline__ float xor_lane(float v, int mask) { return __shfl_xor(v, mask, 64); }

// DPP lane move of a float (bound_ctrl: lanes without a source read 0).
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, true));
}

// v + v of lane l ^ 16 (v_permlane16_swap) and v + v of lane l ^ 32
// (v_permlane32_swap).
__device__ __forceinline__ float swap_sum16(float v) {
  const auto sw = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
}
__device__ __forceinline__ float swap_sum32(float v) {
  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
}

// max(a, b, c) as one v_max3_f32.  fmaxf on matrix-core results costs an
// extra quieting move per input (the compiler cannot tell they are not
// signalling NaNs); softmax row maxima only ever see finite scores or -inf.
__device__ __forceinline__ float vmax3(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

// Maximum of the 16 registers of an accumulator, as a tree of v_max3_f32.
__device__ __forceinline__ float max16(const f32x16& s) {
  const float a = vmax3(s[0], s[1], s[2]), b = vmax3(s[3], s[4], s[5]);
  const float c = vmax3(s[6], s[7], s[8]), d = vmax3(s[9], s[10], s[11]);
  const float e = vmax3(s[12], s[13], s[14]);
  const float f = vmax3(d, e, s[15]);
  return vmax3(vmax3(a, b, c), f, f);
}

// A KV block index read from a caller's list, clamped into [0, nkb): every
// address formed from a list entry then stays inside the tensors whatever
// the list holds (entries outside the range give meaningless results, not
// out-of-bounds accesses; sla_validate_lists reports them).
__device__ __forceinline__ int list_block(int j, int nkb) { return min(max(j, 0), nkb - 1); }

// Workgroup id remapped so that each XCD (the hardware dispatches workgroups
// round-robin over 8 XCDs) owns one contiguous range of logical work items,
// which keeps neighbouring query blocks of one head in the same L2.
__device__ __forceinline__ int xcd_remap(int wg, int n) {
  constexpr int kXcd = 8;
  const int xcd = wg % kXcd;
  const int idx = wg / kXcd;
  const int per = n / kXcd;
  const int rem = n % kXcd;
  return (xcd < rem) ? xcd * (per + 1) + idx : rem * (per + 1) + (xcd - rem) * per + idx;
}

}  // namespace sla
