// Per-block linear-attention states.
//
// [PISA technical summary, "Algoritmo Central"] each KV block j has a
// first-order matrix built from its keys and values; [SPLA technical
// summary, section 2.2] blocks outside the exact set are compressed into a
// compact linear-attention state.  Here:
//   H_j = phi(K_j)^T V_j   (d x d, bf16 out, float32 accumulation)
//   z_j = sum over the block's tokens of phi(k)   (d, float32)
// with phi = softmax over the d features, evaluated in float32, or (the
// exponential map of residual linear attention) phi(k) = exp(k).  H_j is
// stored value-major, element [c][a] = sum_n v_n[c] phi(k_n)[a] (that is,
// H_j^T row-major), the operand layout in which the marginal sums feed the
// matrix cores of the attention kernel directly.
//
// One workgroup per (b, h, j): the 64 x d tiles of K and V are read once
// (coalesced 16-byte loads), phi(K)^T and V^T are staged token-contiguous in
// LDS as bf16, and the d x d product runs on v_mfma_f32_32x32x16_bf16 with
// the 64 tokens as the contraction dimension.  The kernel is HBM-bound: it
// reads 2*64*d and writes d*d elements per block.
#include "device_common.hpp"
#include "fp8_encode.hpp"
#include "sla_internal.hpp"

namespace sla {
namespace {

// EXPMAP: phi(k) = exp(k) elementwise, with no per-token normalisation
// ([SPLA technical summary, section 2.3] parameter-free exponential map).
// QNT (low-bit sparse branch): also the V block's E4M3 codes and float32
// scale ([SLA2 technical summary, section 2.C]; the bytes of the
// stand-alone quantiser), from the V rows already in registers.
// POOLK (bf16 inputs): also the block's pooled key row for the router
// ([SLA2 technical summary, section 2.B]), the float64 mean of the valid
// keys, into the pooled-K rows [B*H][nkb][d] the split routing path reads
// (and float32 into kout when non-null), so routing needs no second pass
// over K.
// The sum runs in the routing pooling kernel's order (rows r, r + RG, ...
// per row group r, then the row groups in order), so the means are that
// kernel's bit for bit.
template <typename T, int D, bool EXPMAP, bool QNT = false, bool POOLK = false>
__global__ void __launch_bounds__(kThreads)
states_kernel(const T* __restrict__ k, const T* __restrict__ v, Geometry g,
              uint16_t* __restrict__ h_out, float* __restrict__ z_out,
              uint8_t* __restrict__ v8 = nullptr, float* __restrict__ v_scale = nullptr,
              double* __restrict__ kpool = nullptr, float* __restrict__ kout = nullptr) {
  constexpr int TS = kBlock + 8;        // token stride of the transposed tiles
  constexpr int HS = D + 8;             // row stride of the staged (value-major) output tile
  constexpr int CW = D / 4;             // features per thread (4 threads per token)
  constexpr int TA = D / 32;            // 32-row tiles per dimension
  constexpr int NT = TA * TA / 4;       // output tiles per wave
  constexpr int SMEM_OP = (2 * D * TS > D * HS) ? 2 * D * TS : D * HS;
  // POOLK: the raw key rows, then float64 partial sums [row groups][D]
  constexpr int SMEM_PK = (64 * HS + 7) / 8 * 8 + (kThreads / (D / 8)) * D * 4;
  constexpr int SMEM = (POOLK && SMEM_PK > SMEM_OP) ? SMEM_PK : SMEM_OP;
  __shared__ __attribute__((aligned(16))) uint16_t smem[SMEM];
  __shared__ float zpart[4][D];
  uint16_t* phi_t = smem;               // [D][TS]: phi(K)^T
  uint16_t* v_t = smem + D * TS;        // [D][TS]: V^T

  const int j = blockIdx.x, bh = blockIdx.y;
  const int b = bh / g.H, h = bh % g.H;
  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);   // wave-uniform (scalar)
  const int row = t >> 2, part = t & 3;
  const int nj = min(kBlock, g.N - j * kBlock);
  const bool valid = row < nj;

  // rows past a short last block load its last row (all loads in flight
  // together); their phi is zeroed below
  const int64_t off = b * g.sb + h * g.sh + static_cast<int64_t>(j * kBlock + min(row, nj - 1)) * g.sn +
                      part * CW;
  float kv[CW], vv[CW];
#pragma unroll
  for (int c = 0; c < CW / 8; ++c) {
    load8_f32(k + off + 8 * c, kv + 8 * c);
    load8_f32(v + off + 8 * c, vv + 8 * c);
  }

  if constexpr (POOLK) {
    // raw keys as bf16 (exact: the inputs are bf16) in the smem rows, then
    // one thread per feature sums its column
    static_assert(sizeof(T) == 2, "pooled keys from the states pass: bf16 inputs");
    constexpr int PRG = kThreads / (D / 8);       // row groups of the pooling kernel
    constexpr int PRPG = kBlock / PRG;            // rows per group
#pragma unroll
    for (int c = 0; c < CW; c += 2)
      *reinterpret_cast<uint32_t*>(&smem[row * HS + part * CW + c]) =
          static_cast<uint32_t>(f32_to_bf16_bits(kv[c])) |
          (static_cast<uint32_t>(f32_to_bf16_bits(kv[c + 1])) << 16);
    __syncthreads();
    // phase 1, all threads: the partial sum of each (row group, feature) in
    // row order, 8 row groups per thread; phase 2: one thread per feature
    // adds its row groups in order
    static_assert(PRG * D / kThreads == 8, "8 row groups per thread");
    double* gsum = reinterpret_cast<double*>(smem + (64 * HS + 7) / 8 * 8);   // [PRG][D]
    {
      const int c = t % D, rg0 = (t / D) * 8;
#pragma unroll
      for (int x = 0; x < 8; ++x) {
        const int rg = rg0 + x;
        double acc = 0.0;
#pragma unroll
        for (int rr = 0; rr < PRPG; ++rr) {
          const int r = rg + rr * PRG;
          acc += r < nj ? static_cast<double>(bf16_to_f32(smem[r * HS + c])) : 0.0;
        }
        gsum[rg * D + c] = acc;
      }
    }
    __syncthreads();
    if (t < D) {
      double sum = 0.0;
#pragma unroll
      for (int rg = 0; rg < PRG; ++rg) sum += gsum[rg * D + t];
      const double m = sum / static_cast<double>(nj);
      kpool[(static_cast<int64_t>(bh) * g.nkb + j) * D + t] = m;
      if (kout) kout[(static_cast<int64_t>(bh) * g.nkb + j) * D + t] = static_cast<float>(m);
    }
    __syncthreads();   // the rows are read before the operand tiles reuse smem
  }

  if constexpr (EXPMAP) {
#pragma unroll
    for (int c = 0; c < CW; ++c) kv[c] = valid ? __builtin_amdgcn_exp2f(kv[c] * kLog2e) : 0.0f;
  } else {
    // phi(k) = softmax over the d features of the token (4 lanes per token:
    // quad_perm DPP moves give the partners)
    float mx = vmax3(kv[0], kv[1], kv[2]);
#pragma unroll
    for (int c = 3; c + 1 < CW; c += 2) mx = vmax3(mx, kv[c], kv[c + 1]);
    if (CW % 2 == 0) mx = vmax3(mx, kv[CW - 1], kv[CW - 1]);
    mx = vmax3(mx, dpp_f<0xB1>(mx), dpp_f<0x4E>(mx));
    mx = vmax3(mx, dpp_f<0x4E>(mx), dpp_f<0x4E>(mx));
    const float mb = mx * kLog2e;
    float sum = 0.0f;
#pragma unroll
    for (int c = 0; c < CW; ++c) {
      kv[c] = __builtin_amdgcn_exp2f(fmaf(kv[c], kLog2e, -mb));
      sum += kv[c];
    }
    sum += dpp_f<0xB1>(sum);
    sum += dpp_f<0x4E>(sum);
    const float inv = valid ? 1.0f / sum : 0.0f;
#pragma unroll
    for (int c = 0; c < CW; ++c) kv[c] *= inv;
  }

  // z: column sums over the wave's 16 tokens (lanes part + 4m: row_ror 4
  // and 8 inside each row of 16, then the row and half swaps), then over
  // the 4 waves
#pragma unroll
  for (int c = 0; c < CW; ++c) {
    float zc = kv[c];
    zc += dpp_f<0x124>(zc);
    zc += dpp_f<0x128>(zc);
    zc = swap_sum16(zc);
    zc = swap_sum32(zc);
    if (lane < 4) zpart[wave][part * CW + c] = zc;
  }

  if constexpr (QNT) {
    __shared__ float wmax[4];
    float amax = 0.0f;
#pragma unroll
    for (int c = 0; c < CW; ++c) amax = fmaxf(amax, valid ? fabsf(vv[c]) : 0.0f);
    amax = workgroup_max4(amax, wmax);
    const float r = e4m3_block_factor(amax);
    if (t == 0) v_scale[static_cast<int64_t>(bh) * g.nq + j] = e4m3_block_scale(amax);
    if (valid) {
      uint8_t* codes = v8 + (static_cast<int64_t>(bh) * g.N + j * kBlock + row) * D + part * CW;
#pragma unroll
      for (int c = 0; c < CW / 8; ++c) *reinterpret_cast<u32x2*>(codes + 8 * c) = e4m3_pack8(vv + 8 * c, r);
    }
  }

  // token-contiguous bf16 operands: phi_t[a][token], v_t[c][token]
#pragma unroll
  for (int c = 0; c < CW; ++c) {
    phi_t[(part * CW + c) * TS + row] = f32_to_bf16_bits(kv[c]);
    v_t[(part * CW + c) * TS + row] = f32_to_bf16_bits(vv[c]);
  }
  __syncthreads();

  const int64_t blk = static_cast<int64_t>(bh) * g.nkb + j;
  if (t < D) z_out[blk * D + t] = zpart[0][t] + zpart[1][t] + zpart[2][t] + zpart[3][t];

  const int l32 = lane & 31, hh = lane >> 5;
  f32x16 acc[NT];
#pragma unroll
  for (int u = 0; u < NT; ++u) {
    const int ti = wave * NT + u;
    const int at = ti / TA, ct = ti % TA;
    acc[u] = zero16();
#pragma unroll
    for (int s = 0; s < kBlock / 16; ++s) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(&phi_t[(at * 32 + l32) * TS + 16 * s + 8 * hh]);
      const bf16x8 bb = *reinterpret_cast<const bf16x8*>(&v_t[(ct * 32 + l32) * TS + 16 * s + 8 * hh]);
      acc[u] = mfma32(a, bb, acc[u]);
    }
  }
  __syncthreads();   // operands consumed; reuse smem as the output tile

  // value-major staging: row c = ct*32 + l32, features a (pairs of
  // consecutive a packed into one 32-bit store)
#pragma unroll
  for (int u = 0; u < NT; ++u) {
    const int ti = wave * NT + u;
    const int at = ti / TA, ct = ti % TA;
    uint16_t* srow = smem + (ct * 32 + l32) * HS;
#pragma unroll
    for (int r = 0; r < 16; r += 2) {
      const int a = at * 32 + 8 * (r >> 2) + 4 * hh + (r & 3);
      *reinterpret_cast<uint32_t*>(srow + a) =
          static_cast<uint32_t>(f32_to_bf16_bits(acc[u][r])) |
          (static_cast<uint32_t>(f32_to_bf16_bits(acc[u][r + 1])) << 16);
    }
  }
  __syncthreads();
  uint16_t* dst = h_out + blk * D * D;
  for (int e = t; e < D * D / 8; e += kThreads) {
    const int c = e / (D / 8), a8 = e % (D / 8);
    *reinterpret_cast<u32x4*>(dst + c * D + a8 * 8) =
        *reinterpret_cast<const u32x4*>(&smem[c * HS + a8 * 8]);
  }
}

template <typename T, int D>
void launch_states_t(const Geometry& g, const void* k, const void* v, uint16_t* hs, float* zs,
                     bool exp_map, hipStream_t stream, uint8_t* v8, float* vs, double* kpool,
                     float* kout) {
  dim3 grid(g.nkb, g.B * g.H);
  if constexpr (sizeof(T) == 2) {
    if (kpool) {
      hipLaunchKernelGGL((states_kernel<T, D, false, false, true>), grid, dim3(kThreads), 0, stream,
                         static_cast<const T*>(k), static_cast<const T*>(v), g, hs, zs, nullptr,
                         nullptr, kpool, kout);
      return;
    }
  }
  if (v8)
    hipLaunchKernelGGL((states_kernel<T, D, false, true>), grid, dim3(kThreads), 0, stream,
                       static_cast<const T*>(k), static_cast<const T*>(v), g, hs, zs, v8, vs);
  else if (exp_map)
    hipLaunchKernelGGL((states_kernel<T, D, true>), grid, dim3(kThreads), 0, stream,
                       static_cast<const T*>(k), static_cast<const T*>(v), g, hs, zs);
  else
    hipLaunchKernelGGL((states_kernel<T, D, false>), grid, dim3(kThreads), 0, stream,
                       static_cast<const T*>(k), static_cast<const T*>(v), g, hs, zs);
}

}  // namespace

hipError_t launch_states(const Geometry& g, const void* k, const void* v, uint16_t* h_states,
                         float* z_states, bool exp_map, hipStream_t stream, uint8_t* v8,
                         float* v_scale, double* kpool, float* kout) {
  if (kpool && (g.dtype != 1 || exp_map || v8)) return hipErrorInvalidValue;
  if (g.dtype == 1) {
    if (g.D == 128) launch_states_t<uint16_t, 128>(g, k, v, h_states, z_states, exp_map, stream, v8, v_scale, kpool, kout);
    else launch_states_t<uint16_t, 64>(g, k, v, h_states, z_states, exp_map, stream, v8, v_scale, kpool, kout);
  } else {
    if (g.D == 128) launch_states_t<float, 128>(g, k, v, h_states, z_states, exp_map, stream, v8, v_scale, nullptr, nullptr);
    else launch_states_t<float, 64>(g, k, v, h_states, z_states, exp_map, stream, v8, v_scale, nullptr, nullptr);
  }
  return hipGetLastError();
}

}  // namespace sla
