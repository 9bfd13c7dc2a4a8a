// Marginal-state sums of the linear branch.
//
// [SLA abstract] marginal KV blocks get O(N) linear attention; [PISA
// technical summary] per-block first-order matrices H_j; the linear branch of
// query block i needs S_i = sum_{j in M_i} H_j and sigma_i = sum_{j in M_i}
// z_j.
//
// Per head, S is a product with the 0/1 marginal mask M ([nq x nkb], exact in
// bf16): S[i, e] = sum_j M[i, j] H[j, e], e running over the d*d entries of
// the value-major states.  It runs as a dense bf16 GEMM on
// v_mfma_f32_32x32x16_bf16 with float32 accumulation, so every product is
// exact and S is the float32 sum of the bf16 states, rounded once to bf16.
//
// Kernel 1 (a few query blocks per workgroup) writes the mask as bit rows,
// laid out chunk-major (64 KV blocks per chunk, two 32-bit words per row) so
// that a chunk's bits for 512 rows are one contiguous 4 KB piece, and splits
// each z_j into two bf16 parts hi + lo (hi = bf16(z), lo = bf16(z - hi)).
// sigma_i = sum_j M[i, j] (hi_j + lo_j) then comes out of the same product
// as S (the parts are exact bf16 values, the sums float32): its float32 sum
// differs from the sum of the float32 z_j by the rounding of lo, about
// 2^-17 of z.
//
// Kernel 2 computes S^T tiles of 64 columns x 512 rows per workgroup, so H is
// streamed from HBM once per head for nq <= 512.  Each 64-block chunk of H
// (64 rows of 128 bytes) and of the bit rows reaches LDS by direct buffer
// loads through a 3-stage ring of separate LDS arrays (the loop is unrolled
// over the stages, so the compiler can tell the stage being read from the
// stages being filled and needs no wait on the loads in flight).  The H^T
// operand comes from the row-major chunk by transposing LDS reads
// (ds_read_b64_tr_b16), and the mask operand is expanded 4 bits at a time
// through a 16-entry LDS table of bf16 0/1 quadruples.
#include "device_common.hpp"
#include "sla_internal.hpp"

#include <type_traits>

namespace sla {
namespace {

constexpr int kGN = 64;                   // S columns per GEMM workgroup
constexpr int kGK = 64;                   // KV blocks per chunk
constexpr int kStages = 3;                // 3 to 6
constexpr int kHBytes = kGK * kGN * 2;    // H chunk bytes (8 KB)
constexpr int kTotParts = 4;              // row ranges of the global-state partial sums

// grid (ceil(nq / RPB), B*H), RPB = 256 / D query blocks per workgroup,
// thread (row, feature a):
//  * the mask bit row of each row's marginal list, OR-ed together in LDS and
//    written chunk-major: word w of row i lands at
//    [(w / 2) * rows_pad + i] * 2 + w % 2;
//  * (nq = nkb) the z row of KV block j = i as bf16 parts, laid out per
//    32-feature group x as [hi of 32x .. 32x+31 | lo of the same], so that
//    one 64-column tile of the product carries both parts of 32 features.
//
// MODE 0: the marginal lists, and the z parts.  MODE 1: the list is each
// row's critical list (k_crit entries) and the bit row written is its
// complement over the valid KV blocks (the residual set of residual linear
// attention: every block that is not critical); no z.  MODE 2: the critical
// lists as they are (the selected set whose states the subtraction form of
// residual linear attention removes from the global state); no z.
template <int D, int MODE>
__global__ void __launch_bounds__(kThreads)
marg_prep_kernel(Geometry g, const int32_t* __restrict__ marg, const float* __restrict__ zs,
                 uint16_t* __restrict__ zhl, uint32_t* __restrict__ bits, int nchunks,
                 int rows_pad) {
  constexpr int RPB = kThreads / D;
  extern __shared__ uint32_t sbits[];        // [RPB][2 * nchunks]
  const int bh = blockIdx.y;
  const int r = threadIdx.x / D, a = threadIdx.x % D;
  const int i0 = blockIdx.x * RPB;
  const int i = i0 + r;
  const int nw = 2 * nchunks;
  for (int e = threadIdx.x; e < RPB * nw; e += kThreads) sbits[e] = 0u;
  __syncthreads();

  constexpr bool COMPL = MODE == 1;
  const int km = MODE == 0 ? g.k_marg : g.k_crit;
  const bool row_ok = i < g.nq;
  const int32_t* __restrict__ mrow = marg + (static_cast<int64_t>(bh) * g.nq + min(i, g.nq - 1)) * km;
  if (row_ok) {
    for (int u = a; u < km; u += D) {
      const int j = list_block(mrow[u], g.nkb);
      atomicOr(&sbits[r * nw + (j >> 5)], 1u << (j & 31));
    }
  }
  if constexpr (MODE == 0) {
    if (i < g.nkb) {
      const float z = zs[(static_cast<int64_t>(bh) * g.nkb + i) * D + a];
      const uint16_t hi = f32_to_bf16_bits(z);
      const uint16_t lo = f32_to_bf16_bits(z - bf16_to_f32(hi));
      uint16_t* zr = zhl + (static_cast<int64_t>(bh) * g.nkb + i) * 2 * D + 64 * (a >> 5) + (a & 31);
      zr[0] = hi;
      zr[32] = lo;
    }
  }
  __syncthreads();

  uint32_t* __restrict__ bout = bits + static_cast<int64_t>(bh) * nchunks * rows_pad * 2;
  for (int e = threadIdx.x; e < RPB * nw; e += kThreads) {
    const int rr = e / nw, w = e % nw;
    uint32_t word = sbits[e];
    if constexpr (COMPL) {
      const int valid = g.nkb - 32 * w;      // KV blocks 32 w .. 32 w + 31 that exist
      word = ~word & (valid >= 32 ? ~0u : (valid <= 0 ? 0u : (1u << valid) - 1u));
    }
    if (i0 + rr < g.nq)
      bout[(static_cast<int64_t>(w >> 1) * rows_pad + i0 + rr) * 2 + (w & 1)] = word;
  }
}

// Physical 16-byte slot of chunk-column c16 in row r of an H chunk (8 slots
// per 128-byte row): flipping bit 2 on rows with bit 1 set makes the
// transposing reads (rows base + 0..3, four slots) hit distinct banks.
__device__ __forceinline__ int hslot(int r, int c16) { return c16 ^ (4 * ((r >> 1) & 1)); }

// One-dimensional grid of row tiles x (RS / 64) column tiles x B*H, the
// row tile fastest in the logical order and each XCD given a contiguous
// range of it, so the row tiles of one column tile share an L2 (each reads
// the same H slabs).  S^T tile: columns e in [64 ct, 64 ct + 64) of the
// value-major states, rows i0 .. i0 + GM - 1 with GM = 128 NT (NT 32-row
// tiles per wave) and i0 = row0 + GM * (row tile).
// RS: elements per row of hs and s_out (d*d, or d*d + d when each row also
// carries a d-vector summed the same way).
// ZC: past the RS / 64 column tiles of the states, 2 D / 64 more tiles
// read the bf16 hi / lo parts of z (zhl, rows of 2 D) and write
// sigma = hi + lo sums as float32 [B,H,nq,D].
// SUB: each output is T[e] - (the product), T[e] = the sum of the kTotParts
// float32 partial totals tot[bh][part][e] (the global state of the head), so
// the row holds the sum over the blocks its bits leave out.
template <int D, int NT, int RS = D * D, bool ZC = false, bool SUB = false>
__global__ void __launch_bounds__(kThreads, 2)
marg_gemm_kernel(Geometry g, const uint32_t* __restrict__ bits, int nchunks, int rows_pad,
                 int row0, int tiles, const uint16_t* __restrict__ hs, uint16_t* __restrict__ s_out,
                 const uint16_t* __restrict__ zhl = nullptr, float* __restrict__ sigma = nullptr,
                 const float* __restrict__ tot = nullptr) {
  constexpr int DD = RS;
  constexpr int kNT = NT;
  constexpr int kGM = 128 * NT;
  constexpr int kBBytes = kGM * 8;          // bit-row chunk bytes
  constexpr int kStageBytes = kHBytes + kBBytes;
  // stages past kStages get one byte (never used)
  constexpr int B3 = kStages > 3 ? kStageBytes : 16, B4 = kStages > 4 ? kStageBytes : 16;
  constexpr int B5 = kStages > 5 ? kStageBytes : 16;
  __shared__ __attribute__((aligned(16))) unsigned char st0[kStageBytes], st1[kStageBytes],
      st2[kStageBytes], st3[B3], st4[B4], st5[B5];
  __shared__ __attribute__((aligned(16))) u32x2 lut[16];

  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int l32 = lane & 31, hh = lane >> 5;
  constexpr int kHCols = RS / kGN;
  constexpr int kCols = kHCols + (ZC ? 2 * D / kGN : 0);
  const int logical = xcd_remap(blockIdx.x, tiles * kCols * g.B * g.H);
  const int rt = logical % tiles;
  const int ct = (logical / tiles) % kCols;
  const int bh = logical / (tiles * kCols);
  const int i0 = row0 + rt * kGM;
  // this workgroup's source rows: the states, or (ZC) the z parts
  const bool zt = ZC && ct >= kHCols;
  const int src_row = zt ? 2 * D : DD;                 // elements per source row
  const int cts = zt ? ct - kHCols : ct;              // column tile within the source row

  if (t < 16) {
    u32x2 e;
    e[0] = ((t & 1) ? 0x3f80u : 0u) | ((t & 2) ? 0x3f800000u : 0u);
    e[1] = ((t & 4) ? 0x3f80u : 0u) | ((t & 8) ? 0x3f800000u : 0u);
    lut[t] = e;
  }

  auto stage_mem = [&](auto sc) -> unsigned char* {
    constexpr int S = decltype(sc)::value;
    if constexpr (S == 0) return st0;
    else if constexpr (S == 1) return st1;
    else if constexpr (S == 2) return st2;
    else if constexpr (S == 3) return st3;
    else if constexpr (S == 4) return st4;
    else return st5;
  };

  // Chunk loads.  H: rows j = 64c + r, bytes 128 ct .. +127 of each block's
  // d*d states; wave w loads rows 16w + 8u + lane/8 (u = 0, 1), lane slot
  // lane%8 holding global 16-byte column (lane%8) ^ swizzle; rows past nkb
  // read as zeros.  Bits: 4 KB, 1 KB per wave.
  const __amdgpu_buffer_rsrc_t hrs =
      zt ? make_rsrc(zhl + static_cast<int64_t>(bh) * g.nkb * 2 * D, static_cast<uint32_t>(g.nkb) * 2 * D * 2)
         : make_rsrc(hs + static_cast<int64_t>(bh) * g.nkb * DD, static_cast<uint32_t>(g.nkb) * DD * 2);
  const __amdgpu_buffer_rsrc_t brs =
      make_rsrc(bits + static_cast<int64_t>(bh) * nchunks * rows_pad * 2,
                static_cast<uint32_t>(nchunks) * rows_pad * 8);
  uint32_t hoff[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int r = 16 * wave + 8 * u + (lane >> 3);
    hoff[u] = static_cast<uint32_t>(r) * src_row * 2 + 128u * cts + 16u * hslot(r, lane & 7);
  }
  const uint32_t boff = static_cast<uint32_t>(i0) * 8 + (kBBytes / 4) * wave + 16u * lane;
  auto issue = [&](int c, unsigned char* sb) {
    const int cc = min(c, nchunks - 1);         // past the end: reload the last chunk (unused)
    const uint32_t hs_off = static_cast<uint32_t>(kGK * cc) * src_row * 2;
#pragma unroll
    for (int u = 0; u < 2; ++u) buffer_load_lds16(hrs, sb + (16 * wave + 8 * u) * 128, hoff[u], hs_off);
    if (kNT == 4 || lane < 16 * kNT)
      buffer_load_lds16(brs, sb + kHBytes + (kBBytes / 4) * wave, boff, static_cast<uint32_t>(cc) * rows_pad * 8);
  };

  // Transposing H^T reads: output lane i of a 16-lane group (G = (lane/16)%2)
  // receives element i%4 of the rows addressed by lanes 4q + i/4; source
  // lane (q, p) = (li/4, li%4) addresses row 16s + 8hh + 4x + q at columns
  // 32mt + 16G + 4p .. +3, so output lane l gets column 32mt + l%32 at the
  // rows j = 16s + 8hh + 4x + q, k-slot 4x + q: the bit order of the mask
  // operand below.
  uint32_t ta[2];
  const uint32_t bofs = static_cast<uint32_t>(kHBytes + (32 * kNT * wave + l32) * 8);
  {
    const int li = lane & 15, q = li >> 2, p = li & 3, G = (lane >> 4) & 1;
    const int r = 8 * hh + q;                       // + 16 s + 4 x (bits 2, 4, 5)
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      const int c16 = 4 * mt + 2 * G + (p >> 1);
      ta[mt] = static_cast<uint32_t>(r * 128 + 16 * hslot(r, c16) + 8 * (p & 1));
    }
  }

  f32x16 acc[2][kNT];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int nt = 0; nt < kNT; ++nt) acc[mt][nt] = zero16();

  // Every wave issues 3 loads per chunk, always (clamped past the end), so
  // "chunk c landed" is vmcnt(3 * (kStages - 2)) at the top of step c.
  auto step = [&](auto sc, int c) {
    constexpr int S = decltype(sc)::value;
    constexpr int SN = (S + kStages - 1) % kStages;
    static_assert(3 * (kStages - 2) < 16, "vmcnt field");
    __builtin_amdgcn_s_waitcnt(0x0F70 | (3 * (kStages - 2)));
    // Barrier without a memory fence: a fence here would also wait for the
    // loads still in flight into the other stages.  Each wave has just
    // waited for its own part of chunk c, so after the barrier the whole
    // chunk is in LDS; the empty asm statements keep the compiler from
    // moving LDS accesses across the barrier.
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    issue(c + kStages - 1, stage_mem(std::integral_constant<int, SN>()));
    if (c >= nchunks) return;
    // This stage's operands in one asm block (it carries no memory operands,
    // so the compiler adds no wait on the loads still filling other stages;
    // the wait for these reads sits inside the block): the 32 mask bits of
    // rows 32 kNT w + 32nt + l32 (with two row tiles the last two reads
    // repeat the first two), and the H^T fragments of both k-steps.
    const uint32_t sb = lds_addr(stage_mem(sc));
    u32x2 wb[4];
    u32x2 tr[16];
    asm volatile(
        "ds_read_b64 %0, %20\n\t"
        "ds_read_b64 %1, %20 offset:256\n\t"
        "ds_read_b64 %2, %20 offset:%23\n\t"
        "ds_read_b64 %3, %20 offset:%24\n\t"
        "ds_read_b64_tr_b16 %4, %21\n\t"
        "ds_read_b64_tr_b16 %5, %21 offset:512\n\t"
        "ds_read_b64_tr_b16 %6, %22\n\t"
        "ds_read_b64_tr_b16 %7, %22 offset:512\n\t"
        "ds_read_b64_tr_b16 %8, %21 offset:2048\n\t"
        "ds_read_b64_tr_b16 %9, %21 offset:2560\n\t"
        "ds_read_b64_tr_b16 %10, %22 offset:2048\n\t"
        "ds_read_b64_tr_b16 %11, %22 offset:2560\n\t"
        "ds_read_b64_tr_b16 %12, %21 offset:4096\n\t"
        "ds_read_b64_tr_b16 %13, %21 offset:4608\n\t"
        "ds_read_b64_tr_b16 %14, %22 offset:4096\n\t"
        "ds_read_b64_tr_b16 %15, %22 offset:4608\n\t"
        "ds_read_b64_tr_b16 %16, %21 offset:6144\n\t"
        "ds_read_b64_tr_b16 %17, %21 offset:6656\n\t"
        "ds_read_b64_tr_b16 %18, %22 offset:6144\n\t"
        "ds_read_b64_tr_b16 %19, %22 offset:6656\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(wb[0]), "=&v"(wb[1]), "=&v"(wb[2]), "=&v"(wb[3]), "=&v"(tr[0]), "=&v"(tr[1]),
          "=&v"(tr[2]), "=&v"(tr[3]), "=&v"(tr[4]), "=&v"(tr[5]), "=&v"(tr[6]), "=&v"(tr[7]),
          "=&v"(tr[8]), "=&v"(tr[9]), "=&v"(tr[10]), "=&v"(tr[11]), "=&v"(tr[12]), "=&v"(tr[13]),
          "=&v"(tr[14]), "=&v"(tr[15])
        : "v"(sb + bofs), "v"(sb + ta[0]), "v"(sb + ta[1]), "i"(256 * (2 % kNT)),
          "i"(256 * (3 % kNT))
        : "memory");
    // mask operand of k-step s for row tile nt: byte 2s + hh of the row's 64
    // chunk bits (word s / 2), one LUT quadruple per nibble
    auto mask_op = [&](int s, int nt) {
      const uint32_t word = wb[nt][s >> 1];
      const uint32_t sh = 16 * (s & 1) + 8 * hh;
      const u32x2 lo = lut[(word >> sh) & 15u];
      const u32x2 hi = lut[(word >> (sh + 4)) & 15u];
      u32x4 w;
      w[0] = lo[0]; w[1] = lo[1]; w[2] = hi[0]; w[3] = hi[1];
      return __builtin_bit_cast(bf16x8, w);
    };
    bf16x8 mb[2][kNT];
#pragma unroll
    for (int nt = 0; nt < kNT; ++nt) mb[0][nt] = mask_op(0, nt);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      if (s + 1 < 4) {
#pragma unroll
        for (int nt = 0; nt < kNT; ++nt) mb[(s + 1) & 1][nt] = mask_op(s + 1, nt);
      }
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        u32x4 w;
        w[0] = tr[4 * s + 2 * mt][0]; w[1] = tr[4 * s + 2 * mt][1];
        w[2] = tr[4 * s + 2 * mt + 1][0]; w[3] = tr[4 * s + 2 * mt + 1][1];
        const bf16x8 ha = __builtin_bit_cast(bf16x8, w);
#pragma unroll
        for (int nt = 0; nt < kNT; ++nt) acc[mt][nt] = mfma32(ha, mb[s & 1][nt], acc[mt][nt]);
      }
    }
  };

  issue(0, st0);
  issue(1, st1);
  if constexpr (kStages > 3) issue(2, st2);
  if constexpr (kStages > 4) issue(3, st3);
  if constexpr (kStages > 5) issue(4, st4);
  for (int c = 0; c < nchunks; c += kStages) {
    step(std::integral_constant<int, 0>(), c);
    step(std::integral_constant<int, 1>(), c + 1);
    step(std::integral_constant<int, 2>(), c + 2);
    if constexpr (kStages > 3) step(std::integral_constant<int, 3>(), c + 3);
    if constexpr (kStages > 4) step(std::integral_constant<int, 4>(), c + 4);
    if constexpr (kStages > 5) step(std::integral_constant<int, 5>(), c + 5);
  }
  wait_vmem();         // the clamped tail loads also write LDS
  __syncthreads();     // every wave is done with the stages

  if (zt) {
    // sigma of features 32 cts + 8(r/4) + 4hh + r%4: hi part (mt = 0) plus
    // lo part (mt = 1), float32, 16 bytes per lane
#pragma unroll
    for (int nt = 0; nt < kNT; ++nt) {
      const int i = i0 + 32 * kNT * wave + 32 * nt + l32;
      if (i >= g.nq) continue;
      float* srow = sigma + (static_cast<int64_t>(bh) * g.nq + i) * D + 32 * cts + 4 * hh;
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        f32x4 w;
#pragma unroll
        for (int x = 0; x < 4; ++x) w[x] = acc[0][nt][4 * r4 + x] + acc[1][nt][4 * r4 + x];
        *reinterpret_cast<f32x4*>(srow + 8 * r4) = w;
      }
    }
    return;
  }
  if constexpr (SUB) {
    // global state entries of this lane's columns e, partial totals summed in
    // a fixed order
    const float* tb = tot + static_cast<int64_t>(bh) * kTotParts * DD;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int e = kGN * ct + 32 * mt + 8 * (r >> 2) + 4 * hh + (r & 3);
        float tv = tb[e];
#pragma unroll
        for (int pp = 1; pp < kTotParts; ++pp) tv += tb[pp * DD + e];
#pragma unroll
        for (int nt = 0; nt < kNT; ++nt) acc[mt][nt][r] = tv - acc[mt][nt][r];
      }
  }
  // Output: acc[mt][nt][r] = S^T[e = 64 ct + 32 mt + 8(r/4) + 4hh + r%4]
  //                              [i = i0 + 128w + 32nt + l32].
  // Each wave stages 32 rows x 128 bytes at a time in its own 4 KB of the
  // first two stage arrays (16-byte chunks XOR-swizzled by row) and writes
  // whole 128-byte rows.
  unsigned char* ob = wave < 2 ? st0 + 4096 * wave : st1 + 4096 * (wave - 2);
#pragma unroll
  for (int nt = 0; nt < kNT; ++nt) {
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int c = 4 * mt + r4;                         // 16-byte chunk of the row
        u32x2 w;
        w[0] = static_cast<uint32_t>(f32_to_bf16_bits(acc[mt][nt][4 * r4])) |
               (static_cast<uint32_t>(f32_to_bf16_bits(acc[mt][nt][4 * r4 + 1])) << 16);
        w[1] = static_cast<uint32_t>(f32_to_bf16_bits(acc[mt][nt][4 * r4 + 2])) |
               (static_cast<uint32_t>(f32_to_bf16_bits(acc[mt][nt][4 * r4 + 3])) << 16);
        *reinterpret_cast<u32x2*>(ob + l32 * 128 + 16 * (c ^ ((l32 >> 1) & 7)) + 8 * hh) = w;
      }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int qc = 64 * k + lane;
      const int row = qc >> 3, c = qc & 7;
      const int i = i0 + 32 * kNT * wave + 32 * nt + row;
      const u32x4 v = *reinterpret_cast<const u32x4*>(ob + row * 128 + 16 * (c ^ ((row >> 1) & 7)));
      if (i < g.nq)
        *reinterpret_cast<u32x4*>(s_out + (static_cast<int64_t>(bh) * g.nq + i) * DD + kGN * ct + 8 * c) = v;
    }
  }
}

// The global state of each head (the sum of every block's state) as
// kTotParts float32 partial sums over consecutive KV block ranges: grid
// (RS / 2048, kTotParts, B*H), thread t of column slice cs sums elements
// 2048 cs + 8 t .. +7 over its part's blocks, four rows in flight at a time,
// in ascending block order.
template <int RS>
__global__ void __launch_bounds__(kThreads)
state_total_kernel(Geometry g, const uint16_t* __restrict__ hs, float* __restrict__ tot) {
  const int cs = blockIdx.x, part = blockIdx.y, bh = blockIdx.z;
  const int per = (g.nkb + kTotParts - 1) / kTotParts;
  const int j0 = min(part * per, g.nkb), j1 = min(j0 + per, g.nkb);
  const int e0 = 2048 * cs + 8 * threadIdx.x;
  const uint16_t* src = hs + static_cast<int64_t>(bh) * g.nkb * RS + e0;
  float a[8];
#pragma unroll
  for (int x = 0; x < 8; ++x) a[x] = 0.0f;
  int j = j0;
  for (; j + 4 <= j1; j += 4) {
    float f[4][8];
#pragma unroll
    for (int u = 0; u < 4; ++u) load8_f32(src + static_cast<int64_t>(j + u) * RS, f[u]);
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int x = 0; x < 8; ++x) a[x] += f[u][x];
  }
  for (; j < j1; ++j) {
    float f[8];
    load8_f32(src + static_cast<int64_t>(j) * RS, f);
#pragma unroll
    for (int x = 0; x < 8; ++x) a[x] += f[x];
  }
  float* dst = tot + (static_cast<int64_t>(bh) * kTotParts + part) * RS + e0;
  *reinterpret_cast<f32x4*>(dst) = f32x4{a[0], a[1], a[2], a[3]};
  *reinterpret_cast<f32x4*>(dst + 4) = f32x4{a[4], a[5], a[6], a[7]};
}

}  // namespace

hipError_t launch_marginal_sums(const Geometry& g, const int32_t* marg, const uint16_t* h_states,
                                const float* z_states, uint16_t* s_sum, float* sigma_sum,
                                uint32_t* bits, uint16_t* zhl, bool complement, hipStream_t stream) {
  const int nchunks = marginal_chunks(g);
  const int rows_pad = marginal_rows_pad(g);
  const int rpb = kThreads / g.D;
  dim3 gs((g.nq + rpb - 1) / rpb, g.B * g.H);
  const size_t lds1 = static_cast<size_t>(rpb) * 2 * nchunks * sizeof(uint32_t);
  auto prep = [&](auto dc, auto mc) {
    constexpr int DK = decltype(dc)::value;
    constexpr int MK = decltype(mc)::value;
    hipLaunchKernelGGL((marg_prep_kernel<DK, MK>), gs, dim3(kThreads), lds1, stream, g, marg,
                       z_states, zhl, bits, nchunks, rows_pad);
  };
  if (g.D == 128) {
    if (complement) prep(std::integral_constant<int, 128>(), std::integral_constant<int, 1>());
    else prep(std::integral_constant<int, 128>(), std::integral_constant<int, 0>());
  } else {
    if (complement) prep(std::integral_constant<int, 64>(), std::integral_constant<int, 1>());
    else prep(std::integral_constant<int, 64>(), std::integral_constant<int, 0>());
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_mask_gemm(g, bits, h_states, s_sum, stream, false, complement ? nullptr : zhl,
                          sigma_sum);
}

hipError_t launch_mask_gemm(const Geometry& g, const uint32_t* bits, const uint16_t* h_states,
                            uint16_t* s_sum, hipStream_t stream, bool with_vector,
                            const uint16_t* zhl, float* sigma, const float* tot) {
  const int nchunks = marginal_chunks(g);
  const int rows_pad = marginal_rows_pad(g);
  // One launch covers every row of the heads, so the row tiles of one
  // column tile (neighbours in the XCD-ordered grid) share the H slabs in
  // L2: a single 512-row tile up to nq = 512 (a 256-row one up to 256), and
  // 256-row tiles beyond (at nq = 1182: five tiles, 1280 rows of work, 5%
  // faster than two 512-row tiles and a separate 256-row launch).
  auto gemm = [&](auto dc, auto ntc, int tiles, int row0) {
    constexpr int DK = decltype(dc)::value, NTK = decltype(ntc)::value;
    if (with_vector) {
      dim3 g2(tiles * ((DK * DK + DK) / kGN) * g.B * g.H);
      hipLaunchKernelGGL((marg_gemm_kernel<DK, NTK, DK * DK + DK>), g2, dim3(kThreads), 0, stream,
                         g, bits, nchunks, rows_pad, row0, tiles, h_states, s_sum);
    } else if (tot) {
      dim3 g2(tiles * (DK * DK / kGN) * g.B * g.H);
      hipLaunchKernelGGL((marg_gemm_kernel<DK, NTK, DK * DK, false, true>), g2, dim3(kThreads), 0,
                         stream, g, bits, nchunks, rows_pad, row0, tiles, h_states, s_sum, nullptr,
                         nullptr, tot);
    } else if (zhl) {
      dim3 g2(tiles * ((DK * DK + 2 * DK) / kGN) * g.B * g.H);
      hipLaunchKernelGGL((marg_gemm_kernel<DK, NTK, DK * DK, true>), g2, dim3(kThreads), 0, stream,
                         g, bits, nchunks, rows_pad, row0, tiles, h_states, s_sum, zhl, sigma);
    } else {
      dim3 g2(tiles * (DK * DK / kGN) * g.B * g.H);
      hipLaunchKernelGGL((marg_gemm_kernel<DK, NTK>), g2, dim3(kThreads), 0, stream, g, bits,
                         nchunks, rows_pad, row0, tiles, h_states, s_sum);
    }
  };
  const bool one512 = g.nq > 256 && g.nq <= 512;
  const int n256 = (g.nq + 255) / 256;
  if (g.D == 128) {
    if (one512) gemm(std::integral_constant<int, 128>(), std::integral_constant<int, 4>(), 1, 0);
    else gemm(std::integral_constant<int, 128>(), std::integral_constant<int, 2>(), n256, 0);
  } else {
    if (one512) gemm(std::integral_constant<int, 64>(), std::integral_constant<int, 4>(), 1, 0);
    else gemm(std::integral_constant<int, 64>(), std::integral_constant<int, 2>(), n256, 0);
  }
  return hipGetLastError();
}

}  // namespace sla

namespace sla {

hipError_t launch_residual_subtract(const Geometry& g, const int32_t* crit, const uint16_t* h_states,
                                    uint16_t* s_sum, uint32_t* bits, float* tot,
                                    hipStream_t stream) {
  const int nchunks = marginal_chunks(g);
  const int rows_pad = marginal_rows_pad(g);
  const int rpb = kThreads / g.D;
  dim3 gs((g.nq + rpb - 1) / rpb, g.B * g.H);
  const size_t lds1 = static_cast<size_t>(rpb) * 2 * nchunks * sizeof(uint32_t);
  const int rs = g.D * g.D;
  if (g.D == 128) {
    hipLaunchKernelGGL((marg_prep_kernel<128, 2>), gs, dim3(kThreads), lds1, stream, g, crit,
                       nullptr, nullptr, bits, nchunks, rows_pad);
    hipLaunchKernelGGL((state_total_kernel<128 * 128>), dim3(rs / 2048, kTotParts, g.B * g.H),
                       dim3(kThreads), 0, stream, g, h_states, tot);
  } else {
    hipLaunchKernelGGL((marg_prep_kernel<64, 2>), gs, dim3(kThreads), lds1, stream, g, crit,
                       nullptr, nullptr, bits, nchunks, rows_pad);
    hipLaunchKernelGGL((state_total_kernel<64 * 64>), dim3(rs / 2048, kTotParts, g.B * g.H),
                       dim3(kThreads), 0, stream, g, h_states, tot);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_mask_gemm(g, bits, h_states, s_sum, stream, false, nullptr, nullptr, tot);
}

size_t residual_total_bytes(const Geometry& g) {
  return static_cast<size_t>(g.B) * g.H * kTotParts * g.D * g.D * sizeof(float);
}

}  // namespace sla
