// Fused sparse + linear attention forward (bf16 matrix cores).
//
// [SLA abstract] exact O(N^2) attention on the critical KV blocks, O(N)
// linear attention on the marginal blocks, negligible blocks skipped, all in
// one kernel; [SLA2 technical summary, section 1 item 1] the sparse softmax
// is renormalised over the kept keys; [SLA2 summary, section 2.A equation]
// O = alpha O_s + (1 - alpha) O_l with alpha per head.
//
// One workgroup per (b, h, query block i), 4 waves: wave = qh + 2*kh, where
// qh picks 32 of the 64 query rows and kh picks 32 of the 64 keys of every
// gathered KV block.  Per critical block (one loop iteration):
//   * the block's K and V tiles [64 keys][d] sit in LDS, row-major with a
//     16-byte-chunk XOR swizzle; two K and two V buffers form a ring that the
//     direct global->LDS loads for the next blocks fill while this one
//     computes;
//   * each wave computes S^T = K Q^T for its 32 keys x 32 queries on
//     v_mfma_f32_32x32x16_bf16, runs the online-softmax update on the S^T
//     registers (query = lane % 32, so a row max is a reduction over the
//     lane's own registers plus the partner lane l ^ 32), and accumulates
//     O^T += V^T P^T with P^T taken straight from the S^T registers and the
//     V^T operand read from the row-major V tile by transposing LDS reads
//     (ds_read_b64_tr_b16).
// The two key halves keep separate running max / sum / output (no per-block
// cross-wave reduction); the shared epilogue merges them, adds the linear
// branch from the precomputed marginal-state sums and stores the alpha mix.
#include "attention_epilogue.hpp"

namespace sla {
namespace {

struct AttnArgs {
  const void* q;
  const void* k;
  const void* v;
  const int32_t* crit;
  const uint16_t* s_sum;
  const float* sigma_sum;
  const float* alpha;
  void* o;
  float* o_sparse;
  float* o_linear;
  Geometry g;
  float c_log2;      // log2(e) / sqrt(d)
};

// XOR swizzle of the 16-byte chunks of a tile row: both the K-row operand
// reads (16 consecutive rows, one chunk) and the transposing V reads (4
// consecutive keys x 4 chunks) hit distinct LDS banks.
template <int D>
__device__ __forceinline__ int swz(int r) {
  if constexpr (D == 128) return 4 * (r & 3) + ((r >> 2) & 3);
  else return (r >> 1) & 7;
}

template <typename T, int D>
__global__ void __launch_bounds__(kThreads, 2)
attention_kernel(AttnArgs A) {
  constexpr int CH = D / 8;                    // 16-byte chunks per row
  constexpr int TILE = kBlock * D;             // elements per K or V tile
  constexpr int NSTAGE = 4;                    // two K buffers, two V buffers
  constexpr int RPI = 64 / CH;                 // rows per 64-lane load instruction
  constexpr int IPW = (kBlock / 4) / RPI;      // load instructions per wave per tile
  constexpr int NS = D / 16;                   // 16-wide k-steps over the features
  constexpr int DT = D / 32;                   // 32-row tiles over the value dims
  constexpr int LOOP_BYTES = NSTAGE * TILE * 2;
  constexpr int EPI_BYTES = epilogue_smem_bytes<D>();
  constexpr int SMEM_BYTES = (LOOP_BYTES > EPI_BYTES ? LOOP_BYTES : EPI_BYTES);
  __shared__ __attribute__((aligned(16))) unsigned char smem_raw[SMEM_BYTES];
  uint16_t* smem = reinterpret_cast<uint16_t*>(smem_raw);

  const Geometry& g = A.g;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int qh = wave & 1, kh = wave >> 1;
  const int l32 = lane & 31, hh = lane >> 5;

  const int total = g.B * g.H * g.nq;
  const int logical = xcd_remap(blockIdx.x, total);
  const int i = logical % g.nq;
  const int bh = logical / g.nq;
  const int b = bh / g.H, h = bh % g.H;
  const int64_t hoff = b * g.sb + h * g.sh;
  const T* __restrict__ qp = static_cast<const T*>(A.q) + hoff;
  const T* __restrict__ kp = static_cast<const T*>(A.k) + hoff;
  const T* __restrict__ vp = static_cast<const T*>(A.v) + hoff;
  const int n_i = min(kBlock, g.N - kBlock * i);
  const float cl = A.c_log2;
  constexpr float kLazy = 8.0f;
  const int64_t sn = g.sn;

  // Q fragments (B operand of S^T = K Q^T): query 32*qh + l32, features
  // 16*s + 8*hh .. +7.  Rows past the last query are clamped (not stored).
  bf16x8 qf[NS];
  const int qrow = 32 * qh + l32;
  {
    const int qr = qrow < n_i ? qrow : n_i - 1;
#pragma unroll
    for (int s = 0; s < NS; ++s)
      qf[s] = load8(qp + static_cast<int64_t>(kBlock * i + qr) * sn + 16 * s + 8 * hh);
  }

  const int32_t* __restrict__ crow = A.crit + (static_cast<int64_t>(bh) * g.nq + i) * g.k_crit;
  const int kc = g.k_crit;
  // The critical list is read once into registers, 64 entries per register
  // (lane l holds entry base + l), and entries are taken with v_readlane, so
  // the loop issues no index loads: a vector load there would make the
  // compiler's vmcnt wait cover the in-flight K/V tile loads as well.
  int cl0 = lane < kc ? crow[lane] : 0;
  int cl1 = 64 + lane < kc ? crow[64 + lane] : 0;
  int cbase = 0;
  auto crit_at = [&](int c) -> int {
    const int o = c - cbase;
    return o < 64 ? __builtin_amdgcn_readlane(cl0, o) : __builtin_amdgcn_readlane(cl1, o - 64);
  };

  // LDS ring: K buffers kbuf[2] and V buffers vbuf[2] (16 KB each at d=128).
  // Iteration it reads K of block it+1 (for the next S) and V of block it;
  // right after its barrier it issues K of block it+2 and V of block it+1
  // straight into LDS (no staging registers), which land while it computes.
  //
  // Wave w fills rows 16w .. 16w+15 of a tile; lane l of instruction u writes
  // row 16w + RPI*u + l/CH at chunk slot l%CH, which holds global chunk
  // (l%CH) ^ swz(row).  Rows past the end of a short last block repeat its
  // last row (those keys are masked to -inf in S).
  const int lrow = lane / CH, lslot = lane % CH;
  uint16_t* kbuf0 = smem;
  uint16_t* vbuf0 = smem + 2 * TILE;
  const uint32_t rowb = static_cast<uint32_t>(sn * sizeof(T));
  uint32_t toff[IPW], tcol[IPW];
#pragma unroll
  for (int u = 0; u < IPW; ++u) {
    const int r = 16 * wave + RPI * u + lrow;
    tcol[u] = static_cast<uint32_t>(8 * (lslot ^ swz<D>(r)) * sizeof(T));
    toff[u] = static_cast<uint32_t>(r) * rowb + tcol[u];
  }
  auto issue_tile = [&](const T* base, int c, uint16_t* dst) {
    const int jb = crit_at(c);
    const int nj = min(kBlock, g.N - kBlock * jb);
    const T* tb = base + static_cast<int64_t>(kBlock * jb) * sn;
#pragma unroll
    for (int u = 0; u < IPW; ++u) {
      const int r0 = 16 * wave + RPI * u;
      uint32_t off = toff[u];
      if (nj < kBlock) {
        const int r = r0 + lrow;
        off = static_cast<uint32_t>(r < nj ? r : nj - 1) * rowb + tcol[u];
      }
      const T* src = reinterpret_cast<const T*>(reinterpret_cast<const char*>(tb) + off);
      if constexpr (sizeof(T) == 2) {
        load_lds16(src, dst + r0 * D);
      } else {
        *reinterpret_cast<bf16x8*>(dst + r0 * D + 8 * lane) = load8(src);
      }
    }
  };

  // S^T of keys 32*kh .. +31 (of the block in kt) and queries 32*qh .. +31
  const int krow = 32 * kh + l32;
  const int ksw = swz<D>(krow);
  auto qk = [&](const uint16_t* kt) {
    bf16x8 kf[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s)
      kf[s] = *reinterpret_cast<const bf16x8*>(&kt[krow * D + 8 * ((2 * s + hh) ^ ksw)]);
    f32x16 acc = zero16();
#pragma unroll
    for (int s = 0; s < NS; ++s) acc = mfma32(kf[s], qf[s], acc);
    return acc;
  };

  // transposing V reads: source role of this lane within its 16-lane group
  const int g16 = lane >> 4, li = lane & 15;
  const int ep = li >> 2, q4 = li & 3, gm = g16 & 1;
  const int key1 = 32 * kh + 4 * hh + ep;                 // + 16 s, and + 8 for the second read
  const int sw1 = swz<D>(key1), sw2 = swz<D>(key1 + 8);   // independent of s (16 s keeps bits 0..3)
  // byte offsets inside a V tile of the (s = 0) transposing reads for each
  // 32-dim tile; s = 1 adds 16 rows
  uint32_t vofs1[DT], vofs2[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
    const int c = 4 * dt + 2 * gm + (q4 >> 1);
    vofs1[dt] = static_cast<uint32_t>((key1 * D + 8 * (c ^ sw1) + 4 * (q4 & 1)) * 2);
    vofs2[dt] = static_cast<uint32_t>(((key1 + 8) * D + 8 * (c ^ sw2) + 4 * (q4 & 1)) * 2);
  }

  float m_run = -INFINITY, l_run = 0.0f;
  f32x16 oacc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) oacc[dt] = zero16();

  f32x16 s_cur = zero16();
  if (kc > 0) {
    issue_tile(kp, 0, kbuf0);
    issue_tile(vp, 0, vbuf0);
    if (kc > 1) issue_tile(kp, 1, kbuf0 + TILE);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    s_cur = qk(kbuf0);
  }
  for (int it = 0; it < kc; ++it) {
    const int cur = it & 1;
    // K(it+2) -> kbuf[cur] (K(it) was read last iteration); V(it+1) -> vbuf[cur^1]
    if (it + 2 < kc) issue_tile(kp, it + 2, kbuf0 + cur * TILE);
    if (it + 1 < kc) issue_tile(vp, it + 1, vbuf0 + (cur ^ 1) * TILE);
    // next S on the matrix cores while this block's softmax runs on the VALU
    f32x16 s_next = zero16();
    if (it + 1 < kc) s_next = qk(kbuf0 + (cur ^ 1) * TILE);

    const int jb = crit_at(it);
    const int nj = min(kBlock, g.N - kBlock * jb);
    if (nj < kBlock) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = 32 * kh + 8 * (r >> 2) + 4 * hh + (r & 3);
        if (key >= nj) s_cur[r] = -INFINITY;
      }
    }
    float mx = s_cur[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s_cur[r]);
    mx = fmaxf(mx, xor_lane(mx, 32));
    // The running reference max m_run only moves when some query's tile max
    // exceeds it by more than kLazy (in log2 units), so p <= 2^kLazy and the
    // output / sum rescale is skipped on most blocks; O and l always share
    // the same reference, so the final O / l is unchanged.
    const bool grow = __ballot((mx - m_run) * cl > kLazy) != 0ull;
    if (grow) {
      const float m_new = fmaxf(m_run, mx);
      const float corr = __builtin_amdgcn_exp2f((m_run - m_new) * cl);
      l_run *= corr;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[dt][r] *= corr;
      m_run = m_new;
    }
    const float mb = (m_run == -INFINITY ? 0.0f : m_run) * cl;
    float ps = 0.0f;
    bf16x8 pb[2];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float p = __builtin_amdgcn_exp2f(fmaf(s_cur[r], cl, -mb));
      ps += p;
      pb[r >> 3][r & 7] = f32_to_bf16(p);
    }
    l_run += ps;

    // O^T += V^T P^T; the V^T operand comes from the row-major V tile through
    // transposing reads: lane l gets dim 32*dt + l%32 at keys
    // 32*kh + 16*s + 8*(e/4) + 4*hh + e%4, matching P^T's k-slots.
    // LDS byte address of this lane's first transposing read in the V tile
    const uint32_t vt_addr = lds_addr(vbuf0 + cur * TILE);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      u32x2 a0, a1, b0, b1;
      // the 4 reads of one 32-dim tile and their wait sit in one asm block
      asm volatile(
          "ds_read_b64_tr_b16 %0, %4\n\t"
          "ds_read_b64_tr_b16 %1, %5\n\t"
          "ds_read_b64_tr_b16 %2, %4 offset:%6\n\t"
          "ds_read_b64_tr_b16 %3, %5 offset:%6\n\t"
          "s_waitcnt lgkmcnt(0)"
          : "=&v"(a0), "=&v"(a1), "=&v"(b0), "=&v"(b1)
          : "v"(vt_addr + vofs1[dt]), "v"(vt_addr + vofs2[dt]), "i"(16 * D * 2)
          : "memory");
      u32x4 w0, w1;
      w0[0] = a0[0]; w0[1] = a0[1]; w0[2] = a1[0]; w0[3] = a1[1];
      w1[0] = b0[0]; w1[1] = b0[1]; w1[2] = b1[0]; w1[3] = b1[1];
      oacc[dt] = mfma32(__builtin_bit_cast(bf16x8, w0), pb[0], oacc[dt]);
      oacc[dt] = mfma32(__builtin_bit_cast(bf16x8, w1), pb[1], oacc[dt]);
    }
    s_cur = s_next;
    if (it + 1 - cbase == 64) {            // entries it+1 .. it+64 now start at register 1
      cbase += 64;
      cl0 = cl1;
      cl1 = cbase + 64 + lane < kc ? crow[cbase + 64 + lane] : 0;
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // this wave's loads for the next step
    __syncthreads();
  }
  __syncthreads();

  attention_finish<T, D>(smem_raw, g, bh, h, i, n_i, qrow, hoff, A.s_sum, A.sigma_sum, A.alpha, A.o,
                         A.o_sparse, A.o_linear, oacc, m_run, l_run, cl, qf);
}

template <typename T, int D>
void launch_attn_t(const AttnArgs& a, hipStream_t stream) {
  const int total = a.g.B * a.g.H * a.g.nq;
  hipLaunchKernelGGL((attention_kernel<T, D>), dim3(total), dim3(kThreads), 0, stream, a);
}

}  // namespace

hipError_t launch_attention(const Geometry& g, const void* q, const void* k, const void* v,
                            const int32_t* crit, const uint16_t* s_sum, const float* sigma_sum,
                            const float* alpha, void* o, float* o_sparse, float* o_linear,
                            hipStream_t stream) {
  AttnArgs a{q, k, v, crit, s_sum, sigma_sum, alpha, o, o_sparse, o_linear, g,
             static_cast<float>(1.4426950408889634 / __builtin_sqrt(static_cast<double>(g.D)))};
  if (g.dtype == 1) {
    if (g.D == 128) launch_attn_t<uint16_t, 128>(a, stream);
    else launch_attn_t<uint16_t, 64>(a, stream);
  } else {
    if (g.D == 128) launch_attn_t<float, 128>(a, stream);
    else launch_attn_t<float, 64>(a, stream);
  }
  return hipGetLastError();
}

}  // namespace sla
