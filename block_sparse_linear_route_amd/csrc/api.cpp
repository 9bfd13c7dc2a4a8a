// C ABI of libsla: argument validation, workspace sizing, device checks and
// kernel dispatch.  Declarations and the contract live in include/sla.h.
#include "sla.h"

#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>

#include "sla_internal.hpp"

namespace {

thread_local std::string g_last_error;

int fail(int status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return status;
}

using sla::kMaxKvBlocks;
constexpr size_t kWsAlign = 256;

size_t align_up(size_t x) { return (x + kWsAlign - 1) / kWsAlign * kWsAlign; }

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int validate_problem(const sla_problem* p) {
  if (!p) return fail(SLA_ERR_INVALID_ARGUMENT, "problem is NULL");
  if (p->batch < 1 || p->heads < 1 || p->seq_len < 1)
    return fail(SLA_ERR_INVALID_ARGUMENT, "batch, heads and seq_len must be >= 1 (got %d, %d, %d)",
                p->batch, p->heads, p->seq_len);
  if (p->head_dim != 64 && p->head_dim != 128)
    return fail(SLA_ERR_UNSUPPORTED, "head_dim %d unsupported (64 or 128)", p->head_dim);
  if (p->block != 64) return fail(SLA_ERR_UNSUPPORTED, "block %d unsupported (64)", p->block);
  if (p->dtype != SLA_F32 && p->dtype != SLA_BF16)
    return fail(SLA_ERR_UNSUPPORTED, "dtype %d unsupported", p->dtype);
  const int64_t nkb = (static_cast<int64_t>(p->seq_len) + 63) / 64;
  if (nkb > kMaxKvBlocks)
    return fail(SLA_ERR_UNSUPPORTED, "%lld KV blocks exceed the supported %d",
                static_cast<long long>(nkb), kMaxKvBlocks);
  if (p->k_crit < 0 || p->k_marg < 0)
    return fail(SLA_ERR_INVALID_ARGUMENT, "k_crit and k_marg must be >= 0");
  const int64_t sum = static_cast<int64_t>(p->k_crit) + p->k_marg;
  if (sum < 1 || sum > nkb)
    return fail(SLA_ERR_INVALID_ARGUMENT, "need 1 <= k_crit + k_marg <= nkb (%lld), got %lld",
                static_cast<long long>(nkb), static_cast<long long>(sum));
  if (p->stride_b < 0 || p->stride_h < 0 || p->stride_n < p->head_dim)
    return fail(SLA_ERR_INVALID_ARGUMENT, "strides must be >= 0 and stride_n >= head_dim");
  const int64_t esz = p->dtype == SLA_BF16 ? 2 : 4;
  if ((p->stride_n * esz) % 16 || (p->stride_h * esz) % 16 || (p->stride_b * esz) % 16)
    return fail(SLA_ERR_INVALID_ARGUMENT, "strides must be multiples of 16 bytes");
  // The tile loads address a head's rows through buffer resources with
  // 32-bit byte offsets and sizes: one head's span must fit in them.
  const int64_t head_span = (static_cast<int64_t>(p->seq_len) - 1) * p->stride_n * esz + p->head_dim * esz;
  if (head_span > static_cast<int64_t>(UINT32_MAX))
    return fail(SLA_ERR_UNSUPPORTED, "one head spans %lld bytes (seq_len x stride_n); at most 4 GiB is supported",
                static_cast<long long>(head_span));
  const int64_t nq_total = static_cast<int64_t>(p->batch) * p->heads * nkb;
  if (2 * nq_total > (1ll << 31) - 1)
    return fail(SLA_ERR_UNSUPPORTED, "2 * batch * heads * blocks exceeds the grid limit");
  return SLA_OK;
}

sla::Geometry geometry(const sla_problem* p) {
  sla::Geometry g;
  g.B = p->batch;
  g.H = p->heads;
  g.N = p->seq_len;
  g.D = p->head_dim;
  g.nq = g.nkb = (p->seq_len + 63) / 64;
  g.k_crit = p->k_crit;
  g.k_marg = p->k_marg;
  g.dtype = p->dtype;
  g.sb = p->stride_b;
  g.sh = p->stride_h;
  g.sn = p->stride_n;
  return g;
}

// -1 unknown, 0 not gfx950, 1 gfx950; indexed by device id.
std::atomic<int> g_dev_ok[64];
std::atomic<bool> g_dev_init{false};

int check_device() {
  if (!g_dev_init.load(std::memory_order_acquire)) {
    for (auto& x : g_dev_ok) x.store(-1, std::memory_order_relaxed);
    g_dev_init.store(true, std::memory_order_release);
  }
  int count = 0;
  if (hipGetDeviceCount(&count) != hipSuccess || count < 1) {
    (void)hipGetLastError();
    return fail(SLA_ERR_NO_DEVICE, "no HIP device available");
  }
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    return fail(SLA_ERR_NO_DEVICE, "hipGetDevice failed");
  }
  if (dev < 0 || dev >= 64) return fail(SLA_ERR_NO_DEVICE, "device id %d out of range", dev);
  int ok = g_dev_ok[dev].load(std::memory_order_relaxed);
  if (ok < 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
      (void)hipGetLastError();
      return fail(SLA_ERR_NO_DEVICE, "hipGetDeviceProperties failed");
    }
    ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 0;
    g_dev_ok[dev].store(ok, std::memory_order_relaxed);
  }
  if (!ok) return fail(SLA_ERR_NO_DEVICE, "device %d is not gfx950", dev);
  return SLA_OK;
}

int launched(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(SLA_ERR_DEVICE, "%s: %s", what, hipGetErrorString(e));
  return SLA_OK;
}

#define SLA_TRY(x)                 \
  do {                             \
    const int _st = (x);           \
    if (_st != SLA_OK) return _st; \
  } while (0)

#define SLA_REQ(ptr, align)                                                              \
  do {                                                                                   \
    if (!(ptr)) return fail(SLA_ERR_INVALID_ARGUMENT, "%s is NULL", #ptr);               \
    if (!aligned((ptr), (align)))                                                        \
      return fail(SLA_ERR_INVALID_ARGUMENT, "%s is not %d-byte aligned", #ptr, (align)); \
  } while (0)

#define SLA_OPT(ptr, align)                                                              \
  do {                                                                                   \
    if ((ptr) && !aligned((ptr), (align)))                                               \
      return fail(SLA_ERR_INVALID_ARGUMENT, "%s is not %d-byte aligned", #ptr, (align)); \
  } while (0)

// Forward workspace: [S bf16 B*H*nq*d*d][sigma f32 B*H*nq*d]
// [mask bits u32 B*H*ceil(nkb/64)*ceil(nq/512)*512*2][z parts bf16 B*H*nkb*2d]
struct FwdWs {
  uint16_t* s_sum;
  float* sigma;
  uint32_t* bits;
  uint16_t* zhl;
};

size_t forward_ws(const sla::Geometry& g) {
  const size_t rows = static_cast<size_t>(g.B) * g.H * g.nq;
  const size_t bit_words = static_cast<size_t>(g.B) * g.H * sla::marginal_chunks(g) *
                           sla::marginal_rows_pad(g) * 2;
  return align_up(rows * g.D * g.D * 2) + align_up(rows * g.D * 4) + align_up(bit_words * 4) +
         align_up(static_cast<size_t>(g.B) * g.H * g.nkb * 2 * g.D * 2);
}

FwdWs carve_forward_ws(const sla::Geometry& g, void* ws) {
  const size_t rows = static_cast<size_t>(g.B) * g.H * g.nq;
  char* p = static_cast<char*>(ws);
  FwdWs w;
  w.s_sum = reinterpret_cast<uint16_t*>(p);
  p += align_up(rows * g.D * g.D * 2);
  w.sigma = reinterpret_cast<float*>(p);
  p += align_up(rows * g.D * 4);
  w.bits = reinterpret_cast<uint32_t*>(p);
  const size_t bit_words = static_cast<size_t>(g.B) * g.H * sla::marginal_chunks(g) *
                           sla::marginal_rows_pad(g) * 2;
  p += align_up(bit_words * 4);
  w.zhl = reinterpret_cast<uint16_t*>(p);
  return w;
}

// Route workspace: [pooled Q f64 B*H*nq*d][pooled K f64 B*H*nkb*d]
// [selection keys u64, route_key_bytes] and, for the second-order score,
// [key variances f64 B*H*nkb*d] (the allocation-free route keeps pooled K
// transposed, B*H*d*nkb, in its static scratch).
size_t route_region(const sla::Geometry& g) {
  return align_up(static_cast<size_t>(g.B) * g.H * g.nq * g.D * 8);
}
size_t route_ws(const sla::Geometry& g) {
  return 2 * route_region(g) + align_up(sla::route_key_bytes(g));
}
size_t route_taylor_ws(const sla::Geometry& g) { return route_ws(g) + route_region(g); }
uint64_t* route_keys(const sla::Geometry& g, void* ws) {
  return reinterpret_cast<uint64_t*>(static_cast<char*>(ws) + 2 * route_region(g));
}

// PISA workspace: [kbar bf16 B*H*npb*64*d][vbar bf16 B*H*npb*64*d]
// [Hbar bf16 B*H*d*d][chunk partials f32 B*H*nchunks*d*d]
struct PisaWs {
  uint16_t* kbar;
  uint16_t* vbar;
  uint16_t* hbar;
  float* part;
};

size_t pisa_ws(const sla::Geometry& g) {
  const size_t bh = static_cast<size_t>(g.B) * g.H;
  const size_t rows = bh * sla::pisa_pseudo_blocks(g) * 64;
  return 2 * align_up(rows * g.D * 2) + align_up(bh * g.D * g.D * 2) +
         align_up(bh * sla::pisa_chunks(g) * g.D * g.D * 4);
}

PisaWs carve_pisa_ws(const sla::Geometry& g, void* ws) {
  const size_t bh = static_cast<size_t>(g.B) * g.H;
  const size_t rows = bh * sla::pisa_pseudo_blocks(g) * 64;
  char* p = static_cast<char*>(ws);
  PisaWs w;
  w.kbar = reinterpret_cast<uint16_t*>(p);
  p += align_up(rows * g.D * 2);
  w.vbar = reinterpret_cast<uint16_t*>(p);
  p += align_up(rows * g.D * 2);
  w.hbar = reinterpret_cast<uint16_t*>(p);
  p += align_up(bh * g.D * g.D * 2);
  w.part = reinterpret_cast<float*>(p);
  return w;
}

// Covariance-aware routing workspace: [PISA workspace, so that the
// statistics serve sla_forward_attend_pisa][route regions][Hbar f32
// B*H*d*d][M_j f64 B*H*nkb]
size_t route_pisa_ws(const sla::Geometry& g) {
  const size_t bh = static_cast<size_t>(g.B) * g.H;
  return pisa_ws(g) + route_ws(g) + align_up(bh * g.D * g.D * 4) + align_up(bh * g.nkb * 8);
}

// Backward workspace: [forward workspace][O scratch, problem layout]
// [O_s f32][O_l f32][lse f32 B*H*N][D_t f32 B*H*N]
// [dS|dsigma bf16 B*H*nq*(d*d + d)][dH|dz bf16 B*H*nkb*(d*d + d)]
// [critical bits^T][marginal bits^T][dalpha partials f32 B*H*nq], each
// region 256-byte aligned
struct BwdWs {
  FwdWs fwd;
  void* o;
  sla::BackwardBuffers b;
};

size_t span_elems(const sla::Geometry& g) {
  return static_cast<size_t>((g.B - 1) * g.sb + (g.H - 1) * g.sh + (g.N - 1) * g.sn + g.D);
}

size_t backward_ws(const sla::Geometry& g) {
  const size_t bh = static_cast<size_t>(g.B) * g.H;
  const size_t rows = bh * g.N;
  const size_t blk = bh * g.nq;
  const size_t nmt = bh * sla::marginal_chunks(g) * sla::marginal_rows_pad(g) * 2;
  return forward_ws(g) + align_up(span_elems(g) * 2) + 2 * align_up(rows * g.D * 4) +
         3 * align_up(rows * 4) + align_up(blk * (g.D * g.D + g.D) * 2) +
         align_up(bh * g.nkb * (g.D * g.D + g.D) * 2) +
         align_up(bh * g.nkb * sla::backward_crit_words(g) * 4) + align_up(nmt * 4) +
         align_up(blk * 4);
}

BwdWs carve_backward_ws(const sla::Geometry& g, void* ws) {
  const size_t bh = static_cast<size_t>(g.B) * g.H;
  const size_t rows = bh * g.N;
  const size_t blk = bh * g.nq;
  const size_t nmt = bh * sla::marginal_chunks(g) * sla::marginal_rows_pad(g) * 2;
  BwdWs w;
  w.fwd = carve_forward_ws(g, ws);
  char* p = static_cast<char*>(ws) + forward_ws(g);
  w.o = p;
  p += align_up(span_elems(g) * 2);
  float* o_s = reinterpret_cast<float*>(p);
  p += align_up(rows * g.D * 4);
  float* o_l = reinterpret_cast<float*>(p);
  p += align_up(rows * g.D * 4);
  float* lse = reinterpret_cast<float*>(p);
  p += align_up(rows * 4);
  float* dd = reinterpret_cast<float*>(p);
  p += align_up(rows * 4);
  float* dol = reinterpret_cast<float*>(p);
  p += align_up(rows * 4);
  uint16_t* ds = reinterpret_cast<uint16_t*>(p);
  p += align_up(blk * (g.D * g.D + g.D) * 2);
  uint16_t* dh = reinterpret_cast<uint16_t*>(p);
  p += align_up(bh * g.nkb * (g.D * g.D + g.D) * 2);
  uint32_t* crit_t = reinterpret_cast<uint32_t*>(p);
  p += align_up(bh * g.nkb * sla::backward_crit_words(g) * 4);
  uint32_t* marg_t = reinterpret_cast<uint32_t*>(p);
  p += align_up(nmt * 4);
  float* dap = reinterpret_cast<float*>(p);
  w.b = sla::BackwardBuffers{o_s, o_l, lse, dd, dol, w.fwd.s_sum, w.fwd.sigma, ds, dh, crit_t,
                             marg_t, dap};
  return w;
}

int check_ws(void* ws, size_t ws_bytes, size_t need) {
  if (need == 0) return SLA_OK;
  if (!ws) return fail(SLA_ERR_WORKSPACE, "workspace is NULL (%zu bytes needed)", need);
  if (!aligned(ws, kWsAlign)) return fail(SLA_ERR_WORKSPACE, "workspace is not 256-byte aligned");
  if (ws_bytes < need)
    return fail(SLA_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the %zu needed", ws_bytes, need);
  return SLA_OK;
}

}  // namespace

extern "C" {

int sla_validate(const sla_problem* problem) {
  const int st = validate_problem(problem);
  if (st == SLA_OK) g_last_error.clear();
  return st;
}

int sla_num_blocks(const sla_problem* problem, int32_t* nq, int32_t* nkb) {
  SLA_TRY(validate_problem(problem));
  if (!nq || !nkb) return fail(SLA_ERR_INVALID_ARGUMENT, "output pointers are NULL");
  *nq = *nkb = (problem->seq_len + 63) / 64;
  return SLA_OK;
}

int sla_workspace_size(const sla_problem* problem, int op, size_t* bytes) {
  SLA_TRY(validate_problem(problem));
  if (!bytes) return fail(SLA_ERR_INVALID_ARGUMENT, "bytes is NULL");
  const sla::Geometry g = geometry(problem);
  switch (op) {
    case SLA_OP_ROUTE: *bytes = route_ws(g); return SLA_OK;
    case SLA_OP_LINEAR_STATES: *bytes = 0; return SLA_OK;
    case SLA_OP_FORWARD: *bytes = forward_ws(g); return SLA_OK;
    case SLA_OP_QUANTIZE_FP8: *bytes = 0; return SLA_OK;
    case SLA_OP_FORWARD_FP8: *bytes = forward_ws(g); return SLA_OK;
    case SLA_OP_ROUTE_TAYLOR: *bytes = route_taylor_ws(g); return SLA_OK;
    case SLA_OP_FORWARD_PISA: *bytes = pisa_ws(g); return SLA_OK;
    case SLA_OP_BACKWARD: *bytes = backward_ws(g); return SLA_OK;
    case SLA_OP_ROUTE_PISA: *bytes = route_pisa_ws(g); return SLA_OK;
    case SLA_OP_RESIDUAL_SUBTRACT: *bytes = forward_ws(g) + align_up(sla::residual_total_bytes(g)); return SLA_OK;
    default: return fail(SLA_ERR_INVALID_ARGUMENT, "unknown op %d", op);
  }
}

int sla_route(const sla_problem* problem, const void* q, const void* k, int32_t* crit_idx,
              int32_t* marg_idx, int8_t* block_class, float* block_logits, float* pooled_q,
              float* pooled_k, void* ws, size_t ws_bytes, void* stream) {
  SLA_TRY(validate_problem(problem));
  SLA_REQ(q, 16);
  SLA_REQ(k, 16);
  if (problem->k_crit > 0) SLA_REQ(crit_idx, 4);
  if (problem->k_marg > 0) SLA_REQ(marg_idx, 4);
  SLA_OPT(block_logits, 4);
  SLA_OPT(pooled_q, 4);
  SLA_OPT(pooled_k, 4);
  const sla::Geometry g = geometry(problem);
  SLA_TRY(check_ws(ws, ws_bytes, route_ws(g)));
  SLA_TRY(check_device());
  double* qpool = static_cast<double*>(ws);
  double* kpool = reinterpret_cast<double*>(static_cast<char*>(ws) + route_region(g));
  return launched(sla::launch_route(g, q, k, crit_idx, marg_idx, block_class, block_logits,
                                    pooled_q, pooled_k, qpool, kpool, nullptr, nullptr,
                                    static_cast<hipStream_t>(stream), nullptr, nullptr,
                                    route_keys(g, ws)),
                  "sla_route launch");
}

int sla_route_states(const sla_problem* problem, const void* q, const void* k, const void* v,
                     int32_t* crit_idx, int32_t* marg_idx, int8_t* block_class, float* block_logits,
                     float* pooled_q, float* pooled_k, void* h_states, float* z_states, void* ws,
                     size_t ws_bytes, void* stream) {
  SLA_TRY(validate_problem(problem));
  SLA_REQ(q, 16);
  SLA_REQ(k, 16);
  SLA_REQ(v, 16);
  SLA_REQ(h_states, 16);
  SLA_REQ(z_states, 16);
  if (problem->k_crit > 0) SLA_REQ(crit_idx, 4);
  if (problem->k_marg > 0) SLA_REQ(marg_idx, 4);
  SLA_OPT(block_logits, 4);
  SLA_OPT(pooled_q, 4);
  SLA_OPT(pooled_k, 4);
  const sla::Geometry g = geometry(problem);
  SLA_TRY(check_ws(ws, ws_bytes, route_ws(g)));
  SLA_TRY(check_device());
  double* qpool = static_cast<double*>(ws);
  double* kpool = reinterpret_cast<double*>(static_cast<char*>(ws) + route_region(g));
  const hipStream_t st = static_cast<hipStream_t>(stream);
  // bf16: the states pass also pools K; float32 inputs take the two passes
  const bool fused = g.dtype == 1;
  SLA_TRY(launched(sla::launch_states(g, k, v, static_cast<uint16_t*>(h_states), z_states, false, st,
                                      nullptr, nullptr, fused ? kpool : nullptr,
                                      fused ? pooled_k : nullptr),
                   "sla_route_states states launch"));
  return launched(sla::launch_route(g, q, k, crit_idx, marg_idx, block_class, block_logits,
                                    pooled_q, pooled_k, qpool, kpool, nullptr, nullptr, st,
                                    nullptr, nullptr, route_keys(g, ws), fused),
                  "sla_route_states route launch");
}

int sla_route_quantize(const sla_problem* problem, const void* q, const void* k, int32_t* crit_idx,
                       int32_t* marg_idx, int8_t* block_class, float* block_logits,
                       float* pooled_q, float* pooled_k, uint8_t* q8, float* q_scales,
                       uint8_t* k8, float* k_scales, void* ws, size_t ws_bytes, void* stream) {
  SLA_TRY(validate_problem(problem));
  SLA_REQ(q, 16);
  SLA_REQ(k, 16);
  if (problem->k_crit > 0) SLA_REQ(crit_idx, 4);
  if (problem->k_marg > 0) SLA_REQ(marg_idx, 4);
  SLA_OPT(block_logits, 4);
  SLA_OPT(pooled_q, 4);
  SLA_OPT(pooled_k, 4);
  SLA_REQ(q8, 16);
  SLA_REQ(k8, 16);
  SLA_REQ(q_scales, 4);
  SLA_REQ(k_scales, 4);
  const sla::Geometry g = geometry(problem);
  SLA_TRY(check_ws(ws, ws_bytes, route_ws(g)));
  SLA_TRY(check_device());
  double* qpool = static_cast<double*>(ws);
  double* kpool = reinterpret_cast<double*>(static_cast<char*>(ws) + route_region(g));
  const sla::Fp8Out f8{q8, q_scales, k8, k_scales};
  return launched(sla::launch_route(g, q, k, crit_idx, marg_idx, block_class, block_logits,
                                    pooled_q, pooled_k, qpool, kpool, nullptr, nullptr,
                                    static_cast<hipStream_t>(stream), nullptr, &f8,
                                    route_keys(g, ws)),
                  "sla_route_quantize launch");
}

int sla_route_noalloc(const sla_problem* problem, const void* q, const void* k, int32_t* crit_idx,
                      int32_t* marg_idx, int8_t* block_class, float* block_logits,
                      float* pooled_q, float* pooled_k, void* stream) {
  SLA_TRY(validate_problem(problem));
  SLA_REQ(q, 16);
  SLA_REQ(k, 16);
  if (problem->k_crit > 0) SLA_REQ(crit_idx, 4);
  if (problem->k_marg > 0) SLA_REQ(marg_idx, 4);
  SLA_OPT(block_logits, 4);
  SLA_OPT(pooled_q, 4);
  SLA_OPT(pooled_k, 4);
  const sla::Geometry g = geometry(problem);
  const size_t need = 2 * route_region(g);   // pooled sums; the fused selection kernel
  if (need > sla::kStaticScratchBytes)
    return fail(SLA_ERR_WORKSPACE,
                "routing needs %zu bytes of scratch; the static scratch holds %zu "
                "(use sla_route with a caller workspace)",
                need, sla::kStaticScratchBytes);
  SLA_TRY(check_device());
  void* ws = nullptr;
  SLA_TRY(launched(sla::static_scratch(&ws), "static scratch lookup"));
  double* qpool = static_cast<double*>(ws);
  double* kpool_t = reinterpret_cast<double*>(static_cast<char*>(ws) + route_region(g));
  return launched(sla::launch_route(g, q, k, crit_idx, marg_idx, block_class, block_logits,
                                    pooled_q, pooled_k, qpool, kpool_t, nullptr, nullptr,
                                    static_cast<hipStream_t>(stream)),
                  "sla_route_noalloc launch");
}

int sla_validate_lists(const sla_problem* problem, const int32_t* crit_idx,
                       const int32_t* marg_idx, void* stream) {
  SLA_TRY(validate_problem(problem));
  if (problem->k_crit > 0) SLA_REQ(crit_idx, 4);
  if (problem->k_marg > 0) SLA_REQ(marg_idx, 4);
  const sla::Geometry g = geometry(problem);
  SLA_TRY(check_device());
  unsigned int bad = 0, first = 0;
  SLA_TRY(launched(sla::validate_lists(g, crit_idx, marg_idx, static_cast<hipStream_t>(stream),
                                       &bad, &first),
                   "sla_validate_lists"));
  if (bad == 0) return SLA_OK;
  const int i = static_cast<int>(first % static_cast<unsigned int>(g.nq));
  const int bh = static_cast<int>(first / static_cast<unsigned int>(g.nq));
  return fail(SLA_ERR_INVALID_ARGUMENT,
              "%u of %lld rows hold an index outside [0, %d), a repeat or a block in both lists; "
              "first at batch %d, head %d, query block %d",
              bad, static_cast<long long>(g.B) * g.H * g.nq, g.nkb, bh / g.H, bh % g.H, i);
}

int sla_route_taylor(const sla_problem* problem, const void* q, const void* k, int32_t* crit_idx,
                     int32_t* marg_idx, int8_t* block_class, float* block_logits,
                     float* pooled_q, float* pooled_k, float* key_var, void* ws, size_t ws_bytes,
                     void* stream) {
  SLA_TRY(validate_problem(problem));
  SLA_REQ(q, 16);
  SLA_REQ(k, 16);
  if (problem->k_crit > 0) SLA_REQ(crit_idx, 4);
  if (problem->k_marg > 0) SLA_REQ(marg_idx, 4);
  SLA_OPT(block_logits, 4);
  SLA_OPT(pooled_q, 4);
  SLA_OPT(pooled_k, 4);
  SLA_OPT(key_var, 4);
  const sla::Geometry g = geometry(problem);
  SLA_TRY(check_ws(ws, ws_bytes, route_taylor_ws(g)));
  SLA_TRY(check_device());
  char* p = static_cast<char*>(ws);
  double* qpool = reinterpret_cast<double*>(p);
  double* kpool = reinterpret_cast<double*>(p + route_region(g));
  double* kvar = reinterpret_cast<double*>(p + route_ws(g));
  return launched(sla::launch_route(g, q, k, crit_idx, marg_idx, block_class, block_logits,
                                    pooled_q, pooled_k, qpool, kpool, kvar, key_var,
                                    static_cast<hipStream_t>(stream), nullptr, nullptr,
                                    route_keys(g, ws)),
                  "sla_route_taylor launch");
}

int sla_linear_states_quantize(const sla_problem* problem, const void* k, const void* v,
                               void* h_states, float* z_states, uint8_t* v8, float* v_scales,
                               void* stream) {
  SLA_TRY(validate_problem(problem));
  SLA_REQ(k, 16);
  SLA_REQ(v, 16);
  SLA_REQ(h_states, 16);
  SLA_REQ(z_states, 16);
  SLA_REQ(v8, 16);
  SLA_REQ(v_scales, 4);
  const sla::Geometry g = geometry(problem);
  SLA_TRY(check_device());
  return launched(sla::launch_states(g, k, v, static_cast<uint16_t*>(h_states), z_states, false,
                                     static_cast<hipStream_t>(stream), v8, v_scales),
                  "sla_linear_states_quantize launch");
}

int sla_linear_states(const sla_problem* problem, const void* k, const void* v, void* h_states,
                      float* z_states, void* stream) {
  SLA_TRY(validate_problem(problem));
  SLA_REQ(k, 16);
  SLA_REQ(v, 16);
  SLA_REQ(h_states, 16);
  SLA_REQ(z_states, 16);
  const sla::Geometry g = geometry(problem);
  SLA_TRY(check_device());
  return launched(sla::launch_states(g, k, v, static_cast<uint16_t*>(h_states), z_states, false,
                                     static_cast<hipStream_t>(stream)),
                  "sla_linear_states launch");
}

int sla_forward(const sla_problem* problem, const void* q, const void* k, const void* v,
                const int32_t* crit_idx, const int32_t* marg_idx, const void* h_states,
                const float* z_states, const float* alpha, void* o, float* o_sparse,
                float* o_linear, void* ws, size_t ws_bytes, void* stream) {
  SLA_TRY(validate_problem(problem));
  SLA_REQ(q, 16);
  SLA_REQ(k, 16);
  SLA_REQ(v, 16);
  SLA_REQ(alpha, 4);
  SLA_REQ(o, 16);
  if (problem->k_crit > 0) SLA_REQ(crit_idx, 4);
  if (problem->k_marg > 0) {
    SLA_REQ(marg_idx, 4);
    SLA_REQ(h_states, 16);
    SLA_REQ(z_states, 16);
  }
  SLA_OPT(o_sparse, 16);
  SLA_OPT(o_linear, 16);
  const sla::Geometry g = geometry(problem);
  SLA_TRY(check_ws(ws, ws_bytes, forward_ws(g)));
  SLA_TRY(check_device());
  const FwdWs w = carve_forward_ws(g, ws);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (g.k_marg > 0)
    SLA_TRY(launched(sla::launch_marginal_sums(g, marg_idx, static_cast<const uint16_t*>(h_states),
                                               z_states, w.s_sum, w.sigma, w.bits, w.zhl, false, s),
                     "marginal-sum launch"));
  return launched(sla::launch_attention(g, q, k, v, crit_idx, w.s_sum, w.sigma, alpha, o, o_sparse,
                                        o_linear, false, s),
                  "attention launch");
}

int sla_marginal_sums(const sla_problem* problem, const int32_t* marg_idx, const void* h_states,
                      const float* z_states, void* ws, size_t ws_bytes, void* stream) {
  SLA_TRY(validate_problem(problem));
  if (problem->k_marg > 0) {
    SLA_REQ(marg_idx, 4);
    SLA_REQ(h_states, 16);
    SLA_REQ(z_states, 16);
  }
  const sla::Geometry g = geometry(problem);
  SLA_TRY(check_ws(ws, ws_bytes, forward_ws(g)));
  SLA_TRY(check_device());
  if (g.k_marg == 0) return SLA_OK;
  const FwdWs w = carve_forward_ws(g, ws);
  return launched(sla::launch_marginal_sums(g, marg_idx, static_cast<const uint16_t*>(h_states),
                                            z_states, w.s_sum, w.sigma, w.bits, w.zhl, false,
                                            static_cast<hipStream_t>(stream)),
                  "marginal-sum launch");
}

int sla_forward_attend(const sla_problem* problem, const void* q, const void* k, const void* v,
                       const int32_t* crit_idx, const float* alpha, void* o, float* o_sparse,
                       float* o_linear, const void* ws, size_t ws_bytes, void* stream) {
  SLA_TRY(validate_problem(problem));
  SLA_REQ(q, 16);
  SLA_REQ(k, 16);
  SLA_REQ(v, 16);
  SLA_REQ(alpha, 4);
  SLA_REQ(o, 16);
  if (problem->k_crit > 0) SLA_REQ(crit_idx, 4);
  SLA_OPT(o_sparse, 16);
  SLA_OPT(o_linear, 16);
  const sla::Geometry g = geometry(problem);
  SLA_TRY(check_ws(const_cast<void*>(ws), ws_bytes, forward_ws(g)));
  SLA_TRY(check_device());
  const FwdWs w = carve_forward_ws(g, const_cast<void*>(ws));
  return launched(sla::launch_attention(g, q, k, v, crit_idx, w.s_sum, w.sigma, alpha, o, o_sparse,
                                        o_linear, false, static_cast<hipStream_t>(stream)),
                  "attention launch");
}

int sla_quantize_fp8(const sla_problem* problem, const void* x, uint8_t* x_e4m3, float* scales,
                     void* stream) {
  SLA_TRY(validate_problem(problem));
  SLA_REQ(x, 16);
  SLA_REQ(x_e4m3, 16);
  SLA_REQ(scales, 4);
  const sla::Geometry g = geometry(problem);
  SLA_TRY(check_device());
  return launched(sla::launch_quantize_fp8(g, x, x_e4m3, scales, static_cast<hipStream_t>(stream)),
                  "sla_quantize_fp8 launch");
}

namespace {

// Checks shared by the two fp8 forward entry points (everything but the
// marginal-state arguments).
int check_fp8_args(const sla_problem* problem, const void* q, const uint8_t* q8, const float* q_s,
                   const uint8_t* k8, const float* k_s, const uint8_t* v8, const float* v_s,
                   const int32_t* crit_idx, const float* alpha, void* o, float* o_sparse,
                   float* o_linear) {
  SLA_TRY(validate_problem(problem));
  if (problem->dtype != SLA_BF16)
    return fail(SLA_ERR_UNSUPPORTED, "the fp8 forward takes bf16 Q and O");
  if (problem->head_dim != 128)
    return fail(SLA_ERR_UNSUPPORTED, "the fp8 forward supports head_dim 128");
  SLA_REQ(q, 16);
  SLA_REQ(q8, 16);
  SLA_REQ(k8, 16);
  SLA_REQ(v8, 16);
  SLA_REQ(q_s, 4);
  SLA_REQ(k_s, 4);
  SLA_REQ(v_s, 4);
  SLA_REQ(alpha, 4);
  SLA_REQ(o, 16);
  if (problem->k_crit > 0) SLA_REQ(crit_idx, 4);
  SLA_OPT(o_sparse, 16);
  SLA_OPT(o_linear, 16);
  return SLA_OK;
}

}  // namespace

int sla_forward_fp8(const sla_problem* problem, const void* q, const uint8_t* q8, const float* q_s,
                    const uint8_t* k8, const float* k_s, const uint8_t* v8, const float* v_s,
                    const int32_t* crit_idx, const int32_t* marg_idx, const void* h_states,
                    const float* z_states, const float* alpha, void* o, float* o_sparse,
                    float* o_linear, void* ws, size_t ws_bytes, void* stream) {
  SLA_TRY(check_fp8_args(problem, q, q8, q_s, k8, k_s, v8, v_s, crit_idx, alpha, o, o_sparse,
                         o_linear));
  if (problem->k_marg > 0) {
    SLA_REQ(marg_idx, 4);
    SLA_REQ(h_states, 16);
    SLA_REQ(z_states, 16);
  }
  const sla::Geometry g = geometry(problem);
  SLA_TRY(check_ws(ws, ws_bytes, forward_ws(g)));
  SLA_TRY(check_device());
  const FwdWs w = carve_forward_ws(g, ws);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (g.k_marg > 0)
    SLA_TRY(launched(sla::launch_marginal_sums(g, marg_idx, static_cast<const uint16_t*>(h_states),
                                               z_states, w.s_sum, w.sigma, w.bits, w.zhl, false, s),
                     "marginal-sum launch"));
  return launched(sla::launch_attention_fp8(g, q, q8, q_s, k8, k_s, v8, v_s, crit_idx, w.s_sum,
                                            w.sigma, alpha, o, o_sparse, o_linear, s),
                  "fp8 attention launch");
}

int sla_forward_attend_fp8(const sla_problem* problem, const void* q, const uint8_t* q8,
                           const float* q_s, const uint8_t* k8, const float* k_s,
                           const uint8_t* v8, const float* v_s, const int32_t* crit_idx,
                           const float* alpha, void* o, float* o_sparse, float* o_linear,
                           const void* ws, size_t ws_bytes, void* stream) {
  SLA_TRY(check_fp8_args(problem, q, q8, q_s, k8, k_s, v8, v_s, crit_idx, alpha, o, o_sparse,
                         o_linear));
  const sla::Geometry g = geometry(problem);
  SLA_TRY(check_ws(const_cast<void*>(ws), ws_bytes, forward_ws(g)));
  SLA_TRY(check_device());
  const FwdWs w = carve_forward_ws(g, const_cast<void*>(ws));
  return launched(sla::launch_attention_fp8(g, q, q8, q_s, k8, k_s, v8, v_s, crit_idx, w.s_sum,
                                            w.sigma, alpha, o, o_sparse, o_linear,
                                            static_cast<hipStream_t>(stream)),
                  "fp8 attention launch");
}

// ---------------------------------------------------------------- residual linear attention

int sla_linear_states_exp(const sla_problem* problem, const void* k, const void* v,
                          void* h_states, float* z_states, void* stream) {
  SLA_TRY(validate_problem(problem));
  SLA_REQ(k, 16);
  SLA_REQ(v, 16);
  SLA_REQ(h_states, 16);
  SLA_REQ(z_states, 16);
  const sla::Geometry g = geometry(problem);
  SLA_TRY(check_device());
  return launched(sla::launch_states(g, k, v, static_cast<uint16_t*>(h_states), z_states, true,
                                     static_cast<hipStream_t>(stream)),
                  "sla_linear_states_exp launch");
}

namespace {
// The residual state covers every non-critical block: k_marg names that count.
int check_rla_counts(const sla_problem* p) {
  const int64_t nkb = (static_cast<int64_t>(p->seq_len) + 63) / 64;
  if (p->k_marg != nkb - p->k_crit)
    return fail(SLA_ERR_INVALID_ARGUMENT,
                "residual linear attention sums every non-critical block: k_marg must be "
                "nkb - k_crit = %lld, got %d", static_cast<long long>(nkb - p->k_crit), p->k_marg);
  return SLA_OK;
}
}  // namespace

int sla_residual_sums(const sla_problem* problem, const int32_t* crit_idx, const void* h_states,
                      void* ws, size_t ws_bytes, void* stream) {
  SLA_TRY(validate_problem(problem));
  SLA_TRY(check_rla_counts(problem));
  if (problem->k_crit > 0) SLA_REQ(crit_idx, 4);
  if (problem->k_marg > 0) SLA_REQ(h_states, 16);
  const sla::Geometry g = geometry(problem);
  SLA_TRY(check_ws(ws, ws_bytes, forward_ws(g)));
  SLA_TRY(check_device());
  if (g.k_marg == 0) return SLA_OK;
  const FwdWs w = carve_forward_ws(g, ws);
  return launched(sla::launch_marginal_sums(g, crit_idx, static_cast<const uint16_t*>(h_states),
                                            nullptr, w.s_sum, nullptr, w.bits, w.zhl, true,
                                            static_cast<hipStream_t>(stream)),
                  "residual-sum launch");
}

int sla_residual_sums_subtract(const sla_problem* problem, const int32_t* crit_idx,
                               const void* h_states, void* ws, size_t ws_bytes, void* stream) {
  SLA_TRY(validate_problem(problem));
  SLA_TRY(check_rla_counts(problem));
  if (problem->k_crit > 0) SLA_REQ(crit_idx, 4);
  if (problem->k_marg > 0) SLA_REQ(h_states, 16);
  const sla::Geometry g = geometry(problem);
  SLA_TRY(check_ws(ws, ws_bytes, forward_ws(g) + align_up(sla::residual_total_bytes(g))));
  SLA_TRY(check_device());
  if (g.k_marg == 0) return SLA_OK;
  const FwdWs w = carve_forward_ws(g, ws);
  float* tot = reinterpret_cast<float*>(static_cast<char*>(ws) + forward_ws(g));
  return launched(sla::launch_residual_subtract(g, crit_idx, static_cast<const uint16_t*>(h_states),
                                                w.s_sum, w.bits, tot,
                                                static_cast<hipStream_t>(stream)),
                  "residual-sum (subtraction form) launch");
}

int sla_forward_attend_rla(const sla_problem* problem, const void* q, const void* k, const void* v,
                           const int32_t* crit_idx, const float* alpha, void* o, float* o_sparse,
                           float* o_linear, const void* ws, size_t ws_bytes, void* stream) {
  SLA_TRY(validate_problem(problem));
  SLA_TRY(check_rla_counts(problem));
  SLA_REQ(q, 16);
  SLA_REQ(k, 16);
  SLA_REQ(v, 16);
  SLA_REQ(alpha, 4);
  SLA_REQ(o, 16);
  if (problem->k_crit > 0) SLA_REQ(crit_idx, 4);
  SLA_OPT(o_sparse, 16);
  SLA_OPT(o_linear, 16);
  const sla::Geometry g = geometry(problem);
  SLA_TRY(check_ws(const_cast<void*>(ws), ws_bytes, forward_ws(g)));
  SLA_TRY(check_device());
  const FwdWs w = carve_forward_ws(g, const_cast<void*>(ws));
  return launched(sla::launch_attention(g, q, k, v, crit_idx, w.s_sum, w.sigma, alpha, o, o_sparse,
                                        o_linear, true, static_cast<hipStream_t>(stream)),
                  "attention launch");
}

int sla_forward_rla(const sla_problem* problem, const void* q, const void* k, const void* v,
                    const int32_t* crit_idx, const void* h_states, const float* alpha, void* o,
                    float* o_sparse, float* o_linear, void* ws, size_t ws_bytes, void* stream) {
  SLA_TRY(sla_residual_sums(problem, crit_idx, h_states, ws, ws_bytes, stream));
  return sla_forward_attend_rla(problem, q, k, v, crit_idx, alpha, o, o_sparse, o_linear, ws,
                                ws_bytes, stream);
}

int sla_pisa_statistics(const sla_problem* problem, const void* k, const void* v, float* hbar,
                        void* ws, size_t ws_bytes, void* stream) {
  SLA_TRY(validate_problem(problem));
  SLA_REQ(k, 16);
  SLA_REQ(v, 16);
  SLA_OPT(hbar, 16);
  const sla::Geometry g = geometry(problem);
  SLA_TRY(check_ws(ws, ws_bytes, pisa_ws(g)));
  SLA_TRY(check_device());
  const PisaWs w = carve_pisa_ws(g, ws);
  return launched(sla::launch_pisa_stats(g, k, v, w.kbar, w.vbar, w.hbar, w.part, hbar,
                                         static_cast<hipStream_t>(stream)),
                  "PISA statistics launch");
}

int sla_route_pisa(const sla_problem* problem, const void* q, const void* k, const void* v,
                   int32_t* crit_idx, int32_t* marg_idx, int8_t* block_class, float* block_logits,
                   float* pooled_q, float* pooled_k, float* block_dev, void* ws, size_t ws_bytes,
                   void* stream) {
  SLA_TRY(validate_problem(problem));
  SLA_REQ(q, 16);
  SLA_REQ(k, 16);
  SLA_REQ(v, 16);
  if (problem->k_crit > 0) SLA_REQ(crit_idx, 4);
  if (problem->k_marg > 0) SLA_REQ(marg_idx, 4);
  SLA_OPT(block_logits, 4);
  SLA_OPT(pooled_q, 4);
  SLA_OPT(pooled_k, 4);
  SLA_OPT(block_dev, 4);
  const sla::Geometry g = geometry(problem);
  SLA_TRY(check_ws(ws, ws_bytes, route_pisa_ws(g)));
  SLA_TRY(check_device());
  const PisaWs w = carve_pisa_ws(g, ws);
  const size_t bh = static_cast<size_t>(g.B) * g.H;
  char* p = static_cast<char*>(ws) + pisa_ws(g);
  double* qpool = reinterpret_cast<double*>(p);
  double* kpool = reinterpret_cast<double*>(p + route_region(g));
  float* hbar_f32 = reinterpret_cast<float*>(p + route_ws(g));
  double* mdev = reinterpret_cast<double*>(p + route_ws(g) + align_up(bh * g.D * g.D * 4));
  const hipStream_t st = static_cast<hipStream_t>(stream);
  SLA_TRY(launched(sla::launch_pisa_stats(g, k, v, w.kbar, w.vbar, w.hbar, w.part, hbar_f32, st),
                   "PISA statistics launch"));
  SLA_TRY(launched(sla::launch_pisa_deviation(g, k, v, w.hbar, w.part, hbar_f32, mdev, block_dev, st),
                   "PISA block deviation launch"));
  return launched(sla::launch_route(g, q, k, crit_idx, marg_idx, block_class, block_logits,
                                    pooled_q, pooled_k, qpool, kpool, nullptr, nullptr, st, mdev,
                                    nullptr, route_keys(g, p)),
                  "sla_route_pisa launch");
}

int sla_forward_attend_pisa(const sla_problem* problem, const void* q, const void* k,
                            const void* v, const int32_t* crit_idx, void* o, float* o_softmax,
                            float* o_correction, const void* ws, size_t ws_bytes, void* stream) {
  SLA_TRY(validate_problem(problem));
  SLA_REQ(q, 16);
  SLA_REQ(k, 16);
  SLA_REQ(v, 16);
  SLA_REQ(o, 16);
  if (problem->k_crit > 0) SLA_REQ(crit_idx, 4);
  SLA_OPT(o_softmax, 16);
  SLA_OPT(o_correction, 16);
  const sla::Geometry g = geometry(problem);
  SLA_TRY(check_ws(const_cast<void*>(ws), ws_bytes, pisa_ws(g)));
  SLA_TRY(check_device());
  const PisaWs w = carve_pisa_ws(g, const_cast<void*>(ws));
  return launched(sla::launch_attention_pisa(g, q, k, v, crit_idx, w.kbar, w.vbar, w.hbar, o,
                                             o_softmax, o_correction,
                                             static_cast<hipStream_t>(stream)),
                  "PISA attention launch");
}

int sla_forward_pisa(const sla_problem* problem, const void* q, const void* k, const void* v,
                     const int32_t* crit_idx, void* o, float* o_softmax, float* o_correction,
                     void* ws, size_t ws_bytes, void* stream) {
  SLA_TRY(sla_pisa_statistics(problem, k, v, nullptr, ws, ws_bytes, stream));
  return sla_forward_attend_pisa(problem, q, k, v, crit_idx, o, o_softmax, o_correction, ws,
                                 ws_bytes, stream);
}

// The forward pass of sla_backward: marginal sums, then the fused kernel
// writing O (to o), O_s, O_l and each row's log2 softmax normaliser into the
// backward workspace.
static int backward_forward_part(const sla::Geometry& g, const void* q, const void* k,
                                 const void* v, const int32_t* crit_idx, const int32_t* marg_idx,
                                 const void* h_states, const float* z_states, const float* alpha,
                                 void* o, const BwdWs& w, hipStream_t st) {
  if (g.k_marg > 0)
    SLA_TRY(launched(sla::launch_marginal_sums(g, marg_idx, static_cast<const uint16_t*>(h_states),
                                               z_states, w.fwd.s_sum, w.fwd.sigma, w.fwd.bits,
                                               w.fwd.zhl, false, st),
                     "backward marginal sums"));
  return launched(sla::launch_attention(g, q, k, v, crit_idx, w.fwd.s_sum, w.fwd.sigma, alpha, o,
                                        const_cast<float*>(w.b.o_s), const_cast<float*>(w.b.o_l),
                                        false, st, const_cast<float*>(w.b.lse)),
                  "backward forward pass");
}

// Argument checks shared by the backward entry points and sla_forward_save.
static int check_backward_args(const sla_problem* problem, const void* q, const void* k,
                               const void* v, const int32_t* crit_idx, const int32_t* marg_idx,
                               const float* alpha) {
  SLA_TRY(validate_problem(problem));
  if (problem->dtype != SLA_BF16)
    return fail(SLA_ERR_UNSUPPORTED, "the backward pass takes bf16 inputs only");
  SLA_REQ(q, 16);
  SLA_REQ(k, 16);
  SLA_REQ(v, 16);
  SLA_REQ(alpha, 4);
  if (problem->k_crit > 0) SLA_REQ(crit_idx, 4);
  if (problem->k_marg > 0) SLA_REQ(marg_idx, 4);
  return SLA_OK;
}

static int check_gradient_args(const void* dout, float* dq, float* dk, float* dv, float* dalpha) {
  SLA_REQ(dout, 16);
  SLA_REQ(dq, 16);
  SLA_REQ(dk, 16);
  SLA_REQ(dv, 16);
  SLA_REQ(dalpha, 4);
  return SLA_OK;
}

int sla_backward(const sla_problem* problem, const void* q, const void* k, const void* v,
                 const void* dout, const int32_t* crit_idx, const int32_t* marg_idx,
                 const void* h_states, const float* z_states, const float* alpha, float* dq,
                 float* dk, float* dv, float* dalpha, void* ws, size_t ws_bytes, void* stream) {
  SLA_TRY(check_backward_args(problem, q, k, v, crit_idx, marg_idx, alpha));
  SLA_TRY(check_gradient_args(dout, dq, dk, dv, dalpha));
  if (problem->k_marg > 0) {
    SLA_REQ(h_states, 16);
    SLA_REQ(z_states, 16);
  }
  const sla::Geometry g = geometry(problem);
  SLA_TRY(check_ws(ws, ws_bytes, backward_ws(g)));
  SLA_TRY(check_device());
  const BwdWs w = carve_backward_ws(g, ws);
  const hipStream_t st = static_cast<hipStream_t>(stream);
  SLA_TRY(backward_forward_part(g, q, k, v, crit_idx, marg_idx, h_states, z_states, alpha, w.o, w,
                                st));
  return launched(sla::launch_backward(g, w.b, q, k, v, dout, crit_idx, marg_idx, alpha, dq, dk,
                                       dv, dalpha, st),
                  "backward launch");
}

int sla_forward_save(const sla_problem* problem, const void* q, const void* k, const void* v,
                     const int32_t* crit_idx, const int32_t* marg_idx, const void* h_states,
                     const float* z_states, const float* alpha, void* o, void* ws,
                     size_t ws_bytes, void* stream) {
  SLA_TRY(check_backward_args(problem, q, k, v, crit_idx, marg_idx, alpha));
  SLA_REQ(o, 16);
  if (problem->k_marg > 0) {
    SLA_REQ(h_states, 16);
    SLA_REQ(z_states, 16);
  }
  const sla::Geometry g = geometry(problem);
  SLA_TRY(check_ws(ws, ws_bytes, backward_ws(g)));
  SLA_TRY(check_device());
  const BwdWs w = carve_backward_ws(g, ws);
  return backward_forward_part(g, q, k, v, crit_idx, marg_idx, h_states, z_states, alpha, o, w,
                               static_cast<hipStream_t>(stream));
}

int sla_forward_save_fp8(const sla_problem* problem, const void* q, const void* k, const void* v,
                         const uint8_t* q8, const float* q_s, const uint8_t* k8, const float* k_s,
                         const uint8_t* v8, const float* v_s, const int32_t* crit_idx,
                         const int32_t* marg_idx, const void* h_states, const float* z_states,
                         const float* alpha, void* o, void* ws, size_t ws_bytes, void* stream) {
  SLA_TRY(check_backward_args(problem, q, k, v, crit_idx, marg_idx, alpha));
  SLA_TRY(check_fp8_args(problem, q, q8, q_s, k8, k_s, v8, v_s, crit_idx, alpha, o, nullptr,
                         nullptr));
  if (problem->k_marg > 0) {
    SLA_REQ(h_states, 16);
    SLA_REQ(z_states, 16);
  }
  const sla::Geometry g = geometry(problem);
  SLA_TRY(check_ws(ws, ws_bytes, backward_ws(g)));
  SLA_TRY(check_device());
  const BwdWs w = carve_backward_ws(g, ws);
  const hipStream_t st = static_cast<hipStream_t>(stream);
  if (g.k_marg > 0)
    SLA_TRY(launched(sla::launch_marginal_sums(g, marg_idx, static_cast<const uint16_t*>(h_states),
                                               z_states, w.fwd.s_sum, w.fwd.sigma, w.fwd.bits,
                                               w.fwd.zhl, false, st),
                     "marginal sums"));
  return launched(sla::launch_attention_fp8(g, q, q8, q_s, k8, k_s, v8, v_s, crit_idx, w.fwd.s_sum,
                                            w.fwd.sigma, alpha, o, const_cast<float*>(w.b.o_s),
                                            const_cast<float*>(w.b.o_l), st,
                                            const_cast<float*>(w.b.lse)),
                  "fp8 forward (saved)");
}

int sla_backward_saved(const sla_problem* problem, const void* q, const void* k, const void* v,
                       const void* dout, const int32_t* crit_idx, const int32_t* marg_idx,
                       const float* alpha, float* dq, float* dk, float* dv, float* dalpha,
                       void* ws, size_t ws_bytes, void* stream) {
  SLA_TRY(check_backward_args(problem, q, k, v, crit_idx, marg_idx, alpha));
  SLA_TRY(check_gradient_args(dout, dq, dk, dv, dalpha));
  const sla::Geometry g = geometry(problem);
  SLA_TRY(check_ws(ws, ws_bytes, backward_ws(g)));
  SLA_TRY(check_device());
  const BwdWs w = carve_backward_ws(g, ws);
  return launched(sla::launch_backward(g, w.b, q, k, v, dout, crit_idx, marg_idx, alpha, dq, dk,
                                       dv, dalpha, static_cast<hipStream_t>(stream)),
                  "backward launch");
}

const char* sla_status_string(int status) {
  switch (status) {
    case SLA_OK: return "ok";
    case SLA_ERR_INVALID_ARGUMENT: return "invalid argument";
    case SLA_ERR_UNSUPPORTED: return "unsupported";
    case SLA_ERR_WORKSPACE: return "workspace too small";
    case SLA_ERR_DEVICE: return "device error";
    case SLA_ERR_NO_DEVICE: return "no gfx950 device";
    default: return "unknown status";
  }
}

const char* sla_last_error_message(void) { return g_last_error.c_str(); }

int sla_version(int* major, int* minor, int* patch) {
  if (!major || !minor || !patch) return fail(SLA_ERR_INVALID_ARGUMENT, "NULL output pointer");
  *major = SLA_VERSION_MAJOR;
  *minor = SLA_VERSION_MINOR;
  *patch = SLA_VERSION_PATCH;
  return SLA_OK;
}

}  // extern "C"
