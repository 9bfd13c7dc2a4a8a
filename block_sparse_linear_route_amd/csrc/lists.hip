// Check of caller-supplied block index lists.
//
// [SLA abstract] each KV block of a query block's row belongs to exactly one
// of the critical, marginal and negligible classes; the compute entry points
// take the first two classes as index lists.  They clamp every entry into
// [0, nkb) before forming an address, so no list content makes them access
// memory outside their tensors, but an invalid list gives meaningless
// results.  This pass reports such lists: per row, every entry must lie in
// [0, nkb), no list may hold an index twice and no index may be in both.
//
// One workgroup per row (b, h, i): the row's blocks are marked in an LDS bit
// row, critical entries first (a bit already set is a repeat), then, after a
// barrier, marginal entries (a set bit is a repeat or a critical block).  The
// number of bad rows and the smallest bad row index go to a two-word report
// that the host clears beforehand with a one-thread kernel.
#include <hip/hip_runtime.h>

#include <mutex>

#include "device_common.hpp"
#include "sla_internal.hpp"

namespace sla {
namespace {

static __device__ __align__(16) unsigned int list_report[2];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
unsigned int* g_report[kMaxDevices] = {};

__global__ void clear_report_kernel(unsigned int* r) {
  r[0] = 0u;
  r[1] = 0xffffffffu;
}

__global__ void __launch_bounds__(kThreads)
validate_lists_kernel(Geometry g, const int32_t* __restrict__ crit,
                      const int32_t* __restrict__ marg, unsigned int* __restrict__ report) {
  __shared__ uint32_t bits[kMaxKvBlocks / 32];
  __shared__ int bad;
  const int t = threadIdx.x;
  const int64_t row = blockIdx.x;                 // bh * nq + i
  const int nw = (g.nkb + 31) / 32;
  for (int w = t; w < nw; w += kThreads) bits[w] = 0u;
  if (t == 0) bad = 0;
  __syncthreads();
  bool my_bad = false;
  auto mark = [&](int j) {
    if (j < 0 || j >= g.nkb) {
      my_bad = true;
      return;
    }
    const uint32_t bit = 1u << (j & 31);
    if (atomicOr(&bits[j >> 5], bit) & bit) my_bad = true;
  };
  for (int u = t; u < g.k_crit; u += kThreads) mark(crit[row * g.k_crit + u]);
  __syncthreads();
  for (int u = t; u < g.k_marg; u += kThreads) mark(marg[row * g.k_marg + u]);
  if (my_bad) bad = 1;
  __syncthreads();
  if (t == 0 && bad) {
    atomicAdd(&report[0], 1u);
    atomicMin(&report[1], static_cast<unsigned int>(row));
  }
}

}  // namespace

hipError_t validate_lists(const Geometry& g, const int32_t* crit, const int32_t* marg,
                          hipStream_t stream, unsigned int* bad_rows, unsigned int* first_bad) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  // one report per GPU: calls on one GPU take turns
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_report[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(list_report));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_report[dev] = static_cast<unsigned int*>(p);
  }
  unsigned int* rep = g_report[dev];
  hipLaunchKernelGGL(clear_report_kernel, dim3(1), dim3(1), 0, stream, rep);
  const int64_t rows = static_cast<int64_t>(g.B) * g.H * g.nq;
  hipLaunchKernelGGL(validate_lists_kernel, dim3(static_cast<unsigned int>(rows)), dim3(kThreads), 0,
                     stream, g, crit, marg, rep);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  unsigned int host[2] = {0u, 0u};
  e = hipMemcpyAsync(host, rep, sizeof(host), hipMemcpyDeviceToHost, stream);
  if (e != hipSuccess) return e;
  e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return e;
  *bad_rows = host[0];
  *first_bad = host[1];
  return hipSuccess;
}

}  // namespace sla
