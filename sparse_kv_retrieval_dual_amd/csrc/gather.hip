// Row gather from the host-resident KV cache into device memory (arXiv page
// of DualDecoder, section 2.2 and Figure 1: the selected entries are
// noncontiguous in host memory and are gathered into the GPU before
// attention; the paper-daily worked example sizes one such transfer).
//
// The kernel reads pinned, device-mapped host rows directly over the host
// link: one row (128-512 B) is read by ROWB/16 lanes with 16-byte loads, and
// every wave keeps 4 row groups of K and V in flight.  The grid is capped:
// the link saturates with a few hundred KB outstanding, and more outstanding
// host reads only slow down HBM traffic of kernels running beside the
// gather (measured on MI355X: with 64 workgroups a concurrent scoring kernel
// ran 50% slower, with 16 about 25%).
#include "dd_internal.h"
#include "gather_body.h"
#include "gather_res.h"

namespace dd {

namespace {

constexpr int kGatherThreads = 256;
constexpr int kDefaultMaxWgs = 1024;

template <int ROWB>
__global__ __launch_bounds__(kGatherThreads) void k_gather(GatherJob g) {
  const int64_t gw = (int64_t)blockIdx.x * (kGatherThreads / 64) + (threadIdx.x >> 6);
  const int64_t nw = (int64_t)gridDim.x * (kGatherThreads / 64);
  gather_rows<ROWB>(g, gw, nw);
}

// The prefetch of a layer whose rows are kept across steps (V plane, one
// row per entry); each wave keeps its two copy queues in LDS.
template <int ROWB>
__global__ __launch_bounds__(kGatherThreads) void k_gather_resident(GatherJob g, GatherRes r) {
  __shared__ ResQueue qh[kGatherThreads / 64];
  __shared__ ResQueue qd[kGatherThreads / 64];
  const int w = threadIdx.x >> 6;
  const int64_t gw = (int64_t)blockIdx.x * (kGatherThreads / 64) + w;
  const int64_t nw = (int64_t)gridDim.x * (kGatherThreads / 64);
  gather_rows_res<ROWB>(g, gw, nw, r, qh[w], qd[w]);
}

}  // namespace

hipError_t launch_gather(const void* k_host, const void* v_host, int64_t n_max, int row_bytes,
                         const int32_t* idx, int m, const int32_t* cnt, int BH, void* k_dst,
                         void* v_dst, int64_t dst_rows_per_bh, int dst_row0, int max_wgs,
                         hipStream_t s, int run_shift) {
  const int64_t total = (int64_t)BH * m;
  if (total == 0) return hipSuccess;
  if ((total << run_shift) > kGatherMaxRows) return hipErrorInvalidValue;
  const int rpi = 64 / (row_bytes / 16);
  const int64_t rows_per_wg = (int64_t)rpi * kGatherUnroll * (kGatherThreads / 64);
  int64_t grid = ((total << run_shift) + rows_per_wg - 1) / rows_per_wg;
  const int cap = max_wgs > 0 ? max_wgs : kDefaultMaxWgs;
  if (grid > cap) grid = cap;
  const GatherJob g{static_cast<const uint8_t*>(k_host), static_cast<const uint8_t*>(v_host),
                    n_max, idx, m, cnt, total, static_cast<uint8_t*>(k_dst),
                    static_cast<uint8_t*>(v_dst), dst_rows_per_bh, dst_row0, run_shift,
                    row_bytes};
  switch (row_bytes) {
    case 128:
      hipLaunchKernelGGL(k_gather<128>, dim3((unsigned)grid), dim3(kGatherThreads), 0, s, g);
      break;
    case 256:
      hipLaunchKernelGGL(k_gather<256>, dim3((unsigned)grid), dim3(kGatherThreads), 0, s, g);
      break;
    default:
      hipLaunchKernelGGL(k_gather<512>, dim3((unsigned)grid), dim3(kGatherThreads), 0, s, g);
      break;
  }
  return hipGetLastError();
}

hipError_t launch_gather_resident(const void* v_host, int64_t n_max, int row_bytes,
                                  const int32_t* idx, int m, int BH, void* v_dst,
                                  int64_t dst_rows_per_bh, const GatherRes& r, int max_wgs,
                                  hipStream_t s) {
  const int64_t total = (int64_t)BH * m;
  if (total == 0) return hipSuccess;
  if (total > kGatherMaxRows || m > dst_rows_per_bh) return hipErrorInvalidValue;
  // A wave classifies 64 entries at a time.
  const int64_t rows_per_wg = 64 * (kGatherThreads / 64);
  int64_t grid = (total + rows_per_wg - 1) / rows_per_wg;
  const int cap = max_wgs > 0 ? max_wgs : kDefaultMaxWgs;
  if (grid > cap) grid = cap;
  const GatherJob g{nullptr, static_cast<const uint8_t*>(v_host), n_max, idx, m, nullptr, total,
                    nullptr, static_cast<uint8_t*>(v_dst), dst_rows_per_bh, 0, 0, row_bytes};
  switch (row_bytes) {
    case 128:
      hipLaunchKernelGGL(k_gather_resident<128>, dim3((unsigned)grid), dim3(kGatherThreads), 0, s,
                         g, r);
      break;
    case 256:
      hipLaunchKernelGGL(k_gather_resident<256>, dim3((unsigned)grid), dim3(kGatherThreads), 0, s,
                         g, r);
      break;
    default:
      hipLaunchKernelGGL(k_gather_resident<512>, dim3((unsigned)grid), dim3(kGatherThreads), 0, s,
                         g, r);
      break;
  }
  return hipGetLastError();
}

int gather_rows_per_wg(int row_bytes) {
  return (64 / (row_bytes / 16)) * kGatherUnroll * (kGatherThreads / 64);
}

}  // namespace dd
