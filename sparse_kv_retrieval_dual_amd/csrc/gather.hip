// Row gather from the host-resident KV cache into device memory (arXiv page
// of DualDecoder, section 2.2 and Figure 1: the selected entries are
// noncontiguous in host memory and are gathered into the GPU before
// attention; the paper-daily worked example sizes one such transfer).
//
// The kernel reads pinned, device-mapped host rows directly over the host
// link: one row (128-512 B) is read by ROWB/16 lanes with 16-byte loads, and
// every wave keeps 4 row groups of K and V in flight, so a few hundred waves
// hold megabytes of reads outstanding, enough to cover the link's latency.
// Host reads are non-temporal; the device-side stores are plain.
#include <cstdlib>

#include "dd_device.h"
#include "dd_internal.h"

namespace dd {

namespace {

constexpr int kGatherThreads = 256;
constexpr int kGatherUnroll = 4;

template <int ROWB>
__global__ __launch_bounds__(kGatherThreads) void k_gather(
    const uint8_t* __restrict__ ksrc, const uint8_t* __restrict__ vsrc, int64_t n_max,
    const int32_t* __restrict__ idx, int m, const int32_t* __restrict__ cnt, int64_t total,
    uint8_t* __restrict__ kdst, uint8_t* __restrict__ vdst, int64_t dst_rows_per_bh,
    int dst_row0, const int32_t* __restrict__ counts, int BH, int64_t* __restrict__ stats) {
  constexpr int LPR = ROWB / 16;
  constexpr int RPI = 64 / LPR;
  constexpr int U = kGatherUnroll;
  const int lane = threadIdx.x & 63;
  const int col = lane % LPR;
  const int rsub = lane / LPR;
  const int64_t gw = (int64_t)blockIdx.x * (kGatherThreads / 64) + (threadIdx.x >> 6);
  const int64_t nw = (int64_t)gridDim.x * (kGatherThreads / 64);

  // Loads are issued unconditionally so that all of them are in flight at
  // once; a lane without a host row to fetch reads a stand-in address in
  // device memory (its own destination slot) and its data is discarded.
  const u32x4 zero = u32x4{0u, 0u, 0u, 0u};
  const bool has_k = ksrc != nullptr;
  const bool has_v = vsrc != nullptr;
  for (int64_t base = gw * (RPI * U); base < total; base += nw * (RPI * U)) {
    const uint8_t* kp[U];
    const uint8_t* vp[U];
    int64_t doff[U];
    bool wr[U], fetch[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      int64_t r = base + u * RPI + rsub;
      wr[u] = r < total;
      if (!wr[u]) r = total - 1;
      const int64_t bh = r / m;
      const int j = (int)(r - bh * m);
      int lim = m;
      if (cnt != nullptr) {
        const int c = cnt[bh];
        lim = c < 0 ? 0 : (c > m ? m : c);
      }
      wr[u] = wr[u] && j < lim;
      doff[u] = (bh * dst_rows_per_bh + dst_row0 + j) * ROWB + col * 16;
      const int32_t ir = idx[r];
      const int32_t i = wr[u] ? ir : -1;
      fetch[u] = i >= 0 && (int64_t)i < n_max;
      const int64_t soff = (bh * n_max + (fetch[u] ? i : 0)) * ROWB + col * 16;
      kp[u] = (fetch[u] && has_k) ? ksrc + soff : kdst + (has_k ? doff[u] : 0);
      vp[u] = (fetch[u] && has_v) ? vsrc + soff : vdst + (has_v ? doff[u] : 0);
    }
    u32x4 kv[U], vv[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (has_k) kv[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kp[u]));
      if (has_v) vv[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(vp[u]));
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (wr[u]) {
        if (has_k) *reinterpret_cast<u32x4*>(kdst + doff[u]) = fetch[u] ? kv[u] : zero;
        if (has_v) *reinterpret_cast<u32x4*>(vdst + doff[u]) = fetch[u] ? vv[u] : zero;
      }
    }
  }

  if (stats != nullptr && blockIdx.x == 0) {
    __shared__ unsigned long long s_acc[3];
    if (threadIdx.x < 3) s_acc[threadIdx.x] = 0ull;
    __syncthreads();
    unsigned long long a0 = 0, a1 = 0, a2 = 0;
    for (int t = threadIdx.x; t < BH; t += kGatherThreads) {
      a0 += (unsigned long long)counts[t];
      a1 += (unsigned long long)counts[BH + t];
      a2 += (unsigned long long)counts[2 * BH + t];
    }
    atomicAdd(&s_acc[0], a0);
    atomicAdd(&s_acc[1], a1);
    atomicAdd(&s_acc[2], a2);
    __syncthreads();
    if (threadIdx.x == 0) {
      stats[0] = (int64_t)s_acc[0];
      stats[1] = (int64_t)s_acc[1];
      stats[2] = (int64_t)(s_acc[2] + s_acc[0]);
    }
  }
}

int gather_grid(int64_t total, int row_bytes) {
  const int rpi = 64 / (row_bytes / 16);
  const int64_t rows_per_wg = (int64_t)rpi * kGatherUnroll * (kGatherThreads / 64);
  int64_t want = (total + rows_per_wg - 1) / rows_per_wg;
  static int cap = -1;
  if (cap < 0) {
    const char* e = getenv("DD_GATHER_WGS");
    cap = (e != nullptr && atoi(e) > 0) ? atoi(e) : 1024;
  }
  if (want > cap) want = cap;
  if (want < 1) want = 1;
  return (int)want;
}

}  // namespace

hipError_t launch_gather(const void* k_host, const void* v_host, int64_t n_max, int row_bytes,
                         const int32_t* idx, int m, const int32_t* cnt, int BH, void* k_dst,
                         void* v_dst, int64_t dst_rows_per_bh, int dst_row0,
                         const int32_t* counts, int64_t* stats, hipStream_t s) {
  const int64_t total = (int64_t)BH * m;
  if (total == 0 && stats == nullptr) return hipSuccess;
  const int grid = gather_grid(total, row_bytes);
  const uint8_t* ks = static_cast<const uint8_t*>(k_host);
  const uint8_t* vs = static_cast<const uint8_t*>(v_host);
  uint8_t* kd = static_cast<uint8_t*>(k_dst);
  uint8_t* vd = static_cast<uint8_t*>(v_dst);
  const int mm = m > 0 ? m : 1;
  switch (row_bytes) {
    case 128:
      hipLaunchKernelGGL(k_gather<128>, dim3(grid), dim3(kGatherThreads), 0, s, ks, vs, n_max, idx,
                         mm, cnt, total, kd, vd, dst_rows_per_bh, dst_row0, counts, BH, stats);
      break;
    case 256:
      hipLaunchKernelGGL(k_gather<256>, dim3(grid), dim3(kGatherThreads), 0, s, ks, vs, n_max, idx,
                         mm, cnt, total, kd, vd, dst_rows_per_bh, dst_row0, counts, BH, stats);
      break;
    default:
      hipLaunchKernelGGL(k_gather<512>, dim3(grid), dim3(kGatherThreads), 0, s, ks, vs, n_max, idx,
                         mm, cnt, total, kd, vd, dst_rows_per_bh, dst_row0, counts, BH, stats);
      break;
  }
  return hipGetLastError();
}

}  // namespace dd
