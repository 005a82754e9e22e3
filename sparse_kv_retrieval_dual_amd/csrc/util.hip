// Device properties, the streaming-copy measurement kernel and a fill.
#include <mutex>

#include "dd_device.h"
#include "dd_internal.h"

namespace dd {

namespace {

constexpr int kMaxDevices = 64;
DeviceInfo g_info[kMaxDevices];
std::once_flag g_once[kMaxDevices];

// Grid-stride 16-byte copy: one read and one write per byte.
__global__ __launch_bounds__(256) void k_stream_copy(const u32x4* __restrict__ src,
                                                     u32x4* __restrict__ dst, int64_t n16) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const u32x4 a = __builtin_nontemporal_load(src + i);
    const u32x4 b = __builtin_nontemporal_load(src + i + stride);
    const u32x4 c = __builtin_nontemporal_load(src + i + 2 * stride);
    const u32x4 d = __builtin_nontemporal_load(src + i + 3 * stride);
    __builtin_nontemporal_store(a, dst + i);
    __builtin_nontemporal_store(b, dst + i + stride);
    __builtin_nontemporal_store(c, dst + i + 2 * stride);
    __builtin_nontemporal_store(d, dst + i + 3 * stride);
  }
  for (; i < n16; i += stride) __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

// Streaming read, the ceiling the scans are measured against: a one-shot
// grid whose workgroups read 16 KB each, every lane with 4 non-temporal
// 16-byte loads in flight (each load instruction of the workgroup covers
// 4 KB), folded into a xor; one word per wave goes to the 64-word sink so
// that the loads cannot be dropped (waves share sink words: the values are
// meaningless).  The fastest of the shapes swept on MI355X for 256 MiB read
// from HBM: 39.5 us, against 39.8-41.0 us for 8 or 16 loads per lane in
// 256- to 1024-thread workgroups or a persistent grid, 41.5 us for the
// scoring kernel's own shape (16 loads per lane, 64 KB per workgroup), and
// 43.6-46.1 us with plain loads.
constexpr int kReadUnroll = 4;
__global__ __launch_bounds__(256) void k_stream_read(const u32x4* __restrict__ src, int64_t n16,
                                                     uint32_t* __restrict__ sink) {
  const int64_t base = (int64_t)blockIdx.x * (256 * kReadUnroll) + threadIdx.x;
  u32x4 v[kReadUnroll];
#pragma unroll
  for (int u = 0; u < kReadUnroll; ++u) {
    const int64_t i = base + 256 * u;
    v[u] = __builtin_nontemporal_load(src + (i < n16 ? i : n16 - 1));
  }
  uint32_t acc = 0u;
#pragma unroll
  for (int u = 0; u < kReadUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
#pragma unroll
  for (int b = 1; b < 64; b <<= 1) acc ^= (uint32_t)__shfl_xor((int)acc, b);
  if ((threadIdx.x & 63) == 0) sink[(blockIdx.x * 4 + threadIdx.x / 64) & 63u] = acc;
}

// A fixed delay: one wave sleeps `rounds` times for the longest s_sleep
// (127 x 64 clocks) and exits; nothing else.  A bounded stall with which a
// test can perturb the timing of a stream.
__global__ __launch_bounds__(64) void k_delay(int rounds) {
  for (int i = 0; i < rounds; ++i) __builtin_amdgcn_s_sleep(127);
}

// Grid-stride fill of n 32-bit words with v.
__global__ __launch_bounds__(256) void k_fill_i32(int32_t* __restrict__ p, int32_t v, int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) p[i] = v;
}

}  // namespace

hipError_t launch_fill_i32(int32_t* p, int32_t v, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  int64_t grid = (n + 255) / 256;
  if (grid > 2048) grid = 2048;
  hipLaunchKernelGGL(k_fill_i32, dim3((unsigned)grid), dim3(256), 0, s, p, v, n);
  return hipGetLastError();
}

const DeviceInfo& device_info() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) dev = 0;
  std::call_once(g_once[dev], [dev]() {
    DeviceInfo di;
    di.device = dev;
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess) di.cus = v;
    v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) == hipSuccess &&
        v > 0)
      di.lds_per_block = v;
    g_info[dev] = di;
  });
  return g_info[dev];
}

hipError_t launch_stream_copy(const void* src, void* dst, size_t bytes, hipStream_t s) {
  const int64_t n16 = (int64_t)(bytes / 16);
  if (n16 == 0) return hipSuccess;
  const DeviceInfo& di = device_info();
  int64_t grid = (n16 + 255) / 256;
  const int64_t cap = (int64_t)(di.cus > 0 ? di.cus : 256) * 16;
  if (grid > cap) grid = cap;
  hipLaunchKernelGGL(k_stream_copy, dim3((unsigned)grid), dim3(256), 0, s,
                     static_cast<const u32x4*>(src), static_cast<u32x4*>(dst), n16);
  return hipGetLastError();
}

hipError_t launch_delay(int us, hipStream_t s) {
  if (us <= 0) return hipSuccess;
  // s_sleep 127 waits 127 x 64 = 8128 clocks, about 3.4 us at 2.4 GHz.
  const int rounds = (int)(((int64_t)us * 2400 + 8127) / 8128);
  hipLaunchKernelGGL(k_delay, dim3(1), dim3(64), 0, s, rounds);
  return hipGetLastError();
}

hipError_t launch_stream_read(const void* src, size_t bytes, void* sink, hipStream_t s) {
  const int64_t n16 = (int64_t)(bytes / 16);
  if (n16 == 0) return hipSuccess;
  const int64_t grid = (n16 + 256 * kReadUnroll - 1) / (256 * kReadUnroll);
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_stream_read, dim3((unsigned)grid), dim3(256), 0, s,
                     static_cast<const u32x4*>(src), n16, static_cast<uint32_t*>(sink));
  return hipGetLastError();
}

}  // namespace dd
