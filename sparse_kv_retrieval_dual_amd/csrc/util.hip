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

}  // namespace dd
