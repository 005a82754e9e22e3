// Chunk landmarks: the compressed per-chunk keys from which the GPU picks
// the important chunks (arXiv page of DualDecoder, section 2.2, on
// ShadowKV's chunk landmarks).  The pages do not define a landmark; here it
// is the mean of the chunk's valid keys, summed in fp32 in row order and
// divided by their count.
//
// HBM-bound: every valid key row is read once (256 B for bf16 D = 128) and
// one fp32 row of D elements is written per chunk.  A chunk is handled by
// LPR lanes (16 B of each row per lane), so a wave covers 64 / LPR chunks
// and each of its load instructions reads one row of each of them.  The
// rows of a chunk are loaded 8 at a time, all in flight together.
#include "dd_device.h"
#include "dd_internal.h"

namespace dd {

namespace {

typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kLmThreads = 256;
constexpr int kLmBatch = 8;  // rows of a chunk in flight per lane

template <typename T, int D>
__global__ __launch_bounds__(kLmThreads) void k_landmarks(const T* __restrict__ keys,
                                                          const int32_t* __restrict__ lens,
                                                          int BH, int H, int64_t n_max,
                                                          int64_t nc_max, int cs,
                                                          float* __restrict__ out) {
  constexpr int EPL = 16 / (int)sizeof(T);
  constexpr int LPR = D / EPL;
  const int64_t t = (int64_t)blockIdx.x * kLmThreads + threadIdx.x;
  const int64_t per_bh = nc_max * LPR;
  const int64_t bh = t / per_bh;
  if (bh >= BH) return;
  const int64_t rem = t - bh * per_bh;
  const int64_t e = rem / LPR;
  const int col = (int)(rem - e * LPR);
  const int64_t len = clamp_len(lens[bh / H], n_max);
  const int64_t r0 = e << cs;
  int64_t cnt = len - r0;
  const int64_t c = (int64_t)1 << cs;
  cnt = cnt < 0 ? 0 : (cnt > c ? c : cnt);

  float acc[EPL];
#pragma unroll
  for (int x = 0; x < EPL; ++x) acc[x] = 0.f;
  const T* base = keys + (bh * n_max + r0) * D + col * EPL;
  for (int64_t i0 = 0; i0 < cnt; i0 += kLmBatch) {
    u32x4 raw[kLmBatch];
#pragma unroll
    for (int u = 0; u < kLmBatch; ++u) {
      const int64_t i = i0 + u < cnt ? i0 + u : cnt - 1;  // stays inside the chunk's valid rows
      raw[u] = *reinterpret_cast<const u32x4*>(base + i * D);
    }
#pragma unroll
    for (int u = 0; u < kLmBatch; ++u) {
      if (i0 + u < cnt) {
        float f[EPL];
        Unpack<T>::run(raw[u], f);
#pragma unroll
        for (int x = 0; x < EPL; ++x) acc[x] += f[x];
      }
    }
  }
  float* o = out + (bh * nc_max + e) * D + col * EPL;
  const float n = (float)cnt;
#pragma unroll
  for (int x = 0; x < EPL; x += 4) {
    f32x4_t v;
    v.x = cnt > 0 ? acc[x] / n : 0.f;
    v.y = cnt > 0 ? acc[x + 1] / n : 0.f;
    v.z = cnt > 0 ? acc[x + 2] / n : 0.f;
    v.w = cnt > 0 ? acc[x + 3] / n : 0.f;
    *reinterpret_cast<f32x4_t*>(o + x) = v;
  }
}

template <typename T, int D>
hipError_t launch_landmarks_t(const void* keys, const int32_t* lens, int BH, int H, int64_t n_max,
                              int cs, float* out, hipStream_t s) {
  constexpr int LPR = D / (16 / (int)sizeof(T));
  const int64_t nc_max = (n_max + ((int64_t)1 << cs) - 1) >> cs;
  const int64_t threads = (int64_t)BH * nc_max * LPR;
  if (threads == 0) return hipSuccess;
  const int64_t grid = (threads + kLmThreads - 1) / kLmThreads;
  if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((k_landmarks<T, D>), dim3((unsigned)grid), dim3(kLmThreads), 0, s,
                     static_cast<const T*>(keys), lens, BH, H, n_max, nc_max, cs, out);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_landmarks(const void* keys, const int32_t* lens, int B, int H, int D,
                            int64_t n_max, int chunk_shift, int dtype, float* out, hipStream_t s) {
  const int BH = B * H;
  if (dtype == kBF16) {
    if (D == 128) return launch_landmarks_t<uint16_t, 128>(keys, lens, BH, H, n_max, chunk_shift, out, s);
    return launch_landmarks_t<uint16_t, 64>(keys, lens, BH, H, n_max, chunk_shift, out, s);
  }
  if (D == 128) return launch_landmarks_t<float, 128>(keys, lens, BH, H, n_max, chunk_shift, out, s);
  return launch_landmarks_t<float, 64>(keys, lens, BH, H, n_max, chunk_shift, out, s);
}

}  // namespace dd
