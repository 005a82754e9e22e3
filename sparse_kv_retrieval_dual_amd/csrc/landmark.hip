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
// rows of a chunk are loaded 8 at a time, all in flight together, with
// non-temporal loads (every key row is read once): 60.6 -> 52.4 us for the
// 7B layer's 256 MiB of keys at c = 8 on MI355X.  The landmarks are stored
// plainly (non-temporal stores took 65.4 us).
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
      raw[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(base + i * D));
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

// One wave per (b, h): the new token's K and V rows (LPR lanes, 16 B each)
// go to row lens[b] of the device keys and of both host planes; with
// landmarks, the landmark of the chunk holding that row is recomputed from
// the chunk's earlier rows (device copy) and the new row, summed in the
// same row order as k_landmarks.  A request whose length is outside
// [0, n_max) is left as it is.
template <typename T, int D>
__global__ __launch_bounds__(64) void k_kv_append(T* __restrict__ k_dev, T* __restrict__ k_host,
                                                  T* __restrict__ v_host,
                                                  const T* __restrict__ new_k,
                                                  const T* __restrict__ new_v,
                                                  const int32_t* __restrict__ lens,
                                                  int32_t* __restrict__ lens_out, int H,
                                                  int64_t n_max, int cs,
                                                  float* __restrict__ landmarks, int64_t nc_max) {
  constexpr int EPL = 16 / (int)sizeof(T);
  constexpr int LPR = D / EPL;
  const int bh = blockIdx.x;
  const int b = bh / H;
  const int lane = threadIdx.x;
  const int32_t len = lens[b];
  const bool ok = len >= 0 && (int64_t)len < n_max;
  if (lens_out != nullptr && bh % H == 0 && lane == 0) lens_out[b] = ok ? len + 1 : len;
  if (!ok || lane >= LPR) return;
  const int64_t src = (int64_t)bh * D + lane * EPL;
  const int64_t dst = ((int64_t)bh * n_max + len) * D + lane * EPL;
  const u32x4 nk = *reinterpret_cast<const u32x4*>(new_k + src);
  const u32x4 nv = *reinterpret_cast<const u32x4*>(new_v + src);
  *reinterpret_cast<u32x4*>(k_dev + dst) = nk;
  *reinterpret_cast<u32x4*>(k_host + dst) = nk;
  *reinterpret_cast<u32x4*>(v_host + dst) = nv;
  if (landmarks == nullptr) return;
  const int64_t e = (int64_t)len >> cs;
  const int64_t r0 = e << cs;
  float acc[EPL];
#pragma unroll
  for (int x = 0; x < EPL; ++x) acc[x] = 0.f;
  for (int64_t r = r0; r < len; ++r) {
    float f[EPL];
    Unpack<T>::run(*reinterpret_cast<const u32x4*>(k_dev + ((int64_t)bh * n_max + r) * D + lane * EPL), f);
#pragma unroll
    for (int x = 0; x < EPL; ++x) acc[x] += f[x];
  }
  float f[EPL];
  Unpack<T>::run(nk, f);
#pragma unroll
  for (int x = 0; x < EPL; ++x) acc[x] += f[x];
  const float n = (float)(len - r0 + 1);
  float* o = landmarks + ((int64_t)bh * nc_max + e) * D + lane * EPL;
#pragma unroll
  for (int x = 0; x < EPL; x += 4) {
    f32x4_t v;
    v.x = acc[x] / n;
    v.y = acc[x + 1] / n;
    v.z = acc[x + 2] / n;
    v.w = acc[x + 3] / n;
    *reinterpret_cast<f32x4_t*>(o + x) = v;
  }
}

template <typename T, int D>
hipError_t launch_kv_append_t(void* k_dev, void* k_host, void* v_host, const void* new_k,
                              const void* new_v, const int32_t* lens, int32_t* lens_out, int BH,
                              int H, int64_t n_max, int cs, float* landmarks, hipStream_t s) {
  const int64_t nc_max = (n_max + ((int64_t)1 << cs) - 1) >> cs;
  hipLaunchKernelGGL((k_kv_append<T, D>), dim3(BH), dim3(64), 0, s, static_cast<T*>(k_dev),
                     static_cast<T*>(k_host), static_cast<T*>(v_host),
                     static_cast<const T*>(new_k), static_cast<const T*>(new_v), lens, lens_out,
                     H, n_max, cs, landmarks, nc_max);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_kv_append(void* k_dev, void* k_host, void* v_host, const void* new_k,
                            const void* new_v, const int32_t* lens, int32_t* lens_out, int B,
                            int H, int D, int64_t n_max, int dtype, int chunk_shift,
                            float* landmarks, hipStream_t s) {
  const int BH = B * H;
  if (BH == 0) return hipSuccess;
  if (dtype == kBF16) {
    if (D == 128)
      return launch_kv_append_t<uint16_t, 128>(k_dev, k_host, v_host, new_k, new_v, lens, lens_out,
                                               BH, H, n_max, chunk_shift, landmarks, s);
    return launch_kv_append_t<uint16_t, 64>(k_dev, k_host, v_host, new_k, new_v, lens, lens_out,
                                            BH, H, n_max, chunk_shift, landmarks, s);
  }
  if (D == 128)
    return launch_kv_append_t<float, 128>(k_dev, k_host, v_host, new_k, new_v, lens, lens_out, BH,
                                          H, n_max, chunk_shift, landmarks, s);
  return launch_kv_append_t<float, 64>(k_dev, k_host, v_host, new_k, new_v, lens, lens_out, BH, H,
                                       n_max, chunk_shift, landmarks, s);
}

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
