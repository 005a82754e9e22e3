// Decode attention over the gathered rows only ("Attention" box of Figure 1
// on the arXiv page of DualDecoder, fed by the sparse KV rows), split over
// chunks of selected entries with an online (log-sum-exp) softmax.
//
// One 256-thread workgroup per (b, h, chunk of 128 entries); each wave owns
// 32 entries.  A row is read by LPR lanes, 16 B each; every lane issues its
// K and V loads for all of its entries at once (one memory round trip), the
// dot products are summed across the LPR lanes by a DPP butterfly that
// leaves every lane with all of its entries' logits, and the wave forms its
// own max, weights and weighted V sum without a workgroup barrier.  The
// four waves are merged in LDS by log-sum-exp.  A chunk's (max, sum of
// weights, weighted V) goes to the workspace and a small kernel merges the
// chunks; with a single chunk the first kernel finishes the output itself.
// Every reduction runs in the order of the entry number j, never of the
// row it is stored in, so the result does not depend on where rows sit.
#include "dd_device.h"
#include "dd_internal.h"

namespace dd {

namespace {

constexpr int kAttnThreads = 256;
constexpr int kAttnWaves = kAttnThreads / 64;
constexpr int kWaveEntries = 32;
constexpr int kChunk = kAttnWaves * kWaveEntries;
constexpr float kLog2e = 1.4426950408889634f;

template <typename T, int D>
struct AttnShape {
  static constexpr int EPL = 16 / (int)sizeof(T);  // elements per lane per load
  static constexpr int LPR = D / EPL;              // lanes per row
  static constexpr int RPI = 64 / LPR;             // rows per wave load instruction
  static constexpr int U = kWaveEntries / RPI;     // entries (K and V loads) per lane
  static_assert(U >= 1 && U * RPI == kWaveEntries, "shape");
};

// All-reduce of NV values over aligned groups of G lanes.
template <int G, int NV>
__device__ __forceinline__ void group_allreduce(float* x) {
  if constexpr (G > 1) {
    constexpr int HALF = G / 2;
#pragma unroll
    for (int v = 0; v < NV; ++v) x[v] += partner<HALF>(x[v]);
    group_allreduce<HALF, NV>(x);
  }
}

// Sums the per-slab counts of the layer step (misses, hits, fetchable
// prediction entries) into stats = {misses, hits, rows over the host link}.
__device__ __forceinline__ void write_stats(const int32_t* __restrict__ counts, int BH,
                                            int64_t* __restrict__ stats) {
  __shared__ unsigned long long s_acc[3];
  if (threadIdx.x < 3) s_acc[threadIdx.x] = 0ull;
  __syncthreads();
  unsigned long long a0 = 0, a1 = 0, a2 = 0;
  for (int t = threadIdx.x; t < BH; t += blockDim.x) {
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

template <typename T, int D>
__global__ __launch_bounds__(kAttnThreads) void k_attn_partial(
    const float* __restrict__ q, int64_t q_stride, const T* __restrict__ krows,
    const T* __restrict__ vrows, const int32_t* __restrict__ pos, const int32_t* __restrict__ cnt,
    int BH, int k, int m, int chunks, float scale, float* __restrict__ out,
    float* __restrict__ lse, float* __restrict__ part, const int32_t* __restrict__ counts,
    int64_t* __restrict__ stats, AttnMiss ms) {
  using S = AttnShape<T, D>;
  __shared__ float s_m[kAttnWaves];
  __shared__ float s_l[kAttnWaves];
  __shared__ float s_o[kAttnWaves][D];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  if (stats != nullptr && blockIdx.x == 0) write_stats(counts, BH, stats);
  int bh, c;
  xcd_tile_map(blockIdx.x, chunks, BH, bh, c);
  int lim = k;
  if (cnt != nullptr) {
    const int cc = cnt[bh];
    lim = cc < 0 ? 0 : (cc > k ? k : cc);
  }
  const int col = lane % S::LPR;
  const int rsub = lane / S::LPR;
  const int e0 = c * kChunk + wave * kWaveEntries;  // this wave's first entry

  // Rows of this lane's entries e0 + u*RPI + rsub (-1: skipped), and for a
  // row past first_miss_row the host row it is fetched from.
  const bool from_host = ms.k_host != nullptr;
  int rows[S::U];
  int hrow[S::U];
#pragma unroll
  for (int u = 0; u < S::U; ++u) {
    const int j = e0 + u * S::RPI + rsub;
    int r = -1, c = -1;
    if (j < lim && m > 0) {
      r = (pos != nullptr) ? pos[(int64_t)bh * k + j] : j;
      if (r < 0 || r >= m) r = -1;
      if (from_host) c = ms.cur[(int64_t)bh * k + j];
    }
    if (r >= ms.first_miss_row && from_host) {
      if (c < 0 || (int64_t)c >= ms.n_max) r = -1;
    } else {
      c = -1;
    }
    rows[u] = r;
    hrow[u] = r >= 0 ? c : -1;
  }
  // K and V of every entry in flight together (slot rows from HBM, missed
  // rows over the host link); a skipped entry reads row 0 of the slab (when
  // there is one) and is masked below.
  const T* kb = krows + (int64_t)bh * m * D + col * S::EPL;
  const T* vb = vrows + (int64_t)bh * m * D + col * S::EPL;
  const T* khb = from_host ? static_cast<const T*>(ms.k_host) + (int64_t)bh * ms.n_max * D + col * S::EPL : kb;
  const T* vhb = from_host ? static_cast<const T*>(ms.v_host) + (int64_t)bh * ms.n_max * D + col * S::EPL : vb;
  const u32x4 zero = u32x4{0u, 0u, 0u, 0u};
  u32x4 kr[S::U], vr[S::U];
  if (m > 0) {
#pragma unroll
    for (int u = 0; u < S::U; ++u) {
      const bool h = hrow[u] >= 0;
      const int64_t off = (int64_t)(h ? hrow[u] : (rows[u] >= 0 ? rows[u] : 0)) * D;
      kr[u] = *reinterpret_cast<const u32x4*>((h ? khb : kb) + off);
      vr[u] = *reinterpret_cast<const u32x4*>((h ? vhb : vb) + off);
    }
    if (from_host) {  // the slot keeps a copy of every fetched miss
#pragma unroll
      for (int u = 0; u < S::U; ++u) {
        if (hrow[u] >= 0) {
          T* kd = const_cast<T*>(kb) + (int64_t)rows[u] * D;
          T* vd = const_cast<T*>(vb) + (int64_t)rows[u] * D;
          *reinterpret_cast<u32x4*>(kd) = kr[u];
          *reinterpret_cast<u32x4*>(vd) = vr[u];
        }
      }
    }
  } else {
#pragma unroll
    for (int u = 0; u < S::U; ++u) kr[u] = vr[u] = zero;
  }
  float qr[S::EPL];
#pragma unroll
  for (int e = 0; e < S::EPL; ++e) qr[e] = q[(int64_t)bh * q_stride + col * S::EPL + e];

  float s[S::U];
#pragma unroll
  for (int u = 0; u < S::U; ++u) {
    float f[S::EPL];
    Unpack<T>::run(kr[u], f);
    float a = 0.f;
#pragma unroll
    for (int e = 0; e < S::EPL; ++e) a = fmaf(f[e], qr[e], a);
    s[u] = a;
  }
  group_allreduce<S::LPR, S::U>(s);

  // Wave-local softmax over its 32 entries (RPI row groups x U).
  float mx = -INFINITY;
#pragma unroll
  for (int u = 0; u < S::U; ++u) {
    s[u] = (rows[u] >= 0) ? s[u] * scale : -INFINITY;
    mx = fmaxf(mx, s[u]);
  }
#pragma unroll
  for (int off = S::LPR; off < 64; off <<= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
  float l = 0.f;
  float o[S::EPL];
#pragma unroll
  for (int e = 0; e < S::EPL; ++e) o[e] = 0.f;
#pragma unroll
  for (int u = 0; u < S::U; ++u) {
    const float w = (rows[u] >= 0) ? exp2f((s[u] - mx) * kLog2e) : 0.f;
    l += w;
    float f[S::EPL];
    Unpack<T>::run(rows[u] >= 0 ? vr[u] : zero, f);
#pragma unroll
    for (int e = 0; e < S::EPL; ++e) o[e] = fmaf(w, f[e], o[e]);
  }
#pragma unroll
  for (int off = S::LPR; off < 64; off <<= 1) {
    l += __shfl_xor(l, off);
#pragma unroll
    for (int e = 0; e < S::EPL; ++e) o[e] += __shfl_xor(o[e], off);
  }
  if (rsub == 0) {
#pragma unroll
    for (int e = 0; e < S::EPL; ++e) s_o[wave][col * S::EPL + e] = o[e];
    if (col == 0) {
      s_m[wave] = mx;
      s_l[wave] = l;
    }
  }
  __syncthreads();

  // Merge the waves (entry order is fixed: wave 0, 1, 2, 3).
  float cm = -INFINITY;
#pragma unroll
  for (int w = 0; w < kAttnWaves; ++w) cm = fmaxf(cm, s_m[w]);
  float f[kAttnWaves];
  float cl = 0.f;
#pragma unroll
  for (int w = 0; w < kAttnWaves; ++w) {
    f[w] = (s_l[w] > 0.f) ? exp2f((s_m[w] - cm) * kLog2e) : 0.f;
    cl += s_l[w] * f[w];
  }
  for (int d = threadIdx.x; d < D; d += kAttnThreads) {
    float od = 0.f;
#pragma unroll
    for (int w = 0; w < kAttnWaves; ++w) od += s_o[w][d] * f[w];
    if (chunks == 1) {
      out[(int64_t)bh * D + d] = (cl > 0.f) ? od / cl : 0.f;
      if (d == 0 && lse != nullptr) lse[bh] = (cl > 0.f) ? cm + logf(cl) : -INFINITY;
    } else {
      float* p = part + ((int64_t)bh * chunks + c) * (D + 2);
      p[d] = od;
      if (d == 0) {
        p[D] = cl > 0.f ? cm : -INFINITY;
        p[D + 1] = cl;
      }
    }
  }
}

// Merge of the chunk partials of one (b, h) by log-sum-exp.
template <int D>
__global__ __launch_bounds__(D) void k_attn_combine(const float* __restrict__ part, int chunks,
                                                    float* __restrict__ out,
                                                    float* __restrict__ lse) {
  const int bh = blockIdx.x;
  const int d = threadIdx.x;
  const float* p = part + (int64_t)bh * chunks * (D + 2);
  float mx = -INFINITY;
  for (int c = 0; c < chunks; ++c) mx = fmaxf(mx, p[c * (D + 2) + D]);
  float tot = 0.f, od = 0.f;
  if (mx > -INFINITY) {
    for (int c = 0; c < chunks; ++c) {
      const float* pc = p + c * (D + 2);
      const float wsum = pc[D + 1];
      if (wsum > 0.f) {
        const float f = exp2f((pc[D] - mx) * kLog2e);
        tot += wsum * f;
        od += pc[d] * f;
      }
    }
  }
  out[(int64_t)bh * D + d] = (tot > 0.f) ? od / tot : 0.f;
  if (d == 0 && lse != nullptr) lse[bh] = (tot > 0.f) ? mx + logf(tot) : -INFINITY;
}

struct AttnLaunch {
  const float* q;
  int64_t q_stride;
  const void* kr;
  const void* vr;
  const int32_t* pos;
  const int32_t* cnt;
  int BH, k, m;
  float scale;
  float* out;
  float* lse;
  void* ws;
  const int32_t* counts;
  int64_t* stats;
  AttnMiss miss;
  hipStream_t s;
};

template <typename T, int D>
hipError_t launch_attn_t(const AttnLaunch& a) {
  const int chunks = (a.k + kChunk - 1) / kChunk;
  float* part = static_cast<float*>(a.ws);
  hipLaunchKernelGGL((k_attn_partial<T, D>), dim3(a.BH * chunks), dim3(kAttnThreads), 0, a.s,
                     a.q, a.q_stride, static_cast<const T*>(a.kr), static_cast<const T*>(a.vr),
                     a.pos, a.cnt, a.BH, a.k, a.m, chunks, a.scale, a.out, a.lse, part, a.counts,
                     a.stats, a.miss);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || chunks == 1) return e;
  hipLaunchKernelGGL((k_attn_combine<D>), dim3(a.BH), dim3(D), 0, a.s, part, chunks, a.out, a.lse);
  return hipGetLastError();
}

}  // namespace

size_t attn_workspace(int B, int H, int k, int D) {
  const int chunks = (k + kChunk - 1) / kChunk;
  if (chunks <= 1) return 0;
  return (size_t)B * H * chunks * (D + 2) * sizeof(float);
}

hipError_t launch_attn(const float* q, int64_t q_stride_bh, const void* k_rows,
                       const void* v_rows, const int32_t* pos, const int32_t* cnt, int B, int H,
                       int k, int m, int D, int dtype, float scale, float* out, float* lse,
                       void* ws, const int32_t* counts, int64_t* stats, const AttnMiss* miss,
                       hipStream_t s) {
  const int BH = B * H;
  if (BH == 0) return hipSuccess;
  AttnLaunch a{q, q_stride_bh, k_rows, v_rows, pos, cnt, BH, k, m, scale, out, lse, ws, counts,
               stats, AttnMiss{nullptr, nullptr, nullptr, 0, 0}, s};
  if (miss != nullptr && miss->k_host != nullptr && miss->v_host != nullptr && miss->cur != nullptr)
    a.miss = *miss;
  if (dtype == kBF16) {
    if (D == 128) return launch_attn_t<uint16_t, 128>(a);
    return launch_attn_t<uint16_t, 64>(a);
  }
  if (D == 128) return launch_attn_t<float, 128>(a);
  return launch_attn_t<float, 64>(a);
}

}  // namespace dd
