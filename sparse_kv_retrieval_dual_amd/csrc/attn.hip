// Decode attention over the gathered rows only ("Attention" box of Figure 1
// on the arXiv page of DualDecoder, fed by the sparse KV rows), split over
// row chunks with an online softmax.
//
// One 256-thread workgroup per (b, h, chunk of 128 selected entries).  The
// chunk's row numbers go to LDS; pass 1 streams the K rows (LPR lanes per
// row, butterfly-reduced dot products) and leaves the scaled logits in LDS;
// the chunk max and the weights exp(s - max) follow in LDS; pass 2 streams
// the V rows and accumulates sum_j w_j V_j per column slice.  A chunk's
// (max, sum of weights, weighted V) goes to the workspace and a small kernel
// merges the chunks by log-sum-exp.  With a single chunk the first kernel
// finishes the output itself.  Every reduction runs in the order of the
// entry number j, never of the row it is stored in, so the result does not
// depend on where the rows sit.
#include "dd_device.h"
#include "dd_internal.h"

namespace dd {

namespace {

constexpr int kAttnThreads = 256;
constexpr int kAttnWaves = kAttnThreads / 64;
constexpr int kChunk = 128;
constexpr float kLog2e = 1.4426950408889634f;

template <typename T, int D>
struct AttnShape {
  static constexpr int EPL = 16 / (int)sizeof(T);
  static constexpr int LPR = D / EPL;
  static constexpr int RPI = 64 / LPR;                 // rows per wave load
  static constexpr int ROWS_PER_WAVE = kChunk / kAttnWaves;
  static constexpr int U1 = ROWS_PER_WAVE / RPI;       // pass-1 loads per lane
  static constexpr int NG = kAttnWaves * RPI;          // pass-2 row groups
  static constexpr int U2 = kChunk / NG;               // pass-2 loads per lane
  static_assert(U1 >= 1 && U1 <= LPR, "pass-1 shape");
  static_assert(U2 >= 1, "pass-2 shape");
};

template <typename T, int D>
__global__ __launch_bounds__(kAttnThreads) void k_attn_partial(
    const float* __restrict__ q, int64_t q_stride, const T* __restrict__ krows,
    const T* __restrict__ vrows, const int32_t* __restrict__ pos, const int32_t* __restrict__ cnt,
    int BH, int k, int m, int chunks, float scale, float* __restrict__ out,
    float* __restrict__ lse, float* __restrict__ part) {
  using S = AttnShape<T, D>;
  __shared__ int s_row[kChunk];
  __shared__ float s_w[kChunk];
  __shared__ float s_red[2 * kAttnWaves];
  __shared__ float s_o[kAttnWaves][D];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  int bh, c;
  xcd_tile_map(blockIdx.x, chunks, BH, bh, c);
  if (m <= 0) {  // no rows at all: nothing takes part
    for (int d = threadIdx.x; d < D; d += kAttnThreads) {
      if (chunks == 1) {
        out[(int64_t)bh * D + d] = 0.f;
        if (d == 0 && lse != nullptr) lse[bh] = -INFINITY;
      } else {
        float* p = part + ((int64_t)bh * chunks + c) * (D + 2);
        p[d] = 0.f;
        if (d == 0) {
          p[D] = -INFINITY;
          p[D + 1] = 0.f;
        }
      }
    }
    return;
  }
  int lim = k;
  if (cnt != nullptr) {
    const int cc = cnt[bh];
    lim = cc < 0 ? 0 : (cc > k ? k : cc);
  }
  const int j0 = c * kChunk;
  for (int t = threadIdx.x; t < kChunk; t += kAttnThreads) {
    const int j = j0 + t;
    int r = -1;
    if (j < lim) {
      r = (pos != nullptr) ? pos[(int64_t)bh * k + j] : j;
      if (r < 0 || r >= m) r = -1;
    }
    s_row[t] = r;
  }
  __syncthreads();

  const int col = lane % S::LPR;
  const int rsub = lane / S::LPR;
  const T* kb = krows + (int64_t)bh * m * D + col * S::EPL;
  const T* vb = vrows + (int64_t)bh * m * D + col * S::EPL;

  // Pass 1: logits of this wave's 32 entries.
  {
    float qr[S::EPL];
#pragma unroll
    for (int e = 0; e < S::EPL; ++e) qr[e] = q[(int64_t)bh * q_stride + col * S::EPL + e];
    const int t0 = wave * S::ROWS_PER_WAVE;
    // Skipped entries load row 0 (m >= 1 here) so that every load is issued
    // unconditionally; their logits are replaced by -inf below.
    u32x4 raw[S::U1];
#pragma unroll
    for (int u = 0; u < S::U1; ++u) {
      const int r = s_row[t0 + u * S::RPI + rsub];
      raw[u] = *reinterpret_cast<const u32x4*>(kb + (int64_t)(r >= 0 ? r : 0) * D);
    }
    float acc[S::U1];
#pragma unroll
    for (int u = 0; u < S::U1; ++u) {
      float f[S::EPL];
      Unpack<T>::run(raw[u], f);
      float a = 0.f;
#pragma unroll
      for (int e = 0; e < S::EPL; ++e) a = fmaf(f[e], qr[e], a);
      acc[u] = a;
    }
    Butterfly<S::LPR, S::U1>::run(acc, lane);
    constexpr int REP = S::LPR / S::U1;  // lanes holding the same total
    if ((col % REP) == 0) {
      const int t = t0 + (col / REP) * S::RPI + rsub;
      s_w[t] = (s_row[t] >= 0) ? acc[0] * scale : -INFINITY;
    }
  }
  __syncthreads();

  // Chunk max, weights and their sum.
  float mx = -INFINITY;
  for (int t = threadIdx.x; t < kChunk; t += kAttnThreads) mx = fmaxf(mx, s_w[t]);
  mx = wave_max(mx);
  if (lane == 0) s_red[wave] = mx;
  __syncthreads();
  mx = -INFINITY;
#pragma unroll
  for (int w = 0; w < kAttnWaves; ++w) mx = fmaxf(mx, s_red[w]);
  float wsum = 0.f;
  for (int t = threadIdx.x; t < kChunk; t += kAttnThreads) {
    const float w = (s_row[t] >= 0) ? exp2f((s_w[t] - mx) * kLog2e) : 0.f;
    s_w[t] = w;
    wsum += w;
  }
  wsum = wave_sum(wsum);
  if (lane == 0) s_red[kAttnWaves + wave] = wsum;
  __syncthreads();
  wsum = 0.f;
#pragma unroll
  for (int w = 0; w < kAttnWaves; ++w) wsum += s_red[kAttnWaves + w];

  // Pass 2: weighted sum of V rows.  Row group g takes entries g, g+NG, ...
  float o[S::EPL];
#pragma unroll
  for (int e = 0; e < S::EPL; ++e) o[e] = 0.f;
  {
    const int g = wave * S::RPI + rsub;
    u32x4 raw[S::U2];
    int rows[S::U2];
#pragma unroll
    for (int u = 0; u < S::U2; ++u) {
      rows[u] = s_row[g + u * S::NG];
      raw[u] = *reinterpret_cast<const u32x4*>(vb + (int64_t)(rows[u] >= 0 ? rows[u] : 0) * D);
    }
#pragma unroll
    for (int u = 0; u < S::U2; ++u) {
      const float w = s_w[g + u * S::NG];
      // A skipped entry has weight 0; zero its stand-in row too so that a
      // non-finite value there cannot turn 0 * x into NaN.
      const u32x4 z = u32x4{0u, 0u, 0u, 0u};
      const u32x4 rv = rows[u] >= 0 ? raw[u] : z;
      float f[S::EPL];
      Unpack<T>::run(rv, f);
#pragma unroll
      for (int e = 0; e < S::EPL; ++e) o[e] = fmaf(w, f[e], o[e]);
    }
  }
  // Fold the RPI row groups of the wave (lanes col, col+LPR, ...).
#pragma unroll
  for (int off = S::LPR; off < 64; off <<= 1)
#pragma unroll
    for (int e = 0; e < S::EPL; ++e) o[e] += __shfl_xor(o[e], off);
  if (rsub == 0) {
#pragma unroll
    for (int e = 0; e < S::EPL; ++e) s_o[wave][col * S::EPL + e] = o[e];
  }
  __syncthreads();

  for (int d = threadIdx.x; d < D; d += kAttnThreads) {
    float od = 0.f;
#pragma unroll
    for (int w = 0; w < kAttnWaves; ++w) od += s_o[w][d];
    if (chunks == 1) {
      out[(int64_t)bh * D + d] = (wsum > 0.f) ? od / wsum : 0.f;
      if (d == 0 && lse != nullptr) lse[bh] = (wsum > 0.f) ? mx + logf(wsum) : -INFINITY;
    } else {
      float* p = part + ((int64_t)bh * chunks + c) * (D + 2);
      p[d] = od;
      if (d == 0) {
        p[D] = mx;
        p[D + 1] = wsum;
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

template <typename T, int D>
hipError_t launch_attn_t(const float* q, int64_t q_stride, const void* kr, const void* vr,
                         const int32_t* pos, const int32_t* cnt, int BH, int k, int m,
                         float scale, float* out, float* lse, void* ws, hipStream_t s) {
  const int chunks = (k + kChunk - 1) / kChunk;
  float* part = static_cast<float*>(ws);
  hipLaunchKernelGGL((k_attn_partial<T, D>), dim3(BH * chunks), dim3(kAttnThreads), 0, s, q,
                     q_stride, static_cast<const T*>(kr), static_cast<const T*>(vr), pos, cnt, BH,
                     k, m, chunks, scale, out, lse, part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || chunks == 1) return e;
  hipLaunchKernelGGL((k_attn_combine<D>), dim3(BH), dim3(D), 0, s, part, chunks, out, lse);
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
                       void* ws, hipStream_t s) {
  const int BH = B * H;
  if (BH == 0) return hipSuccess;
  if (dtype == kBF16) {
    if (D == 128)
      return launch_attn_t<uint16_t, 128>(q, q_stride_bh, k_rows, v_rows, pos, cnt, BH, k, m, scale, out, lse, ws, s);
    return launch_attn_t<uint16_t, 64>(q, q_stride_bh, k_rows, v_rows, pos, cnt, BH, k, m, scale, out, lse, ws, s);
  }
  if (D == 128)
    return launch_attn_t<float, 128>(q, q_stride_bh, k_rows, v_rows, pos, cnt, BH, k, m, scale, out, lse, ws, s);
  return launch_attn_t<float, 64>(q, q_stride_bh, k_rows, v_rows, pos, cnt, BH, k, m, scale, out, lse, ws, s);
}

}  // namespace dd
