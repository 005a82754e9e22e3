// Decode attention over the gathered rows only ("Attention" box of Figure 1
// on the arXiv page of DualDecoder, fed by the sparse KV rows), split over
// chunks of 128 selected entries with an online (log-sum-exp) softmax.
//
// One 256-thread workgroup per (b, h, chunk); the chunk itself is computed
// as described with attend_chunk.  A chunk's (max, sum of weights, weighted
// V) goes to the workspace and a small kernel merges the chunks; with a
// single chunk the first kernel finishes the output itself.
#include "attn_body.h"
#include "dd_device.h"
#include "dd_internal.h"

namespace dd {

namespace {

template <typename T, int D>
__global__ __launch_bounds__(kAttnThreads) void k_attn_partial(
    const float* __restrict__ q, int64_t q_stride, const T* __restrict__ krows,
    const T* __restrict__ vrows, const int32_t* __restrict__ pos, const int32_t* __restrict__ cnt,
    int BH, int k, int m, int chunks, float scale, float* __restrict__ out,
    float* __restrict__ lse, float* __restrict__ part) {
  __shared__ AttnLds<D> lds;
  int bh, c;
  xcd_tile_map(blockIdx.x, chunks, BH, bh, c);
  int lim = k;
  if (cnt != nullptr) {
    const int cc = cnt[bh];
    lim = cc < 0 ? 0 : (cc > k ? k : cc);
  }
  // Rows come from the gathered buffer only (no host rows).
  const AttnRows<T> R{krows + (int64_t)bh * m * D, vrows + (int64_t)bh * m * D, nullptr, nullptr,
                      nullptr, m, m, 0};
  const int32_t* pos_bh = pos != nullptr ? pos + (int64_t)bh * k : nullptr;
  auto entry = [&](int j, int& r, int& hc) {
    r = (pos_bh != nullptr) ? pos_bh[j] : j;
    hc = -1;
  };
  float cm, cl, od;
  attend_chunk<T, D>(q + (int64_t)bh * q_stride, R, c * kAttnChunk, lim, scale, entry, lds, cm,
                     cl, od);
  const int d = threadIdx.x;
  if (d >= D) return;
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

// Merge of the chunk partials of one (b, h) by log-sum-exp.
template <int D>
__global__ __launch_bounds__(D) void k_attn_combine(const float* __restrict__ part, int chunks,
                                                    float* __restrict__ out,
                                                    float* __restrict__ lse) {
  const int bh = blockIdx.x;
  const int d = threadIdx.x;
  float od, l;
  combine_chunks<D>(part + (int64_t)bh * chunks * (D + 2), chunks, d, od, l);
  out[(int64_t)bh * D + d] = od;
  if (d == 0 && lse != nullptr) lse[bh] = l;
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
  hipStream_t s;
};

template <typename T, int D>
hipError_t launch_attn_t(const AttnLaunch& a) {
  const int chunks = (a.k + kAttnChunk - 1) / kAttnChunk;
  float* part = static_cast<float*>(a.ws);
  hipLaunchKernelGGL((k_attn_partial<T, D>), dim3(a.BH * chunks), dim3(kAttnThreads), 0, a.s,
                     a.q, a.q_stride, static_cast<const T*>(a.kr), static_cast<const T*>(a.vr),
                     a.pos, a.cnt, a.BH, a.k, a.m, chunks, a.scale, a.out, a.lse, part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || chunks == 1) return e;
  hipLaunchKernelGGL((k_attn_combine<D>), dim3(a.BH), dim3(D), 0, a.s, part, chunks, a.out, a.lse);
  return hipGetLastError();
}

}  // namespace

size_t attn_workspace(int B, int H, int k, int D) {
  const int chunks = (k + kAttnChunk - 1) / kAttnChunk;
  if (chunks <= 1) return 0;
  return (size_t)B * H * chunks * (D + 2) * sizeof(float);
}

hipError_t launch_attn(const float* q, int64_t q_stride_bh, const void* k_rows,
                       const void* v_rows, const int32_t* pos, const int32_t* cnt, int B, int H,
                       int k, int m, int D, int dtype, float scale, float* out, float* lse,
                       void* ws, hipStream_t s) {
  const int BH = B * H;
  if (BH == 0) return hipSuccess;
  AttnLaunch a{q, q_stride_bh, k_rows, v_rows, pos, cnt, BH, k, m, scale, out, lse, ws, s};
  if (dtype == kBF16) {
    if (D == 128) return launch_attn_t<uint16_t, 128>(a);
    return launch_attn_t<uint16_t, 64>(a);
  }
  if (D == 128) return launch_attn_t<float, 128>(a);
  return launch_attn_t<float, 64>(a);
}

}  // namespace dd
