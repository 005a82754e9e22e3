// Decode attention over the gathered rows only ("Attention" box of Figure 1
// on the arXiv page of DualDecoder, fed by the sparse KV rows), split over
// chunks of 128 selected entries with an online (log-sum-exp) softmax.
//
// A workgroup attends over a run of consecutive chunks of one (b, h), each
// as described with attn_fetch and attn_finish, and keeps every chunk's
// (max, sum of weights, weighted V).  When the (b, h) count alone fills
// the chip, one workgroup of G x 256 threads (G = 1 or 2) takes all chunks
// of its (b, h), G chunks at a time (group g of 256 threads takes chunks
// g, g + G, ...), and merges them from LDS; otherwise every chunk gets its
// own 256-thread workgroup, which writes its partial to the workspace, and
// a small kernel merges them.  The merge is the same log-sum-exp over all
// chunks in chunk order either way, so the result does not depend on the
// split.
#include <mutex>

#include "attn_body.h"
#include "dd_device.h"
#include "dd_internal.h"

// The chunk partials of dd_sparse_attn_noalloc: library memory, one copy on
// every device the library runs on, held until the process ends.  In host
// code this name is only a stand-in for the symbol: its device address on
// each device comes from hipGetSymbolAddress (attn_scratch) and is what
// kernels receive.
static __device__ __align__(256) unsigned char scratch[dd::kAttnScratchMaxBytes];

namespace dd {

namespace {

constexpr int kScratchDevices = 64;
std::once_flag scratch_once[kScratchDevices];
void* scratch_ptr[kScratchDevices];
hipError_t scratch_err[kScratchDevices];

constexpr int kAttnMaxChunks = 4096 / kAttnChunk;  // k <= 4096
// (b, h) count from which each (b, h) gets a single workgroup (the chip is
// busy without splitting), and the one from which that workgroup has two
// 256-thread groups (measured faster there; one group is faster below).
constexpr int kAttnMinWgs = 512;
constexpr int kAttnTwoGroups = 1024;

template <typename T, int D, int G>
__global__ __launch_bounds__(G * kAttnThreads) void k_attn(
    const float* __restrict__ q, int64_t q_stride, const T* __restrict__ krows,
    const T* __restrict__ vrows, const int32_t* __restrict__ pos, const int32_t* __restrict__ cnt,
    int BH, int k, int m, int chunks, int cpw, float scale, float* __restrict__ out,
    float* __restrict__ lse, float* __restrict__ part) {
  __shared__ AttnLds<D> lds[G];
  __shared__ float lp[kAttnMaxChunks * (D + 2)];  // partials, when one workgroup has them all
  const int splits = (chunks + cpw - 1) / cpw;
  int bh, sp;
  xcd_tile_map(blockIdx.x, splits, BH, bh, sp);
  int lim = k;
  if (cnt != nullptr) {
    const int cc = cnt[bh];
    lim = cc < 0 ? 0 : (cc > k ? k : cc);
  }
  // Rows come from the gathered buffer only (no host rows).
  const AttnRows<T> R{krows + (int64_t)bh * m * D, vrows + (int64_t)bh * m * D, nullptr, nullptr,
                      nullptr, m, m, 0};
  const int32_t* pos_bh = pos != nullptr ? pos + (int64_t)bh * k : nullptr;
  auto entry = [&](int j, int& r, int& hc, int& o) {
    r = (pos_bh != nullptr) ? pos_bh[j] : j;
    hc = -1;
    o = -1;
  };
  const float* qb = q + (int64_t)bh * q_stride;
  const int g = threadIdx.x / kAttnThreads;
  const int tid = threadIdx.x % kAttnThreads;
  if (chunks == 1) {  // G == 1 here
    AttnFetch<T, D> f;
    float cm[1], cl[1], od[1];
    attn_fetch<T, D>(R, 0, lim, entry, f, tid);
    attn_finish<T, D, 1>(qb, R, scale, f, lds[0], 1, cm, cl, od, tid);
    if (tid < D) {
      out[(int64_t)bh * D + tid] = (cl[0] > 0.f) ? od[0] / cl[0] : 0.f;
      if (tid == 0 && lse != nullptr) lse[bh] = (cl[0] > 0.f) ? cm[0] + logf(cl[0]) : -INFINITY;
    }
    return;
  }
  const bool whole = splits == 1;
  float* pdst = whole ? lp : part + (int64_t)bh * chunks * (D + 2);
  const int c_beg = sp * cpw;
  const int c_end = min(chunks, c_beg + cpw);
  // Every group runs the same number of rounds (the barriers inside are
  // workgroup-wide); a group past the last chunk attends over no entry and
  // writes nothing.
  for (int c0 = c_beg; c0 < c_end; c0 += G) {
    const int c = c0 + g;
    const bool act = c < c_end;
    AttnFetch<T, D> f;
    float cm[1], cl[1], od[1];
    attn_fetch<T, D>(R, c * kAttnChunk, act ? lim : 0, entry, f, tid);
    attn_finish<T, D, 1>(qb, R, scale, f, lds[g], 1, cm, cl, od, tid);
    if (act && tid < D) {
      float* pc = pdst + c * (D + 2);
      pc[tid] = od[0];
      if (tid == 0) {
        pc[D] = cl[0] > 0.f ? cm[0] : -INFINITY;
        pc[D + 1] = cl[0];
      }
    }
    __syncthreads();  // lds is reused by the next round; lp complete
  }
  if (whole && threadIdx.x < D) {
    float o, l;
    combine_chunks<D>(lp, chunks, threadIdx.x, o, l);
    out[(int64_t)bh * D + threadIdx.x] = o;
    if (threadIdx.x == 0 && lse != nullptr) lse[bh] = l;
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
  const auto args = [&](auto kern, int wgs, int threads, int cpw) {
    hipLaunchKernelGGL(kern, dim3(wgs), dim3(threads), 0, a.s, a.q, a.q_stride,
                       static_cast<const T*>(a.kr), static_cast<const T*>(a.vr), a.pos, a.cnt,
                       a.BH, a.k, a.m, chunks, cpw, a.scale, a.out, a.lse, part);
    return hipGetLastError();
  };
  if (chunks == 1 || a.BH < kAttnMinWgs) {  // a workgroup per chunk
    hipError_t e = args(k_attn<T, D, 1>, a.BH * chunks, kAttnThreads, 1);
    if (e != hipSuccess || chunks == 1) return e;
    hipLaunchKernelGGL((k_attn_combine<D>), dim3(a.BH), dim3(D), 0, a.s, part, chunks, a.out,
                       a.lse);
    return hipGetLastError();
  }
  if (a.BH < kAttnTwoGroups) return args(k_attn<T, D, 1>, a.BH, kAttnThreads, chunks);
  return args(k_attn<T, D, 2>, a.BH, 2 * kAttnThreads, chunks);
}

}  // namespace

size_t attn_workspace(int B, int H, int k, int D) {
  const int chunks = (k + kAttnChunk - 1) / kAttnChunk;
  if (chunks <= 1) return 0;
  return (size_t)B * H * chunks * (D + 2) * sizeof(float);
}

size_t attn_workspace_used(int B, int H, int k, int D) {
  const int chunks = (k + kAttnChunk - 1) / kAttnChunk;
  if (chunks <= 1 || (int64_t)B * H >= kAttnMinWgs) return 0;  // partials stay in LDS
  return attn_workspace(B, H, k, D);
}

hipError_t attn_scratch(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kScratchDevices) return hipErrorInvalidDevice;
  // Once per device, with that device current: the array's address there.
  std::call_once(scratch_once[dev], [dev]() {
    void* p = nullptr;
    scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    scratch_ptr[dev] = scratch_err[dev] == hipSuccess ? p : nullptr;
  });
  *ptr = scratch_ptr[dev];
  return scratch_err[dev];
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
