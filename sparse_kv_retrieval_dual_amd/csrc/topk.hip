// Per-row top-k selection, I = argtopk(alpha, k) (paper-daily summary of
// DualDecoder, core-formulas section; "Top-k" box of Figure 1 on the arXiv
// page), with the prediction bookkeeping of the layer step fused into the
// current-query rows.
//
// One 1024-thread workgroup per row.  Scores become order-preserving 32-bit
// keys; the exact k-th largest key T is found by MSB-first radix selection
// (12 + 12 + 8 bit digits, one LDS histogram per pass, each pass restricted
// to keys matching the digits found so far).  The output is then compacted
// in ascending index order: every key > T, plus the first k - #(> T) keys
// equal to T, which is the lower-index-wins rule.  Rows that fit in LDS are
// cached there once; longer rows are re-read from global memory (L2) by each
// pass.
#include "dd_device.h"
#include "dd_internal.h"

namespace dd {

namespace {

constexpr int kTopkThreads = 1024;
constexpr int kHistBins = 4096;
constexpr int kScratchInts = 64;  // [0,16) scans, [16,18) pass result, [32,64) wave counts

struct CachedKeys {
  const uint32_t* c;
  __device__ __forceinline__ uint32_t operator()(int64_t i) const { return c[i]; }
};

struct GlobalKeys {
  const float* g;
  __device__ __forceinline__ uint32_t operator()(int64_t i) const { return order_key(g[i]); }
};

typedef float f32x4 __attribute__((ext_vector_type(4)));

// Keys of row[0, n) into LDS: 16-byte loads, four per thread in flight.
__device__ __forceinline__ void fill_cache(const float* __restrict__ row, int64_t n,
                                           uint32_t* cache) {
  const int tid = threadIdx.x;
  int64_t done = 0;
  if ((reinterpret_cast<uintptr_t>(row) & 15u) == 0) {
    constexpr int UN = 4;
    const f32x4* r4 = reinterpret_cast<const f32x4*>(row);
    const int64_t n4 = n / 4;
    int64_t i = tid;
    for (; i + (UN - 1) * kTopkThreads < n4; i += UN * kTopkThreads) {
      f32x4 v[UN];
#pragma unroll
      for (int u = 0; u < UN; ++u) v[u] = r4[i + u * kTopkThreads];
#pragma unroll
      for (int u = 0; u < UN; ++u) {
        uint32_t* c = cache + 4 * (i + u * kTopkThreads);
        c[0] = order_key(v[u].x);
        c[1] = order_key(v[u].y);
        c[2] = order_key(v[u].z);
        c[3] = order_key(v[u].w);
      }
    }
    for (; i < n4; i += kTopkThreads) {
      const f32x4 v = r4[i];
      uint32_t* c = cache + 4 * i;
      c[0] = order_key(v.x);
      c[1] = order_key(v.y);
      c[2] = order_key(v.z);
      c[3] = order_key(v.w);
    }
    done = n4 * 4;
  }
  for (int64_t i = done + tid; i < n; i += kTopkThreads) cache[i] = order_key(row[i]);
}

// Finds T, the k-th largest key of src[0, n) (n > k), and how many keys
// equal to T belong to the selection.
template <class Src>
__device__ __forceinline__ void find_threshold(const Src& src, int64_t n, int k, uint32_t* hist,
                                               int* scr, uint32_t& thr, int& take_eq) {
  const int tid = threadIdx.x;
  uint32_t prefix = 0u, pmask = 0u;
  int kr = k;
#pragma unroll 1
  for (int p = 0; p < 3; ++p) {
    const int sh = (p == 0) ? 20 : ((p == 1) ? 8 : 0);
    const uint32_t dm = (p == 2) ? 0xFFu : 0xFFFu;
    for (int i = tid; i < kHistBins; i += kTopkThreads) hist[i] = 0u;
    __syncthreads();
    {
      // Eight keys per thread are loaded before any is counted, so that a
      // row read from global memory has eight loads in flight per lane.
      constexpr int UN = 8;
      int64_t i = tid;
      for (; i + (UN - 1) * kTopkThreads < n; i += UN * kTopkThreads) {
        uint32_t key[UN];
#pragma unroll
        for (int u = 0; u < UN; ++u) key[u] = src(i + u * kTopkThreads);
#pragma unroll
        for (int u = 0; u < UN; ++u)
          if ((key[u] & pmask) == prefix) atomicAdd(&hist[(key[u] >> sh) & dm], 1u);
      }
      for (; i < n; i += kTopkThreads) {
        const uint32_t key = src(i);
        if ((key & pmask) == prefix) atomicAdd(&hist[(key >> sh) & dm], 1u);
      }
    }
    __syncthreads();
    // Thread t owns bins top, top-1, top-2, top-3 (descending digits).
    const int top = kHistBins - 1 - 4 * tid;
    int c[4];
    int local = 0;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      c[u] = (int)hist[top - u];
      local += c[u];
    }
    int total;
    const int above = block_exclusive_scan(local, scr, total);
    if (above < kr && above + local >= kr) {
      int acc = above;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        if (acc + c[u] >= kr) {
          scr[16] = top - u;
          scr[17] = acc;
          break;
        }
        acc += c[u];
      }
    }
    __syncthreads();
    const uint32_t digit = (uint32_t)scr[16];
    const int gt = scr[17];
    __syncthreads();
    prefix |= digit << sh;
    pmask |= dm << sh;
    kr -= gt;
  }
  thr = prefix;
  take_eq = kr;
}

// Writes the selected positions of src[0, n) in ascending order.
template <class Src>
__device__ __forceinline__ void emit_selected(const Src& src, int64_t n, uint32_t thr,
                                              int take_eq, int k, int32_t* __restrict__ out,
                                              int32_t* sel, int* scr) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  constexpr int NW = kTopkThreads / 64;
  const int64_t per_wave = ((n + NW * 64 - 1) / (NW * 64)) * 64;
  const int64_t w0 = (int64_t)wave * per_wave;
  const int64_t w1 = (w0 + per_wave < n) ? (w0 + per_wave) : n;

  // Counting pass, four 64-element chunks per step (loads first).  Lanes
  // past the segment end read the last element and are masked out.
  int gt = 0, eq = 0;
  {
    constexpr int UN = 4;
    for (int64_t base = w0; base < w1; base += UN * 64) {
      uint32_t key[UN];
      bool valid[UN];
#pragma unroll
      for (int u = 0; u < UN; ++u) {
        const int64_t i = base + u * 64 + lane;
        valid[u] = i < w1;
        key[u] = src(valid[u] ? i : w1 - 1);
      }
#pragma unroll
      for (int u = 0; u < UN; ++u) {
        gt += __popcll(__ballot(valid[u] && key[u] > thr));
        eq += __popcll(__ballot(valid[u] && key[u] == thr));
      }
    }
  }
  if (lane == 0) {
    scr[32 + wave] = gt;
    scr[48 + wave] = eq;
  }
  __syncthreads();
  int gt_before = 0, eq_before = 0;
  for (int w = 0; w < wave; ++w) {
    gt_before += scr[32 + w];
    eq_before += scr[48 + w];
  }
  int out_pos = gt_before + (eq_before < take_eq ? eq_before : take_eq);
  int eq_run = eq_before;
  constexpr int UN = 4;
  for (int64_t base = w0; base < w1; base += UN * 64) {
    uint32_t key[UN];
    bool valid[UN];
#pragma unroll
    for (int u = 0; u < UN; ++u) {
      const int64_t i = base + u * 64 + lane;
      valid[u] = i < w1;
      key[u] = src(valid[u] ? i : w1 - 1);
    }
#pragma unroll
    for (int u = 0; u < UN; ++u) {
      const int64_t i = base + u * 64 + lane;
      const bool is_gt = valid[u] && key[u] > thr;
      const bool is_eq = valid[u] && key[u] == thr;
      const uint64_t E = __ballot(is_eq);
      const bool take = is_gt || (is_eq && eq_run + lanes_below(E) < take_eq);
      const uint64_t S = __ballot(take);
      const int slot = out_pos + lanes_below(S);
      if (take && slot < k) {  // exactly k are taken; the bound is a guard
        out[slot] = (int32_t)i;
        if (sel != nullptr) sel[slot] = (int32_t)i;
      }
      out_pos += __popcll(S);
      eq_run += __popcll(E);
    }
  }
}

// Misses of the selected set `sel` (ascending, -1 padded) against the
// prediction, and the slot row of every selected entry: prediction entry p
// sits in slot row p, the t-th miss in slot row k + t.
__device__ __forceinline__ void bookkeeping(const int32_t* sel, int k, int64_t n, int64_t n_max,
                                            const int32_t* __restrict__ pred_row,
                                            int32_t* s_pred, int32_t* __restrict__ pos_row,
                                            int32_t* __restrict__ miss_row,
                                            int32_t* __restrict__ counts, int bh, int BH,
                                            int* scr) {
  int fetchable = 0, nonneg = 0;
  for (int p = threadIdx.x; p < k; p += kTopkThreads) {
    const int v = pred_row != nullptr ? pred_row[p] : -1;
    s_pred[p] = v;
    fetchable += (v >= 0 && (int64_t)v < n_max) ? 1 : 0;
    nonneg += (v >= 0) ? 1 : 0;
  }
  fetchable = block_sum_int(fetchable, scr);
  const int plen = block_sum_int(nonneg, scr);  // entries before the -1 padding

  int misses = 0;
  for (int r0 = 0; r0 < k; r0 += kTopkThreads) {
    const int j = r0 + (int)threadIdx.x;
    const int c = j < k ? sel[j] : -1;
    int hit = -1;
    if (c >= 0) {
      int lo = 0, hi = plen;
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (s_pred[mid] < c) lo = mid + 1;
        else hi = mid;
      }
      if (lo < plen && s_pred[lo] == c) hit = lo;
    }
    const int is_miss = (c >= 0 && hit < 0) ? 1 : 0;
    int tot;
    const int rank = misses + block_exclusive_scan(is_miss, scr, tot);
    if (j < k) pos_row[j] = (c < 0) ? -1 : (hit >= 0 ? hit : k + rank);
    if (is_miss) miss_row[rank] = c;
    misses += tot;
  }
  for (int t = misses + (int)threadIdx.x; t < k; t += kTopkThreads) miss_row[t] = -1;
  if (threadIdx.x == 0) {
    const int valid = (int)(n < k ? n : k);
    counts[bh] = misses;
    counts[BH + bh] = valid - misses;
    counts[2 * BH + bh] = fetchable;
  }
}

__global__ __launch_bounds__(kTopkThreads) void k_topk(
    const float* __restrict__ scores, const int32_t* __restrict__ lens, int H, int Q, int BH,
    int64_t n_max, int k, int32_t* __restrict__ out0, int32_t* __restrict__ out1,
    int64_t out_stride, const int32_t* __restrict__ pred, int32_t* __restrict__ pos,
    int32_t* __restrict__ miss, int32_t* __restrict__ counts, int sel_slots, int cache_cap) {
  extern __shared__ uint32_t smem[];
  uint32_t* hist = smem;
  int* scr = reinterpret_cast<int*>(smem + kHistBins);
  int32_t* sel_buf = reinterpret_cast<int32_t*>(smem + kHistBins + kScratchInts);
  uint32_t* cache = smem + kHistBins + kScratchInts + sel_slots;

  int bh, j;
  xcd_tile_map(blockIdx.x, Q, BH, bh, j);
  const int64_t n = clamp_len(lens[bh / H], n_max);
  const float* row = scores + ((int64_t)bh * Q + j) * n_max;
  int32_t* out = ((j == 0) ? out0 : out1) + (int64_t)bh * out_stride;
  const bool do_book = (pos != nullptr) && j == 0;
  int32_t* sel = do_book ? sel_buf : nullptr;

  if (n <= k) {
    for (int t = threadIdx.x; t < k; t += kTopkThreads) {
      const int32_t v = (t < n) ? t : -1;
      out[t] = v;
      if (sel != nullptr) sel[t] = v;
    }
  } else if (n <= cache_cap) {
    fill_cache(row, n, cache);
    __syncthreads();
    const CachedKeys src{cache};
    uint32_t thr;
    int take_eq;
    find_threshold(src, n, k, hist, scr, thr, take_eq);
    emit_selected(src, n, thr, take_eq, k, out, sel, scr);
  } else {
    const GlobalKeys src{row};
    uint32_t thr;
    int take_eq;
    find_threshold(src, n, k, hist, scr, thr, take_eq);
    emit_selected(src, n, thr, take_eq, k, out, sel, scr);
  }
  if (!do_book) return;
  __syncthreads();
  bookkeeping(sel, k, n, n_max, pred != nullptr ? pred + (int64_t)bh * k : nullptr,
              reinterpret_cast<int32_t*>(hist), pos + (int64_t)bh * k, miss + (int64_t)bh * k,
              counts, bh, BH, scr);
}

}  // namespace

hipError_t launch_topk(const float* scores, const int32_t* lens, int B, int H, int Q,
                       int64_t n_max, int k, int32_t* out0, int32_t* out1,
                       int64_t out_stride_bh, const TopkBook* book, hipStream_t s) {
  const int BH = B * H;
  if (BH == 0) return hipSuccess;
  const DeviceInfo& di = device_info();
  static bool attr_set[64] = {false};
  if (di.device >= 0 && di.device < 64 && !attr_set[di.device]) {
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(k_topk),
                              hipFuncAttributeMaxDynamicSharedMemorySize, di.lds_per_block);
    attr_set[di.device] = true;
  }
  const bool do_book = book != nullptr && book->pos != nullptr;
  const int sel_slots = do_book ? ((k + 3) & ~3) : 0;
  const int64_t fixed = (int64_t)(kHistBins + kScratchInts + sel_slots) * 4;
  int64_t cap = ((int64_t)di.lds_per_block - fixed) / 4;
  if (cap > n_max) cap = n_max;
  if (cap < 1024) cap = 0;
  const size_t shmem = (size_t)(fixed + cap * 4);
  hipLaunchKernelGGL(k_topk, dim3(BH * Q), dim3(kTopkThreads), shmem, s, scores, lens, H, Q, BH,
                     n_max, k, out0, out1, out_stride_bh, do_book ? book->pred : nullptr,
                     do_book ? book->pos : nullptr, do_book ? book->miss : nullptr,
                     do_book ? book->counts : nullptr, sel_slots, (int)cap);
  return hipGetLastError();
}

}  // namespace dd
