// Per-row top-k selection, I = argtopk(alpha, k) (paper-daily summary of
// DualDecoder, core-formulas section; "Top-k" box of Figure 1 on the arXiv
// page), with the prediction bookkeeping of the layer step fused into the
// current-query rows.
//
// One 1024-thread workgroup per row.  Scores become order-preserving 32-bit
// keys and the exact k-th largest key T is found by MSB-first radix
// selection with 11 + 11 + 10 bit digits:
//   pass 0  histogram of digit 0 over the row (fused with caching the row's
//           keys in LDS when the row fits);
//   pass 1  histogram of digit 1 over keys in the chosen digit-0 bin, which
//           are also collected in a candidate list when it fits;
//   pass 2  histogram of digit 2 over the candidates (over the row if the
//           list did not fit).
// The selection is every key > T plus the first k - #(> T) keys equal to T
// (lower index wins), emitted in ascending index order 32768 keys at a
// time: thread t compares keys 32t..32t+31 of the segment with T, which
// gives it one 32-bit word of the "> T" and "== T" bitmaps in registers;
// block scans give the ranks of the T-equal keys and the output offsets,
// and each thread writes its word's set bits in order.  For the
// current-query row of the layer step the same pass looks every selected
// index up in the prediction (binary search in LDS) and assigns slot rows
// to hits and misses.
//
// The cached row is stored XOR-swizzled within 32-word groups (word i at
// i ^ ((i >> 5) & 31)), so that both lane-strided reads (passes 0-2) and
// each thread reading its own 32 consecutive keys (the emit) are free of
// LDS bank conflicts.
#include "dd_device.h"
#include "dd_internal.h"

namespace dd {

namespace {

constexpr int kTopkThreads = 1024;
constexpr int kBins = 2048;
constexpr int kScratchInts = 64;  // [0,16) scans, [16,24) broadcasts
constexpr int kSeg = kTopkThreads * 32;  // keys per emit segment
constexpr int kCandMin = 1024;           // candidate list entries at least
constexpr int kUnroll = 8;

typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ int swz(int i) { return i ^ ((i >> 5) & 31); }

struct CachedKeys {
  const uint32_t* c;
  __device__ __forceinline__ uint32_t operator()(int i) const { return c[swz(i)]; }
  // Keys base..base+31 (base a multiple of 32).  The cache holds whole
  // 32-word groups, so the tail of the last group is readable; entries at
  // or past n are garbage and the caller masks them.
  __device__ __forceinline__ void word(int base, int n, uint32_t (&key)[32]) const {
    (void)n;
    const int s = (base >> 5) & 31;
#pragma unroll
    for (int b = 0; b < 32; ++b) key[b] = c[base + (b ^ s)];
  }
};

struct GlobalKeys {
  const float* g;
  __device__ __forceinline__ uint32_t operator()(int i) const { return order_key(g[i]); }
  __device__ __forceinline__ void word(int base, int n, uint32_t (&key)[32]) const {
    if (base + 32 <= n && (reinterpret_cast<uintptr_t>(g + base) & 15u) == 0) {
      const f32x4* p = reinterpret_cast<const f32x4*>(g + base);
      f32x4 v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = p[u];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        key[4 * u] = order_key(v[u].x);
        key[4 * u + 1] = order_key(v[u].y);
        key[4 * u + 2] = order_key(v[u].z);
        key[4 * u + 3] = order_key(v[u].w);
      }
    } else {
#pragma unroll
      for (int b = 0; b < 32; ++b) key[b] = order_key(g[(base + b < n) ? base + b : n - 1]);
    }
  }
};

// Chooses the digit holding the kr-th largest key from a histogram of
// kBins counters (digit order = key order): returns the digit and the
// number of counted keys in larger digits.
__device__ __forceinline__ void pick_bin(const uint32_t* hist, int kr, int* scr, int& digit,
                                         int& above) {
  const int t = threadIdx.x;
  const int b0 = kBins - 1 - 2 * t;
  const int c0 = (int)hist[b0];
  const int c1 = (int)hist[b0 - 1];
  const int local = c0 + c1;
  int total;
  const int before = block_exclusive_scan(local, scr, total);
  if (before < kr && before + local >= kr) {
    if (before + c0 >= kr) {
      scr[16] = b0;
      scr[17] = before;
    } else {
      scr[16] = b0 - 1;
      scr[17] = before + c0;
    }
  }
  __syncthreads();
  digit = scr[16];
  above = scr[17];
  __syncthreads();
}

__device__ __forceinline__ void clear(uint32_t* p, int words) {
  for (int i = threadIdx.x; i < words; i += kTopkThreads) p[i] = 0u;
}

// Pass 0 when the row is cached: keys go to LDS and into the histogram.
// Odd and even lanes count into separate copies (halving same-address
// atomics within a wave); the copies are summed afterwards.
__device__ __forceinline__ void fill_and_count(const float* __restrict__ row, int n,
                                               uint32_t* cache, uint32_t* hist2) {
  const int tid = threadIdx.x;
  uint32_t* h = hist2 + (tid & 1) * kBins;
  int done = 0;
  if ((reinterpret_cast<uintptr_t>(row) & 15u) == 0) {
    constexpr int UN = 8;  // a 32768-key row is one round trip: 128 KB in flight
    const f32x4* r4 = reinterpret_cast<const f32x4*>(row);
    const int n4 = n >> 2;
    int i = tid;
    for (; i + (UN - 1) * kTopkThreads < n4; i += UN * kTopkThreads) {
      f32x4 v[UN];
#pragma unroll
      for (int u = 0; u < UN; ++u) v[u] = r4[i + u * kTopkThreads];
#pragma unroll
      for (int u = 0; u < UN; ++u) {
        const int b = 4 * (i + u * kTopkThreads);
        const uint32_t k0 = order_key(v[u].x), k1 = order_key(v[u].y);
        const uint32_t k2 = order_key(v[u].z), k3 = order_key(v[u].w);
        cache[swz(b)] = k0;
        cache[swz(b + 1)] = k1;
        cache[swz(b + 2)] = k2;
        cache[swz(b + 3)] = k3;
        atomicAdd(&h[k0 >> 21], 1u);
        atomicAdd(&h[k1 >> 21], 1u);
        atomicAdd(&h[k2 >> 21], 1u);
        atomicAdd(&h[k3 >> 21], 1u);
      }
    }
    for (; i < n4; i += kTopkThreads) {
      const f32x4 v = r4[i];
      const int b = 4 * i;
      const uint32_t k0 = order_key(v.x), k1 = order_key(v.y);
      const uint32_t k2 = order_key(v.z), k3 = order_key(v.w);
      cache[swz(b)] = k0;
      cache[swz(b + 1)] = k1;
      cache[swz(b + 2)] = k2;
      cache[swz(b + 3)] = k3;
      atomicAdd(&h[k0 >> 21], 1u);
      atomicAdd(&h[k1 >> 21], 1u);
      atomicAdd(&h[k2 >> 21], 1u);
      atomicAdd(&h[k3 >> 21], 1u);
    }
    done = n4 * 4;
  }
  for (int i = done + tid; i < n; i += kTopkThreads) {
    const uint32_t a = order_key(row[i]);
    cache[swz(i)] = a;
    atomicAdd(&h[a >> 21], 1u);
  }
}

// Pass 0 over a row read from global memory (two histogram copies).
__device__ __forceinline__ void count_global(const float* __restrict__ row, int n, uint32_t* hist2) {
  uint32_t* h = hist2 + (threadIdx.x & 1) * kBins;
  int i = threadIdx.x;
  for (; i + (kUnroll - 1) * kTopkThreads < n; i += kUnroll * kTopkThreads) {
    uint32_t key[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) key[u] = order_key(row[i + u * kTopkThreads]);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) atomicAdd(&h[key[u] >> 21], 1u);
  }
  for (; i < n; i += kTopkThreads) atomicAdd(&h[order_key(row[i]) >> 21], 1u);
}

// Pass 1: histogram of digit 1 over keys whose digit 0 is d0; when
// `compact`, their positions are appended to cand (order not kept).
template <class Src>
__device__ __forceinline__ void count_digit1(const Src& src, int n, uint32_t d0, bool compact,
                                             uint32_t* hist, int32_t* cand, int* counter) {
  int i0 = threadIdx.x;
  for (; i0 < n; i0 += kUnroll * kTopkThreads) {
    uint32_t key[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int i = i0 + u * kTopkThreads;
      key[u] = src(i < n ? i : n - 1);
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int i = i0 + u * kTopkThreads;
      if (i < n && (key[u] >> 21) == d0) {
        atomicAdd(&hist[(key[u] >> 10) & 0x7FFu], 1u);
        if (compact) cand[atomicAdd(counter, 1)] = i;
      }
    }
  }
}

// Lowest `take` set bits of w (take <= popcount(w)).
__device__ __forceinline__ uint32_t lowest_bits(uint32_t w, int take) {
  uint32_t r = 0u;
  for (int q = 0; q < take; ++q) {
    const uint32_t low = w & (0u - w);
    r |= low;
    w ^= low;
  }
  return r;
}

// Position of c in the ascending list s[0, len), or -1.
__device__ __forceinline__ int find_in(const int32_t* s, int len, int c) {
  int lo = 0, hi = len;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (s[mid] < c) lo = mid + 1;
    else hi = mid;
  }
  return (lo < len && s[lo] == c) ? lo : -1;
}

struct Book {
  const int32_t* s_pred;  // prediction in LDS (nullptr: none)
  int plen;               // entries before its -1 padding
  int32_t* pos;           // row of pos (global), nullptr when not bookkeeping
  int32_t* miss;          // row of miss (global)
};

// Emits the selection {key > T} + first take_eq of {key == T} of src[0, n)
// in ascending index order.  Returns the number of misses (bookkeeping).
template <class Src>
__device__ __forceinline__ int emit_ordered(const Src& src, int n, uint32_t thr, int take_eq,
                                            int k, int32_t* __restrict__ out, const Book& bk,
                                            int* scr) {
  const int t = threadIdx.x;
  int out_run = 0, eq_run = 0, miss_run = 0;
  for (int seg0 = 0; seg0 < n; seg0 += kSeg) {
    const int base = seg0 + 32 * t;
    uint32_t g = 0u, ew = 0u;
    if (base < n) {
      uint32_t key[32];
      src.word(base, n, key);
#pragma unroll
      for (int b = 0; b < 32; ++b) {
        const bool valid = base + b < n;
        g |= (valid && key[b] > thr) ? (1u << b) : 0u;
        ew |= (valid && key[b] == thr) ? (1u << b) : 0u;
      }
    }
    int eq_tot;
    const int eq_before = eq_run + block_exclusive_scan(__popc(ew), scr, eq_tot);
    int take = take_eq - eq_before;
    take = take < 0 ? 0 : (take > __popc(ew) ? __popc(ew) : take);
    const uint32_t sel = g | lowest_bits(ew, take);
    int sel_tot;
    int j = out_run + block_exclusive_scan(__popc(sel), scr, sel_tot);
    if (bk.pos != nullptr) {
      int my_miss = 0;
      for (uint32_t w = sel; w != 0u; w &= w - 1u) {
        const int c = base + __ffs(w) - 1;
        my_miss += (bk.s_pred == nullptr || find_in(bk.s_pred, bk.plen, c) < 0) ? 1 : 0;
      }
      int miss_tot;
      int mr = miss_run + block_exclusive_scan(my_miss, scr, miss_tot);
      for (uint32_t w = sel; w != 0u; w &= w - 1u) {
        const int c = base + __ffs(w) - 1;
        const int hit = bk.s_pred == nullptr ? -1 : find_in(bk.s_pred, bk.plen, c);
        if (j < k) {
          out[j] = c;
          if (hit >= 0) {
            bk.pos[j] = hit;
          } else {
            bk.pos[j] = k + mr;
            bk.miss[mr] = c;
            ++mr;
          }
        }
        ++j;
      }
      miss_run += miss_tot;
    } else {
      for (uint32_t w = sel; w != 0u; w &= w - 1u) {
        if (j < k) out[j] = base + __ffs(w) - 1;
        ++j;
      }
    }
    out_run += sel_tot;
    eq_run += eq_tot;
  }
  return miss_run;
}

// Loads the prediction row into s_pred; returns fetchable | plen << 16.
__device__ __forceinline__ int load_prediction(const int32_t* __restrict__ pred_row, int k,
                                               int64_t n_max, int32_t* s_pred, int* scr) {
  int f = 0, nn = 0;
  for (int p = threadIdx.x; p < k; p += kTopkThreads) {
    const int v = pred_row != nullptr ? pred_row[p] : -1;
    s_pred[p] = v;
    f += (v >= 0 && (int64_t)v < n_max) ? 1 : 0;
    nn += (v >= 0) ? 1 : 0;
  }
  return block_sum_int(f | (nn << 16), scr);
}

__global__ __launch_bounds__(kTopkThreads) void k_topk(
    const float* __restrict__ scores, const int32_t* __restrict__ lens, int H, int Q, int BH,
    int64_t n_max, int k, int32_t* __restrict__ out0, int32_t* __restrict__ out1,
    int64_t out_stride, const int32_t* __restrict__ pred, int32_t* __restrict__ pos,
    int32_t* __restrict__ miss, int32_t* __restrict__ counts, int cand_cap, int cache_cap) {
  extern __shared__ uint32_t smem[];
  uint32_t* hist = smem;  // two copies during pass 0
  int* scr = reinterpret_cast<int*>(smem + 2 * kBins);
  int32_t* cand = reinterpret_cast<int32_t*>(smem + 2 * kBins + kScratchInts);  // also the prediction
  uint32_t* cache = reinterpret_cast<uint32_t*>(cand + cand_cap);

  int bh, j;
  xcd_tile_map(blockIdx.x, Q, BH, bh, j);
  const int n = (int)clamp_len(lens[bh / H], n_max);
  const float* row = scores + ((int64_t)bh * Q + j) * n_max;
  int32_t* out = ((j == 0) ? out0 : out1) + (int64_t)bh * out_stride;
  const bool do_book = (pos != nullptr) && j == 0;
  const int tid = threadIdx.x;
  if (tid == 0) scr[20] = 0;  // running count (candidates, or misses of a short row)
  const int32_t* pred_row = pred != nullptr ? pred + (int64_t)bh * k : nullptr;

  Book bk{nullptr, 0, nullptr, nullptr};
  int fetchable = 0;
  int misses = 0;

  if (n <= k) {
    // Every valid key is selected: entry c is c itself.
    if (do_book) {
      const int packed = load_prediction(pred_row, k, n_max, cand, scr);
      fetchable = packed & 0xFFFF;
      bk = Book{pred_row != nullptr ? cand : nullptr, packed >> 16, pos + (int64_t)bh * k,
                miss + (int64_t)bh * k};
    }
    for (int r0 = 0; r0 < k; r0 += kTopkThreads) {
      const int c = r0 + tid;
      const bool valid = c < n;
      int hit = -1;
      if (do_book && valid && bk.s_pred != nullptr) hit = find_in(bk.s_pred, bk.plen, c);
      int mtot = 0, mr = 0;
      if (do_book) {
        mr = block_exclusive_scan((valid && hit < 0) ? 1 : 0, scr, mtot);
        mr += scr[20];
      }
      if (c < k) {
        out[c] = valid ? c : -1;
        if (do_book) {
          bk.pos[c] = !valid ? -1 : (hit >= 0 ? hit : k + mr);
          if (valid && hit < 0) bk.miss[mr] = c;
        }
      }
      if (do_book) {
        __syncthreads();
        if (tid == 0) scr[20] += mtot;
        __syncthreads();
      }
    }
    if (do_book) misses = scr[20];
  } else {
    const bool cached = ((n + 31) & ~31) <= cache_cap;
    clear(hist, 2 * kBins);
    __syncthreads();
    if (cached) fill_and_count(row, n, cache, hist);
    else count_global(row, n, hist);
    __syncthreads();
    for (int i = tid; i < kBins; i += kTopkThreads) hist[i] += hist[kBins + i];
    __syncthreads();
    int d0, above;
    pick_bin(hist, k, scr, d0, above);
    int kr = k - above;
    const int c0 = (int)hist[d0];
    const bool compact = c0 <= cand_cap;
    __syncthreads();
    clear(hist, kBins);
    __syncthreads();
    if (cached) count_digit1(CachedKeys{cache}, n, (uint32_t)d0, compact, hist, cand, &scr[20]);
    else count_digit1(GlobalKeys{row}, n, (uint32_t)d0, compact, hist, cand, &scr[20]);
    __syncthreads();
    int d1;
    pick_bin(hist, kr, scr, d1, above);
    kr -= above;
    const uint32_t prefix = ((uint32_t)d0 << 21) | ((uint32_t)d1 << 10);
    __syncthreads();
    clear(hist, kBins);
    __syncthreads();
    if (compact) {
      for (int tt = tid; tt < c0; tt += kTopkThreads) {
        const int i = cand[tt];
        const uint32_t key = cached ? cache[swz(i)] : order_key(row[i]);
        if ((key & 0xFFFFFC00u) == prefix) atomicAdd(&hist[key & 0x3FFu], 1u);
      }
    } else {
      for (int i = tid; i < n; i += kTopkThreads) {
        const uint32_t key = cached ? cache[swz(i)] : order_key(row[i]);
        if ((key & 0xFFFFFC00u) == prefix) atomicAdd(&hist[key & 0x3FFu], 1u);
      }
    }
    __syncthreads();
    int d2;
    pick_bin(hist, kr, scr, d2, above);
    kr -= above;
    const uint32_t thr = prefix | (uint32_t)d2;

    if (do_book) {
      const int packed = load_prediction(pred_row, k, n_max, cand, scr);
      fetchable = packed & 0xFFFF;
      bk = Book{pred_row != nullptr ? cand : nullptr, packed >> 16, pos + (int64_t)bh * k,
                miss + (int64_t)bh * k};
    }
    if (cached) misses = emit_ordered(CachedKeys{cache}, n, thr, kr, k, out, bk, scr);
    else misses = emit_ordered(GlobalKeys{row}, n, thr, kr, k, out, bk, scr);
  }

  if (!do_book) return;
  for (int tt = misses + tid; tt < k; tt += kTopkThreads) bk.miss[tt] = -1;
  if (tid == 0) {
    const int valid = n < k ? n : k;
    counts[bh] = misses;
    counts[BH + bh] = valid - misses;
    counts[2 * BH + bh] = fetchable;
  }
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
  // LDS words: two histogram copies, scratch, candidates (also the
  // prediction, so at least k), then the cached row (whole 32-word groups).
  const int64_t lds_words = di.lds_per_block / 4;
  const int64_t fixed = 2 * kBins + kScratchInts;
  const int64_t cand_min = ((k > kCandMin ? k : kCandMin) + 31) & ~int64_t(31);
  const int64_t n_round = (n_max + 31) & ~int64_t(31);
  int64_t cache_cap = (lds_words - fixed - cand_min) & ~int64_t(31);
  if (cache_cap > n_round) cache_cap = n_round;
  if (cache_cap < 4096) cache_cap = 0;
  int64_t cand_cap = (lds_words - fixed - cache_cap) & ~int64_t(31);
  if (cand_cap > 1 << 20) cand_cap = 1 << 20;
  const size_t shmem = (size_t)(fixed + cand_cap + cache_cap) * 4;
  hipLaunchKernelGGL(k_topk, dim3(BH * Q), dim3(kTopkThreads), shmem, s, scores, lens, H, Q, BH,
                     n_max, k, out0, out1, out_stride_bh, do_book ? book->pred : nullptr,
                     do_book ? book->pos : nullptr, do_book ? book->miss : nullptr,
                     do_book ? book->counts : nullptr, (int)cand_cap, (int)cache_cap);
  return hipGetLastError();
}

}  // namespace dd
