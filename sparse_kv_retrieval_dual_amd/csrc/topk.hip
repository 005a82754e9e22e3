// Per-row top-k selection, I = argtopk(alpha, k) (paper-daily summary of
// DualDecoder, core-formulas section; "Top-k" box of Figure 1 on the arXiv
// page), with the prediction bookkeeping of the layer step fused into the
// current-query rows.
//
// One 1024-thread workgroup per row; scores become order-preserving 32-bit
// keys.  The selection is every key > T plus the first k - #(> T) keys equal
// to T (lower index wins), where T is the exact k-th largest key, and it is
// written in ascending index order.
//
// Filter path (rows up to kFilterMaxN keys).  Each thread reads its share
// of the row (8 float4 per 32768-key chunk, coalesced) and keeps the
// maximum of each of its G key groups.  With 1024 * G >= k groups, the
// lowest key of the 11-bit bin holding the k-th largest group maximum is a
// bound B with at least k keys >= B, and only a small multiple of k keys
// pass it on real score rows.  Those candidates (key, index) are compacted
// into LDS, T is found by 11 + 11 + 10 bit radix selection over the
// candidates alone, and the selection is scattered into "> T" / "== T"
// bitmaps of the row; each thread then owns consecutive bitmap words, and
// block scans over their popcounts give the ranks of the T-equal keys and
// the output offsets.  If more than kFilterCap keys pass the bound (a row
// dominated by ties, say), the row takes the radix path instead.
//
// Radix path.  MSB-first radix selection over the whole row:
//   pass 0  histogram of digit 0 over the row (fused with caching the row's
//           keys in LDS when the row fits);
//   pass 1  histogram of digit 1 over keys in the chosen digit-0 bin, which
//           are also collected in a candidate list when it fits;
//   pass 2  histogram of digit 2 over the candidates (over the row if the
//           list did not fit).
// It emits 32768 keys at a time: thread t compares keys 32t..32t+31 of the
// segment with T, which gives it one word of the two bitmaps in registers.
//
// For the current-query row of the layer step either path looks every
// selected index up in the prediction (binary search in LDS) and assigns
// slot rows to hits and misses.
//
// The radix path's cached row is stored XOR-swizzled within 32-word groups
// (word i at i ^ ((i >> 5) & 31)), so that both lane-strided reads and each
// thread reading its own 32 consecutive keys are free of LDS bank conflicts.
#include <algorithm>

#include "dd_device.h"
#include "dd_internal.h"

namespace dd {

namespace {

constexpr int kTopkThreads = 1024;
constexpr int kTopkWaves = kTopkThreads / 64;
constexpr int kBins = 2048;
constexpr int kScratchInts = 128;  // scans and broadcasts
constexpr int kMaxK = 4096;        // largest k (DD_MAX_K)
constexpr int kSeg = kTopkThreads * 32;  // keys per emit segment
constexpr int kCandMin = 1024;           // candidate list entries at least
constexpr int kUnroll = 8;
constexpr int kChunk = kTopkThreads * 32;  // keys per register tile of the filter path
constexpr int kFilterCap = 8192;           // candidates the filter path can hold
constexpr int kFilterMaxN = 1 << 17;       // longest row of the filter path (bitmaps in LDS)
constexpr int kMaxWords = kFilterMaxN / 32 / kTopkThreads;  // bitmap words per thread

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

// ---------------------------------------------------------------- filter path

// Register tiles of NT threads: thread t holds 32 keys of a tile of 32 NT
// entries starting at c0, key[b] = entry c0 + 4 t + koff<NT>(b) with
// koff<NT>(b) = 4 NT (b / 4) + b % 4 (the thread's 8 coalesced float4 loads).
// Entries at or past n read as key 0, which is below the key of every finite
// score; with lim = n - (c0 + 4 t), entry b is in the row iff koff(b) < lim.
template <int NT>
__device__ __forceinline__ constexpr int koff(int b) { return 4 * NT * (b >> 2) + (b & 3); }

// Loads are unconditional, clamped to the first nload entries (n <= nload
// <= n_max), with 32-bit offsets from the row base.  vec: the row is
// 16-byte aligned and n_max is a multiple of 4, so every float4 holding an
// entry < nload lies inside the row's storage.
template <int NT>
__device__ __forceinline__ void load_tile(const float* __restrict__ row, int n, int nload, int c0,
                                          bool vec, uint32_t (&key)[32]) {
  const int lim = n - (c0 + 4 * (int)threadIdx.x);
  const char* base = reinterpret_cast<const char*>(row);
  if (vec) {
    const uint32_t nq = (uint32_t)(nload + 3) >> 2;
    const uint32_t q0 = ((uint32_t)c0 >> 2) + threadIdx.x;
    f32x4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      uint32_t q = q0 + NT * u;
      q = q < nq ? q : nq - 1u;
      v[u] = *reinterpret_cast<const f32x4*>(base + q * 16u);
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      key[4 * u] = order_key(v[u].x);
      key[4 * u + 1] = order_key(v[u].y);
      key[4 * u + 2] = order_key(v[u].z);
      key[4 * u + 3] = order_key(v[u].w);
    }
  } else {
    const uint32_t i0 = (uint32_t)(c0 + 4 * (int)threadIdx.x);
    const int liml = nload - (c0 + 4 * (int)threadIdx.x);
#pragma unroll
    for (int b = 0; b < 32; ++b) {
      const uint32_t i = koff<NT>(b) < liml ? i0 + (uint32_t)koff<NT>(b) : (uint32_t)nload - 1u;
      key[b] = order_key(*reinterpret_cast<const float*>(base + i * 4u));
    }
  }
#pragma unroll
  for (int b = 0; b < 32; ++b) key[b] = koff<NT>(b) < lim ? key[b] : 0u;
}

template <int G>
__device__ __forceinline__ void group_max(const uint32_t (&key)[32], uint32_t (&gmax)[G]) {
#pragma unroll
  for (int b = 0; b < 32; ++b) gmax[b % G] = key[b] > gmax[b % G] ? key[b] : gmax[b % G];
}

// Bit b set iff key[b] is in the row and >= bound.
template <int NT>
__device__ __forceinline__ uint32_t pass_mask(const uint32_t (&key)[32], int c0, int n,
                                              uint32_t bound) {
  const int lim = n - (c0 + 4 * (int)threadIdx.x);
  uint32_t m = 0u;
#pragma unroll
  for (int b = 0; b < 32; ++b) m |= (koff<NT>(b) < lim && key[b] >= bound) ? (1u << b) : 0u;
  return m;
}

// Writes the keys of mask m (entries of tile c0) to ck / ci from slot off
// on, dropping slots >= cap.
template <int NT>
__device__ __forceinline__ void put_candidates(const uint32_t (&key)[32], uint32_t m, int c0,
                                               int off, int cap, uint32_t* ck, int32_t* ci) {
  const int i0 = c0 + 4 * (int)threadIdx.x;
#pragma unroll
  for (int b = 0; b < 32; ++b) {
    if (m & (1u << b)) {
      if (off < cap) {
        ck[off] = key[b];
        ci[off] = i0 + koff<NT>(b);
      }
      ++off;
    }
  }
}

// The digit holding the kr-th largest counted key in a histogram of kBins
// counters (digit order = key order) and the count in larger digits: thread
// t of NT scans the kBins / NT digits below kBins - t kBins / NT, one block
// scan orders the threads, and the thread whose digits reach kr writes both
// to out2 (a second barrier).
template <int NT>
__device__ __forceinline__ void pick_bin_fast(const uint32_t* hist, int kr, ScanBufs& sb,
                                              int* out2, int& digit, int& above) {
  constexpr int BPT = kBins / NT;
  const int top = kBins - BPT * (int)threadIdx.x;  // this thread's digits: [top - BPT, top)
  int c[BPT];
  int sum = 0;
#pragma unroll
  for (int i = 0; i < BPT; ++i) {
    c[i] = (int)hist[top - 1 - i];
    sum += c[i];
  }
  int total;
  const int before = block_scan<NT / 64>(sum, sb, total);
  if (before < kr && before + sum >= kr) {
    int a = before, d = top - BPT;
    bool found = false;
#pragma unroll
    for (int i = 0; i < BPT; ++i) {
      if (!found) {
        if (a + c[i] >= kr) {
          found = true;
          d = top - 1 - i;
        } else {
          a += c[i];
        }
      }
    }
    out2[0] = d;
    out2[1] = a;
  }
  __syncthreads();
  digit = out2[0];
  above = out2[1];
}

// The exact k-th largest key T among the cnt candidate keys (k <= cnt <=
// kFilterCap) and how many keys equal to T the selection takes, by
// MSB-first radix selection with 8-bit digits.  Every thread holds its
// candidates (tid + 1024 r) in registers; pass p counts into its own
// 256-counter histogram h4 + 256 p, which the caller has cleared before a
// barrier that precedes this call.  After each pass's barrier every wave
// scans the histogram itself, so T needs no broadcast.
__device__ __forceinline__ void block_select(const uint32_t* fkey, int cnt, int k, uint32_t* h4,
                                             uint32_t& thr, int& take_eq) {
  constexpr int R = kFilterCap / kTopkThreads;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  uint32_t x[R];
#pragma unroll
  for (int r = 0; r < R; ++r) x[r] = tid + kTopkThreads * r < cnt ? fkey[tid + kTopkThreads * r] : 0u;
  uint32_t prefix = 0u, pmask = 0u;
  int kr = k;
#pragma unroll
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    uint32_t* h = h4 + 256 * pass;
#pragma unroll
    for (int r = 0; r < R; ++r)
      if (tid + kTopkThreads * r < cnt && (x[r] & pmask) == prefix)
        atomicAdd(&h[(x[r] >> shift) & 255u], 1u);
    __syncthreads();
    // lane l holds digits 255 - 4l .. 252 - 4l, highest first
    const u32x4 c = reinterpret_cast<const u32x4*>(h)[63 - lane];
    const int sum = (int)(c.x + c.y + c.z + c.w);
    const int incl = wave_inclusive_scan(sum);
    const int excl = incl - sum;
    const uint64_t hit = __ballot(excl < kr && incl >= kr);
    const int src = (int)__builtin_ctzll(hit);
    int a = excl, d = 252 - 4 * lane;
    if (a + (int)c.w >= kr) {
      d += 3;
    } else if (a + (int)(c.w + c.z) >= kr) {
      a += (int)c.w;
      d += 2;
    } else if (a + (int)(c.w + c.z + c.y) >= kr) {
      a += (int)(c.w + c.z);
      d += 1;
    } else {
      a += (int)(c.w + c.z + c.y);
    }
    d = __builtin_amdgcn_readlane(d, src);
    a = __builtin_amdgcn_readlane(a, src);
    kr -= a;
    prefix |= (uint32_t)d << shift;
    pmask |= 255u << shift;
  }
  thr = prefix;
  take_eq = kr;
}

// Emits the selection held in the "> T" (gt) and "== T" (eq) bitmaps of a
// row of nw words, taking the first take_eq set bits of eq, in ascending
// index order.  Thread t owns words [t W, t W + W).  pf / pn: this thread's
// count of fetchable / non-negative prediction entries (bookkeeping).
// Returns the misses.
__device__ __forceinline__ int emit_bitmaps(const uint32_t* gt, const uint32_t* eq, int nw,
                                            int take_eq, int k, int32_t* __restrict__ out,
                                            const int32_t* s_pred, int32_t* __restrict__ pos_row,
                                            int32_t* __restrict__ miss_row, int pf, int pn,
                                            ScanBufs& sb, int& fetchable) {
  const int W = (nw + kTopkThreads - 1) / kTopkThreads;
  const int w0 = (int)threadIdx.x * W;
  uint32_t g[kMaxWords], e[kMaxWords];
  int gc = 0, ec = 0;
#pragma unroll
  for (int w = 0; w < kMaxWords; ++w) {
    const bool in = w < W && w0 + w < nw;
    g[w] = in ? gt[w0 + w] : 0u;
    e[w] = in ? eq[w0 + w] : 0u;
    gc += __popc(g[w]);
    ec += __popc(e[w]);
  }
  // Both totals are below 2^16 (#gt < k, #eq <= candidates), so one scan
  // of the packed pair gives both prefixes.
  int ex, ep, tx, tp;
  block_scan_pair<kTopkWaves>(gc | (ec << 16), pf | (pn << 16), sb, ex, ep, tx, tp);
  const int gt_before = ex & 0xFFFF;
  const int eq_before = ex >> 16;
  int take = take_eq - eq_before;
  const int j0 = gt_before + (eq_before < take_eq ? eq_before : take_eq);
#pragma unroll
  for (int w = 0; w < kMaxWords; ++w) {
    const int pe = __popc(e[w]);
    const int tw = take < 0 ? 0 : (take > pe ? pe : take);
    g[w] |= lowest_bits(e[w], tw);
    take -= tw;
  }
  int j = j0;
  if (pos_row == nullptr) {
#pragma unroll
    for (int w = 0; w < kMaxWords; ++w) {
      for (uint32_t x = g[w]; x != 0u; x &= x - 1u) {
        if (j < k) out[j] = (w0 + w) * 32 + __ffs(x) - 1;
        ++j;
      }
    }
    return 0;
  }
  // Each selected entry is looked up once: hits get their prediction row
  // now, misses are marked and get slot rows after the scan of miss counts.
  fetchable = tp & 0xFFFF;
  const int plen = tp >> 16;
  uint32_t mm[kMaxWords];
  int my_miss = 0;
#pragma unroll
  for (int w = 0; w < kMaxWords; ++w) {
    mm[w] = 0u;
    for (uint32_t x = g[w]; x != 0u; x &= x - 1u) {
      const int b = __ffs(x) - 1;
      const int c = (w0 + w) * 32 + b;
      const int hit = find_in(s_pred, plen, c);
      if (j < k) {
        out[j] = c;
        if (hit >= 0) {
          pos_row[j] = hit;
        } else {
          mm[w] |= 1u << b;
          ++my_miss;
        }
      }
      ++j;
    }
  }
  int mtot;
  int mr = block_scan<kTopkWaves>(my_miss, sb, mtot);
  int jb = j0;  // output position of word w's first selected entry
#pragma unroll
  for (int w = 0; w < kMaxWords; ++w) {
    for (uint32_t x = mm[w]; x != 0u; x &= x - 1u) {
      const int b = __ffs(x) - 1;
      const int jj = jb + __popc(g[w] & ((1u << b) - 1u));
      pos_row[jj] = k + mr;
      miss_row[mr] = (w0 + w) * 32 + b;
      ++mr;
    }
    jb += __popc(g[w]);
  }
  return mtot;
}

// Filter-path LDS layout (words): the prediction, scratch (same place as
// the radix path's), the selection's four 256-counter histograms, candidate
// keys (whose first
// kBins words hold the bound histogram before any candidate is written),
// candidate indices, then the two bitmaps of the row.
constexpr int kFPred = 0;
constexpr int kFScr = 2 * kBins;
constexpr int kFWaveHist = kFScr + kScratchInts;
constexpr int kFKey = kFWaveHist + 4 * 256;
constexpr int kFIdx = kFKey + kFilterCap;
constexpr int kFBits = kFIdx + kFilterCap;
static_assert(kFPred + kMaxK <= kFScr, "prediction region");
static_assert(4 * kTopkWaves + 24 <= kScratchInts, "scratch region");

struct FilterLds {
  int32_t* s_pred;
  ScanBufs sb;
  int* bcast;  // 8 ints
  uint32_t* whist;  // 4 x 256 counters
  uint32_t* fkey;
  int32_t* fidx;
  uint32_t* bits;
  __device__ explicit FilterLds(uint32_t* smem)
      : s_pred(reinterpret_cast<int32_t*>(smem + kFPred)),
        sb{reinterpret_cast<int*>(smem + kFScr), 0},
        bcast(reinterpret_cast<int*>(smem + kFScr) + 4 * kTopkWaves),
        whist(smem + kFWaveHist),
        fkey(smem + kFKey),
        fidx(reinterpret_cast<int32_t*>(smem + kFIdx)),
        bits(smem + kFBits) {}
};

// Given cnt candidates in LDS (every key of the selection among them; the
// bitmaps and the selection's histograms cleared before a barrier), finds
// T, emits the selection and does the bookkeeping.  Returns the misses.
__device__ __forceinline__ int finish_select(FilterLds& L, int cnt, int n, int64_t n_max, int k,
                                             int32_t* __restrict__ out,
                                             const int32_t* __restrict__ pred_row, bool book,
                                             int32_t* __restrict__ pos_row,
                                             int32_t* __restrict__ miss_row, int& fetchable) {
  constexpr int PR = kMaxK / kTopkThreads;
  const int tid = threadIdx.x;
  const int nw = (n + 31) >> 5;
  uint32_t* gt = L.bits;
  uint32_t* eq = gt + nw;
  // The prediction is loaded now and stored once T is known.
  int32_t pv[PR];
#pragma unroll
  for (int r = 0; r < PR; ++r) {
    const int p = tid + kTopkThreads * r;
    pv[r] = (book && pred_row != nullptr && p < k) ? pred_row[p] : -1;
  }
  uint32_t thr;
  int take_eq;
  block_select(L.fkey, cnt, k, L.whist, thr, take_eq);
  int pf = 0, pn = 0;
  if (book) {
#pragma unroll
    for (int r = 0; r < PR; ++r) {
      const int p = tid + kTopkThreads * r;
      if (p < k) L.s_pred[p] = pv[r];
      pf += (pv[r] >= 0 && (int64_t)pv[r] < n_max) ? 1 : 0;
      pn += pv[r] >= 0 ? 1 : 0;
    }
  }
  for (int i = tid; i < cnt; i += kTopkThreads) {
    const uint32_t x = L.fkey[i];
    const int c = L.fidx[i];
    if (x > thr) atomicOr(&gt[c >> 5], 1u << (c & 31));
    else if (x == thr) atomicOr(&eq[c >> 5], 1u << (c & 31));
  }
  __syncthreads();
  return emit_bitmaps(gt, eq, nw, take_eq, k, out, L.s_pred, book ? pos_row : nullptr, miss_row,
                      pf, pn, L.sb, fetchable);
}

// One-workgroup filter path for a row of n keys (k < n <= kFilterMaxN):
// candidates are the keys >= a bound taken from G group maxima per thread
// (1024 G >= k).  ONE (n_max <= kChunk): the row is loaded over its whole
// storage, so that the loads need not wait for its length, and stays in
// registers.  Returns false, having written nothing, when more than
// kFilterCap keys pass the bound.
template <int G, bool ONE>
__device__ bool filter_select(const float* __restrict__ row, int n, int64_t n_max, int k,
                              uint32_t* smem, int32_t* __restrict__ out,
                              const int32_t* __restrict__ pred_row, bool book,
                              int32_t* __restrict__ pos_row, int32_t* __restrict__ miss_row,
                              int& misses, int& fetchable) {
  FilterLds L(smem);
  uint32_t* hist = L.fkey;  // before any candidate is written
  const int nw = (n + 31) >> 5;
  const bool vec = (reinterpret_cast<uintptr_t>(row) & 15u) == 0 && (n_max & 3) == 0;

  uint32_t key[32];
  uint32_t gmax[G];
#pragma unroll
  for (int g = 0; g < G; ++g) gmax[g] = 0u;
  if (ONE) {
    load_tile<kTopkThreads>(row, n, (int)n_max, 0, vec, key);
    group_max<G>(key, gmax);
  } else {
    for (int c0 = 0; c0 < n; c0 += kChunk) {
      uint32_t kk[32];
      load_tile<kTopkThreads>(row, n, n, c0, vec, kk);
      group_max<G>(kk, gmax);
    }
  }
  clear(hist, kBins);
  clear(L.bits, 2 * nw);
  clear(L.whist, 4 * 256);
  __syncthreads();

  // The bound: lowest key of the bin holding the k-th largest group maximum.
#pragma unroll
  for (int g = 0; g < G; ++g) atomicAdd(&hist[gmax[g] >> 21], 1u);
  __syncthreads();
  int d0, above;
  pick_bin_fast<kTopkThreads>(hist, k, L.sb, L.bcast, d0, above);
  const uint32_t bound = (uint32_t)d0 << 21;

  // Candidates: every key >= bound.
  int cnt = 0;
  for (int c0 = 0; c0 < n; c0 += kChunk) {
    uint32_t kk[32];
    if (ONE) {
#pragma unroll
      for (int b = 0; b < 32; ++b) kk[b] = key[b];
    } else {
      load_tile<kTopkThreads>(row, n, n, c0, vec, kk);
    }
    const uint32_t m = pass_mask<kTopkThreads>(kk, c0, n, bound);
    int tot;
    const int off = cnt + block_scan<kTopkWaves>(__popc(m), L.sb, tot);
    put_candidates<kTopkThreads>(kk, m, c0, off, kFilterCap, L.fkey, L.fidx);
    cnt += tot;
  }
  __syncthreads();
  if (cnt > kFilterCap) return false;
  misses = finish_select(L, cnt, n, n_max, k, out, pred_row, book, pos_row, miss_row, fetchable);
  return true;
}

// ------------------------------------------------------- split filter path

// A row of up to kSplitMaxN keys can be filtered by S = ceil(n_max /
// kSegKeys) workgroups of kSegThreads threads, one per segment of kSegKeys
// entries.  Each hands over the keys of its segment that are >= a bound
// from its own group maxima (at least min(k, keys in the segment) of them,
// so every key of the row's selection that lies in the segment is among
// them), up to kSegCap; the row's workgroup then selects from those.
constexpr int kSegThreads = 256;
constexpr int kSegWaves = kSegThreads / 64;
constexpr int kSegKeys = kSegThreads * 32;
constexpr int kSegCap = 2048;
constexpr int kSplitMaxK = 256;
constexpr int kSplitMaxN = 8 * kSegKeys;

template <int G>
__global__ __launch_bounds__(kSegThreads) void k_topk_seg(
    const float* __restrict__ scores, const int32_t* __restrict__ lens, int H, int Q, int BH,
    int64_t n_max, int k, int S, uint32_t* __restrict__ ckey, int32_t* __restrict__ cidx,
    int32_t* __restrict__ ccnt) {
  __shared__ uint32_t hist[kBins];
  __shared__ int scr[4 * kSegWaves + 8];
  const int tid = threadIdx.x;
  int bh, t;
  xcd_tile_map(blockIdx.x, Q * S, BH, bh, t);
  const int j = t / S;
  const int s = t - j * S;
  const int64_t rowid = (int64_t)bh * Q + j;
  const float* row = scores + rowid * n_max;
  const int seg0 = s * kSegKeys;
  const bool vec = (reinterpret_cast<uintptr_t>(row) & 15u) == 0 && (n_max & 3) == 0;
  // Loads first (they do not depend on the row's length).
  uint32_t key[32];
  load_tile<kSegThreads>(row, (int)n_max, (int)n_max, seg0, vec, key);
  const int n = (int)clamp_len(lens[bh / H], n_max);
  const int lim = n - (seg0 + 4 * tid);
#pragma unroll
  for (int b = 0; b < 32; ++b) key[b] = koff<kSegThreads>(b) < lim ? key[b] : 0u;
  const int seg_n = n - seg0 < 0 ? 0 : (n - seg0 > kSegKeys ? kSegKeys : n - seg0);
  int32_t* cnt_out = ccnt + rowid * S + s;
  if (n <= k || seg_n == 0) {
    if (tid == 0) *cnt_out = 0;
    return;
  }
  const int ks = k < seg_n ? k : seg_n;
  uint32_t gmax[G];
#pragma unroll
  for (int g = 0; g < G; ++g) gmax[g] = 0u;
  group_max<G>(key, gmax);
  for (int i = tid; i < kBins; i += kSegThreads) hist[i] = 0u;
  __syncthreads();
#pragma unroll
  for (int g = 0; g < G; ++g) atomicAdd(&hist[gmax[g] >> 21], 1u);
  __syncthreads();
  ScanBufs sb{scr, 0};
  int d0, above;
  pick_bin_fast<kSegThreads>(hist, ks, sb, scr + 4 * kSegWaves, d0, above);
  const uint32_t m = pass_mask<kSegThreads>(key, seg0, n, (uint32_t)d0 << 21);
  int tot;
  const int off = block_scan<kSegWaves>(__popc(m), sb, tot);
  const int64_t base = (rowid * S + s) * kSegCap;
  put_candidates<kSegThreads>(key, m, seg0, off, kSegCap, ckey + base, cidx + base);
  if (tid == 0) *cnt_out = tot;
}

// The row's side of the split path: gathers the segments' candidates into
// LDS.  Returns false (nothing written) when a segment overflowed or the
// total exceeds kFilterCap.
__device__ bool merge_select(int64_t rowid, int S, const uint32_t* __restrict__ ckey,
                             const int32_t* __restrict__ cidx, const int32_t* __restrict__ ccnt,
                             int n, int64_t n_max, int k, uint32_t* smem,
                             int32_t* __restrict__ out, const int32_t* __restrict__ pred_row,
                             bool book, int32_t* __restrict__ pos_row,
                             int32_t* __restrict__ miss_row, int& misses, int& fetchable) {
  FilterLds L(smem);
  const int tid = threadIdx.x;
  const int nw = (n + 31) >> 5;
  int* seg_cnt = L.bcast + 8;  // S <= 8 counts, then S offsets
  clear(L.bits, 2 * nw);
  clear(L.whist, 4 * 256);
  if (tid < 64) {
    const int c = tid < S ? ccnt[rowid * S + tid] : 0;
    const uint64_t over = __ballot(c > kSegCap);
    const int incl = wave_inclusive_scan(c);
    if (tid < S) {
      seg_cnt[tid] = c;
      seg_cnt[8 + tid] = incl - c;
    }
    if (tid == 63) {
      L.bcast[4] = incl;
      L.bcast[5] = over != 0ull ? 1 : 0;
    }
  }
  __syncthreads();
  const int cnt = L.bcast[4];
  if (L.bcast[5] != 0 || cnt > kFilterCap) return false;
  const int64_t base = rowid * S * kSegCap;
  for (int i = tid; i < S * kSegCap; i += kTopkThreads) {
    const int s = i / kSegCap;
    const int r = i - s * kSegCap;
    if (r < seg_cnt[s]) {
      L.fkey[seg_cnt[8 + s] + r] = ckey[base + i];
      L.fidx[seg_cnt[8 + s] + r] = cidx[base + i];
    }
  }
  __syncthreads();
  misses = finish_select(L, cnt, n, n_max, k, out, pred_row, book, pos_row, miss_row, fetchable);
  return true;
}

// ------------------------------------------------------------------ kernel

enum TopkMode { kModeFilterOne = 0, kModeFilterMulti = 1, kModeMerge = 2 };

struct SplitArgs {
  const uint32_t* ckey;
  const int32_t* cidx;
  const int32_t* ccnt;
  int S;
};

template <int G, int MODE>
__global__ __launch_bounds__(kTopkThreads) void k_topk(
    const float* __restrict__ scores, const int32_t* __restrict__ lens, int H, int Q, int BH,
    int64_t n_max, int k, int32_t* __restrict__ out0, int32_t* __restrict__ out1,
    int64_t out_stride, const int32_t* __restrict__ pred, int32_t* __restrict__ pos,
    int32_t* __restrict__ miss, int32_t* __restrict__ counts, int cand_cap, int cache_cap,
    int filter, SplitArgs split) {
  extern __shared__ uint32_t smem[];
  uint32_t* hist = smem;  // two copies during pass 0
  int* scr = reinterpret_cast<int*>(smem + 2 * kBins);
  int32_t* cand = reinterpret_cast<int32_t*>(smem + 2 * kBins + kScratchInts);  // also the prediction
  uint32_t* cache = reinterpret_cast<uint32_t*>(cand + cand_cap);

  int bh, j;
  xcd_tile_map(blockIdx.x, Q, BH, bh, j);
  const int n = (int)clamp_len(lens[bh / H], n_max);
  const int64_t rowid = (int64_t)bh * Q + j;
  const float* row = scores + rowid * n_max;
  int32_t* out = ((j == 0) ? out0 : out1) + (int64_t)bh * out_stride;
  const bool do_book = (pos != nullptr) && j == 0;
  const int tid = threadIdx.x;
  if (tid == 0) scr[20] = 0;  // running count (candidates, or misses of a short row)
  const int32_t* pred_row = pred != nullptr ? pred + (int64_t)bh * k : nullptr;
  int32_t* pos_row = do_book ? pos + (int64_t)bh * k : nullptr;
  int32_t* miss_row = do_book ? miss + (int64_t)bh * k : nullptr;

  Book bk{nullptr, 0, nullptr, miss_row};
  int fetchable = 0;
  int misses = 0;

  bool done = false;
  if (n <= k) {
    // Every valid key is selected: entry c is c itself.
    if (do_book) {
      const int packed = load_prediction(pred_row, k, n_max, cand, scr);
      fetchable = packed & 0xFFFF;
      bk = Book{pred_row != nullptr ? cand : nullptr, packed >> 16, pos_row, miss_row};
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
    done = true;
  } else if (MODE == kModeMerge) {
    done = merge_select(rowid, split.S, split.ckey, split.cidx, split.ccnt, n, n_max, k, smem,
                        out, pred_row, do_book, pos_row, miss_row, misses, fetchable);
  } else if (filter && n <= kFilterMaxN) {
    done = filter_select<G, MODE == kModeFilterOne>(row, n, n_max, k, smem, out, pred_row,
                                                     do_book, pos_row, miss_row, misses,
                                                     fetchable);
  }
  if (!done) {
    // Radix path over the whole row.
    const bool cached = ((n + 31) & ~31) <= cache_cap;
    clear(hist, 2 * kBins);
    if (tid == 0) scr[20] = 0;  // the filter path may have used this scratch
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
      bk = Book{pred_row != nullptr ? cand : nullptr, packed >> 16, pos_row, miss_row};
    }
    if (cached) misses = emit_ordered(CachedKeys{cache}, n, thr, kr, k, out, bk, scr);
    else misses = emit_ordered(GlobalKeys{row}, n, thr, kr, k, out, bk, scr);
  }

  if (!do_book) return;
  for (int tt = misses + tid; tt < k; tt += kTopkThreads) miss_row[tt] = -1;
  if (tid == 0) {
    const int valid = n < k ? n : k;
    counts[bh] = misses;
    counts[BH + bh] = valid - misses;
    counts[2 * BH + bh] = fetchable;
  }
}

template <int G>
hipError_t launch_seg(const float* scores, const int32_t* lens, int H, int Q, int BH,
                      int64_t n_max, int k, int S, const TopkScratch& ts, hipStream_t s) {
  hipLaunchKernelGGL(k_topk_seg<G>, dim3(BH * Q * S), dim3(kSegThreads), 0, s, scores, lens, H, Q,
                     BH, n_max, k, S, ts.ckey, ts.cidx, ts.ccnt);
  return hipGetLastError();
}

}  // namespace

size_t topk_scratch_bytes(int B, int H, int Q, int64_t n_max, int k) {
  if (k > kSplitMaxK || n_max > kSplitMaxN || n_max <= 0) return 0;
  const int64_t S = (n_max + kSegKeys - 1) / kSegKeys;
  const int64_t rows = (int64_t)B * H * Q;
  return (size_t)(rows * S * kSegCap * 8 + rows * S * 4 + 256);
}

TopkScratch topk_scratch(void* ws, int B, int H, int Q, int64_t n_max) {
  TopkScratch t{nullptr, nullptr, nullptr};
  if (ws == nullptr) return t;
  const int64_t S = (n_max + kSegKeys - 1) / kSegKeys;
  const int64_t rows = (int64_t)B * H * Q;
  uint8_t* p = static_cast<uint8_t*>(ws);
  t.ckey = reinterpret_cast<uint32_t*>(p);
  t.cidx = reinterpret_cast<int32_t*>(p + rows * S * kSegCap * 4);
  t.ccnt = reinterpret_cast<int32_t*>(p + rows * S * kSegCap * 8);
  return t;
}

hipError_t launch_topk(const float* scores, const int32_t* lens, int B, int H, int Q,
                       int64_t n_max, int k, int32_t* out0, int32_t* out1,
                       int64_t out_stride_bh, const TopkBook* book, const TopkScratch* scratch,
                       hipStream_t s) {
  const int BH = B * H;
  if (BH == 0) return hipSuccess;
  const DeviceInfo& di = device_info();
  static bool attr_set[64] = {false};
  if (di.device >= 0 && di.device < 64 && !attr_set[di.device]) {
    const void* fns[] = {reinterpret_cast<const void*>(k_topk<1, kModeFilterOne>),
                         reinterpret_cast<const void*>(k_topk<2, kModeFilterOne>),
                         reinterpret_cast<const void*>(k_topk<4, kModeFilterOne>),
                         reinterpret_cast<const void*>(k_topk<1, kModeFilterMulti>),
                         reinterpret_cast<const void*>(k_topk<2, kModeFilterMulti>),
                         reinterpret_cast<const void*>(k_topk<4, kModeFilterMulti>),
                         reinterpret_cast<const void*>(k_topk<1, kModeMerge>)};
    for (const void* f : fns)
      (void)hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, di.lds_per_block);
    attr_set[di.device] = true;
  }
  const bool do_book = book != nullptr && book->pos != nullptr;
  // LDS words for the radix path: two histogram copies, scratch, candidates
  // (also the prediction, so at least k), then the cached row (whole 32-word
  // groups).
  const int64_t lds_words = di.lds_per_block / 4;
  const int64_t fixed = 2 * kBins + kScratchInts;
  const int64_t cand_min = ((k > kCandMin ? k : kCandMin) + 31) & ~int64_t(31);
  const int64_t n_round = (n_max + 31) & ~int64_t(31);
  int64_t cache_cap = (lds_words - fixed - cand_min) & ~int64_t(31);
  if (cache_cap > n_round) cache_cap = n_round;
  if (cache_cap < 4096) cache_cap = 0;
  int64_t cand_cap = (lds_words - fixed - cache_cap) & ~int64_t(31);
  if (cand_cap > 1 << 20) cand_cap = 1 << 20;
  const int64_t filter_words = kFBits + 2 * ((std::min<int64_t>(n_max, kFilterMaxN) + 31) / 32);
  const int filter = filter_words <= lds_words ? 1 : 0;
  const size_t shmem = (size_t)std::max<int64_t>(fixed + cand_cap + cache_cap,
                                                 filter ? filter_words : 0) * 4;
  SplitArgs split{nullptr, nullptr, nullptr, 0};
  const bool use_split = filter && scratch != nullptr && scratch->ckey != nullptr &&
                         k <= kSplitMaxK && n_max <= kSplitMaxN;
  if (use_split) {
    // Group maxima per segment thread: at least 4k of them over a segment.
    const int S = (int)((n_max + kSegKeys - 1) / kSegKeys);
    const int g = k <= 64 ? 1 : k <= 128 ? 2 : 4;
    hipError_t e = g == 1 ? launch_seg<1>(scores, lens, H, Q, BH, n_max, k, S, *scratch, s)
                 : g == 2 ? launch_seg<2>(scores, lens, H, Q, BH, n_max, k, S, *scratch, s)
                          : launch_seg<4>(scores, lens, H, Q, BH, n_max, k, S, *scratch, s);
    if (e != hipSuccess) return e;
    split = SplitArgs{scratch->ckey, scratch->cidx, scratch->ccnt, S};
  }
  // Groups per thread of the one-workgroup filter: up to 4096 group maxima,
  // at least k of them and 4k where k <= 1024.
  const int g = k <= 256 ? 1 : k <= 512 ? 2 : 4;
  const bool one = n_max <= kChunk;
  auto kern = use_split ? k_topk<1, kModeMerge>
              : one ? (g == 1 ? k_topk<1, kModeFilterOne> : g == 2 ? k_topk<2, kModeFilterOne>
                                                                   : k_topk<4, kModeFilterOne>)
                    : (g == 1 ? k_topk<1, kModeFilterMulti>
                              : g == 2 ? k_topk<2, kModeFilterMulti> : k_topk<4, kModeFilterMulti>);
  hipLaunchKernelGGL(kern, dim3(BH * Q), dim3(kTopkThreads), shmem, s, scores, lens, H, Q, BH,
                     n_max, k, out0, out1, out_stride_bh, do_book ? book->pred : nullptr,
                     do_book ? book->pos : nullptr, do_book ? book->miss : nullptr,
                     do_book ? book->counts : nullptr, (int)cand_cap, (int)cache_cap, filter, split);
  return hipGetLastError();
}

}  // namespace dd
