// Per-row top-k selection, I = argtopk(alpha, k) (paper-daily summary of
// DualDecoder, core-formulas section; "Top-k" box of Figure 1 on the arXiv
// page), with the prediction bookkeeping of the layer step fused into the
// current-query rows.
//
// One workgroup of 512 threads (two waves per SIMD) per row.  Scores become
// order-preserving 32-bit keys; the selection is every key > T plus the
// first k - #(> T) keys equal to T (lower index wins), T being the exact
// k-th largest key, written in ascending index order.
//
// Filter path (rows of up to kFilterMaxN keys).  Thread t reads float4
// t + 512 u of each 32768-key tile (u < 16, coalesced) and keeps the maximum
// of each of its G groups of float4s.  With 512 G >= k groups, the lowest
// key B of the 11-bit digit bin holding the k-th largest group maximum has
// at least k keys >= B, and real score rows have only a small multiple of
// k of them.  Those candidates are located through the float4 maxima (a row
// of one tile is cached in LDS for this) and compacted by index; T is then
// found by 8-bit radix selection over the candidates alone, the selection
// is scattered into "> T" and "== T" bitmaps of the row, and each thread
// emits its consecutive bitmap words after block scans of their popcounts.
// More candidates than the list holds (a row dominated by ties, say) send
// the row to the radix path.
//
// Radix path (every other row): MSB-first radix selection with 11 + 11 + 10
// bit digits over the whole row, then the same comparison emit 32 kNT keys at
// a time.
//
// For the current-query row of the layer step, the filter path marks the
// prediction in a bitmap of the row: a selected entry without a mark is a
// miss and gets slot row k, k + 1, ... in ascending order, and a marked one
// keeps its position in the prediction as its slot row (each prediction
// entry finds its place in the selection from the final bitmap and the
// per-word output positions).  The radix path looks each selected index up
// in the prediction list (each thread walks it forward alongside its own
// ascending entries).
// With attention fused in, that workgroup then runs the sparse decode
// attention of the current query over its selection (DualDecoder, Figure 1
// "Attention" box) from the slot rows and entry numbers it left in LDS,
// reading each miss from host memory and storing it into its slot row.
#include <algorithm>
#include <climits>
#include <mutex>

#include "attn_body.h"
#include "dd_device.h"
#include "dd_internal.h"
#include "gather_body.h"
#include "gather_res.h"

namespace dd {

namespace {

// Threads per row workgroup: two waves per SIMD, so that one wave's LDS
// and barrier latencies overlap the other's work (one wave per SIMD left
// every phase of the selection chain exposed: 19.06 against 17.48 us for
// the 7B layer's top-k, bookkeeping and attention).
constexpr int kNT = 512;
constexpr int kNW = kNT / 64;
constexpr int kBins = 2048;              // 11-bit digits
constexpr int kU = 16;                   // float4 per thread per tile
constexpr int kTile = 4 * kNT * kU;      // 32768 keys
static_assert(kTile == kPrefetchMaxScoreRow, "selection-side prefetch needs cached rows");
constexpr int kMaxK = 4096;              // largest k (DD_MAX_K)
constexpr int kPR = kMaxK / kNT;         // prediction entries per thread
constexpr int kCapCached = 2560;         // candidates of a row cached in LDS
constexpr int kCapLong = 8192;           // candidates of a longer row
constexpr int kFilterMaxN = 1 << 17;     // longest row of the filter path
constexpr int kMaxWords = kFilterMaxN / 32 / kNT;  // bitmap words per thread
constexpr int kScr = 64;                 // scan buffers and broadcasts
constexpr int kSegKeys = 32 * kNT;       // keys per radix-path emit segment
static_assert(kSegKeys < 65536, "a segment's counts fit 16 bits");
constexpr int kAttrDevices = 64;         // devices whose launch attributes are kept

typedef float f32x4 __attribute__((ext_vector_type(4)));

// LDS layout (words): histogram, scratch, candidate indices and keys (the
// attention's scratch once the selection is emitted), then region C: the
// cached row, and once the candidates' keys are read from it, the two
// bitmaps of the row, the prediction and, for the fused attention, every
// entry's slot row and row index.
constexpr int kLHist = 0;                           // kBins counters
constexpr int kLScr = kLHist + kBins;               // kScr ints
constexpr int kLIdx = kLScr + kScr;                 // candidate indices
template <bool CACHED>
struct Lay {
  static constexpr int cap = CACHED ? kCapCached : kCapLong;
  static constexpr int key = kLIdx + cap;           // candidate keys
  static constexpr int c = key + cap;               // region C
  static constexpr int bits = 2 * ((CACHED ? kTile : kFilterMaxN) / 32);
  static constexpr int pred = c + bits;             // prediction, then slot rows, then rows
  static constexpr int end = pred + 3 * kMaxK;
  static constexpr int words = CACHED ? (c + kTile > end ? c + kTile : end) : end;
};
static_assert(Lay<true>::words * 4 <= 160 * 1024, "cached layout exceeds LDS");
static_assert(Lay<false>::words * 4 <= 160 * 1024, "long-row layout exceeds LDS");
static_assert(4 * 256 <= kBins, "selection histograms fit the bound histogram");
// attention scratch, both queries (dual-token): per-wave partials of the
// kNW waves and up to 32 chunk partials of D+2 each; the tail of region C
// for a cached row, the candidate lists otherwise (both free once the
// selection is emitted)
constexpr int kAttnScratchWords =
    (int)(sizeof(AttnLds<128, 2, kNW>) + 15) / 16 * 4 + 2 * 32 * (128 + 2);
static_assert(Lay<true>::end + kAttnScratchWords <= Lay<true>::words, "dual scratch fits (cached)");
static_assert(kLIdx + kAttnScratchWords <= Lay<false>::c, "dual scratch fits (long rows)");
// Rows kept across steps: each entry's row in the previous step's slot (or
// -1), in the candidate lists (free once the selection is emitted), beside
// the attention scratch.
template <bool CACHED>
constexpr int kLOld = CACHED ? kLIdx : kLIdx + kAttnScratchWords;
static_assert(kLOld<true> + kMaxK <= Lay<true>::c, "old rows fit (cached)");
static_assert(kLOld<false> + kMaxK <= Lay<false>::c, "old rows fit (long rows)");

__device__ __forceinline__ void clear(uint32_t* p, int words) {
  for (int i = threadIdx.x; i < words; i += kNT) p[i] = 0u;
}

// Lowest `take` set bits of w (take <= popcount(w)).
__device__ __forceinline__ uint32_t lowest_bits(uint32_t w, int take) {
  uint32_t r = 0u;
#pragma unroll 1
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
#pragma unroll 1
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (s[mid] < c) lo = mid + 1;
    else hi = mid;
  }
  return (lo < len && s[lo] == c) ? lo : -1;
}

// First position of the ascending list s[0, len) whose entry is >= c.
__device__ __forceinline__ int lower_bound_in(const int32_t* s, int len, int c) {
  int lo = 0, hi = len;
#pragma unroll 1
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (s[mid] < c) lo = mid + 1;
    else hi = mid;
  }
  return lo;
}

// Start of a thread's walk through the prediction: none of its entries can
// lie in the thread's words (kNoStart), or to be found by binary search.
constexpr int kNoStart = -1;
constexpr int kSearchStart = -2;

// The smallest fp32 value whose key is >= b (-inf when every value's is).
__device__ __forceinline__ float key_floor(uint32_t b) {
  if (b >= 0x80000000u) return __uint_as_float(b & 0x7FFFFFFFu);
  if (b <= 0x007FFFFFu) return -INFINITY;
  return __uint_as_float(~b);
}

// The digit holding the kr-th largest counted key in a histogram of kBins
// counters (digit order = key order) and the count in larger digits.
// Thread t scans the 8 digits below kBins - 8t, one block scan orders the
// threads, and the thread whose digits reach kr broadcasts through out2.
// With top, also the highest digit that counts anything.
__device__ __forceinline__ void pick_bin(const uint32_t* hist, int kr, ScanBufs& sb, int* out2,
                                         int& digit, int& above, int* top_digit = nullptr) {
  constexpr int BPT = kBins / kNT;
  const int top = kBins - BPT * (int)threadIdx.x;  // this thread's digits: [top - BPT, top)
  int c[BPT];
  int sum = 0;
#pragma unroll
  for (int i = 0; i < BPT; ++i) {
    c[i] = (int)hist[top - 1 - i];
    sum += c[i];
  }
  int total;
  const int before = block_scan<kNW>(sum, sb, total);
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
  if (top_digit != nullptr && before == 0 && sum > 0) {
    int d = top - BPT;
    bool found = false;
#pragma unroll
    for (int i = 0; i < BPT; ++i) {
      if (!found && c[i] > 0) {
        found = true;
        d = top - 1 - i;
      }
    }
    out2[2] = d;
  }
  __syncthreads();
  digit = out2[0];
  above = out2[1];
  if (top_digit != nullptr) *top_digit = out2[2];
}

// The exact k-th largest key T among the cnt candidate keys (k <= cnt <=
// CAP) and how many keys equal to T the selection takes, by MSB-first radix
// selection with 8-bit digits.  Thread t holds candidates t + kNT r in
// registers; pass p counts into its own 256-counter histogram h4 + 256 p,
// cleared by the caller before a barrier that precedes this call.  After
// each pass's barrier every wave scans the histogram itself, so T needs no
// broadcast.  When the chosen digit's keys are exactly the ones still
// needed, all of them are taken and the passes stop: T is then just below
// the digit's lowest key and no key equal to T is taken.  With P > 0 the
// top P bits of T are known to be those of prefix0 (every key that can be
// among the k largest has them); keys without them are not counted, and
// the digits start below them (the last one narrower when 32 - P is not a
// multiple of 8).
template <int CAP>
__device__ __forceinline__ void select_kth(const uint32_t* fkey, int cnt, int k, uint32_t* h4,
                                           uint32_t& thr, int& take_eq, uint32_t prefix0 = 0u,
                                           int P = 0) {
  constexpr int R = CAP / kNT;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // Register r holds candidate tid + kNT r; the loops over r stop at the
  // first r with kNT r >= cnt (a uniform branch), so only the live ones run.
  uint32_t x[R];
#pragma unroll
  for (int r = 0; r < R; ++r) x[r] = 0u;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    if (kNT * r >= cnt) break;
    if (tid + kNT * r < cnt) x[r] = fkey[tid + kNT * r];
  }
  uint32_t pmask = P > 0 ? ~0u << (32 - P) : 0u;
  uint32_t prefix = prefix0 & pmask;
  int kr = k;
#pragma unroll 1
  for (int pass = 0, hi = 32 - P; hi > 0; ++pass, hi -= 8) {
    const int shift = hi > 8 ? hi - 8 : 0;
    const uint32_t dmask = (1u << (hi - shift)) - 1u;
    uint32_t* h = h4 + 256 * pass;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      if (kNT * r >= cnt) break;
      if (tid + kNT * r < cnt && (x[r] & pmask) == prefix) atomicAdd(&h[(x[r] >> shift) & dmask], 1u);
    }
    __syncthreads();
    // lane l holds digits 255 - 4l .. 252 - 4l, highest first
    const u32x4 c = reinterpret_cast<const u32x4*>(h)[63 - lane];
    const int sum = (int)(c.x + c.y + c.z + c.w);
    const int incl = wave_inclusive_scan(sum);
    const int excl = incl - sum;
    const uint64_t hit = __ballot(excl < kr && incl >= kr);
    const int src = (int)__builtin_ctzll(hit);
    int a = excl, d = 252 - 4 * lane, cd = (int)c.x;
    if (a + (int)c.w >= kr) {
      d += 3;
      cd = (int)c.w;
    } else if (a + (int)(c.w + c.z) >= kr) {
      a += (int)c.w;
      d += 2;
      cd = (int)c.z;
    } else if (a + (int)(c.w + c.z + c.y) >= kr) {
      a += (int)(c.w + c.z);
      d += 1;
      cd = (int)c.y;
    } else {
      a += (int)(c.w + c.z + c.y);
    }
    d = __builtin_amdgcn_readlane(d, src);
    a = __builtin_amdgcn_readlane(a, src);
    cd = __builtin_amdgcn_readlane(cd, src);
    kr -= a;
    prefix |= (uint32_t)d << shift;
    pmask |= dmask << shift;
    if (kr == cd && prefix != 0u) {  // every key of this digit is taken
      thr = prefix - 1u;
      take_eq = 0;
      return;
    }
  }
  thr = prefix;
  take_eq = kr;
}

// Where the selection goes: the output row and, for bookkeeping rows, the
// prediction (in LDS) and its length, and the slot row (lpos) and row index
// (lcur) of every selected entry, in LDS for the fused attention.
struct Sink {
  int32_t* out;
  const int32_t* s_pred;  // the prediction list (radix path), or nullptr
  int plen;
  int32_t* lpos;
  int32_t* lcur;
  // Filter path: the prediction as a bitmap of the row (pbits, nwords
  // words), and where the emit leaves the final selection bitmap (gfin) and
  // the output position of each word's first selected entry (wpre).
  const uint32_t* pbits = nullptr;
  uint32_t* gfin = nullptr;
  int32_t* wpre = nullptr;
  int nwords = 0;
  // Position in the caller's prediction of each s_pred entry when the list
  // had to be sorted (nullptr: s_pred is the prediction as given).
  const int32_t* s_ppos = nullptr;
};

// Emits, in ascending index order, the selected entries of this thread's
// bitmap words w0, w0 + 1, ...: g (the "> T" set, extended here by the
// taken "== T" bits of e).  gt_before / eq_before: the counts in lower
// words; misses are numbered from miss_base.  lo: where this thread's walk
// through the prediction starts (kNoStart, kSearchStart or a position).
// Returns this block's misses.
template <int MAXW>
__device__ __forceinline__ int emit_words(uint32_t (&g)[MAXW], const uint32_t (&e)[MAXW], int w0,
                                          int gt_before, int eq_before, int take_eq, int k,
                                          const Sink& sk, ScanBufs& sb, int miss_base, int lo) {
  int take = take_eq - eq_before;
  const int j0 = gt_before + (eq_before < take_eq ? eq_before : take_eq);
#pragma unroll
  for (int w = 0; w < MAXW; ++w) {
    const int pe = __popc(e[w]);
    const int tw = take < 0 ? 0 : (take > pe ? pe : take);
    g[w] |= lowest_bits(e[w], tw);
    take -= tw;
  }
  int j = j0;
  if (sk.pbits != nullptr) {
    // Hits and misses straight from the prediction's bitmap: an entry is a
    // miss where the prediction has no bit.  Every entry's slot row is
    // first a placeholder (INT_MAX); misses get rows k, k + 1, ... after the
    // scan of miss counts, and hits get their prediction position from
    // prediction_rows once the final bitmap and word positions are stored.
    uint32_t mm[MAXW];
    int my_miss = 0;
#pragma unroll
    for (int w = 0; w < MAXW; ++w) {
      const int wi = w0 + w;
      mm[w] = g[w] != 0u ? g[w] & ~sk.pbits[wi] : 0u;
      my_miss += __popc(mm[w]);
#pragma unroll 1
      for (uint32_t x = g[w]; x != 0u; x &= x - 1u) {
        const int c = wi * 32 + __ffs(x) - 1;
        if (j < k) {
          sk.out[j] = c;
          sk.lcur[j] = c;
          sk.lpos[j] = INT_MAX;
        }
        ++j;
      }
    }
    int mtot;
    int mr = miss_base + block_scan<kNW>(my_miss, sb, mtot);
    int jb = j0;  // output position of word w's first selected entry
    const int wn = (sk.nwords + kNT - 1) / kNT;  // words per thread: only those are this thread's
#pragma unroll
    for (int w = 0; w < MAXW; ++w) {
#pragma unroll 1
      for (uint32_t x = mm[w]; x != 0u; x &= x - 1u) {
        const int b = __ffs(x) - 1;
        const int jj = jb + __popc(g[w] & ((1u << b) - 1u));
        if (jj < k) sk.lpos[jj] = k + mr;
        ++mr;
      }
      if (w < wn && w0 + w < sk.nwords) {
        sk.gfin[w0 + w] = g[w];
        sk.wpre[w0 + w] = jb;
      }
      jb += __popc(g[w]);
    }
    return mtot;
  }
  if (sk.s_pred == nullptr) {
#pragma unroll
    for (int w = 0; w < MAXW; ++w) {
#pragma unroll 1
      for (uint32_t x = g[w]; x != 0u; x &= x - 1u) {
        if (j < k) sk.out[j] = (w0 + w) * 32 + __ffs(x) - 1;
        ++j;
      }
    }
    return 0;
  }
  // Each selected entry is looked up once: hits get their prediction row
  // now, misses are marked and get slot rows after the scan of miss counts.
  // The selected entries and the prediction list both ascend (the list was
  // sorted by order_prediction if it had to be), so the lookup walks the
  // list forward from lo; the first of equal entries, the lowest position
  // in the prediction, gives the row.
  if (lo == kSearchStart) {
    bool any = false;
#pragma unroll
    for (int w = 0; w < MAXW; ++w) any = any || g[w] != 0u;
    lo = any ? lower_bound_in(sk.s_pred, sk.plen, w0 * 32) : kNoStart;
  }
  uint32_t mm[MAXW];
  int my_miss = 0;
#pragma unroll
  for (int w = 0; w < MAXW; ++w) {
    mm[w] = 0u;
#pragma unroll 1
    for (uint32_t x = g[w]; x != 0u; x &= x - 1u) {
      const int b = __ffs(x) - 1;
      const int c = (w0 + w) * 32 + b;
      int hit = -1;
      if (lo >= 0) {
#pragma unroll 1
        while (lo < sk.plen && sk.s_pred[lo] < c) ++lo;
        if (lo < sk.plen && sk.s_pred[lo] == c) hit = lo;
      }
      if (j < k) {
        sk.out[j] = c;
        sk.lcur[j] = c;
        if (hit >= 0) {
          sk.lpos[j] = sk.s_ppos != nullptr ? sk.s_ppos[hit] : hit;
        } else {
          mm[w] |= 1u << b;
          ++my_miss;
        }
      }
      ++j;
    }
  }
  int mtot;
  int mr = miss_base + block_scan<kNW>(my_miss, sb, mtot);
  int jb = j0;  // output position of word w's first selected entry
#pragma unroll
  for (int w = 0; w < MAXW; ++w) {
#pragma unroll 1
    for (uint32_t x = mm[w]; x != 0u; x &= x - 1u) {
      const int b = __ffs(x) - 1;
      const int jj = jb + __popc(g[w] & ((1u << b) - 1u));
      sk.lpos[jj] = k + mr;
      ++mr;
    }
    jb += __popc(g[w]);
  }
  return mtot;
}

// Emits the selection held in the "> T" (gt) and "== T" (eq) bitmaps of a
// row of nw words; thread t owns words [t W, t W + W).  pf / pn: this
// thread's count of fetchable / non-negative prediction entries.  Returns
// the misses; sets fetchable and sk.plen from the block totals.  lo: the
// start of this thread's walk through the prediction (see emit_words).
template <int MAXW>
__device__ __forceinline__ int emit_bitmaps(const uint32_t* gt, const uint32_t* eq, int nw,
                                            int take_eq, int k, Sink& sk, int pf, int pn,
                                            ScanBufs& sb, int& fetchable, int lo) {
  const int W = (nw + kNT - 1) / kNT;
  const int w0 = (int)threadIdx.x * W;
  uint32_t g[MAXW], e[MAXW];
  int gc = 0, ec = 0;
#pragma unroll
  for (int w = 0; w < MAXW; ++w) {
    const bool in = w < W && w0 + w < nw;
    g[w] = in ? gt[w0 + w] : 0u;
    e[w] = in ? eq[w0 + w] : 0u;
    gc += __popc(g[w]);
    ec += __popc(e[w]);
  }
  // Both totals are below 2^16 (#gt < k, #eq <= the candidates), so one
  // scan of the packed pair gives both prefixes.
  int ex, ep, tx, tp;
  block_scan_pair<kNW>(gc | (ec << 16), pf | (pn << 16), sb, ex, ep, tx, tp);
  fetchable = tp & 0xFFFF;
  if (sk.s_pred != nullptr) sk.plen = tp >> 16;
  return emit_words<MAXW>(g, e, w0, ex & 0xFFFF, ex >> 16, take_eq, k, sk, sb, 0, lo);
}

// emit_bitmaps for a bookkeeping row of the filter path when no key equal
// to T is taken (take_eq = 0; with distinct scores the last radix pass
// always ends that way): the selection is the "> T" bitmap alone, so each
// thread knows its misses (selected, no mark in the prediction's bitmap)
// before the scan, and one scan of (selected | misses, fetchable | non-
// negative prediction entries) gives every position.  Same outputs as
// emit_bitmaps + emit_words.
template <int MAXW>
__device__ __forceinline__ int emit_book_fast(const uint32_t* gt, int nw, int k, Sink& sk, int pf,
                                              int pn, ScanBufs& sb, int& fetchable) {
  const int W = (nw + kNT - 1) / kNT;
  const int w0 = (int)threadIdx.x * W;
  uint32_t g[MAXW], mm[MAXW];
  int gc = 0, mc = 0;
#pragma unroll
  for (int w = 0; w < MAXW; ++w) {
    const bool in = w < W && w0 + w < nw;
    g[w] = in ? gt[w0 + w] : 0u;
    mm[w] = g[w] != 0u ? g[w] & ~sk.pbits[w0 + w] : 0u;
    gc += __popc(g[w]);
    mc += __popc(mm[w]);
  }
  // Both totals are at most k < 2^16.
  int ex, ep, tx, tp;
  block_scan_pair<kNW>(gc | (mc << 16), pf | (pn << 16), sb, ex, ep, tx, tp);
  fetchable = tp & 0xFFFF;
  int j = ex & 0xFFFF;  // output position of this thread's first entry
  int mr = ex >> 16;    // misses in lower words
#pragma unroll
  for (int w = 0; w < MAXW; ++w) {
    const int jb = j;
#pragma unroll 1
    for (uint32_t x = g[w]; x != 0u; x &= x - 1u) {
      const int b = __ffs(x) - 1;
      const int c = (w0 + w) * 32 + b;
      if (j < k) {
        sk.out[j] = c;
        sk.lcur[j] = c;
        const bool miss = (mm[w] >> b) & 1u;
        sk.lpos[j] = miss ? k + mr : INT_MAX;
        mr += miss ? 1 : 0;
      }
      ++j;
    }
    if (w < W && w0 + w < nw) {
      sk.gfin[w0 + w] = g[w];
      sk.wpre[w0 + w] = jb;
    }
  }
  return tx >> 16;
}

// Stores this thread's prediction entries in s_pred; counts the fetchable
// (in [0, n_max)) and non-negative ones.
__device__ __forceinline__ void store_prediction(const int32_t (&pv)[kPR], int k, int64_t n_max,
                                                 int32_t* s_pred, int& pf, int& pn) {
  pf = pn = 0;
#pragma unroll
  for (int r = 0; r < kPR; ++r) {
    if (kNT * r >= k) break;  // entries r and later are -1 (see the load)
    const int p = (int)threadIdx.x + kNT * r;
    if (p < k) s_pred[p] = pv[r];
    pf += (pv[r] >= 0 && (int64_t)pv[r] < n_max) ? 1 : 0;
    pn += pv[r] >= 0 ? 1 : 0;
  }
}

// Makes the stored prediction list s_pred (k entries) ascend as unsigned
// values, so that hits can be found by walking or binary search and the
// non-negative entries come first; returns the position in the prediction
// of each list entry, or nullptr when the list already ascends (the layer
// step's own speculated sets always do).  Otherwise the (value, position)
// pairs are sorted in LDS (bitonic, sortbuf: 2 * kMaxK words), so that
// among equal entries the lowest position comes first, which is the row the
// prefetch filled first; s_ppos (kMaxK words, inside sortbuf) receives the
// positions.  The caller's barrier after store_prediction must precede.
__device__ __forceinline__ const int32_t* order_prediction(int32_t* s_pred, int k,
                                                           uint32_t* sortbuf, int* flag) {
  const int tid = threadIdx.x;
  int unsorted = 0;
  for (int p = tid + 1; p < k; p += kNT)
    unsorted |= (uint32_t)s_pred[p - 1] > (uint32_t)s_pred[p] ? 1 : 0;
  // Block-wide OR through one LDS word (the runtime's own barrier-OR would
  // add static LDS beside the kernel's full dynamic allocation).
  if (tid == 0) *flag = 0;
  __syncthreads();
  if (unsorted) *flag = 1;
  __syncthreads();
  const bool any = *flag != 0;
  __syncthreads();  // every thread has read the flag before its word is reused
  if (!any) return nullptr;
  int n2 = 1;
  while (n2 < k) n2 <<= 1;
  uint64_t* a = reinterpret_cast<uint64_t*>(sortbuf);
  for (int i = tid; i < n2; i += kNT)
    a[i] = i < k ? ((uint64_t)(uint32_t)s_pred[i] << 32) | (uint32_t)i : ~0ull;
  for (int size = 2; size <= n2; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      __syncthreads();
      for (int t = tid; t < (n2 >> 1); t += kNT) {
        const int lo = 2 * t - (t & (stride - 1));
        const int hi = lo + stride;
        const uint64_t x = a[lo], y = a[hi];
        if ((x > y) == ((lo & size) == 0)) {
          a[lo] = y;
          a[hi] = x;
        }
      }
    }
  }
  __syncthreads();
  // Every entry to registers before the positions overwrite the buffer.
  uint64_t mine[kPR];
#pragma unroll
  for (int r = 0; r < kPR; ++r) {
    const int i = tid + kNT * r;
    mine[r] = i < k ? a[i] : 0ull;
  }
  __syncthreads();
  int32_t* s_ppos = reinterpret_cast<int32_t*>(sortbuf);
#pragma unroll
  for (int r = 0; r < kPR; ++r) {
    const int i = tid + kNT * r;
    if (i < k) {
      s_pred[i] = (int32_t)(uint32_t)(mine[r] >> 32);
      s_ppos[i] = (int32_t)(uint32_t)mine[r];
    }
  }
  __syncthreads();
  return s_ppos;
}

// Filter path, bookkeeping rows: sets the prediction's bit of every entry
// in [0, n) in pbits (cleared before a barrier that precedes this call)
// and counts this thread's fetchable (in [0, n_max)) and non-negative
// prediction entries.
__device__ __forceinline__ void mark_prediction(const int32_t (&pv)[kPR], int k, int n,
                                                int64_t n_max, uint32_t* pbits, int& pf, int& pn) {
  pf = pn = 0;
  // (left to the compiler: with the atomic inside, it keeps this loop rolled)
  for (int r = 0; r < kPR; ++r) {
    if (kNT * r >= k) break;  // entries r and later are -1
    const int c = pv[r];
    if (c >= 0 && c < n) atomicOr(&pbits[c >> 5], 1u << (c & 31));
    pf += (c >= 0 && (int64_t)c < n_max) ? 1 : 0;
    pn += c >= 0 ? 1 : 0;
  }
}

// Filter path, bookkeeping rows, after the emit and a barrier: each
// prediction entry p that the selection holds gives the slot row of that
// entry, p; with repeats the lowest p wins.  Entry j of the selection is
// wpre[w] plus the selected bits below it in word w.
__device__ __forceinline__ void prediction_rows(const int32_t (&pv)[kPR], int k, int n,
                                                const uint32_t* gfin, const int32_t* wpre,
                                                int32_t* lpos) {
#pragma unroll
  for (int r = 0; r < kPR; ++r) {
    if (kNT * r >= k) break;
    const int p = (int)threadIdx.x + kNT * r;
    const int c = pv[r];
    if (p < k && c >= 0 && c < n) {
      const uint32_t gw = gfin[c >> 5];
      const int b = c & 31;
      if ((gw >> b) & 1u) {
        const int j = wpre[c >> 5] + __popc(gw & ((1u << b) - 1u));
        if (j < k) atomicMin(&lpos[j], p);
      }
    }
  }
}

// ---------------------------------------------------------------- filter path

// Float4 q = t + kNT u of the tile starting at entry c0 of the row, u < kU,
// loaded unconditionally (clamped to the first nload entries).  vec: the
// row is 16-byte aligned and n_max is a multiple of 4, so every float4
// holding an entry < nload lies inside the row's storage.
__device__ __forceinline__ void load_tile(const float* __restrict__ row, int nload, int c0,
                                          bool vec, f32x4 (&v)[kU]) {
  const char* base = reinterpret_cast<const char*>(row);
  const uint32_t q0 = ((uint32_t)c0 >> 2) + threadIdx.x;
  if (vec) {
    const uint32_t nq = (uint32_t)(nload + 3) >> 2;
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      uint32_t q = q0 + kNT * u;
      q = q < nq ? q : nq - 1u;
      v[u] = *reinterpret_cast<const f32x4*>(base + q * 16u);
    }
  } else {
    const uint32_t last = (uint32_t)nload - 1u;
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const uint32_t i = 4u * (q0 + kNT * u);
      float f[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t ie = i + e < last ? i + e : last;
        f[e] = *reinterpret_cast<const float*>(base + ie * 4u);
      }
      v[u] = f32x4{f[0], f[1], f[2], f[3]};
    }
  }
}

// Maximum of the entries of float4 v (first entry i) below n; -inf if none.
__device__ __forceinline__ float max_valid(const f32x4& v, int i, int n) {
  const float a = i < n ? v.x : -INFINITY;
  const float b = i + 1 < n ? v.y : -INFINITY;
  const float c = i + 2 < n ? v.z : -INFINITY;
  const float d = i + 3 < n ? v.w : -INFINITY;
  return fmaxf(fmaxf(a, b), fmaxf(c, d));
}

// Component c of v, with no indexing into registers.
__device__ __forceinline__ float f4_at(const f32x4& v, int c) {
  return c == 0 ? v.x : (c == 1 ? v.y : (c == 2 ? v.z : v.w));
}

// Entries of float4 v (first entry i) below n and >= fb, as bits 0..3.
__device__ __forceinline__ uint32_t passing(const f32x4& v, int i, int n, float fb) {
  return ((i < n && v.x >= fb) ? 1u : 0u) | ((i + 1 < n && v.y >= fb) ? 2u : 0u) |
         ((i + 2 < n && v.z >= fb) ? 4u : 0u) | ((i + 3 < n && v.w >= fb) ? 8u : 0u);
}

// The filter path for a row of n keys (k < n <= kFilterMaxN).  CACHED: the
// row fits one tile (n_max <= kTile) and is kept in LDS; otherwise tiles are
// read again from global memory.  G groups of float4s per thread.  Returns
// false, having written nothing, when more than the list's capacity of
// keys pass the bound.
template <int G, bool CACHED, typename AfterRow>
__device__ __forceinline__ bool filter_select(const float* __restrict__ row, int n, int64_t n_max, int k,
                              uint32_t* smem, Sink& sk, bool book, const int32_t (&pv)[kPR],
                              const f32x4 (&v0)[CACHED ? kU : 1], int& misses, int& fetchable,
                              AfterRow&& after_row) {
  using L = Lay<CACHED>;
  constexpr int CAP = L::cap;
  static_assert(G >= 1 && G <= kU, "a group holds at least one float4");
  constexpr int UPG = kU / G;  // float4s per group and tile
  const int tid = threadIdx.x;
  uint32_t* hist = smem + kLHist;
  ScanBufs sb{reinterpret_cast<int*>(smem + kLScr), 0};
  int* bcast = reinterpret_cast<int*>(smem + kLScr) + 4 * kNW;
  int32_t* fidx = reinterpret_cast<int32_t*>(smem + kLIdx);
  uint32_t* fkey = smem + L::key;
  uint32_t* regc = smem + L::c;
  const bool vec = (reinterpret_cast<uintptr_t>(row) & 15u) == 0 && (n_max & 3) == 0;
  const int tiles = CACHED ? 1 : (n + kTile - 1) / kTile;

  // Group maxima (and, for a cached row, the float4 maxima).
  float gmax[G];
#pragma unroll
  for (int g = 0; g < G; ++g) gmax[g] = -INFINITY;
  float f4max[CACHED ? kU : 1];
  for (int tl = 0; tl < tiles; ++tl) {
    const int c0 = tl * kTile;
    f32x4 v[kU];
    // A cached row was loaded over its whole storage at kernel entry (v0),
    // so that the loads need not wait for its length.
    if constexpr (CACHED) {
#pragma unroll
      for (int u = 0; u < kU; ++u) v[u] = v0[u];
    } else {
      load_tile(row, n, c0, vec, v);
    }
    // A tile whose entries are all below n needs no masks (a uniform
    // branch; the same maxima either way).
    if (n >= c0 + kTile) {
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int q = tid + kNT * u;
        if (CACHED) reinterpret_cast<f32x4*>(regc)[q] = v[u];
        const float m = fmaxf(fmaxf(v[u].x, v[u].y), fmaxf(v[u].z, v[u].w));
        if (CACHED) f4max[u] = m;
        gmax[u / UPG] = fmaxf(gmax[u / UPG], m);
      }
    } else {
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int q = tid + kNT * u;
        if (CACHED) reinterpret_cast<f32x4*>(regc)[q] = v[u];
        const float m = max_valid(v[u], c0 + 4 * q, n);
        if (CACHED) f4max[u] = m;
        gmax[u / UPG] = fmaxf(gmax[u / UPG], m);
      }
    }
  }
  __syncthreads();  // also orders the caller's clear of hist
  after_row();      // the caller's work once the row's registers are free

  // The bound: lowest key of the digit bin holding the k-th largest group
  // maximum (kNT G >= k groups).
#pragma unroll
  for (int g = 0; g < G; ++g) atomicAdd(&hist[order_key(gmax[g]) >> 21], 1u);
  __syncthreads();
  int d0, above, dtop;
  pick_bin(hist, k, sb, bcast, d0, above, &dtop);
  const float fb = key_floor((uint32_t)d0 << 21);
  clear(hist, 4 * 256);  // the selection's histograms (ordered by the next barrier)
  // The k largest keys have top digits in [d0, dtop] (dtop: the row
  // maximum's), so they share the leading bits on which d0 and dtop agree.
  const uint32_t ddiff = (uint32_t)(d0 ^ dtop);
  const int kp = ddiff == 0u ? 11 : __clz(ddiff) - 21;

  // Candidates: every entry >= fb, by index.  Count, scan, then write.
  int cnt;
  if (CACHED) {
    uint32_t um = 0u;
    if (n >= kTile) {
#pragma unroll
      for (int u = 0; u < kU; ++u) um |= f4max[u] >= fb ? (1u << u) : 0u;
    } else {
#pragma unroll
      for (int u = 0; u < kU; ++u)
        um |= (4 * (tid + kNT * u) < n && f4max[u] >= fb) ? (1u << u) : 0u;
    }
    // The first two of this thread's candidate float4s are read together
    // and kept in registers for both passes; any others are read per pass.
    const f32x4* rc4 = reinterpret_cast<const f32x4*>(regc);
    uint32_t rest = um;
    const int q0 = rest != 0u ? tid + kNT * (__ffs(rest) - 1) : -1;
    rest &= rest - 1u;
    const int q1 = rest != 0u ? tid + kNT * (__ffs(rest) - 1) : -1;
    rest &= rest - 1u;
    const f32x4 f0 = rc4[q0 >= 0 ? q0 : tid];
    const f32x4 f1 = rc4[q1 >= 0 ? q1 : tid];
    const uint32_t m0 = q0 >= 0 ? passing(f0, 4 * q0, n, fb) : 0u;
    const uint32_t m1 = q1 >= 0 ? passing(f1, 4 * q1, n, fb) : 0u;
    int my = __popc(m0) + __popc(m1);
#pragma unroll 1
    for (uint32_t x = rest; x != 0u; x &= x - 1u) {
      const int q = tid + kNT * (__ffs(x) - 1);
      my += __popc(passing(rc4[q], 4 * q, n, fb));
    }
    int off = block_scan<kNW>(my, sb, cnt);
    if (cnt > CAP) return false;
    // Each candidate's index and key, from the float4 it sits in.
#pragma unroll 1
    for (uint32_t m = m0; m != 0u; m &= m - 1u) {
      const int c = __ffs(m) - 1;
      fidx[off] = 4 * q0 + c;
      fkey[off] = order_key(f4_at(f0, c));
      ++off;
    }
#pragma unroll 1
    for (uint32_t m = m1; m != 0u; m &= m - 1u) {
      const int c = __ffs(m) - 1;
      fidx[off] = 4 * q1 + c;
      fkey[off] = order_key(f4_at(f1, c));
      ++off;
    }
#pragma unroll 1
    for (uint32_t x = rest; x != 0u; x &= x - 1u) {
      const int q = tid + kNT * (__ffs(x) - 1);
      const f32x4 f = rc4[q];
#pragma unroll 1
      for (uint32_t m = passing(f, 4 * q, n, fb); m != 0u; m &= m - 1u) {
        const int c = __ffs(m) - 1;
        fidx[off] = 4 * q + c;
        fkey[off] = order_key(f4_at(f, c));
        ++off;
      }
    }
  } else {
    cnt = 0;
    for (int tl = 0; tl < tiles; ++tl) {
      const int c0 = tl * kTile;
      f32x4 v[kU];
      load_tile(row, n, c0, vec, v);
      uint32_t mk[kU / 8];  // 4 bits per float4
      int my = 0;
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const uint32_t m = passing(v[u], c0 + 4 * (tid + kNT * u), n, fb);
        if ((u & 7) == 0) mk[u >> 3] = 0u;
        mk[u >> 3] |= m << (4 * (u & 7));
        my += __popc(m);
      }
      int tot;
      int off = cnt + block_scan<kNW>(my, sb, tot);
      if (cnt + tot > CAP) return false;
#pragma unroll
      for (int w = 0; w < kU / 8; ++w) {
#pragma unroll 1
        for (uint32_t m = mk[w]; m != 0u; m &= m - 1u) {
          const int b = __ffs(m) - 1;
          const int u = 8 * w + (b >> 2);
          fidx[off++] = c0 + 4 * (tid + kNT * u) + (b & 3);
        }
      }
      cnt += tot;
    }
    __syncthreads();
    for (int i = tid; i < cnt; i += kNT) fkey[i] = order_key(row[fidx[i]]);
  }
  __syncthreads();  // candidate keys written; region C free for bitmaps

  // Bitmaps and the prediction in region C.
  const int nw = (n + 31) >> 5;
  uint32_t* gt = regc;
  uint32_t* eq = regc + nw;
  // The prediction as a bitmap of the row, where the prediction list would
  // sit (the filter path never stores the list).
  uint32_t* pbits = smem + L::pred;
  clear(regc, 2 * nw);
  if (book) clear(pbits, nw);  // ordered before the marks by select_kth's barriers
  int pf = 0, pn = 0;
  uint32_t thr;
  int take_eq;
  select_kth<CAP>(fkey, cnt, k, hist, thr, take_eq, (uint32_t)d0 << 21, kp);
  if (book) {
    mark_prediction(pv, k, n, n_max, pbits, pf, pn);
    sk.pbits = pbits;
    sk.gfin = gt;
    sk.wpre = reinterpret_cast<int32_t*>(eq);  // read into registers by the emit first
    sk.nwords = nw;
  }
  for (int i = tid; i < cnt; i += kNT) {
    const uint32_t x = fkey[i];
    const int c = fidx[i];
    if (x > thr) atomicOr(&gt[c >> 5], 1u << (c & 31));
    else if (x == thr) atomicOr(&eq[c >> 5], 1u << (c & 31));
  }
  __syncthreads();
  // A cached row has at most kTile / 32 bitmap words: 4 per thread.
  constexpr int MAXW = CACHED ? kTile / 32 / kNT : kMaxWords;
  misses = (book && take_eq == 0)
               ? emit_book_fast<MAXW>(gt, nw, k, sk, pf, pn, sb, fetchable)
               : emit_bitmaps<MAXW>(gt, eq, nw, take_eq, k, sk, pf, pn, sb, fetchable, kNoStart);
  if (book) {
    __syncthreads();  // final bitmap and word positions stored
    prediction_rows(pv, k, n, gt, reinterpret_cast<const int32_t*>(eq), sk.lpos);
  }
  return true;
}

// ---------------------------------------------------------------- maxima path

// The filter path from the scoring kernel's group maxima (kMaxGroup keys per
// group), for rows longer than one tile (launches with n_max > kTile; the
// rows of a launch with n_max <= kTile are cached in LDS whole, which is one
// memory round trip where this path makes two, maxima then candidates) of
// up to kFilterMaxN keys with at least k groups.  The
// bound B is the lowest key of the 11-bit digit bin holding the k-th largest
// group maximum, so at least k keys reach it, and a group whose maximum is
// below B holds no key that does: only the groups whose maximum reaches B
// are read, and their keys >= B form the candidate list in ascending index
// order.  T follows by radix selection over the candidates, and the
// selection is emitted straight from the list.  The row itself is never
// streamed whole.
constexpr int kCapM = 4096;                               // candidates
constexpr int kGM4 = kFilterMaxN / kMaxGroup / 4 / kNT;  // maxima float4s per thread (8)
constexpr int kPM = 8;                                    // candidate float4s per thread and round

// LDS of the maxima path: the candidate group list in the bitmap area of
// region C, the candidate indices and keys past the bookkeeping arrays (a
// cached row's layout) or in the candidate area (a longer row's); both are
// free again once the selection is emitted.
template <bool CACHED>
struct LayM {
  static constexpr int groups = Lay<CACHED>::c;
  static constexpr int idx = CACHED ? Lay<true>::end : kLIdx;
  static constexpr int key = idx + kCapM;
};
static_assert(LayM<true>::groups + kTile / kMaxGroup <= Lay<true>::pred, "group list (cached)");
static_assert(LayM<true>::key + kCapM <= Lay<true>::words, "candidates (cached)");
static_assert(LayM<false>::groups + kFilterMaxN / kMaxGroup <= Lay<false>::pred, "group list");
static_assert(LayM<false>::key + kCapM <= Lay<false>::c, "candidates (long rows)");

// Float4s of the maxima row each thread reads (consecutive ones).
__device__ __forceinline__ int maxima_w4(int64_t gstride) {
  const int64_t w = (gstride / 4 + kNT - 1) / kNT;
  return w < kGM4 ? (int)w : kGM4;
}

// This thread's maxima: float4s t W4 .. t W4 + W4 - 1 of the row (clamped to
// the row's storage; entries past the row's groups are masked later).
__device__ __forceinline__ void load_maxima(const float* __restrict__ gm_row, int64_t gstride,
                                            f32x4 (&gv)[kGM4]) {
  const int W4 = maxima_w4(gstride);
  const uint32_t last = (uint32_t)(gstride / 4) - 1u;
  const uint32_t q0 = threadIdx.x * (uint32_t)W4;
#pragma unroll
  for (int w = 0; w < kGM4; ++w) {
    uint32_t q = q0 + (uint32_t)w;
    q = q < last ? q : last;
    gv[w] = w < W4 ? *reinterpret_cast<const f32x4*>(gm_row + 4 * (size_t)q)
                   : f32x4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
  }
}

// First position of the list s[0, len) (ascending as unsigned values) whose
// entry is >= c as an unsigned value.
__device__ __forceinline__ int lower_bound_u32(const int32_t* s, int len, uint32_t c) {
  int lo = 0, hi = len;
#pragma unroll 1
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if ((uint32_t)s[mid] < c) lo = mid + 1;
    else hi = mid;
  }
  return lo;
}

// Returns false, having written nothing to the outputs, when the
// prediction is not in ascending order (the bitmap path takes it) or more
// than kCapM keys reach the bound; hist is then clear again.
template <bool CACHED>
__device__ __forceinline__ bool maxima_select(const float* __restrict__ row,
                                              const f32x4 (&gv)[kGM4], int64_t gstride, int n,
                                              int64_t n_max, int k, uint32_t* smem, Sink& sk,
                                              bool book, const int32_t (&pv)[kPR], int& misses,
                                              int& fetchable) {
  using LM = LayM<CACHED>;
  const int tid = threadIdx.x;
  uint32_t* hist = smem + kLHist;
  ScanBufs sb{reinterpret_cast<int*>(smem + kLScr), 0};
  int* bcast = reinterpret_cast<int*>(smem + kLScr) + 4 * kNW;
  int32_t* cg = reinterpret_cast<int32_t*>(smem + LM::groups);
  int32_t* fidx = reinterpret_cast<int32_t*>(smem + LM::idx);
  uint32_t* fkey = smem + LM::key;
  int32_t* s_pred = reinterpret_cast<int32_t*>(smem + Lay<CACHED>::pred);
  const int ng = (n + kMaxGroup - 1) / kMaxGroup;
  const int W4 = maxima_w4(gstride);
  const int g0 = tid * 4 * W4;  // this thread's first group
  const bool vec = (reinterpret_cast<uintptr_t>(row) & 15u) == 0 && (n_max & 3) == 0;

  int pf = 0, pn = 0;
  if (book) store_prediction(pv, k, n_max, s_pred, pf, pn);

  // The bound: the digit bin of the k-th largest group maximum.
  uint32_t gk[4 * kGM4];
  uint32_t gval = 0u;  // bit i: group g0 + i exists
#pragma unroll
  for (int w = 0; w < kGM4; ++w) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int i = 4 * w + e;
      const bool ok = w < W4 && g0 + i < ng;
      gk[i] = order_key(f4_at(gv[w], e));
      gval |= ok ? (1u << i) : 0u;
      if (ok) atomicAdd(&hist[gk[i] >> 21], 1u);
    }
  }
  __syncthreads();  // histogram complete; the prediction list stored
  int d0, above, dtop;
  pick_bin(hist, k, sb, bcast, d0, above, &dtop);
  const uint32_t bkey = (uint32_t)d0 << 21;
  const float fb = key_floor(bkey);
  clear(hist, 4 * 256);  // the selection's histograms (ordered by the barriers below)
  // As in the filter path: the k largest keys share the leading bits on
  // which d0 and the row maximum's digit agree.
  const uint32_t ddiff = (uint32_t)(d0 ^ dtop);
  const int kp = ddiff == 0u ? 11 : __clz(ddiff) - 21;

  // Candidate groups, and whether the prediction ascends.
  int unsorted = 0;
  if (book)
    for (int p = tid + 1; p < k; p += kNT)
      unsorted |= (uint32_t)s_pred[p - 1] > (uint32_t)s_pred[p] ? 1 : 0;
  uint32_t gsel = 0u;
#pragma unroll
  for (int i = 0; i < 4 * kGM4; ++i) gsel |= ((gval >> i) & 1u) && gk[i] >= bkey ? (1u << i) : 0u;
  int goff, eu, G, tu;
  block_scan_pair<kNW>(__popc(gsel), unsorted, sb, goff, eu, G, tu);
  if (tu != 0) {
    clear(hist, kBins);
    return false;
  }
#pragma unroll 1
  for (uint32_t x = gsel; x != 0u; x &= x - 1u) cg[goff++] = g0 + __ffs(x) - 1;
  __syncthreads();  // group list complete

  // Candidates: slot s of 4 G is float4 s & 3 of group cg[s >> 2]; each
  // round covers kNT * kPM slots, kPM consecutive ones per thread, so the
  // list comes out in ascending index order.
  const int nslots = 4 * G;
  const uint32_t nq = (uint32_t)(n + 3) >> 2;  // float4s holding an entry < n
  int cnt = 0;
#pragma unroll 1
  for (int r0 = 0; r0 < nslots; r0 += kNT * kPM) {
    const int s0 = r0 + tid * kPM;
    f32x4 v[kPM];
    int i0[kPM];
#pragma unroll
    for (int p = 0; p < kPM; ++p) {
      const int sl = s0 + p;
      const int gq = cg[sl < nslots ? sl >> 2 : 0];
      i0[p] = gq * kMaxGroup + 4 * (sl & 3);
      if (vec) {
        uint32_t q = (uint32_t)i0[p] >> 2;
        q = q < nq ? q : nq - 1u;
        v[p] = *reinterpret_cast<const f32x4*>(row + 4 * (size_t)q);
      } else {
        float f[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int ie = i0[p] + e < n ? i0[p] + e : n - 1;
          f[e] = row[ie];
        }
        v[p] = f32x4{f[0], f[1], f[2], f[3]};
      }
    }
    uint32_t m[kPM];
    int my = 0;
#pragma unroll
    for (int p = 0; p < kPM; ++p) {
      m[p] = s0 + p < nslots ? passing(v[p], i0[p], n, fb) : 0u;
      my += __popc(m[p]);
    }
    int tot;
    int off = cnt + block_scan<kNW>(my, sb, tot);
    if (cnt + tot > kCapM) {
      clear(hist, kBins);
      return false;
    }
#pragma unroll
    for (int p = 0; p < kPM; ++p) {
#pragma unroll 1
      for (uint32_t x = m[p]; x != 0u; x &= x - 1u) {
        const int c = __ffs(x) - 1;
        fidx[off] = i0[p] + c;
        fkey[off] = order_key(f4_at(v[p], c));
        ++off;
      }
    }
    cnt += tot;
  }
  __syncthreads();  // candidates complete

  uint32_t thr;
  int take_eq;
  select_kth<kCapM>(fkey, cnt, k, hist, thr, take_eq, bkey, kp);

  // Emit: thread t owns candidates [t E, t E + E) of the ascending list.
  constexpr int EM = kCapM / kNT;
  const int E = (cnt + kNT - 1) / kNT;
  const int c_beg = tid * E;
  uint32_t xs[EM];
  int cs_[EM];
  int gtc = 0, eqc = 0;
#pragma unroll
  for (int e = 0; e < EM; ++e) {
    if (e >= E) break;
    const int i = c_beg + e;
    xs[e] = i < cnt ? fkey[i] : 0u;
    cs_[e] = i < cnt ? fidx[i] : -1;
    gtc += (i < cnt && xs[e] > thr) ? 1 : 0;
    eqc += (i < cnt && xs[e] == thr) ? 1 : 0;
  }
  // Selected: every key > T, and the first take_eq keys equal to T in
  // index order (those need the count of equal keys in lower threads).
  uint32_t selm = 0u;  // bit e: owned candidate e is selected
  int take = 0;
  if (take_eq != 0) {
    int ex, ep, tx, tp;
    block_scan_pair<kNW>(gtc | (eqc << 16), 0, sb, ex, ep, tx, tp);
    take = take_eq - (ex >> 16);
  }
#pragma unroll
  for (int e = 0; e < EM; ++e) {
    if (e >= E) break;
    const bool in = c_beg + e < cnt;
    bool sel = in && xs[e] > thr;
    if (in && xs[e] == thr && take > 0) {
      sel = true;
      --take;
    }
    selm |= sel ? (1u << e) : 0u;
  }
  // Bookkeeping: each selected entry is looked up in the ascending
  // prediction list (binary search for the thread's first, then a walk).
  uint32_t hitm = 0u;
  int hpos[EM];
  if (book) {
    int lo = -1;
#pragma unroll
    for (int e = 0; e < EM; ++e) {
      hpos[e] = -1;
      if (e >= E) break;
      if ((selm >> e) & 1u) {
        const uint32_t c = (uint32_t)cs_[e];
        if (lo < 0) lo = lower_bound_u32(s_pred, k, c);
#pragma unroll 1
        while (lo < k && (uint32_t)s_pred[lo] < c) ++lo;
        if (lo < k && (uint32_t)s_pred[lo] == c) {
          hitm |= 1u << e;
          hpos[e] = lo;
        }
      }
    }
  }
  const int my_sel = __popc(selm);
  const int my_miss = my_sel - __popc(hitm);
  int ex, ep, tx, tp;
  block_scan_pair<kNW>(my_sel | (my_miss << 16), pf | (pn << 16), sb, ex, ep, tx, tp);
  int j = ex & 0xFFFF;  // selected entries in lower threads
  int mr = ex >> 16;
  fetchable = tp & 0xFFFF;
  misses = tx >> 16;
#pragma unroll
  for (int e = 0; e < EM; ++e) {
    if (e >= E) break;
    if ((selm >> e) & 1u) {
      if (j < k) {
        sk.out[j] = cs_[e];
        if (book) {
          sk.lcur[j] = cs_[e];
          sk.lpos[j] = ((hitm >> e) & 1u) ? hpos[e] : k + mr;
        }
      }
      mr += ((hitm >> e) & 1u) ? 0 : 1;
      ++j;
    }
  }
  return true;
}

// ----------------------------------------------------------------- radix path

// Where order_prediction may sort (2 * kMaxK words) on the paths that keep
// the prediction as a list: past the bookkeeping arrays of a cached row
// (the attention's scratch later), the candidate lists of a longer row.
template <bool CACHED>
__device__ __forceinline__ uint32_t* sort_buffer(uint32_t* smem) {
  return smem + (CACHED ? Lay<true>::end : kLIdx);
}
static_assert(Lay<true>::end + 2 * kMaxK <= Lay<true>::words, "prediction sort fits (cached)");
static_assert(kLIdx + 2 * kMaxK <= Lay<false>::c, "prediction sort fits (long rows)");

// Histogram over the row of digit (key >> shift) & dmask, for keys whose
// bits under pmask equal prefix.
__device__ __forceinline__ void row_hist(const float* __restrict__ row, int n, uint32_t pmask,
                                         uint32_t prefix, int shift, uint32_t dmask,
                                         uint32_t* hist) {
  constexpr int UN = 8;
  for (int i0 = threadIdx.x; i0 < n; i0 += UN * kNT) {
    uint32_t key[UN];
#pragma unroll
    for (int u = 0; u < UN; ++u) {
      const int i = i0 + u * kNT;
      key[u] = order_key(row[i < n ? i : n - 1]);
    }
#pragma unroll
    for (int u = 0; u < UN; ++u) {
      if (i0 + u * kNT < n && (key[u] & pmask) == prefix)
        atomicAdd(&hist[(key[u] >> shift) & dmask], 1u);
    }
  }
}

// The radix path: T over the whole row, then, 32 kNT keys at a time, thread
// t compares keys 32 t .. 32 t + 31 of the segment with T.
template <bool CACHED>
__device__ __forceinline__ int radix_select(const float* __restrict__ row, int n, int64_t n_max, int k,
                            uint32_t* smem, Sink& sk, bool book, const int32_t (&pv)[kPR],
                            int& fetchable) {
  const int tid = threadIdx.x;
  uint32_t* hist = smem + kLHist;
  ScanBufs sb{reinterpret_cast<int*>(smem + kLScr), 0};
  int* bcast = reinterpret_cast<int*>(smem + kLScr) + 4 * kNW;
  int32_t* s_pred = reinterpret_cast<int32_t*>(smem + Lay<CACHED>::pred);
  __syncthreads();
  clear(hist, kBins);
  __syncthreads();
  row_hist(row, n, 0u, 0u, 21, 0x7FFu, hist);
  __syncthreads();
  int d0, d1, d2, above;
  pick_bin(hist, k, sb, bcast, d0, above);
  int kr = k - above;
  clear(hist, kBins);
  __syncthreads();
  row_hist(row, n, 0xFFE00000u, (uint32_t)d0 << 21, 10, 0x7FFu, hist);
  __syncthreads();
  pick_bin(hist, kr, sb, bcast, d1, above);
  kr -= above;
  const uint32_t prefix = ((uint32_t)d0 << 21) | ((uint32_t)d1 << 10);
  clear(hist, kBins);
  __syncthreads();
  row_hist(row, n, 0xFFFFFC00u, prefix, 0, 0x3FFu, hist);
  __syncthreads();
  pick_bin(hist, kr, sb, bcast, d2, above);
  kr -= above;
  const uint32_t thr = prefix | (uint32_t)d2;

  int pf = 0, pn = 0;
  if (book) {
    store_prediction(pv, k, n_max, s_pred, pf, pn);
    __syncthreads();
    sk.s_ppos = order_prediction(s_pred, k, sort_buffer<CACHED>(smem), bcast);
    sk.s_pred = s_pred;
  }
  int out_run = 0, eq_run = 0, miss_run = 0;
  for (int seg0 = 0; seg0 < n; seg0 += kSegKeys) {
    const int base = seg0 + 32 * tid;
    uint32_t g[1] = {0u}, e[1] = {0u};
    if (base < n) {
#pragma unroll
      for (int b = 0; b < 32; ++b) {
        const int i = base + b;
        const uint32_t key = order_key(row[i < n ? i : n - 1]);
        g[0] |= (i < n && key > thr) ? (1u << b) : 0u;
        e[0] |= (i < n && key == thr) ? (1u << b) : 0u;
      }
    }
    int ex, ep, tx, tp;
    block_scan_pair<kNW>(__popc(g[0]) | (__popc(e[0]) << 16), pf | (pn << 16), sb, ex, ep, tx,
                         tp);
    if (seg0 == 0) {
      fetchable = tp & 0xFFFF;
      if (sk.s_pred != nullptr) sk.plen = tp >> 16;
    }
    // Per-segment counts stay below 2^16 (kSegKeys = 32 kNT keys).
    const int mtot = emit_words<1>(g, e, base / 32, out_run + (ex & 0xFFFF),
                                   eq_run + (ex >> 16), kr, k, sk, sb, miss_run, kSearchStart);
    out_run += tx & 0xFFFF;
    eq_run += tx >> 16;
    miss_run += mtot;
    pf = pn = 0;
  }
  return miss_run;
}

// ------------------------------------------------------------------ kernel

// Attention of the current query over its own selection (the layer step's
// last stage), done by the workgroup of each bookkeeping row right after its
// emit: slot rows and entry rows come from LDS, chunks of 128 entries as in
// the attention kernel, chunk partials merged the same way.  With selection
// by chunk landmarks (cs > 0) each of the ks selected entries stands for the
// 2^cs consecutive rows of its chunk, rows past the request's length left
// out; the slot holds them at 2^cs times the entry's slot position.  With
// out_spec set, the speculated query (plane 1) attends over the same rows
// too, each K/V row read once for both (the dual-token pipeline runs both
// tokens through the layer); the query count is a run-time value, so one
// body per element type serves both cases.
template <typename T, int D>
__device__ __forceinline__ void fused_attention_t(const FusedAttn& fa, int bh, int ks,
                                                  int32_t len, const int32_t* lpos,
                                                  const int32_t* lcur, const int32_t* lold,
                                                  float* scratch, const float* srow) {
  constexpr int NQ = 2;
  const int nq = fa.out_spec != nullptr ? 2 : 1;
  AttnLds<D, NQ, kNW>& lds = *reinterpret_cast<AttnLds<D, NQ, kNW>*>(scratch);
  float* part = scratch + (sizeof(AttnLds<D, NQ, kNW>) + 15) / 16 * 4;
  const int cs = fa.chunk_shift;
  const int k = ks << cs;  // rows attended (at most)
  const int64_t n_rows = fa.n_rows;
  const int64_t nv = clamp_len(len, n_rows);
  const int64_t slab = (int64_t)bh * 2 * k * D;
  const int64_t hslab = (int64_t)bh * n_rows * D;
  const bool kdev = fa.k_dev != nullptr;
  const AttnRows<T> R{static_cast<const T*>(fa.kslot) + slab, static_cast<const T*>(fa.vslot) + slab,
                      kdev ? nullptr : static_cast<const T*>(fa.k_host) + hslab,
                      static_cast<const T*>(fa.v_host) + hslab,
                      kdev ? static_cast<const T*>(fa.k_dev) + hslab : nullptr, 2 * k, k, n_rows,
                      lold != nullptr ? static_cast<const T*>(fa.old_vslot) + slab : nullptr};
  const int cmask = (1 << cs) - 1;
  auto entry = [&](int j, int& r, int& c, int& o) {
    o = -1;
    if (cs == 0) {  // one row per entry
      r = lpos[j];
      c = lcur[j];
      if (lold != nullptr) o = lold[j];
      return;
    }
    const int e = j >> cs;
    const int i = j & cmask;
    const int pe = lpos[e];
    const int ce = lcur[e];
    const int64_t row = ((int64_t)ce << cs) + i;
    const bool ok = ce >= 0 && pe >= 0 && row < nv;
    r = ok ? (pe << cs) + i : -1;
    c = ok ? (int)row : -1;
  };
  const int chunks = (k + kAttnChunk - 1) / kAttnChunk;
  const float* qrow = fa.q + (int64_t)bh * 2 * D;  // plane 0, then plane 1
  // Output pointers of query qi by value selects (an array indexed by qi
  // would live in scratch memory).
  auto out_of = [&](int qi) { return qi == 0 ? fa.out : fa.out_spec; };
  auto lse_of = [&](int qi) { return qi == 0 ? fa.lse : fa.lse_spec; };
  const int d = threadIdx.x;
  // All kNW waves attend each chunk of kAttnChunk entries, 128 / kNW each.
  for (int ch = 0; ch < chunks; ++ch) {
    float cm[NQ], cl[NQ], od[NQ];
    if (srow != nullptr) {
      AttnFetchS<T, D, NQ, kNW> f;
      attn_fetch_s<T, D, NQ, kNW>(R, srow, n_rows, nq, ch * kAttnChunk,
                                  min(k, (ch + 1) * kAttnChunk), entry, f, threadIdx.x);
      attn_finish_s<T, D, NQ, kNW>(R, f, lds, nq, cm, cl, od, threadIdx.x);
    } else if (kdev && lold == nullptr) {
      attend_chunk_n<T, D, NQ, true, kNW>(qrow, R, ch * kAttnChunk,
                                          min(k, (ch + 1) * kAttnChunk), fa.scale, entry, lds,
                                          nq, cm, cl, od);
    } else {
      attend_chunk_n<T, D, NQ, false, kNW>(qrow, R, ch * kAttnChunk,
                                           min(k, (ch + 1) * kAttnChunk), fa.scale, entry, lds,
                                           nq, cm, cl, od);
    }
    if (d < D) {
#pragma unroll
      for (int qi = 0; qi < NQ; ++qi) {
        if (qi >= nq) break;
        if (chunks == 1) {
          out_of(qi)[(int64_t)bh * D + d] = (cl[qi] > 0.f) ? od[qi] / cl[qi] : 0.f;
          if (d == 0 && lse_of(qi) != nullptr)
            lse_of(qi)[bh] = (cl[qi] > 0.f) ? cm[qi] + logf(cl[qi]) : -INFINITY;
        } else {
          float* pc = part + (qi * chunks + ch) * (D + 2);
          pc[d] = od[qi];
          if (d == 0) {
            pc[D] = cl[qi] > 0.f ? cm[qi] : -INFINITY;
            pc[D + 1] = cl[qi];
          }
        }
      }
    }
    __syncthreads();  // lds is reused by the next chunk; partials complete
  }
  if (chunks > 1 && d < D) {
#pragma unroll
    for (int qi = 0; qi < NQ; ++qi) {
      if (qi >= nq) break;
      float o, l;
      combine_chunks<D>(part + qi * chunks * (D + 2), chunks, d, o, l);
      out_of(qi)[(int64_t)bh * D + d] = o;
      if (d == 0 && lse_of(qi) != nullptr) lse_of(qi)[bh] = l;
    }
  }
}

// Bookkeeping of a layer whose rows are kept across steps, by the
// workgroup of a current-query row after its emit: every miss (slot row
// r >= k, key c) is looked up in the previous step's slot (lold[j]: its row
// there, or -1 when it must come over the host link), and the new slot's
// key list and the key -> row map are brought up to date: the misses' rows,
// then -1 on the rows no miss fills (and on the prediction's rows when
// there was no prediction, so no prefetch wrote them).  Returns the
// workgroup's count of misses read over the link (all threads).
__device__ __forceinline__ int resident_bookkeeping(const FusedAttn& fa, int bh, int k,
                                                    int misses, bool has_pred,
                                                    const int32_t* lpos, const int32_t* lcur,
                                                    int32_t* lold, ScanBufs sb) {
  const int tid = threadIdx.x;
  const int64_t rows = 2 * (int64_t)k;
  const int64_t ib = (int64_t)bh * rows;
  const int64_t wb = (int64_t)bh * fa.n_rows;
  int host = 0;
  for (int j = tid; j < k; j += kNT) {
    const int r = lpos[j];
    const int c = lcur[j];
    int o = -1;
    if (r >= k && r < rows && c >= 0 && (int64_t)c < fa.n_rows) {
      o = resident_row(fa.where, fa.old_idx, fa.n_rows, rows, bh, c);
      host += o < 0 ? 1 : 0;
      fa.new_idx[ib + r] = c;
      fa.where[wb + c] = r;
    }
    lold[j] = o;
  }
  const int64_t m = misses < k ? misses : k;
  for (int64_t r = (has_pred ? k + m : 0) + tid; r < rows; r += kNT)
    if (r < k || r >= k + m) fa.new_idx[ib + r] = -1;
  int total = 0;
  block_scan<kNW>(host, sb, total);
  return total;
}

// scratch: LDS for the attention of both queries (kAttnScratchWords).
// srow (or null): the score rows of (b, h) ([Q][n_rows]: the current query's,
// then the speculated one's); with them the logits of the selected keys
// are those scores, and only V rows are read.
__device__ __forceinline__ void fused_attention(const FusedAttn& fa, int bh, int ks, int32_t len,
                                                const int32_t* lpos, const int32_t* lcur,
                                                const int32_t* lold, float* scratch,
                                                const float* srow) {
  if (fa.dtype == kBF16) {
    if (fa.D == 128)
      fused_attention_t<uint16_t, 128>(fa, bh, ks, len, lpos, lcur, lold, scratch, srow);
    else
      fused_attention_t<uint16_t, 64>(fa, bh, ks, len, lpos, lcur, lold, scratch, srow);
  } else {
    if (fa.D == 128) fused_attention_t<float, 128>(fa, bh, ks, len, lpos, lcur, lold, scratch, srow);
    else fused_attention_t<float, 64>(fa, bh, ks, len, lpos, lcur, lold, scratch, srow);
  }
}

template <int G, bool CACHED, bool PF>
__global__ __launch_bounds__(kNT) void k_topk(
    const float* __restrict__ scores, const int32_t* __restrict__ lens, int H, int Q, int BH,
    int64_t n_max, int k, int32_t* __restrict__ out0, int32_t* __restrict__ out1,
    int64_t out_stride, const int32_t* __restrict__ pred, FusedAttn fa, int len_shift,
    const float* __restrict__ gmax, int64_t gstride) {
  extern __shared__ uint32_t smem[];
  const int tid = threadIdx.x;
  int bh, j;
  xcd_tile_map(blockIdx.x, Q, BH, bh, j);
  const int64_t rowid = (int64_t)bh * Q + j;
  const float* row = scores + rowid * n_max;
  // Bookkeeping and attention: the current-query rows, when attention is fused.
  const bool do_book = fa.q != nullptr && j == 0;
  const int32_t* pred_row = (do_book && pred != nullptr) ? pred + (int64_t)bh * k : nullptr;
  Sink sk{};
  sk.out = ((j == 0) ? out0 : out1) + (int64_t)bh * out_stride;
  sk.lpos = do_book ? reinterpret_cast<int32_t*>(smem + Lay<CACHED>::pred) + kMaxK : nullptr;
  sk.lcur = do_book ? reinterpret_cast<int32_t*>(smem + Lay<CACHED>::pred) + 2 * kMaxK : nullptr;
  // The row's group maxima, when the scoring kernel wrote them, or else a
  // row that fits one tile (over its whole storage), are loaded now, before
  // the row's length is known, so that the loads overlap those of the
  // length and the prediction.
  // The prediction's V rows, when this workgroup prefetches them itself (PF
  // kernels, the last fa.pf_slabs slabs): row r of the slot (entry r >>
  // chunk_shift, row r & mask of its chunk) is read from host memory, 16
  // bytes per thread per 16 rows, and stored before the attention, so that
  // the transfer overlaps the selection.  Loads complete in issue order, so
  // the entries are loaded first, before the score row, and the rows only
  // once the score row is in LDS (pf_issue below), when nothing the
  // selection waits for is issued after them; and every workgroup of a PF
  // kernel issues the same loads (one without rows to fetch reads its
  // slab's slot rows and drops them), so that no join in the kernel has to
  // wait for them.
  constexpr int kPfU = kPrefetchMaxRows * kPrefetchRowBytes / 16 / kNT;
  const bool pf_here = PF && do_book && pred_row != nullptr && bh >= BH - fa.pf_slabs;
  const int pf_rows = k << fa.chunk_shift;
  int pf_e[kPfU];
  if constexpr (PF) {
#pragma unroll
    for (int u = 0; u < kPfU; ++u) {
      const int r = min(tid / 16 + (kNT / 16) * u, pf_rows - 1);
      pf_e[u] = *(pf_here ? pred_row + (r >> fa.chunk_shift) : lens);
    }
  }
  const bool use_gm = gmax != nullptr;
  const bool vec = (reinterpret_cast<uintptr_t>(row) & 15u) == 0 && (n_max & 3) == 0;
  f32x4 v0[CACHED ? kU : 1];
  f32x4 gv[kGM4];
  if (use_gm) {
    load_maxima(gmax + rowid * gstride, gstride, gv);
  } else {
    if constexpr (CACHED) load_tile(row, (int)n_max, 0, vec, v0);
  }
  // The prediction row, loaded now and stored in LDS once it is needed.
  // The loops over a thread's entries stop at the first r with
  // kNT * r >= k (a uniform branch), so a small k runs one iteration of
  // code; entries past that stay -1.
  int32_t pv[kPR];
#pragma unroll
  for (int r = 0; r < kPR; ++r) pv[r] = -1;
#pragma unroll
  for (int r = 0; r < kPR; ++r) {
    if (kNT * r >= k) break;
    const int p = tid + kNT * r;
    if (pred_row != nullptr && p < k) pv[r] = pred_row[p];
  }
  clear(smem + kLHist, kBins);
  const int32_t len_b = lens[bh / H];
  const int n = (int)chunk_len(len_b, len_shift, n_max);
  int misses = 0, fetchable = 0;
  // The rows' loads, issued once the score row has left the registers (the
  // filter path calls this after storing the row in LDS; any other path
  // issues them before the attention).  Rows outside the cache, and rows
  // past the prediction, read the slot row itself (the load is
  // unconditional) and are replaced by zeros or not stored.
  u32x4 pfv[kPfU];
  bool pf_ok[kPfU];
  bool pf_issued = false;
  auto pf_issue = [&]() {
    if constexpr (PF) {
      const int cs = fa.chunk_shift;
      const uint8_t* vh = static_cast<const uint8_t*>(fa.v_host) +
                          (int64_t)bh * fa.n_rows * kPrefetchRowBytes + (tid % 16) * 16;
      const uint8_t* vs = static_cast<const uint8_t*>(fa.vslot) +
                          (int64_t)bh * 2 * pf_rows * kPrefetchRowBytes + (tid % 16) * 16;
#pragma unroll
      for (int u = 0; u < kPfU; ++u) {
        const int r = min(tid / 16 + (kNT / 16) * u, pf_rows - 1);
        const int64_t hr = ((int64_t)pf_e[u] << cs) + (r & ((1 << cs) - 1));
        pf_ok[u] = pf_here && pf_e[u] >= 0 && hr < fa.n_rows;
        const uint8_t* src = pf_ok[u] ? vh + hr * kPrefetchRowBytes : vs + r * kPrefetchRowBytes;
        pfv[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src));
      }
    }
    pf_issued = true;
  };
  if (n <= k) {
    // Every valid key is selected: entry c is c itself.
    ScanBufs sb{reinterpret_cast<int*>(smem + kLScr), 0};
    int32_t* s_pred = reinterpret_cast<int32_t*>(smem + Lay<CACHED>::pred);
    int pf = 0, pn = 0;
    const int32_t* s_ppos = nullptr;
    if (do_book) {
      store_prediction(pv, k, n_max, s_pred, pf, pn);
      __syncthreads();
      s_ppos = order_prediction(s_pred, k, sort_buffer<CACHED>(smem),
                                reinterpret_cast<int*>(smem + kLScr) + 4 * kNW);
    }
    int e0, e1, t0, t1;
    block_scan_pair<kNW>(pf, pn, sb, e0, e1, t0, t1);
    fetchable = t0;
    for (int r0 = 0; r0 < k; r0 += kNT) {
      const int c = r0 + tid;
      const bool valid = c < n;
      int hit = (do_book && valid) ? find_in(s_pred, t1, c) : -1;
      if (hit >= 0 && s_ppos != nullptr) hit = s_ppos[hit];
      int mtot;
      const int mr = misses + block_scan<kNW>((do_book && valid && hit < 0) ? 1 : 0, sb, mtot);
      if (c < k) {
        sk.out[c] = valid ? c : -1;
        if (do_book) {
          sk.lpos[c] = !valid ? -1 : (hit >= 0 ? hit : k + mr);
          sk.lcur[c] = valid ? c : -1;
        }
      }
      misses += mtot;
    }
  } else {
    bool done = false;
    if (use_gm && n <= kFilterMaxN && (n + kMaxGroup - 1) / kMaxGroup >= k)
      done = maxima_select<CACHED>(row, gv, gstride, n, n_max, k, smem, sk, do_book, pv, misses,
                                   fetchable);
    if (!done && n <= kFilterMaxN) {
      if constexpr (CACHED) {
        if (use_gm) load_tile(row, (int)n_max, 0, vec, v0);
      }
      done = filter_select<G, CACHED>(row, n, n_max, k, smem, sk, do_book, pv, v0, misses,
                                      fetchable, pf_issue);
    }
    if (!done) {
      sk.s_pred = nullptr;
      misses = radix_select<CACHED>(row, n, n_max, k, smem, sk, do_book, pv, fetchable);
    }
  }

  if (!do_book) return;
  if constexpr (PF) {  // the prefetched rows into their slot rows (see above)
    if (!pf_issued) pf_issue();
    uint8_t* vs = static_cast<uint8_t*>(const_cast<void*>(fa.vslot)) +
                  (int64_t)bh * 2 * pf_rows * kPrefetchRowBytes + (tid % 16) * 16;
    const u32x4 zero = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int u = 0; u < kPfU; ++u) {
      // An empty statement that takes the row as an operand: the first use
      // of the loaded data stays here, so the compiler cannot move the
      // zero select (and with it the wait for the host reads) up to the
      // loads.
      asm volatile("" : "+v"(pfv[u]));
      const int r = tid / 16 + (kNT / 16) * u;
      if (pf_here && r < pf_rows)
        *reinterpret_cast<u32x4*>(vs + r * kPrefetchRowBytes) = pf_ok[u] ? pfv[u] : zero;
    }
  }
  const int valid = n < k ? n : k;
  const bool resident = fa.where != nullptr;
  if (tid == 0 && fa.stats != nullptr) {
    atomicAdd(reinterpret_cast<unsigned long long*>(fa.stats), (unsigned long long)misses);
    atomicAdd(reinterpret_cast<unsigned long long*>(fa.stats) + 1,
              (unsigned long long)(valid - misses));
    if (!resident)
      atomicAdd(reinterpret_cast<unsigned long long*>(fa.stats) + 2,
                (unsigned long long)(fetchable + misses));
  }
  __syncthreads();  // every entry's slot row and row index are in LDS
  int32_t* lold = nullptr;
  if (resident) {
    lold = reinterpret_cast<int32_t*>(smem + kLOld<CACHED>);
    const int host = resident_bookkeeping(fa, bh, k, misses, pred_row != nullptr, sk.lpos,
                                          sk.lcur, lold,
                                          ScanBufs{reinterpret_cast<int*>(smem + kLScr), 0});
    if (tid == 0) {
      unsigned long long pf = 0;
      if (bh == 0) {  // the layer's prefetch count, taken once and cleared
        pf = *fa.pf_host;
        *fa.pf_host = 0ull;
      }
      if (fa.stats != nullptr)
        atomicAdd(reinterpret_cast<unsigned long long*>(fa.stats) + 2,
                  (unsigned long long)host + pf);
    }
    __syncthreads();  // lold complete
  }
  // Each selected key's logit is already in the score rows when every key
  // was scored (K rows from the scoring copy, one row per entry): the
  // attention then reads only V rows.  Chunk landmarks' scores are not the
  // keys' logits, and K rows from the host are attended from their bytes.
  const bool from_scores = fa.k_dev != nullptr && fa.chunk_shift == 0 && Q == 2;
  fused_attention(fa, bh, k, len_b, sk.lpos, sk.lcur, lold,
                  reinterpret_cast<float*>(smem + (CACHED ? Lay<true>::end : kLIdx)),
                  from_scores ? scores + (int64_t)bh * Q * n_max : nullptr);
}

using TopkKernel = decltype(&k_topk<1, true, false>);

template <bool CACHED>
TopkKernel pick_kernel(int g) {
  switch (g) {
    case 1: return k_topk<1, CACHED, false>;
    case 2: return k_topk<2, CACHED, false>;
    case 4: return k_topk<4, CACHED, false>;
    case 8: return k_topk<8, CACHED, false>;
    default: return k_topk<16, CACHED, false>;
  }
}

// The kernels with the selection-side prefetch: cached rows, k <= 128
// entries (so g is 1 or 2).
TopkKernel pick_pf_kernel(int g) { return g == 1 ? k_topk<1, true, true> : k_topk<2, true, true>; }

}  // namespace

bool topk_uses_maxima(int64_t n_max) { return n_max > kTile; }

hipError_t launch_topk(const float* scores, const int32_t* lens, int B, int H, int Q,
                       int64_t n_max, int k, int32_t* out0, int32_t* out1,
                       int64_t out_stride_bh, const int32_t* pred, const FusedAttn* attn,
                       hipStream_t s, int len_shift, const float* gmax) {
  const int BH = B * H;
  if (BH == 0) return hipSuccess;
  const DeviceInfo& di = device_info();
  const bool cached = n_max <= kTile;
  const int64_t words = cached ? Lay<true>::words : Lay<false>::words;
  if (words * 4 > di.lds_per_block) return hipErrorInvalidConfiguration;
  const size_t shmem = (size_t)words * 4;
  // Groups per thread: at least 4k group maxima (8192 at most).
  int g = 1;
  while (g < kU && kNT * g < 4 * k) g *= 2;
  // Dynamic LDS beyond the runtime's default needs the kernels' opt-in
  // attribute, set once per device (the first caller sets it while any
  // others wait) to what the device leaves beside each kernel's static LDS;
  // a failure is kept and returned by every later launch on that device.
  // Without it a launch was seen to run with a smaller LDS allocation and
  // no error.
  static std::once_flag attr_once[kAttrDevices];
  static hipError_t attr_err[kAttrDevices];
  static size_t attr_room[kAttrDevices][2];  // dynamic bytes allowed: [cached]
  if (di.device < 0 || di.device >= kAttrDevices) return hipErrorInvalidDevice;
  std::call_once(attr_once[di.device], [&di]() {
    hipError_t e = hipSuccess;
    size_t room[2] = {(size_t)di.lds_per_block, (size_t)di.lds_per_block};
    for (int gg = 1; gg <= kU && e == hipSuccess; gg *= 2) {
      for (int c = 0; c < 3 && e == hipSuccess; ++c) {
        if (c == 2 && gg > 2) break;
        const void* fn = c == 2 ? reinterpret_cast<const void*>(pick_pf_kernel(gg))
                         : c  ? reinterpret_cast<const void*>(pick_kernel<true>(gg))
                              : reinterpret_cast<const void*>(pick_kernel<false>(gg));
        hipFuncAttributes fa{};
        e = hipFuncGetAttributes(&fa, fn);
        if (e != hipSuccess) break;
        if (fa.sharedSizeBytes >= (size_t)di.lds_per_block) {
          e = hipErrorInvalidConfiguration;
          break;
        }
        const size_t r = (size_t)di.lds_per_block - fa.sharedSizeBytes;
        if (r < room[c ? 1 : 0]) room[c ? 1 : 0] = r;
        e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)r);
      }
    }
    attr_err[di.device] = e;
    attr_room[di.device][0] = room[0];
    attr_room[di.device][1] = room[1];
  });
  if (attr_err[di.device] != hipSuccess) return attr_err[di.device];
  if (shmem > attr_room[di.device][cached ? 1 : 0]) return hipErrorInvalidConfiguration;
  FusedAttn fa{};
  if (attn != nullptr) fa = *attn;
  // Group maxima rows must be 16-byte aligned for their vector loads.
  if (gmax != nullptr && (reinterpret_cast<uintptr_t>(gmax) & 15u) != 0) return hipErrorInvalidValue;
  const int64_t gstride = max_group_stride(n_max);
  // A selection-side prefetch: V rows of kPrefetchRowBytes from host memory,
  // at most kPrefetchMaxRows of them per slab, with a prediction to read.
  const bool pf = fa.pf_slabs != 0;
  if (pf && (fa.q == nullptr || fa.pf_slabs < 0 || fa.pf_slabs > BH || fa.v_host == nullptr ||
             fa.vslot == nullptr || fa.D * elem_bytes(fa.dtype) != kPrefetchRowBytes ||
             fa.chunk_shift < 0 || fa.chunk_shift > 7 ||
             ((int64_t)k << fa.chunk_shift) > kPrefetchMaxRows || fa.where != nullptr ||
             !cached || g > 2))
    return hipErrorInvalidValue;
  if (pf) {
    hipLaunchKernelGGL(pick_pf_kernel(g), dim3(BH * Q), dim3(kNT), shmem, s, scores, lens, H, Q,
                       BH, n_max, k, out0, out1, out_stride_bh, pred, fa, len_shift, gmax,
                       gstride);
  } else if (cached) {
    hipLaunchKernelGGL(pick_kernel<true>(g), dim3(BH * Q), dim3(kNT), shmem, s, scores, lens, H, Q,
                       BH, n_max, k, out0, out1, out_stride_bh, pred, fa, len_shift, gmax,
                       gstride);
  } else {
    hipLaunchKernelGGL(pick_kernel<false>(g), dim3(BH * Q), dim3(kNT), shmem, s, scores, lens, H,
                       Q, BH, n_max, k, out0, out1, out_stride_bh, pred, fa, len_shift, gmax,
                       gstride);
  }
  return hipGetLastError();
}

}  // namespace dd
