// Rows kept across decode steps: the prefetch of a layer that owns two V
// slots, and the lookup the fused top-k's miss path shares with it.
//
// Each layer owns two slots, the one the previous step filled ("old") and
// the one this step fills ("new"), each with the key index held by every
// row (-1: none).  where[bh][x] is the row that key x was last written to;
// it is trusted only when the old slot's index list confirms it
// (old_idx[row] == x), so it never needs clearing.
#pragma once

#include "gather_body.h"

namespace dd {

struct GatherRes {
  int32_t* where;                  // [BH][n_max]
  const int32_t* old_idx;          // [BH][dst_rows_per_bh]
  int32_t* new_idx;                // [BH][dst_rows_per_bh]
  const uint8_t* old_v;            // [BH][dst_rows_per_bh][row]: the old slot's V plane
  unsigned long long* host_rows;   // rows read over the host link are added here
};

// Row of the old slot that holds key x of slab bh, or -1.
__device__ __forceinline__ int resident_row(const int32_t* where, const int32_t* old_idx,
                                            int64_t n_max, int64_t rows, int bh, int64_t x) {
  const int w = where[(int64_t)bh * n_max + x];
  if (w < 0 || w >= rows) return -1;
  return old_idx[(int64_t)bh * rows + w] == (int32_t)x ? w : -1;
}

// A wave's queue of row copies waiting for a full batch: byte offsets of
// the source (from the queue's base pointer; -1: a zero row) and of the
// destination.  A batch is RPI * kGatherUnroll rows; the queue holds fewer
// than that between classifications, plus the 64 a classification adds.
constexpr int kResQueue = 64 + 64;
struct ResQueue {
  int64_t src[kResQueue];
  int64_t dst[kResQueue];
};

// Copies queue entries [lo, hi) (hi - lo <= one batch): all loads of the
// batch are issued before any store.  A lane with no entry, or with a zero
// row, loads its own destination instead (in device memory) and stores
// nothing, or zeros.
template <int ROWB>
__device__ __forceinline__ void res_batch(const ResQueue& q, int lo, int hi, const uint8_t* base,
                                          uint8_t* vdst) {
  constexpr int LPR = ROWB / 16;
  constexpr int RPI = 64 / LPR;
  constexpr int U = kGatherUnroll;
  const int lane = threadIdx.x & 63;
  const int col = lane % LPR;
  const int rsub = lane / LPR;
  const u32x4 zero = u32x4{0u, 0u, 0u, 0u};
  u32x4 v[U];
  int64_t d[U];
  bool wr[U], fill[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int e = lo + u * RPI + rsub;
    wr[u] = e < hi;
    const int64_t s = wr[u] ? q.src[e] : -1;
    d[u] = (wr[u] ? q.dst[e] : 0) + col * 16;
    fill[u] = s >= 0;
    const uint8_t* p = fill[u] ? base + s + col * 16 : vdst + d[u];
    v[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  }
#pragma unroll
  for (int u = 0; u < U; ++u)
    if (wr[u]) *reinterpret_cast<u32x4*>(vdst + d[u]) = fill[u] ? v[u] : zero;
}

// The prefetch of one layer (V plane, one row per entry, dst_row0 = 0):
// entry j of slab bh (key idx[bh*m + j]) becomes V row j of the new slot,
// copied from the old slot when it holds the key, else read over the host
// link; an out-of-range or negative key gives a zero row.  Every entry's key
// goes to new_idx and where, and the rows read over the link are counted.
//
// A wave classifies 64 entries at a time (one per lane) and appends each
// row to one of two queues in LDS, rows from the host and rows from device
// memory (zero rows go with the latter); a queue is copied a full batch at a
// time.  Every batch of host reads is therefore all host reads, so the
// link sees full batches in flight, and a batch of device copies never
// waits for the host's latency.  The order of the copies is free: every
// row has its own destination.
template <int ROWB>
__device__ __forceinline__ void gather_rows_res(const GatherJob& g, int64_t gw, int64_t nw,
                                                const GatherRes& res, ResQueue& qh,
                                                ResQueue& qd) {
  constexpr int BATCH = (64 / (ROWB / 16)) * kGatherUnroll;
  static_assert(BATCH - 1 + 64 <= kResQueue, "queue too small");
  const int lane = threadIdx.x & 63;
  const int64_t rows = g.dst_rows_per_bh;
  const int64_t total = g.total;
  int nh = 0, nd = 0;    // queue lengths (wave-uniform)
  int host_cnt = 0;      // this lane's entries read over the link
  for (int64_t blk = gw * 64; blk < total; blk += nw * 64) {
    const int64_t r = blk + lane;
    const bool valid = r < total;
    const int bh = valid ? (int)(r / g.m) : 0;
    const int j = valid ? (int)(r - (int64_t)bh * g.m) : 0;
    const int32_t ir = valid ? g.idx[r] : -1;
    const bool fetch = ir >= 0 && (int64_t)ir < g.n_max;
    const int orow = fetch ? resident_row(res.where, res.old_idx, g.n_max, rows, bh, ir) : -1;
    const int64_t drow = (int64_t)bh * rows + j;
    if (valid) {
      res.new_idx[drow] = fetch ? ir : -1;
      if (fetch) res.where[(int64_t)bh * g.n_max + ir] = j;
    }
    const bool host = fetch && orow < 0;
    const bool dev = valid && !host;
    host_cnt += host ? 1 : 0;
    const uint64_t mh = __ballot(host);
    const uint64_t md = __ballot(dev);
    if (host) {
      const int e = nh + lanes_below(mh);
      qh.src[e] = ((int64_t)bh * g.n_max + ir) * ROWB;
      qh.dst[e] = drow * ROWB;
    }
    if (dev) {
      const int e = nd + lanes_below(md);
      qd.src[e] = orow >= 0 ? ((int64_t)bh * rows + orow) * ROWB : -1;
      qd.dst[e] = drow * ROWB;
    }
    nh += __popcll(mh);
    nd += __popcll(md);
    // LDS operations of one wave complete in order; the fence keeps the
    // compiler from moving the reads below above the writes above.
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    while (nh >= BATCH) {
      res_batch<ROWB>(qh, nh - BATCH, nh, g.vsrc, g.vdst);
      nh -= BATCH;
    }
    while (nd >= BATCH) {
      res_batch<ROWB>(qd, nd - BATCH, nd, res.old_v, g.vdst);
      nd -= BATCH;
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  }
  if (nh > 0) res_batch<ROWB>(qh, 0, nh, g.vsrc, g.vdst);
  if (nd > 0) res_batch<ROWB>(qd, 0, nd, res.old_v, g.vdst);
  host_cnt = wave_sum_int(host_cnt);
  if (lane == 0 && host_cnt > 0) atomicAdd(res.host_rows, (unsigned long long)host_cnt);
}

}  // namespace dd
