// The row-gather loop shared by the standalone gather kernel and the
// prefetch workgroups that ride along in the scoring kernel.
#pragma once

#include "dd_device.h"

namespace dd {

struct GatherJob {
  const uint8_t* ksrc;   // pinned host [BH][n_max][row]; either plane may be null
  const uint8_t* vsrc;
  int64_t n_max;
  const int32_t* idx;    // [BH][m]
  int m;
  const int32_t* cnt;    // [BH] or null (all m)
  int64_t total;         // BH * m
  uint8_t* kdst;         // [BH][dst_rows_per_bh][row]
  uint8_t* vdst;
  int64_t dst_rows_per_bh;
  int dst_row0;
};

constexpr int kGatherUnroll = 4;

// Rows handled by wave `gw` of `nw` waves (256-thread workgroups assumed by
// callers only through gw/nw).  Entry j < cnt[bh] of slab bh copies host row
// idx[bh*m + j] (zero row when out of [0, n_max)) to destination row
// bh*dst_rows_per_bh + dst_row0 + j.  Loads are issued unconditionally so
// that all of them are in flight at once; a lane without a host row to
// fetch reads a stand-in address in device memory (its own destination
// slot) and its data is discarded.
template <int ROWB>
__device__ __forceinline__ void gather_rows(const GatherJob& g, int64_t gw, int64_t nw) {
  constexpr int LPR = ROWB / 16;
  constexpr int RPI = 64 / LPR;
  constexpr int U = kGatherUnroll;
  const int lane = threadIdx.x & 63;
  const int col = lane % LPR;
  const int rsub = lane / LPR;
  const u32x4 zero = u32x4{0u, 0u, 0u, 0u};
  const bool has_k = g.ksrc != nullptr;
  const bool has_v = g.vsrc != nullptr;
  for (int64_t base = gw * (RPI * U); base < g.total; base += nw * (RPI * U)) {
    const uint8_t* kp[U];
    const uint8_t* vp[U];
    int64_t doff[U];
    bool wr[U], fetch[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      int64_t r = base + u * RPI + rsub;
      wr[u] = r < g.total;
      if (!wr[u]) r = g.total - 1;
      const int64_t bh = r / g.m;
      const int j = (int)(r - bh * g.m);
      int lim = g.m;
      if (g.cnt != nullptr) {
        const int c = g.cnt[bh];
        lim = c < 0 ? 0 : (c > g.m ? g.m : c);
      }
      wr[u] = wr[u] && j < lim;
      doff[u] = (bh * g.dst_rows_per_bh + g.dst_row0 + j) * ROWB + col * 16;
      const int32_t ir = g.idx[r];
      const int32_t i = wr[u] ? ir : -1;
      fetch[u] = i >= 0 && (int64_t)i < g.n_max;
      const int64_t soff = (bh * g.n_max + (fetch[u] ? i : 0)) * ROWB + col * 16;
      kp[u] = (fetch[u] && has_k) ? g.ksrc + soff : g.kdst + (has_k ? doff[u] : 0);
      vp[u] = (fetch[u] && has_v) ? g.vsrc + soff : g.vdst + (has_v ? doff[u] : 0);
    }
    u32x4 kv[U], vv[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (has_k) kv[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kp[u]));
      if (has_v) vv[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(vp[u]));
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (wr[u]) {
        if (has_k) *reinterpret_cast<u32x4*>(g.kdst + doff[u]) = fetch[u] ? kv[u] : zero;
        if (has_v) *reinterpret_cast<u32x4*>(g.vdst + doff[u]) = fetch[u] ? vv[u] : zero;
      }
    }
  }
}

}  // namespace dd
