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
  int run_shift;         // each index names a run of 2^run_shift rows (a chunk)
  int row_bytes;         // bytes of one K/V row: 128, 256 or 512
};

constexpr int kGatherUnroll = 4;
constexpr int64_t kGatherMaxRows = 0x7fffffff - 1024;  // rows of one job (32-bit row numbers)

// Rows handled by wave `gw` of `nw` waves (256-thread workgroups assumed by
// callers only through gw/nw).  Entry j < cnt[bh] of slab bh copies the run
// of R = 2^run_shift host rows starting at row R * idx[bh*m + j] (a row out
// of [0, n_max), or of a negative index, becomes a zero row) to destination
// rows bh*dst_rows_per_bh + dst_row0 + R*j onwards; with R = 1 a run is one
// row.  The rows of a run are contiguous on both sides, so consecutive
// lanes read consecutive host bytes.  Loads are issued unconditionally so
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
  // Entry and row numbers fit in 32 bits (callers keep total << run_shift
  // below 2^31); byte offsets are 64-bit.
  const int rs = g.run_shift;
  const int rows = (int)(g.total << rs);
  for (int64_t base = gw * (RPI * U); base < rows; base += nw * (RPI * U)) {
    const uint8_t* kp[U];
    const uint8_t* vp[U];
    int64_t doff[U];
    bool wr[U], fetch[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      int row = (int)base + u * RPI + rsub;
      wr[u] = row < rows;
      if (!wr[u]) row = rows - 1;
      const int r = row >> rs;                          // entry
      const int i = row - (r << rs);                    // row within the run
      const int bh = r / g.m;
      const int j = r - bh * g.m;
      int lim = g.m;
      if (g.cnt != nullptr) {
        const int c = g.cnt[bh];
        lim = c < 0 ? 0 : (c > g.m ? g.m : c);
      }
      wr[u] = wr[u] && j < lim;
      doff[u] = ((int64_t)bh * g.dst_rows_per_bh + g.dst_row0 + (j << rs) + i) * ROWB + col * 16;
      const int32_t ir = g.idx[r];
      const int64_t hr = (wr[u] && ir >= 0) ? ((int64_t)ir << rs) + i : -1;
      fetch[u] = hr >= 0 && hr < g.n_max;
      const int64_t soff = ((int64_t)bh * g.n_max + (fetch[u] ? hr : 0)) * ROWB + col * 16;
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
