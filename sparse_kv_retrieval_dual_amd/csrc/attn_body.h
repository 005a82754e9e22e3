// One chunk of sparse decode attention for one (b, h), shared by the
// attention kernel and the layer step's fused top-k + attention kernel.
//
// A chunk of 128 entries is shared by NW waves, 128 / NW consecutive
// entries each: four waves in the attention kernel's 256-thread groups,
// eight in the top-k kernel's 512-thread workgroups (two waves per SIMD,
// so each wave's issue and latency overlap the other's).  A row is read by
// LPR lanes, 16 B each; every lane issues its K and V loads for all of its
// entries at once (one memory round trip), the dot products are summed
// across the LPR lanes by a DPP butterfly that leaves every lane with all
// of its entries' logits, and the wave forms its own max, weights and
// weighted V sum without a workgroup barrier.  The NW waves are merged in
// LDS by log-sum-exp in a fixed order.  Every reduction runs in
// the order of the entry number j, never of the row it is stored in, so the
// result does not depend on where rows sit.
#pragma once

#include "dd_device.h"

namespace dd {

constexpr int kAttnThreads = 256;
constexpr int kAttnWaves = kAttnThreads / 64;
constexpr int kAttnChunk = 128;  // entries per chunk
constexpr float kLog2e = 1.4426950408889634f;

// NW: waves sharing a chunk.
template <typename T, int D, int NW = kAttnWaves>
struct AttnShape {
  static constexpr int WE = kAttnChunk / NW;       // entries per wave
  static constexpr int EPL = 16 / (int)sizeof(T);  // elements per lane per load
  static constexpr int LPR = D / EPL;              // lanes per row
  static constexpr int RPI = 64 / LPR;             // rows per wave load instruction
  static constexpr int U = WE / RPI;               // entries (K and V loads) per lane
  static_assert(WE * NW == kAttnChunk && U >= 1 && U * RPI == WE, "shape");
};

// All-reduce of NV values over aligned groups of G lanes.
template <int G, int NV>
__device__ __forceinline__ void group_allreduce(float* x) {
  if constexpr (G > 1) {
    constexpr int HALF = G / 2;
#pragma unroll
    for (int v = 0; v < NV; ++v) x[v] += partner<HALF>(x[v]);
    group_allreduce<HALF, NV>(x);
  }
}

// The rows of one (b, h): slot rows kb / vb ([m][D]), and for entries whose
// slot row is >= first_miss_row the host rows khb / vhb ([n_max][D]) they
// are read from (and copied into their slot row); vhb null: no host rows.
// kdb (or null): the device copy of the keys ([n_max][D]); when set, every
// entry's K row is read from it by row index and only V rows come from the
// slot or the host (khb is then unused).  vob (or null, with kdb set): the
// previous step's slot ([m][D] V rows); a miss it holds is read from there
// instead of the host.
template <typename T>
struct AttnRows {
  const T* kb;
  const T* vb;
  const T* khb;
  const T* vhb;
  const T* kdb;
  int m;
  int first_miss_row;
  int64_t n_max;
  const T* vob = nullptr;
};

// LDS of one chunk merge, per query: per-wave max, weight sum and weighted V.
template <int D, int NQ = 1, int NW = kAttnWaves>
struct AttnLds {
  float m[NQ][NW];
  float l[NQ][NW];
  float o[NQ][NW][D];
};

// The rows of one chunk in registers: entry slot rows (-1: skipped), the
// host row of each miss (-1 otherwise) and every entry's K and V bytes.
template <typename T, int D, int NW = kAttnWaves>
struct AttnFetch {
  using S = AttnShape<T, D, NW>;
  int rows[S::U];
  int hrow[S::U];
  u32x4 kr[S::U], vr[S::U];
};

// First half of a chunk (entries c0 .. c0 + 127 below lim, handled by the
// NW waves of threads tid = 0 .. 64 NW - 1): resolves each entry's rows through
// entry(j, r, c, o) (slot row r, -1: skipped; host row c; row o of the
// previous step's slot holding a miss, else -1) and issues its K and V loads, all at once (slot rows and device keys from
// HBM, missed rows over the host link); a skipped entry reads row 0 of the
// slab (when there is one) and is masked later.  Nothing waits for the
// loads here, so a caller can fetch the next chunk before it finishes this
// one.
template <typename T, int D, int NW = kAttnWaves, class Entry>
__device__ __forceinline__ void attn_fetch(const AttnRows<T>& R, int c0, int lim, Entry entry,
                                           AttnFetch<T, D, NW>& f, int tid) {
  using S = AttnShape<T, D, NW>;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int col = lane % S::LPR;
  const int rsub = lane / S::LPR;
  const int e0 = c0 + wave * S::WE;  // this wave's first entry
  if (wave >= NW) {  // a larger workgroup's other waves: no entries, no loads
    // The stores in the order of the loads' path below (rows, hrow, then K
    // and V), so that the compiler can merge both paths' stores without
    // selecting between addresses (which would keep f in scratch memory).
#pragma unroll
    for (int u = 0; u < S::U; ++u) {
      f.rows[u] = -1;
      f.hrow[u] = -1;
    }
#pragma unroll
    for (int u = 0; u < S::U; ++u) {
      f.kr[u] = u32x4{0u, 0u, 0u, 0u};
      f.vr[u] = u32x4{0u, 0u, 0u, 0u};
    }
    return;
  }
  const bool from_host = R.vhb != nullptr;
  const bool kdev = R.kdb != nullptr;
  int krow[S::U];  // row of the device key copy (kdev), else -1
  int orow[S::U];  // row of the previous step's slot holding a miss, else -1
#pragma unroll
  for (int u = 0; u < S::U; ++u) {
    const int j = e0 + u * S::RPI + rsub;
    int r = -1, c = -1, o = -1;
    if (j < lim && R.m > 0) {
      entry(j, r, c, o);
      if (r < 0 || r >= R.m) r = -1;
    }
    const bool cvalid = c >= 0 && (int64_t)c < R.n_max;
    const bool miss = r >= R.first_miss_row && from_host;
    if ((miss || kdev) && !cvalid) r = -1;
    f.rows[u] = r;
    f.hrow[u] = (r >= 0 && miss) ? c : -1;
    krow[u] = (r >= 0 && kdev) ? c : -1;
    orow[u] = (r >= 0 && miss && R.vob != nullptr && o >= 0 && o < R.m) ? o : -1;
  }
  const T* kb = R.kb + col * S::EPL;
  const T* vb = R.vb + col * S::EPL;
  const T* khb = (from_host && !kdev) ? R.khb + col * S::EPL : kb;
  const T* vhb = from_host ? R.vhb + col * S::EPL : vb;
  const T* kdb = kdev ? R.kdb + col * S::EPL : kb;
  // Streaming (non-temporal) loads: every row is read once.  One store per
  // element (values selected, not addresses), so the fetch stays in
  // registers.
  const bool any = R.m > 0;
#pragma unroll
  for (int u = 0; u < S::U; ++u) {
    u32x4 kv = u32x4{0u, 0u, 0u, 0u};
    u32x4 vv = kv;
    if (any) {
      const bool h = f.hrow[u] >= 0;
      const int64_t off = (int64_t)(h ? f.hrow[u] : (f.rows[u] >= 0 ? f.rows[u] : 0)) * D;
      const int64_t koff = (int64_t)(krow[u] >= 0 ? krow[u] : 0) * D;
      kv = __builtin_nontemporal_load(
          reinterpret_cast<const u32x4*>(kdev ? kdb + koff : (h ? khb : kb) + off));
      const T* vsrc = (h ? vhb : vb) + off;
      if (orow[u] >= 0) vsrc = R.vob + col * S::EPL + (int64_t)orow[u] * D;
      vv = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(vsrc));
    }
    f.kr[u] = kv;
    f.vr[u] = vv;
  }
}

// attn_fetch for the common case of the layer step: every K row from the
// device key copy by row index (kdb set), no previous slot (vob null).  The
// same rows and addresses as attn_fetch with fewer selects on the way.
template <typename T, int D, int NW = kAttnWaves, class Entry>
__device__ __forceinline__ void attn_fetch_kdev(const AttnRows<T>& R, int c0, int lim, Entry entry,
                                                AttnFetch<T, D, NW>& f, int tid) {
  using S = AttnShape<T, D, NW>;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int col = lane % S::LPR;
  const int rsub = lane / S::LPR;
  const int e0 = c0 + wave * S::WE;
  if (wave >= NW) {  // a larger workgroup's other waves: no entries, no loads
    // The stores in the order of the loads' path below (rows, hrow, then K
    // and V), so that the compiler can merge both paths' stores without
    // selecting between addresses (which would keep f in scratch memory).
#pragma unroll
    for (int u = 0; u < S::U; ++u) {
      f.rows[u] = -1;
      f.hrow[u] = -1;
    }
#pragma unroll
    for (int u = 0; u < S::U; ++u) {
      f.kr[u] = u32x4{0u, 0u, 0u, 0u};
      f.vr[u] = u32x4{0u, 0u, 0u, 0u};
    }
    return;
  }
  const bool from_host = R.vhb != nullptr;
  int krow[S::U];
  // Every entry is looked up first (an entry past lim looks up entry
  // lim - 1 and is dropped), so that the lookups are in flight together.
  int er[S::U], ec[S::U];
#pragma unroll
  for (int u = 0; u < S::U; ++u) er[u] = ec[u] = -1;
  if (lim > 0 && R.m > 0) {
#pragma unroll
    for (int u = 0; u < S::U; ++u) {
      const int j = e0 + u * S::RPI + rsub;
      int o;
      entry(j < lim ? j : lim - 1, er[u], ec[u], o);
    }
  }
#pragma unroll
  for (int u = 0; u < S::U; ++u) {
    const int j = e0 + u * S::RPI + rsub;
    int r = j < lim ? er[u] : -1;
    const int c = ec[u];
    if (r < 0 || r >= R.m) r = -1;
    if (c < 0 || (int64_t)c >= R.n_max) r = -1;
    const bool miss = from_host && r >= R.first_miss_row;
    f.rows[u] = r;
    f.hrow[u] = (r >= 0 && miss) ? c : -1;
    krow[u] = r >= 0 ? c : 0;
  }
  const T* vb = R.vb + col * S::EPL;
  const T* vhb = from_host ? R.vhb + col * S::EPL : vb;
  const T* kdb = R.kdb + col * S::EPL;
  const bool any = R.m > 0;
#pragma unroll
  for (int u = 0; u < S::U; ++u) {
    u32x4 kv = u32x4{0u, 0u, 0u, 0u};
    u32x4 vv = kv;
    if (any) {
      kv = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kdb + (int64_t)krow[u] * D));
      const bool h = f.hrow[u] >= 0;
      const T* vsrc = h ? vhb + (int64_t)f.hrow[u] * D
                        : vb + (int64_t)(f.rows[u] >= 0 ? f.rows[u] : 0) * D;
      vv = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(vsrc));
    }
    f.kr[u] = kv;
    f.vr[u] = vv;
  }
}

// The softmax and weighted V sum of one chunk from its logits, for the
// first nq <= NQ queries: s[qi * U + u] is query qi's scaled logit of the
// lane's entry u (entries with rows[u] < 0 are skipped), vr[u] its V row
// bytes.  Each wave forms its own max, weights and weighted V sum over its
// 128 / NW entries; the NW waves are then merged in LDS in wave order (one
// workgroup barrier; every thread of the workgroup must call it: in a
// workgroup of more than NW waves the others have no entries).
// Afterwards cm[j] and cl[j] (all threads) are query j's max logit and
// weight sum over the chunk, and threads d < D hold od[j] = its weighted V
// sum of column d.  The caller must not touch lds until a barrier after
// this returns.
template <typename T, int D, int NQ, int NW = kAttnWaves>
__device__ __forceinline__ void attn_softmax_merge(float* s, const int* rows, const u32x4* vr,
                                                   AttnLds<D, NQ, NW>& lds, int nq,
                                                   float (&cm)[NQ], float (&cl)[NQ],
                                                   float (&od)[NQ], int tid) {
#pragma clang fp contract(off)
  using S = AttnShape<T, D, NW>;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int col = lane % S::LPR;
  const int rsub = lane / S::LPR;
  const u32x4 zero = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
  for (int qi = 0; qi < NQ; ++qi) {
    if (qi >= nq) break;
    // Wave-local softmax of query qi over its WE entries (RPI row groups x U).
    float mx = -INFINITY;
#pragma unroll
    for (int u = 0; u < S::U; ++u) {
      float& x = s[qi * S::U + u];
      x = (rows[u] >= 0) ? x : -INFINITY;
      mx = fmaxf(mx, x);
    }
#pragma unroll
    for (int off = S::LPR; off < 64; off <<= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
    float l = 0.f;
    float o[S::EPL];
#pragma unroll
    for (int e = 0; e < S::EPL; ++e) o[e] = 0.f;
#pragma unroll
    for (int u = 0; u < S::U; ++u) {
      const float w = (rows[u] >= 0) ? exp2f((s[qi * S::U + u] - mx) * kLog2e) : 0.f;
      l += w;
      float fv[S::EPL];
      u32x4 vv = vr[u];  // a value select: selecting lvalues would put both in memory
      if (rows[u] < 0) vv = zero;
      Unpack<T>::run(vv, fv);
#pragma unroll
      for (int e = 0; e < S::EPL; ++e) o[e] = fmaf(w, fv[e], o[e]);
    }
#pragma unroll
    for (int off = S::LPR; off < 64; off <<= 1) {
      l += __shfl_xor(l, off);
#pragma unroll
      for (int e = 0; e < S::EPL; ++e) o[e] += __shfl_xor(o[e], off);
    }
    if (rsub == 0 && wave < NW) {  // (a larger workgroup's other waves hold nothing)
#pragma unroll
      for (int e = 0; e < S::EPL; ++e) lds.o[qi][wave][col * S::EPL + e] = o[e];
      if (col == 0) {
        lds.m[qi][wave] = mx;
        lds.l[qi][wave] = l;
      }
    }
  }
  __syncthreads();

  // Merge the waves (entry order is fixed: wave 0, 1, ..., NW - 1).
  const int d = tid;
#pragma unroll
  for (int qi = 0; qi < NQ; ++qi) {
    cm[qi] = -INFINITY;
    cl[qi] = 0.f;
    od[qi] = 0.f;
    if (qi >= nq) continue;
    float m = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) m = fmaxf(m, lds.m[qi][w]);
    float fw[NW];
    float tl = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      fw[w] = (lds.l[qi][w] > 0.f) ? exp2f((lds.m[qi][w] - m) * kLog2e) : 0.f;
      tl = fmaf(lds.l[qi][w], fw[w], tl);
    }
    float acc = 0.f;
    if (d < D) {
#pragma unroll
      for (int w = 0; w < NW; ++w) acc = fmaf(lds.o[qi][w][d], fw[w], acc);
    }
    cm[qi] = m;
    cl[qi] = tl;
    od[qi] = acc;
  }
}

// Second half of a chunk fetched by attn_fetch (tid: the thread's index in
// the 64 NW that handle the chunk; every thread of the workgroup must call
// it, since it holds a workgroup barrier), for the first nq <= NQ
// queries at once: query j is q + j * D (D floats; all NQ are read).  Every
// K and V row is read once and serves every query; a missed row is first
// copied into its slot row.  Contraction is off: only the explicit fmaf
// calls fuse, so a query's result is the same bits whatever nq is.
// Outputs as attn_softmax_merge.
template <typename T, int D, int NQ, int NW = kAttnWaves>
__device__ __forceinline__ void attn_finish(const float* __restrict__ q, const AttnRows<T>& R,
                                            float scale, const AttnFetch<T, D, NW>& f,
                                            AttnLds<D, NQ, NW>& lds, int nq, float (&cm)[NQ],
                                            float (&cl)[NQ], float (&od)[NQ], int tid) {
#pragma clang fp contract(off)
  using S = AttnShape<T, D, NW>;
  const int lane = tid & 63;
  const int col = lane % S::LPR;
  const bool from_host = R.vhb != nullptr;
  const bool kdev = R.kdb != nullptr;
  if (from_host && R.m > 0) {  // the slot keeps a copy of every fetched miss
#pragma unroll
    for (int u = 0; u < S::U; ++u) {
      if (f.hrow[u] >= 0) {
        T* vd = const_cast<T*>(R.vb) + col * S::EPL + (int64_t)f.rows[u] * D;
        *reinterpret_cast<u32x4*>(vd) = f.vr[u];
        if (!kdev) {
          T* kd = const_cast<T*>(R.kb) + col * S::EPL + (int64_t)f.rows[u] * D;
          *reinterpret_cast<u32x4*>(kd) = f.kr[u];
        }
      }
    }
  }
  float qr[NQ][S::EPL];
#pragma unroll
  for (int qi = 0; qi < NQ; ++qi)
#pragma unroll
    for (int e = 0; e < S::EPL; ++e) qr[qi][e] = qi < nq ? q[qi * D + col * S::EPL + e] : 0.f;

  // Logits: the first query always, the others only when they attend.
  float s[NQ * S::U];  // s[qi * U + u]
#pragma unroll
  for (int qi = 0; qi < NQ; ++qi) {
    if (qi >= nq) break;
#pragma unroll
    for (int u = 0; u < S::U; ++u) {
      float fk[S::EPL];
      Unpack<T>::run(f.kr[u], fk);
      float a = 0.f;
#pragma unroll
      for (int e = 0; e < S::EPL; ++e) a = fmaf(fk[e], qr[qi][e], a);
      s[qi * S::U + u] = a;
    }
    group_allreduce<S::LPR, S::U>(s + qi * S::U);
#pragma unroll
    for (int u = 0; u < S::U; ++u) s[qi * S::U + u] *= scale;
  }
  attn_softmax_merge<T, D, NQ, NW>(s, f.rows, f.vr, lds, nq, cm, cl, od, tid);
}

// A chunk whose logits are already known (the layer step's own scores of
// the selected keys): the V rows of its entries and their scores, fetched
// in one round trip.
template <typename T, int D, int NQ, int NW = kAttnWaves>
struct AttnFetchS {
  using S = AttnShape<T, D, NW>;
  int rows[S::U];
  int hrow[S::U];
  u32x4 vr[S::U];
  float s[NQ * S::U];
};

// Entries c0 .. c0 + 127 below lim of one (b, h) whose K rows are not
// needed: entry(j, r, c, o) gives the slot row r, the key c and the row o
// of the previous step's slot holding a miss (else -1), as for attn_fetch.
// Every lane loads the V row of each of its entries (slot, host for a miss,
// or the previous slot) and the entry's scaled logit of each of the first
// nq queries, srow[qi * sstride + c].  A skipped entry reads row 0 and
// score 0 and is masked later.
template <typename T, int D, int NQ, int NW = kAttnWaves, class Entry>
__device__ __forceinline__ void attn_fetch_s(const AttnRows<T>& R, const float* __restrict__ srow,
                                             int64_t sstride, int nq, int c0, int lim,
                                             Entry entry, AttnFetchS<T, D, NQ, NW>& f, int tid) {
  using S = AttnShape<T, D, NW>;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int col = lane % S::LPR;
  const int rsub = lane / S::LPR;
  const int e0 = c0 + wave * S::WE;
  if (wave >= NW) {  // a larger workgroup's other waves: no entries, no loads
#pragma unroll
    for (int u = 0; u < S::U; ++u) {
      f.rows[u] = -1;
      f.hrow[u] = -1;
      f.vr[u] = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
      for (int qi = 0; qi < NQ; ++qi) f.s[qi * S::U + u] = 0.f;
    }
    return;
  }
  const bool from_host = R.vhb != nullptr;
  // Every entry is looked up first (an entry past lim looks up entry
  // lim - 1 and is dropped), so that the lookups are in flight together.
  int er[S::U], ec[S::U], eo[S::U];
#pragma unroll
  for (int u = 0; u < S::U; ++u) er[u] = ec[u] = eo[u] = -1;
  if (lim > 0 && R.m > 0) {
#pragma unroll
    for (int u = 0; u < S::U; ++u) {
      const int j = e0 + u * S::RPI + rsub;
      entry(j < lim ? j : lim - 1, er[u], ec[u], eo[u]);
    }
  }
  int cc[S::U], orow[S::U];
#pragma unroll
  for (int u = 0; u < S::U; ++u) {
    const int j = e0 + u * S::RPI + rsub;
    int r = j < lim ? er[u] : -1;
    const int c = ec[u];
    if (r < 0 || r >= R.m) r = -1;
    if (c < 0 || (int64_t)c >= R.n_max) r = -1;
    const bool miss = from_host && r >= R.first_miss_row;
    f.rows[u] = r;
    f.hrow[u] = (r >= 0 && miss) ? c : -1;
    cc[u] = r >= 0 ? c : 0;
    orow[u] = (r >= 0 && miss && R.vob != nullptr && eo[u] >= 0 && eo[u] < R.m) ? eo[u] : -1;
  }
  const T* vb = R.vb + col * S::EPL;
  const T* vhb = from_host ? R.vhb + col * S::EPL : vb;
  const bool any = R.m > 0;
#pragma unroll
  for (int u = 0; u < S::U; ++u) {
    u32x4 vv = u32x4{0u, 0u, 0u, 0u};
    if (any) {
      const bool h = f.hrow[u] >= 0;
      const T* vsrc = h ? vhb + (int64_t)f.hrow[u] * D
                        : vb + (int64_t)(f.rows[u] >= 0 ? f.rows[u] : 0) * D;
      if (orow[u] >= 0) vsrc = R.vob + col * S::EPL + (int64_t)orow[u] * D;
      vv = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(vsrc));
    }
    f.vr[u] = vv;
#pragma unroll
    for (int qi = 0; qi < NQ; ++qi)
      f.s[qi * S::U + u] = qi < nq ? srow[qi * sstride + cc[u]] : 0.f;
  }
}

// Second half of a chunk fetched by attn_fetch_s: a missed row is first
// copied into its slot row, then attn_softmax_merge over the fetched
// logits.  Every thread of the workgroup must call it.
template <typename T, int D, int NQ, int NW = kAttnWaves>
__device__ __forceinline__ void attn_finish_s(const AttnRows<T>& R, AttnFetchS<T, D, NQ, NW>& f,
                                              AttnLds<D, NQ, NW>& lds, int nq, float (&cm)[NQ],
                                              float (&cl)[NQ], float (&od)[NQ], int tid) {
  using S = AttnShape<T, D, NW>;
  const int col = (tid & 63) % S::LPR;
  if (R.vhb != nullptr && R.m > 0) {  // the slot keeps a copy of every fetched miss
#pragma unroll
    for (int u = 0; u < S::U; ++u) {
      if (f.hrow[u] >= 0) {
        T* vd = const_cast<T*>(R.vb) + col * S::EPL + (int64_t)f.rows[u] * D;
        *reinterpret_cast<u32x4*>(vd) = f.vr[u];
      }
    }
  }
  attn_softmax_merge<T, D, NQ, NW>(f.s, f.rows, f.vr, lds, nq, cm, cl, od, tid);
}

// Entries c0 .. c0 + 127 (those < lim): attn_fetch (attn_fetch_kdev when
// KDEV: K rows from the device copy, no previous slot), then attn_finish.
template <typename T, int D, int NQ, bool KDEV = false, int NW = kAttnWaves, class Entry>
__device__ __forceinline__ void attend_chunk_n(const float* __restrict__ q, const AttnRows<T>& R,
                                               int c0, int lim, float scale, Entry entry,
                                               AttnLds<D, NQ, NW>& lds, int nq, float (&cm)[NQ],
                                               float (&cl)[NQ], float (&od)[NQ]) {
  AttnFetch<T, D, NW> f;
  if constexpr (KDEV)
    attn_fetch_kdev<T, D, NW>(R, c0, lim, entry, f, threadIdx.x);
  else
    attn_fetch<T, D, NW>(R, c0, lim, entry, f, threadIdx.x);
  attn_finish<T, D, NQ, NW>(q, R, scale, f, lds, nq, cm, cl, od, threadIdx.x);
}

// Merge of the chunk partials of one (b, h) by log-sum-exp, for column d:
// partial c holds the weighted V sums [0, D), its max logit at D and its
// weight sum at D + 1.
template <int D>
__device__ __forceinline__ void combine_chunks(const float* p, int chunks, int d, float& out_d,
                                               float& lse) {
#pragma clang fp contract(off)
  float mx = -INFINITY;
#pragma unroll 8
  for (int c = 0; c < chunks; ++c) mx = fmaxf(mx, p[c * (D + 2) + D]);
  float tot = 0.f, od = 0.f;
  if (mx > -INFINITY) {
#pragma unroll 8
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
  out_d = (tot > 0.f) ? od / tot : 0.f;
  lse = (tot > 0.f) ? mx + logf(tot) : -INFINITY;
}

}  // namespace dd
