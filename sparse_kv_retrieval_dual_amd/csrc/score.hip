// Dual-query scoring: s = scale * q . K for the current and the speculated
// query against every cached key (paper-daily summary of DualDecoder,
// core-formulas section; its worked example scores the whole key matrix).
//
// HBM-bound: each key row (D elements, 256 B for bf16 D=128) is streamed
// once and serves both queries; 2 flop/B is far below the VALU ridge, so the
// contraction stays on the VALU (MFMA would idle 15/16 of its tile on a
// 2-column operand).  A row is read by LPR lanes, 16 B each, so one wave
// load instruction covers 64*16 contiguous bytes.  Each lane keeps U = LPR/Q
// rows in flight and the Q*U partial dot products are folded across the LPR
// lanes with a transposing butterfly that leaves exactly one finished score
// per lane.
//
// Optionally each wave also writes the maximum score of every group of 16
// consecutive keys, per query (the selection takes its bound from these
// instead of reading the whole score row).
//
// Optionally the first few workgroups of the grid do not score: they gather
// the layer's predicted K/V rows from host memory into its slot (the
// prefetch), so that the host-link transfer overlaps the HBM-bound scan
// inside one kernel, with no second stream and no cross-stream wait.
#include <hip/hip_ext.h>

#include "dd_device.h"
#include "dd_internal.h"
#include "gather_body.h"
#include "gather_res.h"

namespace dd {

namespace {

// A workgroup scores 4 waves x ITERS iterations x (64 / Q) keys: 256 keys
// of 256 B for the two-query bf16 case (64 KB per workgroup).  Smaller tiles
// than that lost to launch overhead and larger ones to the last partial
// round of workgroups (measured on MI355X for 32 x 32768 keys).  Rows of
// 4-byte elements take one iteration, so that a workgroup still reads 64 KB
// at D = 128 (two iterations, 128 KB, scanned the 64 MiB of fp32 chunk
// landmarks 6% slower from HBM: 14.8 against 13.9 us).
constexpr int kScoreWaves = 4;
constexpr int kScoreIters = 2;  // iterations for 2-byte elements

template <typename T, int D, int Q>
struct ScoreShape {
  static constexpr int EPL = 16 / (int)sizeof(T);  // elements per lane per load
  static constexpr int LPR = D / EPL;              // lanes per key row
  static constexpr int RPI = 64 / LPR;             // rows per wave load instruction
  static constexpr int U = LPR / Q;                // loads per lane per iteration
  static constexpr int KPI = U * RPI;              // keys per wave iteration (= 64 / Q)
  static constexpr int ITERS = sizeof(T) == 4 ? 1 : kScoreIters;
  static constexpr int TILE = kScoreWaves * ITERS * KPI;
  static_assert(U >= 1 && U * Q == LPR, "shape");
  // Group maxima: a group of kMaxGroup keys is VPG consecutive vu values of
  // every rsub; GPI groups per wave iteration.
  static constexpr int VPG = kMaxGroup / RPI;
  static constexpr int GPI = KPI / kMaxGroup;
  static_assert(VPG >= 1 && VPG * RPI == kMaxGroup && GPI * kMaxGroup == KPI, "group shape");
};

template <typename T, int D, int Q>
__global__ __launch_bounds__(kScoreWaves * 64) void k_score(
    const float* __restrict__ q, const T* __restrict__ keys, const int32_t* __restrict__ lens,
    int BH, int H, int64_t n_max, int tiles, float scale, float* __restrict__ scores,
    int fill_pad, GatherJob pf, int pf_wgs, int64_t* __restrict__ zero3, int len_shift,
    GatherRes pres, float* __restrict__ gmax, int64_t gstride) {
  using S = ScoreShape<T, D, Q>;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  if (zero3 != nullptr && (int)blockIdx.x == pf_wgs && threadIdx.x < 3) zero3[threadIdx.x] = 0;
  if (tiles == 0) return;
  if ((int)blockIdx.x < pf_wgs) {
    // The gathered rows are K/V rows: the scored rows' size, or half of it
    // when fp32 chunk landmarks are scored for bf16 K/V rows.
    constexpr int RB = D * (int)sizeof(T);
    const int64_t gw = (int64_t)blockIdx.x * kScoreWaves + wave;
    const int64_t nw = (int64_t)pf_wgs * kScoreWaves;
    if (pres.where != nullptr) {  // rows kept across steps: V rows, one per entry
      extern __shared__ ResQueue s_queues[];  // [2][kScoreWaves], launched with them
      gather_rows_res<RB>(pf, gw, nw, pres, s_queues[wave], s_queues[kScoreWaves + wave]);
      return;
    }
    if constexpr (sizeof(T) == 4) {
      if (pf.row_bytes == RB / 2) {
        gather_rows<RB / 2>(pf, gw, nw);
        return;
      }
    }
    gather_rows<RB>(pf, gw, nw);
    return;
  }
  int bh, tile;
  xcd_tile_map((int)blockIdx.x - pf_wgs, tiles, BH, bh, tile);
  const int64_t n = chunk_len(lens[bh / H], len_shift, n_max);
  const int64_t tile0 = (int64_t)tile * S::TILE;
  if (tile0 >= n && !fill_pad) return;

  const int col = lane % S::LPR;
  const int rsub = lane / S::LPR;
  float qr[Q][S::EPL];
#pragma unroll
  for (int j = 0; j < Q; ++j)
#pragma unroll
    for (int e = 0; e < S::EPL; ++e) qr[j][e] = q[((int64_t)bh * Q + j) * D + col * S::EPL + e];

  const T* kb = keys + (int64_t)bh * n_max * D + col * S::EPL;
  float* sb = scores + (int64_t)bh * Q * n_max;
  // The score this lane finishes: value index v = lane % LPR = u * Q + j.
  const int vj = col % Q;
  const int vu = col / Q;

  // Both iterations' rows are loaded before either is scored, so that a
  // lane keeps 2U loads in flight.  Rows past n load row n-1 instead (an
  // iteration with no row below n loads nothing): the loads stay
  // unconditional so all of them are in flight together, and the butterfly
  // never mixes rows, so those lanes' scores are simply not stored.  The
  // keys are read once: non-temporal loads keep them from evicting the
  // scores (and prefetched rows) that the next kernels read from L2.
  u32x4 raw_it[S::ITERS][S::U];
#pragma unroll
  for (int it = 0; it < S::ITERS; ++it) {
    const int64_t key0 = tile0 + ((int64_t)it * kScoreWaves + wave) * S::KPI;
    if (key0 < n) {
#pragma unroll
      for (int u = 0; u < S::U; ++u) {
        const int64_t row = key0 + u * S::RPI + rsub;
        const int64_t rr = row < n ? row : n - 1;
        raw_it[it][u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kb + rr * D));
      }
    }
  }

#pragma unroll
  for (int it = 0; it < S::ITERS; ++it) {
    const int64_t key0 = tile0 + ((int64_t)it * kScoreWaves + wave) * S::KPI;
    if (key0 >= n_max) break;
    const int64_t my_row = key0 + vu * S::RPI + rsub;
    if (key0 >= n) {
      if (fill_pad && my_row < n_max) sb[vj * n_max + my_row] = -INFINITY;
      continue;
    }
    const u32x4 (&raw)[S::U] = raw_it[it];
    float acc[S::U * Q];
#pragma unroll
    for (int u = 0; u < S::U; ++u) {
      float f[S::EPL];
      Unpack<T>::run(raw[u], f);
#pragma unroll
      for (int j = 0; j < Q; ++j) {
        float a = 0.f;
#pragma unroll
        for (int e = 0; e < S::EPL; ++e) a = fmaf(f[e], qr[j][e], a);
        acc[u * Q + j] = a;
      }
    }
    Butterfly<S::LPR, S::U * Q>::run(acc, lane);
    const float sc = acc[0] * scale;
    if (my_row < n) {
      sb[vj * n_max + my_row] = sc;
    } else if (fill_pad && my_row < n_max) {
      sb[vj * n_max + my_row] = -INFINITY;
    }
    if (gmax != nullptr) {
      // Max over the lanes of one group: every rsub (lane bits from LPR up)
      // and VPG consecutive vu (col bits from Q up); keys past n count as
      // -inf.  Lane gi * VPG * Q + j then holds group gi of query j.
      float m = my_row < n ? sc : -INFINITY;
#pragma unroll
      for (int b = S::LPR; b < 64; b <<= 1) m = fmaxf(m, __shfl_xor(m, b));
#pragma unroll
      for (int b = Q; b < Q * S::VPG; b <<= 1) m = fmaxf(m, __shfl_xor(m, b));
      if (lane < S::LPR && vu % S::VPG == 0)
        gmax[((int64_t)bh * Q + vj) * gstride + key0 / kMaxGroup + vu / S::VPG] = m;
    }
  }
}

// One workgroup per score row: max, sum of exp, normalise (0 past len).
__global__ __launch_bounds__(1024) void k_softmax_rows(float* __restrict__ scores,
                                                       const int32_t* __restrict__ lens, int H,
                                                       int Q, int64_t n_max) {
  __shared__ float s_red[16];
  const int row = blockIdx.x;
  const int b = (row / Q) / H;
  const int64_t n = clamp_len(lens[b], n_max);
  float* s = scores + (int64_t)row * n_max;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;

  float m = -INFINITY;
  for (int64_t i = threadIdx.x; i < n; i += blockDim.x) m = fmaxf(m, s[i]);
  m = wave_max(m);
  if (lane == 0) s_red[wave] = m;
  __syncthreads();
  m = -INFINITY;
  for (int w = 0; w < nw; ++w) m = fmaxf(m, s_red[w]);
  __syncthreads();

  float t = 0.f;
  for (int64_t i = threadIdx.x; i < n; i += blockDim.x) t += expf(s[i] - m);
  t = wave_sum(t);
  if (lane == 0) s_red[wave] = t;
  __syncthreads();
  t = 0.f;
  for (int w = 0; w < nw; ++w) t += s_red[w];
  const float inv = 1.0f / t;

  for (int64_t i = threadIdx.x; i < n_max; i += blockDim.x)
    s[i] = (i < n) ? expf(s[i] - m) * inv : 0.f;
}

struct ScoreLaunch {
  const float* q;
  const void* keys;
  const int32_t* lens;
  int B, H;
  int64_t n_max;
  float scale;
  bool fill_pad;
  float* scores;
  GatherJob pf;
  int pf_wgs;
  hipStream_t s;
  hipEvent_t ev_start, ev_stop;
  int64_t* zero3;
  int len_shift;
  GatherRes pres;
  float* gmax;
  int64_t gstride;
};

template <typename T, int D, int Q>
hipError_t launch_score_t(const ScoreLaunch& a) {
  using S = ScoreShape<T, D, Q>;
  const int BH = a.B * a.H;
  const int64_t tiles = (a.n_max + S::TILE - 1) / S::TILE;
  if (BH == 0 || (tiles == 0 && a.pf_wgs == 0 && a.zero3 == nullptr)) return hipSuccess;
  const int64_t grid = (tiles > 0 ? tiles * BH : 1) + a.pf_wgs;
  if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
  // The copy queues of a kept-rows prefetch (dynamic LDS, only then).
  const unsigned lds = a.pres.where != nullptr ? 2 * kScoreWaves * sizeof(ResQueue) : 0;
  if (a.ev_start != nullptr && a.ev_stop != nullptr) {
    // Events taken by the dispatch itself: the kernel's own duration.
    hipExtLaunchKernelGGL((k_score<T, D, Q>), dim3((unsigned)grid), dim3(kScoreWaves * 64), lds,
                          a.s, a.ev_start, a.ev_stop, 0, a.q, static_cast<const T*>(a.keys),
                          a.lens, BH, a.H, a.n_max, (int)tiles, a.scale, a.scores,
                          a.fill_pad ? 1 : 0, a.pf, a.pf_wgs, a.zero3, a.len_shift, a.pres,
                          a.gmax, a.gstride);
  } else {
    hipLaunchKernelGGL((k_score<T, D, Q>), dim3((unsigned)grid), dim3(kScoreWaves * 64), lds, a.s,
                       a.q, static_cast<const T*>(a.keys), a.lens, BH, a.H, a.n_max, (int)tiles,
                       a.scale, a.scores, a.fill_pad ? 1 : 0, a.pf, a.pf_wgs, a.zero3,
                       a.len_shift, a.pres, a.gmax, a.gstride);
  }
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_score_q(int Q, const ScoreLaunch& a) {
  if (Q == 1) return launch_score_t<T, D, 1>(a);
  return launch_score_t<T, D, 2>(a);
}

}  // namespace

hipError_t launch_score(const float* q, const void* keys, const int32_t* lens, int B, int H,
                        int Q, int D, int64_t n_max, int dtype, float scale, bool fill_pad,
                        float* scores, const GatherJob* pf, int pf_wgs, hipStream_t s,
                        hipEvent_t ev_start, hipEvent_t ev_stop, int64_t* zero3,
                        int len_shift, const GatherRes* pres, float* gmax) {
  ScoreLaunch a{q, keys, lens, B, H, n_max, scale, fill_pad, scores, GatherJob{}, 0, s,
                ev_start, ev_stop, zero3, len_shift, GatherRes{}, gmax,
                max_group_stride(n_max)};
  if (pf != nullptr && pf->total > 0 && pf_wgs > 0) {
    // The prefetched K/V rows are the scored rows' size, or (fp32 landmarks
    // of bf16 rows) half of it.
    const int rb = D * (dtype == kBF16 ? 2 : 4);
    if (pf->row_bytes != rb && !(dtype == kF32 && pf->row_bytes == rb / 2))
      return hipErrorInvalidValue;
    if ((pf->total << pf->run_shift) > kGatherMaxRows) return hipErrorInvalidValue;
    a.pf = *pf;
    a.pf_wgs = (pf_wgs + 7) & ~7;  // keeps the scoring tiles' XCD placement
    if (pres != nullptr) {
      // Kept rows: V plane only, one row per entry, the scored rows' size.
      if (pf->ksrc != nullptr || pf->run_shift != 0 || pf->row_bytes != rb ||
          pf->m > pf->dst_rows_per_bh || pf->total > kGatherMaxRows)
        return hipErrorInvalidValue;
      a.pres = *pres;
    }
  }
  if (dtype == kBF16) {
    if (D == 128) return launch_score_q<uint16_t, 128>(Q, a);
    return launch_score_q<uint16_t, 64>(Q, a);
  }
  if (D == 128) return launch_score_q<float, 128>(Q, a);
  return launch_score_q<float, 64>(Q, a);
}

hipError_t launch_softmax_rows(float* scores, const int32_t* lens, int B, int H, int Q,
                               int64_t n_max, hipStream_t s) {
  const int rows = B * H * Q;
  if (rows == 0 || n_max == 0) return hipSuccess;
  hipLaunchKernelGGL(k_softmax_rows, dim3(rows), dim3(1024), 0, s, scores, lens, H, Q, n_max);
  return hipGetLastError();
}

}  // namespace dd
