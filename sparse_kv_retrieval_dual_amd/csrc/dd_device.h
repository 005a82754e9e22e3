// Device-side helpers shared by the gfx950 kernels: bf16 unpacking, DPP
// lane exchanges, the transposing butterfly reduction, block scans, and the
// order-preserving integer key of an fp32 score.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dd {

// Native 16-byte vector (one dwordx4 load or store per lane).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// A packed pair of bf16 values in one 32-bit word: element 0 in the low
// half.  Widening bf16 to fp32 appends sixteen zero bits.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Sixteen bytes of a key/value row -> fp32 elements.
template <typename T>
struct Unpack;

template <>
struct Unpack<uint16_t> {  // bf16 bit patterns
  static constexpr int N = 8;
  __device__ __forceinline__ static void run(const u32x4& r, float (&f)[8]) {
    f[0] = bf16_lo(r.x); f[1] = bf16_hi(r.x);
    f[2] = bf16_lo(r.y); f[3] = bf16_hi(r.y);
    f[4] = bf16_lo(r.z); f[5] = bf16_hi(r.z);
    f[6] = bf16_lo(r.w); f[7] = bf16_hi(r.w);
  }
};

template <>
struct Unpack<float> {
  static constexpr int N = 4;
  __device__ __forceinline__ static void run(const u32x4& r, float (&f)[4]) {
    f[0] = __uint_as_float(r.x); f[1] = __uint_as_float(r.y);
    f[2] = __uint_as_float(r.z); f[3] = __uint_as_float(r.w);
  }
};

// DPP controls (GFX9 encoding).
constexpr int kDppQuadXor1 = 0xB1;      // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;      // quad_perm [2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141;  // lane i <-> 7-i within each 8 lanes
constexpr int kDppRowMirror = 0x140;      // lane i <-> 15-i within each 16 lanes

template <int CTRL>
__device__ __forceinline__ float dpp_move(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// The lane paired with this one at butterfly level HALF (pairs differ in
// the lane bit HALF and lie in the same aligned group of 2*HALF lanes).
template <int HALF>
__device__ __forceinline__ float partner(float v) {
  if constexpr (HALF == 32) return __shfl_xor(v, 32);
  else if constexpr (HALF == 16) return __shfl_xor(v, 16);
  else if constexpr (HALF == 8) return dpp_move<kDppRowMirror>(v);
  else if constexpr (HALF == 4) return dpp_move<kDppRowHalfMirror>(v);
  else if constexpr (HALF == 2) return dpp_move<kDppQuadXor2>(v);
  else return dpp_move<kDppQuadXor1>(v);
}

// Transposing butterfly: G lanes (an aligned group) each hold NV partial
// sums x[0..NV) (NV <= G, both powers of two).  Afterwards x[0] in every
// lane holds the group total of value index (lane % G) / (G / NV); when
// NV < G that total is replicated in G / NV neighbouring lanes.  Each level
// halves the live values, so the work is NV-1 adds instead of NV log2(G).
template <int G, int NV>
struct Butterfly {
  __device__ __forceinline__ static void run(float* x, int lane) {
    if constexpr (G > 1) {
      constexpr int HALF = G / 2;
      if constexpr (NV > 1) {
        const bool upper = (lane & HALF) != 0;
#pragma unroll
        for (int v = 0; v < NV / 2; ++v) {
          const float keep = upper ? x[v + NV / 2] : x[v];
          const float send = upper ? x[v] : x[v + NV / 2];
          x[v] = keep + partner<HALF>(send);
        }
        Butterfly<HALF, NV / 2>::run(x, lane);
      } else {
        x[0] += partner<HALF>(x[0]);
        Butterfly<HALF, 1>::run(x, lane);
      }
    }
  }
};

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

__device__ __forceinline__ int wave_sum_int(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// Number of set bits of `mask` in lanes below this one.
__device__ __forceinline__ int lanes_below(uint64_t mask) {
  return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                        __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// Inclusive prefix sum over the 64 lanes of a wave, all in DPP: shifts by
// 1, 2, 4 and 8 lanes within each row of 16, then the row broadcasts of
// lane 15 (into rows 1 and 3) and lane 31 (into rows 2 and 3).  Lanes with
// no source lane add 0.
constexpr int kDppRowShr1 = 0x111;
constexpr int kDppRowShr2 = 0x112;
constexpr int kDppRowShr4 = 0x114;
constexpr int kDppRowShr8 = 0x118;
constexpr int kDppRowBcast15 = 0x142;
constexpr int kDppRowBcast31 = 0x143;

__device__ __forceinline__ int wave_inclusive_scan(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, kDppRowShr1, 0xF, 0xF, false);
  x += __builtin_amdgcn_update_dpp(0, x, kDppRowShr2, 0xF, 0xF, false);
  x += __builtin_amdgcn_update_dpp(0, x, kDppRowShr4, 0xF, 0xF, false);
  x += __builtin_amdgcn_update_dpp(0, x, kDppRowShr8, 0xF, 0xF, false);
  x += __builtin_amdgcn_update_dpp(0, x, kDppRowBcast15, 0xA, 0xF, false);
  x += __builtin_amdgcn_update_dpp(0, x, kDppRowBcast31, 0xC, 0xF, false);
  return x;
}

// Two alternating LDS scan buffers of 2 * NW ints each.  A block scan
// writes the per-wave totals of one buffer, waits at one barrier and reads
// them back; the next scan uses the other buffer, so a thread still reading
// this one is never overwritten (any writer of it has passed the next
// scan's barrier, which this reader has not reached yet).  All threads make
// the same sequence of scans, so the phase is uniform.
struct ScanBufs {
  int* base;  // 4 * NW ints
  int phase;
  __device__ __forceinline__ int* next(int nw) {
    int* p = base + phase * 2 * nw;
    phase ^= 1;
    return p;
  }
};

// Exclusive prefix sums of a and b over a block of NW waves, with one
// barrier; also returns both block totals.  All threads must call it.
template <int NW>
__device__ __forceinline__ void block_scan_pair(int a, int b, ScanBufs& sb, int& ea, int& eb,
                                                int& ta, int& tb) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  int* buf = sb.next(NW);
  const int ia = wave_inclusive_scan(a);
  const int ib = wave_inclusive_scan(b);
  if (lane == 63) {
    buf[wave] = ia;
    buf[NW + wave] = ib;
  }
  __syncthreads();
  int pa = 0, pb = 0, sa = 0, sbt = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const int va = buf[w];
    const int vb = buf[NW + w];
    pa += (w < wave) ? va : 0;
    pb += (w < wave) ? vb : 0;
    sa += va;
    sbt += vb;
  }
  ea = pa + ia - a;
  eb = pb + ib - b;
  ta = sa;
  tb = sbt;
}

// Exclusive prefix sum of a over a block of NW waves, with one barrier;
// also returns the block total.  All threads must call it.
template <int NW>
__device__ __forceinline__ int block_scan(int a, ScanBufs& sb, int& total) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  int* buf = sb.next(NW);
  const int ia = wave_inclusive_scan(a);
  if (lane == 63) buf[wave] = ia;
  __syncthreads();
  int pa = 0, sa = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const int va = buf[w];
    pa += (w < wave) ? va : 0;
    sa += va;
  }
  total = sa;
  return pa + ia - a;
}

// Exclusive prefix sum over the block (blockDim.x a multiple of 64, at most
// 1024 threads).  s_tmp needs 16 ints.  Returns this thread's exclusive sum
// and the block total; all threads must call it.
__device__ __forceinline__ int block_exclusive_scan(int v, int* s_tmp, int& total) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int nwaves = blockDim.x >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  if (lane == 63) s_tmp[wave] = x;
  __syncthreads();
  int before = 0, tot = 0;
  for (int w = 0; w < nwaves; ++w) {
    const int t = s_tmp[w];
    before += (w < wave) ? t : 0;
    tot += t;
  }
  __syncthreads();
  total = tot;
  return before + x - v;
}

__device__ __forceinline__ int block_sum_int(int v, int* s_tmp) {
  int total;
  (void)block_exclusive_scan(v, s_tmp, total);
  return total;
}

// Order-preserving key of an fp32 value: a < b (as floats, -0 == +0)
// iff key(a) < key(b) (as unsigned integers).
__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Workgroups of one launch are dealt to the 8 XCDs round-robin.  Map the
// 1-D grid so that all tiles of a (b, h) slab land on one XCD (its scores
// then stay in that XCD's L2 for the next kernel), when the slab count
// allows it.
__device__ __forceinline__ void xcd_tile_map(int w, int tiles, int slabs, int& slab, int& tile) {
  if ((slabs & 7) == 0) {
    const int x = w & 7;
    const int r = w >> 3;
    tile = r % tiles;
    slab = (r / tiles) * 8 + x;
  } else {
    slab = w / tiles;
    tile = w - slab * tiles;
  }
}

__device__ __forceinline__ int64_t clamp_len(int32_t len, int64_t n_max) {
  const int64_t n = len;
  return n < 0 ? 0 : (n > n_max ? n_max : n);
}

// Chunks of 2^shift rows that cover the first len rows (len for shift 0),
// at most n_max of them.
__device__ __forceinline__ int64_t chunk_len(int32_t len, int shift, int64_t n_max) {
  const int64_t n = len < 0 ? 0 : (((int64_t)len + (1 << shift) - 1) >> shift);
  return n > n_max ? n_max : n;
}

}  // namespace dd
