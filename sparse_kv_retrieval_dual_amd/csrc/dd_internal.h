// Internal launchers behind the C ABI.  Arguments are validated by the
// callers in abi.cpp; these functions only compute launch shapes and
// enqueue kernels on the given stream.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dd {

constexpr int kF32 = 0;
constexpr int kBF16 = 1;

struct DeviceInfo {
  int device = -1;
  int cus = 0;
  int lds_per_block = 65536;  // usable dynamic LDS bytes for one workgroup
};

// Properties of the current device (queried once per device).
const DeviceInfo& device_info();

inline int elem_bytes(int dtype) { return dtype == kF32 ? 4 : 2; }

struct GatherJob;
struct GatherRes;

// Keys per group of the group maxima the scoring kernel can write, and the
// stride between the maxima rows of [BH][Q][gstride] (16-byte aligned rows).
constexpr int kMaxGroup = 16;
inline int64_t max_group_stride(int64_t n_max) {
  return ((n_max + kMaxGroup - 1) / kMaxGroup + 3) & ~int64_t(3);
}

// Scaled logits of Q queries against every key; rows past lens[b] become
// -inf when fill_pad is set and are left untouched otherwise.  When pf is
// set, pf_wgs extra workgroups (dispatched first) run that row gather
// alongside the scoring (row_bytes = D * element size).  When both events
// are given they are recorded at the kernel's own start and end.  zero3
// (or null): three int64 counters the kernel sets to zero.  len_shift > 0:
// the rows are chunk landmarks, 2^len_shift keys each, and request b has
// ceil(lens[b] / 2^len_shift) of them.  pres (with pf): the prefetch of a
// layer whose rows are kept across steps (see launch_gather_resident).
// gmax (or null): [BH][Q][max_group_stride(n_max)] fp32 receives, for every
// group g of kMaxGroup keys holding a key below the row's length, the
// largest score of its keys below the length (groups past it are left as
// they are).
hipError_t launch_score(const float* q, const void* keys, const int32_t* lens, int B, int H,
                        int Q, int D, int64_t n_max, int dtype, float scale, bool fill_pad,
                        float* scores, const GatherJob* pf, int pf_wgs, hipStream_t s,
                        hipEvent_t ev_start = nullptr, hipEvent_t ev_stop = nullptr,
                        int64_t* zero3 = nullptr, int len_shift = 0,
                        const GatherRes* pres = nullptr, float* gmax = nullptr);

// In-place softmax of each score row over its valid keys; 0 past lens[b].
hipError_t launch_softmax_rows(float* scores, const int32_t* lens, int B, int H, int Q,
                               int64_t n_max, hipStream_t s);

// Attention fused into the top-k of the layer step: after its bookkeeping,
// the workgroup of each current-query row attends that query over the
// selection (slot rows, misses read from host memory and stored into
// their slot rows k + t).
struct FusedAttn {
  const float* q;        // [BH][2][D] (plane 0 attends); null: no attention
  const void* kslot;     // [BH][2k][D]
  const void* vslot;
  const void* k_host;    // pinned [BH][n_max][D] (unused when k_dev is set)
  const void* v_host;
  const void* k_dev;     // device keys [BH][n_rows][D]: K rows read from here
                         // (only V rows travel from the host), or null
  int64_t n_rows;        // rows per slab of the K/V copies
  int chunk_shift;       // entries are chunks of 2^chunk_shift rows (0: rows)
  int D, dtype;
  float scale;
  float* out;            // [BH][D]
  float* lse;            // [BH] or null
  int64_t* stats;        // {misses, hits, rows over the host link}, added to
                         // atomically (zeroed before the launch), or null
  float* out_spec;       // [BH][D]: the speculated query (plane 1) attends over
                         // the same rows, or null
  float* lse_spec;       // [BH] or null
  // Rows kept across steps (null where: every miss comes from the host).
  // vslot is this step's slot; old_vslot / old_idx the previous step's, whose
  // rows serve a miss they hold instead of the host; new_idx ([BH][2k]) and
  // where ([BH][n_rows]) record every row this step's slot holds; pf_host
  // holds the prefetch's count of rows read over the link (read and cleared
  // here).  One row per entry (chunk_shift 0), K rows from k_dev.
  int32_t* where;
  const int32_t* old_idx;
  int32_t* new_idx;
  const void* old_vslot;
  unsigned long long* pf_host;
  // The last pf_slabs slabs' prediction V rows were not prefetched before
  // this kernel: each of their current-query workgroups reads its own from
  // host memory during its selection (k << chunk_shift rows of
  // kPrefetchRowBytes, at most kPrefetchMaxRows) and stores them into slot
  // rows [0, k << chunk_shift) before its attention, as the prefetch gather
  // would (zero rows for entries outside the cache).  0: none.
  int pf_slabs;
};

// The prefetch a selection workgroup can do itself: rows of this size, at
// most this many (one 16-byte load per thread for each 16 rows), for score
// rows of at most kPrefetchMaxScoreRow entries (rows the kernel holds in LDS).
constexpr int kPrefetchRowBytes = 256;
constexpr int kPrefetchMaxRows = 128;
constexpr int64_t kPrefetchMaxScoreRow = 32768;

// Whether launch_topk takes its bound from group maxima for score rows of
// n_max entries (longer than one tile); only then are they worth writing.
bool topk_uses_maxima(int64_t n_max);

// Top-k of each score row.  Plane j of slab bh is written at
// (j == 0 ? out0 : out1) + bh * out_stride_bh.  attn (or null): the plane-0
// rows also do the prediction bookkeeping against pred ([BH][k], or null
// for no prediction) and then the fused attention.  len_shift > 0: the
// scores are of chunk landmarks of 2^len_shift rows, ceil(lens[b] /
// 2^len_shift) per request.  gmax (or null): the rows' group maxima as the
// scoring kernel writes them; rows with enough groups then take their bound
// from these and read only the groups that can hold a selected key.
hipError_t launch_topk(const float* scores, const int32_t* lens, int B, int H, int Q,
                       int64_t n_max, int k, int32_t* out0, int32_t* out1,
                       int64_t out_stride_bh, const int32_t* pred, const FusedAttn* attn,
                       hipStream_t s, int len_shift = 0, const float* gmax = nullptr);

// Row gather from pinned host memory.  Entry j < cnt[bh] (m if cnt is null)
// of slab bh copies the run of R = 2^run_shift host rows from row
// R * idx[bh*m + j] (zero rows where out of range) to destination rows
// bh*dst_rows_per_bh + dst_row0 + R*j onwards.  At most max_wgs workgroups
// (0: a default for a standalone copy) keep rows in flight.
hipError_t launch_gather(const void* k_host, const void* v_host, int64_t n_max, int row_bytes,
                         const int32_t* idx, int m, const int32_t* cnt, int BH, void* k_dst,
                         void* v_dst, int64_t dst_rows_per_bh, int dst_row0, int max_wgs,
                         hipStream_t s, int run_shift = 0);

// The prefetch of a layer whose rows are kept across steps: entry j of
// slab bh (key idx[bh*m + j]) goes to V row j of the new slot, from the old
// slot when it holds the key, else over the host link (see GatherRes).
hipError_t launch_gather_resident(const void* v_host, int64_t n_max, int row_bytes,
                                  const int32_t* idx, int m, int BH, void* v_dst,
                                  int64_t dst_rows_per_bh, const GatherRes& r, int max_wgs,
                                  hipStream_t s);

// Sets n 32-bit words at p to v.
hipError_t launch_fill_i32(int32_t* p, int32_t v, int64_t n, hipStream_t s);

size_t attn_workspace(int B, int H, int k, int D);

// Bytes of workspace launch_attn actually writes for these sizes (0 when
// one chunk per (b, h), or when a workgroup per (b, h) keeps every chunk
// partial in LDS).
size_t attn_workspace_used(int B, int H, int k, int D);

// Largest workspace the library's own attention scratch holds (4 MiB).
constexpr size_t kAttnScratchMaxBytes = size_t(4) << 20;

// The device address of the library's own attention scratch on the current
// device (kAttnScratchMaxBytes, 256-byte aligned), looked up once per device.
hipError_t attn_scratch(void** ptr);

// Sparse attention over gathered rows (entry j is row pos[j], or j).
hipError_t launch_attn(const float* q, int64_t q_stride_bh, const void* k_rows,
                       const void* v_rows, const int32_t* pos, const int32_t* cnt, int B, int H,
                       int k, int m, int D, int dtype, float scale, float* out, float* lse,
                       void* ws, hipStream_t s);

hipError_t launch_stream_copy(const void* src, void* dst, size_t bytes, hipStream_t s);

// A single-wave kernel that stalls its stream for about `us` microseconds
// (a fixed number of sleeps; it always ends).
hipError_t launch_delay(int us, hipStream_t s);

// Streaming read of bytes (a multiple of 16) at src; sink: 64 device words.
hipError_t launch_stream_read(const void* src, size_t bytes, void* sink, hipStream_t s);

// Chunk landmarks: out[bh][e] (fp32, D wide, ceil(n_max / 2^chunk_shift)
// rows per slab) = the mean of keys[bh][i] over the rows i of chunk e below
// lens[b]; zero for a chunk with no such row.
hipError_t launch_landmarks(const void* keys, const int32_t* lens, int B, int H, int D,
                            int64_t n_max, int chunk_shift, int dtype, float* out, hipStream_t s);

// Appends new_k / new_v ([BH][D]) at row lens[b] of k_dev, k_host and
// v_host, writes lens_out[b] = lens[b] + 1 (lens_out may be null), and, with
// landmarks, recomputes the landmark of the chunk holding the new row.
hipError_t launch_kv_append(void* k_dev, void* k_host, void* v_host, const void* new_k,
                            const void* new_v, const int32_t* lens, int32_t* lens_out, int B,
                            int H, int D, int64_t n_max, int dtype, int chunk_shift,
                            float* landmarks, hipStream_t s);

}  // namespace dd
