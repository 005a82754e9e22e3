// The C ABI: argument validation, error reporting, pinned host memory, the
// per-stage entry points and the layer step (the layer-aware transfer
// schedule over a ring of layer-scoped slots, arXiv page of DualDecoder,
// section 1; paper-daily summary, technical-method section).
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <string>
#include <vector>

#include "dd.h"
#include "dd_internal.h"
#include "gather_body.h"
#include "gather_res.h"

struct dd_ctx {
  int device = -1;
  int ring_slots = 1;
  int gather_cus = 0;
  int prefetch_wgs = 0;             // 0: sized per layer (prefetch_wgs_for)
  int prefetch_mode = DD_PREFETCH_AUTO;
  int k_rows = DD_KROWS_DEVICE;
  int perturb_side_us = 0;          // race detection: stalls before each side /
  int perturb_main_us = 0;          // main-stream stage of the layer step
  int select_prefetch_slabs = 0;    // 0: split by sizes; > 0: that many; -1: none
  hipStream_t side = nullptr;       // prefetch gathers
  hipStream_t main_own = nullptr;   // CU-masked main stream (gather_cus > 0 only)
  hipEvent_t ev_start = nullptr;    // caller stream at entry
  hipEvent_t ev_end = nullptr;      // own main stream at exit
  std::vector<hipEvent_t> ev_gathered;  // per slot: prefetch finished
  std::vector<hipEvent_t> ev_free;      // per slot: attention finished
};

namespace {

// Workgroups of a kept-rows prefetch per prefetch_wgs: 4 (128 at the default
// 32) was the fastest of 1 to 8, on the side stream and inside the scoring
// kernel alike, for a 4-layer decode step at batch 16, k = 1024 on MI355X.
constexpr int kResidentWgsScale = 4;

// Host-link bytes a layer's selection kernel hides before its attention
// needs the prediction's rows: about 5 us at about 50 GB/s.  256 KiB (8
// slabs of 32 KiB) was the fastest of 6 to 20 slabs for the 7B layer at
// c = 8 (38.1-38.4 us a step, against 39.5-40.4 us with 12) and at c = 16
// (36.4-36.6 against 37.8-37.9 us) on MI355X.
constexpr int64_t kSelectWindowLinkBytes = int64_t(256) << 10;
// Bytes the key scan streams from HBM while the host link moves one byte
// of prefetch beside it.
constexpr int64_t kScanBytesPerLinkByte = 100;
// Smallest per-layer prefetch that DD_PREFETCH_AUTO puts on the side stream
// when there are several layers.
constexpr int64_t kSideMinPrefetchBytes = int64_t(16) << 20;

// Workgroups of one layer's prefetch when the context leaves it open: 32 for
// a small prefetch (1 MiB at batch 1, k = 128: 16 to 32 were equal, 8 too
// few); inside the scoring kernel 64 from 16 MiB up (84 MiB at batch 4 x 40
// heads, k = 2048: 2.06 ms per layer against 2.14 ms with 32), while on the
// side stream 64 slowed a 32-layer step at batch 16, k = 1024 from 102.5 to
// 107.6 ms; times kResidentWgsScale for kept rows.
int prefetch_wgs_for(const dd_ctx* c, int64_t rows, int row_bytes, bool resident, bool fused) {
  int w = c->prefetch_wgs;
  if (w == 0) w = fused && !resident && rows * row_bytes >= (int64_t(16) << 20) ? 64 : 32;
  return resident ? kResidentWgsScale * w : w;
}

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(DD_ERR_HIP, "%s: %s (%d)", what, hipGetErrorString(e), (int)e);
}

#define DD_CHECK_HIP(expr, what)              \
  do {                                        \
    hipError_t e_ = (expr);                   \
    if (e_ != hipSuccess) return hip_fail(e_, what); \
  } while (0)

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t align_up(size_t v) { return (v + 255) & ~size_t(255); }

int check_shape(int B, int H, int D, int64_t n_max, int dtype) {
  if (B < 0 || H < 0) return fail(DD_ERR_INVALID_ARG, "B and H must be >= 0 (B=%d H=%d)", B, H);
  if ((int64_t)B * H > (int64_t)1 << 24) return fail(DD_ERR_UNSUPPORTED, "B*H too large");
  if (D != 64 && D != 128) return fail(DD_ERR_UNSUPPORTED, "D must be 64 or 128 (got %d)", D);
  if (dtype != DD_F32 && dtype != DD_BF16)
    return fail(DD_ERR_UNSUPPORTED, "dtype must be DD_F32 or DD_BF16 (got %d)", dtype);
  if (n_max < 0 || n_max >= ((int64_t)1 << 31))
    return fail(DD_ERR_UNSUPPORTED, "n_max must be in [0, 2^31) (got %lld)", (long long)n_max);
  return DD_OK;
}

int check_k(int k) {
  if (k < 1 || k > DD_MAX_K) return fail(DD_ERR_UNSUPPORTED, "k must be in [1, %d] (got %d)", DD_MAX_K, k);
  return DD_OK;
}

// Workspace of the layer step, carved in this order: the two score planes
// of a layer and their group maxima (kMaxGroup keys per group).
struct StepLayout {
  size_t scores, gmax, total;
};

StepLayout step_layout(int B, int H, int D, int64_t n_max, int k) {
  const size_t BH = (size_t)B * H;
  StepLayout l{};
  size_t off = 0;
  l.scores = off;
  off += align_up(BH * 2 * (size_t)n_max * sizeof(float));
  l.gmax = off;
  off += align_up(BH * 2 * (size_t)dd::max_group_stride(n_max) * sizeof(float));
  l.total = off;
  (void)D;
  (void)k;
  return l;
}

size_t slot_bytes(int B, int H, int D, int k, int dtype) {
  return 2 * (size_t)B * H * 2 * k * D * dd::elem_bytes(dtype);
}

// Rows kept across steps, per layer (byte offsets, 256-byte aligned): two
// slots of V rows ([BH][2k][D] each), their key lists ([BH][2k] int32
// each), the key -> row map ([BH][n_max] int32) and the prefetch's host-row
// counter; `layer` is the stride between layers.
struct ResidentLayout {
  size_t vbytes, ibytes;  // one slot's V rows, one slot's key list
  size_t vslot, idx, where, counter, layer;
};

ResidentLayout resident_layout(int B, int H, int D, int64_t n_max, int k, int dtype) {
  const size_t BH = (size_t)B * H;
  const size_t rows = 2 * (size_t)k;
  ResidentLayout r{};
  r.vbytes = align_up(BH * rows * D * dd::elem_bytes(dtype));
  r.ibytes = align_up(BH * rows * sizeof(int32_t));
  r.vslot = 0;
  r.idx = 2 * r.vbytes;
  r.where = r.idx + 2 * r.ibytes;
  r.counter = r.where + align_up(BH * (size_t)n_max * sizeof(int32_t));
  r.layer = r.counter + 256;
  return r;
}

}  // namespace

extern "C" {

DD_API const char* dd_last_error(void) { return g_err.c_str(); }

DD_API int dd_version(void) { return 100; }

DD_API int dd_host_alloc(size_t bytes, void** host_ptr) {
  if (host_ptr == nullptr) return fail(DD_ERR_INVALID_ARG, "host_ptr is NULL");
  *host_ptr = nullptr;
  if (bytes == 0) return DD_OK;
  void* p = nullptr;
  hipError_t e = hipHostMalloc(&p, bytes, hipHostMallocMapped | hipHostMallocPortable);
  if (e != hipSuccess || p == nullptr)
    return fail(DD_ERR_ALLOC, "hipHostMalloc(%zu) failed: %s", bytes, hipGetErrorString(e));
  void* dp = nullptr;
  e = hipHostGetDevicePointer(&dp, p, 0);
  if (e != hipSuccess || dp != p) {
    (void)hipHostFree(p);
    return fail(DD_ERR_ALLOC, "pinned memory is not mapped at the same address on the device");
  }
  *host_ptr = p;
  return DD_OK;
}

DD_API int dd_host_free(void* host_ptr) {
  if (host_ptr == nullptr) return DD_OK;
  DD_CHECK_HIP(hipHostFree(host_ptr), "hipHostFree");
  return DD_OK;
}

DD_API int dd_score(const float* q, const void* keys, const int32_t* lens, int B, int H, int Q,
                    int D, int64_t n_max, int kv_dtype, float scale, int kind, float* scores,
                    hipStream_t stream) {
  int rc = check_shape(B, H, D, n_max, kv_dtype);
  if (rc) return rc;
  if (Q != 1 && Q != 2) return fail(DD_ERR_UNSUPPORTED, "Q must be 1 or 2 (got %d)", Q);
  if (kind != DD_LOGITS && kind != DD_ALPHA) return fail(DD_ERR_UNSUPPORTED, "unknown kind %d", kind);
  if ((int64_t)B * H == 0 || n_max == 0) return DD_OK;
  if (!q || !keys || !lens || !scores) return fail(DD_ERR_INVALID_ARG, "null pointer argument");
  if (!aligned16(keys)) return fail(DD_ERR_INVALID_ARG, "keys must be 16-byte aligned");
  const float sc = scale > 0.f ? scale : 1.0f / sqrtf((float)D);
  hipError_t e = dd::launch_score(q, keys, lens, B, H, Q, D, n_max, kv_dtype, sc, true, scores,
                                  nullptr, 0, stream);
  if (e != hipSuccess) return hip_fail(e, "score kernel launch");
  if (kind == DD_ALPHA) {
    e = dd::launch_softmax_rows(scores, lens, B, H, Q, n_max, stream);
    if (e != hipSuccess) return hip_fail(e, "softmax kernel launch");
  }
  return DD_OK;
}

DD_API int dd_topk(const float* scores, const int32_t* lens, int B, int H, int Q, int64_t n_max,
                   int k, int32_t* idx, hipStream_t stream) {
  int rc = check_shape(B, H, 64, n_max, DD_F32);
  if (rc) return rc;
  rc = check_k(k);
  if (rc) return rc;
  if (Q != 1 && Q != 2) return fail(DD_ERR_UNSUPPORTED, "Q must be 1 or 2 (got %d)", Q);
  if ((int64_t)B * H == 0) return DD_OK;
  if (!lens || !idx || (!scores && n_max > 0)) return fail(DD_ERR_INVALID_ARG, "null pointer argument");
  hipError_t e = dd::launch_topk(scores, lens, B, H, Q, n_max, k, idx, idx + k, (int64_t)Q * k,
                                 nullptr, nullptr, stream);
  if (e != hipSuccess) return hip_fail(e, "top-k kernel launch");
  return DD_OK;
}

DD_API int dd_gather(const void* k_host, const void* v_host, const int32_t* idx,
                     const int32_t* cnt, int B, int H, int m, int D, int64_t n_max, int dtype,
                     void* k_rows, void* v_rows, hipStream_t stream) {
  int rc = check_shape(B, H, D, n_max, dtype);
  if (rc) return rc;
  if (m < 0) return fail(DD_ERR_INVALID_ARG, "m must be >= 0 (got %d)", m);
  if ((int64_t)B * H * m == 0) return DD_OK;
  if (!idx) return fail(DD_ERR_INVALID_ARG, "idx is NULL");
  if (!k_host && !v_host) return fail(DD_ERR_INVALID_ARG, "both host planes are NULL");
  if ((k_host && !k_rows) || (v_host && !v_rows))
    return fail(DD_ERR_INVALID_ARG, "destination missing for a host plane");
  if ((k_host && (!aligned16(k_host) || !aligned16(k_rows))) ||
      (v_host && (!aligned16(v_host) || !aligned16(v_rows))))
    return fail(DD_ERR_INVALID_ARG, "host and row buffers must be 16-byte aligned");
  const int rowb = D * dd::elem_bytes(dtype);
  hipError_t e = dd::launch_gather(k_host, v_host, n_max, rowb, idx, m, cnt, B * H,
                                   k_host ? k_rows : nullptr, v_host ? v_rows : nullptr, m, 0, 0,
                                   stream);
  if (e != hipSuccess) return hip_fail(e, "gather kernel launch");
  return DD_OK;
}

static int chunk_shift_of(int chunk, int* cs) {
  int s = 0;
  while (s < 7 && (1 << s) < chunk) ++s;
  if (chunk < 1 || chunk > 64 || (1 << s) != chunk)
    return fail(DD_ERR_INVALID_ARG, "chunk must be a power of two in [1, 64] (got %d)", chunk);
  *cs = s;
  return DD_OK;
}

DD_API int dd_gather_chunks(const void* k_host, const void* v_host, const int32_t* idx,
                            const int32_t* cnt, int B, int H, int m, int chunk, int D,
                            int64_t n_max, int dtype, void* k_rows, void* v_rows,
                            hipStream_t stream) {
  int rc = check_shape(B, H, D, n_max, dtype);
  if (rc) return rc;
  int cs = 0;
  rc = chunk_shift_of(chunk, &cs);
  if (rc) return rc;
  if (m < 0) return fail(DD_ERR_INVALID_ARG, "m must be >= 0 (got %d)", m);
  if ((int64_t)m * chunk > 0x7fffffff) return fail(DD_ERR_INVALID_ARG, "m * chunk too large");
  if ((int64_t)B * H * m == 0) return DD_OK;
  if (!idx) return fail(DD_ERR_INVALID_ARG, "idx is NULL");
  if (!k_host && !v_host) return fail(DD_ERR_INVALID_ARG, "both host planes are NULL");
  if ((k_host && !k_rows) || (v_host && !v_rows))
    return fail(DD_ERR_INVALID_ARG, "destination missing for a host plane");
  if ((k_host && (!aligned16(k_host) || !aligned16(k_rows))) ||
      (v_host && (!aligned16(v_host) || !aligned16(v_rows))))
    return fail(DD_ERR_INVALID_ARG, "host and row buffers must be 16-byte aligned");
  const int rowb = D * dd::elem_bytes(dtype);
  hipError_t e = dd::launch_gather(k_host, v_host, n_max, rowb, idx, m, cnt, B * H,
                                   k_host ? k_rows : nullptr, v_host ? v_rows : nullptr,
                                   (int64_t)m * chunk, 0, 0, stream, cs);
  if (e != hipSuccess) return hip_fail(e, "gather kernel launch");
  return DD_OK;
}

DD_API int dd_landmarks(const void* keys, const int32_t* lens, int B, int H, int D,
                        int64_t n_max, int chunk, int dtype, float* landmarks,
                        hipStream_t stream) {
  int rc = check_shape(B, H, D, n_max, dtype);
  if (rc) return rc;
  int cs = 0;
  rc = chunk_shift_of(chunk, &cs);
  if (rc) return rc;
  if ((int64_t)B * H == 0 || n_max == 0) return DD_OK;
  if (!keys || !lens || !landmarks) return fail(DD_ERR_INVALID_ARG, "null pointer argument");
  if (!aligned16(keys) || !aligned16(landmarks))
    return fail(DD_ERR_INVALID_ARG, "keys and landmarks must be 16-byte aligned");
  hipError_t e = dd::launch_landmarks(keys, lens, B, H, D, n_max, cs, dtype, landmarks, stream);
  if (e != hipSuccess) return hip_fail(e, "landmark kernel launch");
  return DD_OK;
}

DD_API int dd_kv_append(void* k_dev, void* k_host, void* v_host, const void* new_k,
                        const void* new_v, const int32_t* lens, int32_t* lens_out, int B, int H,
                        int D, int64_t n_max, int dtype, int chunk, float* landmarks,
                        hipStream_t stream) {
  int rc = check_shape(B, H, D, n_max, dtype);
  if (rc) return rc;
  int cs = 0;
  if (landmarks != nullptr) {
    rc = chunk_shift_of(chunk, &cs);
    if (rc) return rc;
  }
  if ((int64_t)B * H == 0) return DD_OK;
  if (!k_dev || !k_host || !v_host || !new_k || !new_v || !lens)
    return fail(DD_ERR_INVALID_ARG, "null pointer argument");
  if (lens_out == lens) return fail(DD_ERR_INVALID_ARG, "lens_out must not alias lens");
  if (!aligned16(k_dev) || !aligned16(k_host) || !aligned16(v_host) || !aligned16(new_k) ||
      !aligned16(new_v) || (landmarks && !aligned16(landmarks)))
    return fail(DD_ERR_INVALID_ARG, "buffers must be 16-byte aligned");
  hipError_t e = dd::launch_kv_append(k_dev, k_host, v_host, new_k, new_v, lens, lens_out, B, H,
                                      D, n_max, dtype, cs, landmarks, stream);
  if (e != hipSuccess) return hip_fail(e, "append kernel launch");
  return DD_OK;
}

DD_API size_t dd_attn_workspace(int B, int H, int k, int D) {
  if (B <= 0 || H <= 0 || k <= 0) return 0;
  return dd::attn_workspace(B, H, k, D);
}

DD_API int dd_sparse_attn(const float* q, int64_t q_stride_bh, const void* k_rows,
                          const void* v_rows, const int32_t* pos, const int32_t* cnt, int B,
                          int H, int k, int m, int D, int dtype, float scale, float* out,
                          float* lse, void* ws, size_t ws_bytes, hipStream_t stream) {
  int rc = check_shape(B, H, D, 0, dtype);
  if (rc) return rc;
  rc = check_k(k);
  if (rc) return rc;
  if (m < 0) return fail(DD_ERR_INVALID_ARG, "m must be >= 0 (got %d)", m);
  if ((int64_t)B * H == 0) return DD_OK;
  if (!q || !out || (m > 0 && (!k_rows || !v_rows)))
    return fail(DD_ERR_INVALID_ARG, "null pointer argument");
  if (q_stride_bh < D) return fail(DD_ERR_INVALID_ARG, "q_stride_bh must be >= D");
  if (m > 0 && (!aligned16(k_rows) || !aligned16(v_rows)))
    return fail(DD_ERR_INVALID_ARG, "row buffers must be 16-byte aligned");
  const size_t need = dd::attn_workspace(B, H, k, D);
  if (ws_bytes < need || (need > 0 && ws == nullptr))
    return fail(DD_ERR_WORKSPACE, "workspace too small: need %zu bytes, got %zu", need, ws_bytes);
  const float sc = scale > 0.f ? scale : 1.0f / sqrtf((float)D);
  hipError_t e = dd::launch_attn(q, q_stride_bh, k_rows, v_rows, pos, cnt, B, H, k, m, D, dtype,
                                 sc, out, lse, ws, stream);
  if (e != hipSuccess) return hip_fail(e, "attention kernel launch");
  return DD_OK;
}

DD_API int dd_sparse_attn_noalloc(const float* q, int64_t q_stride_bh, const void* k_rows,
                                  const void* v_rows, const int32_t* pos, const int32_t* cnt,
                                  int B, int H, int k, int m, int D, int dtype, float scale,
                                  float* out, float* lse, hipStream_t stream) {
  int rc = check_shape(B, H, D, 0, dtype);
  if (rc) return rc;
  rc = check_k(k);
  if (rc) return rc;
  if (m < 0) return fail(DD_ERR_INVALID_ARG, "m must be >= 0 (got %d)", m);
  if ((int64_t)B * H == 0) return DD_OK;
  if (!q || !out || (m > 0 && (!k_rows || !v_rows)))
    return fail(DD_ERR_INVALID_ARG, "null pointer argument");
  if (q_stride_bh < D) return fail(DD_ERR_INVALID_ARG, "q_stride_bh must be >= D");
  if (m > 0 && (!aligned16(k_rows) || !aligned16(v_rows)))
    return fail(DD_ERR_INVALID_ARG, "row buffers must be 16-byte aligned");
  const size_t need = dd::attn_workspace_used(B, H, k, D);
  if (need > dd::kAttnScratchMaxBytes)
    return fail(DD_ERR_WORKSPACE,
                "dd_sparse_attn_noalloc: these sizes need %zu bytes of chunk partials, more than "
                "the library's %zu-byte scratch (fewer chunks per (b, h), or B*H >= 512, fit; "
                "dd_sparse_attn takes a workspace of any size)",
                need, dd::kAttnScratchMaxBytes);
  void* ws = nullptr;
  if (need > 0) DD_CHECK_HIP(dd::attn_scratch(&ws), "scratch address");
  const float sc = scale > 0.f ? scale : 1.0f / sqrtf((float)D);
  hipError_t e = dd::launch_attn(q, q_stride_bh, k_rows, v_rows, pos, cnt, B, H, k, m, D, dtype,
                                 sc, out, lse, ws, stream);
  if (e != hipSuccess) return hip_fail(e, "attention kernel launch");
  return DD_OK;
}

DD_API size_t dd_ring_bytes(int ring_slots, int B, int H, int D, int k, int dtype) {
  if (ring_slots <= 0 || B <= 0 || H <= 0 || k <= 0) return 0;
  return (size_t)ring_slots * slot_bytes(B, H, D, k, dtype);
}

DD_API size_t dd_resident_bytes(int L, int B, int H, int D, int64_t n_max, int k, int dtype) {
  if (L <= 0 || B <= 0 || H <= 0 || k <= 0 || n_max <= 0 || D <= 0) return 0;
  return (size_t)L * resident_layout(B, H, D, n_max, k, dtype).layer;
}

DD_API size_t dd_layer_step_workspace(int B, int H, int D, int64_t n_max, int k) {
  if (B <= 0 || H <= 0 || k <= 0 || n_max < 0) return 0;
  return step_layout(B, H, D, n_max, k).total;
}

DD_API int dd_ctx_create(const dd_ctx_config* cfg, dd_ctx** ctx) {
  if (!cfg || !ctx) return fail(DD_ERR_INVALID_ARG, "null pointer argument");
  *ctx = nullptr;
  if (cfg->ring_slots < 1 || cfg->ring_slots > 64)
    return fail(DD_ERR_INVALID_ARG, "ring_slots must be in [1, 64] (got %d)", cfg->ring_slots);
  if (cfg->gather_cus < 0 || cfg->prefetch_wgs < 0)
    return fail(DD_ERR_INVALID_ARG, "gather_cus and prefetch_wgs must be >= 0");
  if (cfg->prefetch_mode < DD_PREFETCH_AUTO || cfg->prefetch_mode > DD_PREFETCH_FUSED)
    return fail(DD_ERR_INVALID_ARG, "unknown prefetch_mode %d", cfg->prefetch_mode);
  if (cfg->k_rows != DD_KROWS_DEVICE && cfg->k_rows != DD_KROWS_HOST)
    return fail(DD_ERR_INVALID_ARG, "unknown k_rows %d", cfg->k_rows);
  if (cfg->perturb_side_us < 0 || cfg->perturb_main_us < 0 || cfg->perturb_side_us > 100000 ||
      cfg->perturb_main_us > 100000)
    return fail(DD_ERR_INVALID_ARG, "perturb_side_us / perturb_main_us must be in [0, 100000]");
  if (cfg->select_prefetch_slabs < -1)
    return fail(DD_ERR_INVALID_ARG, "select_prefetch_slabs must be >= -1");
  dd_ctx* c = new dd_ctx();
  c->ring_slots = cfg->ring_slots;
  c->gather_cus = cfg->gather_cus;
  c->prefetch_wgs = cfg->prefetch_wgs;
  c->prefetch_mode = cfg->prefetch_mode;
  c->k_rows = cfg->k_rows;
  c->perturb_side_us = cfg->perturb_side_us;
  c->perturb_main_us = cfg->perturb_main_us;
  c->select_prefetch_slabs = cfg->select_prefetch_slabs;
  hipError_t e = hipGetDevice(&c->device);
  const int cus = dd::device_info().cus;
  if (e == hipSuccess && c->gather_cus > 0) {
    if (c->gather_cus >= cus) {
      delete c;
      return fail(DD_ERR_INVALID_ARG, "gather_cus must be below the CU count (%d)", cus);
    }
    // Side stream on the last gather_cus CUs, own main stream on the rest.
    std::vector<uint32_t> side_mask((cus + 31) / 32, 0u), main_mask((cus + 31) / 32, 0u);
    for (int i = 0; i < cus; ++i) {
      if (i >= cus - c->gather_cus) side_mask[i / 32] |= 1u << (i % 32);
      else main_mask[i / 32] |= 1u << (i % 32);
    }
    e = hipExtStreamCreateWithCUMask(&c->side, (uint32_t)side_mask.size(), side_mask.data());
    if (e == hipSuccess)
      e = hipExtStreamCreateWithCUMask(&c->main_own, (uint32_t)main_mask.size(), main_mask.data());
  } else if (e == hipSuccess) {
    e = hipStreamCreateWithFlags(&c->side, hipStreamNonBlocking);
  }
  if (e == hipSuccess) e = hipEventCreateWithFlags(&c->ev_start, hipEventDisableTiming);
  if (e == hipSuccess) e = hipEventCreateWithFlags(&c->ev_end, hipEventDisableTiming);
  for (int i = 0; e == hipSuccess && i < c->ring_slots; ++i) {
    hipEvent_t a = nullptr, b = nullptr;
    e = hipEventCreateWithFlags(&a, hipEventDisableTiming);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&b, hipEventDisableTiming);
    if (a) c->ev_gathered.push_back(a);
    if (b) c->ev_free.push_back(b);
  }
  if (e != hipSuccess) {
    dd_ctx_destroy(c);
    return hip_fail(e, "context creation");
  }
  *ctx = c;
  return DD_OK;
}

DD_API int dd_ctx_destroy(dd_ctx* c) {
  if (c == nullptr) return DD_OK;
  if (c->side) (void)hipStreamSynchronize(c->side);
  if (c->main_own) (void)hipStreamSynchronize(c->main_own);
  for (hipEvent_t e : c->ev_gathered) (void)hipEventDestroy(e);
  for (hipEvent_t e : c->ev_free) (void)hipEventDestroy(e);
  if (c->ev_start) (void)hipEventDestroy(c->ev_start);
  if (c->ev_end) (void)hipEventDestroy(c->ev_end);
  if (c->side) (void)hipStreamDestroy(c->side);
  if (c->main_own) (void)hipStreamDestroy(c->main_own);
  delete c;
  return DD_OK;
}

DD_API int dd_layer_step(dd_ctx* c, const dd_layer_step_args* a) {
  if (!c || !a) return fail(DD_ERR_INVALID_ARG, "null pointer argument");
  int dev = -1;
  DD_CHECK_HIP(hipGetDevice(&dev), "hipGetDevice");
  if (dev != c->device) return fail(DD_ERR_INVALID_ARG, "context belongs to device %d, current is %d", c->device, dev);
  int rc = check_shape(a->B, a->H, a->D, a->n_max, a->dtype);
  if (rc) return rc;
  rc = check_k(a->k);
  if (rc) return rc;
  if (a->L < 0) return fail(DD_ERR_INVALID_ARG, "L must be >= 0");
  if (a->L == 0 || (int64_t)a->B * a->H == 0) return DD_OK;
  // With K rows read from the scoring copy the host K plane is never read,
  // so it may be absent.
  const bool k_from_dev = c->k_rows == DD_KROWS_DEVICE;
  if (!a->lens || !a->q || !a->k_dev || (!a->k_host && !k_from_dev) || !a->v_host ||
      !a->cur_idx || !a->spec_idx || !a->out)
    return fail(DD_ERR_INVALID_ARG, "null pointer argument");
  for (int l = 0; l < a->L; ++l) {
    const void* kh = a->k_host ? a->k_host[l] : nullptr;
    if (!a->q[l] || !a->k_dev[l] || (!kh && !k_from_dev) || !a->v_host[l] || !a->cur_idx[l] ||
        !a->spec_idx[l] || !a->out[l])
      return fail(DD_ERR_INVALID_ARG, "null pointer for layer %d", l);
    if (!aligned16(a->k_dev[l]) || (kh && !aligned16(kh)) || !aligned16(a->v_host[l]))
      return fail(DD_ERR_INVALID_ARG, "K/V buffers of layer %d must be 16-byte aligned", l);
  }
  // Selection by chunk landmarks: ks chunks of 2^cs rows each, k rows in all.
  int cs = 0;
  if (a->chunk > 1) {
    while ((1 << cs) < a->chunk) ++cs;
    if ((1 << cs) != a->chunk || a->chunk > 64)
      return fail(DD_ERR_INVALID_ARG, "chunk must be 0, 1 or a power of two up to 64 (got %d)",
                  a->chunk);
    if (a->k % a->chunk != 0)
      return fail(DD_ERR_INVALID_ARG, "k (%d) must be a multiple of chunk (%d)", a->k, a->chunk);
    if (!a->landmarks) return fail(DD_ERR_INVALID_ARG, "chunk > 1 needs landmarks");
    for (int l = 0; l < a->L; ++l)
      if (!a->landmarks[l] || !aligned16(a->landmarks[l]))
        return fail(DD_ERR_INVALID_ARG, "landmarks of layer %d missing or not 16-byte aligned", l);
  } else if (a->chunk < 0) {
    return fail(DD_ERR_INVALID_ARG, "chunk must be >= 0");
  }
  const int B = a->B, H = a->H, D = a->D, k = a->k, BH = B * H;
  const int ks = k >> cs;                                      // entries selected per query
  const int64_t n_sel = (a->n_max + (1 << cs) - 1) >> cs;      // rows of the scored matrix
  const size_t sbytes = slot_bytes(B, H, D, k, a->dtype);
  // Rows kept across steps: each layer's own pair of slots replaces the ring.
  const bool resident = a->resident != nullptr;
  const ResidentLayout RL = resident_layout(B, H, D, a->n_max, k, a->dtype);
  if (resident) {
    if (cs != 0) return fail(DD_ERR_UNSUPPORTED, "rows kept across steps need chunk 0 or 1");
    if (c->k_rows != DD_KROWS_DEVICE)
      return fail(DD_ERR_UNSUPPORTED, "rows kept across steps need K rows from k_dev "
                                      "(DD_KROWS_DEVICE)");
    if (a->parity != 0 && a->parity != 1)
      return fail(DD_ERR_INVALID_ARG, "parity must be 0 or 1 (got %d)", a->parity);
    const size_t need = (size_t)a->L * RL.layer;
    if (a->resident_bytes < need || !aligned16(a->resident))
      return fail(DD_ERR_WORKSPACE, "resident state too small: need %zu bytes, got %zu", need,
                  a->resident_bytes);
  } else {
    const size_t ring_need = (size_t)c->ring_slots * sbytes;
    if (!a->ring || a->ring_bytes < ring_need || !aligned16(a->ring))
      return fail(DD_ERR_WORKSPACE, "ring too small: need %zu bytes, got %zu", ring_need,
                  a->ring_bytes);
  }
  const StepLayout lay = step_layout(B, H, D, a->n_max, k);
  if (!a->ws || a->ws_bytes < lay.total)
    return fail(DD_ERR_WORKSPACE, "workspace too small: need %zu bytes, got %zu", lay.total, a->ws_bytes);
  if (!aligned16(a->ws)) return fail(DD_ERR_INVALID_ARG, "workspace must be 16-byte aligned");

  const float sc = a->scale > 0.f ? a->scale : 1.0f / sqrtf((float)D);
  const int rowb = D * dd::elem_bytes(a->dtype);
  char* ws = static_cast<char*>(a->ws);
  float* scores = reinterpret_cast<float*>(ws + lay.scores);
  // Group maxima of the score rows, for a selection that reads only the
  // groups that can hold a selected key (rows longer than one tile).
  float* gmax = dd::topk_uses_maxima(n_sel) ? reinterpret_cast<float*>(ws + lay.gmax) : nullptr;
  const int R = c->ring_slots;
  hipStream_t caller = a->stream;
  hipStream_t ms = c->main_own ? c->main_own : caller;
  hipStream_t side = c->side;

  bool any_pred = false;
  if (a->pred)
    for (int l = 0; l < a->L; ++l) any_pred = any_pred || (a->pred[l] != nullptr);
  // Where the prediction is fetched: on the side stream ahead of the layer
  // (it can then overlap the previous layer's work), or by extra workgroups
  // of the layer's own scoring kernel (no second stream, no cross-stream
  // wait; the transfer overlaps that layer's key scan only).
  // With rows kept across steps, a layer's prefetch has its own slot to
  // fill and no slot to wait for; inside the layer's scoring kernel it
  // disturbed the main stream least (a 4-layer step at batch 16, k = 1024:
  // 5.96 ms against 6.70 ms on the side stream).  Without them the side
  // stream pays only where a layer's prefetch is large: its cross-stream
  // waits cost about 13 us per layer in graph replays (8 layers of the 7B
  // shape at batch 1, 1 MiB per layer: 78.5 against 66.1 us per layer, and
  // 54.0 against 40.9 with 8-key chunks), while at batch 16, k = 1024 (128
  // MiB per layer) it was 1% ahead.
  const int64_t pf_layer_bytes =
      (int64_t)BH * k * rowb * (c->k_rows == DD_KROWS_DEVICE ? 1 : 2);
  const bool fused = c->prefetch_mode == DD_PREFETCH_FUSED ||
                     (c->prefetch_mode == DD_PREFETCH_AUTO &&
                      (a->L == 1 || resident || pf_layer_bytes < kSideMinPrefetchBytes));
  const bool use_side = any_pred && !fused;
  // Where a fused prefetch runs.  Inside the scoring kernel it overlaps the
  // layer's key scan; the slabs whose transfer the scan cannot hide (HBM
  // streams about kScanBytesPerLinkByte bytes while the host link moves
  // one), up to what the link moves during a selection, are read instead by
  // their own selection workgroups, overlapping the selection (V rows of
  // kPrefetchRowBytes, at most kPrefetchMaxRows per slab, cached score rows).
  int pf_sel_slabs = 0;
  if (any_pred && fused && !resident && c->k_rows == DD_KROWS_DEVICE &&
      D * dd::elem_bytes(a->dtype) == dd::kPrefetchRowBytes && k <= dd::kPrefetchMaxRows &&
      n_sel <= dd::kPrefetchMaxScoreRow) {
    const int64_t per_slab = (int64_t)k * dd::kPrefetchRowBytes;
    const int64_t scan = (int64_t)BH * n_sel * D * (cs ? 4 : dd::elem_bytes(a->dtype));
    const int64_t hidden = scan / (kScanBytesPerLinkByte * per_slab);
    const int64_t window = kSelectWindowLinkBytes / per_slab;
    if (c->select_prefetch_slabs > 0)
      pf_sel_slabs = c->select_prefetch_slabs < BH ? c->select_prefetch_slabs : BH;
    else if (c->select_prefetch_slabs == 0 && hidden < BH)
      pf_sel_slabs = (int)(BH - hidden < window ? BH - hidden : window);
  }
  const int pf_score_slabs = BH - pf_sel_slabs;

  if (resident && a->reset) {  // both slots hold nothing; counters at zero
    for (int l = 0; l < a->L; ++l) {
      char* base = static_cast<char*>(a->resident) + (size_t)l * RL.layer;
      hipError_t e = dd::launch_fill_i32(reinterpret_cast<int32_t*>(base + RL.idx), -1,
                                         (int64_t)(2 * RL.ibytes / sizeof(int32_t)), caller);
      if (e == hipSuccess)
        e = dd::launch_fill_i32(reinterpret_cast<int32_t*>(base + RL.counter), 0, 2, caller);
      if (e != hipSuccess) return hip_fail(e, "resident state reset");
    }
  }
  // The start event orders the context's own streams after the caller's
  // work; with neither in use (one stream, the prefetch inside the scoring
  // kernel) it is not recorded at all.
  if (ms != caller || use_side)
    DD_CHECK_HIP(hipEventRecord(c->ev_start, caller), "record start");
  if (ms != caller) DD_CHECK_HIP(hipStreamWaitEvent(ms, c->ev_start, 0), "main waits start");
  if (use_side) DD_CHECK_HIP(hipStreamWaitEvent(side, c->ev_start, 0), "side waits start");

  auto tev = [&](int l, int i) -> hipEvent_t {
    return a->timing ? a->timing[(size_t)l * DD_STAGE_EVENTS + i] : nullptr;
  };

  for (int l = 0; l < a->L; ++l) {
    const int slot = l % R;
    char* kslot = resident ? nullptr : static_cast<char*>(a->ring) + (size_t)slot * sbytes;
    char* vslot = resident ? nullptr : kslot + sbytes / 2;
    // Rows kept across steps: this step fills slot `parity` of the layer and
    // reads rows the previous step left in the other one.
    dd::GatherRes res{};
    const void* old_v = nullptr;
    if (resident) {
      char* base = static_cast<char*>(a->resident) + (size_t)l * RL.layer;
      const int p = a->parity;
      vslot = base + RL.vslot + (size_t)p * RL.vbytes;
      kslot = vslot;  // unused: K rows come from k_dev
      old_v = base + RL.vslot + (size_t)(1 - p) * RL.vbytes;
      res = dd::GatherRes{reinterpret_cast<int32_t*>(base + RL.where),
                          reinterpret_cast<const int32_t*>(base + RL.idx + (size_t)(1 - p) * RL.ibytes),
                          reinterpret_cast<int32_t*>(base + RL.idx + (size_t)p * RL.ibytes),
                          static_cast<const uint8_t*>(old_v),
                          reinterpret_cast<unsigned long long*>(base + RL.counter)};
    }
    const int32_t* P = a->pred ? a->pred[l] : nullptr;
    // With K rows read from the scoring copy, only V rows cross the host
    // link (the slot's K plane stays unused).
    const bool kdev = c->k_rows == DD_KROWS_DEVICE;
    const void* khost = kdev ? nullptr : a->k_host[l];  // present unless kdev
    const dd::GatherJob pf{static_cast<const uint8_t*>(khost),
                           static_cast<const uint8_t*>(a->v_host[l]), a->n_max, P, ks, nullptr,
                           (int64_t)(fused ? pf_score_slabs : BH) * ks,
                           reinterpret_cast<uint8_t*>(kslot),
                           reinterpret_cast<uint8_t*>(vslot), 2 * (int64_t)k, 0, cs, rowb};
    // Bytes the prefetch moves: V rows (and K rows from the host).
    const int pf_wgs = prefetch_wgs_for(c, pf.total << cs, rowb * (kdev ? 1 : 2),
                                        resident, fused);

    if (P && use_side) {
      if (l >= R && !resident)
        DD_CHECK_HIP(hipStreamWaitEvent(side, c->ev_free[slot], 0), "side waits slot");
      if (c->perturb_side_us > 0)
        DD_CHECK_HIP(dd::launch_delay(c->perturb_side_us, side), "side-stream stall");
      if (tev(l, 5)) DD_CHECK_HIP(hipEventRecord(tev(l, 5), side), "timing");
      // A kept-rows prefetch runs on more workgroups: each wave's
      // lookups (index, then the old slot's row) leave its host loads idle
      // for a while, and its own layer's slots free it from waiting.
      hipError_t e =
          resident ? dd::launch_gather_resident(a->v_host[l], a->n_max, rowb, P, ks, BH, vslot,
                                                2 * (int64_t)k, res, pf_wgs,
                                                side)
                   : dd::launch_gather(khost, a->v_host[l], a->n_max, rowb, P, ks, nullptr, BH,
                                       kslot, vslot, 2 * (int64_t)k, 0, pf_wgs, side, cs);
      if (e != hipSuccess) return hip_fail(e, "prefetch gather launch");
      if (tev(l, 6)) DD_CHECK_HIP(hipEventRecord(tev(l, 6), side), "timing");
      DD_CHECK_HIP(hipEventRecord(c->ev_gathered[slot], side), "record gathered");
    }

    // Events 0 and 1 are taken by the scoring dispatch itself (its start and
    // end), so they time exactly that kernel.  The scoring kernel also zeroes
    // the layer's statistics, which the next kernel adds to.
    int64_t* st = a->stats ? a->stats + 3 * (size_t)l : nullptr;
    const bool score_ev = tev(l, 0) && tev(l, 1);
    if (tev(l, 0) && !score_ev) DD_CHECK_HIP(hipEventRecord(tev(l, 0), ms), "timing");
    hipError_t e = dd::launch_score(a->q[l], cs ? static_cast<const void*>(a->landmarks[l]) : a->k_dev[l],
                                    a->lens, B, H, 2, D, n_sel, cs ? DD_F32 : a->dtype,
                                    sc, false, scores, (P && fused && pf.total > 0) ? &pf : nullptr,
                                    pf_wgs, ms,
                                    score_ev ? tev(l, 0) : nullptr,
                                    score_ev ? tev(l, 1) : nullptr, st, cs,
                                    (P && fused && resident) ? &res : nullptr, gmax);
    if (e != hipSuccess) return hip_fail(e, "score kernel launch");
    if (tev(l, 1) && !score_ev) DD_CHECK_HIP(hipEventRecord(tev(l, 1), ms), "timing");
    if (P && use_side) DD_CHECK_HIP(hipStreamWaitEvent(ms, c->ev_gathered[slot], 0), "main waits prefetch");
    if (c->perturb_main_us > 0)
      DD_CHECK_HIP(dd::launch_delay(c->perturb_main_us, ms), "main-stream stall");
    // Top-k of both queries, the bookkeeping of the current one and its
    // attention in one kernel: each current-query row's workgroup attends
    // right after its selection, reading misses from host memory itself
    // (and storing them into their slot rows k + t); K rows come from the
    // scoring copy when kdev.
    const dd::FusedAttn fa{a->q[l], kslot, vslot, khost, a->v_host[l],
                           kdev ? a->k_dev[l] : nullptr, a->n_max, cs, D, a->dtype, sc,
                           a->out[l], a->lse ? a->lse[l] : nullptr, st,
                           a->out_spec ? a->out_spec[l] : nullptr,
                           (a->out_spec && a->out_spec[l] && a->lse_spec) ? a->lse_spec[l] : nullptr,
                           res.where, res.old_idx, res.new_idx, old_v, res.host_rows,
                           P ? pf_sel_slabs : 0};
    e = dd::launch_topk(scores, a->lens, B, H, 2, n_sel, ks, a->cur_idx[l], a->spec_idx[l], ks,
                        P, &fa, ms, cs, gmax);
    if (e != hipSuccess) return hip_fail(e, "top-k and attention kernel launch");
    for (int ev = 2; ev <= 4; ++ev)
      if (tev(l, ev)) DD_CHECK_HIP(hipEventRecord(tev(l, ev), ms), "timing");
    if (use_side) DD_CHECK_HIP(hipEventRecord(c->ev_free[slot], ms), "record slot free");
  }
  if (ms != caller) {
    DD_CHECK_HIP(hipEventRecord(c->ev_end, ms), "record end");
    DD_CHECK_HIP(hipStreamWaitEvent(caller, c->ev_end, 0), "caller waits end");
  }
  return DD_OK;
}

DD_API int dd_stream_copy(const void* src, void* dst, size_t bytes, hipStream_t stream) {
  if (bytes == 0) return DD_OK;
  if (!src || !dst) return fail(DD_ERR_INVALID_ARG, "null pointer argument");
  if ((bytes & 15) != 0 || !aligned16(src) || !aligned16(dst))
    return fail(DD_ERR_INVALID_ARG, "bytes and pointers must be multiples of 16");
  hipError_t e = dd::launch_stream_copy(src, dst, bytes, stream);
  if (e != hipSuccess) return hip_fail(e, "copy kernel launch");
  return DD_OK;
}

DD_API int dd_stream_read(const void* src, size_t bytes, void* sink, hipStream_t stream) {
  if (bytes == 0) return DD_OK;
  if (!src || !sink) return fail(DD_ERR_INVALID_ARG, "null pointer argument");
  if ((bytes & 15) != 0 || !aligned16(src) || !aligned16(sink))
    return fail(DD_ERR_INVALID_ARG, "bytes and pointers must be multiples of 16");
  hipError_t e = dd::launch_stream_read(src, bytes, sink, stream);
  if (e != hipSuccess) return hip_fail(e, "read kernel launch");
  return DD_OK;
}

}  // extern "C"
