/*
 * dd.h -- predictive sparse-KV decode hot path on MI355X (gfx950).
 *
 * The operations follow "DualDecoder: Accelerate Long Context LLM Inference
 * by Predictive Prefetch" (arXiv 2607.26475; abstract, sections 1 and 2.2,
 * Figure 1) and the paper-daily summary of it (core-formulas and
 * worked-example sections).  For one transformer layer of a batched decode
 * step they are:
 *
 *   1. score   s = q K^T / sqrt(d_k) for the current token's query and the
 *              speculated next token's query against every cached key
 *              (alpha = softmax(s) on request);
 *   2. topk    I = argtopk(alpha, k) per request, head and query;
 *   3. gather  copy the selected K/V rows from the host-resident full KV
 *              cache into a small layer-scoped GPU buffer;
 *   4. attend  decode attention of the current query over those rows only;
 *   and the layer step that chains them, prefetching the rows predicted by
 *   the previous step's speculated token on a side stream while the layer
 *   computes, and fetching the prediction's misses on the critical path.
 *
 * Conventions shared by every call:
 *   - All entry points are extern "C", return an int status (DD_OK = 0) and
 *     never throw.  On a non-OK status a message is kept per thread and
 *     returned by dd_last_error(); nothing has been enqueued.
 *   - Calls are asynchronous and ordered on the HIP stream passed in (NULL
 *     is the legacy default stream).  Faults inside a kernel surface at the
 *     caller's next synchronisation.
 *   - The caller owns every buffer.  Device pointers are HIP device memory;
 *     "host" pointers are pinned, device-mapped memory from dd_host_alloc.
 *     The compute calls allocate nothing.
 *   - Layouts are row-major and densely packed.  (b, h) addresses a slab;
 *     offsets are computed in 64 bits.  Indices are int32.
 *   - Supported: head dimension D in {64, 128}; K/V element type DD_F32 or
 *     DD_BF16 (raw bfloat16 bit patterns); Q in {1, 2}; 1 <= k <= DD_MAX_K;
 *     0 <= n_max < 2^31.  Other values return DD_ERR_UNSUPPORTED.
 *   - Values read from device memory are never trusted for addressing:
 *     lens[b] is clamped to [0, n_max]; an index outside the valid range
 *     produces a zero row (gather) or is skipped (attention).  These cases
 *     are defined behaviour, not errors.
 */
#ifndef DD_H
#define DD_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DD_API __attribute__((visibility("default")))

enum {
  DD_OK = 0,
  DD_ERR_INVALID_ARG = 1, /* null pointer, negative size, inconsistent shapes */
  DD_ERR_UNSUPPORTED = 2, /* D, dtype, Q or k outside the supported set */
  DD_ERR_WORKSPACE = 3,   /* workspace or ring smaller than required */
  DD_ERR_HIP = 4,         /* a HIP runtime call or kernel launch failed */
  DD_ERR_ALLOC = 5        /* dd_host_alloc could not pin the memory */
};

enum { DD_F32 = 0, DD_BF16 = 1 };      /* element type of K and V */
enum { DD_LOGITS = 0, DD_ALPHA = 1 };  /* what dd_score writes */

#define DD_MAX_K 4096
/* Events per layer recorded by dd_layer_step when args.timing is set (an
 * entry may be NULL to skip it): [0] start and [1] end of the scoring
 * kernel (taken by that dispatch itself when both are given); [2], [3] and
 * [4] all after the kernel that selects, does the bookkeeping, fetches the
 * misses and attends (a wait for a side-stream prefetch comes before it) --
 * all on the main stream -- and [5] before and [6] after the prefetch
 * gather on the side stream (left unrecorded when the prediction is fetched
 * inside the scoring kernel or the layer has none). */
#define DD_STAGE_EVENTS 7

/* Text of the last non-OK status returned on this thread ("" if none). */
DD_API const char* dd_last_error(void);

/* Library version: major * 10000 + minor * 100 + patch. */
DD_API int dd_version(void);

/* Pinned, device-mapped host memory for the full KV cache (arXiv page,
 * section 2.2: the full cache lives in host memory and selected entries are
 * brought back to the GPU).  The returned pointer is valid on the host and,
 * unchanged, in kernels on every device.  bytes == 0 returns NULL and DD_OK.
 * Free with dd_host_free.  DD_ERR_ALLOC if the runtime cannot pin. */
DD_API int dd_host_alloc(size_t bytes, void** host_ptr);
DD_API int dd_host_free(void* host_ptr);

/* Scoring (paper-daily summary, core-formulas section:
 * alpha = softmax(q K^T / sqrt(d_k)); its worked example scores every cached
 * key of the layer).
 *   q       device fp32 [B][H][Q][D]; plane 0 = current query, plane 1 =
 *           speculated next-token query.
 *   keys    device [B][H][n_max][D] of kv_dtype.  Each key row is read once
 *           for all Q queries.
 *   lens    device int32 [B]: keys [0, lens[b]) are valid.
 *   scale   multiplier of the dot products; <= 0 selects 1/sqrt(D).
 *   kind    DD_LOGITS: scores = scale * q.K (fp32 accumulation);
 *           DD_ALPHA: the softmax of those logits over the valid keys.
 *   scores  device fp32 [B][H][Q][n_max]; positions >= lens[b] are written
 *           as -inf (logits) or 0 (alpha).
 */
DD_API int dd_score(const float* q, const void* keys, const int32_t* lens, int B, int H,
                    int Q, int D, int64_t n_max, int kv_dtype, float scale, int kind,
                    float* scores, hipStream_t stream);

/* Selection I = argtopk(alpha, k) (paper-daily summary, core-formulas
 * section; Figure 1 "Top-k" on the arXiv page).  Softmax is increasing, so
 * selecting on logits gives the same set.
 *   scores  device fp32 [B][H][Q][n_max] (logits or alpha); entries at
 *           positions < lens[b] must not be NaN.
 *   idx     device int32 [B][H][Q][k]: the chosen positions in ascending
 *           order.  Ties go to the lower index; -0.0 equals +0.0.  When
 *           lens[b] < k, the first lens[b] slots hold 0..lens[b]-1 and the
 *           rest hold -1.
 */
DD_API int dd_topk(const float* scores, const int32_t* lens, int B, int H, int Q,
                   int64_t n_max, int k, int32_t* idx, hipStream_t stream);

/* Gather of selected rows from the host KV cache into device memory
 * (arXiv page, section 2.2 and Figure 1, "Sparse KV" / "Gather"; the
 * paper-daily worked example sizes one such transfer).  The rows are read
 * by a kernel directly over the host link.
 *   k_host, v_host  pinned host [B][H][n_max][D] of dtype (dd_host_alloc).
 *                   Either may be NULL to skip that plane.
 *   idx     device int32 [B][H][m]: row positions to fetch.
 *   cnt     device int32 [B][H] or NULL: only entries j < cnt[b][h] are
 *           processed (all m when NULL); rows j >= cnt are not written.
 *   k_rows, v_rows  device [B][H][m][D] of dtype (the one whose host plane
 *           is non-NULL must be non-NULL).  Row j = host row idx[j], byte for
 *           byte; an index outside [0, n_max) gives an all-zero row.
 */
DD_API int dd_gather(const void* k_host, const void* v_host, const int32_t* idx,
                     const int32_t* cnt, int B, int H, int m, int D, int64_t n_max,
                     int dtype, void* k_rows, void* v_rows, hipStream_t stream);

/* Chunk gather (arXiv page, section 2.2: the GPU picks important chunks
 * and retrieves their entries from host memory).  Entry j < cnt[b][h] (m if
 * cnt is NULL) names chunk idx[b][h][j]: its `chunk` consecutive host rows
 * from row chunk * idx are copied, byte for byte, to rows
 * [j * chunk, (j + 1) * chunk) of k_rows / v_rows ([B][H][m * chunk][D]).
 * A negative index, and every row at or past n_max, gives zero rows; entries
 * at or past cnt are left untouched.  chunk: a power of two in [1, 64].  The
 * rows of a chunk are contiguous in host memory, so the link carries runs of
 * chunk * D * element-size bytes.  Either plane may be NULL (not both). */
DD_API int dd_gather_chunks(const void* k_host, const void* v_host, const int32_t* idx,
                            const int32_t* cnt, int B, int H, int m, int chunk, int D,
                            int64_t n_max, int dtype, void* k_rows, void* v_rows,
                            hipStream_t stream);

/* Chunk landmarks: the compressed per-chunk keys that selection scores
 * (arXiv page, section 2.2, ShadowKV's chunk landmarks).  The pages do not
 * define a landmark; here it is the mean key of the chunk.
 *   landmarks[b][h][e][:] (fp32, ceil(n_max / chunk) rows per (b, h)) =
 *   the mean of keys[b][h][i][:] over the rows i of chunk e (i in
 *   [e * chunk, (e + 1) * chunk)) below lens[b], summed in fp32 in row order
 *   and divided by their count; 0 for a chunk with no such row.
 * keys: device [B][H][n_max][D] (dtype); chunk: a power of two in [1, 64].
 * Landmarks are built once per cache (and as it grows), not per step. */
DD_API int dd_landmarks(const void* keys, const int32_t* lens, int B, int H, int D,
                        int64_t n_max, int chunk, int dtype, float* landmarks,
                        hipStream_t stream);

/* KV append (arXiv page, section 2.1: each decoding step computes the new
 * token's key and value and appends them to the cache).  For every (b, h)
 * the new rows new_k[b][h], new_v[b][h] (device, [B][H][D], dtype) are
 * written to row lens[b] of k_dev (the device keys that are scored), k_host
 * and v_host (the pinned host cache), all [B][H][n_max][D].  lens_out (or
 * NULL) receives lens[b] + 1; it must not alias lens, since every (b, h)
 * reads lens[b].  A request with lens[b] outside [0, n_max) is left as it is
 * (lens_out[b] = lens[b]).  landmarks (or NULL): the chunk landmarks of the
 * cache (chunk as in dd_landmarks); the landmark of the chunk holding the new
 * row is recomputed, with the same arithmetic as dd_landmarks, so it equals
 * a rebuild of the grown cache bit for bit. */
DD_API int dd_kv_append(void* k_dev, void* k_host, void* v_host, const void* new_k,
                        const void* new_v, const int32_t* lens, int32_t* lens_out, int B, int H,
                        int D, int64_t n_max, int dtype, int chunk, float* landmarks,
                        hipStream_t stream);

/* Workspace bytes dd_sparse_attn needs for these sizes (0 when k <= 128:
 * one chunk, nothing to merge).  It holds the chunk partials. */
DD_API size_t dd_attn_workspace(int B, int H, int k, int D);

/* Decode attention over gathered rows only (Figure 1 "Attention" on the
 * arXiv page, fed by the sparse KV rows).  Split over row chunks with an
 * online softmax, then combined.
 *   q        device fp32; the query of (b, h) starts at q + (b*H+h)*q_stride_bh
 *            (D for a [B][H][D] array, 2*D for plane 0 of [B][H][2][D]).
 *   k_rows, v_rows  device [B][H][m][D] of dtype.
 *   pos      device int32 [B][H][k] or NULL: entry j uses row pos[j] (row j
 *            when NULL); a row outside [0, m) is skipped.
 *   cnt      device int32 [B][H] or NULL: entries j < cnt take part (k when
 *            NULL).
 *   out      device fp32 [B][H][D]: sum_j softmax_j(scale q.K_j) V_j; zeros
 *            when no entry takes part.
 *   lse      device fp32 [B][H] or NULL: log-sum-exp of the scaled logits
 *            (-inf when no entry takes part).
 *   ws       device workspace of at least dd_attn_workspace(B, H, k, D) bytes
 *            (no initial contents needed; calls that overlap on one
 *            workspace race).
 * The reduction order depends only on j, never on pos, so the result for
 * a given list of rows is bitwise the same wherever the rows sit.
 */
DD_API int dd_sparse_attn(const float* q, int64_t q_stride_bh, const void* k_rows,
                          const void* v_rows, const int32_t* pos, const int32_t* cnt, int B,
                          int H, int k, int m, int D, int dtype, float scale, float* out,
                          float* lse, void* ws, size_t ws_bytes, hipStream_t stream);

/* dd_sparse_attn for callers that cannot allocate memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation):
 * the same computation and arguments, without ws / ws_bytes.  The chunk
 * partials live in a 4 MiB scratch array inside the library, one per device
 * the library runs on, kept until the process ends; no call allocates or
 * frees anything.  Sizes whose partials exceed it (more than 4 MiB when
 * B*H < 512 and k > 128: B*H * ceil(k / 128) * (D + 2) * 4 bytes) return
 * DD_ERR_WORKSPACE with nothing enqueued.  The scratch needs no initial
 * contents.  All calls on one device share it: calls whose executions
 * overlap on one device (concurrent streams, host threads) race and must be
 * ordered by the caller.  The output is bitwise that of dd_sparse_attn. */
DD_API int dd_sparse_attn_noalloc(const float* q, int64_t q_stride_bh, const void* k_rows,
                                  const void* v_rows, const int32_t* pos, const int32_t* cnt,
                                  int B, int H, int k, int m, int D, int dtype, float scale,
                                  float* out, float* lse, hipStream_t stream);

/* ------------------------------------------------------------------------ */
/* Layer step: the layer-aware transfer schedule and the layer-scoped buffer */
/* (arXiv page, section 1: predicted entries are fetched early enough to hide */
/* the host-to-device transfer, prediction misses are corrected on the        */
/* critical path, and a layer-scoped memory manager keeps the runtime sparse  */
/* KV buffer small; paper-daily summary: transfers overlap the forward pass   */
/* on separate streams, and the buffer is O(k d) instead of O(n d)).          */

typedef struct dd_ctx dd_ctx;

typedef struct dd_ctx_config {
  int ring_slots;  /* layer slots in the ring buffer, >= 1 (2 lets layer l+1
                      prefetch while layer l attends) */
  int gather_cus;  /* 0: side stream without a CU mask.  > 0: the side stream
                      is restricted to this many CUs and the layer step's own
                      main stream to the others */
  int prefetch_wgs; /* workgroups of the prefetch gather (0: 32, or 64 for a
                      layer prefetch of 16 MiB or more inside the scoring
                      kernel; four times as many when rows are kept across
                      steps).  Fewer keep
                      fewer host reads outstanding, which disturbs the
                      concurrent HBM-bound scoring less; enough of them
                      still saturate the host link */
  int prefetch_mode; /* DD_PREFETCH_AUTO (fused for L == 1, when rows are
                      kept across steps, or when a layer's prefetch is under
                      16 MiB; side stream otherwise), DD_PREFETCH_SIDE or
                      DD_PREFETCH_FUSED */
  int k_rows;       /* DD_KROWS_DEVICE (0) or DD_KROWS_HOST: where attention
                      reads the K rows of the selected entries */
  /* Race detection: when > 0, dd_layer_step enqueues a fixed stall of about
     this many microseconds (a single-wave kernel that sleeps and ends) on
     the side stream before each prefetch gather (side) or on the main stream
     before each selection + attention kernel (main), so that tests can move
     the two streams' relative timing.  Results must not change; 0 in
     production. */
  int perturb_side_us;
  int perturb_main_us;
  /* Where a fused prefetch (no rows kept across steps) of 256-byte V rows
     (k <= 128 rows, score rows of at most 32768 entries, K rows from k_dev)
     runs: 0 splits it by the layer's sizes between the scoring kernel
     (beside the key scan) and the selection kernel (beside the selection;
     the last slabs); n > 0 gives the last min(n, B*H) slabs to the
     selection kernel; -1 keeps it all in the scoring kernel.  Other
     prefetches ignore it.  Results are identical for any value. */
  int select_prefetch_slabs;
} dd_ctx_config;

/* DD_PREFETCH_SIDE: the prediction of layer l is fetched on the side stream
 * as soon as its ring slot is free, so it overlaps earlier layers' work.
 * DD_PREFETCH_FUSED: it is fetched by extra workgroups of layer l's own
 * scoring kernel (one stream, no cross-stream wait; it overlaps that
 * layer's key scan).  Results are identical either way. */
enum { DD_PREFETCH_AUTO = 0, DD_PREFETCH_SIDE = 1, DD_PREFETCH_FUSED = 2 };

/* DD_KROWS_DEVICE: the layer step already holds every key in HBM for
 * scoring (k_dev), so attention reads the K row of each selected entry
 * there, and only V rows are fetched from the host (prefetch and misses);
 * the slot's K plane stays unused.  DD_KROWS_HOST: K and V rows both come
 * from the host copy into the slot, as for a system that keeps only
 * compressed keys on the GPU (arXiv page, section 2.2).  K bytes are the
 * same in both places, so the outputs are bitwise identical. */
enum { DD_KROWS_DEVICE = 0, DD_KROWS_HOST = 1 };

/* Creates the side stream and events on the current device.  The context
 * may only be used with that device current. */
DD_API int dd_ctx_create(const dd_ctx_config* cfg, dd_ctx** ctx);
DD_API int dd_ctx_destroy(dd_ctx* ctx);

/* Bytes of the ring for ring_slots slots.  A slot holds, per (b, h), 2k rows
 * of K and 2k rows of V: rows [0, k) are the prefetched prediction, rows
 * [k, 2k) the misses. */
DD_API size_t dd_ring_bytes(int ring_slots, int B, int H, int D, int k, int dtype);

/* Workspace bytes of dd_layer_step (the scores of one layer, reused layer
 * after layer). */
DD_API size_t dd_layer_step_workspace(int B, int H, int D, int64_t n_max, int k);

typedef struct dd_layer_step_args {
  int L, B, H, D, k, dtype;
  int64_t n_max;
  float scale;                  /* <= 0 selects 1/sqrt(D) */
  const int32_t* lens;          /* device int32 [B], shared by all layers */
  /* Host arrays of L pointers each: */
  const float* const* q;        /* device fp32 [B][H][2][D]: current, speculated */
  const void* const* k_dev;     /* device [B][H][n_max][D]: keys for scoring */
  const void* const* k_host;    /* pinned host [B][H][n_max][D]: the full cache.
                                   May be NULL (or hold NULL entries) when the
                                   context reads K rows from k_dev
                                   (DD_KROWS_DEVICE): the host K plane is then
                                   never read, and only V needs pinned memory */
  const void* const* v_host;    /* pinned host [B][H][n_max][D] */
  const int32_t* const* pred;   /* NULL (no prediction) or device int32 [B][H][k]
                                   per layer (an entry may be NULL): the previous
                                   step's speculated set, ascending, -1 at the end */
  int32_t* const* cur_idx;      /* out, device int32 [B][H][k]: true set */
  int32_t* const* spec_idx;     /* out, device int32 [B][H][k]: speculated set,
                                   the next step's prediction */
  float* const* out;            /* out, device fp32 [B][H][D] */
  float* const* lse;            /* NULL, or per layer device fp32 [B][H] (entries may be NULL) */
  int64_t* stats;               /* NULL or device int64 [L][3]: misses, hits, rows
                                   fetched over the host link (prefetched + misses) */
  void* ring;                   /* device, >= dd_ring_bytes(ring_slots, ...) */
  size_t ring_bytes;
  void* ws;                     /* device, >= dd_layer_step_workspace(...) */
  size_t ws_bytes;
  hipStream_t stream;           /* caller's stream; all work is ordered after
                                   earlier work on it and before later work */
  hipEvent_t* timing;           /* NULL or L * DD_STAGE_EVENTS events (see above) */
  /* Selection by chunk landmarks (arXiv page, section 2.2: chunks of adjacent
   * entries with compressed landmarks, from which the GPU picks important
   * chunks and retrieves their entries).  chunk 0 or 1: every key is scored
   * and k keys are selected (the default).  chunk = c in {2, 4, ..., 64}:
   * the c-row landmarks of each layer are scored instead of k_dev, k / c
   * chunks are selected per query (k must be a multiple of c), pred /
   * cur_idx / spec_idx hold chunk indices ([B][H][k / c]), every selected
   * chunk brings its c rows (those below lens[b]) to the slot and to
   * attention, and stats count chunks. */
  int chunk;
  const float* const* landmarks; /* chunk > 1: per layer device fp32
                                    [B][H][ceil(n_max / chunk)][D] (dd_landmarks) */
  /* Dual-token attention (arXiv page, section 1: the dual-token pipeline runs
   * the normal token and the retrieval-guiding token through the same
   * decoding flow).  NULL, or per layer (entries may be NULL) device fp32
   * [B][H][D]: the speculated query (plane 1 of q) attends over the same
   * selected rows as the current one, each K/V row read once for both; its
   * log-sum-exp goes to lse_spec (NULL, or per layer [B][H], entries may be
   * NULL).  out is unchanged bit for bit. */
  float* const* out_spec;
  float* const* lse_spec;
  /* Rows kept across steps (arXiv page, section 1: the prefetched entries of
   * a layer are those its next step is predicted to need).  NULL: the ring
   * of ring_slots slots is shared by the layers and every step fetches the
   * whole prediction over the host link.  Otherwise device memory of at
   * least dd_resident_bytes(L, B, H, D, n_max, k, dtype) bytes that gives
   * every layer two slots of its own, used in turn (ring and ring_bytes are
   * then unused): a predicted or missed row that the layer's previous step
   * already brought in is copied from there in HBM instead of crossing the
   * host link again.  Outputs are bitwise those of the ring; stats count as
   * rows fetched only the rows read over the link.  Needs chunk 0 or 1 and
   * DD_KROWS_DEVICE.  The host rows
   * must not change while they may be held, except by dd_kv_append (an
   * appended row was never selected before).  The state belongs to one
   * sequence of steps over the same layers and shapes. */
  void* resident;
  size_t resident_bytes;
  int parity;  /* 0 or 1, flipped by the caller from one step to the next */
  int reset;   /* non-zero: the state is cleared first (the first step, or
                  after the host cache was rewritten); nothing is read from it */
} dd_layer_step_args;

/* Bytes of the state of rows kept across steps for L layers (see
 * dd_layer_step_args.resident). */
DD_API size_t dd_resident_bytes(int L, int B, int H, int D, int64_t n_max, int k, int dtype);

/* Runs the layer step for layers 0..L-1.  Per layer, on the main stream:
 * score both queries, select both top-k sets, compare the true set with the
 * prediction (misses and the slot row of every selected entry), fetch the
 * misses into the slot, attend the current query over the true set.  On the
 * side stream, ahead of it: fetch the predicted rows into the layer's slot
 * as soon as the slot is free.  The outputs do not depend on the prediction
 * (bitwise): a prediction only changes which rows travel early. */
DD_API int dd_layer_step(dd_ctx* ctx, const dd_layer_step_args* args);

/* Measurement utility: a plain streaming device-to-device copy kernel
 * (bytes must be a multiple of 16, pointers 16-byte aligned).  Used to
 * calibrate hardware counters and to measure the achievable HBM rate. */
DD_API int dd_stream_copy(const void* src, void* dst, size_t bytes, hipStream_t stream);

/* Measurement utility: a plain streaming read of bytes at src (a multiple of
 * 16, 16-byte aligned) with the non-temporal loads the scoring kernel uses;
 * the achievable HBM read rate, the scoring kernel's own kind of traffic.
 * sink: device memory of at least 256 bytes (16-byte aligned) whose
 * contents afterwards are meaningless. */
DD_API int dd_stream_read(const void* src, size_t bytes, void* sink, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* DD_H */
