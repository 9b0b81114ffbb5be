/*
 * gqa_decode.h — C ABI of the MI355X (gfx950) single-token grouped-query
 * decode-attention library (libgqa_decode.so).
 *
 * Operation. For every request b and query head h (Hq = 32 or 16 per
 * request, sharing 8 KV heads, head dimension 128, so head h reads KV head
 * h / G with G = Hq / 8):
 *
 *     s_j     = q_scale * k_scale / sqrt(128) * dot(q[b,h,:], K[b,h/G,j,:])
 *     out[b,h,:] = v_scale * sum_{j < L_b} softmax_j(s) * V[b,h/G,j,:]
 *
 * with L_b = seq_lens[b]. For an INT8 cache, K[b,g,j,:] = k8[b,g,j,:] *
 * ks[b,g,j] and V[b,g,j,:] = v8[b,g,j,:] * vs[b,g,j] with one bf16 scale per
 * (position, KV head) row. Sources: the FlashInfer sm110_gqa_decode article
 * (cf-1.com news 5454068): "why a separate SM110 GQA decode path" (fixed
 * 32/8/128 geometry, one query token per request), "input contract" (layout
 * and the device-only lengths), "convenience API" (signature, the grouped
 * q view, the log2-domain scale), "prepared continuous decode" (prepare
 * phase, the three differences, lifecycle and concurrency, num_splits and
 * the FP32 split workspace); and the Thor FP8 KV-cache porting notes
 * (kipfel.ltd), section 1, patches 1-2 (uint8 bytes reinterpreted as
 * float8_e4m3fn; scores *= k_scale, normalised output *= v_scale); and the
 * Qwen3-VL on Jetson Orin doc (stargazers.cn, FlashRT), "INT8 KV cache"
 * (INT8 mirrors with one BF16 scale per (position, KV head) row, decode
 * geometry 16 query heads / 8 KV heads / head_dim 128).
 *
 * Layouts (all dense, contiguous, row-major, device memory, 16-byte aligned):
 *   q         [batch, Hq, 128]                 q_dtype (F16 or BF16)
 *   kv        [batch, 2, 8, capacity, 128]     kv_dtype; plane 0 = K, 1 = V
 *                                              (FP8: OCP E4M3FN bytes;
 *                                               INT8_ROWSCALE: int8 values)
 *   kv_scales [batch, 2, 8, capacity]          bf16 row scales, INT8 only
 *                                              (plane 0 = K, 1 = V)
 *   seq_lens  [batch] int32, read on the device only (4-byte aligned)
 *   out       [batch, Hq, 128]                 q_dtype (written by the call)
 *
 * Ownership. The caller owns q, kv, seq_lens and out and must keep them
 * alive until the enqueued work (and any captured graph containing it)
 * has retired. A prepared handle stores their addresses, never copies, and
 * owns only its split workspace.
 *
 * Lengths. Keeping 1 <= seq_lens[b] <= capacity is the caller's job; the
 * host never reads them. Kernels clamp each length to [0, capacity] so they
 * never read outside the cache: a length <= 0 yields an all-zero output row
 * block and a length > capacity behaves as capacity. Slots at or beyond the
 * length are never loaded (their contents, NaN included, cannot matter).
 *
 * Errors. Every entry point returns a gqa_status_t and never throws. On any
 * error nothing is enqueued and out is untouched; gqa_last_error() returns a
 * thread-local message describing the most recent failure on this thread.
 * Every kernel launch is checked.
 */
#ifndef GQA_DECODE_H_
#define GQA_DECODE_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GQA_API __attribute__((visibility("default")))

#define GQA_NUM_Q_HEADS 32
/* The other accepted query-head count: 2 query heads per KV head. */
#define GQA_NUM_Q_HEADS_2TO1 16
#define GQA_NUM_KV_HEADS 8
#define GQA_HEAD_DIM 128
/* Capacities up to this value take the short route (one workgroup per
 * (request, KV head), no workspace), as the article's routing paragraph
 * does for capacity <= 64. */
#define GQA_SHORT_CAPACITY_MAX 64
/* Split chunks are multiples of this many tokens (one wave tile). */
#define GQA_CHUNK_GRANULE 16
/* Largest accepted capacity (keeps every per-head K/V plane below 2 GiB). */
#define GQA_MAX_CAPACITY (1 << 22)

typedef enum gqa_status {
  GQA_OK = 0,
  GQA_ERR_INVALID_ARG = 1,        /* bad pointer, geometry, dtype, scale, split */
  GQA_ERR_ALIAS = 2,              /* out overlaps q, kv or seq_lens */
  GQA_ERR_UNSUPPORTED_DEVICE = 3, /* current device is not gfx950 */
  GQA_ERR_CAPTURE = 4,            /* convenience call would allocate during capture */
  GQA_ERR_OUT_OF_MEMORY = 5,      /* workspace allocation failed */
  GQA_ERR_HIP = 6                 /* a HIP runtime call or launch failed */
} gqa_status_t;

typedef enum gqa_dtype {
  GQA_F16 = 0,
  GQA_BF16 = 1,
  GQA_FP8_E4M3 = 2,     /* KV only: OCP E4M3FN bytes (torch.float8_e4m3fn) */
  GQA_INT8_ROWSCALE = 3 /* KV only: int8 values + one bf16 scale per (slot, KV head)
                           row, passed separately (gqa_decode_int8) */
} gqa_dtype_t;

/* Problem descriptor. Fields are int32/float so the struct has one layout
 * for every caller. Accepted dtype pairs (q, kv): (F16, F16), (BF16, BF16),
 * (F16, FP8_E4M3), (BF16, FP8_E4M3), (F16, INT8_ROWSCALE),
 * (BF16, INT8_ROWSCALE); every pair with 32 or 16 query heads. out has q's
 * dtype. k_scale and v_scale must be finite and > 0, and must equal 1.0 for
 * a 16-bit cache (a scale there is rejected rather than silently ignored);
 * on an INT8 cache they multiply on top of the row scales. */
typedef struct gqa_desc {
  int32_t batch;        /* >= 0; 0 makes every call a no-op */
  int32_t capacity;     /* 1 .. GQA_MAX_CAPACITY (kv.shape[-2]) */
  int32_t num_q_heads;  /* 32 or 16 (GQA_NUM_Q_HEADS_2TO1) */
  int32_t num_kv_heads; /* must be 8 */
  int32_t head_dim;     /* must be 128 */
  int32_t q_dtype;      /* gqa_dtype_t */
  int32_t kv_dtype;     /* gqa_dtype_t */
  float k_scale;        /* multiplies every score (fp8 / int8 cache) */
  float v_scale;        /* multiplies the normalised output (fp8 / int8 cache) */
  int32_t flags;        /* GQA_FLAG_* bits; 0 for the defaults */
} gqa_desc_t;

/* Split plans merge their chunks with a log-sum-exp combine kernel launched
 * right after the attention kernel on the same stream, or, in one launch,
 * inside the attention kernel: the last workgroup to finish a (request, KV
 * head) merges it (a per-head counter in the workspace, reset by that
 * workgroup, tells it that it is last; the partials travel through
 * device-coherent stores and loads, with no cache-wide fence). The automatic
 * plan takes the one-launch merge for small problems (a chunked split of at
 * most 16 chunks per head and 384 workgroups over a contiguous cache), where
 * it saves the second launch; on large grids the workgroups' waits on their
 * counters cost more than that launch. This flag asks for the one-launch
 * merge on any chunked plan (and keeps the plan off the balanced split). */
#define GQA_FLAG_FUSED_COMBINE 1

/* Launch plan chosen for a descriptor (host arithmetic only).
 * route 0 (short, capacity <= 64) and single-chunk plans: one workgroup per
 * (request, KV head), output normalised in place, no workspace.
 * route 1 (chunked split: explicit num_splits >= 2, the fused-merge flag, or
 * an automatic plan for a problem too small for the balanced split, whose
 * chunks then hold about an eighth of the capacity, 64 to 256 slots):
 * num_splits chunks of chunk_tokens slots per (request, KV head) -> FP32
 * partials -> log-sum-exp combine, as the article's split routes.
 * route 2 (balanced split, the automatic choice above capacity 64 for up to
 * 4096 requests when the cache holds at least 768 slabs of 64 slots across
 * all (request, KV head) pairs; smaller problems use the chunked split): a
 * persistent grid of num_workgroups workgroups (all resident at once)
 * shares the step's 64-slot slabs out in proportion to how fast the
 * hardware serves each workgroup (computed on the device from the lengths);
 * heads a workgroup covers whole are written directly, the rest are merged
 * by the combine kernel. num_splits is 0 (varies per head), chunk_tokens 64. */
typedef struct gqa_plan {
  int32_t route;
  int32_t num_splits;      /* chunks per (request, KV head); 1 = no combine; 0 = balanced */
  int32_t chunk_tokens;    /* tokens per chunk (multiple of GQA_CHUNK_GRANULE) or slab (64) */
  int32_t num_workgroups;  /* workgroups of the attention kernel */
  uint64_t workspace_bytes;/* FP32 partials (+ counters / slab prefix); 0 when no merge */
  int32_t fused_merge;     /* 1: one launch, the last workgroup of each head merges it
                              (GQA_FLAG_FUSED_COMBINE, or a small automatic split) */
} gqa_plan_t;

typedef struct gqa_prepared gqa_prepared_t;

/* Convenience call: validate, plan (num_splits chosen automatically) and
 * enqueue the whole decode step on `stream`, asynchronously. Split partials
 * live in a library-owned workspace cached per (device, stream) that only
 * grows; growing it allocates, so a call made while `stream` is capturing
 * that would need to grow it returns GQA_ERR_CAPTURE instead. Calls on the
 * same stream are ordered and may share the cache. Calls from several host
 * threads are safe: the cache lookup, any growth (which synchronises the
 * stream before freeing the old buffer) and the enqueue happen under one
 * lock, so no call launches with a buffer another call has freed. Entries
 * live until the process ends and are keyed by the stream handle: a stream
 * created later with the same handle value reuses the entry, so synchronise a
 * stream before destroying it. The prepared pair below is the capture-safe
 * interface. */
GQA_API gqa_status_t gqa_decode(const gqa_desc_t* desc, const void* q, const void* kv,
                                const int32_t* seq_lens, float q_scale, void* out,
                                hipStream_t stream);

/* Prepare phase (run outside any capture): validates the descriptor and the
 * buffers (non-null, 16-byte aligned, out not overlapping q/kv/seq_lens by
 * address range), requires q_scale finite and > 0, picks the route, and
 * allocates the FP32 split workspace once with hipMalloc on the current
 * device. num_splits: 0 = automatic (the balanced split, sized for the current
 * device); 1 = one chunk per (request, KV head)
 * with the output normalised in place; n >= 2 = exactly n chunks — a value
 * the chunking cannot honour exactly (ceil(capacity / chunk) != n with chunk
 * a multiple of 16) is rejected with GQA_ERR_INVALID_ARG, never replaced.
 * On success *handle owns the workspace; release it with
 * gqa_prepared_destroy. */
GQA_API gqa_status_t prepare_gqa_decode(const gqa_desc_t* desc, const void* q,
                                        const void* kv, const int32_t* seq_lens,
                                        float q_scale, void* out, int32_t num_splits,
                                        gqa_prepared_t** handle);

/* Enqueue a prepared decode step on `stream`: no allocation, no host read of
 * device memory, no synchronisation — hipGraph-capturable. Buffer contents
 * (q, kv, seq_lens within [1, capacity]) may change between launches. The
 * workspace is mutable: a handle must not run on two unordered streams (or
 * graphs) at once; streams ordered by events may share it. Partials of an
 * earlier launch are never read: the combine derives the number of valid
 * chunks from the current lengths. */
GQA_API gqa_status_t launch_gqa_decode_prepared(gqa_prepared_t* handle, hipStream_t stream);

/* launch_gqa_decode_prepared with instrumentation: records `ev_start` on
 * `stream` before the attention kernel, `ev_mid` right after it and `ev_end`
 * after the combine kernel (immediately after `ev_mid` when there is no
 * combine). The events must have been created by the caller on the handle's
 * device; any of them may be NULL to skip it. For timing tools. */
GQA_API gqa_status_t launch_gqa_decode_prepared_timed(gqa_prepared_t* handle, hipStream_t stream,
                                                      hipEvent_t ev_start, hipEvent_t ev_mid,
                                                      hipEvent_t ev_end);

/* INT8 cache with per-row scales (Qwen3-VL on Jetson Orin doc, "INT8 KV
 * cache"): as gqa_decode / prepare_gqa_decode, for desc->kv_dtype ==
 * GQA_INT8_ROWSCALE only, with the bf16 row scales kv_scales [batch, 2, 8,
 * capacity] (16-byte aligned, caller-owned like kv; slots at or beyond a
 * request's length are never read). Token j's K scale multiplies its score,
 * its V scale its softmax weight in the output sum. The plain entry points
 * reject an INT8 descriptor (they have no scales argument); these reject any
 * other kv dtype. out must not overlap kv_scales either. The handle runs with
 * launch_gqa_decode_prepared like any other. */
GQA_API gqa_status_t gqa_decode_int8(const gqa_desc_t* desc, const void* q, const void* kv,
                                     const void* kv_scales, const int32_t* seq_lens,
                                     float q_scale, void* out, hipStream_t stream);
GQA_API gqa_status_t prepare_gqa_decode_int8(const gqa_desc_t* desc, const void* q,
                                             const void* kv, const void* kv_scales,
                                             const int32_t* seq_lens, float q_scale, void* out,
                                             int32_t num_splits, gqa_prepared_t** handle);

/* ---- Allocation-free decode -------------------------------------------------
 * For callers that cannot allocate device memory at all: code under hipGraph
 * capture, tight serving loops, harnesses that forbid hipMalloc. As
 * gqa_decode (kv_scales NULL) or gqa_decode_int8 (kv_dtype INT8_ROWSCALE,
 * kv_scales given): the same validation, plan, kernels and results, but the
 * split workspace is a static device array of GQA_NO_ALLOC_SCRATCH_BYTES
 * inside the library (one per GPU, held until the process ends) instead of
 * an allocated buffer, so the call never allocates or frees anything. A plan
 * whose workspace exceeds that size (very large batches on the chunked
 * route) is rejected with GQA_ERR_INVALID_ARG, as is any flag. The caller
 * still passes every input and out. All calls on one GPU share the one
 * array: calls that can overlap on the device (different streams, or several
 * host threads) race on it and must be ordered by the caller; calls on one
 * stream are ordered. The first call on a device looks up the array's device
 * address (hipGetSymbolAddress) and keeps it. */
#define GQA_NO_ALLOC_SCRATCH_BYTES ((size_t)4 << 20)
GQA_API gqa_status_t gqa_decode_no_alloc(const gqa_desc_t* desc, const void* q, const void* kv,
                                         const void* kv_scales, const int32_t* seq_lens,
                                         float q_scale, void* out, hipStream_t stream);

/* ---- Paged cache, several query tokens per request -------------------------
 * The decode step over a page pool, for one or more query tokens per request
 * (the verify pass of speculative decoding). The pages name a paged-KV decode
 * backend (FreeToken Turing notes, change 2) and a draft-and-verify loop of K
 * draft tokens per step (Thor vLLM notes, MTP) without fixing a layout; the
 * one below is this library's reading.
 *
 * Layouts (device memory):
 *   q           [batch, q_tokens, Hq, 128]       q_dtype, 16-byte aligned
 *   kv_pages    [num_pages, 2, 8, page_size, 128] kv_dtype (plane 0 = K), 16-byte aligned
 *   kv_scales   [num_pages, 2, 8, page_size]     bf16, INT8_ROWSCALE only (else NULL);
 *               with GQA_PAGED_SCALES_BY_POSITION instead
 *               [batch, 2, 8, max_pages * page_size]: the scale of request b's
 *               slot j at [b, plane, g, j], whatever page holds the row
 *   block_table [batch, max_pages] int32: request b's slot j is row j % page_size of
 *               page block_table[b][j / page_size]; read on the device only
 *   seq_lens    [batch] int32, device only: L_b counts the q_tokens new slots
 *   out         [batch, q_tokens, Hq, 128]       q_dtype
 * Query token t of request b is at slot L_b - q_tokens + t and attends slots
 * j < L_b - q_tokens + 1 + t (causal among the new tokens; q_tokens = 1 is
 * the plain decode step). Lengths are clamped to [0, max_pages * page_size];
 * a token whose limit leaves no slot (L_b < q_tokens) gets zeros. Block-table
 * entries for slots below L_b must name pages of the pool; the kernels clamp
 * entries into [0, num_pages), so a bad entry yields a wrong result, never an
 * access outside the pool. Entries past a request's last page are never read.
 * A contiguous cache [batch, 2, 8, C, 128] with C a power of two >= 16 is the
 * pool with page_size = C and block_table[b] = {b}. */
#define GQA_MAX_PAGE_SIZE (1 << 16)
/* q_tokens x (query heads per KV head) may not exceed this (one MFMA tile). */
#define GQA_PAGED_MAX_ROWS 16
/* gqa_paged_desc_t.flags bit, INT8_ROWSCALE pools only: the row scales are
 * indexed by position ([batch, 2, 8, max_pages * page_size], the contiguous
 * INT8 cache's scale layout) instead of living beside their rows in the pool.
 * The Orin Qwen3-VL doc ("INT8 KV cache") keeps one bf16 scale per (position,
 * KV head) row without fixing where it is stored. With pages of 16 or 32
 * slots, a head's scales for one page fill only 32 or 64 bytes of a 128-byte
 * line in the pool layout, and the kernels fetch the whole line; indexed by
 * position, each line holds 64 consecutive scales of one head. The decode
 * and append entry points must be given the same layout. */
#define GQA_PAGED_SCALES_BY_POSITION 2

typedef struct gqa_paged_desc {
  int32_t batch;        /* >= 0; 0 makes every call a no-op */
  int32_t q_tokens;     /* >= 1; q_tokens * num_q_heads / 8 <= GQA_PAGED_MAX_ROWS */
  int32_t num_q_heads;  /* 32 or 16 */
  int32_t num_kv_heads; /* must be 8 */
  int32_t head_dim;     /* must be 128 */
  int32_t q_dtype;      /* gqa_dtype_t, as for gqa_desc_t */
  int32_t kv_dtype;     /* gqa_dtype_t, as for gqa_desc_t */
  float k_scale;        /* as for gqa_desc_t */
  float v_scale;
  int32_t flags;        /* 0, or GQA_PAGED_SCALES_BY_POSITION for an INT8_ROWSCALE pool
                           (the one-launch merge is not offered here) */
  int32_t page_size;    /* slots per page: a power of two in [16, GQA_MAX_PAGE_SIZE] */
  int32_t num_pages;    /* pages in the pool, >= 1 */
  int32_t max_pages;    /* block_table row length, >= 1; max_pages * page_size <= GQA_MAX_CAPACITY */
} gqa_paged_desc_t;

/* As gqa_decode / prepare_gqa_decode / gqa_validate_args / gqa_plan_decode
 * (same routes, num_splits rules, workspace ownership, capture rules and
 * status codes), over a page pool. The prepared handle runs with
 * launch_gqa_decode_prepared. out must not overlap q, kv_pages, kv_scales,
 * block_table or seq_lens (GQA_ERR_ALIAS). */
GQA_API gqa_status_t gqa_decode_paged(const gqa_paged_desc_t* desc, const void* q,
                                      const void* kv_pages, const void* kv_scales,
                                      const int32_t* block_table, const int32_t* seq_lens,
                                      float q_scale, void* out, hipStream_t stream);
GQA_API gqa_status_t prepare_gqa_decode_paged(const gqa_paged_desc_t* desc, const void* q,
                                              const void* kv_pages, const void* kv_scales,
                                              const int32_t* block_table, const int32_t* seq_lens,
                                              float q_scale, void* out, int32_t num_splits,
                                              gqa_prepared_t** handle);
GQA_API gqa_status_t gqa_validate_args_paged(const gqa_paged_desc_t* desc, const void* q,
                                             const void* kv_pages, const void* kv_scales,
                                             const int32_t* block_table, const int32_t* seq_lens,
                                             float q_scale, const void* out, int32_t num_splits);
GQA_API gqa_status_t gqa_plan_decode_paged(const gqa_paged_desc_t* desc, int32_t num_splits,
                                           gqa_plan_t* plan);

/* Free the workspace and the handle (after its work has retired). NULL is a no-op. */
GQA_API void gqa_prepared_destroy(gqa_prepared_t* handle);

/* Workspace bytes owned by the handle (0 for NULL or single-chunk plans). */
GQA_API size_t gqa_prepared_workspace_bytes(const gqa_prepared_t* handle);

/* Copy of the handle's launch plan; GQA_ERR_INVALID_ARG for NULL arguments. */
GQA_API gqa_status_t gqa_prepared_plan(const gqa_prepared_t* handle, gqa_plan_t* plan);

/* Append one token per request to the cache: writes the K row k_new[b, g, :]
 * and the V row v_new[b, g, :] of every KV head g at slot positions[b] of
 * request b (the cache write that precedes each decode step; Thor Qwen3-VL
 * doc, "Runtime architecture", RoPE and KV writes). Layouts: k_new, v_new
 * [batch, 8, 128] in desc->q_dtype (F16 or BF16), 16-byte aligned; positions
 * int32 [batch], read on the device only, 4-byte aligned; kv as for
 * gqa_decode, written in place. A 16-bit cache (kv dtype == q dtype) stores
 * the values as they are. An FP8_E4M3 cache stores e4m3(x / k_scale) for K
 * and e4m3(x / v_scale) for V (Thor FP8-KV notes, section 1): IEEE fp32
 * division, nearest E4M3FN code with ties to even, magnitudes >= 448
 * saturating to +-448, NaN stored as 0x7F. Positions outside [0, capacity)
 * write nothing. kv must not overlap k_new, v_new or positions
 * (GQA_ERR_ALIAS). Asynchronous on `stream`; allocates nothing. An INT8
 * cache is rejected (GQA_ERR_INVALID_ARG); gqa_kv_append_int8 writes one. */
GQA_API gqa_status_t gqa_kv_append(const gqa_desc_t* desc, const void* k_new, const void* v_new,
                                   const int32_t* positions, void* kv, hipStream_t stream);

/* As gqa_kv_append, for an INT8_ROWSCALE cache: writes each new K and V row
 * of 128 values as int8 codes into kv and its bf16 row scale into kv_scales
 * [batch, 2, 8, capacity] (2-byte aligned; the layout gqa_decode_int8 reads).
 * The Orin Qwen3-VL doc ("INT8 KV cache") keeps INT8 mirrors with one BF16
 * scale per (position, KV head) row without saying how a row is quantised;
 * this follows that doc's symmetric INT8 weight rule (scale = amax / 127,
 * "Weight quantization" table) per row: y = x / k_scale (V: v_scale),
 * s = max|y| / 127 rounded to bf16 (nearest, ties to even), code = y / s
 * rounded to the nearest integer (ties to even) and clamped to +-127; a row
 * whose s is 0 stores code 0. Every division is an IEEE fp32 division, so the
 * decode's code * s * k_scale gives back x to within half a step. Rows with a
 * non-finite value store unspecified codes and scale. kv_scales must not
 * overlap kv, k_new, v_new or positions (GQA_ERR_ALIAS); a non-INT8
 * descriptor is rejected (GQA_ERR_INVALID_ARG). Asynchronous on `stream`;
 * allocates nothing. */
GQA_API gqa_status_t gqa_kv_append_int8(const gqa_desc_t* desc, const void* k_new,
                                        const void* v_new, const int32_t* positions, void* kv,
                                        void* kv_scales, hipStream_t stream);

/* Append desc->q_tokens new tokens per request to a page pool: token t of
 * request b lands at slot s = positions[b] + t, i.e. row s % page_size of
 * page block_table[b][s / page_size], with the K row k_new[b, t, g, :] and
 * the V row v_new[b, t, g, :] of every KV head g. It is the cache write
 * before a step over a paged cache (FreeToken Turing notes, change 2, name a
 * paged-KV decode backend; Thor Qwen3-VL doc, "Runtime architecture", for
 * the write), several tokens at once for a verify pass over draft tokens
 * (Thor vLLM notes on MTP); with positions[b] = L_b - q_tokens the tokens
 * are the ones gqa_decode_paged then attends with the same descriptor.
 * Layouts: k_new, v_new [batch, q_tokens, 8, 128] in desc->q_dtype (F16 or
 * BF16), 16-byte aligned; positions int32 [batch] and block_table
 * [batch, max_pages] int32, both read on the device only, 4-byte aligned;
 * kv_pages as for gqa_decode_paged, written in place. Encoding as for
 * gqa_kv_append (16-bit: stored as is; FP8_E4M3: e4m3 of x / k_scale or
 * x / v_scale, saturating). Slots outside [0, max_pages * page_size) and
 * block-table entries outside [0, num_pages) write nothing. Two new tokens
 * must not land on the same page row (which one is stored is then
 * unspecified). kv_pages must not overlap k_new, v_new, positions or
 * block_table (GQA_ERR_ALIAS). Asynchronous on `stream`; allocates nothing.
 * An INT8 pool is rejected (GQA_ERR_INVALID_ARG); gqa_kv_append_paged_int8
 * writes one. */
GQA_API gqa_status_t gqa_kv_append_paged(const gqa_paged_desc_t* desc, const void* k_new,
                                         const void* v_new, const int32_t* positions,
                                         const int32_t* block_table, void* kv_pages,
                                         hipStream_t stream);

/* As gqa_kv_append_paged, for an INT8_ROWSCALE pool: each row is quantised
 * as in gqa_kv_append_int8 and its bf16 scale goes to row `s % page_size` of
 * page block_table[b][s / page_size] in kv_scales [num_pages, 2, 8,
 * page_size] (2-byte aligned; the layout gqa_decode_paged reads), or, with
 * GQA_PAGED_SCALES_BY_POSITION, to [b, plane, g, s] of kv_scales [batch, 2,
 * 8, max_pages * page_size]. A token whose slot or page entry is skipped
 * writes no scale either. kv_scales must not overlap kv_pages, k_new, v_new,
 * positions or block_table (GQA_ERR_ALIAS); a non-INT8 descriptor is
 * rejected (GQA_ERR_INVALID_ARG). */
GQA_API gqa_status_t gqa_kv_append_paged_int8(const gqa_paged_desc_t* desc, const void* k_new,
                                              const void* v_new, const int32_t* positions,
                                              const int32_t* block_table, void* kv_pages,
                                              void* kv_scales, hipStream_t stream);

/* Host-only validation of a call's arguments (never touches a device, so it
 * runs without a GPU). Same checks and status codes as prepare_gqa_decode,
 * except the device check; the _int8 form as prepare_gqa_decode_int8. */
GQA_API gqa_status_t gqa_validate_args(const gqa_desc_t* desc, const void* q, const void* kv,
                                       const int32_t* seq_lens, float q_scale,
                                       const void* out, int32_t num_splits);
GQA_API gqa_status_t gqa_validate_args_int8(const gqa_desc_t* desc, const void* q, const void* kv,
                                            const void* kv_scales, const int32_t* seq_lens,
                                            float q_scale, const void* out, int32_t num_splits);

/* Host-only planning: the route, chunking and workspace a call would use
 * (num_splits as for prepare_gqa_decode). Runs without a GPU, so a balanced
 * plan assumes a nominal 768 workgroups (256 CUs x 3); prepare sizes the grid
 * for the device and the cache type (on MI355X 512 workgroups for 16-bit and
 * fp8 caches, up to 768 for INT8) and reports it in its plan. With a 16-bit or
 * INT8 cache, a single request or a cache of at most 256 MiB of K+V at
 * capacity takes one workgroup per CU instead (256 here and on MI355X). */
GQA_API gqa_status_t gqa_plan_decode(const gqa_desc_t* desc, int32_t num_splits,
                                     gqa_plan_t* plan);

/* Thread-local description of the last error on this thread ("" if none). */
GQA_API const char* gqa_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* GQA_DECODE_H_ */
