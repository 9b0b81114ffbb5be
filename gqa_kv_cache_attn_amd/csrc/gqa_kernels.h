// Internal interface between the C-ABI layer (gqa_api.hip) and the gfx950
// kernels (gqa_kernels.hip). Not installed; callers use include/gqa_decode.h.
#pragma once

#include <stdint.h>

#include <hip/hip_runtime_api.h>

namespace gqa {

enum DType : int { kF16 = 0, kBF16 = 1, kFP8 = 2, kI8 = 3 };

// The balanced split keeps the per-request slab prefix in LDS.
constexpr int kMaxBalancedBatch = 4096;
// Tiers of workgroup shares in the balanced split (StepArgs::share).
constexpr int kShareTiers = 4;

// Arguments of one decode step, passed to the kernels by value.
struct StepArgs {
  const void* q;             // [batch, Hq, 128] q dtype
  const void* kv;            // [batch, 2, 8, capacity, 128] kv dtype
  const void* kv_scales;     // [batch, 2, 8, capacity] bf16 row scales (INT8 cache), else null
  const int32_t* seq_lens;   // [batch]
  void* out;                 // [batch, Hq, 128] q dtype
  float* part_o;             // [batch, Hq, num_splits, 128] unnormalised chunk outputs
  float* part_ml;            // [batch, Hq, num_splits, 2] chunk (max, sum), log2 domain
  uint32_t* counters;        // [batch, 8] finished chunks per (request, KV head); 0 between launches
  int32_t* slab_prefix;      // [batch + 1] balanced split: 8 * slabs before each request
  int32_t* head_pieces;      // [2, batch * 8] balanced split, per (request, KV head): the slot
                             // of its first piece (-1: written whole), then the workgroup
                             // holding its last piece
  int32_t batch;
  int32_t num_q_heads;       // Hq: 32 (4 per KV head) or 16 (2 per KV head)
  int32_t capacity;
  int32_t num_splits;        // chunks per (request, KV head); 1 = normalise in place
  int32_t chunk_tokens;      // multiple of 16
  float scale_log2;          // q_scale * k_scale * log2(e) / sqrt(128)
  float v_scale;
  int32_t fused_combine;     // 1: last workgroup of a head combines; 0: separate combine kernel
  int32_t grid_wgs;          // > 0: balanced split with this many persistent workgroups
  // Balanced split shares: workgroup w takes a share of the slabs proportional
  // to share[2 * min(w / tier_size, kShareTiers - 1) + (w & 1)].
  int32_t tier_size;         // workgroups per tier (the device's CU count)
  int32_t share[2 * 4];
  // Paged cache (gqa_paged.hip only; kv then is the page pool
  // [num_pages, 2, 8, page_size, 128] and kv_scales [num_pages, 2, 8, page_size]).
  const int32_t* block_table;  // [batch, max_pages]: page of each request's page-sized run of slots
  int32_t max_pages;
  int32_t page_shift;        // log2(page_size)
  int32_t num_pages;
  int32_t q_tokens;          // T query tokens per request (q, out: [batch, T, Hq, 128]); 1 otherwise
  int32_t scales_by_position;  // INT8 pool: kv_scales is [batch, 2, 8, capacity], indexed by
                               // the request's slot instead of the page row
};

// Arguments of one KV append (one new token per request).
struct AppendArgs {
  const void* k_new;         // [batch, tokens, 8, 128] 16-bit
  const void* v_new;         // [batch, tokens, 8, 128] 16-bit
  const int32_t* positions;  // [batch] slot of the first new token; slots outside
                             // [0, capacity) are skipped
  void* kv;                  // contiguous [batch, 2, 8, capacity, 128] or page pool
                             // [num_pages, 2, 8, 1 << page_shift, 128], kv dtype
  int32_t batch;
  int32_t tokens = 1;        // new tokens per request
  int32_t capacity;          // slots a request can address (paged: max_pages << page_shift)
  float k_scale;             // fp8 cache: stored code = e4m3(k / k_scale); INT8: rows of k / k_scale
  float v_scale;
  void* kv_scales = nullptr; // INT8 cache: bf16 row scales, [batch, 2, 8, capacity] or
                             // [num_pages, 2, 8, 1 << page_shift]
  // Page pool (block_table != nullptr): slot j of request b is row j % page
  // size of page block_table[b * max_pages + j / page size]; entries outside
  // [0, num_pages) are skipped.
  const int32_t* block_table = nullptr;
  int32_t max_pages = 0;
  int32_t page_shift = 0;
  int32_t num_pages = 0;
  // INT8 pool: the row scales are [batch, 2, 8, capacity], indexed by slot.
  int32_t scales_by_position = 0;
};

hipError_t enqueue_kv_append(const AppendArgs& args, int src_dtype, int kv_dtype, hipStream_t stream);

// Device address, on device `dev` (which must be current), of the static
// scratch array gqa_decode_no_alloc uses as its split workspace
// (GQA_NO_ALLOC_SCRATCH_BYTES, 256-byte aligned). Looked up once per device.
hipError_t no_alloc_scratch(int dev, void** ptr);

// Workgroups of the balanced split that the current device keeps resident at
// once (CUs x resident workgroups per CU); 0 if the query fails.
int balanced_grid_size(int q_dtype, int kv_dtype, int num_q_heads);

// Enqueue the attention kernel (and, for num_splits > 1, the combine kernel).
// Returns the first launch error. Arguments are assumed validated. When given,
// `ev_mid` is recorded between the two kernels (or after the only one).
hipError_t enqueue_decode_step(const StepArgs& args, int q_dtype, int kv_dtype,
                               hipStream_t stream, hipEvent_t ev_mid = nullptr);

// Paged cache, T query tokens per request (gqa_paged.hip). The balanced split
// keeps 16 partial rows per slot (kPagedSlotRows).
constexpr int kPagedSlotRows = 16;
int paged_balanced_grid_size(int q_dtype, int kv_dtype, int num_q_heads);
hipError_t enqueue_paged_decode_step(const StepArgs& args, int q_dtype, int kv_dtype,
                                     hipStream_t stream, hipEvent_t ev_mid = nullptr);

}  // namespace gqa
