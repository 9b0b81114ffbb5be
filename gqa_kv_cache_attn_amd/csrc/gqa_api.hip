// C-ABI layer of libgqa_decode.so: argument validation, launch planning, the
// prepared handle with its split workspace, and the convenience call.
//
// The entry points mirror the FlashInfer sm110_gqa_decode article's API
// (convenience call; prepare + launch-prepared pair; "three differences":
// caller-owned non-aliasing output, finite positive q_scale, a launch that
// allocates nothing and reads nothing on the host; num_splits never replaced
// silently) in plain C: pointers, sizes, a status code.
//
// Host code here never reads device memory; lengths stay on the device.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <map>
#include <mutex>
#include <new>
#include <string>
#include <utility>

#include "../../include/gqa_decode.h"
#include "gqa_kernels.h"

namespace {

thread_local std::string g_last_error;

gqa_status_t fail(gqa_status_t st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

gqa_status_t ok() {
  g_last_error.clear();
  return GQA_OK;
}

// Paged cache and query tokens (zero-initialised: the contiguous cache with
// one query token per request).
struct Paging {
  bool on = false;
  int32_t q_tokens = 1;
  int32_t page_shift = 0;
  int32_t num_pages = 0;
  int32_t max_pages = 0;
  const int32_t* block_table = nullptr;
  bool scales_by_position = false;   // INT8 pool: row scales [batch, 2, 8, capacity]
};

// Automatic split planning (measured on MI355X: ~1 MiB of K+V per chunk was
// best for 16-bit and fp8 caches alike; 768 = 256 CUs x 3 resident workgroups).
constexpr int64_t kChunkBytes = 1 << 20;
constexpr int64_t kFillWorkgroups = 768;
// Balanced split: host-only plans assume a nominal 256 CUs x 3 workgroups;
// prepare and the convenience call size the grid for the device and cache
// type (balanced_wgs_per_cu: 2 per CU for 16-bit and fp8, 3 for INT8 on
// MI355X), capped at kMaxBalancedGrid.
constexpr int kNominalBalancedGrid = 768;
constexpr int kMaxBalancedGrid = 4096;
// Small problems with a 16-bit or INT8 cache take one balanced workgroup per
// CU instead: a single request, or at most kSmallBalancedBytes of K+V at
// capacity (an upper bound of the step's bytes, the only size the host knows).
// Measured on MI355X, contiguous and paged: a single request ran 4-41% faster
// that way, caches of up to 256 MiB 3-26% faster; batches of larger ragged
// caches ran 2-7% slower (coarser pieces balance worse). fp8 caches keep the
// resident grid: their tiles carry half the bytes, and one workgroup per CU
// ran 2-6% slower on single requests of 128k-256k slots.
constexpr int64_t kSmallBalancedBytes = int64_t(256) << 20;
// Automatic chunked plans that merge inside the attention kernel: at most
// this many chunks per head and workgroups per launch.
constexpr int64_t kOneLaunchMaxSplits = 16;
constexpr int64_t kOneLaunchMaxWorkgroups = 384;
constexpr int kNominalCUs = 256;
// A dispatch counts its work-items in 32 bits: at most this many 256-thread
// workgroups per launch (decode and append kernels alike).
constexpr int64_t kMaxLaunchWorkgroups = (int64_t)UINT32_MAX / 256;


// Resident balanced-kernel workgroups per (device, dtype pair, query heads),
// queried once.
std::mutex g_grid_mu;
std::map<std::pair<int, int>, int> g_grid;

int device_balanced_grid(int dev, const gqa_desc_t* d, bool paged) {
  std::lock_guard<std::mutex> lk(g_grid_mu);
  const std::pair<int, int> key{dev, ((d->num_q_heads * 8 + d->q_dtype) * 8 + d->kv_dtype) * 2 + paged};
  auto it = g_grid.find(key);
  if (it != g_grid.end()) return it->second;
  const int W = paged ? gqa::paged_balanced_grid_size(d->q_dtype, d->kv_dtype, d->num_q_heads)
                      : gqa::balanced_grid_size(d->q_dtype, d->kv_dtype, d->num_q_heads);
  g_grid.emplace(key, W);
  return W;
}

// Compute units of a device (the size of one tier of balanced-split shares), queried once.
std::map<int, int> g_cus;

int device_cus(int dev) {
  std::lock_guard<std::mutex> lk(g_grid_mu);
  auto it = g_cus.find(dev);
  if (it != g_cus.end()) return it->second;
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) {
    (void)hipGetLastError();
    cus = 0;
  }
  g_cus.emplace(dev, cus);
  return cus;
}

// Relative shares (per mille) of the balanced split's workgroups by tier (the
// k-th workgroup resident on a CU: workgroups tier * CUs .. (tier + 1) * CUs - 1)
// and by parity (odd workgroups run on odd-numbered XCDs). Measured on MI355X
// with equal shares (per-workgroup timestamps, 64k bf16 and 128k fp8
// workloads): the second and third workgroup of each CU took 1.1-1.2x and
// 1.25-1.45x as long as the first, whatever slabs they read; the tier shares
// (a sweep of five sets) lift the long-context kernels by 1-3 points of HBM
// peak. With two workgroups per CU the second is barely slower: a sweep of
// its share (780-960) was fastest at 960 on both workloads (0.4-0.7% over
// 840). Build-time knobs; shares only move range boundaries, never the
// result's correctness.
#ifndef GQA_SHARE_TIER1
#define GQA_SHARE_TIER1 840
#endif
#ifndef GQA_SHARE_TIER1_OF_TWO
#define GQA_SHARE_TIER1_OF_TWO 960   // second workgroup when two share each CU
#endif
#ifndef GQA_SHARE_TIER2
#define GQA_SHARE_TIER2 670
#endif
#ifndef GQA_SHARE_TIER3
#define GQA_SHARE_TIER3 670
#endif
// Odd-XCD share with two or three workgroups per CU, contiguous and paged.
// Interleaved A/B runs on five boxes (three alternating samples per variant
// and box) improved every long workload monotonically from 920 up to
// 1000-1060: 128k fp8 -2.1%, 128k INT8 -2.5%, 64k bf16 -1.9%, the ragged
// batch -2.3%, the fp8 / INT8 / bf16 page pools -2.9 / -2.6 / -1.6% at 1060;
// 1100 was about as fast and 1150-1300 slower again.
#ifndef GQA_SHARE_ODD
#define GQA_SHARE_ODD 1060
#endif
// With one workgroup per CU (single requests and small 16-bit or INT8
// caches; fp8 keeps two per CU) a bf16 request of 100k slots ran 1.7-1.8%
// faster at 1000 than at 920 on two boxes, while INT8 ran 0.6-0.9% slower,
// so 16-bit grids take 1000 there and INT8 grids keep 920.
#ifndef GQA_SHARE_ODD_ONE_PER_CU
#define GQA_SHARE_ODD_ONE_PER_CU 1000
#endif
#ifndef GQA_SHARE_ODD_ONE_PER_CU_INT8
#define GQA_SHARE_ODD_ONE_PER_CU_INT8 920
#endif

// a.grid_wgs must be set: the shares depend on how many workgroups share a CU.
void set_shares(gqa::StepArgs& a, int tier_size, int kv_dtype) {
  int tier[gqa::kShareTiers] = {1000, GQA_SHARE_TIER1, GQA_SHARE_TIER2, GQA_SHARE_TIER3};
  const bool two = tier_size > 0 && a.grid_wgs == 2 * tier_size;
  if (two) tier[1] = GQA_SHARE_TIER1_OF_TWO;
  const int odd = tier_size > 0 && a.grid_wgs > tier_size ? GQA_SHARE_ODD
                  : kv_dtype == GQA_INT8_ROWSCALE       ? GQA_SHARE_ODD_ONE_PER_CU_INT8
                                                        : GQA_SHARE_ODD_ONE_PER_CU;
  // tier_size 0 (unknown) or a grid of one tier: plain equal shares
  a.tier_size = tier_size > 0 ? tier_size : (1 << 28);
  for (int t = 0; t < gqa::kShareTiers; ++t) {
    a.share[2 * t] = tier[t];
    a.share[2 * t + 1] = tier[t] * odd / 1000;
  }
}

int elem_bytes(int dt) { return (dt == GQA_FP8_E4M3 || dt == GQA_INT8_ROWSCALE) ? 1 : 2; }

// K+V bytes one cache slot of one KV head occupies (row scales included).
int64_t slot_bytes(int dt) {
  return 2 * (GQA_HEAD_DIM * (int64_t)elem_bytes(dt) + (dt == GQA_INT8_ROWSCALE ? 2 : 0));
}

bool ranges_overlap(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
  return na != 0 && nb != 0 && a0 < b0 + nb && b0 < a0 + na;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool scale_ok(float s) { return std::isfinite(s) && s > 0.0f; }

gqa_status_t check_desc(const gqa_desc_t* d) {
  if (d == nullptr) return fail(GQA_ERR_INVALID_ARG, "desc is NULL");
  if ((d->num_q_heads != GQA_NUM_Q_HEADS && d->num_q_heads != GQA_NUM_Q_HEADS_2TO1) ||
      d->num_kv_heads != GQA_NUM_KV_HEADS || d->head_dim != GQA_HEAD_DIM)
    return fail(GQA_ERR_INVALID_ARG,
                "geometry must be 32 or 16 query heads / 8 KV heads / head_dim 128 (got %d/%d/%d)",
                d->num_q_heads, d->num_kv_heads, d->head_dim);
  if (d->batch < 0) return fail(GQA_ERR_INVALID_ARG, "batch must be >= 0 (got %d)", d->batch);
  if (d->capacity < 1 || d->capacity > GQA_MAX_CAPACITY)
    return fail(GQA_ERR_INVALID_ARG, "capacity must be in [1, %d] (got %d)", GQA_MAX_CAPACITY,
                d->capacity);
  if (d->q_dtype != GQA_F16 && d->q_dtype != GQA_BF16)
    return fail(GQA_ERR_INVALID_ARG, "q dtype must be F16 or BF16 (got %d)", d->q_dtype);
  const bool kv_ok = d->kv_dtype == GQA_FP8_E4M3 || d->kv_dtype == GQA_INT8_ROWSCALE ||
                     d->kv_dtype == d->q_dtype;
  if (!kv_ok)
    return fail(GQA_ERR_INVALID_ARG,
                "unsupported (q, kv) dtype pair (%d, %d): kv must match q or be FP8_E4M3 or "
                "INT8_ROWSCALE",
                d->q_dtype, d->kv_dtype);
  if (!scale_ok(d->k_scale) || !scale_ok(d->v_scale))
    return fail(GQA_ERR_INVALID_ARG, "k_scale and v_scale must be finite and > 0");
  if (d->kv_dtype == d->q_dtype && (d->k_scale != 1.0f || d->v_scale != 1.0f))
    return fail(GQA_ERR_INVALID_ARG,
                "k_scale/v_scale apply to an fp8 or int8 cache only; a 16-bit cache needs 1.0");
  if ((d->flags & ~GQA_FLAG_FUSED_COMBINE) != 0)
    return fail(GQA_ERR_INVALID_ARG, "unknown flags 0x%x", (unsigned)d->flags);
  return GQA_OK;
}

// Workspace: control words | part_o [R,128] f32 | part_ml [R,2] f32 | slab
// prefix [B+1] and head pieces [2, B*8] int32 (balanced split only). The control words (the opt-in
// fused merge's per-(request, KV head) counters [B*8]) come first, at an
// offset no plan changes, and every launch leaves them at zero (the last
// workgroup of each head resets its counter). R is the number of partial
// rows: chunked split R = B*T*Hq*S (query-row-major; T = 1 for the contiguous
// cache), balanced split R = 2W*4 (two slots per workgroup, 4 query rows
// each; 16 for the paged cache).
struct WorkspaceLayout {
  uint64_t ctrl_bytes, o_offset, ml_offset, aux_offset, total;
};

WorkspaceLayout workspace_layout(uint64_t ctrl_bytes, uint64_t rows, uint64_t aux_ints) {
  WorkspaceLayout w;
  w.ctrl_bytes = ctrl_bytes;
  w.o_offset = ctrl_bytes;
  w.ml_offset = w.o_offset + rows * GQA_HEAD_DIM * sizeof(float);
  w.aux_offset = w.ml_offset + rows * 2 * sizeof(float);
  w.total = w.aux_offset + ((aux_ints * sizeof(int32_t) + 255) & ~255ull);
  return w;
}

WorkspaceLayout plan_layout(const gqa_desc_t* d, const gqa_plan_t& p, const Paging& pg) {
  if (p.route == 2)   // aux: slab prefix [B+1] | head pieces [2, B*8]
    return workspace_layout(0, 2ull * (uint64_t)p.num_workgroups * (pg.on ? gqa::kPagedSlotRows : 4),
                            (uint64_t)d->batch + 1 + 2ull * (uint64_t)d->batch * GQA_NUM_KV_HEADS);
  const uint64_t ctrl =
      p.fused_merge ? (((uint64_t)d->batch * GQA_NUM_KV_HEADS * sizeof(uint32_t) + 255) & ~255ull)
                    : 0;
  return workspace_layout(ctrl,
                          (uint64_t)d->batch * (uint64_t)pg.q_tokens * (uint64_t)d->num_q_heads *
                              (uint64_t)p.num_splits,
                          0);
}

// grid_wgs: resident workgroups of the balanced kernel on the target device,
// cus: its compute units (0, 0: the nominal kNominalBalancedGrid and
// kNominalCUs, for host-only planning). one_launch_ok: an automatic chunked
// plan may merge in the attention kernel (contiguous cache with an allocated
// workspace; the paged kernels and the static no-alloc scratch have no
// zeroed per-head counters).
gqa_status_t make_plan(const gqa_desc_t* d, int32_t num_splits, gqa_plan_t* p, int grid_wgs = 0,
                       const Paging& pg = Paging(), int cus = 0, bool one_launch_ok = true) {
  const int64_t C = d->capacity;
  p->fused_merge = (d->flags & GQA_FLAG_FUSED_COMBINE) ? 1 : 0;
  if (num_splits < 0) return fail(GQA_ERR_INVALID_ARG, "num_splits must be >= 0 (got %d)", num_splits);
  const int64_t slabs_per_head = (C + 63) / 64;
  const int64_t slabs_at_capacity = (int64_t)d->batch * GQA_NUM_KV_HEADS * slabs_per_head;
  if (num_splits == 0 && C > GQA_SHORT_CAPACITY_MAX && !(d->flags & GQA_FLAG_FUSED_COMBINE) &&
      d->batch <= gqa::kMaxBalancedBatch && slabs_at_capacity <= INT32_MAX &&
      slabs_at_capacity >= kNominalBalancedGrid) {
    // Balanced split: a persistent grid shares the step's slabs evenly.
    const int resident = grid_wgs > 0 ? grid_wgs : kNominalBalancedGrid;
    const int64_t cap_bytes = (int64_t)d->batch * GQA_NUM_KV_HEADS * C * slot_bytes(d->kv_dtype);
    const bool small = d->kv_dtype != GQA_FP8_E4M3 &&
                       (d->batch == 1 || cap_bytes <= kSmallBalancedBytes);
    const int one_per_cu = cus > 0 ? cus : kNominalCUs;
    const int G = std::max(1, std::min(small ? std::min(resident, one_per_cu) : resident,
                                       kMaxBalancedGrid));
    p->route = 2;
    p->num_splits = 0;
    p->chunk_tokens = 64;
    p->num_workgroups = G;
    p->workspace_bytes = d->batch > 0 ? plan_layout(d, *p, pg).total : 0;
    return GQA_OK;
  }
  const int64_t granules = (C + GQA_CHUNK_GRANULE - 1) / GQA_CHUNK_GRANULE;
  int64_t chunk_granules;
  bool small_auto = false;
  if (num_splits == 0) {
    if (C <= GQA_SHORT_CAPACITY_MAX) {
      chunk_granules = granules;
    } else if (slabs_at_capacity < kNominalBalancedGrid) {
      // Small problems (too few 64-slot slabs for the balanced grid):
      // chunks of about an eighth of the capacity, in 64-slot steps, from 64
      // to 256 slots. Measured on MI355X over 1-5 requests and capacities of
      // 128-6000 slots: within 2-8% of the best chunk size at every shape,
      // where fixed 64-slot chunks were up to 1.7x slower beyond 2k slots.
      const int64_t per = (C + 7) / 8;
      const int64_t chunk = std::min<int64_t>(256, std::max<int64_t>(64, (per + 63) / 64 * 64));
      chunk_granules = chunk / GQA_CHUNK_GRANULE;
      small_auto = true;
    } else {
      // Automatic, in whole workgroup steps (64 tokens): chunks of about
      // kChunkBytes of K+V each (long enough to amortise a workgroup's
      // prologue and merge, short enough to balance), but small enough that
      // the grid still fills every CU once at full capacity.
      constexpr int64_t kStepGranules = 64 / GQA_CHUNK_GRANULE;
      const int64_t steps = (C + 63) / 64;
      const int64_t step_bytes = 64 * slot_bytes(d->kv_dtype);
      const int64_t by_bytes = std::max<int64_t>(1, kChunkBytes / step_bytes);
      const int64_t total = std::max<int64_t>(1, (int64_t)d->batch * GQA_NUM_KV_HEADS * steps);
      const int64_t by_fill = std::max<int64_t>(1, total / kFillWorkgroups);
      const int64_t chunk_steps = std::min(std::min(by_bytes, by_fill), steps);
      chunk_granules = chunk_steps * kStepGranules;
    }
  } else if (num_splits == 1) {
    chunk_granules = granules;
  } else {
    const int64_t per = (C + num_splits - 1) / num_splits;
    chunk_granules = (per + GQA_CHUNK_GRANULE - 1) / GQA_CHUNK_GRANULE;
    const int64_t chunk = chunk_granules * GQA_CHUNK_GRANULE;
    if ((C + chunk - 1) / chunk != num_splits)
      return fail(GQA_ERR_INVALID_ARG,
                  "num_splits=%d cannot be honoured for capacity %lld with %d-token chunks "
                  "(would give %lld); pass 0 for automatic",
                  num_splits, (long long)C, GQA_CHUNK_GRANULE, (long long)((C + chunk - 1) / chunk));
  }
  const int64_t chunk = chunk_granules * GQA_CHUNK_GRANULE;
  const int64_t S = (C + chunk - 1) / chunk;
  const int64_t wgs = (int64_t)d->batch * GQA_NUM_KV_HEADS * S;
  if (wgs > kMaxLaunchWorkgroups)
    return fail(GQA_ERR_INVALID_ARG, "problem too large for one launch (%lld workgroups)",
                (long long)wgs);
  p->route = C <= GQA_SHORT_CAPACITY_MAX ? 0 : 1;
  p->num_splits = (int32_t)S;
  p->chunk_tokens = (int32_t)chunk;
  p->num_workgroups = (int32_t)wgs;
  // A small automatic split merges in the attention kernel (one launch): its
  // last workgroup per head merges the head. Measured on MI355X, that beat
  // the second launch while a head has at most 16 chunks and the grid at
  // most 384 workgroups (single requests: 5-16% faster per step); beyond
  // that the grid's workgroups each waiting on their counter cost more.
  if (small_auto && one_launch_ok && !pg.on && S > 1 && S <= kOneLaunchMaxSplits &&
      wgs <= kOneLaunchMaxWorkgroups)
    p->fused_merge = 1;
  if (S <= 1) p->fused_merge = 0;
  p->workspace_bytes = S > 1 ? plan_layout(d, *p, pg).total : 0;
  return GQA_OK;
}

// with_scales: the _int8 entry points (kv dtype INT8_ROWSCALE, scales given);
// the plain ones reject an INT8 descriptor.
gqa_status_t check_args(const gqa_desc_t* d, const void* q, const void* kv, const void* scales,
                        bool with_scales, const int32_t* lens, float q_scale, const void* out) {
  gqa_status_t st = check_desc(d);
  if (st != GQA_OK) return st;
  if (with_scales && d->kv_dtype != GQA_INT8_ROWSCALE)
    return fail(GQA_ERR_INVALID_ARG, "the _int8 entry points need kv dtype INT8_ROWSCALE (got %d)",
                d->kv_dtype);
  if (!with_scales && d->kv_dtype == GQA_INT8_ROWSCALE)
    return fail(GQA_ERR_INVALID_ARG,
                "an INT8_ROWSCALE cache needs its row scales: use gqa_decode_int8 / "
                "prepare_gqa_decode_int8");
  if (!scale_ok(q_scale))
    return fail(GQA_ERR_INVALID_ARG, "q_scale must be finite and > 0 (got %g)", (double)q_scale);
  if (d->batch == 0) return GQA_OK;
  if (!q || !kv || !lens || !out || (with_scales && !scales))
    return fail(GQA_ERR_INVALID_ARG,
                with_scales ? "q, kv, kv_scales, seq_lens and out must be non-NULL"
                            : "q, kv, seq_lens and out must be non-NULL");
  if (!aligned(q, 16) || !aligned(kv, 16) || !aligned(out, 16) || !aligned(lens, 4) ||
      (with_scales && !aligned(scales, 16)))
    return fail(GQA_ERR_INVALID_ARG,
                "q, kv, kv_scales and out must be 16-byte aligned and seq_lens 4-byte aligned");
  const size_t B = (size_t)d->batch;
  const size_t q_bytes = B * (size_t)d->num_q_heads * GQA_HEAD_DIM * elem_bytes(d->q_dtype);
  const size_t kv_bytes =
      B * 2 * GQA_NUM_KV_HEADS * (size_t)d->capacity * GQA_HEAD_DIM * elem_bytes(d->kv_dtype);
  const size_t sc_bytes = with_scales ? B * 2 * GQA_NUM_KV_HEADS * (size_t)d->capacity * 2 : 0;
  const size_t len_bytes = B * sizeof(int32_t);
  if (ranges_overlap(out, q_bytes, q, q_bytes) || ranges_overlap(out, q_bytes, kv, kv_bytes) ||
      ranges_overlap(out, q_bytes, lens, len_bytes) ||
      (with_scales && ranges_overlap(out, q_bytes, scales, sc_bytes)))
    return fail(GQA_ERR_ALIAS, with_scales ? "out must not overlap q, kv, kv_scales or seq_lens"
                                           : "out must not overlap q, kv or seq_lens");
  return GQA_OK;
}

// --- device gate (gfx950 only) ------------------------------------------------
std::mutex g_dev_mu;
std::map<int, bool> g_dev_ok;

gqa_status_t check_device(int* dev_out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(GQA_ERR_HIP, "hipGetDevice failed: %s", hipGetErrorString(e));
  *dev_out = dev;
  std::lock_guard<std::mutex> lk(g_dev_mu);
  auto it = g_dev_ok.find(dev);
  if (it == g_dev_ok.end()) {
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess)
      return fail(GQA_ERR_HIP, "hipGetDeviceProperties failed: %s", hipGetErrorString(e));
    const bool good = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    it = g_dev_ok.emplace(dev, good).first;
    if (!good)
      return fail(GQA_ERR_UNSUPPORTED_DEVICE, "device %d is %s; this library is built for gfx950",
                  dev, prop.gcnArchName);
  }
  if (!it->second) return fail(GQA_ERR_UNSUPPORTED_DEVICE, "device %d is not gfx950", dev);
  return GQA_OK;
}

gqa::StepArgs step_args(const gqa_desc_t* d, const void* q, const void* kv, const void* scales,
                        const int32_t* lens, float q_scale, void* out, const gqa_plan_t& p,
                        void* ws, const Paging& pg, int tier_size) {
  gqa::StepArgs a;
  a.q = q;
  a.kv = kv;
  a.kv_scales = scales;
  a.num_q_heads = d->num_q_heads;
  a.seq_lens = lens;
  a.out = out;
  const WorkspaceLayout wl = plan_layout(d, p, pg);
  char* base = static_cast<char*>(ws);
  a.part_o = ws ? reinterpret_cast<float*>(base + wl.o_offset) : nullptr;
  a.part_ml = ws ? reinterpret_cast<float*>(base + wl.ml_offset) : nullptr;
  a.counters = (ws && p.route != 2) ? reinterpret_cast<uint32_t*>(base) : nullptr;
  a.slab_prefix = (ws && p.route == 2) ? reinterpret_cast<int32_t*>(base + wl.aux_offset) : nullptr;
  a.head_pieces = a.slab_prefix ? a.slab_prefix + d->batch + 1 : nullptr;
  a.fused_combine = p.fused_merge;
  a.grid_wgs = p.route == 2 ? p.num_workgroups : 0;
  set_shares(a, tier_size, d->kv_dtype);
  a.batch = d->batch;
  a.capacity = d->capacity;
  a.num_splits = p.num_splits;
  a.chunk_tokens = p.chunk_tokens;
  // log2-domain score scale, computed once on the host in double precision.
  const double scale = (double)q_scale * (double)d->k_scale / std::sqrt((double)GQA_HEAD_DIM) /
                       std::log(2.0);
  a.scale_log2 = (float)scale;
  a.v_scale = d->v_scale;
  a.block_table = pg.block_table;
  a.max_pages = pg.max_pages;
  a.page_shift = pg.page_shift;
  a.num_pages = pg.num_pages;
  a.q_tokens = pg.q_tokens;
  a.scales_by_position = pg.scales_by_position ? 1 : 0;
  return a;
}

gqa_status_t enqueue(const gqa::StepArgs& a, const gqa_desc_t* d, bool paged, hipStream_t stream,
                     hipEvent_t ev_mid = nullptr) {
  hipError_t e = paged ? gqa::enqueue_paged_decode_step(a, d->q_dtype, d->kv_dtype, stream, ev_mid)
                       : gqa::enqueue_decode_step(a, d->q_dtype, d->kv_dtype, stream, ev_mid);
  if (e != hipSuccess) return fail(GQA_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  return ok();
}

// --- convenience-call workspace cache, per (device, stream) ----------------------
struct CacheEntry {
  void* ptr = nullptr;
  size_t bytes = 0;
  size_t zero_bytes = 0;   // leading bytes known to be zero (the control words of the last plan)
};
std::mutex g_cache_mu;
std::map<std::pair<int, uintptr_t>, CacheEntry> g_cache;

}  // namespace

struct gqa_prepared {
  gqa_desc_t desc;
  gqa_plan_t plan;
  const void* q;
  const void* kv;
  const void* kv_scales;   // INT8 cache only
  const int32_t* seq_lens;
  void* out;
  float q_scale;
  void* workspace;
  int device;
  int tier_size;           // the device's CU count (balanced-split shares)
  Paging pg;               // paged cache / several query tokens
};

namespace {

// The steps after argument checking, shared by the contiguous and the paged
// entry points (pg: paging and query tokens; default = contiguous, one token).
gqa_status_t prepare_checked(const gqa_desc_t* desc, const void* q, const void* kv,
                             const void* scales, const int32_t* seq_lens, float q_scale, void* out,
                             int32_t num_splits, const Paging& pg, gqa_prepared_t** handle) {
  gqa_plan_t p;
  gqa_status_t st = make_plan(desc, num_splits, &p, 0, pg);
  if (st != GQA_OK) return st;
  int dev = -1;
  st = check_device(&dev);
  if (st != GQA_OK) return st;
  if (p.route == 2) {   // size the balanced grid for this device
    st = make_plan(desc, num_splits, &p, device_balanced_grid(dev, desc, pg.on), pg,
                   device_cus(dev));
    if (st != GQA_OK) return st;
  }
  void* ws = nullptr;
  if (p.workspace_bytes > 0 && desc->batch > 0) {
    hipError_t e = hipMalloc(&ws, p.workspace_bytes);
    if (e != hipSuccess) {
      (void)hipGetLastError();
      return fail(GQA_ERR_OUT_OF_MEMORY, "hipMalloc(%llu) for the split workspace failed: %s",
                  (unsigned long long)p.workspace_bytes, hipGetErrorString(e));
    }
    // The per-head counters must start at zero; launches keep them at zero.
    e = hipMemset(ws, 0, p.workspace_bytes);
    if (e != hipSuccess) {
      (void)hipFree(ws);
      return fail(GQA_ERR_HIP, "hipMemset of the workspace failed: %s", hipGetErrorString(e));
    }
  }
  gqa_prepared* h = new (std::nothrow) gqa_prepared;
  if (h == nullptr) {
    if (ws) (void)hipFree(ws);
    return fail(GQA_ERR_OUT_OF_MEMORY, "out of host memory");
  }
  h->desc = *desc;
  h->plan = p;
  h->q = q;
  h->kv = kv;
  h->kv_scales = scales;
  h->seq_lens = seq_lens;
  h->out = out;
  h->q_scale = q_scale;
  h->workspace = ws;
  h->device = dev;
  h->tier_size = device_cus(dev);
  h->pg = pg;
  *handle = h;
  return ok();
}

gqa_status_t decode_checked(const gqa_desc_t* desc, const void* q, const void* kv,
                            const void* scales, const int32_t* seq_lens, float q_scale, void* out,
                            const Paging& pg, hipStream_t stream) {
  gqa_plan_t p;
  gqa_status_t st = make_plan(desc, 0, &p, 0, pg);
  if (st != GQA_OK) return st;
  if (desc->batch == 0) return ok();
  int dev = -1;
  st = check_device(&dev);
  if (st != GQA_OK) return st;
  if (p.route == 2) {
    st = make_plan(desc, 0, &p, device_balanced_grid(dev, desc, pg.on), pg, device_cus(dev));
    if (st != GQA_OK) return st;
  }

  void* ws = nullptr;
  // Held until the kernels are enqueued: another host thread that grows the
  // same (device, stream) entry frees the old buffer only after this call's
  // launches are in the stream ahead of its synchronisation.
  std::unique_lock<std::mutex> lk(g_cache_mu, std::defer_lock);
  if (p.workspace_bytes > 0) {
    lk.lock();
    CacheEntry& ce = g_cache[{dev, reinterpret_cast<uintptr_t>(stream)}];
    if (ce.bytes < p.workspace_bytes) {
      hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
      hipError_t e = hipStreamIsCapturing(stream, &cs);
      if (e != hipSuccess) {
        (void)hipGetLastError();
        return fail(GQA_ERR_HIP, "hipStreamIsCapturing failed: %s", hipGetErrorString(e));
      }
      if (cs != hipStreamCaptureStatusNone)
        return fail(GQA_ERR_CAPTURE,
                    "the convenience call would allocate %llu workspace bytes while the stream "
                    "is capturing; use the prepare / launch_gqa_decode_prepared pair",
                    (unsigned long long)p.workspace_bytes);
      if (ce.ptr) {
        // Work already enqueued on this stream may still use the old buffer.
        e = hipStreamSynchronize(stream);
        if (e != hipSuccess) return fail(GQA_ERR_HIP, "hipStreamSynchronize failed: %s", hipGetErrorString(e));
        (void)hipFree(ce.ptr);
        ce.ptr = nullptr;
        ce.bytes = 0;
      }
      e = hipMalloc(&ce.ptr, p.workspace_bytes);
      if (e != hipSuccess) {
        (void)hipGetLastError();
        ce.ptr = nullptr;
        return fail(GQA_ERR_OUT_OF_MEMORY, "hipMalloc(%llu) for the split workspace failed: %s",
                    (unsigned long long)p.workspace_bytes, hipGetErrorString(e));
      }
      // Zero it (counters) on the stream, ahead of the launch that uses it.
      e = hipMemsetAsync(ce.ptr, 0, p.workspace_bytes, stream);
      if (e != hipSuccess) {
        (void)hipFree(ce.ptr);
        ce.ptr = nullptr;
        return fail(GQA_ERR_HIP, "hipMemsetAsync of the workspace failed: %s", hipGetErrorString(e));
      }
      ce.bytes = p.workspace_bytes;
      ce.zero_bytes = p.workspace_bytes;
    }
    // The control words must start at zero. A plan with more of them than the
    // last one finds partials of the earlier plan there: clear those bytes
    // (not during a capture, where that would record a memset; an automatic
    // one-launch plan then takes the two-launch merge, which needs none).
    size_t ctrl = (size_t)plan_layout(desc, p, pg).ctrl_bytes;
    if (ctrl > ce.zero_bytes) {
      hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
      hipError_t e = hipStreamIsCapturing(stream, &cs);
      if (e != hipSuccess) {
        (void)hipGetLastError();
        return fail(GQA_ERR_HIP, "hipStreamIsCapturing failed: %s", hipGetErrorString(e));
      }
      if (cs != hipStreamCaptureStatusNone && !(desc->flags & GQA_FLAG_FUSED_COMBINE)) {
        st = make_plan(desc, 0, &p, 0, pg, 0, /*one_launch_ok=*/false);
        if (st != GQA_OK) return st;
        ctrl = (size_t)plan_layout(desc, p, pg).ctrl_bytes;   // 0: no control words
      } else if (cs != hipStreamCaptureStatusNone) {
        return fail(GQA_ERR_CAPTURE,
                    "the convenience call would clear %llu workspace bytes while the stream is "
                    "capturing; use the prepare / launch_gqa_decode_prepared pair",
                    (unsigned long long)(ctrl - ce.zero_bytes));
      } else {
        e = hipMemsetAsync(static_cast<char*>(ce.ptr) + ce.zero_bytes, 0, ctrl - ce.zero_bytes,
                           stream);
        if (e != hipSuccess)
          return fail(GQA_ERR_HIP, "hipMemsetAsync of the workspace failed: %s",
                      hipGetErrorString(e));
      }
    }
    // Launches leave the control words at zero; everything after them is now dirty.
    ce.zero_bytes = ctrl;
    ws = ce.ptr;
  }
  return enqueue(step_args(desc, q, kv, scales, seq_lens, q_scale, out, p, ws, pg, device_cus(dev)),
                 desc, pg.on, stream);
}

gqa_status_t validate_impl(const gqa_desc_t* desc, const void* q, const void* kv,
                           const void* scales, bool with_scales, const int32_t* seq_lens,
                           float q_scale, const void* out, int32_t num_splits) {
  gqa_status_t st = check_args(desc, q, kv, scales, with_scales, seq_lens, q_scale, out);
  if (st != GQA_OK) return st;
  gqa_plan_t p;
  st = make_plan(desc, num_splits, &p);
  if (st != GQA_OK) return st;
  return ok();
}

gqa_status_t prepare_impl(const gqa_desc_t* desc, const void* q, const void* kv,
                          const void* scales, bool with_scales, const int32_t* seq_lens,
                          float q_scale, void* out, int32_t num_splits, gqa_prepared_t** handle) {
  if (handle == nullptr) return fail(GQA_ERR_INVALID_ARG, "handle is NULL");
  *handle = nullptr;
  gqa_status_t st = check_args(desc, q, kv, scales, with_scales, seq_lens, q_scale, out);
  if (st != GQA_OK) return st;
  return prepare_checked(desc, q, kv, scales, seq_lens, q_scale, out, num_splits, Paging(), handle);
}

// gqa_decode / gqa_decode_int8 with the static scratch as the split
// workspace: the same plan, kernels and results, and no allocation.
gqa_status_t decode_no_alloc_checked(const gqa_desc_t* desc, const void* q, const void* kv,
                                     const void* scales, const int32_t* seq_lens, float q_scale,
                                     void* out, hipStream_t stream) {
  if (desc->flags != 0)
    return fail(GQA_ERR_INVALID_ARG, "gqa_decode_no_alloc takes no flags (got 0x%x)",
                (unsigned)desc->flags);
  auto too_big = [](const gqa_plan_t& p) {
    return fail(GQA_ERR_INVALID_ARG,
                "this plan needs %llu workspace bytes; gqa_decode_no_alloc's static scratch "
                "holds %llu (use gqa_decode or the prepared pair)",
                (unsigned long long)p.workspace_bytes,
                (unsigned long long)GQA_NO_ALLOC_SCRATCH_BYTES);
  };
  gqa_plan_t p;
  gqa_status_t st = make_plan(desc, 0, &p, 0, Paging(), 0, /*one_launch_ok=*/false);
  if (st != GQA_OK) return st;
  // The host-only plan already decides the chunked routes' workspace (and
  // bounds the balanced one by a nominal grid), so an oversized request is
  // refused before any device is touched.
  if (p.route != 2 && p.workspace_bytes > GQA_NO_ALLOC_SCRATCH_BYTES) return too_big(p);
  if (desc->batch == 0) return ok();
  int dev = -1;
  st = check_device(&dev);
  if (st != GQA_OK) return st;
  if (p.route == 2) {
    st = make_plan(desc, 0, &p, device_balanced_grid(dev, desc, false), Paging(), device_cus(dev),
                   /*one_launch_ok=*/false);
    if (st != GQA_OK) return st;
  }
  void* ws = nullptr;
  if (p.workspace_bytes > 0) {
    if (p.workspace_bytes > GQA_NO_ALLOC_SCRATCH_BYTES) return too_big(p);
    const hipError_t e = gqa::no_alloc_scratch(dev, &ws);
    if (e != hipSuccess)
      return fail(GQA_ERR_HIP, "looking up the no-alloc scratch on device %d failed: %s", dev,
                  hipGetErrorString(e));
  }
  // Nothing in the workspace needs to start at zero here: without the
  // one-launch merge (never planned for this entry point), every partial row
  // and bookkeeping word a launch reads was written by that launch.
  return enqueue(step_args(desc, q, kv, scales, seq_lens, q_scale, out, p, ws, Paging(),
                           device_cus(dev)),
                 desc, false, stream);
}

gqa_status_t decode_impl(const gqa_desc_t* desc, const void* q, const void* kv,
                         const void* scales, bool with_scales, const int32_t* seq_lens,
                         float q_scale, void* out, hipStream_t stream) {
  gqa_status_t st = check_args(desc, q, kv, scales, with_scales, seq_lens, q_scale, out);
  if (st != GQA_OK) return st;
  return decode_checked(desc, q, kv, scales, seq_lens, q_scale, out, Paging(), stream);
}

// --- paged cache ---------------------------------------------------------------
// Checks a paged descriptor; on success fills the equivalent contiguous
// descriptor (capacity = max_pages * page_size, the longest length a
// block-table row can address) and the paging record (without a table).
gqa_status_t check_paged_desc(const gqa_paged_desc_t* pd, gqa_desc_t* d, Paging* pg) {
  if (pd == nullptr) return fail(GQA_ERR_INVALID_ARG, "desc is NULL");
  const int P = pd->page_size;
  if (P < 16 || P > GQA_MAX_PAGE_SIZE || (P & (P - 1)) != 0)
    return fail(GQA_ERR_INVALID_ARG, "page_size must be a power of two in [16, %d] (got %d)",
                GQA_MAX_PAGE_SIZE, P);
  if (pd->num_pages < 1 || pd->max_pages < 1)
    return fail(GQA_ERR_INVALID_ARG, "num_pages and max_pages must be >= 1 (got %d, %d)",
                pd->num_pages, pd->max_pages);
  if ((int64_t)pd->max_pages * P > GQA_MAX_CAPACITY)
    return fail(GQA_ERR_INVALID_ARG, "max_pages * page_size must be <= %d (got %lld)",
                GQA_MAX_CAPACITY, (long long)pd->max_pages * P);
  if ((pd->flags & ~GQA_PAGED_SCALES_BY_POSITION) != 0)
    return fail(GQA_ERR_INVALID_ARG,
                "the paged entry points take no flags but GQA_PAGED_SCALES_BY_POSITION (got 0x%x)",
                (unsigned)pd->flags);
  if ((pd->flags & GQA_PAGED_SCALES_BY_POSITION) && pd->kv_dtype != GQA_INT8_ROWSCALE)
    return fail(GQA_ERR_INVALID_ARG,
                "GQA_PAGED_SCALES_BY_POSITION needs an INT8_ROWSCALE pool (kv dtype %d)",
                pd->kv_dtype);
  *d = gqa_desc_t{};
  d->batch = pd->batch;
  d->capacity = pd->max_pages * P;
  d->num_q_heads = pd->num_q_heads;
  d->num_kv_heads = pd->num_kv_heads;
  d->head_dim = pd->head_dim;
  d->q_dtype = pd->q_dtype;
  d->kv_dtype = pd->kv_dtype;
  d->k_scale = pd->k_scale;
  d->v_scale = pd->v_scale;
  d->flags = 0;
  gqa_status_t st = check_desc(d);
  if (st != GQA_OK) return st;
  const int group = pd->num_q_heads / GQA_NUM_KV_HEADS;
  if (pd->q_tokens < 1 || pd->q_tokens * group > GQA_PAGED_MAX_ROWS)
    return fail(GQA_ERR_INVALID_ARG,
                "q_tokens must be in [1, %d] for %d query heads (q_tokens x query heads per KV "
                "head <= %d; got %d)",
                GQA_PAGED_MAX_ROWS / group, pd->num_q_heads, GQA_PAGED_MAX_ROWS, pd->q_tokens);
  pg->on = true;
  pg->q_tokens = pd->q_tokens;
  pg->page_shift = __builtin_ctz((unsigned)P);
  pg->num_pages = pd->num_pages;
  pg->max_pages = pd->max_pages;
  pg->block_table = nullptr;
  pg->scales_by_position = (pd->flags & GQA_PAGED_SCALES_BY_POSITION) != 0;
  return GQA_OK;
}

// Bytes of the pool's K/V rows.
size_t pool_bytes_of(const gqa_paged_desc_t* pd) {
  return (size_t)pd->num_pages * 2 * GQA_NUM_KV_HEADS * (size_t)pd->page_size * GQA_HEAD_DIM *
         elem_bytes(pd->kv_dtype);
}

// Bytes of an INT8 pool's row scales, in the layout the flags select.
size_t scale_bytes_of(const gqa_paged_desc_t* pd) {
  const size_t per_head = (pd->flags & GQA_PAGED_SCALES_BY_POSITION)
                              ? (size_t)pd->batch * (size_t)pd->max_pages * (size_t)pd->page_size
                              : (size_t)pd->num_pages * (size_t)pd->page_size;
  return per_head * 2 * GQA_NUM_KV_HEADS * 2;
}

// Checks a paged descriptor and a decode call's buffers (see check_paged_desc).
gqa_status_t check_paged_args(const gqa_paged_desc_t* pd, const void* q, const void* pool,
                              const void* scales, const int32_t* table, const int32_t* lens,
                              float q_scale, const void* out, gqa_desc_t* d, Paging* pg) {
  gqa_status_t st = check_paged_desc(pd, d, pg);
  if (st != GQA_OK) return st;
  if (!scale_ok(q_scale))
    return fail(GQA_ERR_INVALID_ARG, "q_scale must be finite and > 0 (got %g)", (double)q_scale);
  const bool int8 = pd->kv_dtype == GQA_INT8_ROWSCALE;
  pg->block_table = table;
  if (pd->batch == 0) return GQA_OK;
  if (!q || !pool || !table || !lens || !out || (int8 && !scales))
    return fail(GQA_ERR_INVALID_ARG, int8 ? "q, kv_pages, kv_scales, block_table, seq_lens and out "
                                            "must be non-NULL"
                                          : "q, kv_pages, block_table, seq_lens and out must be "
                                            "non-NULL");
  if (!int8 && scales)
    return fail(GQA_ERR_INVALID_ARG, "kv_scales must be NULL unless the cache is INT8_ROWSCALE");
  if (!aligned(q, 16) || !aligned(pool, 16) || !aligned(out, 16) || !aligned(table, 4) ||
      !aligned(lens, 4) || (int8 && !aligned(scales, 16)))
    return fail(GQA_ERR_INVALID_ARG,
                "q, kv_pages, kv_scales and out must be 16-byte aligned, block_table and "
                "seq_lens 4-byte aligned");
  const size_t B = (size_t)pd->batch;
  const size_t q_bytes =
      B * (size_t)pd->q_tokens * (size_t)pd->num_q_heads * GQA_HEAD_DIM * elem_bytes(pd->q_dtype);
  const size_t pool_bytes = pool_bytes_of(pd);
  const size_t sc_bytes = int8 ? scale_bytes_of(pd) : 0;
  const size_t table_bytes = B * (size_t)pd->max_pages * sizeof(int32_t);
  if (ranges_overlap(out, q_bytes, q, q_bytes) || ranges_overlap(out, q_bytes, pool, pool_bytes) ||
      ranges_overlap(out, q_bytes, lens, B * sizeof(int32_t)) ||
      ranges_overlap(out, q_bytes, table, table_bytes) ||
      (int8 && ranges_overlap(out, q_bytes, scales, sc_bytes)))
    return fail(GQA_ERR_ALIAS,
                "out must not overlap q, kv_pages, kv_scales, block_table or seq_lens");
  return GQA_OK;
}

// The KV append entry points; int8 = the _int8 forms, which write an
// INT8_ROWSCALE cache and its bf16 row scales (the others reject one).
gqa_status_t check_append_dtype(int kv_dtype, bool int8, const char* name) {
  if (int8 && kv_dtype != GQA_INT8_ROWSCALE)
    return fail(GQA_ERR_INVALID_ARG, "%s_int8 needs kv dtype INT8_ROWSCALE (got %d)", name, kv_dtype);
  if (!int8 && kv_dtype == GQA_INT8_ROWSCALE)
    return fail(GQA_ERR_INVALID_ARG, "%s does not write an INT8_ROWSCALE cache; use %s_int8", name,
                name);
  return GQA_OK;
}

gqa_status_t append_contiguous(const gqa_desc_t* desc, const void* k_new, const void* v_new,
                               const int32_t* positions, void* kv, void* kv_scales, bool int8,
                               hipStream_t stream) {
  gqa_status_t st = check_desc(desc);
  if (st != GQA_OK) return st;
  st = check_append_dtype(desc->kv_dtype, int8, "gqa_kv_append");
  if (st != GQA_OK) return st;
  if (desc->batch == 0) return ok();
  if (!k_new || !v_new || !positions || !kv || (int8 && !kv_scales))
    return fail(GQA_ERR_INVALID_ARG, "k_new, v_new, positions, kv%s must be non-NULL",
                int8 ? " and kv_scales" : "");
  if (!aligned(k_new, 16) || !aligned(v_new, 16) || !aligned(kv, 16) || !aligned(positions, 4) ||
      (int8 && !aligned(kv_scales, 2)))
    return fail(GQA_ERR_INVALID_ARG,
                "k_new, v_new and kv must be 16-byte aligned, positions 4-byte aligned%s",
                int8 ? " and kv_scales 2-byte aligned" : "");
  if (desc->batch > kMaxLaunchWorkgroups)   // one workgroup per request
    return fail(GQA_ERR_INVALID_ARG, "batch too large for one append launch (%d)", desc->batch);
  const size_t B = (size_t)desc->batch;
  const size_t row_bytes = B * GQA_NUM_KV_HEADS * GQA_HEAD_DIM * elem_bytes(desc->q_dtype);
  const size_t rows = B * 2 * GQA_NUM_KV_HEADS * (size_t)desc->capacity;
  const size_t kv_bytes = rows * GQA_HEAD_DIM * elem_bytes(desc->kv_dtype);
  const size_t pos_bytes = B * sizeof(int32_t);
  if (ranges_overlap(kv, kv_bytes, k_new, row_bytes) || ranges_overlap(kv, kv_bytes, v_new, row_bytes) ||
      ranges_overlap(kv, kv_bytes, positions, pos_bytes))
    return fail(GQA_ERR_ALIAS, "kv must not overlap k_new, v_new or positions");
  if (int8) {
    const size_t sc_bytes = rows * 2;
    if (ranges_overlap(kv_scales, sc_bytes, kv, kv_bytes) ||
        ranges_overlap(kv_scales, sc_bytes, k_new, row_bytes) ||
        ranges_overlap(kv_scales, sc_bytes, v_new, row_bytes) ||
        ranges_overlap(kv_scales, sc_bytes, positions, pos_bytes))
      return fail(GQA_ERR_ALIAS, "kv_scales must not overlap kv, k_new, v_new or positions");
  }
  int dev = -1;
  st = check_device(&dev);
  if (st != GQA_OK) return st;
  gqa::AppendArgs a;
  a.k_new = k_new;
  a.v_new = v_new;
  a.positions = positions;
  a.kv = kv;
  a.kv_scales = kv_scales;
  a.batch = desc->batch;
  a.capacity = desc->capacity;
  a.k_scale = desc->k_scale;
  a.v_scale = desc->v_scale;
  hipError_t e = gqa::enqueue_kv_append(a, desc->q_dtype, desc->kv_dtype, stream);
  if (e != hipSuccess) return fail(GQA_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  return ok();
}

gqa_status_t append_paged(const gqa_paged_desc_t* desc, const void* k_new, const void* v_new,
                          const int32_t* positions, const int32_t* block_table, void* kv_pages,
                          void* kv_scales, bool int8, hipStream_t stream) {
  gqa_desc_t d;
  Paging pg;
  gqa_status_t st = check_paged_desc(desc, &d, &pg);
  if (st != GQA_OK) return st;
  st = check_append_dtype(desc->kv_dtype, int8, "gqa_kv_append_paged");
  if (st != GQA_OK) return st;
  if (desc->batch == 0) return ok();
  if (!k_new || !v_new || !positions || !block_table || !kv_pages || (int8 && !kv_scales))
    return fail(GQA_ERR_INVALID_ARG,
                "k_new, v_new, positions, block_table, kv_pages%s must be non-NULL",
                int8 ? " and kv_scales" : "");
  if (!aligned(k_new, 16) || !aligned(v_new, 16) || !aligned(kv_pages, 16) ||
      !aligned(positions, 4) || !aligned(block_table, 4) || (int8 && !aligned(kv_scales, 2)))
    return fail(GQA_ERR_INVALID_ARG,
                "k_new, v_new and kv_pages must be 16-byte aligned, positions and block_table "
                "4-byte aligned%s", int8 ? ", kv_scales 2-byte aligned" : "");
  if ((int64_t)desc->batch * desc->q_tokens > kMaxLaunchWorkgroups)   // one workgroup per token
    return fail(GQA_ERR_INVALID_ARG, "batch x q_tokens too large for one append launch");
  const size_t B = (size_t)desc->batch;
  const size_t row_bytes =
      B * (size_t)desc->q_tokens * GQA_NUM_KV_HEADS * GQA_HEAD_DIM * elem_bytes(desc->q_dtype);
  const size_t pool_bytes = pool_bytes_of(desc);
  const size_t pos_bytes = B * sizeof(int32_t);
  const size_t table_bytes = B * (size_t)desc->max_pages * sizeof(int32_t);
  if (ranges_overlap(kv_pages, pool_bytes, k_new, row_bytes) ||
      ranges_overlap(kv_pages, pool_bytes, v_new, row_bytes) ||
      ranges_overlap(kv_pages, pool_bytes, positions, pos_bytes) ||
      ranges_overlap(kv_pages, pool_bytes, block_table, table_bytes))
    return fail(GQA_ERR_ALIAS, "kv_pages must not overlap k_new, v_new, positions or block_table");
  if (int8) {
    const size_t sc_bytes = scale_bytes_of(desc);
    if (ranges_overlap(kv_scales, sc_bytes, kv_pages, pool_bytes) ||
        ranges_overlap(kv_scales, sc_bytes, k_new, row_bytes) ||
        ranges_overlap(kv_scales, sc_bytes, v_new, row_bytes) ||
        ranges_overlap(kv_scales, sc_bytes, positions, pos_bytes) ||
        ranges_overlap(kv_scales, sc_bytes, block_table, table_bytes))
      return fail(GQA_ERR_ALIAS,
                  "kv_scales must not overlap kv_pages, k_new, v_new, positions or block_table");
  }
  int dev = -1;
  st = check_device(&dev);
  if (st != GQA_OK) return st;
  gqa::AppendArgs a;
  a.k_new = k_new;
  a.v_new = v_new;
  a.positions = positions;
  a.kv = kv_pages;
  a.kv_scales = kv_scales;
  a.batch = desc->batch;
  a.tokens = desc->q_tokens;
  a.capacity = d.capacity;
  a.k_scale = desc->k_scale;
  a.v_scale = desc->v_scale;
  a.block_table = block_table;
  a.max_pages = desc->max_pages;
  a.page_shift = pg.page_shift;
  a.num_pages = desc->num_pages;
  a.scales_by_position = pg.scales_by_position ? 1 : 0;
  hipError_t e = gqa::enqueue_kv_append(a, desc->q_dtype, desc->kv_dtype, stream);
  if (e != hipSuccess) return fail(GQA_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  return ok();
}

}  // namespace

extern "C" {

GQA_API const char* gqa_last_error(void) { return g_last_error.c_str(); }

GQA_API gqa_status_t gqa_validate_args(const gqa_desc_t* desc, const void* q, const void* kv,
                                       const int32_t* seq_lens, float q_scale, const void* out,
                                       int32_t num_splits) {
  return validate_impl(desc, q, kv, nullptr, false, seq_lens, q_scale, out, num_splits);
}

GQA_API gqa_status_t gqa_validate_args_int8(const gqa_desc_t* desc, const void* q, const void* kv,
                                            const void* kv_scales, const int32_t* seq_lens,
                                            float q_scale, const void* out, int32_t num_splits) {
  return validate_impl(desc, q, kv, kv_scales, true, seq_lens, q_scale, out, num_splits);
}

GQA_API gqa_status_t gqa_plan_decode(const gqa_desc_t* desc, int32_t num_splits, gqa_plan_t* plan) {
  if (plan == nullptr) return fail(GQA_ERR_INVALID_ARG, "plan is NULL");
  gqa_status_t st = check_desc(desc);
  if (st != GQA_OK) return st;
  st = make_plan(desc, num_splits, plan);
  if (st != GQA_OK) return st;
  return ok();
}

GQA_API gqa_status_t prepare_gqa_decode(const gqa_desc_t* desc, const void* q, const void* kv,
                                        const int32_t* seq_lens, float q_scale, void* out,
                                        int32_t num_splits, gqa_prepared_t** handle) {
  return prepare_impl(desc, q, kv, nullptr, false, seq_lens, q_scale, out, num_splits, handle);
}

GQA_API gqa_status_t prepare_gqa_decode_int8(const gqa_desc_t* desc, const void* q,
                                             const void* kv, const void* kv_scales,
                                             const int32_t* seq_lens, float q_scale, void* out,
                                             int32_t num_splits, gqa_prepared_t** handle) {
  return prepare_impl(desc, q, kv, kv_scales, true, seq_lens, q_scale, out, num_splits, handle);
}

GQA_API gqa_status_t launch_gqa_decode_prepared_timed(gqa_prepared_t* h, hipStream_t stream,
                                                      hipEvent_t ev_start, hipEvent_t ev_mid,
                                                      hipEvent_t ev_end) {
  if (h == nullptr) return fail(GQA_ERR_INVALID_ARG, "handle is NULL");
  if (h->desc.batch == 0) return ok();
  int cur = -1;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return fail(GQA_ERR_HIP, "hipGetDevice failed: %s", hipGetErrorString(e));
  if (cur != h->device && (e = hipSetDevice(h->device)) != hipSuccess)
    return fail(GQA_ERR_HIP, "hipSetDevice(%d) failed: %s", h->device, hipGetErrorString(e));
  gqa_status_t st = GQA_OK;
  if (ev_start != nullptr && (e = hipEventRecord(ev_start, stream)) != hipSuccess)
    st = fail(GQA_ERR_HIP, "hipEventRecord failed: %s", hipGetErrorString(e));
  if (st == GQA_OK) {
    const gqa::StepArgs a = step_args(&h->desc, h->q, h->kv, h->kv_scales, h->seq_lens, h->q_scale,
                                      h->out, h->plan, h->workspace, h->pg, h->tier_size);
    st = enqueue(a, &h->desc, h->pg.on, stream, ev_mid);
  }
  if (st == GQA_OK && ev_end != nullptr && (e = hipEventRecord(ev_end, stream)) != hipSuccess)
    st = fail(GQA_ERR_HIP, "hipEventRecord failed: %s", hipGetErrorString(e));
  if (cur != h->device) (void)hipSetDevice(cur);
  return st;
}

GQA_API gqa_status_t launch_gqa_decode_prepared(gqa_prepared_t* h, hipStream_t stream) {
  return launch_gqa_decode_prepared_timed(h, stream, nullptr, nullptr, nullptr);
}

GQA_API void gqa_prepared_destroy(gqa_prepared_t* h) {
  if (h == nullptr) return;
  if (h->workspace) (void)hipFree(h->workspace);
  delete h;
}

GQA_API size_t gqa_prepared_workspace_bytes(const gqa_prepared_t* h) {
  return (h && h->workspace) ? (size_t)h->plan.workspace_bytes : 0;
}

GQA_API gqa_status_t gqa_prepared_plan(const gqa_prepared_t* h, gqa_plan_t* plan) {
  if (h == nullptr || plan == nullptr) return fail(GQA_ERR_INVALID_ARG, "NULL argument");
  *plan = h->plan;
  return ok();
}

GQA_API gqa_status_t gqa_decode(const gqa_desc_t* desc, const void* q, const void* kv,
                                const int32_t* seq_lens, float q_scale, void* out,
                                hipStream_t stream) {
  return decode_impl(desc, q, kv, nullptr, false, seq_lens, q_scale, out, stream);
}

GQA_API gqa_status_t gqa_decode_int8(const gqa_desc_t* desc, const void* q, const void* kv,
                                     const void* kv_scales, const int32_t* seq_lens,
                                     float q_scale, void* out, hipStream_t stream) {
  return decode_impl(desc, q, kv, kv_scales, true, seq_lens, q_scale, out, stream);
}

GQA_API gqa_status_t gqa_decode_no_alloc(const gqa_desc_t* desc, const void* q, const void* kv,
                                         const void* kv_scales, const int32_t* seq_lens,
                                         float q_scale, void* out, hipStream_t stream) {
  const bool int8 = desc != nullptr && desc->kv_dtype == GQA_INT8_ROWSCALE;
  gqa_status_t st = check_args(desc, q, kv, kv_scales, int8, seq_lens, q_scale, out);
  if (st != GQA_OK) return st;
  if (!int8 && kv_scales != nullptr)
    return fail(GQA_ERR_INVALID_ARG, "kv_scales must be NULL unless the cache is INT8_ROWSCALE");
  return decode_no_alloc_checked(desc, q, kv, kv_scales, seq_lens, q_scale, out, stream);
}

GQA_API gqa_status_t gqa_validate_args_paged(const gqa_paged_desc_t* desc, const void* q,
                                             const void* kv_pages, const void* kv_scales,
                                             const int32_t* block_table, const int32_t* seq_lens,
                                             float q_scale, const void* out, int32_t num_splits) {
  gqa_desc_t d;
  Paging pg;
  gqa_status_t st = check_paged_args(desc, q, kv_pages, kv_scales, block_table, seq_lens, q_scale,
                                     out, &d, &pg);
  if (st != GQA_OK) return st;
  gqa_plan_t p;
  st = make_plan(&d, num_splits, &p, 0, pg);
  if (st != GQA_OK) return st;
  return ok();
}

GQA_API gqa_status_t gqa_plan_decode_paged(const gqa_paged_desc_t* desc, int32_t num_splits,
                                           gqa_plan_t* plan) {
  if (plan == nullptr) return fail(GQA_ERR_INVALID_ARG, "plan is NULL");
  gqa_desc_t d;
  Paging pg;
  // Descriptor checks only: with batch 0 no buffer is looked at.
  gqa_paged_desc_t probe = desc ? *desc : gqa_paged_desc_t{};
  const int32_t batch = probe.batch;
  probe.batch = 0;
  gqa_status_t st = check_paged_args(desc ? &probe : nullptr, nullptr, nullptr, nullptr, nullptr,
                                     nullptr, 1.0f, nullptr, &d, &pg);
  if (st != GQA_OK) return st;
  if (batch < 0) return fail(GQA_ERR_INVALID_ARG, "batch must be >= 0 (got %d)", batch);
  d.batch = batch;
  st = make_plan(&d, num_splits, plan, 0, pg);
  if (st != GQA_OK) return st;
  return ok();
}

GQA_API gqa_status_t prepare_gqa_decode_paged(const gqa_paged_desc_t* desc, const void* q,
                                              const void* kv_pages, const void* kv_scales,
                                              const int32_t* block_table, const int32_t* seq_lens,
                                              float q_scale, void* out, int32_t num_splits,
                                              gqa_prepared_t** handle) {
  if (handle == nullptr) return fail(GQA_ERR_INVALID_ARG, "handle is NULL");
  *handle = nullptr;
  gqa_desc_t d;
  Paging pg;
  gqa_status_t st = check_paged_args(desc, q, kv_pages, kv_scales, block_table, seq_lens, q_scale,
                                     out, &d, &pg);
  if (st != GQA_OK) return st;
  return prepare_checked(&d, q, kv_pages, kv_scales, seq_lens, q_scale, out, num_splits, pg, handle);
}

GQA_API gqa_status_t gqa_decode_paged(const gqa_paged_desc_t* desc, const void* q,
                                      const void* kv_pages, const void* kv_scales,
                                      const int32_t* block_table, const int32_t* seq_lens,
                                      float q_scale, void* out, hipStream_t stream) {
  gqa_desc_t d;
  Paging pg;
  gqa_status_t st = check_paged_args(desc, q, kv_pages, kv_scales, block_table, seq_lens, q_scale,
                                     out, &d, &pg);
  if (st != GQA_OK) return st;
  return decode_checked(&d, q, kv_pages, kv_scales, seq_lens, q_scale, out, pg, stream);
}

GQA_API gqa_status_t gqa_kv_append(const gqa_desc_t* desc, const void* k_new, const void* v_new,
                                   const int32_t* positions, void* kv, hipStream_t stream) {
  return append_contiguous(desc, k_new, v_new, positions, kv, nullptr, false, stream);
}

GQA_API gqa_status_t gqa_kv_append_int8(const gqa_desc_t* desc, const void* k_new,
                                        const void* v_new, const int32_t* positions, void* kv,
                                        void* kv_scales, hipStream_t stream) {
  return append_contiguous(desc, k_new, v_new, positions, kv, kv_scales, true, stream);
}

GQA_API gqa_status_t gqa_kv_append_paged(const gqa_paged_desc_t* desc, const void* k_new,
                                         const void* v_new, const int32_t* positions,
                                         const int32_t* block_table, void* kv_pages,
                                         hipStream_t stream) {
  return append_paged(desc, k_new, v_new, positions, block_table, kv_pages, nullptr, false, stream);
}

GQA_API gqa_status_t gqa_kv_append_paged_int8(const gqa_paged_desc_t* desc, const void* k_new,
                                              const void* v_new, const int32_t* positions,
                                              const int32_t* block_table, void* kv_pages,
                                              void* kv_scales, hipStream_t stream) {
  return append_paged(desc, k_new, v_new, positions, block_table, kv_pages, kv_scales, true,
                      stream);
}

}  // extern "C"
