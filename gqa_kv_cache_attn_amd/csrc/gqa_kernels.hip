// gfx950 kernels for single-token grouped-query decode attention.
//
// The step (FlashInfer sm110_gqa_decode article, "input contract" and
// "convenience API"): G = 4 query rows of one request share one KV head (or
// G = 2 in the 16-query-head geometry of the Orin Qwen3-VL doc's INT8-KV
// decode); scores are taken in the log2 domain, exp2(scale_log2 * s) with
// scale_log2 = q_scale / sqrt(128) / ln 2 (times k_scale for an fp8 cache,
// Thor FP8 KV notes, patch 2), and the output is the softmax-weighted sum of
// the V rows of the valid prefix, times v_scale. An INT8 cache carries one
// bf16 scale per (position, KV head) row (Orin Qwen3-VL doc, "INT8 KV
// cache"): the K row scale multiplies that token's score, the V row scale
// its weight in the PV product.
//
// Routes (the tile step, loads and merges they share are in gqa_device.h):
//   * chunked split (gqa_attention_kernel): a workgroup of 4 waves owns one
//     chunk of `chunk_tokens` slots of one (request, KV head); one chunk per
//     head normalises and writes the output in place (the short route is the
//     one-chunk case), several write FP32 (m, l, O) partials -- the split-KV
//     scheme of the article's "default routes and num_splits" section -- that
//     gqa_combine_kernel merges per query head (or, opt-in, the head's last
//     workgroup merges them inside the attention kernel);
//   * balanced split (gqa_balanced_attention_kernel): a persistent grid
//     shares the step's 64-slot slabs across workgroups from the actual
//     lengths, weighted by how fast the hardware serves each workgroup;
//     heads a workgroup covers whole are written directly and the pieces of
//     the others merged by gqa_balanced_combine_kernel;
//   * KV append (gqa_kv_append_kernel): the cache write before a step, into
//     the contiguous cache or a page pool.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <map>
#include <mutex>
#include <type_traits>

#include "../../include/gqa_decode.h"
#include "gqa_device.h"
#include "gqa_kernels.h"

// Split workspace of gqa_decode_no_alloc: a device array of fixed size in the
// library's own code object, so that entry point never allocates. Each GPU
// the library runs on holds its own copy until the process ends. In host
// code `scratch` names a host-side stand-in, not device memory: only the
// per-device address from hipGetSymbolAddress (gqa::no_alloc_scratch) is
// ever passed to a kernel.
static __device__ __align__(256) unsigned char scratch[GQA_NO_ALLOC_SCRATCH_BYTES];

namespace gqa {
namespace {

// Merge of the chunked split for the G query heads of (request b, KV head g):
// wave r < G takes head G g + r. Only the chunks that start below the current
// length are read, so partials left by an earlier launch with longer lengths
// never enter the result.
template <int QT, int G, bool kCoherent = false>
__device__ __forceinline__ void combine_head_group(const StepArgs& a, int b, int g, int L) {
  using E = Elem<QT>;
  const int lane = threadIdx.x & 63;
  const int r = threadIdx.x >> 6;
  if (r >= G) return;
  const int S = a.num_splits;
  const size_t head = ((size_t)b * kKvHeads + g) * G + r;
  char* outp = static_cast<char*>(a.out) + (head * kHeadDim + 2 * lane) * 2;
  const int n = (L + a.chunk_tokens - 1) / a.chunk_tokens;
  if (n == 0) {
    E::store2(outp, 0.f, 0.f);
    return;
  }
  merge_rows<QT, kCoherent>(a, n, [&](int k) -> size_t { return head * (size_t)S + k; }, outp);
}

// One workgroup attends the G query rows of (request b, KV head g) over the
// cache slots [c0, c1) (c0 < c1 <= length). On return thread t holds, for
// row t / 64 (meaningful for rows < G) and dims 2 (t % 64) + {0, 1}: the
// chunk's log2-domain max M, its sum of weights l and its unnormalised output
// (o0, o1). Ends with a barrier, so the caller may call it again for another
// range.
// kBlocks (INT8 cache only, for long ranges): waves take whole 64-slot
// blocks instead of every fourth tile; see the loop below.
template <int QT, int KVT, int G, bool kBlocks = false>
__device__ __forceinline__ void attend_range(const StepArgs& a, int b, int g, int c0, int c1,
                                             WorkgroupLds& lds, float& M, float& lsum, float& o0,
                                             float& o1) {
  constexpr int kRowBytes = kHeadDim * (kByteKv<KVT> ? 1 : 2);
  // (b, g, c0, c1) are the same in every lane. Stating it keeps the buffer
  // descriptors in scalar registers: one the compiler takes for divergent
  // costs a waterfall loop around every load.
  b = __builtin_amdgcn_readfirstlane(b);
  g = __builtin_amdgcn_readfirstlane(g);
  c0 = __builtin_amdgcn_readfirstlane(c0);
  c1 = __builtin_amdgcn_readfirstlane(c1);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int n16 = lane & 15;
  const int grp = lane >> 4;

  const char* kvb = static_cast<const char*>(a.kv);
  const size_t plane = (size_t)a.capacity * kRowBytes;
  const char* kplane = kvb + ((size_t)(b * 2 + 0) * kKvHeads + g) * plane;
  const char* vplane = kvb + ((size_t)(b * 2 + 1) * kKvHeads + g) * plane;
  Planes pl;
  pl.k = make_rsrc(kplane, (u32)c1 * kRowBytes);
  pl.v = make_rsrc(vplane, (u32)c1 * kRowBytes);
  pl.c1 = c1;
  pl.quads = (a.capacity & 3) == 0;
  if constexpr (KVT == kI8) {
    const char* sb = static_cast<const char*>(a.kv_scales);
    const size_t splane = (size_t)a.capacity * 2;
    pl.ks = make_rsrc(sb + ((size_t)(b * 2 + 0) * kKvHeads + g) * splane, (u32)c1 * 2);
    pl.vs = make_rsrc(sb + ((size_t)(b * 2 + 1) * kKvHeads + g) * splane, (u32)c1 * 2);
  }

  // Query fragment: B operand of the QK product, row n16 (< G), dim block per
  // instruction as the K loads deliver it. Rows G..15 are zero.
  u32x4 qf[4];
  {
    const char* qrow = static_cast<const char*>(a.q) +
                       (((size_t)b * kKvHeads + g) * G + (n16 & (G - 1))) * (kHeadDim * 2);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(qrow + 16 * qk_dim_block<KVT>(i, grp));
      qf[i] = (n16 < G) ? v : (u32x4){0u, 0u, 0u, 0u};
    }
  }

  Softmax st;
  st.m = -INFINITY;
  st.l = 0.f;
#pragma unroll
  for (int c = 0; c < 8; ++c) st.o[c] = (f32x4){0.f, 0.f, 0.f, 0.f};

  if constexpr (KVT == kI8 && kBlocks) {
    // INT8: each wave takes whole 64-slot blocks (wave w the blocks at
    // c0 + 64 w + 256 k, four tiles each), so every 128-byte line of a scale
    // plane is read once, by one wave, with one load a block ahead. With the
    // waves' tiles interleaved, four waves read each line at different times
    // and, streamed, it was fetched again (1.8% more HBM bytes). Short ranges
    // (a chunk of one block) would leave three waves idle: they keep the
    // interleaved order.
    int base = __builtin_amdgcn_readfirstlane(c0 + 64 * wave);
    if (base < c1) {
      u32x4* sk = lds.k[wave];
      Tile<KVT> ta, tb;
      BlockScales sc = load_block_scales(pl, base, lane);
      load_tile<KVT, false>(ta, pl, base, lane);
      // One iteration per block; the next block's scales are requested with
      // its first tile's predecessor and handed over after the block's last
      // tile, so waiting for them never holds up a tile.
      for (;;) {
        load_tile<KVT, false>(tb, pl, base + kTile, lane);        // past c1: reads 0
        const BlockScales sc_next = load_block_scales(pl, base + 4 * kStep, lane);
        tile_scales(ta, sc, 0, lane);
        process_tile<QT, KVT, G>(st, ta, qf, sk, base, c1, lane, a.scale_log2);
        if (base + kTile >= c1) break;
        load_tile<KVT, false>(ta, pl, base + 2 * kTile, lane);
        tile_scales(tb, sc, 1, lane);
        process_tile<QT, KVT, G>(st, tb, qf, sk, base + kTile, c1, lane, a.scale_log2);
        if (base + 2 * kTile >= c1) break;
        load_tile<KVT, false>(tb, pl, base + 3 * kTile, lane);
        tile_scales(ta, sc, 2, lane);
        process_tile<QT, KVT, G>(st, ta, qf, sk, base + 2 * kTile, c1, lane, a.scale_log2);
        if (base + 3 * kTile >= c1) break;
        load_tile<KVT, false>(ta, pl, base + 4 * kStep, lane);    // the next block's first tile
        tile_scales(tb, sc, 3, lane);
        process_tile<QT, KVT, G>(st, tb, qf, sk, base + 3 * kTile, c1, lane, a.scale_log2);
        base += 4 * kStep;
        if (base >= c1) break;
        sc = sc_next;
      }
    }
  } else {
    int j0 = c0 + kTile * wave;
    if (j0 < c1) {
      u32x4* sk = lds.k[wave];
      Tile<KVT> ta, tb;
      load_tile<KVT>(ta, pl, j0, lane);
      for (;;) {
        load_tile<KVT>(tb, pl, j0 + kStep, lane);   // past c1: reads 0, no traffic
        process_tile<QT, KVT, G>(st, ta, qf, sk, j0, c1, lane, a.scale_log2);
        j0 += kStep;
        if (j0 >= c1) break;
        load_tile<KVT>(ta, pl, j0 + kStep, lane);
        process_tile<QT, KVT, G>(st, tb, qf, sk, j0, c1, lane, a.scale_log2);
        j0 += kStep;
        if (j0 >= c1) break;
      }
    }
  }

  // ---- merge the 4 waves ----------------------------------------------------
  float l = st.l;
  l += __shfl_xor(l, 16);
  l += __shfl_xor(l, 32);
  if (lane < kGroup) {
    lds.m[wave][lane] = st.m;
    lds.l[wave][lane] = l;
  }
  if (grp == 0) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float4* dst = reinterpret_cast<float4*>(&lds.o[wave][r][8 * n16]);
      dst[0] = make_float4(st.o[0][r], st.o[1][r], st.o[2][r], st.o[3][r]);
      dst[1] = make_float4(st.o[4][r], st.o[5][r], st.o[6][r], st.o[7][r]);
    }
  }
  __syncthreads();
  const int er = tid >> 6;
  const int ed = (tid & 63) * 2;
  M = lds.m[0][er];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) M = fmaxf(M, lds.m[w][er]);
  o0 = 0.f;
  o1 = 0.f;
  lsum = 0.f;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    const float f = fast_exp2(lds.m[w][er] - M);  // idle waves: m = -inf -> 0
    o0 += f * lds.o[w][er][ed];
    o1 += f * lds.o[w][er][ed + 1];
    lsum += f * lds.l[w][er];
  }
  __syncthreads();
}

// Chunked split: workgroup = one chunk of `chunk_tokens` slots of one
// (request, KV head); grid B * 8 * num_splits.
template <int QT, int KVT, int G, int kMode>
__global__ __launch_bounds__(kThreads, GQA_MIN_WAVES_PER_SIMD) void gqa_attention_kernel(StepArgs a) {
  using E = Elem<QT>;
  __shared__ WorkgroupLds lds;
  __shared__ int s_last;

  const int tid = threadIdx.x;
  const int S = a.num_splits;
  const int split = (int)blockIdx.x % S;
  const int bg = (int)blockIdx.x / S;
  const int g = bg % kKvHeads;
  const int b = bg / kKvHeads;
  const int L = min(max(a.seq_lens[b], 0), a.capacity);
  const int c0 = split * a.chunk_tokens;

  // Epilogue coordinates: 256 threads cover 4 rows x 64 dim pairs; rows < G
  // are query heads G g + er.
  const int er = tid >> 6;
  const int ed = (tid & 63) * 2;
  const size_t head = ((size_t)b * kKvHeads + g) * G + er;

  if (c0 >= L) {
    // Chunks past the length take no part. An empty request (L = 0) has no
    // chunk at all: unless a combine kernel follows, chunk 0 writes its zeros.
    if (kMode != kModeSplit && split == 0 && er < G)
      E::store2(static_cast<char*>(a.out) + (head * kHeadDim + ed) * 2, 0.f, 0.f);
    return;
  }
  const int c1 = min(c0 + a.chunk_tokens, L);
  float M, lsum, o0, o1;
  attend_range<QT, KVT, G>(a, b, g, c0, c1, lds, M, lsum, o0, o1);

  if constexpr (kMode == kModeDirect) {
    const float inv = a.v_scale / lsum;
    if (er < G)
      E::store2(static_cast<char*>(a.out) + (head * kHeadDim + ed) * 2, o0 * inv, o1 * inv);
  } else {
    // With the one-launch merge another workgroup of this launch reads the
    // partial: device-coherent stores (store_partial).
    constexpr bool kShared = kMode == kModeSplitFused;
    const size_t slot = head * (size_t)S + split;
    if (er < G) {
      store_partial<kShared>(reinterpret_cast<float2*>(a.part_o + slot * kHeadDim + ed),
                             make_float2(o0, o1));
      if ((tid & 63) == 0)
        store_partial<kShared>(reinterpret_cast<float2*>(a.part_ml + slot * 2),
                               make_float2(M, lsum));
    }
    if constexpr (kMode == kModeSplitFused) {
      // Count this chunk; the head's last chunk merges all of them.
      const unsigned n_valid = (unsigned)((L + a.chunk_tokens - 1) / a.chunk_tokens);
      if (!publish_piece(a.counters + bg, 1u, n_valid, &s_last)) return;
      combine_head_group<QT, G, true>(a, b, g, L);
    }
  }
}

// Separate log-sum-exp combine for the chunked split: one workgroup per
// (request, KV head).
template <int QT, int G>
__global__ __launch_bounds__(kThreads) void gqa_combine_kernel(StepArgs a) {
  const int bg = blockIdx.x;
  const int b = bg / kKvHeads;
  const int L = min(max(a.seq_lens[b], 0), a.capacity);
  combine_head_group<QT, G>(a, b, bg % kKvHeads, L);
}

// ---------------------------------------------------------------------------
// Balanced split. The work of a step is N = 8 * sum_b ceil(L_b / 64) slabs
// of 64 slots, ordered request-major then KV head. A persistent grid of W
// workgroups (all resident at once: balanced_wgs_per_cu per CU) gives
// workgroup w the slab range [bound(w), bound(w + 1)), bound(w) = N S(w) /
// S(W) with S(w) the summed shares of workgroups 0 .. w-1, so each workgroup
// streams a share of the bytes matched to how fast the hardware serves it,
// whatever the length mix. A range crosses (request, KV head)
// boundaries: heads it covers whole are normalised and written directly; its
// first and last piece, when they are only part of a head, become partials
// in slots 2w and 2w + 1, which the balanced combine merges per head.
// ---------------------------------------------------------------------------
// Partial rows of the balanced split: slot k holds kGroup rows (rows >= G
// unused), so the slot stride does not depend on the geometry.
//
// The balanced-split range of workgroup u: slabs [s0, s1) (s0 < s1), in
// pieces of one (request, KV head) each. Heads covered whole are written
// directly; the first and last piece, when only part of a head, go to slots
// 2u and 2u + 1.
template <int QT, int KVT, int G>
__device__ __forceinline__ void balanced_unit(const StepArgs& a, const int* s_pref, int s0, int s1,
                                              int u, WorkgroupLds& lds) {
  using E = Elem<QT>;
  const int tid = threadIdx.x;
  const int B = a.batch;
  const int er = tid >> 6;
  const int ed = (tid & 63) * 2;
#pragma nounroll
  for (int s = s0; s < s1;) {
    // request b with pref[b] <= s < pref[b + 1]
    int lo = 0, hi = B;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (s_pref[mid] <= s) lo = mid; else hi = mid;
    }
    const int b = __builtin_amdgcn_readfirstlane(lo);
    const int pref_b = __builtin_amdgcn_readfirstlane(s_pref[b]);
    const int nsb = (__builtin_amdgcn_readfirstlane(s_pref[b + 1]) - pref_b) / kKvHeads;   // >= 1
    const int g = (s - pref_b) / nsb;
    const int seg_start = pref_b + g * nsb;
    const int seg_end = seg_start + nsb;
    const int pe = min(s1, seg_end);
    const int L = min(max(__builtin_amdgcn_readfirstlane(a.seq_lens[b]), 0), a.capacity);
    const int c0 = (s - seg_start) * kSlab;
    const int c1 = min((pe - seg_start) * kSlab, L);
    float M, lsum, o0, o1;
    attend_range<QT, KVT, G, KVT == kI8>(a, b, g, c0, c1, lds, M, lsum, o0, o1);
    const size_t head = ((size_t)b * kKvHeads + g) * G + er;
    const bool whole = s == seg_start && pe == seg_end;
    const size_t slot = 2 * (size_t)u + (s == s0 ? 0 : 1);
    record_piece(a, b * kKvHeads + g, whole, s == seg_start, pe == seg_end, slot, u);
    if (whole) {
      const float inv = a.v_scale / lsum;
      if (er < G)
        E::store2(static_cast<char*>(a.out) + (head * kHeadDim + ed) * 2, o0 * inv, o1 * inv);
    } else {
      const size_t row = slot * kGroup + er;
      *reinterpret_cast<float2*>(a.part_o + row * kHeadDim + ed) = make_float2(o0, o1);
      if ((tid & 63) == 0) *reinterpret_cast<float2*>(a.part_ml + row * 2) = make_float2(M, lsum);
    }
    s = pe;
  }
}

template <int QT, int KVT, int G>
__global__ __launch_bounds__(kThreads, GQA_BALANCED_MIN_WAVES_PER_SIMD) void gqa_balanced_attention_kernel(
    StepArgs a) {
  __shared__ WorkgroupLds lds;
  __shared__ int s_pref[kMaxBalancedBatch + 1];
  __shared__ int s_wave_tot[kWaves];

  const int tid = threadIdx.x;
  const int B = a.batch;
  build_slab_prefix(a, s_pref, s_wave_tot);
  // Values read from LDS are the same in every lane; saying so keeps the
  // loop control in scalar registers. Slab counts fit in int32 (checked when
  // the plan is made).
  const int N = __builtin_amdgcn_readfirstlane(s_pref[B]);
  const int W = (int)gridDim.x;
  const int w = (int)blockIdx.x;
  if (w == 0)   // the combine kernel reads the same prefix
    for (int i = tid; i <= B; i += kThreads) a.slab_prefix[i] = s_pref[i];

  const int64_t total = share_prefix(a, W);
  const int s0 = balanced_bound(a, w, N, total);
  const int s1 = balanced_bound(a, w + 1, N, total);
  if (s0 == s1) {
    // Fewer slabs than workgroups: mark slot 2w empty for the combine, which
    // may look at it when this workgroup falls inside a head's range of workgroups.
    const int er = tid >> 6;
    if ((tid & 63) == 0)
      *reinterpret_cast<float2*>(a.part_ml + ((size_t)2 * w * kGroup + er) * 2) =
          make_float2(-INFINITY, 0.f);
    return;
  }
  balanced_unit<QT, KVT, G>(a, s_pref, s0, s1, w, lds);
}

// Merge of the balanced split, one workgroup per (request, KV head); wave
// r < G takes query head G g + r. Heads that one workgroup covered whole were
// written by it; empty heads get zeros.
template <int QT, int G>
__global__ __launch_bounds__(kThreads) void gqa_balanced_combine_kernel(StepArgs a) {
  using E = Elem<QT>;
  const int bg = blockIdx.x;
  const int b = bg / kKvHeads;
  const int g = bg % kKvHeads;
  const int lane = threadIdx.x & 63;
  const int r = threadIdx.x >> 6;
  if (r >= G) return;
  const size_t head = ((size_t)b * kKvHeads + g) * G + r;
  char* outp = static_cast<char*>(a.out) + (head * kHeadDim + 2 * lane) * 2;
  // Where the attention kernel put the head's pieces: the first piece's slot
  // (-1: written whole) and the workgroup of the last piece. The workgroups
  // in between hold the head in their first slot (or, with no slab, mark it
  // empty). The empty asm takes the four values at once, so their loads
  // issue together instead of one after another behind the branches below.
  int first_slot = a.head_pieces[bg];
  int wl = a.head_pieces[a.batch * kKvHeads + bg];
  int p0 = a.slab_prefix[b], p1 = a.slab_prefix[b + 1];
  asm volatile("" : "+s"(first_slot), "+s"(wl), "+s"(p0), "+s"(p1));
  const int nsb = (p1 - p0) / kKvHeads;
  if (nsb == 0) {
    E::store2(outp, 0.f, 0.f);
    return;
  }
  if (first_slot < 0) return;
  const int wf = first_slot >> 1;
  merge_rows<QT>(a, wl - wf + 1,
                 [&](int k) -> size_t {
                   return (k == 0 ? (size_t)first_slot : 2 * (size_t)(wf + k)) * kGroup + r;
                 },
                 outp);
}

template <int QT, int KVT, int G>
hipError_t enqueue_typed(const StepArgs& a, hipStream_t stream, hipEvent_t ev_mid) {
  hipError_t e;
  if (a.grid_wgs > 0) {   // balanced split
    hipLaunchKernelGGL((gqa_balanced_attention_kernel<QT, KVT, G>), dim3(a.grid_wgs), dim3(kThreads),
                       0, stream, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (ev_mid != nullptr && (e = hipEventRecord(ev_mid, stream)) != hipSuccess) return e;
    hipLaunchKernelGGL((gqa_balanced_combine_kernel<QT, G>), dim3((unsigned)a.batch * kKvHeads),
                       dim3(kThreads), 0, stream, a);
    return hipGetLastError();
  }
  const unsigned wgs = (unsigned)a.batch * kKvHeads * (unsigned)a.num_splits;
  const bool separate = a.num_splits > 1 && !a.fused_combine;
  if (a.num_splits == 1) {
    hipLaunchKernelGGL((gqa_attention_kernel<QT, KVT, G, kModeDirect>), dim3(wgs), dim3(kThreads), 0,
                       stream, a);
  } else if (separate) {
    hipLaunchKernelGGL((gqa_attention_kernel<QT, KVT, G, kModeSplit>), dim3(wgs), dim3(kThreads), 0,
                       stream, a);
  } else {
    hipLaunchKernelGGL((gqa_attention_kernel<QT, KVT, G, kModeSplitFused>), dim3(wgs),
                       dim3(kThreads), 0, stream, a);
  }
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (ev_mid != nullptr && (e = hipEventRecord(ev_mid, stream)) != hipSuccess) return e;
  if (!separate) return hipSuccess;
  hipLaunchKernelGGL((gqa_combine_kernel<QT, G>), dim3((unsigned)a.batch * kKvHeads), dim3(kThreads),
                     0, stream, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// KV append: write the K and V rows of every KV head of T new tokens per
// request at slots positions[b] + t (the cache write that precedes each
// decode step; T > 1 for the draft tokens a verify pass attends), into the
// contiguous cache or through the block table into a page pool. An fp8
// cache stores e4m3(x / scale), per-tensor scales as in the Thor FP8-KV
// notes; the division is an IEEE fp32 division and the code the nearest
// E4M3FN value (ties to even), saturating at +-448. An INT8 cache (the Orin
// Qwen3-VL doc's INT8 mirrors, one bf16 scale per (position, KV head) row)
// stores each row symmetrically, as that doc quantises its INT8 weights:
// y = x / scale, row scale s = bf16(max|y| / 127), code = the integer nearest
// to y / s (ties to even) clamped to +-127, all in fp32 (0 where s is 0).
// ---------------------------------------------------------------------------
// fp32 -> bf16 bits, nearest with ties to even (finite and infinite inputs):
// add just under half of the kept unit, plus one if the kept part is odd.
__device__ __forceinline__ u32 f32_to_bf16_rne(float x) {
  const u32 b = __float_as_uint(x);
  return (b + 0x7fffu + ((b >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ u32 f32_to_e4m3fn_sat(float x) {
  const u32 bits = __float_as_uint(x);
  const u32 sign = (bits >> 24) & 0x80u;
  const u32 mag = bits & 0x7fffffffu;
  if (mag > 0x7f800000u) return 0x7fu;           // NaN
  if (mag >= 0x43e00000u) return sign | 0x7eu;   // |x| >= 448, infinities included
  if (mag < 0x3c800000u) {                       // |x| < 2^-6: codes m * 2^-9, m = 0..8
    const float v = __uint_as_float(mag) * 512.0f;   // exact
    return sign | (u32)__builtin_rintf(v);            // round half to even
  }
  u32 e = (mag >> 23) - 120u;                    // exponent field 1..15
  u32 q = (mag >> 20) & 7u;                      // top 3 mantissa bits
  const u32 rest = mag & 0xfffffu;
  if (rest > 0x80000u || (rest == 0x80000u && (q & 1u))) ++q;
  if (q == 8u) {
    q = 0u;
    ++e;
  }
  return sign | (e << 3) | q;
}

template <int QT, int KVT>
__global__ __launch_bounds__(256) void gqa_kv_append_kernel(AppendArgs a) {
  using E = Elem<QT>;
  // One thread per 8 dims of one (request, new token, plane, KV head) row:
  // the 256 threads of a workgroup write the 16 rows of one new token.
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int T = a.tokens;
  if (t >= (int64_t)a.batch * T * 2 * kKvHeads * (kHeadDim / 8)) return;
  const int chunk = (int)(t % (kHeadDim / 8));
  const int64_t row = t / (kHeadDim / 8);
  const int g = (int)(row % kKvHeads);
  const int plane = (int)((row / kKvHeads) % 2);
  const int64_t bt = row / (2 * kKvHeads);   // request * T + token
  const int token = (int)(bt % T);
  const int b = (int)(bt / T);
  const int64_t pos = (int64_t)a.positions[b] + token;
  if (pos < 0 || pos >= a.capacity) return;
  size_t dst_row;   // destination row, in rows of 128 values
  if (a.block_table == nullptr) {
    dst_row = ((size_t)(b * 2 + plane) * kKvHeads + g) * (size_t)a.capacity + (size_t)pos;
  } else {
    const int page = a.block_table[(size_t)b * a.max_pages + (size_t)(pos >> a.page_shift)];
    if (page < 0 || page >= a.num_pages) return;
    dst_row = ((((size_t)page * 2 + plane) * kKvHeads + g) << a.page_shift) +
              (size_t)(pos & ((1 << a.page_shift) - 1));
  }
  const char* src = static_cast<const char*>(plane ? a.v_new : a.k_new) +
                    ((bt * kKvHeads + g) * kHeadDim + chunk * 8) * 2;
  const u32x4 in = *reinterpret_cast<const u32x4*>(src);
  const size_t dst = dst_row * kHeadDim + chunk * 8;
  if constexpr (KVT == kFP8) {
    const float scale = plane ? a.v_scale : a.k_scale;
    u32 w[2] = {0u, 0u};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float x = (i & 1) ? E::hi(in[i >> 1]) : E::lo(in[i >> 1]);
      w[i >> 2] |= f32_to_e4m3fn_sat(__fdiv_rn(x, scale)) << (8 * (i & 3));
    }
    *reinterpret_cast<u32x2*>(static_cast<char*>(a.kv) + dst) = (u32x2){w[0], w[1]};
  } else if constexpr (KVT == kI8) {
    const float scale = plane ? a.v_scale : a.k_scale;
    float y[8];
    float m = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      y[i] = __fdiv_rn((i & 1) ? E::hi(in[i >> 1]) : E::lo(in[i >> 1]), scale);
      m = fmaxf(m, fabsf(y[i]));
    }
    // The 16 threads of a row are lanes 16k .. 16k + 15 of one wave, and a
    // row's threads leave early only together (slot and page are per row).
#pragma unroll
    for (int o = 8; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
    const u32 sb = f32_to_bf16_rne(__fdiv_rn(m, 127.f));
    const float s = __uint_as_float(sb << 16);
    u32 w[2] = {0u, 0u};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float q = s > 0.f ? fminf(fmaxf(__builtin_rintf(__fdiv_rn(y[i], s)), -127.f), 127.f)
                              : 0.f;
      w[i >> 2] |= ((u32)(int)q & 0xffu) << (8 * (i & 3));
    }
    *reinterpret_cast<u32x2*>(static_cast<char*>(a.kv) + dst) = (u32x2){w[0], w[1]};
    if (chunk == 0) {
      const size_t scale_row =
          a.scales_by_position
              ? ((size_t)(b * 2 + plane) * kKvHeads + g) * (size_t)a.capacity + (size_t)pos
              : dst_row;
      static_cast<uint16_t*>(a.kv_scales)[scale_row] = (uint16_t)sb;
    }
  } else {
    *reinterpret_cast<u32x4*>(static_cast<char*>(a.kv) + dst * 2) = in;
  }
}

template <int QT, int KVT>
hipError_t enqueue_append_typed(const AppendArgs& a, hipStream_t stream) {
  // 256 threads per new token (2 planes x 8 heads x 16 chunks): one workgroup each
  const unsigned blocks = (unsigned)((int64_t)a.batch * a.tokens);
  hipLaunchKernelGGL((gqa_kv_append_kernel<QT, KVT>), dim3(blocks), dim3(256), 0, stream, a);
  return hipGetLastError();
}

template <int QT, int KVT, int G>
int balanced_grid_typed() {
  int dev = 0, cus = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
          &per_cu, reinterpret_cast<const void*>(&gqa_balanced_attention_kernel<QT, KVT, G>),
          kThreads, 0) != hipSuccess)
    return 0;
  if (balanced_wgs_per_cu<KVT>() > 0) per_cu = std::min(per_cu, balanced_wgs_per_cu<KVT>());
  return cus * per_cu;
}

}  // namespace

hipError_t no_alloc_scratch(int dev, void** ptr) {
  static std::mutex mu;
  static std::map<int, void*> addr;
  std::lock_guard<std::mutex> lk(mu);
  auto it = addr.find(dev);
  if (it == addr.end()) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) {
      (void)hipGetLastError();
      return e;
    }
    if (p == nullptr) return hipErrorInvalidSymbol;
    it = addr.emplace(dev, p).first;
  }
  *ptr = it->second;
  return hipSuccess;
}

int balanced_grid_size(int q_dtype, int kv_dtype, int num_q_heads) {
  return dispatch(q_dtype, kv_dtype, num_q_heads, 0,
                  []<int QT, int KVT, int G>() { return balanced_grid_typed<QT, KVT, G>(); });
}

hipError_t enqueue_kv_append(const AppendArgs& a, int src_dtype, int kv_dtype, hipStream_t stream) {
  if (src_dtype == kBF16 && kv_dtype == kBF16) return enqueue_append_typed<kBF16, kBF16>(a, stream);
  if (src_dtype == kF16 && kv_dtype == kF16) return enqueue_append_typed<kF16, kF16>(a, stream);
  if (src_dtype == kBF16 && kv_dtype == kFP8) return enqueue_append_typed<kBF16, kFP8>(a, stream);
  if (src_dtype == kF16 && kv_dtype == kFP8) return enqueue_append_typed<kF16, kFP8>(a, stream);
  if (a.kv_scales != nullptr && src_dtype == kBF16 && kv_dtype == kI8)
    return enqueue_append_typed<kBF16, kI8>(a, stream);
  if (a.kv_scales != nullptr && src_dtype == kF16 && kv_dtype == kI8)
    return enqueue_append_typed<kF16, kI8>(a, stream);
  return hipErrorInvalidValue;
}

hipError_t enqueue_decode_step(const StepArgs& a, int q_dtype, int kv_dtype, hipStream_t stream,
                               hipEvent_t ev_mid) {
  return dispatch(q_dtype, kv_dtype, a.num_q_heads, hipErrorInvalidValue,
                  [&]<int QT, int KVT, int G>() { return enqueue_typed<QT, KVT, G>(a, stream, ev_mid); });
}

}  // namespace gqa
