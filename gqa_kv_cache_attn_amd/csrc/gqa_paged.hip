// gfx950 kernels for decode over a paged KV cache with T query tokens per
// request (the verify pass of speculative decoding).
//
// Cache. A pool of pages [num_pages, 2, 8, page_size, 128]: every page holds
// the same [2, 8, slots, 128] block as the contiguous cache (FlashInfer
// sm110_gqa_decode article, "input contract"), and an int32 block table
// [batch, max_pages] maps request b's slot j to row j % page_size of page
// block_table[b][j / page_size]. The pages name a paged-KV decode backend
// (FreeToken Turing notes, change 2) without a layout; this one is the
// library's reading. An INT8 pool carries its bf16 row scales as
// [num_pages, 2, 8, page_size] (Orin Qwen3-VL doc, "INT8 KV cache"), or,
// indexed by position, as [batch, 2, 8, max_pages * page_size].
//
// Queries. q and out are [batch, T, Hq, 128]: the T tokens are the last T of
// the request's L slots, and token t attends slots j < L - T + 1 + t, so the
// T tokens a draft model proposed are verified in one pass (Thor vLLM notes
// on MTP: K draft tokens per step, T = K + 1).
//
// The T tokens x G query heads of one (request, KV head) fill up to 16 rows
// of the MFMA operand (T <= 16 / G), so the verify pass streams each page
// once for all its tokens; each row masks the slots past its own causal
// limit. Page sizes are powers of two >= 16, so a 16-token tile never
// crosses a page: every tile gets its own buffer descriptors, bounded at the
// last slot of the range inside that page. Each wave keeps the page ids of
// its next 64 tiles in one register (lane i: tile i), loaded ahead of the
// tiles, and takes the current one with readlane, so no page lookup waits on
// memory inside the loop. Work split, partials and merges are those of the
// contiguous kernels, with 16 partial rows per (request, KV head) piece.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <type_traits>

#include "gqa_device.h"
#include "gqa_kernels.h"

namespace gqa {
namespace {

constexpr int kRowsMax = kPagedSlotRows;   // MFMA rows that may hold queries

// Build-time knob: minimum resident waves per SIMD the paged balanced kernel
// is compiled for (the register budget: 2 -> 256 VGPRs, 3 -> 168).
#ifndef GQA_PAGED_MIN_WAVES_PER_SIMD
#define GQA_PAGED_MIN_WAVES_PER_SIMD 2
#endif

// LDS of one workgroup: the waves' K staging slices, merge buffers for one
// group of 4 rows at a time, and the per-wave (m, l) of all 16 rows.
struct PagedLds {
  u32x4 k[kWaves][kKStageSlots];
  float o[kWaves][4][kHeadDim];
  float m[kWaves][kRowsMax];
  float l[kWaves][kRowsMax];
};

// Addressing of one (request, KV head) of the pool, for a range ending at c1.
template <int KVT>
struct PagedHead {
  const char* kv;
  const char* scales;
  const char* ks_pos;   // scales indexed by position: this (request, KV head)'s K and V
  const char* vs_pos;   // scale rows (null for the pool layout)
  const int32_t* table_row;
  int g, shift, num_pages, c1;

  // Descriptors of the tile at slot j0, which lies in page `page`; `row` is
  // j0's row in that page. They end at the range's last slot in the page (0
  // bytes when the page starts at or past c1: such a tile reads zeros and
  // touches no memory).
  __device__ __forceinline__ Planes planes(int j0, int page, int& row) const {
    constexpr int kRowBytes = kHeadDim * (kByteKv<KVT> ? 1 : 2);
    const int P = 1 << shift;
    const int page_start = j0 & ~(P - 1);
    const int nrows = max(0, min(c1 - page_start, P));
    row = j0 - page_start;
    const size_t plane = (size_t)P * kRowBytes;
    Planes pl;
    pl.k = make_rsrc(kv + ((size_t)(page * 2 + 0) * kKvHeads + g) * plane, (u32)nrows * kRowBytes);
    pl.v = make_rsrc(kv + ((size_t)(page * 2 + 1) * kKvHeads + g) * plane, (u32)nrows * kRowBytes);
    pl.c1 = nrows;
    pl.quads = true;   // pages hold multiples of 16 rows: scale quads are 8-byte aligned
    if constexpr (KVT == kI8) {
      if (ks_pos != nullptr) {   // by position: the page's slots in the request's scale rows
        pl.ks = make_rsrc(ks_pos + (size_t)page_start * 2, (u32)nrows * 2);
        pl.vs = make_rsrc(vs_pos + (size_t)page_start * 2, (u32)nrows * 2);
      } else {
        const size_t splane = (size_t)P * 2;
        pl.ks = make_rsrc(scales + ((size_t)(page * 2 + 0) * kKvHeads + g) * splane,
                          (u32)nrows * 2);
        pl.vs = make_rsrc(scales + ((size_t)(page * 2 + 1) * kKvHeads + g) * splane,
                          (u32)nrows * 2);
      }
    }
    return pl;
  }

  // Lane i: page id of the tile (or block) that starts at slot first +
  // stride i. Indices past the range's last page read that page (such tiles
  // read nothing); ids are clamped into the pool, so a bad table entry can
  // give a wrong result but never an access outside the pool.
  __device__ __forceinline__ int page_ids(int first, int last_index, int lane,
                                          int stride = kStep) const {
    const int idx = min((first + stride * lane) >> shift, last_index);
    return min(max(table_row[idx], 0), num_pages - 1);
  }
};

// The workgroup attends the T*G query rows of (request b, KV head g) over the
// slots [c0, c1) (c0 < c1 <= L). For every row group rg < ceil(T*G / 4),
// thread t calls emit(row = 4 rg + t / 64, M, l, o0, o1) with the range's
// log2-domain max, sum of weights and unnormalised output at dims
// 2 (t % 64) + {0, 1}; a row that saw no slot of the range gets M = -inf,
// l = 0. Rows >= T*G are passed too and must be ignored. Ends with a barrier.
//
// kBlocks (INT8 pools; the caller checks): each wave takes whole 64-slot
// blocks, as the contiguous balanced kernel does, so each 128-byte line of a
// scale plane is read once. 1: pages of at least 64 slots (a block lies in
// one page); 2: pages of 16 or 32 slots (a block spans 4 or 2 pages; the
// scale pool must fit 32-bit offsets); 3: scales indexed by position, any
// page size (a block's scales are 128 contiguous bytes per plane). 0: the
// waves take interleaved tiles.
template <int QT, int KVT, int G, int kBlocks = 0, class Emit>
__device__ __forceinline__ void attend_paged(const StepArgs& a, int b, int g, int c0, int c1,
                                             int L, PagedLds& lds, Emit&& emit) {
  b = __builtin_amdgcn_readfirstlane(b);
  g = __builtin_amdgcn_readfirstlane(g);
  c0 = __builtin_amdgcn_readfirstlane(c0);
  c1 = __builtin_amdgcn_readfirstlane(c1);
  L = __builtin_amdgcn_readfirstlane(L);
  constexpr int Hq = kKvHeads * G;
  int tid = threadIdx.x;
  if constexpr (KVT == kI8) {
    // Hide the thread index from the optimiser (an empty asm statement, no
    // instruction): otherwise the lane-derived addresses and constants of the
    // tile loop are hoisted out of the balanced kernel's loop over pieces and
    // stay live across it, 171-174 VGPRs instead of 155, which leaves room
    // for two workgroups per CU instead of the three INT8 needs.
    asm volatile("" : "+v"(tid));
  }
  const int lane = tid & 63;
  // Uniform per wave; saying so keeps each tile's descriptors (which depend on
  // the wave's slot) in scalar registers instead of a waterfall loop per load.
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n16 = lane & 15;
  const int grp = lane >> 4;
  const int T = a.q_tokens;
  const int R = T * G;

  PagedHead<KVT> ph;
  ph.kv = static_cast<const char*>(a.kv);
  ph.scales = static_cast<const char*>(a.kv_scales);
  ph.ks_pos = nullptr;
  ph.vs_pos = nullptr;
  if constexpr (KVT == kI8) {
    if (a.scales_by_position) {
      const size_t srow = (size_t)a.capacity * 2;
      ph.ks_pos = ph.scales + ((size_t)(b * 2 + 0) * kKvHeads + g) * srow;
      ph.vs_pos = ph.scales + ((size_t)(b * 2 + 1) * kKvHeads + g) * srow;
    }
  }
  ph.table_row = a.block_table + (size_t)b * a.max_pages;
  ph.g = g;
  ph.shift = a.page_shift;
  ph.num_pages = a.num_pages;
  ph.c1 = c1;

  // Row n16 is token n16 / G, query head G g + n16 % G; its causal limit.
  const int lim = n16 < R ? min(c1, L - T + 1 + n16 / G) : c1;
  u32x4 qf[4];
  {
    const int r = n16 < R ? n16 : 0;
    const char* qrow = static_cast<const char*>(a.q) +
                       (((size_t)b * T + r / G) * Hq + (size_t)g * G + r % G) * (kHeadDim * 2);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(qrow + 16 * qk_dim_block<KVT>(i, grp));
      qf[i] = (n16 < R) ? v : (u32x4){0u, 0u, 0u, 0u};
    }
  }

  Softmax st;
  st.m = -INFINITY;
  st.l = 0.f;
#pragma unroll
  for (int c = 0; c < 8; ++c) st.o[c] = (f32x4){0.f, 0.f, 0.f, 0.f};

  if constexpr (KVT == kI8 && (kBlocks == 2 || kBlocks == 3)) {
    // Whole 64-slot blocks over pages of any size: each of a block's four
    // tiles gets the descriptors of its own page, and the block's row scales
    // come from one 2-byte load per lane and plane. Pool layout (2, pages of
    // 16 or 32 slots): through a descriptor over the whole scale pool, at the
    // lane's page (slots at or past c1 get an offset past the pool: they read
    // 0). By position (3): through descriptors over the request's K and V
    // scale rows, bounded at c1. Page ids come from the table four per block
    // (its tiles' pages), sixteen blocks per load.
    int base = __builtin_amdgcn_readfirstlane(c0 + 64 * wave);
    if (base < c1) {
      u32x4* sk = lds.k[wave];
      const int last_index = (c1 - 1) >> ph.shift;
      const int P = 1 << ph.shift;
      constexpr int kBlock = 4 * kStep;              // slots between a wave's blocks
      const int base0 = base;
      // lane i: page of slot first + 256 (i / 4) + 16 (i % 4)
      auto tile_ids = [&](int first) -> int {
        const int idx = min((first + kBlock * (lane >> 2) + kTile * (lane & 3)) >> ph.shift,
                            last_index);
        return min(max(ph.table_row[idx], 0), ph.num_pages - 1);
      };
      int kb0 = 0;                                   // block held by lanes 0..3
      int ids = tile_ids(base0);
      __amdgpu_buffer_rsrc_t ks_src, vs_src;
      if constexpr (kBlocks == 3) {
        ks_src = make_rsrc(ph.ks_pos, (u32)c1 * 2);   // the K scale row, up to c1
        vs_src = make_rsrc(ph.vs_pos, (u32)c1 * 2);
      } else {
        const u32 pool_bytes = (u32)a.num_pages * (u32)(2 * kKvHeads * 2) * (u32)P;
        ks_src = make_rsrc(ph.scales, pool_bytes);
        vs_src = ks_src;
      }
      // Byte offset of the K scale of slot bbase + lane. Pool layout: the V
      // scale is one plane further on (+ 8 P 2 bytes), and slots at or past
      // c1 get an offset past the pool. By position: the slot's offset in
      // both rows (the descriptors end at c1).
      auto scale_offset = [&](int kb, int bbase) -> u32 {
        const int slot = bbase + lane;
        if constexpr (kBlocks == 3) {
          return (u32)slot * 2u;
        } else {
          const int page = __shfl(ids, 4 * (kb - kb0) + (lane >> 4));
          return slot < c1 ? (u32)page * (u32)(2 * kKvHeads * 2 * P) + (u32)(g * 2 * P) +
                                 (u32)((slot & (P - 1)) * 2)
                           : 0xffffffffu;
        }
      };
      auto load_scales = [&](u32 off) -> BlockScales {
        BlockScales r;
        r.k = __builtin_amdgcn_raw_buffer_load_b16(ks_src, off, 0, kLoadAux);
        if constexpr (kBlocks == 3) {
          r.v = __builtin_amdgcn_raw_buffer_load_b16(vs_src, off, 0, kLoadAux);
        } else {
          r.v = __builtin_amdgcn_raw_buffer_load_b16(
              ks_src, off == 0xffffffffu ? off : off + (u32)(kKvHeads * 2 * P), 0, kLoadAux);
        }
        return r;
      };
      int kb = 0, row;
      BlockQuads sc = pack_block_scales(load_scales(scale_offset(0, base)), lane);
      Tile<KVT> ta, tb;
      {
        const Planes p0 = ph.planes(base, __builtin_amdgcn_readlane(ids, 0), row);
        load_tile<KVT, false>(ta, p0, row, lane);
      }
      for (;;) {
        // this block's tile pages, read before the ids may move on
        const int o = 4 * (kb - kb0);
        const int pg1 = __builtin_amdgcn_readlane(ids, o + 1);
        const int pg2 = __builtin_amdgcn_readlane(ids, o + 2);
        const int pg3 = __builtin_amdgcn_readlane(ids, o + 3);
        if (kb + 1 - kb0 >= 16) {
          kb0 = kb + 1;
          ids = tile_ids(base0 + kBlock * kb0);
        }
        const int pgn = __builtin_amdgcn_readlane(ids, 4 * (kb + 1 - kb0));
        {
          const Planes p1 = ph.planes(base + kTile, pg1, row);
          load_tile<KVT, false>(tb, p1, row, lane);                 // past c1: reads 0
        }
        const BlockScales sc_next = load_scales(scale_offset(kb + 1, base + kBlock));
        tile_scales(ta, sc, 0, lane);
        process_tile<QT, KVT, kRowsMax>(st, ta, qf, sk, base, lim, lane, a.scale_log2);
        if (base + kTile >= c1) break;
        {
          const Planes p2 = ph.planes(base + 2 * kTile, pg2, row);
          load_tile<KVT, false>(ta, p2, row, lane);
        }
        tile_scales(tb, sc, 1, lane);
        process_tile<QT, KVT, kRowsMax>(st, tb, qf, sk, base + kTile, lim, lane, a.scale_log2);
        if (base + 2 * kTile >= c1) break;
        {
          const Planes p3 = ph.planes(base + 3 * kTile, pg3, row);
          load_tile<KVT, false>(tb, p3, row, lane);
        }
        tile_scales(ta, sc, 2, lane);
        process_tile<QT, KVT, kRowsMax>(st, ta, qf, sk, base + 2 * kTile, lim, lane,
                                        a.scale_log2);
        if (base + 3 * kTile >= c1) break;
        {
          const Planes pn = ph.planes(base + kBlock, pgn, row);   // the next block's first tile
          load_tile<KVT, false>(ta, pn, row, lane);
        }
        tile_scales(tb, sc, 3, lane);
        process_tile<QT, KVT, kRowsMax>(st, tb, qf, sk, base + 3 * kTile, lim, lane,
                                        a.scale_log2);
        base += kBlock;
        ++kb;
        if (base >= c1) break;
        sc = pack_block_scales(sc_next, lane);
      }
    }
  } else if constexpr (KVT == kI8 && kBlocks == 1) {
    // Whole 64-slot blocks, wave w the blocks at c0 + 64 w + 256 k; a block
    // lies in one page (ranges start on 64-slot boundaries), so it takes one
    // set of descriptors, and its scales one 2-byte load per lane and plane,
    // fetched a block ahead like its first tile.
    int base = __builtin_amdgcn_readfirstlane(c0 + 64 * wave);
    if (base < c1) {
      u32x4* sk = lds.k[wave];
      const int last_index = (c1 - 1) >> ph.shift;
      constexpr int kBlock = 4 * kStep;              // slots between a wave's blocks
      int kb0 = 0;                                   // block index held by lane 0
      int ids = ph.page_ids(base, last_index, lane, kBlock);
      const int base0 = base;
      auto page_of_block = [&](int kb) -> int {      // kb is uniform and never decreases
        if (kb - kb0 >= 64) {
          kb0 = kb;
          ids = ph.page_ids(base0 + kBlock * kb0, last_index, lane, kBlock);
        }
        return __builtin_amdgcn_readlane(ids, kb - kb0);
      };
      int kb = 0, row, row_next;
      Planes pl = ph.planes(base, page_of_block(0), row);
      BlockQuads sc = pack_block_scales(load_block_scales(pl, row, lane), lane);
      Tile<KVT> ta, tb;
      load_tile<KVT, false>(ta, pl, row, lane);
      for (;;) {
        const Planes pl_next = ph.planes(base + kBlock, page_of_block(kb + 1), row_next);
        load_tile<KVT, false>(tb, pl, row + kTile, lane);          // past c1: reads 0
        const BlockScales sc_next = load_block_scales(pl_next, row_next, lane);
        tile_scales(ta, sc, 0, lane);
        process_tile<QT, KVT, kRowsMax>(st, ta, qf, sk, base, lim, lane, a.scale_log2);
        if (base + kTile >= c1) break;
        load_tile<KVT, false>(ta, pl, row + 2 * kTile, lane);
        tile_scales(tb, sc, 1, lane);
        process_tile<QT, KVT, kRowsMax>(st, tb, qf, sk, base + kTile, lim, lane, a.scale_log2);
        if (base + 2 * kTile >= c1) break;
        load_tile<KVT, false>(tb, pl, row + 3 * kTile, lane);
        tile_scales(ta, sc, 2, lane);
        process_tile<QT, KVT, kRowsMax>(st, ta, qf, sk, base + 2 * kTile, lim, lane,
                                        a.scale_log2);
        if (base + 3 * kTile >= c1) break;
        load_tile<KVT, false>(ta, pl_next, row_next, lane);       // the next block's first tile
        tile_scales(tb, sc, 3, lane);
        process_tile<QT, KVT, kRowsMax>(st, tb, qf, sk, base + 3 * kTile, lim, lane,
                                        a.scale_log2);
        base += kBlock;
        ++kb;
        if (base >= c1) break;
        sc = pack_block_scales(sc_next, lane);
        pl = pl_next;
        row = row_next;
      }
    }
  } else {
    const int first = c0 + kTile * wave;   // this wave's tile k starts at first + 64 k
    if (first < c1) {
      u32x4* sk = lds.k[wave];
      const int last_index = (c1 - 1) >> ph.shift;
      int base = 0;                                      // tile index held by lane 0
      int ids = ph.page_ids(first, last_index, lane);
      auto page_of = [&](int k) -> int {                 // k is uniform and never decreases
        if (k - base >= 64) {
          base = k;
          ids = ph.page_ids(first + kStep * base, last_index, lane);
        }
        return __builtin_amdgcn_readlane(ids, k - base);
      };
      Tile<KVT> ta, tb;
      int row;
      int j0 = first;
      int k = 0;
      {
        const Planes pl = ph.planes(j0, page_of(0), row);
        load_tile<KVT>(ta, pl, row, lane);
      }
      for (;;) {
        {
          const Planes pl = ph.planes(j0 + kStep, page_of(k + 1), row);
          load_tile<KVT>(tb, pl, row, lane);
        }
        process_tile<QT, KVT, kRowsMax>(st, ta, qf, sk, j0, lim, lane, a.scale_log2);
        j0 += kStep;
        ++k;
        if (j0 >= c1) break;
        {
          const Planes pl = ph.planes(j0 + kStep, page_of(k + 1), row);
          load_tile<KVT>(ta, pl, row, lane);
        }
        process_tile<QT, KVT, kRowsMax>(st, tb, qf, sk, j0, lim, lane, a.scale_log2);
        j0 += kStep;
        ++k;
        if (j0 >= c1) break;
      }
    }
  }

  // ---- merge the 4 waves, one group of 4 rows at a time ---------------------
  float l = st.l;
  l += __shfl_xor(l, 16);
  l += __shfl_xor(l, 32);
  if (lane < kRowsMax) {
    lds.m[wave][lane] = st.m;
    lds.l[wave][lane] = l;
  }
  const int er = tid >> 6;
  const int ed = (tid & 63) * 2;
  const int groups = (R + 3) >> 2;
  for (int rg = 0; rg < groups; ++rg) {
    if (grp == rg) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float4* dst = reinterpret_cast<float4*>(&lds.o[wave][r][8 * n16]);
        dst[0] = make_float4(st.o[0][r], st.o[1][r], st.o[2][r], st.o[3][r]);
        dst[1] = make_float4(st.o[4][r], st.o[5][r], st.o[6][r], st.o[7][r]);
      }
    }
    __syncthreads();
    const int row = 4 * rg + er;
    float M = lds.m[0][row];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) M = fmaxf(M, lds.m[w][row]);
    float o0 = 0.f, o1 = 0.f, lsum = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float f = fast_exp2(lds.m[w][row] - M);   // waves that saw nothing: 0
        o0 += f * lds.o[w][er][ed];
        o1 += f * lds.o[w][er][ed + 1];
        lsum += f * lds.l[w][row];
      }
    }
    emit(row, M, lsum, o0, o1);
    __syncthreads();
  }
}

// Index of query row `row` (= t G + h) of (request b, KV head g) in q/out
// [batch, T, Hq, 128], counted in rows of 128.
template <int G>
__device__ __forceinline__ size_t query_row(int b, int g, int row, int T) {
  return ((size_t)b * T + row / G) * (kKvHeads * G) + (size_t)g * G + row % G;
}

// Zeros for every query row of (request b, KV head g): a request of length
// <= 0, or rows whose causal limit leaves no slot.
// Query rows of a head in the combine kernels: wave w of workgroup (head,
// y) takes rows 4 y + w, 4 y + w + 4 gridDim.y, ...; the launch gives each
// head ceil(T G / 4) workgroups, so every row has a wave of its own and the
// merges of a head's rows wait for their loads together.
__device__ __forceinline__ int first_row() { return (int)blockIdx.y * kWaves + (threadIdx.x >> 6); }
__device__ __forceinline__ int row_stride() { return (int)gridDim.y * kWaves; }

template <int QT, int G>
__device__ __forceinline__ void zero_rows(const StepArgs& a, int b, int g) {
  const int T = a.q_tokens;
  const int ed = (threadIdx.x & 63) * 2;
  for (int row = first_row(); row < T * G; row += row_stride())
    Elem<QT>::store2(static_cast<char*>(a.out) + (query_row<G>(b, g, row, T) * kHeadDim + ed) * 2,
                     0.f, 0.f);
}

// Chunked split: workgroup = one chunk of `chunk_tokens` slots of one
// (request, KV head); grid B * 8 * num_splits.
template <int QT, int KVT, int G, int kMode>
__global__ __launch_bounds__(kThreads, GQA_MIN_WAVES_PER_SIMD) void gqa_paged_attention_kernel(
    StepArgs a) {
  using E = Elem<QT>;
  __shared__ PagedLds lds;
  const int S = a.num_splits;
  const int split = (int)blockIdx.x % S;
  const int bg = (int)blockIdx.x / S;
  const int g = bg % kKvHeads;
  const int b = bg / kKvHeads;
  const int L = min(max(a.seq_lens[b], 0), a.capacity);
  const int c0 = split * a.chunk_tokens;
  const int T = a.q_tokens;
  const int R = T * G;
  if (c0 >= L) {
    if (kMode == kModeDirect && split == 0) zero_rows<QT, G>(a, b, g);
    return;
  }
  const int c1 = min(c0 + a.chunk_tokens, L);
  const int lane = threadIdx.x & 63;
  const int ed = lane * 2;
  attend_paged<QT, KVT, G>(a, b, g, c0, c1, L, lds,
                           [&](int row, float M, float lsum, float o0, float o1) {
    if (row >= R) return;
    const size_t qrow = query_row<G>(b, g, row, T);
    if constexpr (kMode == kModeDirect) {
      const float inv = lsum > 0.f ? a.v_scale / lsum : 0.f;   // 0: the row sees no slot
      E::store2(static_cast<char*>(a.out) + (qrow * kHeadDim + ed) * 2, o0 * inv, o1 * inv);
    } else {
      const size_t slot = qrow * (size_t)S + split;
      *reinterpret_cast<float2*>(a.part_o + slot * kHeadDim + ed) = make_float2(o0, o1);
      if (lane == 0) *reinterpret_cast<float2*>(a.part_ml + slot * 2) = make_float2(M, lsum);
    }
  });
}

// Causal limit of query row `row`: the slots [0, limit) it attends.
template <int G>
__device__ __forceinline__ int row_limit(int L, int T, int row) {
  return L - T + 1 + row / G;
}

// Log-sum-exp combine of the chunked split: one workgroup per (request, KV
// head); wave w merges rows w, w + 4, ... Only the chunks that start below a
// row's causal limit hold data for it (every one of them holds at least one
// of its slots), so only those are read.
template <int QT, int G>
__global__ __launch_bounds__(kThreads) void gqa_paged_combine_kernel(StepArgs a) {
  using E = Elem<QT>;
  const int bg = blockIdx.x;
  const int b = bg / kKvHeads;
  const int g = bg % kKvHeads;
  const int L = min(max(a.seq_lens[b], 0), a.capacity);
  const int T = a.q_tokens;
  const int lane = threadIdx.x & 63;
  const int S = a.num_splits;
  for (int row = first_row(); row < T * G; row += row_stride()) {
    const size_t qrow = query_row<G>(b, g, row, T);
    char* outp = static_cast<char*>(a.out) + (qrow * kHeadDim + 2 * lane) * 2;
    const int limit = min(row_limit<G>(L, T, row), L);
    if (limit <= 0) {
      E::store2(outp, 0.f, 0.f);
      continue;
    }
    const int n = (limit + a.chunk_tokens - 1) / a.chunk_tokens;
    merge_rows<QT>(a, n, [&](int k) -> size_t { return qrow * (size_t)S + k; }, outp);
  }
}

// Balanced split over the logical slots (the contiguous kernel's scheme):
// workgroup w takes slabs [bound(w), bound(w + 1)); heads covered whole are
// written directly, first and last pieces go to slots 2w and 2w + 1 of
// kRowsMax rows each. kBlocks: see attend_paged (INT8 pools: 1 for pages of
// at least 64 slots, 2 for pages of 16 or 32, 3 for scales indexed by
// position).
template <int QT, int KVT, int G, int kBlocks>
__global__ __launch_bounds__(kThreads, GQA_PAGED_MIN_WAVES_PER_SIMD) void
gqa_paged_balanced_kernel(StepArgs a) {
  using E = Elem<QT>;
  __shared__ PagedLds lds;
  __shared__ int s_pref[kMaxBalancedBatch + 1];
  __shared__ int s_wave_tot[kWaves];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int B = a.batch;
  const int T = a.q_tokens;
  const int R = T * G;
  build_slab_prefix(a, s_pref, s_wave_tot);
  const int64_t N = __builtin_amdgcn_readfirstlane(s_pref[B]);
  const int W = (int)gridDim.x;
  const int w = (int)blockIdx.x;
  if (w == 0)   // the combine kernel reads the same prefix
    for (int i = tid; i <= B; i += kThreads) a.slab_prefix[i] = s_pref[i];

  const int64_t total = share_prefix(a, W);
  const int s0 = balanced_bound(a, w, N, total);
  const int s1 = balanced_bound(a, w + 1, N, total);
  if (s0 == s1) {   // no slab: mark slot 2w empty for the combine
    if (tid < kRowsMax)
      *reinterpret_cast<float2*>(a.part_ml + ((size_t)2 * w * kRowsMax + tid) * 2) =
          make_float2(-INFINITY, 0.f);
    return;
  }
#pragma nounroll
  for (int s = s0; s < s1;) {
    int lo = 0, hi = B;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (s_pref[mid] <= s) lo = mid; else hi = mid;
    }
    const int b = __builtin_amdgcn_readfirstlane(lo);
    const int pref_b = __builtin_amdgcn_readfirstlane(s_pref[b]);
    const int nsb = (__builtin_amdgcn_readfirstlane(s_pref[b + 1]) - pref_b) / kKvHeads;
    const int g = (s - pref_b) / nsb;
    const int seg_start = pref_b + g * nsb;
    const int seg_end = seg_start + nsb;
    const int pe = min(s1, seg_end);
    const int L = min(max(__builtin_amdgcn_readfirstlane(a.seq_lens[b]), 0), a.capacity);
    const int c0 = (s - seg_start) * kSlab;
    const int c1 = min((pe - seg_start) * kSlab, L);
    const bool whole = s == seg_start && pe == seg_end;
    const size_t slot = 2 * (size_t)w + (s == s0 ? 0 : 1);
    record_piece(a, b * kKvHeads + g, whole, s == seg_start, pe == seg_end, slot, w);
    attend_paged<QT, KVT, G, kBlocks>(a, b, g, c0, c1, L, lds,
                                      [&](int row, float M, float lsum, float o0, float o1) {
      if (row >= R) return;
      int ed = lane * 2;
      if constexpr (kBlocks != 0) asm volatile("" : "+v"(ed));   // not hoisted across pieces
      if (whole) {
        const float inv = lsum > 0.f ? a.v_scale / lsum : 0.f;
        E::store2(static_cast<char*>(a.out) + (query_row<G>(b, g, row, T) * kHeadDim + ed) * 2,
                  o0 * inv, o1 * inv);
      } else {
        const size_t prow = slot * kRowsMax + row;
        *reinterpret_cast<float2*>(a.part_o + prow * kHeadDim + ed) = make_float2(o0, o1);
        if (lane == 0) *reinterpret_cast<float2*>(a.part_ml + prow * 2) = make_float2(M, lsum);
      }
    });
    s = pe;
  }
}

// Merge of the balanced split, one workgroup per (request, KV head); wave w
// merges rows w, w + 4, ... of the workgroups whose ranges cover the head.
template <int QT, int G>
__global__ __launch_bounds__(kThreads) void gqa_paged_balanced_combine_kernel(StepArgs a) {
  using E = Elem<QT>;
  const int bg = blockIdx.x;
  const int b = bg / kKvHeads;
  const int g = bg % kKvHeads;
  const int lane = threadIdx.x & 63;
  const int T = a.q_tokens;
  // The head's first-piece slot (-1: written whole) and last workgroup, as
  // the attention kernel recorded them. The empty asm takes them with the
  // length and the request's slab bounds at once, so the five loads issue
  // together instead of one after another behind the branches below.
  int first_slot = a.head_pieces[bg];
  int wl = a.head_pieces[a.batch * kKvHeads + bg];
  int len = a.seq_lens[b];
  int p0 = a.slab_prefix[b], p1 = a.slab_prefix[b + 1];
  asm volatile("" : "+s"(first_slot), "+s"(wl), "+s"(len), "+s"(p0), "+s"(p1));
  const int L = min(max(len, 0), a.capacity);
  const int nsb = (p1 - p0) / kKvHeads;
  if (nsb == 0) {
    zero_rows<QT, G>(a, b, g);
    return;
  }
  if (first_slot < 0) return;
  const int wf = first_slot >> 1;
  for (int row = first_row(); row < T * G; row += row_stride()) {
    char* outp = static_cast<char*>(a.out) + (query_row<G>(b, g, row, T) * kHeadDim + 2 * lane) * 2;
    if (row_limit<G>(L, T, row) <= 0) {   // sees no slot: every piece is empty
      E::store2(outp, 0.f, 0.f);
      continue;
    }
    merge_rows<QT>(a, wl - wf + 1,
                   [&](int k) -> size_t {
                     return (k == 0 ? (size_t)first_slot : 2 * (size_t)(wf + k)) * kRowsMax + row;
                   },
                   outp);
  }
}

template <int QT, int KVT, int G>
hipError_t enqueue_paged_typed(const StepArgs& a, hipStream_t stream, hipEvent_t ev_mid) {
  hipError_t e;
  // Combine grid: per head, one workgroup per 4 query rows (one wave a row).
  const dim3 heads((unsigned)a.batch * kKvHeads, (unsigned)((a.q_tokens * G + kWaves - 1) / kWaves));
  if (a.grid_wgs > 0) {
    // INT8 pools: whole 64-slot blocks per wave, within one page (pages of
    // 64+ slots) or across the pages of 16 or 32 slots a block spans, when
    // the scale pool's offsets fit 32 bits.
    int blocks = 0;
    if constexpr (KVT == kI8) {
      const int64_t scale_pool = (int64_t)a.num_pages * (2 * kKvHeads * 2) << a.page_shift;
      blocks = a.scales_by_position ? 3
               : a.page_shift >= 6  ? 1
                                    : (scale_pool < (int64_t)UINT32_MAX ? 2 : 0);
      if (blocks == 3)
        hipLaunchKernelGGL((gqa_paged_balanced_kernel<QT, KVT, G, 3>), dim3(a.grid_wgs),
                           dim3(kThreads), 0, stream, a);
      else if (blocks == 1)
        hipLaunchKernelGGL((gqa_paged_balanced_kernel<QT, KVT, G, 1>), dim3(a.grid_wgs),
                           dim3(kThreads), 0, stream, a);
      else if (blocks == 2)
        hipLaunchKernelGGL((gqa_paged_balanced_kernel<QT, KVT, G, 2>), dim3(a.grid_wgs),
                           dim3(kThreads), 0, stream, a);
    }
    if (blocks == 0)
      hipLaunchKernelGGL((gqa_paged_balanced_kernel<QT, KVT, G, 0>), dim3(a.grid_wgs),
                         dim3(kThreads), 0, stream, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (ev_mid != nullptr && (e = hipEventRecord(ev_mid, stream)) != hipSuccess) return e;
    hipLaunchKernelGGL((gqa_paged_balanced_combine_kernel<QT, G>), heads, dim3(kThreads), 0, stream,
                       a);
    return hipGetLastError();
  }
  const dim3 grid((unsigned)a.batch * kKvHeads * (unsigned)a.num_splits);
  if (a.num_splits == 1) {
    hipLaunchKernelGGL((gqa_paged_attention_kernel<QT, KVT, G, kModeDirect>), grid, dim3(kThreads), 0,
                       stream, a);
  } else {
    hipLaunchKernelGGL((gqa_paged_attention_kernel<QT, KVT, G, kModeSplit>), grid, dim3(kThreads), 0,
                       stream, a);
  }
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (ev_mid != nullptr && (e = hipEventRecord(ev_mid, stream)) != hipSuccess) return e;
  if (a.num_splits == 1) return hipSuccess;
  hipLaunchKernelGGL((gqa_paged_combine_kernel<QT, G>), heads, dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

template <int QT, int KVT, int G>
int paged_balanced_grid_typed() {
  int dev = 0, cus = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
          &per_cu, reinterpret_cast<const void*>(&gqa_paged_balanced_kernel<QT, KVT, G, 0>), kThreads,
          0) != hipSuccess)
    return 0;
  if (balanced_wgs_per_cu<KVT>() > 0) per_cu = std::min(per_cu, balanced_wgs_per_cu<KVT>());
  return cus * per_cu;
}

}  // namespace

int paged_balanced_grid_size(int q_dtype, int kv_dtype, int num_q_heads) {
  return dispatch(q_dtype, kv_dtype, num_q_heads, 0,
                  []<int QT, int KVT, int G>() { return paged_balanced_grid_typed<QT, KVT, G>(); });
}

hipError_t enqueue_paged_decode_step(const StepArgs& a, int q_dtype, int kv_dtype,
                                     hipStream_t stream, hipEvent_t ev_mid) {
  return dispatch(q_dtype, kv_dtype, a.num_q_heads, hipErrorInvalidValue,
                  [&]<int QT, int KVT, int G>() {
                    return enqueue_paged_typed<QT, KVT, G>(a, stream, ev_mid);
                  });
}

}  // namespace gqa
