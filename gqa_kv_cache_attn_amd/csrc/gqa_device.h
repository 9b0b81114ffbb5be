// Device building blocks shared by the decode kernels (gqa_kernels.hip: the
// contiguous cache; gqa_paged.hip: the paged cache with several query tokens
// per request): element traits of the MFMA operand types, whole-row tile
// loads through buffer descriptors, the per-tile step of the online softmax
// (QK^T and PV on the matrix cores), the log-sum-exp merge of partial rows,
// and the balanced split's bookkeeping. Included by the .hip sources only.
//
// Tile step. A wave takes 16 cache slots at a time. The query rows of one
// (request, KV head) -- G = 4 (or 2) grouped heads, times the query tokens of
// a paged call -- form the 16-column B operand (unused columns zero; the
// matrix cores have far more throughput than this stream needs):
//   scores^T[16 tok, 16 rows] = K_tile[16 tok, 128] x Q^T[128, 16]
//       4 x v_mfma_f32_16x16x32_{bf16,f16}; the coalesced loads deliver K
//       one row per 16 (or 8) lanes, so each wave passes its K tile through a
//       private, XOR-swizzled LDS slice to get one token per lane;
//   O[16 rows, 128]           += P[16 rows, 16 tok] x V_tile[16 tok, 128]
//       8 x v_mfma_f32_16x16x16_{bf16,f16} (16 with the bf16 hi + lo weight
//       split); the score accumulator already is the P operand layout, and
//       byte permutes turn the V load layout into the B operand.
// fp8 e4m3 and int8 bytes are widened exactly in registers (fp8 with the
// gfx950 packed converts), so the cache is read once, at 1 byte per element.
// The online softmax runs in fp32 in the log2 domain. Loads are raw buffer
// loads whose range ends at the range's last valid slot: slots past a length
// read as 0 without touching memory, which also makes the one-tile-ahead
// prefetch free at the end of a range.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "gqa_kernels.h"

namespace gqa {
namespace {

constexpr int kHeadDim = 128;
constexpr int kKvHeads = 8;
constexpr int kGroup = 4;               // MFMA rows carried per KV head (G <= 4 are real)
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kTile = 16;               // tokens per wave step
constexpr int kStep = kTile * kWaves;   // tokens per workgroup step
constexpr int kSlab = kStep;            // unit of work of the balanced split
constexpr uint32_t kRsrcWord3 = 0x00020000u;  // raw buffer, 32-bit data format

// Build-time tuning knobs (defaults are the measured best on MI355X).
#ifndef GQA_MIN_WAVES_PER_SIMD
#define GQA_MIN_WAVES_PER_SIMD 2
#endif
#ifndef GQA_BALANCED_MIN_WAVES_PER_SIMD
#define GQA_BALANCED_MIN_WAVES_PER_SIMD 2
#endif
#ifndef GQA_BALANCED_WGS_PER_CU
#define GQA_BALANCED_WGS_PER_CU 0  // build-time override of balanced_wgs_per_cu (0: none)
#endif
#ifndef GQA_KV_LOAD_POLICY
#define GQA_KV_LOAD_POLICY 2   // cache-policy bits of the K/V loads: 2 = non-temporal
#endif
constexpr int kLoadAux = GQA_KV_LOAD_POLICY;

typedef uint32_t u32;
typedef u32 u32x4 __attribute__((ext_vector_type(4)));
typedef u32 u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// Element-type traits for the MFMA operand type (= query dtype).
// ---------------------------------------------------------------------------
template <int QT>
struct Elem;

template <>
struct Elem<kBF16> {
  static __device__ __forceinline__ f32x4 qk(u32x4 k, u32x4 q, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, k),
                                                   __builtin_bit_cast(bf16x8, q), c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4 pv(u32x2 p, u32x2 v, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4, p),
                                                     __builtin_bit_cast(i16x4, v), c, 0, 0, 0);
  }
  static __device__ __forceinline__ u32 pack(float a, float b) {
    bf16x2 v = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(u32, v);
  }
  static __device__ __forceinline__ float lo(u32 x) { return __uint_as_float(x << 16); }
  static __device__ __forceinline__ float hi(u32 x) { return __uint_as_float(x & 0xffff0000u); }
  // Two e4m3 codes (bytes 2*sel, 2*sel+1 of x) -> two bf16 (exact).
  template <bool kHiWord>
  static __device__ __forceinline__ u32 from_fp8(u32 x) {
    return __builtin_bit_cast(u32, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x, 1.0f, kHiWord));
  }
  // Two signed int8 values (bytes 2*sel, 2*sel+1 of x) -> two bf16 (exact).
  template <bool kHiWord>
  static __device__ __forceinline__ u32 from_i8(u32 x) {
    return pack((float)(signed char)(x >> (kHiWord ? 16 : 0)),
                (float)(signed char)(x >> (kHiWord ? 24 : 8)));
  }
  static __device__ __forceinline__ void store2(void* p, float a, float b) {
    *reinterpret_cast<u32*>(p) = pack(a, b);
  }
};

template <>
struct Elem<kF16> {
  static __device__ __forceinline__ f32x4 qk(u32x4 k, u32x4 q, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, k),
                                                  __builtin_bit_cast(f16x8, q), c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4 pv(u32x2 p, u32x2 v, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4, p),
                                                 __builtin_bit_cast(f16x4, v), c, 0, 0, 0);
  }
  static __device__ __forceinline__ u32 pack(float a, float b) {
    f16x2 v = {(_Float16)a, (_Float16)b};
    return __builtin_bit_cast(u32, v);
  }
  static __device__ __forceinline__ float lo(u32 x) {
    return (float)__builtin_bit_cast(f16x2, x)[0];
  }
  static __device__ __forceinline__ float hi(u32 x) {
    return (float)__builtin_bit_cast(f16x2, x)[1];
  }
  template <bool kHiWord>
  static __device__ __forceinline__ u32 from_fp8(u32 x) {
    return __builtin_bit_cast(u32, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(x, 1.0f, kHiWord));
  }
  template <bool kHiWord>
  static __device__ __forceinline__ u32 from_i8(u32 x) {
    return pack((float)(signed char)(x >> (kHiWord ? 16 : 0)),
                (float)(signed char)(x >> (kHiWord ? 24 : 8)));
  }
  static __device__ __forceinline__ void store2(void* p, float a, float b) {
    *reinterpret_cast<u32*>(p) = pack(a, b);
  }
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, u32 bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, kRsrcWord3);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Dim-block (8 dims) that lane group `grp` feeds to QK instruction `i`.
// 16-bit cache: block 4i+grp.
// byte cache:   the lane's 16-byte chunk 4p+grp of a K row holds blocks
//               8p + 2grp + {0,1}, fed to instructions 2p and 2p+1.
// One-byte caches (fp8 e4m3, int8 with row scales) share the row layout and
// the load/stage/widen path; only the widening and the row scales differ.
template <int KVT>
constexpr bool kByteKv = KVT == kFP8 || KVT == kI8;

template <int KVT>
__device__ __forceinline__ int qk_dim_block(int i, int grp) {
  if constexpr (kByteKv<KVT>) {
    return 8 * (i >> 1) + 2 * grp + (i & 1);
  } else {
    return 4 * i + grp;
  }
}

// Registers of one 16-token tile, as loaded. Every load instruction reads
// whole cache rows (K and V alike): a 16-bit row is 256 bytes = 16 lanes x 16
// bytes, an fp8 row 128 bytes = 8 lanes x 16 bytes (K) or 16 lanes x 8 bytes (V).
template <int KVT>
struct Tile;

template <>
struct Tile<kF16> {
  u32x4 k[4];  // K: token 4grp+e, 16-byte chunk n16 (dims [8 n16, 8 n16 + 8))
  u32x4 v[4];  // V: token 4grp+e, dims [8 n16, 8 n16 + 8)
};
template <>
struct Tile<kBF16> : Tile<kF16> {};
template <>
struct Tile<kFP8> {
  u32x4 k[2];  // K: token 8u + lane/8, 16-byte chunk lane%8
  u32x2 v[4];  // V: token 4grp+e, dims [8 n16, 8 n16 + 8)
};
template <>
struct Tile<kI8> : Tile<kFP8> {
  u32x2 ks;    // bf16 K row scales of tokens 4grp .. 4grp+3
  u32x2 vs;    // bf16 V row scales of the same tokens
};

// Buffer resources of the (request, KV head) planes a workgroup reads; each
// ends at the range's last slot c1, so loads past it read 0 and cost nothing.
struct Planes {
  __amdgpu_buffer_rsrc_t k, v;    // K and V rows
  __amdgpu_buffer_rsrc_t ks, vs;  // bf16 row scales (INT8 cache only)
  int c1;                         // slots in range
  bool quads;                     // scale planes 8-byte aligned (capacity % 4 == 0)
};

// Four consecutive bf16 row scales from slot `tok` (a multiple of 4) on;
// slots at or past c1 read 0. A quad that straddles c1, or any quad of a
// plane that is not 8-byte aligned, is read one scale at a time, so no load
// reaches past the range's end whatever the hardware's range-check
// granularity, and none is misaligned. The scales stream like the rows they
// belong to (read once per step) and take the same non-temporal policy: with
// the default one they stay cached between back-to-back steps, which a model
// that runs other layers in between never sees, and a step that starts on
// caches full of other data ran 20% slower than with the streaming policy.
// (The contiguous cache reads its scales a block at a time instead; see
// load_block_scales. The paged cache reads them per tile here.)
__device__ __forceinline__ u32x2 load_scale_quad(__amdgpu_buffer_rsrc_t r, int tok, int c1,
                                                 bool quads) {
  if (quads && (tok + 4 <= c1 || tok >= c1))
    return __builtin_amdgcn_raw_buffer_load_b64(r, tok * 2, 0, kLoadAux);
  u32 h[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    h[i] = __builtin_amdgcn_raw_buffer_load_b16(r, (tok + i) * 2, 0, kLoadAux);
  return (u32x2){h[0] | (h[1] << 16), h[2] | (h[3] << 16)};
}

// kScales = false leaves an INT8 tile's row scales to the caller.
template <int KVT, bool kScales = true>
__device__ __forceinline__ void load_tile(Tile<KVT>& t, const Planes& pl, int j0, int lane) {
  const int n16 = lane & 15, grp = lane >> 4;
  const __amdgpu_buffer_rsrc_t rk = pl.k, rv = pl.v;
  if constexpr (kByteKv<KVT>) {
    const int ko = (j0 + (lane >> 3)) * kHeadDim + 16 * (lane & 7);
#pragma unroll
    for (int u = 0; u < 2; ++u)
      t.k[u] = __builtin_amdgcn_raw_buffer_load_b128(rk, ko + u * 8 * kHeadDim, 0, kLoadAux);
    const int vo = (j0 + 4 * grp) * kHeadDim + 8 * n16;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      t.v[e] = __builtin_amdgcn_raw_buffer_load_b64(rv, vo + e * kHeadDim, 0, kLoadAux);
    if constexpr (KVT == kI8 && kScales) {
      t.ks = load_scale_quad(pl.ks, j0 + 4 * grp, pl.c1, pl.quads);
      t.vs = load_scale_quad(pl.vs, j0 + 4 * grp, pl.c1, pl.quads);
    }
  } else {
    const int ko = (j0 + 4 * grp) * (2 * kHeadDim) + 16 * n16;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      t.k[e] = __builtin_amdgcn_raw_buffer_load_b128(rk, ko + e * (2 * kHeadDim), 0, kLoadAux);
    const int vo = ko;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      t.v[e] = __builtin_amdgcn_raw_buffer_load_b128(rv, vo + e * (2 * kHeadDim), 0, kLoadAux);
  }
}

// The bf16 row scales of a 64-slot block (four tiles) of an INT8 cache, read
// by one wave with one 2-byte load per lane and plane: lane l holds slot
// base + l (one 128-byte line per plane; slots at or past c1 read 0). One
// path for every block, whatever the alignment, so a wait for these loads
// can be counted exactly. Tile t of the block gathers its scales with lane
// shuffles.
struct BlockScales {
  u32 k, v;   // bf16 bits in the low half
};

__device__ __forceinline__ BlockScales load_block_scales(const Planes& pl, int base, int lane) {
  BlockScales s;
  s.k = __builtin_amdgcn_raw_buffer_load_b16(pl.ks, (base + lane) * 2, 0, kLoadAux);
  s.v = __builtin_amdgcn_raw_buffer_load_b16(pl.vs, (base + lane) * 2, 0, kLoadAux);
  return s;
}

// Scales of slots 16 t + 4 grp .. + 3 of the block into tile `t`.
__device__ __forceinline__ void tile_scales(Tile<kI8>& t, const BlockScales& s, int tile,
                                            int lane) {
  const int src = 16 * tile + 4 * (lane >> 4);
  u32 k[4], v[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    k[r] = (u32)__shfl((int)s.k, src + r);
    v[r] = (u32)__shfl((int)s.v, src + r);
  }
  t.ks = (u32x2){k[0] | (k[1] << 16), k[2] | (k[3] << 16)};
  t.vs = (u32x2){v[0] | (v[1] << 16), v[2] | (v[3] << 16)};
}

// The same scales repacked once per block into quads: lane m (< 16) holds the
// scales of slots 4 m .. 4 m + 3 of the block (lanes 16-63 repeat lanes 0-15),
// so a tile gathers its quads with two shuffles per plane from one source
// lane per lane group, instead of four. Fewer lane addresses stay live across
// the tile loop.
struct BlockQuads {
  u32x2 k, v;
};

__device__ __forceinline__ BlockQuads pack_block_scales(const BlockScales& s, int lane) {
  const int src = 4 * (lane & 15);
  u32 k[4], v[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    k[r] = (u32)__shfl((int)s.k, src + r);
    v[r] = (u32)__shfl((int)s.v, src + r);
  }
  BlockQuads q;
  q.k = (u32x2){k[0] | (k[1] << 16), k[2] | (k[3] << 16)};
  q.v = (u32x2){v[0] | (v[1] << 16), v[2] | (v[3] << 16)};
  return q;
}

// Quads of slots 16 t + 4 grp .. + 3 of the block into tile `t`.
__device__ __forceinline__ void tile_scales(Tile<kI8>& t, const BlockQuads& q, int tile, int lane) {
  const int src = 4 * tile + (lane >> 4);
  t.ks = (u32x2){(u32)__shfl((int)q.k[0], src), (u32)__shfl((int)q.k[1], src)};
  t.vs = (u32x2){(u32)__shfl((int)q.v[0], src), (u32)__shfl((int)q.v[1], src)};
}

// The QK product wants K with one token per lane (lane n16 = token, 8 dims
// per lane), the opposite of the row-per-16-lanes layout the coalesced loads
// deliver. The wave passes its K tile through its own LDS slice: token t's
// 16-byte chunk c is stored at slot c ^ f(t) of row t, with f(t) = t for
// 16-bit rows (16 chunks) and f(t) = (t >> 1) & 7 for fp8 rows (8 chunks), so
// both the stores (16 lanes = one row) and the loads (16 lanes = 16 rows, one
// chunk each) hit 16 distinct 16-byte bank groups.
constexpr int kKStageSlots = 16 * 16;  // 16-byte slots per wave (one 16-bit tile)
// Running state of one wave.
struct Softmax {
  float m;      // running max of log2-domain scores of row n16 (uniform per row)
  float l;      // this lane's share of the running sum
  f32x4 o[8];   // O[row 4grp+r][dim 8 n16 + c] in o[c][r] (rows 4grp..4grp+3 in group grp)
};

// Two one-byte cache values (bytes 2*sel, 2*sel+1 of x) -> two MFMA operands
// of type T.
template <int T, int KVT, bool kHiWord>
__device__ __forceinline__ u32 widen(u32 x) {
  if constexpr (KVT == kFP8) {
    return Elem<T>::template from_fp8<kHiWord>(x);
  } else {
    return Elem<T>::template from_i8<kHiWord>(x);
  }
}

// Operand type of the PV product. An INT8 cache multiplies each weight by its
// token's V row scale, whose range is not f16's, so its weights (and V) go in
// as bf16 hi + lo pairs whatever the query dtype; otherwise the query dtype.
template <int QT, int KVT>
constexpr int kPvType = KVT == kI8 ? (int)kBF16 : QT;

// One 16-token tile starting at slot j0: scores, online softmax and PV for
// the lane's row n16. Slots at or past `lim` are masked for that row (the
// range end; with several query tokens per request also the row's causal
// limit). kRows bounds the rows that hold real queries: G (<= 4) with one
// query token per request, where every row shares the tile's valid slots;
// up to 16 with several tokens, where a row may see no slot of a tile.
template <int QT, int KVT, int kRows>
__device__ __forceinline__ void process_tile(Softmax& st, const Tile<KVT>& t, const u32x4 (&qf)[4],
                                             u32x4* sk, int j0, int lim, int lane, float scale_log2) {
  using E = Elem<QT>;
  constexpr int PT = kPvType<QT, KVT>;
  using P = Elem<PT>;
  using B16 = Elem<kBF16>;   // row scales are bf16 whatever the query dtype
  const int n16 = lane & 15, grp = lane >> 4;
  // ---- scores^T[token 4grp + r][row n16] ------------------------------------
  f32x4 s = {0.f, 0.f, 0.f, 0.f};
  if constexpr (kByteKv<KVT>) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int tok = 8 * u + (lane >> 3);
      sk[tok * 8 + ((lane & 7) ^ ((tok >> 1) & 7))] = t.k[u];
    }
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const u32x4 k16 = sk[n16 * 8 + ((4 * p + grp) ^ ((n16 >> 1) & 7))];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const u32 w0 = k16[2 * h], w1 = k16[2 * h + 1];
        u32x4 kk = {widen<QT, KVT, false>(w0), widen<QT, KVT, true>(w0),
                    widen<QT, KVT, false>(w1), widen<QT, KVT, true>(w1)};
        s = E::qk(kk, qf[2 * p + h], s);
      }
    }
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int tok = 4 * grp + e;
      sk[tok * 16 + (n16 ^ tok)] = t.k[e];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) s = E::qk(sk[n16 * 16 + ((4 * i + grp) ^ n16)], qf[i], s);
  }

  // ---- online softmax, log2 domain -----------------------------------------
  float x[4];
  const int tok0 = j0 + 4 * grp;
  if constexpr (KVT == kI8) {   // K row scale of each token multiplies its score
    s[0] *= B16::lo(t.ks[0]);
    s[1] *= B16::hi(t.ks[0]);
    s[2] *= B16::lo(t.ks[1]);
    s[3] *= B16::hi(t.ks[1]);
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) x[r] = (tok0 + r < lim) ? s[r] * scale_log2 : -INFINITY;
  float mx = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
  mx = fmaxf(mx, __shfl_xor(mx, 16));
  mx = fmaxf(mx, __shfl_xor(mx, 32));
  const float m_new = fmaxf(st.m, mx);   // finite when the row sees a slot of this tile
  float m_ref = m_new;
  if constexpr (kRows > 4) {
    // A row that has seen no slot yet keeps m = -inf; exponents are then taken
    // against 0 (its weights and alpha come out 0, never NaN).
    m_ref = m_new == -INFINITY ? 0.f : m_new;
  }
  const float alpha = fast_exp2(st.m - m_ref);
  float p[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) p[r] = fast_exp2(x[r] - m_ref);
  // Weights the PV product sees: with an INT8 cache, each token's V row scale
  // multiplies its weight (l still sums the plain weights).
  float pw[4] = {p[0], p[1], p[2], p[3]};
  if constexpr (KVT == kI8) {
    pw[0] *= B16::lo(t.vs[0]);
    pw[1] *= B16::hi(t.vs[0]);
    pw[2] *= B16::lo(t.vs[1]);
    pw[3] *= B16::hi(t.vs[1]);
  }
  const u32 p01 = P::pack(pw[0], pw[1]);
  const u32 p23 = P::pack(pw[2], pw[3]);
  // bf16 keeps 8 significant bits of a weight; the PV product then takes the
  // weights as hi + lo bf16 pairs (16 bits), so only fp32 rounding is left and
  // l sums the fp32 weights. f16 weights (11 bits) go in one piece and l sums
  // the rounded weights the product sees.
  u32 q01 = 0u, q23 = 0u;
  if constexpr (PT == kBF16) {
    q01 = P::pack(pw[0] - P::lo(p01), pw[1] - P::hi(p01));
    q23 = P::pack(pw[2] - P::lo(p23), pw[3] - P::hi(p23));
    st.l = st.l * alpha + ((p[0] + p[1]) + (p[2] + p[3]));
  } else {
    st.l = st.l * alpha + ((P::lo(p01) + P::hi(p01)) + (P::lo(p23) + P::hi(p23)));
  }
  st.m = m_new;

  if constexpr (kRows <= 4) {
    // Rows 0..kRows-1 of O live in lanes 0..15; they need alpha of those rows.
    float al[4];
#pragma unroll
    for (int r = 0; r < 4; ++r)
      al[r] = r < kRows ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(alpha), r)) : 1.f;
    if (al[0] != 1.f || al[1] != 1.f || al[2] != 1.f || al[3] != 1.f) {
#pragma unroll
      for (int c = 0; c < 8; ++c) {
#pragma unroll
        for (int r = 0; r < kRows; ++r) st.o[c][r] *= al[r];
      }
    }
  } else {
    // Row 4grp+r of O lives in lane group grp; its alpha sits in lane 4grp+r.
    float al[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) al[r] = __shfl(alpha, 4 * grp + r);
    if (__any(al[0] != 1.f || al[1] != 1.f || al[2] != 1.f || al[3] != 1.f)) {
#pragma unroll
      for (int c = 0; c < 8; ++c) {
#pragma unroll
        for (int r = 0; r < 4; ++r) st.o[c][r] *= al[r];
      }
    }
  }

  // ---- O += P x V ------------------------------------------------------------
  const u32x2 pa = {p01, p23};
  const u32x2 pl = {q01, q23};
  auto pv = [&](f32x4 acc, u32x2 bv) {
    acc = P::pv(pa, bv, acc);
    if constexpr (PT == kBF16) acc = P::pv(pl, bv, acc);
    return acc;
  };
  if constexpr (kByteKv<KVT>) {
    // For dim 8 n16 + c the B operand is {V[tok0+0..3][c]}: interleave the
    // bytes of two tokens, then widen byte pairs.
#pragma unroll
    for (int w = 0; w < 2; ++w) {
      u32 lo_a[2], lo_b[2];
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const u32 x0 = t.v[2 * q][w], x1 = t.v[2 * q + 1][w];
        lo_a[q] = __builtin_amdgcn_perm(x1, x0, 0x05010400u);  // x0.b0 x1.b0 x0.b1 x1.b1
        lo_b[q] = __builtin_amdgcn_perm(x1, x0, 0x07030602u);  // x0.b2 x1.b2 x0.b3 x1.b3
      }
      const u32x2 b0 = {widen<PT, KVT, false>(lo_a[0]), widen<PT, KVT, false>(lo_a[1])};
      const u32x2 b1 = {widen<PT, KVT, true>(lo_a[0]), widen<PT, KVT, true>(lo_a[1])};
      const u32x2 b2 = {widen<PT, KVT, false>(lo_b[0]), widen<PT, KVT, false>(lo_b[1])};
      const u32x2 b3 = {widen<PT, KVT, true>(lo_b[0]), widen<PT, KVT, true>(lo_b[1])};
      st.o[4 * w + 0] = pv(st.o[4 * w + 0], b0);
      st.o[4 * w + 1] = pv(st.o[4 * w + 1], b1);
      st.o[4 * w + 2] = pv(st.o[4 * w + 2], b2);
      st.o[4 * w + 3] = pv(st.o[4 * w + 3], b3);
    }
  } else {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const u32 v0 = t.v[0][w], v1 = t.v[1][w], v2 = t.v[2][w], v3 = t.v[3][w];
      const u32x2 be = {(v0 & 0xffffu) | (v1 << 16), (v2 & 0xffffu) | (v3 << 16)};
      const u32x2 bo = {(v0 >> 16) | (v1 & 0xffff0000u), (v2 >> 16) | (v3 & 0xffff0000u)};
      st.o[2 * w + 0] = pv(st.o[2 * w + 0], be);
      st.o[2 * w + 1] = pv(st.o[2 * w + 1], bo);
    }
  }
}

// How a workgroup finishes its chunk.
enum Mode : int {
  kModeDirect = 0,      // single chunk per head: normalise and write the output
  kModeSplit = 1,       // write the chunk partial; a separate kernel combines
  kModeSplitFused = 2,  // write the partial; the head's last workgroup combines
};

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

// ---------------------------------------------------------------------------
// Partials read back inside the launch that wrote them (the one-launch
// merge). Each XCD has its own L2, not coherent with the others', so a partial
// that a workgroup on another XCD reads within the same launch goes through
// device-coherent accesses: the loads and stores the compiler emits for
// relaxed agent-scope atomics (stores write through the L2, loads are not
// served from a stale L2 line). Ordering comes from waiting for the stores
// to complete before the counter update that announces them (publish_piece).
// An agent-scope release/acquire fence pair would instead write back and
// invalidate the whole L2 of the XCD for every piece.
// ---------------------------------------------------------------------------
template <bool kCoherent>
__device__ __forceinline__ float2 load_partial(const float2* p) {
  if constexpr (kCoherent) {
    const unsigned long long v = __hip_atomic_load(reinterpret_cast<const unsigned long long*>(p),
                                                   __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return __builtin_bit_cast(float2, v);
  } else {
    return *p;
  }
}

template <bool kCoherent>
__device__ __forceinline__ void store_partial(float2* p, float2 v) {
  if constexpr (kCoherent) {
    __hip_atomic_store(reinterpret_cast<unsigned long long*>(p),
                       __builtin_bit_cast(unsigned long long, v), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
  } else {
    *p = v;
  }
}

// Announce a piece of `total` units of one head: every thread of the
// workgroup has stored its share of the piece with store_partial<true>; once
// those stores have completed (s_waitcnt vmcnt(0) in each wave, then the
// barrier), one thread adds the piece's `units` to the head's counter with a
// device-scope atomic. Returns, in every thread, whether this piece completed
// the head (the caller then merges it); that thread also resets the counter,
// so every launch finds it at zero. s_flag is a workgroup-shared int.
__device__ __forceinline__ bool publish_piece(uint32_t* counter, uint32_t units, uint32_t total,
                                              int* s_flag) {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t prev =
        __hip_atomic_fetch_add(counter, units, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const bool last = prev + units == total;
    if (last) __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *s_flag = last;
  }
  __syncthreads();
  return *s_flag != 0;
}

// NB partial O rows base + j0 + u (u < NB) of a merge, loaded together and
// accumulated with their weights, which lane j of wk holds for row base + j.
// Rows at or past cnt get weight 0 and read the fallback row instead.
template <int NB, bool kCoherent = false, typename RowFn>
__device__ __forceinline__ void merge_batch(const float2* po, RowFn& row, size_t fallback, int base,
                                            int j0, int cnt, float wk, int lane, float& o0,
                                            float& o1) {
  float f[NB];
  float2 v[NB];
#pragma unroll
  for (int u = 0; u < NB; ++u) {
    const int j = j0 + u;
    f[u] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wk), min(j, 63)));
    if (j >= cnt) f[u] = 0.f;
    const size_t r = f[u] != 0.f ? row(base + j) : fallback;
    v[u] = load_partial<kCoherent>(po + r * (kHeadDim / 2) + lane);
  }
#pragma unroll
  for (int u = 0; u < NB; ++u) {
    o0 += f[u] * v[u].x;
    o1 += f[u] * v[u].y;
  }
}

// merge_rows for n <= NB rows: the (m, l) pair of row k (lane k) and all NB
// partial O rows are loaded before any of them is waited on, so the merge
// costs one round trip to memory. Addresses depend only on n, not on the
// weights; rows at or past n read the first row again and, like empty rows
// (max -inf, O possibly stale), enter with weight 0 through a select.
template <int NB, int QT, bool kCoherent, typename RowFn>
__device__ __forceinline__ void merge_few(const StepArgs& a, int n, RowFn& row, char* outp) {
  using E = Elem<QT>;
  const int lane = threadIdx.x & 63;
  const float2* ml = reinterpret_cast<const float2*>(a.part_ml);
  const float2* po = reinterpret_cast<const float2*>(a.part_o);
  const size_t fallback = row(0);
  const float2 mv = load_partial<kCoherent>(ml + (lane < n ? row(lane) : fallback));
  float2 v[NB];
#pragma unroll
  for (int u = 0; u < NB; ++u)
    v[u] = load_partial<kCoherent>(po + (u < n ? row(u) : fallback) * (kHeadDim / 2) + lane);
  const float mk = lane < n ? mv.x : -INFINITY;
  const float M = wave_max(mk);   // finite: at least one row holds data
  const float wk = mk != -INFINITY ? fast_exp2(mk - M) : 0.f;
  const float lsum = wave_sum(wk != 0.f ? wk * mv.y : 0.f);
  float o0 = 0.f, o1 = 0.f;
#pragma unroll
  for (int u = 0; u < NB; ++u) {
    const float f = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wk), u));
    o0 = fmaf(f, f != 0.f ? v[u].x : 0.f, o0);
    o1 = fmaf(f, f != 0.f ? v[u].y : 0.f, o1);
  }
  const float inv = a.v_scale / lsum;
  E::store2(outp, o0 * inv, o1 * inv);
}

// Log-sum-exp merge of n partial rows of one query head, run by one wave
// (lane l owns dims 2l and 2l + 1):
//   M = max_k m_k,  out = v_scale * sum_k 2^(m_k - M) O_k / sum_k 2^(m_k - M) l_k
// row(k) gives the k-th partial row. A row whose max is -inf is empty (a
// workgroup that had no slabs marked it): it gets weight 0 and its O row,
// possibly stale, never enters the sum. Up to 32 rows take merge_few's
// single round of loads. Beyond that the (m, l) pairs of 64 rows at a time are
// loaded one per lane; the O rows follow in batches of 32, 16 and then 8
// independent loads, so a head split into 64 pieces (one request spread over
// the whole grid) waits for two rounds of loads, not eight. kCoherent: the
// rows were written in this launch (load_partial).
template <int QT, bool kCoherent = false, typename RowFn>
__device__ __forceinline__ void merge_rows(const StepArgs& a, int n, RowFn row, char* outp) {
  if (n <= 8) return merge_few<8, QT, kCoherent>(a, n, row, outp);
  if (n <= 16) return merge_few<16, QT, kCoherent>(a, n, row, outp);
  if (n <= 32) return merge_few<32, QT, kCoherent>(a, n, row, outp);
  using E = Elem<QT>;
  const int lane = threadIdx.x & 63;
  const float2* ml = reinterpret_cast<const float2*>(a.part_ml);
  const float2* po = reinterpret_cast<const float2*>(a.part_o);
  float mloc = -INFINITY;
  for (int k = lane; k < n; k += 64) mloc = fmaxf(mloc, load_partial<kCoherent>(ml + row(k)).x);
  const float M = wave_max(mloc);   // finite: at least one row holds data
  const size_t fallback = row(0);   // a row that holds data, read with weight 0
  float lloc = 0.f, o0 = 0.f, o1 = 0.f;
  for (int base = 0; base < n; base += 64) {
    const int k = base + lane;
    float wk = 0.f;
    if (k < n) {
      const float2 v = load_partial<kCoherent>(ml + row(k));
      if (v.x != -INFINITY) {
        wk = fast_exp2(v.x - M);
        lloc += wk * v.y;
      }
    }
    const int cnt = min(64, n - base);
    int j0 = 0;
    for (; cnt - j0 >= 32; j0 += 32)
      merge_batch<32, kCoherent>(po, row, fallback, base, j0, cnt, wk, lane, o0, o1);
    if (cnt - j0 >= 16) {
      merge_batch<16, kCoherent>(po, row, fallback, base, j0, cnt, wk, lane, o0, o1);
      j0 += 16;
    }
    for (; j0 < cnt; j0 += 8)
      merge_batch<8, kCoherent>(po, row, fallback, base, j0, cnt, wk, lane, o0, o1);
  }
  const float inv = a.v_scale / wave_sum(lloc);
  E::store2(outp, o0 * inv, o1 * inv);
}

// LDS of one workgroup: the 4 waves' K staging slices and the merge buffers
// (for the 4 MFMA rows; rows >= G carry zero queries and are never stored).
struct WorkgroupLds {
  u32x4 k[kWaves][kKStageSlots];
  float o[kWaves][kGroup][kHeadDim];
  float m[kWaves][kGroup];
  float l[kWaves][kGroup];
};

// Balanced split: workgroup w's range is [bound(w), bound(w + 1)), with
// bound(w) = N * S(w) / S(W) and S(w) the sum of the shares of workgroups
// 0 .. w-1 (integer arithmetic).
// The shares follow how the hardware serves co-resident workgroups: on each
// CU the workgroup dispatched first streams fastest, and workgroups of
// odd-numbered XCDs (w odd: XCDs take workgroups round-robin) stream slower.
__device__ __forceinline__ int64_t share_prefix(const StepArgs& a, int w) {
  const int ts = a.tier_size;
  int64_t acc = 0;
  for (int t = 0; t < kShareTiers; ++t) {
    const int lo = t * ts;
    const int hi = t == kShareTiers - 1 ? w : min(w, lo + ts);
    if (hi <= lo) break;
    const int evens = (hi + 1) / 2 - (lo + 1) / 2;
    const int odds = hi / 2 - lo / 2;
    acc += (int64_t)evens * a.share[2 * t] + (int64_t)odds * a.share[2 * t + 1];
  }
  return acc;
}

__device__ __forceinline__ int balanced_bound(const StepArgs& a, int w, int64_t N, int64_t total) {
  return (int)(N * share_prefix(a, w) / total);
}

// Balanced split bookkeeping for the combine: the slot of the head's first
// piece (-1 when one workgroup wrote the head whole) and the workgroup that
// holds its last piece. Every head with a slab gets its first entry written
// by every launch, so nothing of an earlier launch is read.
__device__ __forceinline__ void record_piece(const StepArgs& a, int head, bool whole, bool first,
                                             bool last, size_t slot, int w) {
  if (threadIdx.x != 0) return;
  const int heads = a.batch * kKvHeads;
  if (whole) {
    a.head_pieces[head] = -1;
    return;
  }
  if (first) a.head_pieces[head] = (int)slot;
  if (last) a.head_pieces[heads + head] = w;
}

// Resident workgroups per CU of the balanced grids, contiguous and paged (0:
// as many as fit): 2 for 16-bit and fp8 caches, all that fit for INT8.
// Measured against 3 per CU: 0.3% / 0.9% / 0.7% faster on the 64k bf16,
// 128k fp8 and ragged f16 steps and 1.7-1.9% on fp8 page pools, but 2.5%
// slower on the 128k INT8 step, whose byte widening needs the third
// workgroup's waves to hide its ALU latency. One per CU won 1.2% on 64k bf16
// and lost 6% on fp8, 2.5% on the ragged batch and 47% on INT8.
template <int KVT>
constexpr int balanced_wgs_per_cu() {
  return GQA_BALANCED_WGS_PER_CU > 0 ? GQA_BALANCED_WGS_PER_CU : (KVT == kI8 ? 0 : 2);
}

// Balanced split: slabs of 64 slots per (request, KV head).
__device__ __forceinline__ int slabs_of(int len, int capacity) {
  return (min(max(len, 0), capacity) + kSlab - 1) / kSlab;
}

// pref[b] = 8 * sum_{b' < b} slabs(b'), b = 0..B (B <= kMaxBalancedBatch).
__device__ __forceinline__ void build_slab_prefix(const StepArgs& a, int* pref, int* wave_tot) {
  const int B = a.batch;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int per = (B + kThreads - 1) / kThreads;
  const int lo = min(tid * per, B);
  const int hi = min(lo + per, B);
  int own = 0;
  for (int i = lo; i < hi; ++i) own += slabs_of(a.seq_lens[i], a.capacity);
  int x = own;   // inclusive scan across the wave
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  if (lane == 63) wave_tot[wave] = x;
  __syncthreads();
  int run = x - own;
  for (int w = 0; w < wave; ++w) run += wave_tot[w];
  for (int i = lo; i < hi; ++i) {
    pref[i] = kKvHeads * run;
    run += slabs_of(a.seq_lens[i], a.capacity);
  }
  if (tid == kThreads - 1) pref[B] = kKvHeads * run;
  __syncthreads();
}

// Calls f.template operator()<QT, KVT, G>() for a supported combination, else
// returns `bad`.
template <typename R, typename F>
R dispatch(int q_dtype, int kv_dtype, int num_q_heads, R bad, F&& f) {
  auto by_group = [&](auto qt, auto kvt) -> R {
    constexpr int QT = decltype(qt)::value, KVT = decltype(kvt)::value;
    if (num_q_heads == 4 * kKvHeads) return f.template operator()<QT, KVT, 4>();
    if (num_q_heads == 2 * kKvHeads) return f.template operator()<QT, KVT, 2>();
    return bad;
  };
  using BF = std::integral_constant<int, kBF16>;
  using F16 = std::integral_constant<int, kF16>;
  using F8 = std::integral_constant<int, kFP8>;
  using I8 = std::integral_constant<int, kI8>;
  if (q_dtype == kBF16 && kv_dtype == kBF16) return by_group(BF{}, BF{});
  if (q_dtype == kF16 && kv_dtype == kF16) return by_group(F16{}, F16{});
  if (q_dtype == kBF16 && kv_dtype == kFP8) return by_group(BF{}, F8{});
  if (q_dtype == kF16 && kv_dtype == kFP8) return by_group(F16{}, F8{});
  if (q_dtype == kBF16 && kv_dtype == kI8) return by_group(BF{}, I8{});
  if (q_dtype == kF16 && kv_dtype == kI8) return by_group(F16{}, I8{});
  return bad;
}

}  // namespace
}  // namespace gqa
