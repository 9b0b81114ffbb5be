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
// Work split. A workgroup (4 waves of 64 lanes) owns one chunk of one
// (request, KV head): `chunk_tokens` consecutive cache slots. Within the
// chunk the waves take 16-token tiles round-robin. Every chunk keeps an fp32
// online softmax (running max m, running sum l, unnormalised output O) in the
// log2 domain; the 4 waves merge through LDS at the end. With one chunk per
// head the workgroup normalises and writes the output; otherwise it writes
// (m, l, O) as FP32 partials — the split-KV scheme of the article's
// "default routes and num_splits" section — and a log-sum-exp combine kernel
// merges the chunks of each query head.
//
// Tile math on the matrix cores. The 4 grouped query rows form a 16-row MFMA
// operand (rows 4..15 zero; the cores have ~10x the throughput this stream
// needs, so the padding costs nothing measurable):
//   scores^T[16 tok, 16 rows] = K_tile[16 tok, 128] x Q^T[128, 16]
//       4 x v_mfma_f32_16x16x32_{bf16,f16}; K arrives straight from HBM in
//       the A-operand layout (lane = token, 8 consecutive dims per lane).
//   O[16 rows, 128]           += P[16 rows, 16 tok] x V_tile[16 tok, 128]
//       8 x v_mfma_f32_16x16x16_{bf16,f16}; the score accumulator already is
//       the P A-operand layout, and each lane loads 16 contiguous bytes of a
//       V row (a wave covers 4 whole rows per load), which a byte permute
//       turns into the B-operand layout (4 tokens of one dim per lane).
// fp8 e4m3 K/V bytes are widened to bf16/f16 in registers with the gfx950
// packed converts (exact: every e4m3 value is representable), so the cache
// is read once, at 1 byte per element.
//
// Loads are raw buffer loads whose range ends at the chunk's last valid
// slot: slots past the request's length are never fetched (they read as 0
// without touching memory), which also makes the one-tile-ahead prefetch
// free at the end of a chunk.

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
// granularity, and none is misaligned.
__device__ __forceinline__ u32x2 load_scale_quad(__amdgpu_buffer_rsrc_t r, int tok, int c1,
                                                 bool quads) {
  if (quads && (tok + 4 <= c1 || tok >= c1))
    return __builtin_amdgcn_raw_buffer_load_b64(r, tok * 2, 0, 0);
  u32 h[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) h[i] = __builtin_amdgcn_raw_buffer_load_b16(r, (tok + i) * 2, 0, 0);
  return (u32x2){h[0] | (h[1] << 16), h[2] | (h[3] << 16)};
}

template <int KVT>
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
    if constexpr (KVT == kI8) {
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
  f32x4 o[8];   // O[row 4grp+r][dim 8 n16 + c] in o[c][r] (rows 0..3 live in grp 0)
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

template <int QT, int KVT, int G>
__device__ __forceinline__ void process_tile(Softmax& st, const Tile<KVT>& t, const u32x4 (&qf)[4],
                                             u32x4* sk, int j0, int c1, int lane, float scale_log2) {
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
  for (int r = 0; r < 4; ++r) x[r] = (tok0 + r < c1) ? s[r] * scale_log2 : -INFINITY;
  float mx = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
  mx = fmaxf(mx, __shfl_xor(mx, 16));
  mx = fmaxf(mx, __shfl_xor(mx, 32));
  const float m_new = fmaxf(st.m, mx);   // finite: the tile holds >= 1 valid token
  const float alpha = fast_exp2(st.m - m_new);
  float p[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) p[r] = fast_exp2(x[r] - m_new);
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

  // Rows 0..G-1 of O live in lanes 0..15; they need alpha of rows 0..G-1.
  float al[4];
#pragma unroll
  for (int r = 0; r < 4; ++r)
    al[r] = r < G ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(alpha), r)) : 1.f;
  if (al[0] != 1.f || al[1] != 1.f || al[2] != 1.f || al[3] != 1.f) {
#pragma unroll
    for (int c = 0; c < 8; ++c) {
#pragma unroll
      for (int r = 0; r < G; ++r) st.o[c][r] *= al[r];
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

// Log-sum-exp merge of n partial rows of one query head, run by one wave
// (lane l owns dims 2l and 2l + 1):
//   M = max_k m_k,  out = v_scale * sum_k 2^(m_k - M) O_k / sum_k 2^(m_k - M) l_k
// row(k) gives the k-th partial row. A row whose max is -inf is empty (a
// workgroup that had no slabs marked it): it gets weight 0 and its O row,
// possibly stale, is never read. The (m, l) pairs of 64 rows at a time are
// loaded one per lane, so the whole merge costs two dependent loads.
template <int QT, typename RowFn>
__device__ __forceinline__ void merge_rows(const StepArgs& a, int n, RowFn row, char* outp) {
  using E = Elem<QT>;
  const int lane = threadIdx.x & 63;
  const float2* ml = reinterpret_cast<const float2*>(a.part_ml);
  const float2* po = reinterpret_cast<const float2*>(a.part_o);
  float mloc = -INFINITY;
  for (int k = lane; k < n; k += 64) mloc = fmaxf(mloc, ml[row(k)].x);
  const float M = wave_max(mloc);   // finite: at least one row holds data
  const size_t fallback = row(0);   // a row that holds data, read with weight 0
  float lloc = 0.f, o0 = 0.f, o1 = 0.f;
  for (int base = 0; base < n; base += 64) {
    const int k = base + lane;
    float wk = 0.f;
    if (k < n) {
      const float2 v = ml[row(k)];
      if (v.x != -INFINITY) {
        wk = fast_exp2(v.x - M);
        lloc += wk * v.y;
      }
    }
    const int cnt = min(64, n - base);
    for (int j0 = 0; j0 < cnt; j0 += 8) {   // 8 independent row loads in flight
      float f[8];
      float2 v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int j = j0 + u;
        f[u] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wk), min(j, 63)));
        if (j >= cnt) f[u] = 0.f;
        const size_t r = f[u] != 0.f ? row(base + j) : fallback;
        v[u] = po[r * (kHeadDim / 2) + lane];
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        o0 += f[u] * v[u].x;
        o1 += f[u] * v[u].y;
      }
    }
  }
  const float inv = a.v_scale / wave_sum(lloc);
  E::store2(outp, o0 * inv, o1 * inv);
}

// Merge of the chunked split for the G query heads of (request b, KV head g):
// wave r < G takes head G g + r. Only the chunks that start below the current
// length are read, so partials left by an earlier launch with longer lengths
// never enter the result.
template <int QT, int G>
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
  merge_rows<QT>(a, n, [&](int k) -> size_t { return head * (size_t)S + k; }, outp);
}

// LDS of one workgroup: the 4 waves' K staging slices and the merge buffers
// (for the 4 MFMA rows; rows >= G carry zero queries and are never stored).
struct WorkgroupLds {
  u32x4 k[kWaves][kKStageSlots];
  float o[kWaves][kGroup][kHeadDim];
  float m[kWaves][kGroup];
  float l[kWaves][kGroup];
};

// One workgroup attends the G query rows of (request b, KV head g) over the
// cache slots [c0, c1) (c0 < c1 <= length). On return thread t holds, for
// row t / 64 (meaningful for rows < G) and dims 2 (t % 64) + {0, 1}: the
// chunk's log2-domain max M, its sum of weights l and its unnormalised output
// (o0, o1). Ends with a barrier, so the caller may call it again for another
// range.
template <int QT, int KVT, int G>
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
    const size_t slot = head * (size_t)S + split;
    if (er < G) {
      *reinterpret_cast<float2*>(a.part_o + slot * kHeadDim + ed) = make_float2(o0, o1);
      if ((tid & 63) == 0) *reinterpret_cast<float2*>(a.part_ml + slot * 2) = make_float2(M, lsum);
    }
    if constexpr (kMode == kModeSplitFused) {
      // Publish this chunk, count it, and let the head's last chunk combine.
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
      __syncthreads();
      if (tid == 0) {
        const unsigned n_valid = (unsigned)((L + a.chunk_tokens - 1) / a.chunk_tokens);
        const unsigned prev = atomicAdd(a.counters + bg, 1u);
        const int last = (prev + 1u == n_valid);
        if (last) atomicExch(a.counters + bg, 0u);   // ready for the next launch
        s_last = last;
      }
      __syncthreads();
      if (!s_last) return;
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
      combine_head_group<QT, G>(a, b, g, L);
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
// Balanced split. The work of a step is 8 * sum_b ceil(L_b / 64) slabs of 64
// slots, ordered request-major then KV head. A persistent grid of W
// workgroups (as many as the device keeps resident) gives workgroup w the
// slab range [w N / W, (w+1) N / W), so every workgroup streams the same
// number of bytes whatever the length mix. A range crosses (request, KV head)
// boundaries: heads it covers whole are normalised and written directly; its
// first and last piece, when they are only part of a head, become partials
// in slots 2w and 2w + 1, which the balanced combine merges per head.
// ---------------------------------------------------------------------------
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

// Partial rows of the balanced split: slot k holds kGroup rows (rows >= G
// unused), so the slot stride does not depend on the geometry.
template <int QT, int KVT, int G>
__global__ __launch_bounds__(kThreads, GQA_BALANCED_MIN_WAVES_PER_SIMD) void gqa_balanced_attention_kernel(
    StepArgs a) {
  using E = Elem<QT>;
  __shared__ WorkgroupLds lds;
  __shared__ int s_pref[kMaxBalancedBatch + 1];
  __shared__ int s_wave_tot[kWaves];

  const int tid = threadIdx.x;
  const int B = a.batch;
  build_slab_prefix(a, s_pref, s_wave_tot);
  // Values read from LDS are the same in every lane; saying so keeps the
  // loop control in scalar registers.
  const int64_t N = __builtin_amdgcn_readfirstlane(s_pref[B]);
  const int W = (int)gridDim.x;
  const int w = (int)blockIdx.x;
  if (w == 0)   // the combine kernel reads the same prefix
    for (int i = tid; i <= B; i += kThreads) a.slab_prefix[i] = s_pref[i];

  const int er = tid >> 6;
  const int ed = (tid & 63) * 2;
  // Slab counts fit in int32 (checked when the plan is made).
  const int s0 = (int)((int64_t)w * N / W);
  const int s1 = (int)((int64_t)(w + 1) * N / W);
  if (s0 == s1) {
    // Fewer slabs than workgroups: mark slot 2w empty for the combine, which
    // may look at it when this workgroup falls inside a head's range of workgroups.
    if ((tid & 63) == 0)
      *reinterpret_cast<float2*>(a.part_ml + ((size_t)2 * w * kGroup + er) * 2) =
          make_float2(-INFINITY, 0.f);
    return;
  }
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
    attend_range<QT, KVT, G>(a, b, g, c0, c1, lds, M, lsum, o0, o1);
    const size_t head = ((size_t)b * kKvHeads + g) * G + er;
    if (s == seg_start && pe == seg_end) {
      const float inv = a.v_scale / lsum;
      if (er < G)
        E::store2(static_cast<char*>(a.out) + (head * kHeadDim + ed) * 2, o0 * inv, o1 * inv);
    } else {
      const size_t slot = 2 * (size_t)w + (s == s0 ? 0 : 1);
      const size_t row = slot * kGroup + er;
      *reinterpret_cast<float2*>(a.part_o + row * kHeadDim + ed) = make_float2(o0, o1);
      if ((tid & 63) == 0) *reinterpret_cast<float2*>(a.part_ml + row * 2) = make_float2(M, lsum);
    }
    s = pe;
  }
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
  const int64_t N = a.slab_prefix[a.batch];
  const int nsb = (a.slab_prefix[b + 1] - a.slab_prefix[b]) / kKvHeads;
  if (nsb == 0) {
    E::store2(outp, 0.f, 0.f);
    return;
  }
  const int64_t W = a.grid_wgs;
  const int64_t seg_start = a.slab_prefix[b] + (int64_t)g * nsb;
  const int64_t seg_end = seg_start + nsb;
  // workgroup whose range holds slab t: the largest w with w N / W <= t
  const int wf = (int)(((seg_start + 1) * W - 1) / N);
  const int wl = (int)((seg_end * W - 1) / N);
  if (wf == wl) return;
  // wf's range may begin in an earlier head: then this head is its last piece
  const int first_slot_bump = ((int64_t)wf * N / W < seg_start) ? 1 : 0;
  merge_rows<QT>(a, wl - wf + 1,
                 [&](int k) -> size_t {
                   return (2 * (size_t)(wf + k) + (k == 0 ? first_slot_bump : 0)) * kGroup + r;
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
// KV append: write one new token's K and V rows of every KV head at slot
// positions[b] (the cache write that precedes each decode step). An fp8
// cache stores e4m3(x / scale), per-tensor scales as in the Thor FP8-KV
// notes; the division is an IEEE fp32 division and the code the nearest
// E4M3FN value (ties to even), saturating at +-448.
// ---------------------------------------------------------------------------
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
  // one thread per 8 dims of one (request, plane, KV head) row
  const int t = (int)(blockIdx.x * 256 + threadIdx.x);
  if (t >= a.batch * 2 * kKvHeads * (kHeadDim / 8)) return;
  const int chunk = t % (kHeadDim / 8);
  const int row = t / (kHeadDim / 8);
  const int g = row % kKvHeads;
  const int plane = (row / kKvHeads) % 2;
  const int b = row / (2 * kKvHeads);
  const int pos = a.positions[b];
  if (pos < 0 || pos >= a.capacity) return;
  const char* src = static_cast<const char*>(plane ? a.v_new : a.k_new) +
                    (((size_t)b * kKvHeads + g) * kHeadDim + chunk * 8) * 2;
  const u32x4 in = *reinterpret_cast<const u32x4*>(src);
  const size_t dst = ((((size_t)b * 2 + plane) * kKvHeads + g) * a.capacity + pos) * kHeadDim + chunk * 8;
  if constexpr (KVT == kFP8) {
    const float scale = plane ? a.v_scale : a.k_scale;
    u32 w[2] = {0u, 0u};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float x = (i & 1) ? E::hi(in[i >> 1]) : E::lo(in[i >> 1]);
      w[i >> 2] |= f32_to_e4m3fn_sat(__fdiv_rn(x, scale)) << (8 * (i & 3));
    }
    *reinterpret_cast<u32x2*>(static_cast<char*>(a.kv) + dst) = (u32x2){w[0], w[1]};
  } else {
    *reinterpret_cast<u32x4*>(static_cast<char*>(a.kv) + dst * 2) = in;
  }
}

template <int QT, int KVT>
hipError_t enqueue_append_typed(const AppendArgs& a, hipStream_t stream) {
  const int threads = a.batch * 2 * kKvHeads * (kHeadDim / 8);
  hipLaunchKernelGGL((gqa_kv_append_kernel<QT, KVT>), dim3((threads + 255) / 256), dim3(256), 0,
                     stream, a);
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
  return cus * per_cu;
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

int balanced_grid_size(int q_dtype, int kv_dtype, int num_q_heads) {
  return dispatch(q_dtype, kv_dtype, num_q_heads, 0,
                  []<int QT, int KVT, int G>() { return balanced_grid_typed<QT, KVT, G>(); });
}

hipError_t enqueue_kv_append(const AppendArgs& a, int src_dtype, int kv_dtype, hipStream_t stream) {
  if (src_dtype == kBF16 && kv_dtype == kBF16) return enqueue_append_typed<kBF16, kBF16>(a, stream);
  if (src_dtype == kF16 && kv_dtype == kF16) return enqueue_append_typed<kF16, kF16>(a, stream);
  if (src_dtype == kBF16 && kv_dtype == kFP8) return enqueue_append_typed<kBF16, kFP8>(a, stream);
  if (src_dtype == kF16 && kv_dtype == kFP8) return enqueue_append_typed<kF16, kFP8>(a, stream);
  return hipErrorInvalidValue;
}

hipError_t enqueue_decode_step(const StepArgs& a, int q_dtype, int kv_dtype, hipStream_t stream,
                               hipEvent_t ev_mid) {
  return dispatch(q_dtype, kv_dtype, a.num_q_heads, hipErrorInvalidValue,
                  [&]<int QT, int KVT, int G>() { return enqueue_typed<QT, KVT, G>(a, stream, ev_mid); });
}

}  // namespace gqa
