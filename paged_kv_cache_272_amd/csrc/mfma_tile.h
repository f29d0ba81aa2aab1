// Register-level building blocks of the MFMA paged-attention kernels
// (gfx950): one 16-token K/V block of one KV head held by a wave, the query
// operand of up to 16 query columns, and the online-softmax state.
//
// Layout, per block, with lane l = 16*c + r (r = l%16, c = l/16):
//   QK:  S^T[token][column] = K[token][:] . Q[column][:]  with D/32 MFMAs
//        16x16x32 bf16.  A = K: lane holds 8 consecutive d of token r
//        (row r), B = Q^T: lane holds the same 8 d of query column r.  The d
//        chunk for k-step i and lane group c is (D/32)*c + i, so a lane reads
//        one contiguous D/4-element run of its token's row.
//        Result: lane holds s[j] = S^T[token 4c+j][column r], j = 0..3.
//   softmax: logits taken relative to a per-column reference max by one
//        FMA, mask by select; the reference moves (and the output is
//        rescaled) only when a logit exceeds it by more than 2^kLazyMax,
//        which the lane's own maximum shows without any cross-lane step.
//   PV:  O^T[d][column] += V^T[d][token] . P^T[token][column] with D/16
//        MFMAs 16x16x16 bf16.  B = P^T: lane holds p[j] for tokens 4c..4c+3
//        of column r, which is exactly the QK result layout, so P never
//        leaves registers.  A = V^T: lane holds tokens 4c..4c+3 of one d; V
//        is loaded row-contiguously (16 lanes per 256-byte token row) and the
//        4x(D/16) sub-tile is transposed in registers with byte permutes.
//        Tile n covers d = (D/16)*r + n, so lane (r, c) ends up holding the
//        contiguous output run d in [(D/4)c, (D/4)(c+1)) of column r.
// e4m3 codes are widened to bf16 exactly (every e4m3 value is a bf16
// value); int4 codes become the bf16 value 128 + code (one and-or per pair
// of codes), and the 136-times bias terms this adds are taken off per
// column.  The per-(block, head) scales multiply the logits (K) and the
// block's fp32 P.V product (V).
#pragma once

#include "pa_device.h"

namespace pa {
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef short short4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));


// All-reduce over the lane pairs (l, l^32) and (l, l^16): each permlane swap
// returns, per lane, its own value and its partner's (in some order).
__device__ __forceinline__ float max_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float sum_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const bf16x2_t v = {(__bf16)lo, (__bf16)hi};   // round to nearest even
  return __builtin_bit_cast(uint32_t, v);
}

// Two e4m3 codes (bytes 0,1 or 2,3 of `w`) -> two bf16 values, exactly.
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t w, bool hi) {
  const bf16x2_t v = hi ? __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true)
                        : __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false);
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ int clamp_block(int blk, int num_blocks) {
  return blk < 0 ? 0 : (blk >= num_blocks ? num_blocks - 1 : blk);
}

// KV storage formats: bf16 values; e4m3 codes with per-(block, head) scales;
// int4 codes (value + 8, two per byte, element 2i in the low nibble) with
// per-(block, head) scales.
constexpr int kFmtBf16 = 0, kFmtFp8 = 1, kFmtInt4 = 2;

template <int D, int kFmt>
struct Tile {
  static constexpr int kKSteps = D / 32;                  // QK MFMAs (16x16x32)
  static constexpr int kE = D / 16;                       // V elements per lane per token = PV MFMAs
  static constexpr int kBits = kFmt == kFmtBf16 ? 16 : (kFmt == kFmtFp8 ? 8 : 4);
  static constexpr int kKWords = kKSteps * 8 * kBits / 32;   // K words per lane per block
  static constexpr int kVWords = kE * kBits / 32;            // V words per lane per token
  static constexpr bool kScaled = kFmt != kFmtBf16;
  static_assert(kVWords >= 1, "int4 needs head_dim 128");
  // byte offset of element `e` of the pool
  static __device__ __forceinline__ int64_t bytes(int64_t e) { return e * kBits / 8; }
};

// int4 code c (value c - 8) -> bf16 bits of 128 + c = value + 136, exactly
// (bf16 holds every integer up to 256).  A dot product over such values is
// the true one plus 136 times the sum of the other operand.
constexpr float kInt4Bias = 136.0f;

// Byte selectors of v_perm_b32 (__builtin_amdgcn_perm(src0, src1, sel)):
// output byte k takes byte sel[k] of the 8-byte value src0:src1 (0-3 from
// src1, 4-7 from src0).
__device__ __forceinline__ constexpr uint32_t perm_sel(uint32_t b0, uint32_t b1, uint32_t b2, uint32_t b3) {
  return b0 | (b1 << 8) | (b2 << 16) | (b3 << 24);
}

// 0x43004300 | (two codes at bits 0-3 and 16-19 of x): a word of bf16 pairs
// 128 + code, exactly (bf16 holds every integer up to 256).
// (One v_and_or_b32: the compiler would split it in two, since gfx950's
// three-operand encodings take no literal and at most one scalar operand.)
__device__ __forceinline__ uint32_t int4_halves_to_bf16x2(uint32_t x) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(x), "s"(0x000f000fu), "v"(0x43004300u));
  return r;
}

// 8 int4 codes of one K row (one word, element 2i in the low nibble of byte
// i) -> 4 words of bf16 pairs holding elements (0,4), (1,5), (2,6), (3,7):
// one shift and one and-or per word.  The query operand is put in the same
// order (int4_query_order), so the dot product is unchanged.
__device__ __forceinline__ void int4x8_to_bf16x8(uint32_t w, uint32_t* out) {
  out[0] = int4_halves_to_bf16x2(w);
  out[1] = int4_halves_to_bf16x2(w >> 4);
  out[2] = int4_halves_to_bf16x2(w >> 8);
  out[3] = int4_halves_to_bf16x2(w >> 12);
}

// 8 bf16 query elements in order -> the order int4x8_to_bf16x8 gives a K row.
__device__ __forceinline__ uint4 int4_query_order(uint4 q) {
  return make_uint4(__builtin_amdgcn_perm(q.z, q.x, perm_sel(0, 1, 4, 5)), __builtin_amdgcn_perm(q.z, q.x, perm_sel(2, 3, 6, 7)),
                    __builtin_amdgcn_perm(q.w, q.y, perm_sel(0, 1, 4, 5)), __builtin_amdgcn_perm(q.w, q.y, perm_sel(2, 3, 6, 7)));
}

// Load `W` 32-bit words from a 4*W-byte aligned address.
template <int W>
__device__ __forceinline__ void load_words(const uint8_t* p, uint32_t* w) {
  if constexpr (W % 4 == 0) {
#pragma unroll
    for (int i = 0; i < W / 4; ++i) {
      const uint4 v = reinterpret_cast<const uint4*>(p)[i];
      w[4 * i] = v.x; w[4 * i + 1] = v.y; w[4 * i + 2] = v.z; w[4 * i + 3] = v.w;
    }
  } else if constexpr (W == 2) {
    const uint2 v = *reinterpret_cast<const uint2*>(p);
    w[0] = v.x; w[1] = v.y;
  } else {
    static_assert(W == 1, "unsupported load width");
    w[0] = *reinterpret_cast<const uint32_t*>(p);
  }
}

// Store `W` 32-bit words to a 4*W-byte aligned address.
template <int W>
__device__ __forceinline__ void store_words(uint8_t* p, const uint32_t* w) {
  if constexpr (W % 4 == 0) {
#pragma unroll
    for (int i = 0; i < W / 4; ++i)
      reinterpret_cast<uint4*>(p)[i] = make_uint4(w[4 * i], w[4 * i + 1], w[4 * i + 2], w[4 * i + 3]);
  } else if constexpr (W == 2) {
    *reinterpret_cast<uint2*>(p) = make_uint2(w[0], w[1]);
  } else {
    static_assert(W == 1, "unsupported store width");
    *reinterpret_cast<uint32_t*>(p) = w[0];
  }
}

// NV bf16 values (NV/2 words) -> NV e4m3 codes (NV/4 words) of x / scale,
// IEEE division, saturating round-to-nearest-even (as the slot scatter does).
template <int NV>
__device__ __forceinline__ void quantize_bf16_words(const uint32_t* src, float scale, uint32_t* dst) {
#pragma unroll
  for (int i = 0; i < NV / 4; ++i) {
    uint32_t code = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int v = 4 * i + k;
      const uint32_t bits = (v & 1) ? (src[v / 2] >> 16) : (src[v / 2] & 0xffffu);
      code |= f32_to_e4m3_sat_rne(__fdiv_rn(bf16_bits_to_f32(bits), scale)) << (8 * k);
    }
    dst[i] = code;
  }
}

// NV bf16 values (NV/2 words) -> NV int4 codes (NV/8 words) of x / scale,
// IEEE division, round half to even, clamped to [-8, 7] (as the slot scatter does).
template <int NV>
__device__ __forceinline__ void quantize_bf16_words_int4(const uint32_t* src, float scale, uint32_t* dst) {
#pragma unroll
  for (int i = 0; i < NV / 8; ++i) {
    uint32_t code = 0;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int v = 8 * i + k;
      const uint32_t bits = (v & 1) ? (src[v / 2] >> 16) : (src[v / 2] & 0xffffu);
      code |= f32_to_int4_code(__fdiv_rn(bf16_bits_to_f32(bits), scale)) << (4 * k);
    }
    dst[i] = code;
  }
}

// One 16-token K/V block of one KV head, as this lane holds it.
template <int D, int kFmt>
struct BlockRegs {
  uint32_t k[Tile<D, kFmt>::kKWords];
  uint32_t v[4][Tile<D, kFmt>::kVWords];
};

template <int D, int kFmt>
__device__ __forceinline__ void load_block(BlockRegs<D, kFmt>& br, const uint8_t* kbase, const uint8_t* vbase,
                                           int64_t blk, int num_kv_heads, int g, int r, int c) {
  using T = Tile<D, kFmt>;
  // (a block base common to the wave plus a 32-bit lane offset: no 64-bit
  // address per lane to compute or keep)
  const int64_t head_bytes = T::bytes((blk * num_kv_heads + g) * kBlockTokens * D);
  const uint8_t* kb = kbase + head_bytes;
  const uint8_t* vb = vbase + head_bytes;
  load_words<T::kKWords>(kb + (uint32_t)T::bytes(r * D + (D / 4) * c), br.k);
#pragma unroll
  for (int e = 0; e < 4; ++e) load_words<T::kVWords>(vb + (uint32_t)T::bytes((4 * c + e) * D + T::kE * r), br.v[e]);
}

// The Q^T operand of HeadState::begin as raw registers: query rows
// q_row0 .. q_row0+G-1, lane r reading row min(r, G-1), so every lane issues
// the same loads with no lane-dependent branch (a caller can place them
// ahead of block loads).  Nothing here uses the loaded words, so they are
// only waited for where begin_loaded() takes them and zeroes lanes r >= G.
template <int D>
__device__ __forceinline__ void load_query(const uint16_t* q, int64_t q_row0, int G, int r, int c, uint4* qw) {
  const uint16_t* qp = q + q_row0 * D + (uint32_t)(min(r, G - 1) * D + (D / 4) * c);
#pragma unroll
  for (int i = 0; i < D / 32; ++i) qw[i] = reinterpret_cast<const uint4*>(qp)[i];
}

// A operands of a block's P.V MFMAs (V^T as bf16, one per d tile), built
// once per block and shared by every tile of query columns that folds the
// block in.  Tokens past `valid` get V = 0 by selection (their slots may
// hold NaN); a full block needs no selection.
template <int D, int kFmt>
struct VOperands {
  short4_t v[Tile<D, kFmt>::kE];
};

template <int D, int kFmt>
__device__ __forceinline__ VOperands<D, kFmt> make_voperands(const BlockRegs<D, kFmt>& br, int valid, int c) {
  using T = Tile<D, kFmt>;
  if constexpr (kFmt == kFmtInt4) {
    VOperands<D, kFmt> vo;
    // nibble nn of the 4 tokens' words -> [t0 t1 | t2 t3] as bf16 of 128 + code.
    // y01a: bytes 0-1 (codes 0-3) of tokens 0 and 1, one token per 16-bit
    // half; y01b: bytes 2-3 (codes 4-7); y23a, y23b the same for tokens 2, 3.
    // Code nn then sits at bits 4*(nn%4) of each half.  (Tokens past `valid`
    // need no masking here: every code gives a finite value, and their P is 0.)
    const uint32_t y01a = __builtin_amdgcn_perm(br.v[1][0], br.v[0][0], perm_sel(0, 1, 4, 5));
    const uint32_t y01b = __builtin_amdgcn_perm(br.v[1][0], br.v[0][0], perm_sel(2, 3, 6, 7));
    const uint32_t y23a = __builtin_amdgcn_perm(br.v[3][0], br.v[2][0], perm_sel(0, 1, 4, 5));
    const uint32_t y23b = __builtin_amdgcn_perm(br.v[3][0], br.v[2][0], perm_sel(2, 3, 6, 7));
#pragma unroll
    for (int nn = 0; nn < T::kE; ++nn) {
      const int sh = 4 * (nn % 4);
      const uint32_t lo = int4_halves_to_bf16x2((nn < 4 ? y01a : y01b) >> sh);
      const uint32_t hi = int4_halves_to_bf16x2((nn < 4 ? y23a : y23b) >> sh);
      vo.v[nn] = __builtin_bit_cast(short4_t, make_uint2(lo, hi));
    }
    return vo;
  }
  uint32_t vw[4][T::kVWords];
  if (valid < kBlockTokens) {
#pragma unroll
    for (int e = 0; e < 4; ++e)
#pragma unroll
      for (int w = 0; w < T::kVWords; ++w) vw[e][w] = 4 * c + e < valid ? br.v[e][w] : 0u;
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e)
#pragma unroll
      for (int w = 0; w < T::kVWords; ++w) vw[e][w] = br.v[e][w];
  }
  VOperands<D, kFmt> vo;
#pragma unroll
  for (int nn = 0; nn < T::kE; ++nn) {
    uint32_t lo, hi;
    if constexpr (kFmt == kFmtFp8) {
      // byte nn%4 of word nn/4 from each of the 4 tokens -> [t0 t1 | t2 t3] codes -> bf16 pairs
      const int w = nn / 4, byte = nn % 4;
      const uint32_t sel = (uint32_t)byte | ((uint32_t)(byte + 4) << 8) | 0x0c0c0000u;
      const uint32_t c01 = __builtin_amdgcn_perm(vw[1][w], vw[0][w], sel);
      const uint32_t c23 = __builtin_amdgcn_perm(vw[3][w], vw[2][w], sel);
      lo = fp8x2_to_bf16x2(c01, false);
      hi = fp8x2_to_bf16x2(c23, false);
    } else {
      const int w = nn / 2;
      const uint32_t sel = (nn & 1) ? 0x07060302u : 0x05040100u;
      lo = __builtin_amdgcn_perm(vw[1][w], vw[0][w], sel);
      hi = __builtin_amdgcn_perm(vw[3][w], vw[2][w], sel);
    }
    vo.v[nn] = __builtin_bit_cast(short4_t, make_uint2(lo, hi));
  }
  return vo;
}

// Probabilities are formed against a per-column reference max m (base 2)
// that moves only when a logit exceeds it by more than this: p = 2^(x - m)
// may reach 2^kLazyMax, harmless in fp32 and in bf16 (whose exponent range
// is fp32's), and the final division by l cancels the choice of m exactly.
constexpr float kLazyMax = 8.0f;

// Running state of one wave: G query heads of one KV head over a run of blocks.
template <int D, int kFmt>
struct HeadState {
  using T = Tile<D, kFmt>;
  static constexpr int kE = T::kE;
  static constexpr bool kInt4 = kFmt == kFmtInt4;
  bf16x8_t qop[T::kKSteps];
  f32x4_t acc[kE];
  float m, l;    // reference max (-inf until the column sees a token) and the sum of 2^(x - m)
  float nm;      // -m, or 0 while m = -inf: the offset of the FMA that forms relative logits
  float thr;     // a relative logit above this moves the reference: kLazyMax, or -inf while m = -inf
  float qbias;   // int4: 136 * (sum of this lane's query column): removed from every logit
  bool query_pending = false;   // int4: query still to be reordered and summed (begin_row)
  float vbias;   // int4: sum over blocks of V scale * (sum of the bf16 P of this lane's tokens),
                 // rescaled like acc; the column's total is the sum over its 4 lanes

  // Q^T operand for query rows q_row0 .. q_row0+G-1 (lane r < G), d chunk (D/32)*c + i.
  __device__ __forceinline__ void begin(const uint16_t* q, int64_t q_row0, int G, int r, int c) {
    const uint16_t* qp = q + (q_row0 + r) * D + (D / 4) * c;
#pragma unroll
    for (int i = 0; i < T::kKSteps; ++i) {
      uint4 w = make_uint4(0, 0, 0, 0);
      if (r < G) w = reinterpret_cast<const uint4*>(qp)[i];
      qop[i] = __builtin_bit_cast(bf16x8_t, w);
    }
    reset();
    take_query();
  }

  // Start a run from the words load_query() fetched (lanes r >= G get zeros).
  __device__ __forceinline__ void begin_loaded(const uint4* qw, int G, int r) {
#pragma unroll
    for (int i = 0; i < T::kKSteps; ++i) qop[i] = __builtin_bit_cast(bf16x8_t, r < G ? qw[i] : make_uint4(0, 0, 0, 0));
    reset();
    take_query();
  }

  // Q^T operand with an arbitrary query row per column: lane r takes row
  // `row`; a column that will see no token (every step masks it whole) may
  // pass -1 and gets row 0.  Every lane issues the same loads and nothing
  // here uses their values, so they are waited for at the first step (the
  // int4 reordering and query sum are done there too).
  __device__ __forceinline__ void begin_row(const uint16_t* q, int64_t row, int c) {
    const uint16_t* qp = q + (row < 0 ? 0 : row) * D + (D / 4) * c;
#pragma unroll
    for (int i = 0; i < T::kKSteps; ++i) qop[i] = __builtin_bit_cast(bf16x8_t, reinterpret_cast<const uint4*>(qp)[i]);
    reset();
    query_pending = kInt4;
  }

  // int4: put the query operand in the element order of the K operand
  // (int4x8_to_bf16x8) and take 136 times the column's query sum (the 4 lane
  // groups hold D/4 each).
  __device__ __forceinline__ void take_query() {
    qbias = 0.0f;
    if constexpr (kInt4) {
#pragma unroll
      for (int i = 0; i < T::kKSteps; ++i)
        qop[i] = __builtin_bit_cast(bf16x8_t, int4_query_order(__builtin_bit_cast(uint4, qop[i])));
      float s = 0.0f;
#pragma unroll
      for (int i = 0; i < T::kKSteps; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) s += (float)qop[i][j];
      qbias = kInt4Bias * sum_xor16(sum_xor32(s));
    }
  }

  __device__ __forceinline__ void reset() {
    m = -INFINITY;
    nm = 0.0f;
    thr = -INFINITY;
    l = 0.0f;
    vbias = 0.0f;
#pragma unroll
    for (int t = 0; t < kE; ++t) acc[t] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  }

  // Fold one block in.  `valid` = tokens of the block inside the context
  // (1..16), `sc` = scale*log2(e) (times the block's K scale for e4m3),
  // `vs` = the block's V scale.  Every column sees the same tokens.
  __device__ __forceinline__ void step(const BlockRegs<D, kFmt>& br, int valid, float sc, float vs, int c) {
    const VOperands<D, kFmt> vo = make_voperands<D, kFmt>(br, valid, c);
    step_impl<false>(br, vo, valid, 0, sc, vs, c);
  }

  // Fold one block in with a causal horizon per column: column r (this
  // lane's) sees only the block's first `col_valid` tokens (any integer;
  // <= 0 hides the whole block, >= 16 hides nothing).  `valid` still bounds
  // the tokens whose V rows hold data.  A column may see no token at all
  // (then m stays -inf, l = 0, acc = 0).  `vo`: the block's P.V operands
  // (make_voperands), shared by every tile that folds this block in.
  __device__ __forceinline__ void step_cols(const BlockRegs<D, kFmt>& br, const VOperands<D, kFmt>& vo, int valid,
                                            int col_valid, float sc, float vs, int c) {
    step_impl<true>(br, vo, valid, col_valid, sc, vs, c);
  }

  template <bool kCols>
  __device__ __forceinline__ void step_impl(const BlockRegs<D, kFmt>& br, const VOperands<D, kFmt>& vo, int valid,
                                            int col_valid, float sc, float vs, int c) {
    ready();
    // ---- S^T = K . Q^T
    f32x4_t s = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int st = 0; st < T::kKSteps; ++st)
      s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k_operand(br, st), qop[st], s, 0, 0, 0);
    float x[4];
    rel_logits(s, sc, x);
    if (valid < kBlockTokens) hide_tokens(x, valid, c);
    if constexpr (kCols) {
      // (a block every column sees in full needs no mask: wave-uniform test)
      if (__ballot(col_valid < kBlockTokens) != 0) hide_tokens(x, col_valid, c);
    }
    // ---- online softmax (base 2)
    fold<4>(x);
    const short4_t pop = probs(x, vs);
    pv(vo, pop, vs);
  }

  // Before a QK product: the query work begin_row deferred (int4).
  __device__ __forceinline__ void ready() {
    if constexpr (kInt4) {
      if (query_pending) {
        take_query();
        query_pending = false;
      }
    }
  }

  // The K operand of QK MFMA step st (K rows as bf16 pairs), the same for
  // every tile that folds the block in.
  static __device__ __forceinline__ bf16x8_t k_operand(const BlockRegs<D, kFmt>& br, int st) {
    uint4 kw;
    if constexpr (kFmt == kFmtFp8) {
      kw = make_uint4(fp8x2_to_bf16x2(br.k[2 * st], false), fp8x2_to_bf16x2(br.k[2 * st], true),
                      fp8x2_to_bf16x2(br.k[2 * st + 1], false), fp8x2_to_bf16x2(br.k[2 * st + 1], true));
    } else if constexpr (kInt4) {
      uint32_t w4[4];
      int4x8_to_bf16x8(br.k[st], w4);
      kw = make_uint4(w4[0], w4[1], w4[2], w4[3]);
    } else {
      kw = make_uint4(br.k[4 * st], br.k[4 * st + 1], br.k[4 * st + 2], br.k[4 * st + 3]);
    }
    return __builtin_bit_cast(bf16x8_t, kw);
  }

  // Base-2 logits of this lane's 4 scores relative to the reference max:
  // s * sc - m in one FMA (int4: also less 136 times the query sum, the
  // bias the MFMA saw).
  __device__ __forceinline__ void rel_logits(const f32x4_t& s, float sc, float* x) {
    const float off = kInt4 ? __builtin_fmaf(-qbias, sc, nm) : nm;
#pragma unroll
    for (int j = 0; j < 4; ++j) x[j] = __builtin_fmaf(s[j], sc, off);
  }

  // Remove the block's tokens from `limit` on (this lane's tokens 4c..4c+3).
  static __device__ __forceinline__ void hide_tokens(float* x, int limit, int c) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (4 * c + j >= limit) x[j] = -INFINITY;
  }

  // Take N relative logits of this lane's column into account: if any
  // exceeds the threshold (wave-uniform test), the columns concerned move
  // their reference to their maximum over these logits (across the 4 lane
  // groups), rescale l and the output by 2^(m - m_new), and shift x into
  // the new frame.  A column that has seen no token keeps m = -inf and
  // never forms -inf - (-inf).
  template <int N>
  __device__ __forceinline__ void fold(float* x) {
    float lm = x[0];
#pragma unroll
    for (int j = 1; j < N; ++j) lm = fmaxf(lm, x[j]);
    if (__ballot(lm > thr) != 0) {
      const float bm = max_xor16(max_xor32(lm));          // this column's maximum, relative to m
      const bool grow = bm > thr;
      const float m_new = grow ? bm - nm : m;              // (nm = 0 while m = -inf)
      const float alpha = grow ? __builtin_amdgcn_exp2f(m - m_new) : 1.0f;
      l *= alpha;
      if constexpr (kInt4) vbias *= alpha;
#pragma unroll
      for (int t = 0; t < kE; ++t) acc[t] *= alpha;
      const float shift = grow ? bm : 0.0f;
#pragma unroll
      for (int j = 0; j < N; ++j) x[j] -= shift;
      m = m_new;
      nm = grow ? -m_new : nm;
      thr = grow ? kLazyMax : thr;
    }
  }

  // The block's probabilities 2^x, added to l; returns them as the bf16 P
  // operand of the P.V MFMAs.
  __device__ __forceinline__ short4_t probs(const float* x, float vs) {
    float p[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) p[j] = __builtin_amdgcn_exp2f(x[j]);
    l += (p[0] + p[1]) + (p[2] + p[3]);
    // e4m3/int4: the block's V scale is applied in fp32 to the block's P.V
    // product (folding it into the bf16 P would put a relative 2^-9 error on
    // every V row); a bf16 cache has no V scale (callers pass vs = 1)
    const uint2 pbits = make_uint2(pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]));
    if constexpr (kInt4) {
      // the P.V MFMA sees V + 136: keep V scale * (sum of the bf16 P it used) to take off at the end
      // (this lane's 4 tokens, two dot products with (1, 1); the lanes are summed at the end)
      const bf16x2_t ones = __builtin_bit_cast(bf16x2_t, 0x3f803f80u);
      const float ps = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pbits.y), ones,
                                                       __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pbits.x), ones, 0.0f, false),
                                                       false);
      vbias = __builtin_fmaf(ps, vs, vbias);
    }
    return __builtin_bit_cast(short4_t, pbits);
  }

  // ---- O^T += V^T . P^T, one MFMA per d tile n (d = kE*r + n)
  __device__ __forceinline__ void pv(const VOperands<D, kFmt>& vo, short4_t pop, float vs) {
#pragma unroll
    for (int nn = 0; nn < kE; ++nn) {
      if constexpr (T::kScaled) {
        const f32x4_t t = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vo.v[nn], pop, f32x4_t{0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0);
        acc[nn] += t * vs;
      } else {
        acc[nn] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vo.v[nn], pop, acc[nn], 0, 0, 0);
      }
    }
  }

  __device__ __forceinline__ float total_l() const { return sum_xor16(sum_xor32(l)); }

  // int4: take the V bias out of acc itself (for callers that read acc directly)
  __device__ __forceinline__ void settle() {
    if constexpr (kInt4) {
      const float vb = kInt4Bias * sum_xor16(sum_xor32(vbias));
#pragma unroll
      for (int t = 0; t < kE; ++t) acc[t] -= vb;
      vbias = 0.0f;
    }
  }

  // Output run of this lane: d = (D/4)*c + kE*j + n  ->  o[kE*j + n].
  __device__ __forceinline__ void unpack(float* o) const {
    const float vb = kInt4 ? kInt4Bias * sum_xor16(sum_xor32(vbias)) : 0.0f;
#pragma unroll
    for (int nn = 0; nn < kE; ++nn)
#pragma unroll
      for (int j = 0; j < 4; ++j) o[kE * j + nn] = kInt4 ? acc[nn][j] - vb : acc[nn][j];
  }
};

// Fold one block into two tiles of columns (step_cols of each), phase by
// phase: both tiles' QK products, then both softmax updates, then both P.V
// products, so that one tile's MFMAs run under the other's vector work.
// The K operand is converted once for both.
template <int D, int kFmt>
__device__ __forceinline__ void step_cols2(HeadState<D, kFmt>& ha, HeadState<D, kFmt>& hb, const BlockRegs<D, kFmt>& br,
                                           const VOperands<D, kFmt>& vo, int valid, int col_valid_a, int col_valid_b,
                                           float sc, float vs, int c) {
  using H = HeadState<D, kFmt>;
  ha.ready();
  hb.ready();
  f32x4_t sa = {0.0f, 0.0f, 0.0f, 0.0f}, sb = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int st = 0; st < Tile<D, kFmt>::kKSteps; ++st) {
    const bf16x8_t k = H::k_operand(br, st);
    sa = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k, ha.qop[st], sa, 0, 0, 0);
    sb = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k, hb.qop[st], sb, 0, 0, 0);
  }
  float xa[4], xb[4];
  ha.rel_logits(sa, sc, xa);
  hb.rel_logits(sb, sc, xb);
  // one wave-uniform test for the context end and both tiles' horizons
  if (valid < kBlockTokens || __ballot(col_valid_a < kBlockTokens || col_valid_b < kBlockTokens) != 0) {
    H::hide_tokens(xa, min(valid, col_valid_a), c);
    H::hide_tokens(xb, min(valid, col_valid_b), c);
  }
  ha.template fold<4>(xa);
  hb.template fold<4>(xb);
  const short4_t pa = ha.probs(xa, vs), pb = hb.probs(xb, vs);
  ha.pv(vo, pa, vs);
  hb.pv(vo, pb, vs);
}

// The same value, which the compiler must take as computed at this point
// (an empty asm statement): an address built from it cannot be hoisted and
// kept in registers across a loop.
__device__ __forceinline__ int fresh(int v) {
  asm volatile("" : "+v"(v));
  return v;
}

// Finished rows leave a wave through LDS, this many rows per pass.
constexpr int kStageRows = 8;

// Make this wave's LDS writes visible to its other lanes' later LDS reads
// (and finish its reads before later writes): wait for the wave's LDS
// operations, and keep the compiler from moving LDS accesses across.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_s_waitcnt(0xc07f);    // lgkmcnt(0); vmcnt and expcnt left alone
  __builtin_amdgcn_wave_barrier();
}

// Write D/4 normalised values of one query row as bf16 (16-byte stores).
template <int D>
__device__ __forceinline__ void store_bf16_run(uint16_t* dst_row, int d0, const float* o, float inv) {
  uint32_t* dst = reinterpret_cast<uint32_t*>(dst_row + d0);
#pragma unroll
  for (int i = 0; i < D / 8; i += 4) {
    const uint4 w = make_uint4(pack_bf16x2(o[2 * i] * inv, o[2 * i + 1] * inv),
                               pack_bf16x2(o[2 * i + 2] * inv, o[2 * i + 3] * inv),
                               pack_bf16x2(o[2 * i + 4] * inv, o[2 * i + 5] * inv),
                               pack_bf16x2(o[2 * i + 6] * inv, o[2 * i + 7] * inv));
    *reinterpret_cast<uint4*>(dst + i) = w;
  }
}

// Write D/4 unnormalised fp32 values of one workspace row.
template <int D>
__device__ __forceinline__ void store_f32_run(float* dst_row, int d0, const float* o) {
  float4* dst = reinterpret_cast<float4*>(dst_row + d0);
#pragma unroll
  for (int i = 0; i < D / 16; ++i) dst[i] = make_float4(o[4 * i], o[4 * i + 1], o[4 * i + 2], o[4 * i + 3]);
}

}  // namespace pa
