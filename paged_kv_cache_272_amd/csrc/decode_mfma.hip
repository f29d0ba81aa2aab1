// Paged decode on the matrix cores (gfx950 MFMA), bf16 query with a bf16 or
// e4m3 KV cache.
//
// What is computed is the attention of "系统级优化…" section 3.1 for one
// query token per sequence, over K/V gathered page by page through the block
// table (section 2.3), with the online-softmax tiling idea of section 3.2
// (the running-max rescale that page omits is applied exactly).
//
// Work split.  One workgroup of 4 waves per (partition, KV head, sequence);
// wave w takes the partition's 16-token blocks w, w+4, ... and keeps its
// own running max / sum / output; the 4 waves merge through LDS at the end.
// A single wave holds one K/V block in registers and applies it to all G
// query heads of the GQA group at once: the heads are the N dimension of
// the MFMAs, so each block is read from HBM exactly once per group.
//
// Per block (16 tokens), lane l = 16*c + r (r = l%16, c = l/16):
//   QK:  S^T[token][head] = K[token][:] . Q[head][:]  with D/32 MFMAs
//        16x16x32 bf16.  A = K: lane holds 8 consecutive d of token r
//        (row r), B = Q^T: lane holds the same 8 d of head r.  The d chunk
//        for k-step i and lane group c is (D/32)*c + i, so a lane reads one
//        contiguous D/4-element run of its token's row.
//        Result: lane holds s[j] = S^T[token 4c+j][head r], j = 0..3.
//   softmax: scale, mask past the context by select, block max over the
//        4 lane groups (permlane swaps), running max / sum update; the
//        output is rescaled only when some running max grew.
//   PV:  O^T[d][head] += V^T[d][token] . P^T[token][head] with D/16 MFMAs
//        16x16x16 bf16.  B = P^T: lane holds p[j] for tokens 4c..4c+3 of
//        head r, which is exactly the QK result layout, so P never leaves
//        registers.  A = V^T: lane holds tokens 4c..4c+3 of one d; V is
//        loaded row-contiguously (16 lanes per 256-byte token row) and the
//        4x(D/16) sub-tile is transposed in registers with byte permutes.
//        Tile n covers d = (D/16)*r + n, so lane (r, c) ends up holding the
//        contiguous output run d in [(D/4)c, (D/4)(c+1)) of head r.
// e4m3 codes are widened to bf16 exactly (every e4m3 value is a bf16
// value); the per-(block, head) scales multiply the logits (K) and the
// probabilities fed to P.V (V).
#include "pa_device.h"
#include "pa_internal.h"

namespace pa {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef short short4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;

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

template <int D, bool kFp8>
struct Tile {
  static constexpr int kKSteps = D / 32;                  // QK MFMAs (16x16x32)
  static constexpr int kE = D / 16;                       // V elements per lane per token = PV MFMAs
  static constexpr int kEb = kFp8 ? 1 : 2;
  static constexpr int kKWords = kKSteps * 8 * kEb / 4;   // K words per lane per block
  static constexpr int kVWords = kE * kEb / 4;            // V words per lane per token
};

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

template <int D, bool kFp8>
struct BlockRegs {
  uint32_t k[Tile<D, kFp8>::kKWords];
  uint32_t v[4][Tile<D, kFp8>::kVWords];
};

template <int D, bool kFp8>
__device__ __forceinline__ void load_block(BlockRegs<D, kFp8>& br, const uint8_t* kbase, const uint8_t* vbase,
                                           int64_t blk, int num_kv_heads, int g, int r, int c) {
  using T = Tile<D, kFp8>;
  const int64_t head_base = (blk * num_kv_heads + g) * kBlockTokens;            // token row index
  load_words<T::kKWords>(kbase + ((head_base + r) * D + (D / 4) * c) * T::kEb, br.k);
#pragma unroll
  for (int e = 0; e < 4; ++e)
    load_words<T::kVWords>(vbase + ((head_base + 4 * c + e) * D + T::kE * r) * T::kEb, br.v[e]);
}

template <int D, bool kFp8>
__global__ __launch_bounds__(kThreads) void decode_mfma_kernel(DecodeArgs a) {
  using T = Tile<D, kFp8>;
  constexpr int kE = T::kE;
  __shared__ float lds_m[kWaves][16];
  __shared__ float lds_l[kWaves][16];
  __shared__ f32x4_t lds_acc[kWaves][kE][64];

  const int part = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r = lane & 15, c = lane >> 4;
  const int G = a.num_q_heads / a.num_kv_heads;
  const int P = a.partition_tokens;

  int ctx = a.context_lens[b];
  ctx = ctx < 0 ? 0 : min(min(ctx, a.max_context_len), a.max_blocks_per_seq * kBlockTokens);
  const int nparts = (ctx + P - 1) / P;
  const int64_t head0 = (int64_t)b * a.num_q_heads + (int64_t)g * G;
  uint16_t* out = reinterpret_cast<uint16_t*>(a.out);
  if (ctx == 0) {
    if (part == 0)
      for (int i = threadIdx.x; i < G * D; i += kThreads) out[head0 * D + i] = 0;
    return;
  }
  const int t0 = part * P;
  if (t0 >= ctx) return;
  const int n = min(P, ctx - t0);
  const int nblk = (n + kBlockTokens - 1) / kBlockTokens;
  const int nw = wave < nblk ? (nblk - wave + kWaves - 1) / kWaves : 0;   // blocks of this wave

  // Q^T operand: head r (zero for r >= G), d chunk (D/32)*c + i.
  bf16x8_t qop[T::kKSteps];
  {
    const uint16_t* q = reinterpret_cast<const uint16_t*>(a.q) + (head0 + r) * D + (D / 4) * c;
#pragma unroll
    for (int i = 0; i < T::kKSteps; ++i) {
      uint4 w = make_uint4(0, 0, 0, 0);
      if (r < G) w = reinterpret_cast<const uint4*>(q)[i];
      qop[i] = __builtin_bit_cast(bf16x8_t, w);
    }
  }
  // physical ids (and fp8 scales) of this wave's blocks: lane j holds block j
  int my_blk = 0;
  float my_ks = 1.0f, my_vs = 1.0f;
  if (lane < nw) {
    int blk = a.block_tables[(int64_t)b * a.max_blocks_per_seq + t0 / kBlockTokens + wave + kWaves * lane];
    my_blk = blk < 0 ? 0 : (blk >= a.num_blocks ? a.num_blocks - 1 : blk);
    if constexpr (kFp8) {
      my_ks = a.k_scale[(int64_t)my_blk * a.num_kv_heads + g];
      my_vs = a.v_scale[(int64_t)my_blk * a.num_kv_heads + g];
    }
  }

  const uint8_t* kbase = reinterpret_cast<const uint8_t*>(a.k_cache);
  const uint8_t* vbase = reinterpret_cast<const uint8_t*>(a.v_cache);
  float m = -INFINITY, l = 0.0f;
  f32x4_t acc[kE];
#pragma unroll
  for (int t = 0; t < kE; ++t) acc[t] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};

  auto compute = [&](const BlockRegs<D, kFp8>& br, int i) {
    // ---- S^T = K . Q^T
    f32x4_t s = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int st = 0; st < T::kKSteps; ++st) {
      uint4 kw;
      if constexpr (kFp8) {
        kw = make_uint4(fp8x2_to_bf16x2(br.k[2 * st], false), fp8x2_to_bf16x2(br.k[2 * st], true),
                        fp8x2_to_bf16x2(br.k[2 * st + 1], false), fp8x2_to_bf16x2(br.k[2 * st + 1], true));
      } else {
        kw = make_uint4(br.k[4 * st], br.k[4 * st + 1], br.k[4 * st + 2], br.k[4 * st + 3]);
      }
      s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, kw), qop[st], s, 0, 0, 0);
    }
    float sc = a.scale_log2;
    float vs = 1.0f;
    if constexpr (kFp8) {
      sc *= __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(my_ks), i));
      vs = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(my_vs), i));
    }
    float sv[4] = {s[0] * sc, s[1] * sc, s[2] * sc, s[3] * sc};
    const int valid = n - (wave + kWaves * i) * kBlockTokens;   // tokens of this block inside the context
    uint32_t vmask = 0xffffffffu;                                // per-token keep mask for V (bit e)
    if (valid < kBlockTokens) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (4 * c + j >= valid) sv[j] = -INFINITY;
      vmask = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) vmask |= (4 * c + e < valid) ? (1u << e) : 0u;
    }
    // ---- online softmax (base 2)
    float mx = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
    mx = max_xor16(max_xor32(mx));
    const float m_new = fmaxf(m, mx);
    if (__ballot(m_new > m) != 0) {
      const float alpha = __builtin_amdgcn_exp2f(m - m_new);
      l *= alpha;
#pragma unroll
      for (int t = 0; t < kE; ++t) acc[t] *= alpha;
      m = m_new;
    }
    float p[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) p[j] = __builtin_amdgcn_exp2f(sv[j] - m);
    l += (p[0] + p[1]) + (p[2] + p[3]);
    const short4_t pop = __builtin_bit_cast(
        short4_t, make_uint2(pack_bf16x2(p[0] * vs, p[1] * vs), pack_bf16x2(p[2] * vs, p[3] * vs)));
    // ---- O^T += V^T . P^T, one MFMA per d tile n (d = kE*r + n)
    uint32_t vw[4][T::kVWords];
#pragma unroll
    for (int e = 0; e < 4; ++e)
#pragma unroll
      for (int w = 0; w < T::kVWords; ++w) vw[e][w] = (vmask >> e & 1u) ? br.v[e][w] : 0u;
#pragma unroll
    for (int nn = 0; nn < kE; ++nn) {
      uint32_t lo, hi;
      if constexpr (kFp8) {
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
      const short4_t vop = __builtin_bit_cast(short4_t, make_uint2(lo, hi));
      acc[nn] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vop, pop, acc[nn], 0, 0, 0);
    }
  };

  // software pipeline: the next block's loads are in flight while this one computes
  BlockRegs<D, kFp8> b0, b1;
  if (nw > 0) load_block<D, kFp8>(b0, kbase, vbase, __builtin_amdgcn_readlane(my_blk, 0), a.num_kv_heads, g, r, c);
  for (int i = 0; i < nw; i += 2) {
    if (i + 1 < nw)
      load_block<D, kFp8>(b1, kbase, vbase, __builtin_amdgcn_readlane(my_blk, i + 1), a.num_kv_heads, g, r, c);
    compute(b0, i);
    if (i + 1 < nw) {
      if (i + 2 < nw)
        load_block<D, kFp8>(b0, kbase, vbase, __builtin_amdgcn_readlane(my_blk, i + 2), a.num_kv_heads, g, r, c);
      compute(b1, i + 1);
    }
  }

  // ---- wave totals, then the 4-wave merge through LDS
  l = sum_xor16(sum_xor32(l));
  if (c == 0) {
    lds_m[wave][r] = m;
    lds_l[wave][r] = l;
  }
#pragma unroll
  for (int t = 0; t < kE; ++t) lds_acc[wave][t][lane] = acc[t];
  __syncthreads();
  if (wave != 0) return;

  float mw[kWaves], M = -INFINITY;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    mw[w] = lds_m[w][r];
    M = fmaxf(M, mw[w]);
  }
  float L = 0.0f, wt[kWaves];
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    wt[w] = __builtin_amdgcn_exp2f(mw[w] - M);   // waves without blocks have m = -inf -> 0
    L += wt[w] * lds_l[w][r];
  }
  float o[4 * kE];   // d = (D/4)*c + kE*j + nn  ->  o[kE*j + nn]
#pragma unroll
  for (int nn = 0; nn < kE; ++nn) {
    f32x4_t v = lds_acc[0][nn][lane] * wt[0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) v += lds_acc[w][nn][lane] * wt[w];
#pragma unroll
    for (int j = 0; j < 4; ++j) o[kE * j + nn] = v[j];
  }
  if (r >= G) return;
  const int64_t row = head0 + r;
  const int d0 = (D / 4) * c;
  if (nparts == 1) {
    const float inv = 1.0f / L;
    uint32_t* dst = reinterpret_cast<uint32_t*>(out + row * D + d0);
#pragma unroll
    for (int i = 0; i < 2 * kE; i += 4) {
      uint4 w = make_uint4(pack_bf16x2(o[2 * i] * inv, o[2 * i + 1] * inv),
                           pack_bf16x2(o[2 * i + 2] * inv, o[2 * i + 3] * inv),
                           pack_bf16x2(o[2 * i + 4] * inv, o[2 * i + 5] * inv),
                           pack_bf16x2(o[2 * i + 6] * inv, o[2 * i + 7] * inv));
      *reinterpret_cast<uint4*>(dst + i) = w;
    }
  } else {
    const int64_t wr = row * a.num_parts + part;
    float4* dst = reinterpret_cast<float4*>(a.ws_acc + wr * D + d0);
#pragma unroll
    for (int i = 0; i < kE; ++i) dst[i] = make_float4(o[4 * i], o[4 * i + 1], o[4 * i + 2], o[4 * i + 3]);
    if (c == 0) {
      a.ws_m[wr] = M;
      a.ws_l[wr] = L;
    }
  }
}

}  // namespace

hipError_t launch_decode_mfma(const DecodeArgs& a, hipStream_t stream) {
  const dim3 grid(a.num_parts, a.num_kv_heads, a.num_seqs);
  const bool fp8 = a.cache_dtype == PA_DTYPE_FP8_E4M3;
  if (a.head_dim == 128) {
    if (fp8) hipLaunchKernelGGL((decode_mfma_kernel<128, true>), grid, dim3(kThreads), 0, stream, a);
    else hipLaunchKernelGGL((decode_mfma_kernel<128, false>), grid, dim3(kThreads), 0, stream, a);
  } else {
    if (fp8) hipLaunchKernelGGL((decode_mfma_kernel<64, true>), grid, dim3(kThreads), 0, stream, a);
    else hipLaunchKernelGGL((decode_mfma_kernel<64, false>), grid, dim3(kThreads), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace pa
