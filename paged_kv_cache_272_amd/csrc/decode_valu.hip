// Paged decode on the vector ALUs for an fp32 query and an fp32 cache (the
// matrix cores take bf16 operands, so this path keeps full fp32 precision).
//
// out[b, h] = softmax(scale * q[b, h] . K_b^T) V_b for one query token per
// sequence ("系统级优化…", section 3.1), where K_b, V_b are gathered page by
// page through the block table ("系统级优化…", section 2.3).  Query head h
// reads KV head h / G (consecutive groups).
//
// One workgroup (4 waves) per (partition, KV head, sequence).  A partition
// is a run of `partition_tokens` tokens; its G query heads' scores live in
// LDS, so the partition is processed with an exact softmax over its tokens
// and emitted as (max, sum, unnormalised output) for the merge kernel, or
// as the final output when the sequence has a single partition.  Logits are
// kept in the base-2 domain (q is pre-scaled by scale*log2 e).
//
// Masking: tokens at or past the context length get a score of -inf by
// selection, and the P.V loop never touches them, so NaN in unused slots
// cannot reach the output.
//
// The merge kernel below also serves the matrix-core partition grid (bf16
// query), whose partial rows have the same layout.
#include "pa_device.h"
#include "pa_internal.h"

namespace pa {
namespace {

constexpr int kThreads = 256;
constexpr int kMaxGroup = 16;

// Load N consecutive fp32 cache elements (16-byte aligned, N a multiple of 4).
template <int N>
__device__ __forceinline__ void load_elems(const float* p, float* out) {
  const float4* v = reinterpret_cast<const float4*>(p);
#pragma unroll
  for (int i = 0; i < N / 4; ++i) {
    const float4 w = v[i];
    out[4 * i] = w.x; out[4 * i + 1] = w.y; out[4 * i + 2] = w.z; out[4 * i + 3] = w.w;
  }
}

template <bool kQBf16>
__device__ __forceinline__ void store_out(void* out, int64_t idx, float v) {
  if constexpr (kQBf16) reinterpret_cast<uint16_t*>(out)[idx] = (uint16_t)f32_to_bf16_bits_rne(v);
  else reinterpret_cast<float*>(out)[idx] = v;
}

__device__ __forceinline__ int seq_context(const DecodeArgs& a, int b) {
  int ctx = a.context_lens[b];
  ctx = ctx < 0 ? 0 : ctx;
  ctx = min(ctx, a.max_context_len);
  return min(ctx, a.max_blocks_per_seq * kBlockTokens);
}

__device__ __forceinline__ int64_t phys_block(const DecodeArgs& a, int b, int logical) {
  int blk = a.block_tables[(int64_t)b * a.max_blocks_per_seq + logical];
  blk = blk < 0 ? 0 : (blk >= a.num_blocks ? a.num_blocks - 1 : blk);
  return blk;
}

template <int D>
__global__ __launch_bounds__(kThreads) void decode_valu_kernel(DecodeArgs a) {
  constexpr int kDQ = D / 4;            // elements of a K row per lane (4 lanes per token)
  __shared__ float q_s[kMaxGroup][D];
  __shared__ float s_s[kMaxGroup][kMaxPartitionTokens];
  __shared__ float m_s[kMaxGroup], l_s[kMaxGroup];

  const int part = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int G = a.num_q_heads / a.num_kv_heads;
  const int P = a.partition_tokens;
  const int ctx = seq_context(a, b);
  const int nparts = (ctx + P - 1) / P;
  const int64_t head0 = (int64_t)b * a.num_q_heads + (int64_t)g * G;   // first query head row

  if (ctx == 0) {
    if (part == 0)
      for (int i = threadIdx.x; i < G * D; i += kThreads) store_out<false>(a.out, head0 * D + i, 0.0f);
    return;
  }
  const int t0 = part * P;
  if (t0 >= ctx) return;
  const int n = min(P, ctx - t0);

  for (int i = threadIdx.x; i < G * D; i += kThreads)
    q_s[i / D][i % D] = reinterpret_cast<const float*>(a.q)[head0 * D + i] * a.scale_log2;
  __syncthreads();

  // Phase 1: scores.  Wave w takes blocks w, w+4, ...; lane -> (token lane/4, quarter lane%4).
  const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
  const int tok = lane / 4, quarter = lane % 4;
  const int nblk = (n + kBlockTokens - 1) / kBlockTokens;
  const float* kbase = reinterpret_cast<const float*>(a.k_cache);
  for (int i = wave; i < nblk; i += 4) {
    const int logical = t0 / kBlockTokens + i;
    const int64_t phys = phys_block(a, b, logical);
    const int64_t row = ((phys * a.num_kv_heads + g) * kBlockTokens + tok) * D + quarter * kDQ;
    float kv[kDQ];
    load_elems<kDQ>(kbase + row, kv);
    const int t = i * kBlockTokens + tok;   // token index inside the partition
    for (int h = 0; h < G; ++h) {
      float acc = 0.0f;
#pragma unroll
      for (int d = 0; d < kDQ; ++d) acc += q_s[h][quarter * kDQ + d] * kv[d];
      acc += __shfl_xor(acc, 1, 64);
      acc += __shfl_xor(acc, 2, 64);
      if (quarter == 0) s_s[h][t] = (t < n) ? acc : -INFINITY;
    }
  }
  __syncthreads();

  // Phase 2: per-head max and sum over the partition's tokens.
  for (int h = wave; h < G; h += 4) {
    float m = -INFINITY;
    for (int t = lane; t < n; t += 64) m = fmaxf(m, s_s[h][t]);
    m = wave_max(m);
    float l = 0.0f;
    for (int t = lane; t < n; t += 64) {
      const float e = exp2f(s_s[h][t] - m);
      s_s[h][t] = e;
      l += e;
    }
    l = wave_sum(l);
    if (lane == 0) { m_s[h] = m; l_s[h] = l; }
  }
  __syncthreads();

  // Phase 3: P.V.  Thread -> (column d, head slice hs); heads hs, hs+HS, ...
  constexpr int kHS = kThreads / D;
  constexpr int kMaxPer = kMaxGroup / kHS;
  const int d = threadIdx.x % D, hs = threadIdx.x / D;
  float acc[kMaxPer];
#pragma unroll
  for (int j = 0; j < kMaxPer; ++j) acc[j] = 0.0f;
  const float* vbase = reinterpret_cast<const float*>(a.v_cache);
  for (int i = 0; i < nblk; ++i) {
    const int64_t phys = phys_block(a, b, t0 / kBlockTokens + i);
    const int64_t base = (phys * a.num_kv_heads + g) * kBlockTokens * D + d;
    const int tn = min(kBlockTokens, n - i * kBlockTokens);
    for (int tt = 0; tt < tn; ++tt) {
      const float v = vbase[base + (int64_t)tt * D];
      const int t = i * kBlockTokens + tt;
#pragma unroll
      for (int j = 0; j < kMaxPer; ++j) {
        const int h = hs + j * kHS;
        if (h < G) acc[j] += s_s[h][t] * v;
      }
    }
  }

  if (nparts == 1) {
#pragma unroll
    for (int j = 0; j < kMaxPer; ++j) {
      const int h = hs + j * kHS;
      if (h < G) store_out<false>(a.out, (head0 + h) * D + d, acc[j] / l_s[h]);
    }
  } else {
#pragma unroll
    for (int j = 0; j < kMaxPer; ++j) {
      const int h = hs + j * kHS;
      if (h < G) {
        const int64_t r = (head0 + h) * a.num_recs + part;     // (a record per partition here)
        a.ws_acc[r * D + d] = acc[j];
        if (d == 0) { a.ws_m[r] = m_s[h]; a.ws_l[r] = l_s[h]; }
      }
    }
  }
}

// Merge: one workgroup per (query head, sequence) over its partial records
// (one per partition from the kernel above; one per group of parts_per_rec
// partitions from the matrix-core grid).  Thread (lp, ch) owns the 4-wide
// output chunk ch and the records lp, lp + P', ... (P' = 256 / (D/4) lanes),
// folded with a running maximum four at a time so their loads are in flight
// together; the lanes are combined in LDS.
//   out = sum_p 2^(m_p - M) acc_p / sum_p 2^(m_p - M) l_p,  M = max_p m_p.
constexpr int kMergeThreads = 256;

template <bool kQBf16, int D>
__global__ __launch_bounds__(kMergeThreads) void decode_merge_kernel(DecodeArgs a) {
  constexpr int kChunks = D / 4;
  constexpr int kLanesP = kMergeThreads / kChunks;
  __shared__ float s_m[kLanesP][kChunks];
  __shared__ float s_l[kLanesP][kChunks];
  __shared__ float4 s_acc[kLanesP][kChunks];
  const int h = blockIdx.x, b = blockIdx.y;
  const int ch = threadIdx.x % kChunks, lp = threadIdx.x / kChunks;
  const int P = a.partition_tokens * a.parts_per_rec;    // tokens per record
  const int ctx = seq_context(a, b);
  const int nparts = (ctx + P - 1) / P;                  // records of this sequence
  if (nparts <= 1) return;            // written by the partition kernel
  const int64_t row = (int64_t)b * a.num_q_heads + h;
  const float* m = a.ws_m + row * a.num_recs;
  const float* l = a.ws_l + row * a.num_recs;
  const float4* acc = reinterpret_cast<const float4*>(a.ws_acc + row * a.num_recs * D);
  float M = -INFINITY, den = 0.0f;
  float4 num = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  for (int p0 = lp; p0 < nparts; p0 += 4 * kLanesP) {
    float mv[4], lv[4];
    float4 av[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int p = p0 + k * kLanesP;
      if (p < nparts) {
        mv[k] = m[p];
        lv[k] = l[p];
        av[k] = acc[(int64_t)p * kChunks + ch];
      } else {
        mv[k] = -INFINITY;
        lv[k] = 0.0f;
        av[k] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
      }
    }
    const float Mn = fmaxf(M, fmaxf(fmaxf(mv[0], mv[1]), fmaxf(mv[2], mv[3])));
    const float sc = exp2f(M - Mn);                 // 0 while M is still -inf
    den *= sc;
    num.x *= sc; num.y *= sc; num.z *= sc; num.w *= sc;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float w = exp2f(mv[k] - Mn);            // 0 for the padding entries
      den += w * lv[k];
      num.x += w * av[k].x; num.y += w * av[k].y; num.z += w * av[k].z; num.w += w * av[k].w;
    }
    M = Mn;
  }
  s_m[lp][ch] = M;
  s_l[lp][ch] = den;
  s_acc[lp][ch] = num;
  __syncthreads();
  if (lp != 0) return;
  float MM = -INFINITY;
#pragma unroll
  for (int i = 0; i < kLanesP; ++i) MM = fmaxf(MM, s_m[i][ch]);
  float dd = 0.0f;
  float4 nn = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
#pragma unroll
  for (int i = 0; i < kLanesP; ++i) {
    const float w = s_m[i][ch] == -INFINITY ? 0.0f : exp2f(s_m[i][ch] - MM);   // lanes without partitions
    dd += w * s_l[i][ch];
    const float4 v = s_acc[i][ch];
    nn.x += w * v.x; nn.y += w * v.y; nn.z += w * v.z; nn.w += w * v.w;
  }
  const float inv = 1.0f / dd;
  const int64_t o = row * D + 4 * ch;
  store_out<kQBf16>(a.out, o, nn.x * inv);
  store_out<kQBf16>(a.out, o + 1, nn.y * inv);
  store_out<kQBf16>(a.out, o + 2, nn.z * inv);
  store_out<kQBf16>(a.out, o + 3, nn.w * inv);
}

hipError_t launch_valu(const DecodeArgs& a, hipStream_t stream) {
  const dim3 grid(a.num_parts, a.num_kv_heads, a.num_seqs);
  if (a.head_dim == 64)
    hipLaunchKernelGGL((decode_valu_kernel<64>), grid, dim3(kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL((decode_valu_kernel<128>), grid, dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_partitions(const DecodeArgs& a, hipStream_t stream) {
  if (a.q_dtype == PA_DTYPE_F32) return launch_valu(a, stream);
  return launch_decode_mfma(a, stream);
}

hipError_t launch_decode_merge(const DecodeArgs& a, hipStream_t stream) {
  const dim3 grid(a.num_q_heads, a.num_seqs);
  const bool bf16 = a.q_dtype == PA_DTYPE_BF16;
  const dim3 block(kMergeThreads);
  if (a.head_dim == 64) {
    if (bf16) hipLaunchKernelGGL((decode_merge_kernel<true, 64>), grid, block, 0, stream, a);
    else hipLaunchKernelGGL((decode_merge_kernel<false, 64>), grid, block, 0, stream, a);
  } else {
    if (bf16) hipLaunchKernelGGL((decode_merge_kernel<true, 128>), grid, block, 0, stream, a);
    else hipLaunchKernelGGL((decode_merge_kernel<false, 128>), grid, block, 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace pa
