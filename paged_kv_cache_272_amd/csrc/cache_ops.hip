// Slot scatter of new K/V into pages, and whole-block copy for copy-on-write.
//
// Slot scatter: the paged form of appending new keys/values to a KV cache
// ("推理优化", section 二 Step 1), with token positions mapped to
// (block, offset) through the block table ("系统级优化…", section 2.3).
// Block copy: the copy step of copy-on-write ("17 · 连续批处理与
// PagedAttention", section 三).
//
// Both are pure data movement (plus the e4m3 or int4 encode of new rows):
// one workgroup per (token or pair, K or V), vector loads and stores,
// 64-bit address arithmetic.
#include "pa_device.h"
#include "pa_internal.h"

namespace pa {
namespace {

constexpr int kCopyThreads = 256;
constexpr int kWriteThreads = 128;

// Slot of token t: given, or the newest position of sequence t.
__device__ __forceinline__ int64_t token_slot(const CacheWriteArgs& a, int t) {
  if (a.slot_mapping) return a.slot_mapping[t];
  const int ctx = a.context_lens[t];
  if (ctx <= 0 || ctx > a.max_blocks_per_seq * kBlockTokens) return -1;
  const int blk = a.block_tables[(int64_t)t * a.max_blocks_per_seq + (ctx - 1) / kBlockTokens];
  return (int64_t)blk * kBlockTokens + (ctx - 1) % kBlockTokens;
}

// Copy one token's [Hkv, D] row (bit copy; f32 or bf16).
__global__ __launch_bounds__(kWriteThreads) void cache_write_copy_kernel(CacheWriteArgs a, int elem_bytes) {
  const int t = blockIdx.x;
  const bool is_v = blockIdx.y != 0;
  const int64_t slot = token_slot(a, t);
  if (slot < 0 || slot >= (int64_t)a.num_blocks * kBlockTokens) return;
  const int64_t blk = slot / kBlockTokens;
  const int off = (int)(slot % kBlockTokens);
  const int row_chunks = a.head_dim * elem_bytes / 16;   // 16-byte chunks per head row
  const int chunks = a.num_kv_heads * row_chunks;
  const uint4* src = reinterpret_cast<const uint4*>(is_v ? a.v : a.k) + (int64_t)t * chunks;
  uint4* cache = reinterpret_cast<uint4*>(is_v ? a.v_cache : a.k_cache);
  for (int i = threadIdx.x; i < chunks; i += kWriteThreads) {
    const int h = i / row_chunks, c = i % row_chunks;
    const int64_t dst = ((blk * a.num_kv_heads + h) * kBlockTokens + off) * row_chunks + c;
    cache[dst] = src[i];
  }
}

// Quantise one token's [Hkv, D] row to e4m3 with the destination block's scale.
template <bool kSrcBf16>
__global__ __launch_bounds__(kWriteThreads) void cache_write_fp8_kernel(CacheWriteArgs a) {
  const int t = blockIdx.x;
  const bool is_v = blockIdx.y != 0;
  const int64_t slot = token_slot(a, t);
  if (slot < 0 || slot >= (int64_t)a.num_blocks * kBlockTokens) return;
  const int64_t blk = slot / kBlockTokens;
  const int off = (int)(slot % kBlockTokens);
  const int row_groups = a.head_dim / 8;                 // groups of 8 values -> 8 code bytes
  const int groups = a.num_kv_heads * row_groups;
  const float* scales = is_v ? a.v_scale : a.k_scale;
  uint2* cache = reinterpret_cast<uint2*>(is_v ? a.v_cache : a.k_cache);
  for (int i = threadIdx.x; i < groups; i += kWriteThreads) {
    const int h = i / row_groups, c = i % row_groups;
    float x[8];
    if constexpr (kSrcBf16) {
      const uint4 w = reinterpret_cast<const uint4*>(is_v ? a.v : a.k)[(int64_t)t * groups + i];
      const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        x[2 * j] = bf16_bits_to_f32(ws[j] & 0xffffu);
        x[2 * j + 1] = bf16_bits_to_f32(ws[j] >> 16);
      }
    } else {
      const float4* s4 = reinterpret_cast<const float4*>(is_v ? a.v : a.k) + ((int64_t)t * groups + i) * 2;
      const float4 lo = s4[0], hi = s4[1];
      x[0] = lo.x; x[1] = lo.y; x[2] = lo.z; x[3] = lo.w;
      x[4] = hi.x; x[5] = hi.y; x[6] = hi.z; x[7] = hi.w;
    }
    const float s = scales[blk * a.num_kv_heads + h];
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      lo |= f32_to_e4m3_sat_rne(__fdiv_rn(x[j], s)) << (8 * j);
      hi |= f32_to_e4m3_sat_rne(__fdiv_rn(x[4 + j], s)) << (8 * j);
    }
    const int64_t dst = ((blk * a.num_kv_heads + h) * kBlockTokens + off) * row_groups + c;
    cache[dst] = make_uint2(lo, hi);
  }
}

// Quantise one token's [Hkv, D] row to int4 codes with the destination
// block's scale: 8 values -> one 32-bit word (element 2i in the low nibble
// of byte i).
template <bool kSrcBf16>
__global__ __launch_bounds__(kWriteThreads) void cache_write_int4_kernel(CacheWriteArgs a) {
  const int t = blockIdx.x;
  const bool is_v = blockIdx.y != 0;
  const int64_t slot = token_slot(a, t);
  if (slot < 0 || slot >= (int64_t)a.num_blocks * kBlockTokens) return;
  const int64_t blk = slot / kBlockTokens;
  const int off = (int)(slot % kBlockTokens);
  const int row_groups = a.head_dim / 8;                 // groups of 8 values -> one word of codes
  const int groups = a.num_kv_heads * row_groups;
  const float* scales = is_v ? a.v_scale : a.k_scale;
  uint32_t* cache = reinterpret_cast<uint32_t*>(is_v ? a.v_cache : a.k_cache);
  for (int i = threadIdx.x; i < groups; i += kWriteThreads) {
    const int h = i / row_groups, c = i % row_groups;
    float x[8];
    if constexpr (kSrcBf16) {
      const uint4 w = reinterpret_cast<const uint4*>(is_v ? a.v : a.k)[(int64_t)t * groups + i];
      const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        x[2 * j] = bf16_bits_to_f32(ws[j] & 0xffffu);
        x[2 * j + 1] = bf16_bits_to_f32(ws[j] >> 16);
      }
    } else {
      const float4* s4 = reinterpret_cast<const float4*>(is_v ? a.v : a.k) + ((int64_t)t * groups + i) * 2;
      const float4 lo = s4[0], hi = s4[1];
      x[0] = lo.x; x[1] = lo.y; x[2] = lo.z; x[3] = lo.w;
      x[4] = hi.x; x[5] = hi.y; x[6] = hi.z; x[7] = hi.w;
    }
    const float s = scales[blk * a.num_kv_heads + h];
    uint32_t code = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) code |= f32_to_int4_code(__fdiv_rn(x[j], s)) << (4 * j);
    cache[((blk * a.num_kv_heads + h) * kBlockTokens + off) * row_groups + c] = code;
  }
}

__global__ __launch_bounds__(kCopyThreads) void copy_blocks_kernel(CopyBlocksArgs a, int block_chunks) {
  const int i = blockIdx.x;
  const bool is_v = blockIdx.y != 0;
  const int src = a.pairs[2 * i], dst = a.pairs[2 * i + 1];
  if (src < 0 || dst < 0 || src >= a.num_blocks || dst >= a.num_blocks) return;
  uint4* cache = reinterpret_cast<uint4*>(is_v ? a.v_cache : a.k_cache);
  const uint4* s = cache + (int64_t)src * block_chunks;
  uint4* d = cache + (int64_t)dst * block_chunks;
  for (int c = threadIdx.x; c < block_chunks; c += kCopyThreads) d[c] = s[c];
  float* scales = is_v ? a.v_scale : a.k_scale;
  if (scales != nullptr && threadIdx.x < a.num_kv_heads)
    scales[(int64_t)dst * a.num_kv_heads + threadIdx.x] = scales[(int64_t)src * a.num_kv_heads + threadIdx.x];
}

}  // namespace

hipError_t launch_cache_write(const CacheWriteArgs& a, hipStream_t stream) {
  const dim3 grid(a.num_tokens, 2);
  if (a.cache_dtype == PA_DTYPE_FP8_E4M3) {
    if (a.src_dtype == PA_DTYPE_BF16)
      hipLaunchKernelGGL(cache_write_fp8_kernel<true>, grid, dim3(kWriteThreads), 0, stream, a);
    else
      hipLaunchKernelGGL(cache_write_fp8_kernel<false>, grid, dim3(kWriteThreads), 0, stream, a);
  } else if (a.cache_dtype == PA_DTYPE_INT4) {
    if (a.src_dtype == PA_DTYPE_BF16)
      hipLaunchKernelGGL(cache_write_int4_kernel<true>, grid, dim3(kWriteThreads), 0, stream, a);
    else
      hipLaunchKernelGGL(cache_write_int4_kernel<false>, grid, dim3(kWriteThreads), 0, stream, a);
  } else {
    const int e = a.cache_dtype == PA_DTYPE_F32 ? 4 : 2;
    hipLaunchKernelGGL(cache_write_copy_kernel, grid, dim3(kWriteThreads), 0, stream, a, e);
  }
  return hipGetLastError();
}

hipError_t launch_copy_blocks(const CopyBlocksArgs& a, hipStream_t stream) {
  const int bits = a.cache_dtype == PA_DTYPE_F32 ? 32 : (a.cache_dtype == PA_DTYPE_BF16 ? 16 :
                   (a.cache_dtype == PA_DTYPE_INT4 ? 4 : 8));
  const int block_chunks = a.num_kv_heads * kBlockTokens * a.head_dim * bits / 8 / 16;
  CopyBlocksArgs b = a;
  if (a.cache_dtype != PA_DTYPE_FP8_E4M3 && a.cache_dtype != PA_DTYPE_INT4) b.k_scale = b.v_scale = nullptr;
  hipLaunchKernelGGL(copy_blocks_kernel, dim3(a.num_pairs, 2), dim3(kCopyThreads), 0, stream, b,
                     block_chunks);
  return hipGetLastError();
}

}  // namespace pa
