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

// ---- slot scatter that sets the (block, head) scales itself
//
// The rows a call writes into one block are consecutive tokens of the call
// (a "run"); the workgroup of the run's first token handles the whole run,
// head by head: a = max |x| over the run's values; a block started by the
// run takes scale a / top, an append whose values exceed old_scale * top
// grows the scale and re-encodes the rows already in the block
// (value = code value * old scale, code = encode(value / new scale)), and
// the new rows are encoded with the final scale.  top = 448 (e4m3) or 7
// (int4).  All arithmetic is binary32, products and quotients rounded once.
constexpr int kScaleThreads = 256;

template <bool kInt4, bool kSrcBf16>
__global__ __launch_bounds__(kScaleThreads) void cache_write_autoscale_kernel(CacheWriteArgs a, float* k_scale,
                                                                              float* v_scale) {
  __shared__ float s_red[kScaleThreads / 64];
  const int t0 = blockIdx.x;
  const bool is_v = blockIdx.y != 0;
  const int64_t slot0 = a.slot_mapping[t0];
  const int64_t pool = (int64_t)a.num_blocks * kBlockTokens;
  if (slot0 < 0 || slot0 >= pool) return;
  const int64_t blk = slot0 / kBlockTokens;
  if (t0 > 0) {
    const int64_t prev = a.slot_mapping[t0 - 1];
    if (prev >= 0 && prev < pool && prev / kBlockTokens == blk) return;      // not the run's first token
  }
  int n = 1;                                                                // run length (<= 16)
  while (n < kBlockTokens && t0 + n < a.num_tokens) {
    const int64_t s = a.slot_mapping[t0 + n];
    if (s < 0 || s >= pool || s / kBlockTokens != blk) break;
    ++n;
  }
  const int o0 = (int)(slot0 % kBlockTokens);
  const int D = a.head_dim;
  const int row_bytes = kInt4 ? D / 2 : D;
  const float top = kInt4 ? 7.0f : 448.0f;
  float* scales = is_v ? v_scale : k_scale;
  uint8_t* cache = reinterpret_cast<uint8_t*>(is_v ? a.v_cache : a.k_cache);
  const uint8_t* src = reinterpret_cast<const uint8_t*>(is_v ? a.v : a.k);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  auto load = [&](int i, int h, int d) -> float {     // value d of head h of the run's row i
    const int64_t e = ((int64_t)(t0 + i) * a.num_kv_heads + h) * D + d;
    if constexpr (kSrcBf16) return bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(src)[e]);
    else return reinterpret_cast<const float*>(src)[e];
  };
  auto encode = [&](float x) -> uint32_t {
    if constexpr (kInt4) return f32_to_int4_code(x);
    else return f32_to_e4m3_sat_rne(x);
  };
  for (int h = 0; h < a.num_kv_heads; ++h) {
    // a = max |x| over the run's new values of this head
    float amax = 0.0f;
    for (int i = tid; i < n * D; i += kScaleThreads) amax = fmaxf(amax, fabsf(load(i / D, h, i % D)));
    amax = wave_max(amax);
    if (lane == 0) s_red[wave] = amax;
    __syncthreads();
    amax = fmaxf(fmaxf(s_red[0], s_red[1]), fmaxf(s_red[2], s_red[3]));
    __syncthreads();
    const float old = scales[blk * a.num_kv_heads + h];
    float s = old;
    bool grow = false;
    if (o0 == 0) {
      s = amax > 0.0f ? __fdiv_rn(amax, top) : 1.0f;
    } else if (amax > old * top) {
      s = __fdiv_rn(amax, top);
      grow = true;
    }
    uint8_t* head_rows = cache + ((blk * a.num_kv_heads + h) * kBlockTokens) * row_bytes;
    if (grow) {                                         // re-encode the rows already in the block
      for (int i = tid; i < o0 * row_bytes; i += kScaleThreads) {
        const uint32_t b = head_rows[i];
        uint32_t out;
        if constexpr (kInt4) {
          const float lo = (float)((int)(b & 15u) - 8) * old, hi = (float)((int)(b >> 4) - 8) * old;
          out = encode(__fdiv_rn(lo, s)) | (encode(__fdiv_rn(hi, s)) << 4);
        } else {
          out = encode(__fdiv_rn(e4m3_to_f32(b) * old, s));
        }
        head_rows[i] = (uint8_t)out;
      }
    }
    // the new rows with the block's final scale
    for (int i = tid; i < n * row_bytes; i += kScaleThreads) {
      const int r = i / row_bytes, j = i % row_bytes;
      uint32_t out;
      if constexpr (kInt4)
        out = encode(__fdiv_rn(load(r, h, 2 * j), s)) | (encode(__fdiv_rn(load(r, h, 2 * j + 1), s)) << 4);
      else out = encode(__fdiv_rn(load(r, h, j), s));
      head_rows[(int64_t)(o0 + r) * row_bytes + j] = (uint8_t)out;
    }
    if (tid == 0) scales[blk * a.num_kv_heads + h] = s;
    __syncthreads();
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

hipError_t launch_cache_write_autoscale(const CacheWriteArgs& a, float* k_scale, float* v_scale,
                                       hipStream_t stream) {
  const dim3 grid(a.num_tokens, 2);
  const bool int4 = a.cache_dtype == PA_DTYPE_INT4, bf16 = a.src_dtype == PA_DTYPE_BF16;
  if (int4) {
    if (bf16) hipLaunchKernelGGL((cache_write_autoscale_kernel<true, true>), grid, dim3(kScaleThreads), 0, stream, a,
                                 k_scale, v_scale);
    else hipLaunchKernelGGL((cache_write_autoscale_kernel<true, false>), grid, dim3(kScaleThreads), 0, stream, a,
                            k_scale, v_scale);
  } else {
    if (bf16) hipLaunchKernelGGL((cache_write_autoscale_kernel<false, true>), grid, dim3(kScaleThreads), 0, stream,
                                 a, k_scale, v_scale);
    else hipLaunchKernelGGL((cache_write_autoscale_kernel<false, false>), grid, dim3(kScaleThreads), 0, stream, a,
                            k_scale, v_scale);
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
