// Internal interface between the C-ABI layer (pa_api.hip) and the kernel
// translation units.  Every launcher enqueues on `stream` and returns the
// hipError_t of the launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/pa.h"

namespace pa {

struct CacheWriteArgs {
  const void* k;
  const void* v;
  void* k_cache;
  void* v_cache;
  const float* k_scale;
  const float* v_scale;
  const int64_t* slot_mapping;
  int32_t num_tokens, num_kv_heads, head_dim, num_blocks;
  pa_dtype src_dtype, cache_dtype;
};

struct CopyBlocksArgs {
  void* k_cache;
  void* v_cache;
  float* k_scale;
  float* v_scale;
  const int32_t* pairs;
  int32_t num_pairs, num_kv_heads, head_dim, num_blocks;
  pa_dtype cache_dtype;
};

// Everything the decode kernels read.  Workspace sections (fp32):
//   ws_m   [num_seqs, num_q_heads, num_parts]      running max (log2 domain)
//   ws_l   [num_seqs, num_q_heads, num_parts]      running sum
//   ws_acc [num_seqs, num_q_heads, num_parts, D]   unnormalised output
struct DecodeArgs {
  void* out;
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const float* k_scale;
  const float* v_scale;
  const int32_t* block_tables;
  const int32_t* context_lens;
  float* ws_m;
  float* ws_l;
  float* ws_acc;
  int32_t max_blocks_per_seq, max_context_len, num_seqs, num_q_heads, num_kv_heads;
  int32_t head_dim, num_blocks, partition_tokens, num_parts;
  float scale_log2;  // scale * log2(e): logits are kept in the base-2 domain
  pa_dtype q_dtype, cache_dtype;
};

hipError_t launch_cache_write(const CacheWriteArgs& a, hipStream_t stream);
hipError_t launch_copy_blocks(const CopyBlocksArgs& a, hipStream_t stream);

// Partition kernel: one workgroup per (partition, KV head, sequence).
// Writes `out` directly for sequences that fit one partition, partial
// results into the workspace otherwise.
hipError_t launch_decode_partitions(const DecodeArgs& a, hipStream_t stream);
// Matrix-core partition kernel for a bf16 query (bf16 or e4m3 cache); the
// generic VALU kernel serves the fp32 path.
hipError_t launch_decode_mfma(const DecodeArgs& a, hipStream_t stream);
// Merge kernel: combines the partial results of multi-partition sequences.
hipError_t launch_decode_merge(const DecodeArgs& a, hipStream_t stream);

// Largest partition the partition kernels accept.
constexpr int kMaxPartitionTokens = 512;

// Workspace layout helpers (shared by size queries and launches).
size_t workspace_section_floats(int32_t num_seqs, int32_t num_q_heads, int32_t num_parts);
size_t align_floats(size_t n);

hipError_t launch_probe_stream_read(const void* buf, size_t bytes, void* sink, hipStream_t stream);
hipError_t launch_probe_copy(void* dst, const void* src, size_t bytes, hipStream_t stream);
size_t probe_sink_bytes();

}  // namespace pa
