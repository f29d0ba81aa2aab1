// Internal interface between the C-ABI layer (pa_api.hip) and the kernel
// translation units.  Every launcher enqueues on `stream` and returns the
// hipError_t of the launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "pa.h"

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

// Everything the decode kernels read.
//
// Two work splits share the same per-block arithmetic:
//  * partition grid (`balanced == 0`): one workgroup per (partition of
//    `partition_tokens` tokens, KV head, sequence).  Workspace rows are
//    indexed (sequence, query head, partition):
//      ws_m, ws_l [num_seqs * num_q_heads * num_parts], ws_acc [... * D];
//  * balanced (`balanced == 1`): `num_wgs` workgroups; workgroup x takes an
//    equal, contiguous slice of the list of (sequence, 16-token block) units
//    laid end to end, one wave per KV head.  A sequence cut by a slice edge
//    leaves a partial result in slot 0 (it began before the slice) or slot 1
//    (it began inside the slice); rows are indexed (x, slot, query head):
//      ws_m, ws_l [num_wgs * 2 * num_q_heads], ws_acc [... * D];
//    ws_seq_start [num_seqs + 1] receives each sequence's first unit.
// m is kept in the base-2 domain (logits times log2 e).
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
  int32_t* ws_seq_start;
  int32_t max_blocks_per_seq, max_context_len, num_seqs, num_q_heads, num_kv_heads;
  int32_t head_dim, num_blocks, partition_tokens, num_parts;
  int32_t balanced, num_wgs, waves_per_wg, head_groups;
  float scale_log2;  // scale * log2(e): logits are kept in the base-2 domain
  pa_dtype q_dtype, cache_dtype;
};

hipError_t launch_cache_write(const CacheWriteArgs& a, hipStream_t stream);
hipError_t launch_copy_blocks(const CopyBlocksArgs& a, hipStream_t stream);

// Partition kernels (partition grid): writes `out` directly for sequences
// that fit one partition, partial results into the workspace otherwise.
hipError_t launch_decode_partitions(const DecodeArgs& a, hipStream_t stream);
// Matrix-core kernels for a bf16 query (bf16 or e4m3 cache); the generic
// VALU kernel serves the fp32 path.
hipError_t launch_decode_mfma(const DecodeArgs& a, hipStream_t stream);
hipError_t launch_decode_mfma_balanced(const DecodeArgs& a, hipStream_t stream);
// Merge kernels: combine the partial results of sequences split across
// partitions (partition grid) or across workgroup slices (balanced).
hipError_t launch_decode_merge(const DecodeArgs& a, hipStream_t stream);
hipError_t launch_decode_merge_balanced(const DecodeArgs& a, hipStream_t stream);

// Balanced split: at most this many sequences (their start units live in LDS),
// about this many waves in flight over the whole device.
constexpr int kBalancedMaxSeqs = 4096;
constexpr int kBalancedTargetWaves = 2048;
constexpr int kBalancedMaxWaves = 8;

// Largest partition the partition kernels accept.
constexpr int kMaxPartitionTokens = 512;

// Workspace layout helpers (shared by size queries and launches).
size_t workspace_section_floats(int32_t num_seqs, int32_t num_q_heads, int32_t num_parts);
size_t align_floats(size_t n);

hipError_t launch_probe_stream_read(const void* buf, size_t bytes, void* sink, hipStream_t stream);
hipError_t launch_probe_copy(void* dst, const void* src, size_t bytes, hipStream_t stream);
size_t probe_sink_bytes();

}  // namespace pa
