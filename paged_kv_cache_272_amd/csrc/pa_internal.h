// Internal interface between the C-ABI layer (pa_api.hip) and the kernel
// translation units.  Every launcher enqueues on `stream` and returns the
// hipError_t of the launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "pa.h"

#define PA_EXPORT extern "C" __attribute__((visibility("default")))

namespace pa {

// Slot scatter.  With slot_mapping == nullptr the slot of token t is the
// position context_lens[t] - 1 of sequence t (its newest token), taken
// through block_tables; sequences with no token are skipped.
struct CacheWriteArgs {
  const void* k;
  const void* v;
  void* k_cache;
  void* v_cache;
  const float* k_scale;
  const float* v_scale;
  const int64_t* slot_mapping;
  const int32_t* block_tables;
  const int32_t* context_lens;
  int32_t num_tokens, num_kv_heads, head_dim, num_blocks, max_blocks_per_seq;
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
//  * partition grid (`balanced == 0`): partitions of `partition_tokens`
//    tokens; a workgroup per (record, KV head, sequence), a record covering
//    `parts_per_rec` consecutive partitions (the matrix-core kernel: 4, one
//    per wave, merged in LDS; the fp32 kernel: 1).  Workspace rows are
//    indexed (sequence, query head, record):
//      ws_m, ws_l [num_seqs * num_q_heads * num_recs], ws_acc [... * D];
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
  // Appending decode: the newest token (position context_lens[b] - 1) of
  // every sequence is taken from k_new/v_new [B, Hkv, D] (query type) and
  // written to its slot by the wave that reads that block.
  const void* k_new;
  const void* v_new;
  int32_t append;
  int32_t max_blocks_per_seq, max_context_len, num_seqs, num_q_heads, num_kv_heads;
  int32_t head_dim, num_blocks, partition_tokens, num_parts, parts_per_rec, num_recs;
  int32_t balanced, num_wgs, waves_per_wg, head_groups;
  int32_t out_words;  // balanced: 4-byte LDS words of each wave's outbox of finished rows
  float scale_log2;  // scale * log2(e): logits are kept in the base-2 domain
  pa_dtype q_dtype, cache_dtype;
};

hipError_t launch_cache_write(const CacheWriteArgs& a, hipStream_t stream);
hipError_t launch_copy_blocks(const CopyBlocksArgs& a, hipStream_t stream);
// Slot scatter into an e4m3/int4 cache that sets the (block, head) scales.
hipError_t launch_cache_write_autoscale(const CacheWriteArgs& a, float* k_scale, float* v_scale,
                                       hipStream_t stream);

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
// about this many waves in flight over the whole device, at most this many
// waves per workgroup.  bf16 and e4m3 caches run two waves per SIMD (8-wave
// workgroups, up to 256 VGPRs); an int4 cache, bound by vector work rather
// than HBM, runs three (4-wave workgroups, three per CU, up to 168 VGPRs).
constexpr int kBalancedMaxSeqs = 4096;
// LDS of a balanced-split workgroup: start[B + 1] and ctx[B] (padded to 16
// bytes, plus 16 words for the kernel's static LDS), then each wave's outbox
// of finished rows (DecodeArgs::out_words words, at least kBalancedStageRows
// rows of head_dim floats).
constexpr int kBalancedStageRows = 8;
__host__ __device__ constexpr int balanced_stage_offset_words(int num_seqs) { return (2 * num_seqs + 1 + 3) / 4 * 4; }
__host__ __device__ constexpr int balanced_lds_fixed_words(int num_seqs) { return balanced_stage_offset_words(num_seqs) + 16; }
constexpr int kBalancedTargetWaves = 2048;
constexpr int kBalancedMaxWaves = 8;
constexpr int kBalancedTargetWavesInt4 = 3072;
constexpr int kBalancedMaxWavesInt4 = 4;

// Largest partition the partition kernels accept.
constexpr int kMaxPartitionTokens = 512;

// Workspace layout helpers (shared by size queries and launches).
size_t workspace_section_floats(int32_t num_seqs, int32_t num_q_heads, int32_t num_parts);
size_t align_floats(size_t n);

// ---- planned attention (pa_plan_attention / pa_attend_planned)
//
// A packed plan is five arrays, one after the other (each 16-byte aligned):
//   items[num_items], columns[num_columns], merge_rows[num_merge_rows],
//   entries[num_merge_entries] (int32 record ids), wg_start[num_wgs + 1]
//   (workgroup x runs items wg_start[x] .. wg_start[x+1]-1).
// Item k reads logical blocks [blk_lo, blk_hi) of block-table row `seq` for
// the `ncols` query columns columns[col0 .. col0+ncols-1]; tokens at or past
// kv_len hold no data.  rec0 < 0: the item is the column's only
// contribution and writes `out`; otherwise column c's partial result goes
// to record rec0 + c.  A merge row combines the records entries[e0 .. e0+n-1]
// into the output row of (q_row, j).
struct PlanItem {
  int32_t seq, blk_lo, blk_hi, col0, ncols, kv_len, rec0, pad;
};
struct PlanColumn {
  int32_t q_row, j, horizon, pad;   // query head = kv_head * G + j; sees positions < horizon
};
struct PlanMergeRow {
  int32_t q_row, j, e0, n;
};
// A wide group: up to kWideTiles items of one segment (the same sequence and
// first block, other query columns) run by one workgroup per KV head, each
// wave one item, every block read once into LDS for all of them.
struct PlanWideGroup {
  int32_t item0, nitems, blk_lo, blk_hi;
};
constexpr int kWideTiles = 4;

struct PlanLayout {
  size_t items_off, cols_off, rows_off, entries_off, wg_off, wide_off, bytes;
};

inline size_t align16(size_t n) { return (n + 15) / 16 * 16; }

inline PlanLayout plan_layout(const pa_plan_info& info) {
  PlanLayout l;
  l.items_off = 0;
  l.cols_off = align16(l.items_off + (size_t)info.num_items * sizeof(PlanItem));
  l.rows_off = align16(l.cols_off + (size_t)info.num_columns * sizeof(PlanColumn));
  l.entries_off = align16(l.rows_off + (size_t)info.num_merge_rows * sizeof(PlanMergeRow));
  l.wg_off = align16(l.entries_off + (size_t)info.num_merge_entries * sizeof(int32_t));
  l.wide_off = align16(l.wg_off + (size_t)(info.num_wgs > 0 ? info.num_wgs + 1 : 0) * sizeof(int32_t));
  l.bytes = align16(l.wide_off + (size_t)info.num_wide_groups * sizeof(PlanWideGroup));
  return l;
}

// Records: [num_kv_heads, num_records] rows of m, l (floats) and acc[head_dim]
// (one KV head's records adjacent, so a wave's columns are consecutive rows).
inline size_t planned_workspace_bytes(const pa_plan_info& info) {
  const size_t rows = (size_t)info.num_records * info.num_kv_heads;
  if (rows == 0) return 0;
  const size_t sec = (rows + 63) / 64 * 64;
  return (2 * sec + rows * info.head_dim) * sizeof(float);
}

struct PlannedArgs {
  void* out;
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const float* k_scale;
  const float* v_scale;
  const int32_t* block_tables;
  // the plan arrays are read-only and alias nothing the kernels write, so
  // their wave-uniform reads can go through scalar loads
  const PlanItem* __restrict__ items;
  const PlanColumn* __restrict__ cols;
  const PlanMergeRow* __restrict__ rows;
  const int32_t* __restrict__ entries;
  const int32_t* __restrict__ wg_start;
  const PlanWideGroup* __restrict__ wide;
  float* ws_m;
  float* ws_l;
  float* ws_acc;
  int32_t num_items, num_columns, num_records, num_merge_rows, num_merge_entries, num_wgs, max_item_columns;
  int32_t num_wide_groups;
  int32_t num_seqs, num_q_tokens, num_q_heads, num_kv_heads, head_dim;
  int32_t max_blocks_per_seq, num_blocks;
  int32_t waves_per_wg, head_groups;
  int32_t box_entries;  // sliced items: record entries each wave's LDS outbox holds (set at launch)
  float scale_log2;
  pa_dtype cache_dtype;
};

hipError_t launch_attend_planned(const PlannedArgs& a, hipStream_t stream);
hipError_t launch_attend_planned_merge(const PlannedArgs& a, hipStream_t stream);
hipError_t launch_attend_wide(const PlannedArgs& a, hipStream_t stream);

hipError_t launch_probe_stream_read(const void* buf, size_t bytes, void* sink, hipStream_t stream);
hipError_t launch_probe_copy(void* dst, const void* src, size_t bytes, hipStream_t stream);
hipError_t launch_upload(void* dst, const void* src, size_t bytes, hipStream_t stream);
size_t probe_sink_bytes();

}  // namespace pa
