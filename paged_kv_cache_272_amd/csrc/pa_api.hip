// C-ABI layer of libpa: argument validation, dtype/shape dispatch, partition
// choice, workspace layout, launches, status codes and the timing hooks.
//
// Validation happens entirely on the host and before any HIP call, so a
// rejected call never touches the GPU.
#include <cmath>
#include <cstdint>
#include <mutex>
#include <vector>

#include "pa_device.h"
#include "pa_internal.h"


namespace pa {

size_t align_floats(size_t n) { return (n + 63) / 64 * 64; }  // 256-byte sections

size_t workspace_section_floats(int32_t num_seqs, int32_t num_q_heads, int32_t num_parts) {
  return align_floats((size_t)num_seqs * num_q_heads * num_parts);
}

namespace {

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline bool valid_dtype(int d) {
  return d == PA_DTYPE_F32 || d == PA_DTYPE_BF16 || d == PA_DTYPE_FP8_E4M3 || d == PA_DTYPE_INT4;
}
// caches whose codes are scaled per (block, head)
inline bool scaled_dtype(int d) { return d == PA_DTYPE_FP8_E4M3 || d == PA_DTYPE_INT4; }

// Automatic partition length: whole sequences when they are short, else
// 512-token partitions (a multiple of the 16-token block).
int32_t auto_partition(int32_t max_context_len) {
  if (max_context_len <= kMaxPartitionTokens) {
    const int32_t p = (max_context_len + 15) / 16 * 16;
    return p < 16 ? 16 : p;
  }
  return kMaxPartitionTokens;
}

int check_decode_shape(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                       int32_t max_context_len, int32_t partition_tokens) {
  if (num_seqs < 0 || num_seqs > 65535) return PA_ERR_BAD_SHAPE;
  if (num_q_heads < 1 || num_kv_heads < 1 || num_kv_heads > 65535) return PA_ERR_BAD_SHAPE;
  if (num_q_heads % num_kv_heads) return PA_ERR_BAD_SHAPE;
  if (num_q_heads / num_kv_heads > 16) return PA_ERR_UNSUPPORTED;
  if (head_dim != 64 && head_dim != 128) return PA_ERR_UNSUPPORTED;
  if (max_context_len < 0) return PA_ERR_BAD_SHAPE;
  if (partition_tokens < 0 || partition_tokens % 16 || partition_tokens > kMaxPartitionTokens)
    return PA_ERR_BAD_SHAPE;
  return PA_OK;
}

struct WorkspaceLayout {
  bool balanced = false;
  int32_t partition_tokens = 0;
  int32_t num_parts = 1;
  int32_t parts_per_rec = 1, num_recs = 1;   // partition grid: records of parts_per_rec partitions
  int32_t num_wgs = 0, waves_per_wg = 0, head_groups = 0;
  int32_t out_words = 0;                     // balanced: LDS outbox words per wave
  size_t bytes = 0;
  size_t m_off = 0, l_off = 0, acc_off = 0, start_off = 0;  // in 4-byte words
};

// Partition grid: partial rows (sequence, query head, record), a record per
// parts_per_rec consecutive partitions (4 for the matrix-core kernel, whose
// waves each take one partition; 1 for the fp32 kernel).
WorkspaceLayout partition_layout(int32_t num_seqs, int32_t num_q_heads, int32_t head_dim, int32_t max_context_len,
                                 int32_t partition_tokens, int32_t parts_per_rec) {
  WorkspaceLayout w;
  w.partition_tokens = partition_tokens > 0 ? partition_tokens : auto_partition(max_context_len);
  const int32_t parts = (max_context_len + w.partition_tokens - 1) / w.partition_tokens;
  w.num_parts = parts < 1 ? 1 : parts;
  w.parts_per_rec = parts_per_rec;
  w.num_recs = (w.num_parts + parts_per_rec - 1) / parts_per_rec;
  if (w.num_recs <= 1) return w;
  const size_t sec = workspace_section_floats(num_seqs, num_q_heads, w.num_recs);
  w.m_off = 0;
  w.l_off = sec;
  w.acc_off = 2 * sec;
  w.bytes = (2 * sec + align_floats((size_t)num_seqs * num_q_heads * w.num_recs * head_dim)) * sizeof(float);
  return w;
}

// Partitions per partial record in the partition grid: the matrix-core
// kernel (bf16 query) merges the 4 partitions of a workgroup itself.
int32_t parts_per_record(pa_dtype q_dtype) { return q_dtype == PA_DTYPE_F32 ? 1 : 4; }

// Balanced split: partial rows (workgroup, slot 0/1, query head), plus the
// per-sequence unit starts.  One wave per KV head, at most 8 waves per
// workgroup (int4: 4), about kBalancedTargetWaves waves over the device
// (int4: kBalancedTargetWavesInt4).
WorkspaceLayout balanced_layout(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                pa_dtype cache_dtype) {
  WorkspaceLayout w;
  w.balanced = true;
  const bool int4 = cache_dtype == PA_DTYPE_INT4;
  const int32_t max_waves = int4 ? kBalancedMaxWavesInt4 : kBalancedMaxWaves;
  const int32_t target = int4 ? kBalancedTargetWavesInt4 : kBalancedTargetWaves;
  w.waves_per_wg = num_kv_heads < max_waves ? num_kv_heads : max_waves;
  w.head_groups = (num_kv_heads + w.waves_per_wg - 1) / w.waves_per_wg;
  const int32_t wgs = target / (w.waves_per_wg * w.head_groups);
  w.num_wgs = wgs < 1 ? 1 : wgs;
  const size_t rows = (size_t)w.num_wgs * 2 * num_q_heads;
  w.m_off = 0;
  w.l_off = align_floats(rows);
  w.acc_off = 2 * align_floats(rows);
  w.start_off = w.acc_off + align_floats(rows * head_dim);
  w.bytes = (w.start_off + align_floats((size_t)num_seqs + 1)) * sizeof(float);
  // bf16 and e4m3: each wave keeps the rows it finishes in an LDS outbox and
  // stores them after its loop (with the newest token's K and V rows of a
  // bf16 append).  Its size: room for two partial, two final and two
  // new-row entries of this group size, within what one workgroup may take of
  // the CU's 160 KB at eight waves per CU (less 2 KB for the allocation
  // granularity and static LDS, at most 64 KB a workgroup) after start[] and
  // ctx[]; at least one staging pass of kBalancedStageRows rows.  int4: the
  // deferred stores gained nothing (its loop is bound by vector work, not by
  // the loads the stores delay) and the outbox writes cost 1-4%, so its rows
  // are stored when each sequence ends, through one staging pass.
  const size_t floor_words = (size_t)kBalancedStageRows * head_dim;
  size_t words = floor_words;
  if (!int4) {
    const size_t G = (size_t)(num_q_heads / num_kv_heads);
    const size_t partial_words = 4 + ((2 * G + 3) & ~(size_t)3) + G * head_dim, final_words = 4 + G * head_dim / 2;
    const size_t splice_words = 4 + (size_t)head_dim;          // the newest token's K and V rows (bf16)
    const size_t want = (2 * partial_words + 2 * final_words + 2 * splice_words + 3) / 4 * 4;
    const size_t wgs_per_cu = 8 / (size_t)w.waves_per_wg > 0 ? 8 / (size_t)w.waves_per_wg : 1;
    size_t budget = ((size_t)160 << 10) / wgs_per_cu - 2048;
    if (budget > ((size_t)64 << 10)) budget = (size_t)64 << 10;
    const size_t fixed = (size_t)balanced_lds_fixed_words(num_seqs) * sizeof(int);
    const size_t room = budget > fixed ? (budget - fixed) / sizeof(int) / (size_t)w.waves_per_wg / 4 * 4 : 0;
    words = room < want ? room : want;
    if (words < floor_words) words = floor_words;
  }
  w.out_words = (int32_t)words;
  return w;
}

bool use_balanced(pa_dtype q_dtype, int32_t num_seqs, int32_t partition_tokens) {
  return partition_tokens == 0 && q_dtype == PA_DTYPE_BF16 && num_seqs <= kBalancedMaxSeqs;
}

// ---- timing hooks -----------------------------------------------------------

struct TimingRecord {
  hipEvent_t start, mid, end;
  bool merged;
};

struct Timing {
  std::mutex mu;
  int every = 0;            // record one decode call in `every`; 0 = off
  int64_t seen = 0;         // decode calls since enabling
  std::vector<TimingRecord> pool;
  size_t used = 0;
} g_timing;

constexpr size_t kMaxTimedCalls = 65536;

TimingRecord* timing_slot() {
  std::lock_guard<std::mutex> lock(g_timing.mu);
  if (g_timing.every <= 0 || g_timing.used >= kMaxTimedCalls) return nullptr;
  if (g_timing.seen++ % g_timing.every != 0) return nullptr;
  if (g_timing.used == g_timing.pool.size()) {
    TimingRecord r{};
    // timing-only events: no system-scope fence when they are recorded, so
    // no cache writeback and invalidation lands between the kernels they time
    const unsigned f = hipEventDisableSystemFence;
    if (hipEventCreateWithFlags(&r.start, f) != hipSuccess || hipEventCreateWithFlags(&r.mid, f) != hipSuccess ||
        hipEventCreateWithFlags(&r.end, f) != hipSuccess)
      return nullptr;
    g_timing.pool.push_back(r);
  }
  return &g_timing.pool[g_timing.used++];
}

}  // namespace
}  // namespace pa

using namespace pa;

PA_EXPORT const char* pa_status_string(int status) {
  switch (status) {
    case PA_OK: return "ok";
    case PA_ERR_NULL_POINTER: return "a required pointer is NULL";
    case PA_ERR_BAD_SHAPE: return "a size is negative, inconsistent or out of range";
    case PA_ERR_BAD_DTYPE: return "unknown dtype or unsupported dtype combination";
    case PA_ERR_UNSUPPORTED: return "head_dim or group size outside the supported set";
    case PA_ERR_WORKSPACE: return "workspace missing or too small";
    case PA_ERR_MISALIGNED: return "a q/out/cache pointer is not 16-byte aligned";
    case PA_ERR_LAUNCH: return "the HIP runtime rejected a kernel launch";
    case PA_ERR_OUT_OF_BLOCKS: return "the block pool cannot hold the request";
    default: return "unknown status";
  }
}

PA_EXPORT int pa_cache_write(const void* k, const void* v, pa_dtype src_dtype, void* k_cache, void* v_cache,
                             pa_dtype cache_dtype, const float* k_scale, const float* v_scale,
                             const int64_t* slot_mapping, int32_t num_tokens, int32_t num_kv_heads,
                             int32_t head_dim, int32_t num_blocks, void* stream) {
  if (num_tokens < 0 || num_kv_heads < 1 || num_blocks < 1) return PA_ERR_BAD_SHAPE;
  if (!valid_dtype(src_dtype) || !valid_dtype(cache_dtype)) return PA_ERR_BAD_DTYPE;
  if (scaled_dtype(cache_dtype)) {
    if (scaled_dtype(src_dtype)) return PA_ERR_BAD_DTYPE;
  } else if (src_dtype != cache_dtype) {
    return PA_ERR_BAD_DTYPE;
  }
  if (head_dim != 64 && head_dim != 128) return PA_ERR_UNSUPPORTED;
  if (cache_dtype == PA_DTYPE_INT4 && head_dim != 128) return PA_ERR_UNSUPPORTED;
  if (num_tokens == 0) return PA_OK;
  if (!k || !v || !k_cache || !v_cache || !slot_mapping) return PA_ERR_NULL_POINTER;
  if (scaled_dtype(cache_dtype) && (!k_scale || !v_scale)) return PA_ERR_NULL_POINTER;
  if (!aligned16(k) || !aligned16(v) || !aligned16(k_cache) || !aligned16(v_cache)) return PA_ERR_MISALIGNED;
  CacheWriteArgs a{k, v, k_cache, v_cache, k_scale, v_scale, slot_mapping, nullptr, nullptr, num_tokens,
                   num_kv_heads, head_dim, num_blocks, 0, src_dtype, cache_dtype};
  return launch_cache_write(a, reinterpret_cast<hipStream_t>(stream)) == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

PA_EXPORT int pa_cache_write_autoscale(const void* k, const void* v, pa_dtype src_dtype, void* k_cache,
                                       void* v_cache, pa_dtype cache_dtype, float* k_scale, float* v_scale,
                                       const int64_t* slot_mapping, int32_t num_tokens, int32_t num_kv_heads,
                                       int32_t head_dim, int32_t num_blocks, void* stream) {
  if (num_tokens < 0 || num_kv_heads < 1 || num_blocks < 1) return PA_ERR_BAD_SHAPE;
  if (!valid_dtype(src_dtype) || !valid_dtype(cache_dtype)) return PA_ERR_BAD_DTYPE;
  if (!scaled_dtype(cache_dtype)) return PA_ERR_BAD_DTYPE;
  if (src_dtype != PA_DTYPE_F32 && src_dtype != PA_DTYPE_BF16) return PA_ERR_BAD_DTYPE;
  if (head_dim != 64 && head_dim != 128) return PA_ERR_UNSUPPORTED;
  if (cache_dtype == PA_DTYPE_INT4 && head_dim != 128) return PA_ERR_UNSUPPORTED;
  if (num_tokens == 0) return PA_OK;
  if (!k || !v || !k_cache || !v_cache || !slot_mapping || !k_scale || !v_scale) return PA_ERR_NULL_POINTER;
  CacheWriteArgs a{k, v, k_cache, v_cache, k_scale, v_scale, slot_mapping, nullptr, nullptr, num_tokens,
                   num_kv_heads, head_dim, num_blocks, 0, src_dtype, cache_dtype};
  return launch_cache_write_autoscale(a, k_scale, v_scale, reinterpret_cast<hipStream_t>(stream)) == hipSuccess
             ? PA_OK : PA_ERR_LAUNCH;
}

PA_EXPORT int32_t pa_decode_partition_tokens(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                             int32_t head_dim, int32_t max_context_len,
                                             int32_t partition_tokens) {
  const int st = check_decode_shape(num_seqs, num_q_heads, num_kv_heads, head_dim, max_context_len,
                                    partition_tokens);
  if (st != PA_OK) return st;
  return partition_layout(num_seqs, num_q_heads, head_dim, max_context_len, partition_tokens, 1).partition_tokens;
}

PA_EXPORT size_t pa_decode_workspace_size(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                          int32_t head_dim, int32_t max_context_len, int32_t partition_tokens) {
  if (check_decode_shape(num_seqs, num_q_heads, num_kv_heads, head_dim, max_context_len, partition_tokens) !=
      PA_OK)
    return 0;
  // the automatic choice depends on the query type, which this query does not
  // take: report enough for either split (a record per partition is the larger grid)
  size_t bytes = partition_layout(num_seqs, num_q_heads, head_dim, max_context_len, partition_tokens, 1).bytes;
  if (use_balanced(PA_DTYPE_BF16, num_seqs, partition_tokens)) {
    for (pa_dtype cd : {PA_DTYPE_BF16, PA_DTYPE_INT4}) {   // (nor the cache type: the larger of the two shapes)
      const size_t b2 = balanced_layout(num_seqs, num_q_heads, num_kv_heads, head_dim, cd).bytes;
      bytes = b2 > bytes ? b2 : bytes;
    }
  }
  return bytes;
}

namespace {

// pa_decode and pa_decode_append.  k_new/v_new non-null: appending.
// need_only non-null: validate every argument except the workspace, store
// the scratch bytes the call needs there, and launch nothing.
int decode_impl(void* out, const void* q, pa_dtype q_dtype, const void* k_new, const void* v_new, const void* k_cache,
                const void* v_cache, pa_dtype cache_dtype, const float* k_scale, const float* v_scale,
                const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* context_lens,
                int32_t max_context_len, int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                int32_t head_dim, int32_t num_blocks, float scale, int32_t partition_tokens, void* workspace,
                size_t workspace_bytes, void* stream, bool timed = true, size_t* need_only = nullptr) {
  const bool append = k_new != nullptr || v_new != nullptr;
  int st = check_decode_shape(num_seqs, num_q_heads, num_kv_heads, head_dim, max_context_len, partition_tokens);
  if (st != PA_OK) return st;
  if (!valid_dtype(q_dtype) || !valid_dtype(cache_dtype)) return PA_ERR_BAD_DTYPE;
  const bool combo_ok = (q_dtype == PA_DTYPE_F32 && cache_dtype == PA_DTYPE_F32) ||
                        (q_dtype == PA_DTYPE_BF16 && cache_dtype == PA_DTYPE_BF16) ||
                        (q_dtype == PA_DTYPE_BF16 && scaled_dtype(cache_dtype));
  if (!combo_ok) return PA_ERR_BAD_DTYPE;
  if (cache_dtype == PA_DTYPE_INT4 && head_dim != 128) return PA_ERR_UNSUPPORTED;
  if (num_blocks < 1 || max_blocks_per_seq < 1) return PA_ERR_BAD_SHAPE;
  if ((int64_t)max_context_len > (int64_t)max_blocks_per_seq * PA_BLOCK_SIZE) return PA_ERR_BAD_SHAPE;
  if (need_only) *need_only = 0;
  if (num_seqs == 0) return PA_OK;
  if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens) return PA_ERR_NULL_POINTER;
  if (append && (!k_new || !v_new)) return PA_ERR_NULL_POINTER;
  if (append && (!aligned16(k_new) || !aligned16(v_new))) return PA_ERR_MISALIGNED;
  if (scaled_dtype(cache_dtype) && (!k_scale || !v_scale)) return PA_ERR_NULL_POINTER;
  if (!aligned16(out) || !aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache)) return PA_ERR_MISALIGNED;
  const WorkspaceLayout w = use_balanced(q_dtype, num_seqs, partition_tokens)
                                ? balanced_layout(num_seqs, num_q_heads, num_kv_heads, head_dim, cache_dtype)
                                : partition_layout(num_seqs, num_q_heads, head_dim, max_context_len,
                                                   partition_tokens, parts_per_record(q_dtype));
  if (need_only) {
    *need_only = w.bytes;
    return PA_OK;
  }
  if (w.bytes > 0 && (!workspace || workspace_bytes < w.bytes)) return PA_ERR_WORKSPACE;
  if (w.bytes > 0 && !aligned16(workspace)) return PA_ERR_MISALIGNED;

  DecodeArgs a{};
  a.out = out;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  float* ws = reinterpret_cast<float*>(workspace);
  a.ws_m = w.bytes ? ws + w.m_off : nullptr;
  a.ws_l = w.bytes ? ws + w.l_off : nullptr;
  a.ws_acc = w.bytes ? ws + w.acc_off : nullptr;
  a.ws_seq_start = w.balanced ? reinterpret_cast<int32_t*>(ws + w.start_off) : nullptr;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.max_context_len = max_context_len;
  a.num_seqs = num_seqs;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.head_dim = head_dim;
  a.num_blocks = num_blocks;
  a.partition_tokens = w.partition_tokens;
  a.num_parts = w.num_parts;
  a.parts_per_rec = w.parts_per_rec;
  a.num_recs = w.num_recs;
  a.balanced = w.balanced ? 1 : 0;
  a.num_wgs = w.num_wgs;
  a.waves_per_wg = w.waves_per_wg;
  a.head_groups = w.head_groups;
  a.out_words = w.out_words;
  a.scale_log2 = scale * kLog2e;
  a.q_dtype = q_dtype;
  a.cache_dtype = cache_dtype;
  // the balanced kernel writes the newest tokens itself; other paths scatter first
  a.append = append && w.balanced ? 1 : 0;
  a.k_new = a.append ? k_new : nullptr;
  a.v_new = a.append ? v_new : nullptr;

  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (append && !a.append) {
    CacheWriteArgs cw{k_new, v_new, const_cast<void*>(k_cache), const_cast<void*>(v_cache), k_scale, v_scale,
                      nullptr, block_tables, context_lens, num_seqs, num_kv_heads, head_dim, num_blocks,
                      max_blocks_per_seq, q_dtype, cache_dtype};
    if (launch_cache_write(cw, s) != hipSuccess) return PA_ERR_LAUNCH;
  }
  TimingRecord* rec = timed ? timing_slot() : nullptr;
  if (rec) (void)hipEventRecord(rec->start, s);
  const hipError_t e1 = w.balanced ? launch_decode_mfma_balanced(a, s) : launch_decode_partitions(a, s);
  if (e1 != hipSuccess) return PA_ERR_LAUNCH;
  if (rec) (void)hipEventRecord(rec->mid, s);
  const bool merge = w.balanced || w.num_recs > 1;
  if (merge) {
    const hipError_t e2 = w.balanced ? launch_decode_merge_balanced(a, s) : launch_decode_merge(a, s);
    if (e2 != hipSuccess) return PA_ERR_LAUNCH;
  }
  if (rec) {
    rec->merged = merge;
    (void)hipEventRecord(rec->end, s);
  }
  return PA_OK;
}

}  // namespace

PA_EXPORT int pa_decode(void* out, const void* q, pa_dtype q_dtype, const void* k_cache, const void* v_cache,
                        pa_dtype cache_dtype, const float* k_scale, const float* v_scale,
                        const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* context_lens,
                        int32_t max_context_len, int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                        int32_t head_dim, int32_t num_blocks, float scale, int32_t partition_tokens,
                        void* workspace, size_t workspace_bytes, void* stream) {
  return decode_impl(out, q, q_dtype, nullptr, nullptr, k_cache, v_cache, cache_dtype, k_scale, v_scale,
                     block_tables, max_blocks_per_seq, context_lens, max_context_len, num_seqs, num_q_heads,
                     num_kv_heads, head_dim, num_blocks, scale, partition_tokens, workspace, workspace_bytes, stream);
}

PA_EXPORT int pa_decode_append(void* out, const void* q, pa_dtype q_dtype, const void* k_new, const void* v_new,
                               void* k_cache, void* v_cache, pa_dtype cache_dtype, const float* k_scale,
                               const float* v_scale, const int32_t* block_tables, int32_t max_blocks_per_seq,
                               const int32_t* context_lens, int32_t max_context_len, int32_t num_seqs,
                               int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t num_blocks,
                               float scale, int32_t partition_tokens, void* workspace, size_t workspace_bytes,
                               void* stream) {
  if (num_seqs > 0 && (!k_new || !v_new)) return PA_ERR_NULL_POINTER;
  return decode_impl(out, q, q_dtype, k_new, v_new, k_cache, v_cache, cache_dtype, k_scale, v_scale, block_tables,
                     max_blocks_per_seq, context_lens, max_context_len, num_seqs, num_q_heads, num_kv_heads,
                     head_dim, num_blocks, scale, partition_tokens, workspace, workspace_bytes, stream);
}

// ---- pa_decode_noalloc: pa_decode with its scratch in a static device array
//
// For callers that cannot allocate device memory (work captured into a HIP
// graph, tight serving loops, harnesses that forbid allocation).  The array
// below exists once per device the library runs on and lives until the
// process ends.  In host code its name is only a host-side stand-in: the
// device address of each device's copy is looked up once with
// hipGetSymbolAddress (with that device current) and only that address is
// handed to kernels.  The decode writes every workspace byte it later reads
// within the same call, so nothing needs clearing; calls that overlap on one
// device share the array and therefore race.

namespace pa {
namespace {

constexpr size_t kStaticScratchBytes = PA_DECODE_NOALLOC_MAX_WORKSPACE;
constexpr int kMaxDevices = 64;

__device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

struct StaticScratch {
  std::mutex mu;
  void* ptr[kMaxDevices] = {};
} g_scratch;

// The current device's copy of `scratch`, or nullptr (status in *err).
void* static_scratch(int* err) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    *err = PA_ERR_LAUNCH;
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_scratch.mu);
  if (!g_scratch.ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
      *err = PA_ERR_LAUNCH;
      return nullptr;
    }
    g_scratch.ptr[dev] = p;
  }
  return g_scratch.ptr[dev];
}

}  // namespace
}  // namespace pa

PA_EXPORT int pa_decode_noalloc(void* out, const void* q, pa_dtype q_dtype, const void* k_cache, const void* v_cache,
                                pa_dtype cache_dtype, const float* k_scale, const float* v_scale,
                                const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* context_lens,
                                int32_t max_context_len, int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                int32_t head_dim, int32_t num_blocks, float scale, int32_t partition_tokens,
                                void* stream) {
  // every check (the size limit included) before the first HIP call
  size_t need = 0;
  const int st = decode_impl(out, q, q_dtype, nullptr, nullptr, k_cache, v_cache, cache_dtype, k_scale, v_scale,
                             block_tables, max_blocks_per_seq, context_lens, max_context_len, num_seqs, num_q_heads,
                             num_kv_heads, head_dim, num_blocks, scale, partition_tokens, nullptr, 0, stream, false,
                             &need);
  if (st != PA_OK || num_seqs == 0) return st;
  if (need > kStaticScratchBytes) return PA_ERR_WORKSPACE;
  int err = PA_OK;
  void* ws = static_scratch(&err);
  if (!ws) return err;
  return decode_impl(out, q, q_dtype, nullptr, nullptr, k_cache, v_cache, cache_dtype, k_scale, v_scale,
                     block_tables, max_blocks_per_seq, context_lens, max_context_len, num_seqs, num_q_heads,
                     num_kv_heads, head_dim, num_blocks, scale, partition_tokens, ws, kStaticScratchBytes, stream,
                     false);
}

PA_EXPORT int pa_copy_blocks(void* k_cache, void* v_cache, pa_dtype cache_dtype, float* k_scale, float* v_scale,
                             const int32_t* block_pairs, int32_t num_pairs, int32_t num_kv_heads,
                             int32_t head_dim, int32_t num_blocks, void* stream) {
  if (num_pairs < 0 || num_kv_heads < 1 || num_blocks < 1) return PA_ERR_BAD_SHAPE;
  if (!valid_dtype(cache_dtype)) return PA_ERR_BAD_DTYPE;
  if (head_dim != 64 && head_dim != 128) return PA_ERR_UNSUPPORTED;
  if (num_kv_heads > 256) return PA_ERR_BAD_SHAPE;   // scales are copied by one workgroup's lanes
  if (cache_dtype == PA_DTYPE_INT4 && head_dim != 128) return PA_ERR_UNSUPPORTED;
  if (num_pairs == 0) return PA_OK;
  if (!k_cache || !v_cache || !block_pairs) return PA_ERR_NULL_POINTER;
  if (scaled_dtype(cache_dtype) && (!k_scale || !v_scale)) return PA_ERR_NULL_POINTER;
  if (!aligned16(k_cache) || !aligned16(v_cache)) return PA_ERR_MISALIGNED;
  CopyBlocksArgs a{k_cache, v_cache, k_scale, v_scale, block_pairs, num_pairs, num_kv_heads, head_dim,
                   num_blocks, cache_dtype};
  return launch_copy_blocks(a, reinterpret_cast<hipStream_t>(stream)) == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

PA_EXPORT int pa_upload(void* dst, const void* src, size_t bytes, void* stream) {
  if (bytes == 0) return PA_OK;
  if (!dst || !src) return PA_ERR_NULL_POINTER;
  if (bytes % 16) return PA_ERR_BAD_SHAPE;
  if (!aligned16(dst) || !aligned16(src)) return PA_ERR_MISALIGNED;
  // the kernel reads src through its device mapping: only page-locked,
  // device-mapped host memory qualifies, and dst must be device memory
  hipPointerAttribute_t sa{}, da{};
  if (hipPointerGetAttributes(&sa, src) != hipSuccess) {
    (void)hipGetLastError();                      // pageable memory: clear the query's error
    return PA_ERR_UNSUPPORTED;
  }
  if (sa.type != hipMemoryTypeHost || !sa.devicePointer || !sa.hostPointer) return PA_ERR_UNSUPPORTED;
  if (hipPointerGetAttributes(&da, dst) != hipSuccess) {
    (void)hipGetLastError();
    return PA_ERR_UNSUPPORTED;
  }
  if (da.type != hipMemoryTypeDevice) return PA_ERR_UNSUPPORTED;
  // the device address of src itself (the mapping's device pointer shifted by src's offset from its host pointer)
  const char* dev_src = static_cast<const char*>(sa.devicePointer) +
                        (static_cast<const char*>(src) - static_cast<const char*>(sa.hostPointer));
  return launch_upload(dst, dev_src, bytes, reinterpret_cast<hipStream_t>(stream)) == hipSuccess ? PA_OK
                                                                                                 : PA_ERR_LAUNCH;
}

PA_EXPORT int pa_attend_planned(void* out, const void* q, pa_dtype q_dtype, const void* k_cache,
                                const void* v_cache, pa_dtype cache_dtype, const float* k_scale,
                                const float* v_scale, const int32_t* block_tables, int32_t max_blocks_per_seq,
                                int32_t num_blocks, float scale, const void* plan, const pa_plan_info* info,
                                void* workspace, size_t workspace_bytes, void* stream) {
  if (!info) return PA_ERR_NULL_POINTER;
  const pa_plan_info& in = *info;
  if (in.num_seqs < 0 || in.num_q_tokens < 0 || in.num_items < 0 || in.num_columns < 0 || in.num_records < 0 ||
      in.num_merge_rows < 0 || in.num_merge_entries < 0 || in.num_wgs < 0 || in.max_item_columns < 0 ||
      in.max_item_columns > 32 || in.num_wide_groups < 0)
    return PA_ERR_BAD_SHAPE;
  if (in.num_q_heads < 1 || in.num_kv_heads < 1 || in.num_q_heads % in.num_kv_heads) return PA_ERR_BAD_SHAPE;
  if (in.num_q_heads / in.num_kv_heads > 16) return PA_ERR_UNSUPPORTED;
  if (in.head_dim != 64 && in.head_dim != 128) return PA_ERR_UNSUPPORTED;
  if (num_blocks < 1 || max_blocks_per_seq < 1) return PA_ERR_BAD_SHAPE;
  if (!valid_dtype(q_dtype) || !valid_dtype(cache_dtype)) return PA_ERR_BAD_DTYPE;
  if (q_dtype != PA_DTYPE_BF16 || cache_dtype == PA_DTYPE_F32) return PA_ERR_BAD_DTYPE;
  if (cache_dtype == PA_DTYPE_INT4 && in.head_dim != 128) return PA_ERR_UNSUPPORTED;
  const PlanLayout lay = plan_layout(in);
  if ((int64_t)lay.bytes != in.plan_bytes) return PA_ERR_BAD_SHAPE;
  if ((int64_t)planned_workspace_bytes(in) != in.workspace_bytes) return PA_ERR_BAD_SHAPE;
  if (in.num_items == 0 || in.num_seqs == 0 || in.num_q_tokens == 0) return PA_OK;
  if (in.num_columns < 1 || (in.num_wgs < 1 && in.num_wide_groups < 1)) return PA_ERR_BAD_SHAPE;
  if (in.num_merge_rows > 0 && (in.num_records < 1 || in.num_merge_entries < 1)) return PA_ERR_BAD_SHAPE;
  if (!out || !q || !k_cache || !v_cache || !block_tables || !plan) return PA_ERR_NULL_POINTER;
  if (scaled_dtype(cache_dtype) && (!k_scale || !v_scale)) return PA_ERR_NULL_POINTER;
  if (!aligned16(out) || !aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(plan))
    return PA_ERR_MISALIGNED;
  const size_t ws_need = planned_workspace_bytes(in);
  if (ws_need > 0 && (!workspace || workspace_bytes < ws_need)) return PA_ERR_WORKSPACE;
  if (ws_need > 0 && !aligned16(workspace)) return PA_ERR_MISALIGNED;

  PlannedArgs a{};
  a.out = out;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.block_tables = block_tables;
  const uint8_t* p = static_cast<const uint8_t*>(plan);
  a.items = reinterpret_cast<const PlanItem*>(p + lay.items_off);
  a.cols = reinterpret_cast<const PlanColumn*>(p + lay.cols_off);
  a.rows = reinterpret_cast<const PlanMergeRow*>(p + lay.rows_off);
  a.entries = reinterpret_cast<const int32_t*>(p + lay.entries_off);
  a.wg_start = reinterpret_cast<const int32_t*>(p + lay.wg_off);
  a.wide = reinterpret_cast<const PlanWideGroup*>(p + lay.wide_off);
  if (ws_need > 0) {
    const size_t rows = (size_t)in.num_records * in.num_kv_heads;
    float* ws = static_cast<float*>(workspace);
    a.ws_m = ws;
    a.ws_l = ws + align_floats(rows);
    a.ws_acc = ws + 2 * align_floats(rows);
  }
  a.num_items = in.num_items;
  a.num_columns = in.num_columns;
  a.num_records = in.num_records;
  a.num_merge_rows = in.num_merge_rows;
  a.num_merge_entries = in.num_merge_entries;
  a.num_wgs = in.num_wgs;
  a.num_wide_groups = in.num_wide_groups;
  a.max_item_columns = in.max_item_columns;
  a.num_seqs = in.num_seqs;
  a.num_q_tokens = in.num_q_tokens;
  a.num_q_heads = in.num_q_heads;
  a.num_kv_heads = in.num_kv_heads;
  a.head_dim = in.head_dim;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.num_blocks = num_blocks;
  a.waves_per_wg = in.num_kv_heads < kBalancedMaxWaves ? in.num_kv_heads : kBalancedMaxWaves;
  a.head_groups = (in.num_kv_heads + a.waves_per_wg - 1) / a.waves_per_wg;
  a.scale_log2 = scale * kLog2e;
  a.cache_dtype = cache_dtype;

  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  TimingRecord* rec = timing_slot();
  if (rec) (void)hipEventRecord(rec->start, s);
  if (in.num_wide_groups > 0 && launch_attend_wide(a, s) != hipSuccess) return PA_ERR_LAUNCH;
  if (in.num_wgs > 0 && launch_attend_planned(a, s) != hipSuccess) return PA_ERR_LAUNCH;
  if (rec) (void)hipEventRecord(rec->mid, s);
  const bool merge = in.num_merge_rows > 0;
  if (merge && launch_attend_planned_merge(a, s) != hipSuccess) return PA_ERR_LAUNCH;
  if (rec) {
    rec->merged = merge;
    (void)hipEventRecord(rec->end, s);
  }
  return PA_OK;
}

PA_EXPORT int pa_timing_enable(int every) {
  if (every < 0) return PA_ERR_BAD_SHAPE;
  std::lock_guard<std::mutex> lock(g_timing.mu);
  g_timing.every = every;
  g_timing.seen = 0;
  return PA_OK;
}

PA_EXPORT int pa_timing_read(double* partition_ms, double* merge_ms, int64_t* calls) {
  if (!partition_ms || !merge_ms || !calls) return PA_ERR_NULL_POINTER;
  std::lock_guard<std::mutex> lock(g_timing.mu);
  double part = 0.0, merge = 0.0;
  for (size_t i = 0; i < g_timing.used; ++i) {
    TimingRecord& r = g_timing.pool[i];
    if (hipEventSynchronize(r.end) != hipSuccess) return PA_ERR_LAUNCH;
    float ms = 0.0f;
    if (hipEventElapsedTime(&ms, r.start, r.mid) != hipSuccess) return PA_ERR_LAUNCH;
    part += ms;
    if (r.merged) {
      if (hipEventElapsedTime(&ms, r.mid, r.end) != hipSuccess) return PA_ERR_LAUNCH;
      merge += ms;
    }
  }
  *partition_ms = part;
  *merge_ms = merge;
  *calls = (int64_t)g_timing.used;
  g_timing.used = 0;
  return PA_OK;
}

PA_EXPORT size_t pa_probe_sink_bytes(void) { return probe_sink_bytes(); }

PA_EXPORT int pa_probe_stream_read(const void* buf, size_t bytes, void* sink, void* stream) {
  if (!buf || !sink) return PA_ERR_NULL_POINTER;
  if (bytes % 16) return PA_ERR_BAD_SHAPE;
  if (!aligned16(buf) || !aligned16(sink)) return PA_ERR_MISALIGNED;
  return launch_probe_stream_read(buf, bytes, sink, reinterpret_cast<hipStream_t>(stream)) == hipSuccess
             ? PA_OK
             : PA_ERR_LAUNCH;
}

PA_EXPORT int pa_probe_copy(void* dst, const void* src, size_t bytes, void* stream) {
  if (!dst || !src) return PA_ERR_NULL_POINTER;
  if (bytes % 16) return PA_ERR_BAD_SHAPE;
  if (!aligned16(dst) || !aligned16(src)) return PA_ERR_MISALIGNED;
  return launch_probe_copy(dst, src, bytes, reinterpret_cast<hipStream_t>(stream)) == hipSuccess ? PA_OK
                                                                                                  : PA_ERR_LAUNCH;
}
