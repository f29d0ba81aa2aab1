/*
 * pa.h — C ABI of libpa, a paged-KV decode library for AMD MI355X (gfx950).
 *
 * The operations follow the paged KV cache described on the pages:
 *   - "系统级优化：批处理、PagedAttention 与 FlashAttention", section 2.3:
 *     the KV cache is cut into pages of 16 tokens; a per-request block
 *     table maps logical pages to physical pages anywhere in a pool.
 *   - "17 · 连续批处理与 PagedAttention", section 三: physical blocks come
 *     from a global pool, are reference counted, may be shared, and are
 *     copied only when a sharer diverges (copy-on-write).
 *   - "系统级优化…", section 3.1 (attention equation) and 3.3 (scale
 *     head_dim ** -0.5): out = softmax(q K^T * scale) V.
 *   - "推理优化", section 五 exercise 3: grouped-query attention, several
 *     query heads reading one KV head.
 *
 * Layouts (row-major, element counts in brackets):
 *   q, out          [num_seqs, num_q_heads, head_dim]
 *   k_cache, v_cache [num_blocks, num_kv_heads, 16, head_dim]
 *   k_scale, v_scale [num_blocks, num_kv_heads] fp32 (fp8 caches only)
 *   block_tables    [num_seqs, max_blocks_per_seq] int32 physical block ids
 *   context_lens    [num_seqs] int32
 *   slot_mapping    [num_tokens] int64, slot = block * 16 + offset, < 0 = skip
 *   block_pairs     [num_pairs, 2] int32 (src, dst)
 *
 * Ownership: every array argument is device memory owned by the caller.
 * The library allocates no device memory at run time and keeps no per-call
 * state; the only device memory it owns is the static scratch array of
 * pa_decode_noalloc (one per device, created when the library's code is
 * loaded onto that device).
 * All calls enqueue work on `stream` (a hipStream_t; NULL = the default
 * stream) and return without synchronising.  The return value reports
 * host-side validation and launch errors only; a fault inside a kernel
 * surfaces at the caller's next synchronisation.  No C++ exception crosses
 * this boundary.  Calls are thread-safe.
 *
 * Query heads map to KV heads by consecutive groups: query head h reads KV
 * head h / (num_q_heads / num_kv_heads) (the pages do not fix this mapping).
 *
 * The fp8 type is OCP e4m3 ("E4M3FN": bias 7, max 448, no infinities),
 * gfx950's native 8-bit float.  The pages name "fp8" only as a KV-cache
 * setting ("17 · 连续批处理与 PagedAttention", section 四).
 *
 * The int4 type stores a signed integer in [-8, 7] as the 4-bit code
 * value + 8, two per byte (element 2i in the low nibble of byte i), so an
 * int4 cache is [num_blocks, kv_heads, 16, head_dim / 2] bytes; values are
 * code - 8 times the (block, head) scale, and a write stores
 * clamp(round_half_even(x / scale), -8, 7).  The pages compare FP16, FP8
 * and INT4 KV caches ("推理优化", section 五, exercise 1).  Wherever this
 * header says "FP8_E4M3 with k_scale/v_scale", INT4 works the same way
 * (with head_dim 128).
 */
#ifndef PA_H_
#define PA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PA_BLOCK_SIZE 16
/* bytes of the static scratch array behind pa_decode_noalloc */
#define PA_DECODE_NOALLOC_MAX_WORKSPACE ((size_t)64 << 20)

typedef enum pa_dtype {
  PA_DTYPE_F32 = 0,
  PA_DTYPE_BF16 = 1,
  PA_DTYPE_FP8_E4M3 = 2,
  PA_DTYPE_INT4 = 3        /* caches only: value + 8 in 4 bits, two per byte; head_dim 128 */
} pa_dtype;

typedef enum pa_status {
  PA_OK = 0,
  PA_ERR_NULL_POINTER = -1, /* a required pointer is NULL */
  PA_ERR_BAD_SHAPE = -2,    /* a size is negative, inconsistent or out of range */
  PA_ERR_BAD_DTYPE = -3,    /* unknown dtype or unsupported dtype combination */
  PA_ERR_UNSUPPORTED = -4,  /* head_dim or group size outside the supported set */
  PA_ERR_WORKSPACE = -5,    /* workspace missing or smaller than pa_decode_workspace_size() */
  PA_ERR_MISALIGNED = -6,   /* a q/out/cache pointer is not 16-byte aligned */
  PA_ERR_LAUNCH = -7,       /* the HIP runtime rejected a kernel launch */
  PA_ERR_OUT_OF_BLOCKS = -8 /* the block pool cannot hold the request (nothing changed) */
} pa_status;

/*
 * pa_cache_write — scatter one decode step's new K/V rows into their pages.
 *
 * For every token t with slot_mapping[t] >= 0:
 *   k_cache[slot / 16, h, slot % 16, :] = k[t, h, :]   for every KV head h
 *   (same for v).
 * This is the paged form of appending new keys and values to a KV cache
 * ("推理优化", section 二 Step 1, where new K/V are written after the
 * current length of a contiguous cache).
 *
 * k, v:      [num_tokens, num_kv_heads, head_dim] of src_dtype.
 * cache_dtype F32 or BF16: src_dtype must equal it; bits are copied.
 * cache_dtype FP8_E4M3: src_dtype F32 or BF16; each value x is stored as the
 *   e4m3 code of float32(x) / k_scale[block, h] (IEEE division), rounded to
 *   nearest even and saturated to +-448.  k_scale/v_scale must be given.
 * Preconditions not checked on the device: live slots are unique and below
 * num_blocks * 16 (a slot outside the pool is skipped by the kernel).
 * Errors: NULL_POINTER, BAD_SHAPE (num_tokens < 0, num_kv_heads < 1,
 * num_blocks < 1), BAD_DTYPE, UNSUPPORTED (head_dim not 64 or 128),
 * MISALIGNED, LAUNCH.  num_tokens == 0 is a no-op.
 */
int pa_cache_write(const void* k, const void* v, pa_dtype src_dtype,
                   void* k_cache, void* v_cache, pa_dtype cache_dtype,
                   const float* k_scale, const float* v_scale,
                   const int64_t* slot_mapping, int32_t num_tokens,
                   int32_t num_kv_heads, int32_t head_dim, int32_t num_blocks,
                   void* stream);

/*
 * pa_cache_write_autoscale — slot scatter into an e4m3 or int4 cache that
 * sets the per-(block, head) scales itself (k_scale/v_scale are read and
 * written).
 *
 * The rows one call writes into one block must be consecutive tokens of the
 * call with consecutive offsets (a prefill chunk, or one decode token per
 * sequence); such a run starting at offset o0 is handled per KV head with
 * a = max |x| over its values and top = 448 (e4m3) or 7 (int4):
 *   - o0 == 0 (the run starts the block): scale = a / top (1 if a == 0);
 *   - else if a > scale * top: the scale grows to a / top and the rows
 *     already in the block are re-encoded (code value * old scale, divided
 *     by the new scale, encoded again);
 *   - else the scale stays.
 * The new rows are then encoded with the block's scale as pa_cache_write
 * does.  So no value is clipped, and the scales need no calibration pass
 * ("推理优化" section 五 exercise 1 and "17 · 连续批处理与 PagedAttention"
 * section 四 name fp8/int4 KV caches; how their scales are chosen is this
 * library's reading).  src_dtype F32 or BF16.  Errors as pa_cache_write.
 */
int pa_cache_write_autoscale(const void* k, const void* v, pa_dtype src_dtype,
                             void* k_cache, void* v_cache, pa_dtype cache_dtype,
                             float* k_scale, float* v_scale,
                             const int64_t* slot_mapping, int32_t num_tokens,
                             int32_t num_kv_heads, int32_t head_dim, int32_t num_blocks,
                             void* stream);

/*
 * pa_decode_partition_tokens — the partition length pa_decode uses.
 *
 * Returns `partition_tokens` itself when it is positive, otherwise the
 * automatic choice for this shape (a multiple of 16).  Returns a negative
 * pa_status for invalid arguments.
 */
int32_t pa_decode_partition_tokens(int32_t num_seqs, int32_t num_q_heads,
                                   int32_t num_kv_heads, int32_t head_dim,
                                   int32_t max_context_len,
                                   int32_t partition_tokens);

/*
 * pa_decode_workspace_size — bytes of scratch pa_decode needs.
 *
 * Zero when every sequence fits one partition (then workspace may be
 * NULL).  Otherwise room for per-(sequence, query head, partition) partial
 * results: running max, running sum and an unnormalised fp32 output row.
 * Returns 0 for invalid arguments as well; pa_decode then reports the error.
 */
size_t pa_decode_workspace_size(int32_t num_seqs, int32_t num_q_heads,
                                int32_t num_kv_heads, int32_t head_dim,
                                int32_t max_context_len,
                                int32_t partition_tokens);

/*
 * pa_decode — one query token per sequence attending over its paged cache.
 *
 * For sequence b, query head h, KV head g = h / (num_q_heads/num_kv_heads):
 *   out[b, h, :] = sum_t softmax_t(scale * q[b,h,:] . K_b[g,t,:]) V_b[g,t,:]
 * over tokens t < context_lens[b], where token t of sequence b is
 *   K_b[g, t, :] = k_cache[block_tables[b, t / 16], g, t % 16, :]
 * (for FP8 caches, times k_scale[block, g]; V likewise with v_scale).
 * ("系统级优化…" sections 2.3 and 3.1; "17 · 连续批处理与 PagedAttention"
 * section 三.)  Long contexts are split into partitions of
 * pa_decode_partition_tokens() tokens whose partial results are merged
 * exactly by log-sum-exp.  Accumulation is fp32; out has q's dtype and is
 * rounded to nearest even.  context_lens[b] == 0 gives a zero row.
 *
 * Supported: (q F32, cache F32), (q BF16, cache BF16), (q BF16, cache
 * FP8_E4M3 with k_scale/v_scale); head_dim 64 or 128; num_q_heads a
 * multiple of num_kv_heads with a group of at most 16.
 * max_context_len is a host-side upper bound of context_lens (it sizes the
 * launch) and must not exceed max_blocks_per_seq * 16; partition_tokens is
 * 0 (automatic) or a positive multiple of 16.
 * Preconditions not checked on the device: block ids used by a sequence lie
 * in [0, num_blocks) (the kernel clamps them, so a bad table gives wrong
 * numbers, not a fault) and context_lens[b] <= max_context_len.
 * Errors: NULL_POINTER, BAD_SHAPE, BAD_DTYPE, UNSUPPORTED, WORKSPACE,
 * MISALIGNED, LAUNCH.  num_seqs == 0 is a no-op.
 * pa_decode writes only `out` and `workspace`.
 */
int pa_decode(void* out, const void* q, pa_dtype q_dtype,
              const void* k_cache, const void* v_cache, pa_dtype cache_dtype,
              const float* k_scale, const float* v_scale,
              const int32_t* block_tables, int32_t max_blocks_per_seq,
              const int32_t* context_lens, int32_t max_context_len,
              int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
              int32_t head_dim, int32_t num_blocks, float scale,
              int32_t partition_tokens, void* workspace, size_t workspace_bytes,
              void* stream);

/*
 * pa_decode_append — one decode step: write each sequence's newest token
 * into its slot and attend over the cache including it.
 *
 * For every sequence b with context_lens[b] = n >= 1, the token at position
 * n - 1 (slot block_tables[b, (n-1)/16] * 16 + (n-1) % 16) receives
 * k_new[b, :, :] and v_new[b, :, :] exactly as pa_cache_write would store
 * them (bit copy, or the e4m3 encode with the block's scale), and out[b] is
 * what pa_decode returns for the cache after that write.  This is the
 * decode-time append of "推理优化" section 二 Step 1 (new keys/values
 * joined to the cache, then attention over all of them) done in one pass:
 * with a bf16 query and partition_tokens == 0 the wave that reads a
 * sequence's last block takes the new row from k_new/v_new and writes it to
 * the cache itself, so no separate scatter kernel runs.  Otherwise the call
 * runs the scatter and then pa_decode.
 *
 * k_new, v_new: [num_seqs, num_kv_heads, head_dim] in q's dtype.  All other
 * arguments, the workspace rules and the errors are those of pa_decode and
 * pa_cache_write.  Precondition not checked on the device: the block holding
 * a sequence's newest token is not shared with another sequence in the
 * batch (copy-on-write has given it a private copy).
 */
int pa_decode_append(void* out, const void* q, pa_dtype q_dtype,
                     const void* k_new, const void* v_new,
                     void* k_cache, void* v_cache, pa_dtype cache_dtype,
                     const float* k_scale, const float* v_scale,
                     const int32_t* block_tables, int32_t max_blocks_per_seq,
                     const int32_t* context_lens, int32_t max_context_len,
                     int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                     int32_t head_dim, int32_t num_blocks, float scale,
                     int32_t partition_tokens, void* workspace,
                     size_t workspace_bytes, void* stream);

/*
 * pa_decode_noalloc — pa_decode for callers that cannot allocate device
 * memory: code captured into a HIP graph, tight serving loops, harnesses
 * that forbid allocation.
 *
 * Arguments, results, supported set and errors are those of pa_decode,
 * without the workspace: the scratch lives in a static device array of
 * PA_DECODE_NOALLOC_MAX_WORKSPACE bytes (64 MiB) that the library holds on
 * every device it runs on until the process ends.  Calls whose scratch
 * (pa_decode_workspace_size) exceeds it return PA_ERR_WORKSPACE before any
 * launch: every automatic (balanced) split fits; a partition grid fits when
 * num_seqs * num_q_heads * records * (head_dim + 2) * 4 bytes does, a record
 * covering 4 partitions for a BF16 query and 1 for F32.
 * The call allocates nothing and records no timing events.  All calls on
 * one device share that device's array: calls that may overlap on one
 * device (other streams, other threads) race and must be serialised by the
 * caller.  The first call on a device looks up that device's copy of the
 * array (the current device, hipGetDevice).
 */
int pa_decode_noalloc(void* out, const void* q, pa_dtype q_dtype,
                      const void* k_cache, const void* v_cache, pa_dtype cache_dtype,
                      const float* k_scale, const float* v_scale,
                      const int32_t* block_tables, int32_t max_blocks_per_seq,
                      const int32_t* context_lens, int32_t max_context_len,
                      int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                      int32_t head_dim, int32_t num_blocks, float scale,
                      int32_t partition_tokens, void* stream);

/*
 * pa_copy_blocks — the copy step of copy-on-write.
 *
 * For every pair i: block block_pairs[i,1] of k_cache and of v_cache becomes
 * a copy of block block_pairs[i,0] (all KV heads, all 16 slots), and for
 * FP8 caches k_scale/v_scale[dst, :] = [src, :].  ("17 · 连续批处理与
 * PagedAttention", section 三: a shared block is copied when a sharer
 * diverges; "推理优化", section "PagedAttention".)
 * Preconditions not checked on the device: destinations are unique and no
 * destination is also a source (pairs run in parallel); ids outside
 * [0, num_blocks) are skipped.
 * Errors: NULL_POINTER, BAD_SHAPE, BAD_DTYPE, UNSUPPORTED, MISALIGNED,
 * LAUNCH.  num_pairs == 0 is a no-op.
 */
int pa_copy_blocks(void* k_cache, void* v_cache, pa_dtype cache_dtype,
                   float* k_scale, float* v_scale,
                   const int32_t* block_pairs, int32_t num_pairs,
                   int32_t num_kv_heads, int32_t head_dim, int32_t num_blocks,
                   void* stream);

/*
 * Planned attention: several query tokens per sequence, and prefixes shared
 * between sequences read once.
 *
 * pa_decode serves one new token per sequence.  Three other steps attend
 * over the same paged cache with several new tokens of one sequence at
 * once: a chunk of a chunked prefill ("17 · 连续批处理与 PagedAttention",
 * section 二, remedy ① for decode stalls), the K draft tokens a target model
 * checks in one pass ("推理优化", section 一, speculative decoding), and the
 * suffix computed after a prefix-cache hit (same section, prefix caching).
 * The new tokens are the last q_len positions of their sequence, their K/V
 * are already in the cache (pa_cache_write), and new token i (position
 * ctx - q_len + i) attends to every position <= its own: the causal mask of
 * "系统级优化…" section 3.3, aligned to the end of the context.
 *
 * Sequences whose block tables start with the same physical blocks share
 * those blocks' K/V ("17 · 连续批处理与 PagedAttention", section 三: a
 * shared prefix is stored once and referenced by every sharer; "推理优化"
 * section 一, prefix caching).  With PA_PLAN_SHARE_PREFIX the plan reads
 * such a run of blocks once for all sharers (their query columns side by
 * side in the MFMA tiles of one wave) and merges that partial result with each sharer's
 * own suffix by log-sum-exp; the result equals the unshared computation.
 *
 * The work is described by a plan built on the host from host copies of
 * the lengths (and, for prefix sharing, of the block tables), copied by the
 * caller to device memory, then executed by pa_attend_planned.
 */
#define PA_PLAN_SHARE_PREFIX 1

typedef struct pa_plan_info {
  int32_t num_seqs, num_q_tokens, num_q_heads, num_kv_heads, head_dim;
  int32_t num_items;          /* work items: (<= 32 query columns, run of blocks) */
  int32_t num_columns;        /* query columns: (new token, query head within its group) */
  int32_t num_records;        /* partial results, each [num_kv_heads] x (m, l, acc[head_dim]) */
  int32_t num_merge_rows;     /* columns whose result is merged from partial results */
  int32_t num_merge_entries;
  int32_t num_shared_groups;  /* runs of prefix blocks read once for several sequences */
  int32_t num_wgs;            /* workgroups (equal slices of the work) per KV-head group */
  int32_t max_item_columns;   /* most query columns of one item (<= 32) */
  int32_t num_wide_groups;    /* groups of up to 4 items of one long segment sharing each block (see below) */
  int64_t plan_bytes;         /* size of the packed plan */
  int64_t workspace_bytes;    /* scratch pa_attend_planned needs (0: none) */
  int64_t block_reads;        /* blocks read per KV head (a wide group reads a block once for its items) */
} pa_plan_info;

/*
 * pa_plan_attention — build the plan on the host.
 *
 * All arrays are HOST memory.  q_start [num_seqs + 1]: sequence b owns the
 * new tokens (rows of q) q_start[b] .. q_start[b+1]-1, with q_start[0] == 0
 * and 0 <= q_len <= context_lens[b]; NULL means one new token per sequence
 * (q_start[b] = b, the decode case).  context_lens [num_seqs] count every
 * token of the sequence including the new ones.  block_tables
 * [num_seqs, max_blocks_per_seq] is read only with PA_PLAN_SHARE_PREFIX
 * (NULL allowed otherwise).  target_slices: how many equal slices
 * (workgroups) to cut the work into (0 = automatic: about 2048 waves over
 * the device; never more slices than 16-token blocks to read).  A
 * segment with many query columns (a chunked-prefill chunk: q_len x group
 * columns, at least 4 tiles of 32) goes to wide groups instead: up to 4 of
 * its 32-column items, one workgroup per KV head, every block read once
 * into LDS for all of them; their block runs are split into pieces only
 * when the groups alone would not fill the device, and the groups are
 * ordered longest run first within the groups that share an XCD (the
 * earlier-started of two workgroups on a CU runs faster).  `plan` receives
 * info->plan_bytes bytes; pass plan = NULL to learn the sizes only.  Errors: NULL_POINTER, BAD_SHAPE
 * (inconsistent lengths, context past the block table), UNSUPPORTED
 * (group > 16, head_dim not 64/128), WORKSPACE (plan_capacity too small).
 * Pure host computation; thread-safe.
 */
int pa_plan_attention(const int32_t* q_start, const int32_t* context_lens,
                      const int32_t* block_tables, int32_t max_blocks_per_seq,
                      int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                      int32_t head_dim, int32_t flags, int32_t target_slices,
                      void* plan, size_t plan_capacity, pa_plan_info* info);

/*
 * pa_attend_planned — run a plan.
 *
 * out, q: [info->num_q_tokens, num_q_heads, head_dim] bf16 (device).
 * Caches, scales and block_tables as for pa_decode (device).  `plan` is a
 * device copy of the bytes pa_plan_attention wrote, and `info` (host) is
 * the info it returned with them; the shapes in `info` must match the
 * other arguments.  workspace: at least info->workspace_bytes
 * bytes of device memory (any contents).  Supported: q BF16 with a BF16 or
 * FP8_E4M3 cache.  A plan that does not come from pa_plan_attention gives
 * wrong numbers, not a fault (indices are clamped on the device).  Errors:
 * NULL_POINTER, BAD_SHAPE, BAD_DTYPE, UNSUPPORTED, WORKSPACE, MISALIGNED,
 * LAUNCH.  Writes only `out` and `workspace`.
 */
int pa_attend_planned(void* out, const void* q, pa_dtype q_dtype,
                      const void* k_cache, const void* v_cache, pa_dtype cache_dtype,
                      const float* k_scale, const float* v_scale,
                      const int32_t* block_tables, int32_t max_blocks_per_seq,
                      int32_t num_blocks, float scale, const void* plan,
                      const pa_plan_info* info, void* workspace,
                      size_t workspace_bytes, void* stream);

/*
 * pa_upload — move a step's small host arrays (block tables, lengths,
 * copy pairs) to the device on the compute stream.
 *
 * The continuous-batching step of "17 · 连续批处理与 PagedAttention"
 * (section 二: the batch is re-formed every iteration) sends its freshly
 * built block tables to the device before every decode step.  An ordinary
 * asynchronous copy goes through a DMA engine, and the compute stream then
 * waits on it and the DMA engine on the compute stream: tens of
 * microseconds of idle GPU per iteration at the decode's scale.  pa_upload
 * instead runs a copy kernel on `stream` that reads the pinned host buffer
 * directly.
 *
 * src: page-locked host memory mapped for the device (hipHostMalloc, or a
 * pinned torch tensor); dst: device memory; both 16-byte aligned; bytes a
 * multiple of 16.  The host must not change src until the kernel has run
 * (record an event after the call).  Errors: NULL_POINTER, BAD_SHAPE
 * (bytes not a multiple of 16), MISALIGNED, UNSUPPORTED (src is not
 * device-mapped host memory, or dst is not device memory), LAUNCH.
 * bytes == 0 is a no-op.
 */
int pa_upload(void* dst, const void* src, size_t bytes, void* stream);

/*
 * Host block manager and the continuous-batching step (host memory only).
 *
 * A global pool of num_blocks physical blocks of 16 tokens, one block table
 * per sequence, and reference counts ("系统级优化…" section 2.3: one manager
 * hands out equal pages, a request's pages need not be contiguous, pages a
 * finished request frees are reused at once; "17 · 连续批处理与
 * PagedAttention" section 三: blocks are shared by reference count and a
 * shared block is copied only when a sharer writes into it).  A sequence of
 * n tokens holds ceil(n/16) blocks.  Free blocks are handed out from the
 * front of a free list that starts as `free_order` (NULL: 0..num_blocks-1);
 * a freed block goes back to the front (reused first); a freed sequence
 * releases its blocks last to first, so they come back in table order.
 *
 * Sequences are named by caller-chosen int32 ids.  Every call validates
 * before it changes anything: a call that returns an error leaves the
 * manager as it was.  OUT_OF_BLOCKS means the pool is too small for the
 * request; the caller preempts (frees) a sequence and retries ("17 ·
 * 连续批处理与 PagedAttention" section 五: running requests are evicted when
 * the KV cache runs out, and recomputed later).  A manager is not
 * thread-safe; distinct managers are independent.
 */
typedef struct pa_block_manager pa_block_manager;

typedef struct pa_bm_stats {
  int32_t num_blocks, free_blocks, num_seqs, reserved;
  int64_t logical_tokens;   /* sum of the sequences' token counts */
  int64_t block_refs;       /* sum of the sequences' block counts (shared blocks counted per sharer) */
  int64_t stored_tokens;    /* tokens held in distinct blocks (a shared block counts once) */
} pa_bm_stats;

/* NULL if num_blocks < 1, free_order is not a permutation, or no memory. */
pa_block_manager* pa_bm_create(int32_t num_blocks, const int32_t* free_order);
void pa_bm_destroy(pa_block_manager* m);
/* A new sequence holding num_tokens tokens (a prompt): ceil(n/16) fresh blocks. */
int pa_bm_add(pa_block_manager* m, int32_t seq, int32_t num_tokens);
/* child references every block of parent (parallel sampling, beam search). */
int pa_bm_fork(pa_block_manager* m, int32_t parent, int32_t child);
/* Drop the sequence; blocks whose count reaches zero return to the pool. */
int pa_bm_free(pa_block_manager* m, int32_t seq);
/* One more token: returns its slot (block * 16 + offset); a new block when
 * the last is full; when the last block is shared, a private copy
 * (*cow_src -> *cow_dst, else both -1) whose contents the caller copies
 * with pa_copy_blocks before writing the token. */
int pa_bm_append(pa_block_manager* m, int32_t seq, int64_t* slot, int32_t* cow_src, int32_t* cow_dst);
/* The sequence's block ids (table may be NULL to query the counts). */
int pa_bm_table(const pa_block_manager* m, int32_t seq, int32_t* table, int32_t capacity,
                int32_t* num_blocks, int64_t* num_tokens);
int pa_bm_get_stats(const pa_block_manager* m, pa_bm_stats* out);
/*
 * One decode iteration of continuous batching ("17 · 连续批处理与
 * PagedAttention" section 二: the batch is re-formed at every token): append
 * one token to each of seqs[0..num_seqs-1] (distinct ids) and write the
 * batch's arrays for pa_copy_blocks / pa_decode_append (or pa_cache_write +
 * pa_decode): block_tables [num_seqs, max_blocks_per_seq] (unused entries
 * repeat the last block), context_lens [num_seqs] (including the new
 * token), slot_mapping [num_seqs] (the new token's slot), cow_pairs
 * [num_seqs, 2] with *num_cow pairs used.  All or nothing: if the pool
 * cannot hold the step, returns OUT_OF_BLOCKS with *blocks_short = how many
 * blocks are missing, and changes nothing.
 */
int pa_bm_step(pa_block_manager* m, const int32_t* seqs, int32_t num_seqs, int32_t max_blocks_per_seq,
               int32_t* block_tables, int32_t* context_lens, int64_t* slot_mapping, int32_t* cow_pairs,
               int32_t* num_cow, int32_t* blocks_short);

/* pa_status_string — static text for a status code (never NULL). */
const char* pa_status_string(int status);

/*
 * Measurement hooks (not part of the method; used to report achieved
 * bandwidth against the hardware's).
 *
 * pa_timing_enable(n), n >= 1, makes every n-th pa_decode /
 * pa_decode_append call from then on record HIP events on its stream
 * around its decode kernel and its merge kernel (n = 0 turns recording
 * off; sampling keeps the events' own cost out of most calls).
 * pa_timing_read() waits for the recorded events, returns the summed kernel
 * times in milliseconds and the number of calls recorded, and clears the
 * record.  At most 65536 calls are recorded between reads.  The events are
 * timing-only (created without the system-scope fence, so recording them
 * writes back no caches between the kernels they bracket): they order
 * nothing and publish no results to the host.
 */
int pa_timing_enable(int every);
int pa_timing_read(double* partition_ms, double* merge_ms, int64_t* calls);

/*
 * pa_probe_stream_read — read `bytes` (a multiple of 16) from `buf` with
 * 16-byte loads and write one 16-byte checksum per workgroup into `sink`
 * (at least pa_probe_sink_bytes() bytes), so the loads cannot be elided.
 * pa_probe_copy — copy `bytes` (a multiple of 16) from src to dst.
 * Both measure what the memory system sustains for a plain stream.
 */
size_t pa_probe_sink_bytes(void);
int pa_probe_stream_read(const void* buf, size_t bytes, void* sink, void* stream);
int pa_probe_copy(void* dst, const void* src, size_t bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PA_H_ */
