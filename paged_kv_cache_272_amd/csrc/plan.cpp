// Host planner for pa_attend_planned: cuts attention over the paged cache
// into work items of at most 16 query columns by a run of 16-token blocks.
//
// A query column is one (new token, query head within its GQA group) pair;
// it becomes one N-column of the MFMA tile, so up to 16 of them share every
// K/V block a wave loads.  New token i of a sequence with q_len new tokens
// and context ctx sits at position ctx - q_len + i and sees positions
// 0 .. ctx - q_len + i (the causal mask of "系统级优化…" section 3.3,
// aligned to the end of the context; the multi-token steps are chunked
// prefill, "17 · 连续批处理与 PagedAttention" section 二, and speculative
// verification / prefix-cache suffixes, "推理优化" section 一).
//
// Prefix sharing ("17 · 连续批处理与 PagedAttention", section 三: sharers
// reference the same physical blocks): sequences whose tables begin with
// the same physical blocks, visible in full to every one of their columns,
// form a group; the group's common blocks become one segment whose columns
// are all the members' columns, and each member keeps a segment for its
// remaining blocks.  Partial results of a column's segments are merged by
// log-sum-exp (exact in real arithmetic).
//
// Work balance: every tile's block run is cut into near-equal pieces of
// about total_blocks / target_items blocks (at least kMinChunk).  Items that
// read the same blocks (tiles of one segment) are kept on one XCD: the GPU
// hands workgroup x to XCD x mod 8, so the planner fills 8 queues with
// bundles of sibling items (least-loaded queue first) and interleaves them.
#include <algorithm>
#include <cstring>
#include <map>
#include <vector>

#include "pa_internal.h"

namespace pa {
namespace {

constexpr int kBlockTokens = PA_BLOCK_SIZE;
constexpr int kMinChunk = 16;          // blocks per item, at least
constexpr int kDefaultTargetItems = 1024;
constexpr int kXcds = 8;

struct Segment {
  int seq;                       // block-table row the blocks are read from
  int lo, hi;                    // logical block range
  std::vector<int> cols;         // column ids
  bool partial;                  // its columns have other contributions
};

struct PlanBuild {
  std::vector<PlanItem> items;
  std::vector<PlanColumn> cols;
  std::vector<PlanMergeRow> rows;
  std::vector<int32_t> entries;
  int32_t records = 0;
  int32_t groups = 0;
  int64_t block_reads = 0;
};

int ceil_div(int64_t a, int64_t b) { return (int)((a + b - 1) / b); }

// Column ids are q_row * G + j; q_row is the new token's row in q.
void sequence_columns(int q0, int q_len, int G, std::vector<int>& out) {
  for (int i = 0; i < q_len; ++i)
    for (int j = 0; j < G; ++j) out.push_back((q0 + i) * G + j);
}

int build_plan(const int32_t* q_start, const int32_t* context_lens, const int32_t* block_tables,
               int32_t max_blocks_per_seq, int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
               int32_t flags, int32_t target_items, PlanBuild& pb) {
  const int G = num_q_heads / num_kv_heads;
  const bool share = (flags & PA_PLAN_SHARE_PREFIX) != 0;
  const int64_t B = num_seqs;
  auto qs = [&](int64_t b) -> int64_t { return q_start ? q_start[b] : b; };
  if (q_start && q_start[0] != 0) return PA_ERR_BAD_SHAPE;
  for (int64_t b = 0; b < B; ++b) {
    const int64_t q_len = qs(b + 1) - qs(b);
    const int64_t ctx = context_lens[b];
    if (q_len < 0 || ctx < 0 || q_len > ctx) return PA_ERR_BAD_SHAPE;
    if (ctx > (int64_t)max_blocks_per_seq * kBlockTokens) return PA_ERR_BAD_SHAPE;
  }
  const int64_t T = qs(B);
  if (T * G > INT32_MAX / 2) return PA_ERR_BAD_SHAPE;

  // ---- columns: (q_row, j, horizon), id = q_row * G + j
  pb.cols.assign((size_t)(T * G), PlanColumn{0, 0, 0, 0});
  for (int64_t b = 0; b < B; ++b) {
    const int q_len = (int)(qs(b + 1) - qs(b)), ctx = context_lens[b];
    for (int i = 0; i < q_len; ++i)
      for (int j = 0; j < G; ++j) {
        const int64_t id = (qs(b) + i) * G + j;
        pb.cols[id] = PlanColumn{(int32_t)(qs(b) + i), j, ctx - q_len + i + 1, 0};
      }
  }

  // ---- segments
  std::vector<Segment> segs;
  std::vector<int> own_lo(B, 0);        // first block of a sequence's own segment
  std::vector<char> grouped(B, 0);
  if (share && B > 1) {
    // candidates: the blocks every column of b sees in full
    std::map<int32_t, std::vector<int>> by_first;
    for (int64_t b = 0; b < B; ++b) {
      const int q_len = (int)(qs(b + 1) - qs(b));
      if (q_len == 0) continue;
      const int full = (context_lens[b] - q_len + 1) / kBlockTokens;
      if (full >= 1) by_first[block_tables[b * max_blocks_per_seq]].push_back((int)b);
    }
    for (auto& kv : by_first) {
      const std::vector<int>& mem = kv.second;
      if (mem.size() < 2) continue;
      const int32_t* t0 = block_tables + (int64_t)mem[0] * max_blocks_per_seq;
      int npre = max_blocks_per_seq;
      for (int b : mem) {
        const int q_len = (int)(qs(b + 1) - qs(b));
        const int full = (context_lens[b] - q_len + 1) / kBlockTokens;
        const int32_t* tb = block_tables + (int64_t)b * max_blocks_per_seq;
        int k = 0;
        const int lim = std::min(full, npre);
        while (k < lim && tb[k] == t0[k]) ++k;
        npre = k;
      }
      if (npre < 1) continue;
      Segment g{mem[0], 0, npre, {}, true};
      for (int b : mem) {
        sequence_columns((int)qs(b), (int)(qs(b + 1) - qs(b)), G, g.cols);
        own_lo[b] = npre;
        grouped[b] = 1;
      }
      segs.push_back(std::move(g));
      ++pb.groups;
    }
  }
  for (int64_t b = 0; b < B; ++b) {
    const int q_len = (int)(qs(b + 1) - qs(b));
    if (q_len == 0) continue;
    const int nblk = ceil_div(context_lens[b], kBlockTokens);
    if (own_lo[b] >= nblk) continue;                 // everything was in the shared run
    Segment s{(int)b, own_lo[b], nblk, {}, grouped[b] != 0};
    sequence_columns((int)qs(b), q_len, G, s.cols);
    segs.push_back(std::move(s));
  }

  // ---- tiles (16 columns each) and their block runs
  struct Tile {
    int seg, col0, ncols, lo, hi, kv_len;
  };
  std::vector<Tile> tiles;
  int64_t total = 0;
  for (size_t si = 0; si < segs.size(); ++si) {
    const Segment& s = segs[si];
    for (size_t c0 = 0; c0 < s.cols.size(); c0 += 16) {
      const int n = (int)std::min<size_t>(16, s.cols.size() - c0);
      int max_h = 0;
      for (int k = 0; k < n; ++k) max_h = std::max(max_h, (int)pb.cols[s.cols[c0 + k]].horizon);
      const int hi = std::min(s.hi, ceil_div(max_h, kBlockTokens));
      if (hi <= s.lo) continue;                      // no column of this tile sees these blocks
      tiles.push_back(Tile{(int)si, (int)c0, n, s.lo, hi, max_h});
      total += hi - s.lo;
    }
  }
  const int target = target_items > 0 ? target_items : kDefaultTargetItems;
  const int chunk = std::max<int>(kMinChunk, ceil_div(total, target));

  // ---- items, records and bundles of sibling items (same blocks, other tiles)
  std::vector<std::vector<int>> col_recs(pb.cols.size());
  std::vector<PlanColumn> item_cols;                 // columns laid out per item
  std::vector<PlanItem> raw;
  std::vector<std::pair<int, int>> bundles;          // [first, last) into raw
  std::vector<int64_t> bundle_load;
  // the tiles of one segment are consecutive; cut each into the same pieces
  for (size_t t0 = 0; t0 < tiles.size();) {
    size_t t1 = t0;
    while (t1 < tiles.size() && tiles[t1].seg == tiles[t0].seg) ++t1;
    const Segment& s = segs[tiles[t0].seg];
    // pieces of the segment's longest run; a tile uses the pieces that overlap its run
    int seg_hi = s.lo;
    for (size_t t = t0; t < t1; ++t) seg_hi = std::max(seg_hi, tiles[t].hi);
    const int len = seg_hi - s.lo;
    const int pieces = std::max(1, ceil_div(len, chunk));
    for (int p = 0; p < pieces; ++p) {
      const int lo = s.lo + (int)((int64_t)p * len / pieces);
      const int hi = s.lo + (int)((int64_t)(p + 1) * len / pieces);
      const int first = (int)raw.size();
      int64_t load = 0;
      for (size_t t = t0; t < t1; ++t) {
        const Tile& tl = tiles[t];
        const int ilo = lo, ihi = std::min(hi, tl.hi);
        if (ihi <= ilo) continue;
        const bool direct = !s.partial && pieces == 1;
        PlanItem it{};
        it.seq = s.seq;
        it.blk_lo = ilo;
        it.blk_hi = ihi;
        it.col0 = (int32_t)item_cols.size();
        it.ncols = tl.ncols;
        it.kv_len = tl.kv_len;
        it.rec0 = direct ? -1 : pb.records;
        for (int k = 0; k < tl.ncols; ++k) {
          const int id = s.cols[tl.col0 + k];
          item_cols.push_back(pb.cols[id]);
          if (!direct) col_recs[id].push_back(pb.records + k);
        }
        if (!direct) pb.records += tl.ncols;
        raw.push_back(it);
        load += ihi - ilo;
        pb.block_reads += ihi - ilo;
      }
      if ((int)raw.size() > first) {
        bundles.emplace_back(first, (int)raw.size());
        bundle_load.push_back(load);
      }
    }
    t0 = t1;
  }

  // ---- XCD queues: a bundle's items go to one queue, in order
  std::vector<std::vector<int>> queue(kXcds);
  std::vector<int64_t> qload(kXcds, 0);
  for (size_t k = 0; k < bundles.size(); ++k) {
    const int q = (int)(std::min_element(qload.begin(), qload.end()) - qload.begin());
    for (int i = bundles[k].first; i < bundles[k].second; ++i) queue[q].push_back(i);
    qload[q] += bundle_load[k];
  }
  size_t depth = 0;
  for (auto& q : queue) depth = std::max(depth, q.size());
  pb.items.clear();
  pb.items.reserve(depth * kXcds);
  const PlanItem empty{0, 0, 0, 0, 0, 0, -1, 0};
  for (size_t d = 0; d < depth; ++d)
    for (int q = 0; q < kXcds; ++q) pb.items.push_back(d < queue[q].size() ? raw[queue[q][d]] : empty);
  pb.cols = std::move(item_cols);

  // ---- merge rows: every column with partial records, in column order
  for (size_t id = 0; id < col_recs.size(); ++id) {
    if (col_recs[id].empty()) continue;
    const int32_t q_row = (int32_t)(id / G), j = (int32_t)(id % G);
    pb.rows.push_back(PlanMergeRow{q_row, j, (int32_t)pb.entries.size(), (int32_t)col_recs[id].size()});
    for (int r : col_recs[id]) pb.entries.push_back(r);
  }
  return PA_OK;
}

}  // namespace
}  // namespace pa

using namespace pa;

PA_EXPORT int pa_plan_attention(const int32_t* q_start, const int32_t* context_lens, const int32_t* block_tables,
                                int32_t max_blocks_per_seq, int32_t num_seqs, int32_t num_q_heads,
                                int32_t num_kv_heads, int32_t head_dim, int32_t flags, int32_t target_items,
                                void* plan, size_t plan_capacity, pa_plan_info* info) {
  if (!info) return PA_ERR_NULL_POINTER;
  std::memset(info, 0, sizeof(*info));
  if (num_seqs < 0 || num_q_heads < 1 || num_kv_heads < 1 || max_blocks_per_seq < 1) return PA_ERR_BAD_SHAPE;
  if (num_q_heads % num_kv_heads) return PA_ERR_BAD_SHAPE;
  if (num_q_heads / num_kv_heads > 16) return PA_ERR_UNSUPPORTED;
  if (head_dim != 64 && head_dim != 128) return PA_ERR_UNSUPPORTED;
  if (target_items < 0 || (flags & ~PA_PLAN_SHARE_PREFIX)) return PA_ERR_BAD_SHAPE;
  if (num_seqs > 0 && !context_lens) return PA_ERR_NULL_POINTER;
  if ((flags & PA_PLAN_SHARE_PREFIX) && num_seqs > 0 && !block_tables) return PA_ERR_NULL_POINTER;
  PlanBuild pb;
  const int st = build_plan(q_start, context_lens, block_tables, max_blocks_per_seq, num_seqs, num_q_heads,
                            num_kv_heads, flags, target_items, pb);
  if (st != PA_OK) return st;
  info->num_seqs = num_seqs;
  info->num_q_tokens = q_start ? q_start[num_seqs] : num_seqs;
  info->num_q_heads = num_q_heads;
  info->num_kv_heads = num_kv_heads;
  info->head_dim = head_dim;
  info->num_items = (int32_t)pb.items.size();
  info->num_columns = (int32_t)pb.cols.size();
  info->num_records = pb.records;
  info->num_merge_rows = (int32_t)pb.rows.size();
  info->num_merge_entries = (int32_t)pb.entries.size();
  info->num_shared_groups = pb.groups;
  const PlanLayout lay = plan_layout(*info);
  info->plan_bytes = (int64_t)lay.bytes;
  info->workspace_bytes = (int64_t)planned_workspace_bytes(*info);
  info->block_reads = pb.block_reads;
  if (!plan) return PA_OK;
  if (plan_capacity < lay.bytes) return PA_ERR_WORKSPACE;
  uint8_t* p = static_cast<uint8_t*>(plan);
  std::memset(p, 0, lay.bytes);
  if (!pb.items.empty()) std::memcpy(p + lay.items_off, pb.items.data(), pb.items.size() * sizeof(PlanItem));
  if (!pb.cols.empty()) std::memcpy(p + lay.cols_off, pb.cols.data(), pb.cols.size() * sizeof(PlanColumn));
  if (!pb.rows.empty()) std::memcpy(p + lay.rows_off, pb.rows.data(), pb.rows.size() * sizeof(PlanMergeRow));
  if (!pb.entries.empty())
    std::memcpy(p + lay.entries_off, pb.entries.data(), pb.entries.size() * sizeof(int32_t));
  return PA_OK;
}
