// Host planner for pa_attend_planned: cuts attention over the paged cache
// into work items of at most 32 query columns by a run of 16-token blocks.
//
// A query column is one (new token, query head within its GQA group) pair;
// it becomes one N-column of an MFMA tile.  A wave holds up to two tiles of
// 16 columns, so up to 32 columns share every K/V block the wave loads.
// New token i of a sequence with q_len new tokens and context ctx sits at
// position ctx - q_len + i and sees positions
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
// Work balance: the tiles' block runs are laid end to end (the tiles of one
// segment taking turns piece by piece) and cut into about 2048 / (waves per
// workgroup) equal slices, one workgroup each, as the balanced decode does
// with sequences; every (run, slice) overlap is an item, and a workgroup
// runs its slice's items in order.  No compute unit idles at the end of the
// launch for lack of work.
//
// A segment with many tiles (a prefill chunk: hundreds of query columns
// over the same blocks) would have each block read once per tile.  Its
// tiles go to wide groups instead: up to kWideTiles (4) items of 32
// columns, one workgroup per KV head, one wave per item, each block read
// once into LDS for the group.
#include <algorithm>
#include <cstring>
#include <map>
#include <numeric>
#include <vector>

#include "pa_internal.h"

namespace pa {
namespace {

constexpr int kBlockTokens = PA_BLOCK_SIZE;
constexpr int kTileCols = 32;          // query columns per item (two 16-column MFMA tiles)
constexpr int kTargetWaves = 2048;     // waves over the device, about 8 per compute unit
constexpr int kMaxWavesPerWg = 8;      // one wave per KV head, at most 8 per workgroup
constexpr int kWideMinTiles = 4;       // a segment with this many tiles goes to wide groups
constexpr int kWideMinPiece = 8;       // blocks per piece of a cut wide group, at least

struct Segment {
  int seq;                       // block-table row the blocks are read from
  int lo, hi;                    // logical block range
  std::vector<int> cols;         // column ids
  bool partial;                  // its columns have other contributions
};

struct PlanBuild {
  std::vector<PlanItem> items;
  std::vector<int32_t> wg_start;       // [num_wgs + 1]: workgroup x runs items wg_start[x] .. wg_start[x+1]-1
  std::vector<PlanWideGroup> wide;     // wide groups; their items follow the sliced ones
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
               int32_t flags, int32_t target_slices, PlanBuild& pb) {
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

  // ---- tiles (up to kTileCols columns each) and their block runs.  A
  // segment of at least kWideMinTiles tiles (a prefill chunk) goes to wide
  // groups, the others to the equal slices.
  struct Tile {
    int seg, col0, ncols, lo, hi, kv_len;
  };
  std::vector<Tile> tiles, wtiles;
  int64_t total = 0;
  for (size_t si = 0; si < segs.size(); ++si) {
    const Segment& s = segs[si];
    std::vector<Tile> st;
    for (size_t c0 = 0; c0 < s.cols.size(); c0 += kTileCols) {
      const int n = (int)std::min<size_t>(kTileCols, s.cols.size() - c0);
      int max_h = 0;
      for (int k = 0; k < n; ++k) max_h = std::max(max_h, (int)pb.cols[s.cols[c0 + k]].horizon);
      const int hi = std::min(s.hi, ceil_div(max_h, kBlockTokens));
      if (hi <= s.lo) continue;                      // no column of this tile sees these blocks
      st.push_back(Tile{(int)si, (int)c0, n, s.lo, hi, max_h});
    }
    if ((int)st.size() >= kWideMinTiles) {
      wtiles.insert(wtiles.end(), st.begin(), st.end());
    } else {
      for (const Tile& t : st) total += t.hi - t.lo;
      tiles.insert(tiles.end(), st.begin(), st.end());
    }
  }
  // ---- runs of units in work order.  A segment with one tile is one run; the
  // tiles of a segment with several tiles (the same blocks, other columns)
  // take turns piece by piece, so they read each piece at about the same
  // time and the second read is served from cache.
  const int waves_per_wg = std::min(num_kv_heads, kMaxWavesPerWg);
  const int head_groups = ceil_div(num_kv_heads, waves_per_wg);
  const int64_t want = target_slices > 0 ? target_slices : std::max(1, kTargetWaves / (waves_per_wg * head_groups));
  const int n = (int)std::min<int64_t>(want, total);             // slices; none is empty
  const int piece = std::max(1, ceil_div(total, std::max(n, 1)));
  struct Run {
    int tile, lo, hi;
  };
  std::vector<Run> runs;
  for (size_t t0 = 0; t0 < tiles.size();) {
    size_t t1 = t0;
    while (t1 < tiles.size() && tiles[t1].seg == tiles[t0].seg) ++t1;
    if (t1 - t0 == 1) {
      runs.push_back(Run{(int)t0, tiles[t0].lo, tiles[t0].hi});
    } else {
      int seg_hi = tiles[t0].lo;
      for (size_t t = t0; t < t1; ++t) seg_hi = std::max(seg_hi, tiles[t].hi);
      for (int lo = tiles[t0].lo; lo < seg_hi; lo += piece)
        for (size_t t = t0; t < t1; ++t) {
          const int hi = std::min(lo + piece, tiles[t].hi);
          if (hi > lo) runs.push_back(Run{(int)t, lo, hi});
        }
    }
    t0 = t1;
  }

  // ---- cut the runs at slice boundaries: slice x owns units
  // [floor(x*total/n), floor((x+1)*total/n)); every (run, slice) overlap is an item
  struct Cut {
    int tile, lo, hi, slice;
  };
  std::vector<Cut> cuts;
  std::vector<int> items_of_tile(tiles.size(), 0);
  {
    int64_t u = 0;
    int x = 0;
    for (const Run& r : runs) {
      int lo = r.lo;
      while (lo < r.hi) {
        while (x + 1 < n && (int64_t)(x + 1) * total / n <= u) ++x;
        const int64_t slice_end = (int64_t)(x + 1) * total / n;
        const int take = (int)std::min<int64_t>(r.hi - lo, slice_end - u);
        cuts.push_back(Cut{r.tile, lo, lo + take, x});
        ++items_of_tile[r.tile];
        lo += take;
        u += take;
      }
    }
  }

  // ---- items, records and the slices' item ranges
  std::vector<std::vector<int>> col_recs(pb.cols.size());
  std::vector<PlanColumn> item_cols;                 // columns laid out per item
  std::vector<int32_t> tile_col0(tiles.size(), -1);  // a tile's columns are laid out once
  pb.items.clear();
  pb.wg_start.assign(n > 0 ? (size_t)n + 1 : 0, 0);
  for (const Cut& ct : cuts) {
    const Tile& tl = tiles[ct.tile];
    const Segment& s = segs[tl.seg];
    const bool direct = !s.partial && items_of_tile[ct.tile] == 1;
    if (tile_col0[ct.tile] < 0) {
      tile_col0[ct.tile] = (int32_t)item_cols.size();
      for (int k = 0; k < tl.ncols; ++k) item_cols.push_back(pb.cols[s.cols[tl.col0 + k]]);
    }
    PlanItem it{};
    it.seq = s.seq;
    it.blk_lo = ct.lo;
    it.blk_hi = ct.hi;
    it.col0 = tile_col0[ct.tile];
    it.ncols = tl.ncols;
    it.kv_len = tl.kv_len;
    it.rec0 = direct ? -1 : pb.records;
    if (!direct) {
      for (int k = 0; k < tl.ncols; ++k) col_recs[s.cols[tl.col0 + k]].push_back(pb.records + k);
      pb.records += tl.ncols;
    }
    pb.items.push_back(it);
    pb.block_reads += ct.hi - ct.lo;
    pb.wg_start[ct.slice + 1] = (int32_t)pb.items.size();
  }
  for (int x = 1; x <= n; ++x) pb.wg_start[x] = std::max(pb.wg_start[x], pb.wg_start[x - 1]);

  // ---- wide groups: up to kWideTiles consecutive tiles of one segment (the
  // same first block); their runs are cut into pieces only when the groups
  // times the KV heads would not give about kTargetWaves / kWideTiles
  // workgroups, each piece at least kWideMinPiece blocks.  A tile's item is
  // direct when its segment is its columns' only one and it is not cut.
  std::vector<int32_t> wtile_col0(wtiles.size(), -1);
  struct Group {
    size_t t0, t1;
    int lo, hi;
  };
  std::vector<Group> groups;
  for (size_t t0 = 0; t0 < wtiles.size();) {
    size_t t1 = t0;
    int hi = wtiles[t0].lo;
    while (t1 < wtiles.size() && wtiles[t1].seg == wtiles[t0].seg && t1 - t0 < (size_t)kWideTiles)
      hi = std::max(hi, wtiles[t1++].hi);
    groups.push_back(Group{t0, t1, wtiles[t0].lo, hi});
    t0 = t1;
  }
  const int64_t have = (int64_t)groups.size() * num_kv_heads;
  const int64_t want_wide = kTargetWaves / kWideTiles;
  const int pieces = have > 0 && have < want_wide ? (int)((want_wide + have - 1) / have) : 1;
  for (const Group& gr : groups) {
    const int len = gr.hi - gr.lo;
    const int np = std::max(1, std::min(pieces, len / kWideMinPiece));
    for (int k = 0; k < np; ++k) {
      const int plo = gr.lo + (int)((int64_t)k * len / np), phi = gr.lo + (int)((int64_t)(k + 1) * len / np);
      PlanWideGroup wg{(int32_t)pb.items.size(), 0, plo, plo};
      for (size_t t = gr.t0; t < gr.t1; ++t) {
        const Tile& tl = wtiles[t];
        const Segment& s = segs[tl.seg];
        const int hi = std::min(phi, tl.hi);
        if (hi <= plo) continue;                     // this tile's columns see none of the piece
        if (wtile_col0[t] < 0) {
          wtile_col0[t] = (int32_t)item_cols.size();
          for (int c = 0; c < tl.ncols; ++c) item_cols.push_back(pb.cols[s.cols[tl.col0 + c]]);
        }
        const bool direct = !s.partial && np == 1;
        PlanItem it{};
        it.seq = s.seq;
        it.blk_lo = plo;
        it.blk_hi = hi;
        it.col0 = wtile_col0[t];
        it.ncols = tl.ncols;
        it.kv_len = tl.kv_len;
        it.rec0 = direct ? -1 : pb.records;
        if (!direct) {
          for (int c = 0; c < tl.ncols; ++c) col_recs[s.cols[tl.col0 + c]].push_back(pb.records + c);
          pb.records += tl.ncols;
        }
        pb.items.push_back(it);
        ++wg.nitems;
        wg.blk_hi = std::max(wg.blk_hi, hi);
      }
      if (wg.nitems == 0) continue;
      pb.block_reads += wg.blk_hi - wg.blk_lo;
      pb.wide.push_back(wg);
    }
  }
  pb.cols = std::move(item_cols);
  // Longest groups first, within each run of groups that lands on one XCD.
  // The wide kernel sends workgroup j = (KV head, group), head-major, to XCD
  // j / per_xcd; an XCD starts its workgroups in order, and of two sharing a
  // CU the earlier one's waves win issue arbitration (about 14% more blocks
  // per microsecond on a prefill chunk), so the earlier slots should take the
  // longer runs.  Sorting chunks of gcd(groups, per_xcd) groups keeps every
  // group of every head on the XCD it had (its L2 still serves the blocks
  // that the groups of one segment share).
  const int64_t ngroups = (int64_t)pb.wide.size();
  const int64_t per_xcd = (ngroups * num_kv_heads + 7) / 8;
  if (ngroups > 1 && per_xcd > 0) {
    const int64_t chunk = std::gcd(ngroups, per_xcd);
    for (int64_t c0 = 0; c0 < ngroups; c0 += chunk)
      std::stable_sort(pb.wide.begin() + c0, pb.wide.begin() + c0 + chunk,
                       [](const PlanWideGroup& a, const PlanWideGroup& b) {
                         return a.blk_hi - a.blk_lo > b.blk_hi - b.blk_lo;
                       });
  }

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
                                int32_t num_kv_heads, int32_t head_dim, int32_t flags, int32_t target_slices,
                                void* plan, size_t plan_capacity, pa_plan_info* info) {
  if (!info) return PA_ERR_NULL_POINTER;
  std::memset(info, 0, sizeof(*info));
  if (num_seqs < 0 || num_q_heads < 1 || num_kv_heads < 1 || max_blocks_per_seq < 1) return PA_ERR_BAD_SHAPE;
  if (num_q_heads % num_kv_heads) return PA_ERR_BAD_SHAPE;
  if (num_q_heads / num_kv_heads > 16) return PA_ERR_UNSUPPORTED;
  if (head_dim != 64 && head_dim != 128) return PA_ERR_UNSUPPORTED;
  if (target_slices < 0 || (flags & ~PA_PLAN_SHARE_PREFIX)) return PA_ERR_BAD_SHAPE;
  if (num_seqs > 0 && !context_lens) return PA_ERR_NULL_POINTER;
  if ((flags & PA_PLAN_SHARE_PREFIX) && num_seqs > 0 && !block_tables) return PA_ERR_NULL_POINTER;
  PlanBuild pb;
  const int st = build_plan(q_start, context_lens, block_tables, max_blocks_per_seq, num_seqs, num_q_heads,
                            num_kv_heads, flags, target_slices, pb);
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
  info->num_wgs = pb.wg_start.empty() ? 0 : (int32_t)pb.wg_start.size() - 1;
  info->num_wide_groups = (int32_t)pb.wide.size();
  for (const PlanItem& it : pb.items) info->max_item_columns = std::max(info->max_item_columns, it.ncols);
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
  if (!pb.wg_start.empty())
    std::memcpy(p + lay.wg_off, pb.wg_start.data(), pb.wg_start.size() * sizeof(int32_t));
  if (!pb.wide.empty()) std::memcpy(p + lay.wide_off, pb.wide.data(), pb.wide.size() * sizeof(PlanWideGroup));
  return PA_OK;
}
