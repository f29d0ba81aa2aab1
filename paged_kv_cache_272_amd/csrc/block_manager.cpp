// Host block manager for the paged KV cache: a global pool of 16-token
// physical blocks, per-sequence block tables, reference counts, sharing and
// copy-on-write, and the per-iteration step of continuous batching.
//
// Model ("系统级优化…" section 2.3, the PagedAttention diagram; "17 · 连续批处理与
// PagedAttention" sections 二 and 三):
//   * every block holds 16 tokens; one manager hands blocks out of a global
//     pool, and a sequence's blocks need not be contiguous;
//   * a sequence of n tokens holds ceil(n / 16) blocks, so at most one
//     partly filled block per sequence is wasted;
//   * blocks freed by a finished sequence are handed out again at once (the
//     free list is a stack: the most recently freed block goes out first);
//   * sequences may share blocks (a forked sample references its parent's
//     blocks; reference counts track the sharers), and a shared block is
//     copied only when a sharer writes into it (copy-on-write);
//   * continuous batching appends one token to every running sequence per
//     iteration and admits or retires sequences between iterations; when the
//     pool cannot hold the next iteration a sequence must be preempted (its
//     blocks freed, to be recomputed later), which the caller decides.
// Everything here is host code, single-threaded per manager.
#include <algorithm>
#include <cstring>
#include <deque>
#include <new>
#include <unordered_map>
#include <vector>

#include "pa_internal.h"

struct pa_block_manager {
  struct Seq {
    std::vector<int32_t> blocks;
    int64_t tokens = 0;
  };
  int32_t num_blocks = 0;
  std::deque<int32_t> free_list;               // front = next handed out
  std::vector<int32_t> refcount;
  std::unordered_map<int32_t, Seq> seqs;
};

namespace pa {
namespace {

constexpr int kBlockTokens = PA_BLOCK_SIZE;

int32_t blocks_for(int64_t tokens) { return (int32_t)((tokens + kBlockTokens - 1) / kBlockTokens); }

int32_t take_block(pa_block_manager& m) {
  const int32_t b = m.free_list.front();
  m.free_list.pop_front();
  m.refcount[b] = 1;
  return b;
}

void drop_block(pa_block_manager& m, int32_t b) {
  if (--m.refcount[b] == 0) m.free_list.push_front(b);
}

// Blocks one more token needs: a new block when the last is full (or there
// is none), a private copy when the last block is shared.
int32_t blocks_for_append(const pa_block_manager& m, const pa_block_manager::Seq& s) {
  if (s.tokens % kBlockTokens == 0) return 1;
  return m.refcount[s.blocks.back()] > 1 ? 1 : 0;
}

// Append one token; returns its slot, and the (src, dst) copy pair when the
// last block had to be copied (else src = dst = -1).  The caller has checked
// that a free block exists when one is needed.
int64_t append_token(pa_block_manager& m, pa_block_manager::Seq& s, int32_t* src, int32_t* dst) {
  *src = *dst = -1;
  if (s.tokens % kBlockTokens == 0) {
    s.blocks.push_back(take_block(m));
  } else if (m.refcount[s.blocks.back()] > 1) {
    const int32_t old = s.blocks.back();
    const int32_t fresh = take_block(m);
    drop_block(m, old);
    s.blocks.back() = fresh;
    *src = old;
    *dst = fresh;
  }
  const int64_t pos = s.tokens++;
  return (int64_t)s.blocks[pos / kBlockTokens] * kBlockTokens + pos % kBlockTokens;
}

}  // namespace
}  // namespace pa

using namespace pa;

PA_EXPORT pa_block_manager* pa_bm_create(int32_t num_blocks, const int32_t* free_order) {
  if (num_blocks < 1) return nullptr;
  pa_block_manager* m = new (std::nothrow) pa_block_manager();
  if (!m) return nullptr;
  m->num_blocks = num_blocks;
  m->refcount.assign(num_blocks, 0);
  if (free_order) {
    std::vector<char> seen(num_blocks, 0);
    for (int32_t i = 0; i < num_blocks; ++i) {
      const int32_t b = free_order[i];
      if (b < 0 || b >= num_blocks || seen[b]) {
        delete m;
        return nullptr;
      }
      seen[b] = 1;
      m->free_list.push_back(b);
    }
  } else {
    for (int32_t b = 0; b < num_blocks; ++b) m->free_list.push_back(b);
  }
  return m;
}

PA_EXPORT void pa_bm_destroy(pa_block_manager* m) { delete m; }

PA_EXPORT int pa_bm_add(pa_block_manager* m, int32_t seq, int32_t num_tokens) {
  if (!m) return PA_ERR_NULL_POINTER;
  if (num_tokens < 0) return PA_ERR_BAD_SHAPE;
  if (m->seqs.count(seq)) return PA_ERR_BAD_SHAPE;
  const int32_t need = blocks_for(num_tokens);
  if ((size_t)need > m->free_list.size()) return PA_ERR_OUT_OF_BLOCKS;
  pa_block_manager::Seq s;
  for (int32_t i = 0; i < need; ++i) s.blocks.push_back(take_block(*m));
  s.tokens = num_tokens;
  m->seqs.emplace(seq, std::move(s));
  return PA_OK;
}

PA_EXPORT int pa_bm_fork(pa_block_manager* m, int32_t parent, int32_t child) {
  if (!m) return PA_ERR_NULL_POINTER;
  auto it = m->seqs.find(parent);
  if (it == m->seqs.end() || m->seqs.count(child)) return PA_ERR_BAD_SHAPE;
  pa_block_manager::Seq s = it->second;
  for (int32_t b : s.blocks) ++m->refcount[b];
  m->seqs.emplace(child, std::move(s));
  return PA_OK;
}

PA_EXPORT int pa_bm_free(pa_block_manager* m, int32_t seq) {
  if (!m) return PA_ERR_NULL_POINTER;
  auto it = m->seqs.find(seq);
  if (it == m->seqs.end()) return PA_ERR_BAD_SHAPE;
  // release from the last block back: the blocks return to the front of the free list in table order
  for (auto b = it->second.blocks.rbegin(); b != it->second.blocks.rend(); ++b) drop_block(*m, *b);
  m->seqs.erase(it);
  return PA_OK;
}

PA_EXPORT int pa_bm_append(pa_block_manager* m, int32_t seq, int64_t* slot, int32_t* cow_src, int32_t* cow_dst) {
  if (!m || !slot || !cow_src || !cow_dst) return PA_ERR_NULL_POINTER;
  auto it = m->seqs.find(seq);
  if (it == m->seqs.end()) return PA_ERR_BAD_SHAPE;
  if ((size_t)blocks_for_append(*m, it->second) > m->free_list.size()) return PA_ERR_OUT_OF_BLOCKS;
  *slot = append_token(*m, it->second, cow_src, cow_dst);
  return PA_OK;
}

PA_EXPORT int pa_bm_table(const pa_block_manager* m, int32_t seq, int32_t* table, int32_t capacity,
                          int32_t* num_blocks, int64_t* num_tokens) {
  if (!m || !num_blocks || !num_tokens) return PA_ERR_NULL_POINTER;
  auto it = m->seqs.find(seq);
  if (it == m->seqs.end()) return PA_ERR_BAD_SHAPE;
  const auto& s = it->second;
  *num_blocks = (int32_t)s.blocks.size();
  *num_tokens = s.tokens;
  if (!table) return PA_OK;
  if (capacity < (int32_t)s.blocks.size()) return PA_ERR_WORKSPACE;
  std::copy(s.blocks.begin(), s.blocks.end(), table);
  return PA_OK;
}

PA_EXPORT int pa_bm_get_stats(const pa_block_manager* m, pa_bm_stats* out) {
  if (!m || !out) return PA_ERR_NULL_POINTER;
  std::memset(out, 0, sizeof(*out));
  out->num_blocks = m->num_blocks;
  out->free_blocks = (int32_t)m->free_list.size();
  out->num_seqs = (int32_t)m->seqs.size();
  int64_t refs = 0;
  for (const auto& kv : m->seqs) {
    out->logical_tokens += kv.second.tokens;
    refs += (int64_t)kv.second.blocks.size();
  }
  out->block_refs = refs;
  // tokens actually stored: a shared block holds its furthest sharer's tokens once
  std::vector<int32_t> used(m->num_blocks, 0);
  for (const auto& kv : m->seqs) {
    const auto& s = kv.second;
    for (size_t i = 0; i < s.blocks.size(); ++i) {
      const int32_t n = (int32_t)std::min<int64_t>(kBlockTokens, s.tokens - (int64_t)i * kBlockTokens);
      used[s.blocks[i]] = std::max(used[s.blocks[i]], n);
    }
  }
  for (int32_t b = 0; b < m->num_blocks; ++b) out->stored_tokens += used[b];
  return PA_OK;
}

PA_EXPORT int pa_bm_step(pa_block_manager* m, const int32_t* seqs, int32_t num_seqs, int32_t max_blocks_per_seq,
                         int32_t* block_tables, int32_t* context_lens, int64_t* slot_mapping, int32_t* cow_pairs,
                         int32_t* num_cow, int32_t* blocks_short) {
  if (!m || !num_cow || !blocks_short) return PA_ERR_NULL_POINTER;
  *num_cow = 0;
  *blocks_short = 0;
  if (num_seqs < 0 || max_blocks_per_seq < 1) return PA_ERR_BAD_SHAPE;
  if (num_seqs == 0) return PA_OK;
  if (!seqs || !block_tables || !context_lens || !slot_mapping || !cow_pairs) return PA_ERR_NULL_POINTER;
  // check everything before changing anything: the step is all or nothing
  std::vector<pa_block_manager::Seq*> batch(num_seqs);
  int64_t need = 0;
  for (int32_t i = 0; i < num_seqs; ++i) {
    auto it = m->seqs.find(seqs[i]);
    if (it == m->seqs.end()) return PA_ERR_BAD_SHAPE;
    for (int32_t k = 0; k < i; ++k)
      if (batch[k] == &it->second) return PA_ERR_BAD_SHAPE;     // a sequence twice in one step
    batch[i] = &it->second;
    if (blocks_for(it->second.tokens + 1) > max_blocks_per_seq) return PA_ERR_BAD_SHAPE;
    need += blocks_for_append(*m, it->second);
  }
  // a block shared only inside this batch is copied by the first sharer that
  // writes it; the later sharer then owns it alone and needs no copy, so
  // `need` can only overestimate
  if (need > (int64_t)m->free_list.size()) {
    *blocks_short = (int32_t)(need - (int64_t)m->free_list.size());
    return PA_ERR_OUT_OF_BLOCKS;
  }
  for (int32_t i = 0; i < num_seqs; ++i) {
    int32_t src, dst;
    slot_mapping[i] = append_token(*m, *batch[i], &src, &dst);
    if (src >= 0) {
      cow_pairs[2 * *num_cow] = src;
      cow_pairs[2 * *num_cow + 1] = dst;
      ++*num_cow;
    }
  }
  for (int32_t i = 0; i < num_seqs; ++i) {
    const auto& s = *batch[i];
    int32_t* row = block_tables + (int64_t)i * max_blocks_per_seq;
    std::copy(s.blocks.begin(), s.blocks.end(), row);
    std::fill(row + s.blocks.size(), row + max_blocks_per_seq, s.blocks.empty() ? 0 : s.blocks.back());
    context_lens[i] = (int32_t)s.tokens;
  }
  return PA_OK;
}
