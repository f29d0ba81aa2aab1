// Executor of a host-built attention plan on the matrix cores (gfx950):
// several query tokens per sequence with a causal horizon per query column,
// and prefix blocks shared by several sequences read once for all of them.
//
// What is computed: for every query column (new token, query head) the
// attention of "系统级优化…" section 3.1 over the positions its token sees
// (the causal mask of section 3.3, aligned to the end of the context), with
// K/V gathered page by page through the block table (section 2.3).
//
// One workgroup per slice of the plan (a list of items), one wave per KV
// head.  A wave loads each 16-token K/V block of an item's run once and
// applies it to the item's query columns (up to two tiles of 16) as the N
// dimension of the MFMAs (mfma_tile.h);
// columns may belong to different tokens of one sequence or to different
// sequences that share the block.  An item that is its columns' only
// contribution writes the output; otherwise it leaves (m, l, acc) partials
// that the merge kernel combines by log-sum-exp.
//
// Every index read from the plan is clamped into its array, so a corrupt
// plan yields wrong numbers rather than an out-of-bounds access.
#include "mfma_tile.h"
#include "pa_device.h"
#include "pa_internal.h"

namespace pa {
namespace {

__device__ __forceinline__ int clampi(int v, int lo, int hi) { return v < lo ? lo : (v > hi ? hi : v); }

template <int D, int kFmt>
struct PlannedPending {
  BlockRegs<D, kFmt> regs;
  int i;              // logical block
  bool live;          // false: a fetch past the item's end (a copy of its last block, folded in as a no-op)
  float ks, vs;
};

// This lane's query column of each tile of an item (columns past ncols are
// zero and see nothing).  Every lane loads (a clamped index) so that the
// number of loads does not depend on the lanes; the loaded values are only
// zeroed where used (run_item).
template <int kTiles>
__device__ __forceinline__ void load_item_columns(const PlannedArgs& a, int col0, int r, PlanColumn (&cols)[kTiles]) {
#pragma unroll
  for (int t = 0; t < kTiles; ++t) cols[t] = a.cols[clampi(col0 + 16 * t + r, 0, a.num_columns - 1)];
}

// Wait for loads into these registers here (not where the compiler would
// first copy them).
__device__ __forceinline__ void settle_reg(int& v) { asm volatile("" : "+v"(v)); }
template <int kTiles>
__device__ __forceinline__ void settle_cols(PlanColumn (&cols)[kTiles]) {
#pragma unroll
  for (int t = 0; t < kTiles; ++t) {
    settle_reg(cols[t].q_row);
    settle_reg(cols[t].j);
    settle_reg(cols[t].horizon);
  }
}

// What a wave needs of the item after the current one, loaded while the
// current one runs: its columns and the physical ids of its first 64 blocks.
template <int kTiles>
struct NextItem {
  PlanColumn cols[kTiles];
  int blk;              // lane j: physical id of block blk_lo + j
};

template <int kTiles>
__device__ __forceinline__ void load_next(const PlannedArgs& a, const PlanItem& it, int lane, NextItem<kTiles>& nx) {
  load_item_columns<kTiles>(a, it.col0, lane & 15, nx.cols);
  const int seq = clampi(it.seq, 0, a.num_seqs - 1);
  const int lo = max(it.blk_lo, 0);
  // every lane loads (an entry inside the table row); lanes past the item's blocks are never read out
  nx.blk = a.block_tables[(int64_t)seq * a.max_blocks_per_seq + clampi(lo + lane, 0, a.max_blocks_per_seq - 1)];
}

// Results of an item's tiles leave through this wave's LDS stage,
// kStageRows columns per pass, as whole 16-byte pieces with consecutive
// lanes on consecutive pieces (each lane holds a 16-byte-strided run of one
// column).  Records of a KV head are adjacent, so an item's records are
// consecutive rows; an output row's address comes from the lane that owns
// its column.
// A column's row from tiles in the transposed layout (lane (r, c): dims
// 16 nn + 4c + i in acc[nn][i]) into a stage row, as bf16 times `inv` or as fp32.
template <int D>
__device__ __forceinline__ void stage_tr_bf16(uint16_t* srow, const f32x4_t* acc, int c, float inv) {
#pragma unroll
  for (int nn = 0; nn < D / 16; ++nn)
    *reinterpret_cast<uint2*>(srow + 16 * nn + 4 * c) =
        make_uint2(pack_bf16x2(acc[nn][0] * inv, acc[nn][1] * inv), pack_bf16x2(acc[nn][2] * inv, acc[nn][3] * inv));
}
template <int D>
__device__ __forceinline__ void stage_tr_f32(float* srow, const f32x4_t* acc, int c) {
#pragma unroll
  for (int nn = 0; nn < D / 16; ++nn)
    *reinterpret_cast<float4*>(srow + 16 * nn + 4 * c) = make_float4(acc[nn][0], acc[nn][1], acc[nn][2], acc[nn][3]);
}

template <int D, int kFmt, int kTiles, bool kTr = false>
__device__ __forceinline__ void store_item_tiles(const PlannedArgs& a, const PlanItem& it,
                                                 const HeadState<D, kFmt> (&hs)[kTiles], const int64_t (&row)[kTiles],
                                                 int ncols, bool second, int g, int lane, float* stage) {
  static_assert(!kTr || kFmt == kFmtBf16, "transposed tiles carry no int4 bias");
  const int r = lane & 15, c = lane >> 4;
  const int d0 = (D / 4) * c;
#pragma unroll
  for (int t = 0; t < kTiles; ++t) {
    if (t > 0 && !second) break;
    const float L = hs[t].total_l();
    float o[4 * Tile<D, kFmt>::kE];
    hs[t].unpack(o);
    const int nt = min(16, ncols - 16 * t);                 // live columns of this tile
    const bool direct = it.rec0 < 0 || a.num_records <= 0;   // (no workspace: a plan not built here)
    // the tile's nt records stay inside this head's records even for a plan that was not built here
    const int64_t rec_row0 = (int64_t)g * a.num_records + clampi(it.rec0 + 16 * t, 0, max(a.num_records - nt, 0));
    if (!direct && c == 0 && r < nt) {
      const int64_t wr = (int64_t)g * a.num_records + clampi(it.rec0 + 16 * t + r, 0, a.num_records - 1);
      a.ws_m[wr] = hs[t].m;
      a.ws_l[wr] = L;
    }
    for (int rr = 0; rr < nt; rr += kStageRows) {
      const int nr = min(kStageRows, nt - rr);
      const bool mine = r >= rr && r < rr + nr;
      wave_lds_sync();                                      // the previous pass's reads are done
      if (direct) {
        if (mine) {
          uint16_t* srow = reinterpret_cast<uint16_t*>(stage) + (r - rr) * D;
          const float inv = L > 0.0f ? 1.0f / L : 0.0f;
          if constexpr (kTr) stage_tr_bf16<D>(srow, hs[t].acc, c, inv);
          else store_bf16_run<D>(srow, d0, o, inv);
        }
        wave_lds_sync();
        for (int pc = lane; pc < nr * D / 8; pc += 64) {
          const int col = rr + pc / (D / 8);
          const int64_t orow = __shfl(row[t], col, 64);       // lane col holds that column's output row
          reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(a.out) + orow * D)[pc % (D / 8)] =
              reinterpret_cast<const uint4*>(stage)[pc];
        }
      } else {
        if (mine) {
          if constexpr (kTr) stage_tr_f32<D>(stage + (r - rr) * D, hs[t].acc, c);
          else store_f32_run<D>(stage + (r - rr) * D, d0, o);
        }
        wave_lds_sync();
        // (rows past head g's records, only for a plan with fewer records than a tile has columns, are dropped)
        const int nw = (int)min<int64_t>(nr, (int64_t)(g + 1) * a.num_records - (rec_row0 + rr));
        float4* dst = reinterpret_cast<float4*>(a.ws_acc + (rec_row0 + rr) * D);
        for (int pc = lane; pc < nw * D / 4; pc += 64) dst[pc] = reinterpret_cast<const float4*>(stage)[pc];
      }
    }
  }
}

// The partial records of a wave's items other than its last wait in the
// wave's LDS outbox and are stored after the last item: a store is counted
// with the loads in vmcnt, so records stored when an item ends would make
// the next item's first waits also wait for them.  One entry per item, of
// fixed size: 8 header words (per tile the first record row, low and high
// word, then per tile its live columns), then per tile m[16], l[16] and 16
// rows of D floats.  Rows stored at once (the last item's, a direct item's,
// or an item that finds the outbox full) are staged through the same LDS
// after the outbox has been emptied.
template <int D, int kTiles>
__host__ __device__ constexpr int box_entry_words() { return 8 + kTiles * (32 + 16 * D); }

template <int D, int kFmt, int kTiles>
__device__ __forceinline__ void box_item_records(const PlannedArgs& a, const PlanItem& it,
                                                 const HeadState<D, kFmt> (&hs)[kTiles], int ncols, bool second,
                                                 int g, int lane, uint32_t* e) {
  const int r = lane & 15, c = lane >> 4;
  const int d0 = (D / 4) * c;
  uint32_t head[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
  for (int t = 0; t < kTiles; ++t) {
    if (t > 0 && !second) break;
    const int nt = min(16, ncols - 16 * t);
    const int64_t rec_row0 = (int64_t)g * a.num_records + clampi(it.rec0 + 16 * t, 0, max(a.num_records - nt, 0));
    head[2 * t] = (uint32_t)rec_row0;
    head[2 * t + 1] = (uint32_t)((uint64_t)rec_row0 >> 32);
    head[4 + t] = (uint32_t)nt;
    const float L = hs[t].total_l();
    float o[4 * Tile<D, kFmt>::kE];
    hs[t].unpack(o);
    float* ml = reinterpret_cast<float*>(e + 8 + t * (32 + 16 * D));
    if (c == 0 && r < nt) {
      ml[r] = hs[t].m;
      ml[16 + r] = L;
    }
    if (r < nt) store_f32_run<D>(ml + 32 + r * D, d0, o);
  }
  if (lane == 0) {
    reinterpret_cast<uint4*>(e)[0] = make_uint4(head[0], head[1], head[2], head[3]);
    reinterpret_cast<uint4*>(e)[1] = make_uint4(head[4], head[5], head[6], head[7]);
  }
}

// Store the outbox's n entries and empty it.
template <int D, int kTiles>
__device__ __forceinline__ void box_flush(const PlannedArgs& a, const uint32_t* box, int& n, int g, int lane) {
  if (n == 0) return;
  wave_lds_sync();                                    // every lane's entry writes are visible
  for (int k = 0; k < n; ++k) {
    const uint32_t* e = box + k * box_entry_words<D, kTiles>();
#pragma unroll
    for (int t = 0; t < kTiles; ++t) {
      const int nt = (int)__builtin_amdgcn_readfirstlane(e[4 + t]);
      if (nt <= 0) continue;
      const int64_t row0 = (int64_t)(((uint64_t)__builtin_amdgcn_readfirstlane(e[2 * t + 1]) << 32) |
                                     __builtin_amdgcn_readfirstlane(e[2 * t]));
      const float* ml = reinterpret_cast<const float*>(e + 8 + t * (32 + 16 * D));
      // rows past head g's records (only a plan with fewer records than a tile has columns) are dropped
      const int nw = (int)min<int64_t>(nt, (int64_t)(g + 1) * a.num_records - row0);
      if (lane < nw) {
        a.ws_m[row0 + lane] = ml[lane];
        a.ws_l[row0 + lane] = ml[16 + lane];
      }
      const float4* src = reinterpret_cast<const float4*>(ml + 32);
      float4* dst = reinterpret_cast<float4*>(a.ws_acc + row0 * D);
      for (int pc = lane; pc < nw * D / 4; pc += 64) dst[pc] = src[pc];
    }
  }
  wave_lds_sync();                                    // every read of the entries is done before they are rewritten
  n = 0;
}

// One plan item on one wave (KV head g): stream the item's blocks through
// kTiles MFMA tiles of 16 columns (columns 16t .. 16t+15 in tile t), then
// write the output or the partial records.  `cur` holds the item's columns
// and first block ids (loaded during the previous item); those of `next_it`
// (the following item, or this one again after the last) are loaded into
// `nx` once this item's own loads are issued, on every path alike.
//
// Vector memory operations complete in issue order and each wait is a count
// the compiler fixes per program point from the path with the fewest
// operations issued after the awaited one, so the block loop issues the same
// loads on every path (one loop exit; past the item's end a dead copy of its
// last block) and the wait before a block leaves the next block in flight.
template <int D, int kFmt, int kTiles>
__device__ __forceinline__ void run_item(const PlannedArgs& a, const PlanItem& it, const NextItem<kTiles>& cur,
                                         const PlanItem& next_it, NextItem<kTiles>& nx, int g, int lane,
                                         uint32_t* box, int& box_n, bool last) {
  const int r = lane & 15, c = lane >> 4;
  const int ncols = min(it.ncols, 16 * kTiles);
  const int G = a.num_q_heads / a.num_kv_heads;
  const int seq = clampi(it.seq, 0, a.num_seqs - 1);
  const int lo = max(it.blk_lo, 0), hi = min(it.blk_hi, a.max_blocks_per_seq);
  const int32_t* table = a.block_tables + (int64_t)seq * a.max_blocks_per_seq;
  const uint8_t* kbase = reinterpret_cast<const uint8_t*>(a.k_cache);
  const uint8_t* vbase = reinterpret_cast<const uint8_t*>(a.v_cache);

  int horizon[kTiles];
  int64_t row[kTiles];
  HeadState<D, kFmt> hs[kTiles];
#pragma unroll
  for (int t = 0; t < kTiles; ++t) {
    const bool live = 16 * t + r < ncols;
    horizon[t] = live ? cur.cols[t].horizon : 0;
    row[t] = live ? (int64_t)clampi(cur.cols[t].q_row, 0, a.num_q_tokens - 1) * a.num_q_heads + (int64_t)g * G +
                        clampi(cur.cols[t].j, 0, G - 1)
                  : 0;
    hs[t].begin_row(reinterpret_cast<const uint16_t*>(a.q), live ? row[t] : -1, c);
  }
  load_next<kTiles>(a, next_it, lane, nx);
  const bool second = kTiles > 1 && ncols > 16;     // wave-uniform

  // physical ids of 64 blocks at a time (lane j: block idbase + j)
  int idbase = lo, my_blk = cur.blk;
  auto fetch = [&](PlannedPending<D, kFmt>& p, int i) {
    p.live = i < hi;
    i = min(i, hi - 1);
    if (i - idbase >= 64) {
      // a new chunk of ids, waited for here (once per 64 blocks)
      idbase += 64;
      my_blk = table[clampi(idbase + lane, 0, a.max_blocks_per_seq - 1)];
      settle_reg(my_blk);
    }
    p.i = i;
    const int64_t blk = clampi(__builtin_amdgcn_readlane(my_blk, i - idbase), 0, a.num_blocks - 1);
    if constexpr (kFmt != kFmtBf16) {
      p.ks = a.k_scale[blk * a.num_kv_heads + g];
      p.vs = a.v_scale[blk * a.num_kv_heads + g];
    } else {
      p.ks = p.vs = 1.0f;
    }
    load_block<D, kFmt>(p.regs, kbase, vbase, blk, a.num_kv_heads, g, r, c);
    __builtin_amdgcn_sched_barrier(0);               // keep the loads ahead of the next consume's waits
  };
  auto consume = [&](const PlannedPending<D, kFmt>& p) {
    const int t0 = p.i * kBlockTokens;
    // a dead copy sees no token: the running max, sum and accumulator stay as they are
    const int valid = p.live ? min(kBlockTokens, it.kv_len - t0) : 0;
    const VOperands<D, kFmt> vo = make_voperands<D, kFmt>(p.regs, valid, c);
    hs[0].step_cols(p.regs, vo, valid, horizon[0] - t0, a.scale_log2 * p.ks, p.vs, c);
    if constexpr (kTiles > 1)
      if (second) hs[1].step_cols(p.regs, vo, valid, horizon[1] - t0, a.scale_log2 * p.ks, p.vs, c);
  };

  // two blocks in flight
  if (lo < hi) {
    PlannedPending<D, kFmt> p0, p1;
    fetch(p0, lo);
    for (int i = lo; i < hi; i += 2) {
      fetch(p1, i + 1);
      consume(p0);
      fetch(p0, i + 2);
      consume(p1);
    }
  }
  // the next item's loads have long landed: take their wait here
  settle_cols<kTiles>(nx.cols);
  settle_reg(nx.blk);
  if (ncols <= 0) return;

  // records of an item before the wave's last wait in the outbox
  const bool direct = it.rec0 < 0 || a.num_records <= 0;
  if (!direct && !last && box_n < a.box_entries) {
    box_item_records<D, kFmt, kTiles>(a, it, hs, ncols, second, g, lane, box + box_n * box_entry_words<D, kTiles>());
    ++box_n;
    return;
  }
  box_flush<D, kTiles>(a, box, box_n, g, lane);
  store_item_tiles<D, kFmt, kTiles>(a, it, hs, row, ncols, second, g, lane, reinterpret_cast<float*>(box));
}

// Workgroup x runs the items of slice x in order, one wave per KV head.
template <int D, int kFmt, int kTiles>
__global__ __launch_bounds__(64 * kBalancedMaxWaves) void attend_planned_kernel(PlannedArgs a) {
  // (the wave index in a scalar register, so addresses built from it are wave-uniform to the compiler)
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int g = blockIdx.y * a.waves_per_wg + wave;
  if (g >= a.num_kv_heads) return;
  // per wave: an outbox of box_entries entries, or kStageRows x D floats if larger
  extern __shared__ uint32_t s_box[];
  const int k0 = clampi(a.wg_start[blockIdx.x], 0, a.num_items);
  const int k1 = clampi(a.wg_start[blockIdx.x + 1], k0, a.num_items);
  if (k0 >= k1) return;
  uint32_t* box = s_box + wave * max(a.box_entries * box_entry_words<D, kTiles>(), kStageRows * D);
  int box_n = 0;
  // item headers, 64 at a time: lane j holds item kb + j
  int kb = k0;
  PlanItem mine{0, 0, 0, 0, 0, 0, -1, 0};
  auto load_headers = [&]() {
    if (kb + lane < k1) mine = a.items[kb + lane];
    settle_reg(mine.seq);
    settle_reg(mine.blk_lo);
    settle_reg(mine.blk_hi);
    settle_reg(mine.col0);
    settle_reg(mine.ncols);
    settle_reg(mine.kv_len);
    settle_reg(mine.rec0);
  };
  auto header = [&](int k) {
    const int j = k - kb;
    return PlanItem{__builtin_amdgcn_readlane(mine.seq, j),  __builtin_amdgcn_readlane(mine.blk_lo, j),
                    __builtin_amdgcn_readlane(mine.blk_hi, j), __builtin_amdgcn_readlane(mine.col0, j),
                    __builtin_amdgcn_readlane(mine.ncols, j),  __builtin_amdgcn_readlane(mine.kv_len, j),
                    __builtin_amdgcn_readlane(mine.rec0, j),   0};
  };
  load_headers();
  PlanItem it = header(k0);
  NextItem<kTiles> cur, nx;
  load_next<kTiles>(a, it, lane, cur);
  settle_cols<kTiles>(cur.cols);        // (the item loop then finds them settled on every path)
  settle_reg(cur.blk);
  for (int k = k0; k < k1; ++k) {
    PlanItem next_it = it;
    if (k + 1 < k1) {
      if (k + 1 - kb >= 64) {
        kb += 64;
        load_headers();
      }
      next_it = header(k + 1);
    }
    run_item<D, kFmt, kTiles>(a, it, cur, next_it, nx, g, lane, box, box_n, k + 1 == k1);
    it = next_it;
    cur = nx;
  }
  box_flush<D, kTiles>(a, box, box_n, g, lane);
}

// ---------------------------------------------------------------------------
// Wide groups: workgroup (group, KV head g), wave w runs item item0 + w of
// the group (up to two 16-column tiles).  The group's items share their
// sequence and first block, so every block of the group's run is read from
// memory once, by the whole workgroup, into LDS, and each wave folds it into
// its own tiles from there: the 4 items of a prefill chunk cost one read of
// each block instead of four.  Blocks alternate between two LDS buffers:
// block i+1 is written to one while block i is folded in from the other.
// Two workgroups share a CU.

// LDS block buffers: two alternating buffers of one block, of a pair of
// blocks for bf16 (which folds blocks in pairs)
template <int kFmt>
constexpr int wide_block_bufs() { return kFmt == kFmtBf16 ? 4 : 2; }
constexpr int kWideAhead = 4;   // blocks in flight per thread (6 and 8 measured no faster)

// A bf16 block's P.V operands are read from LDS with transpose reads
// (ds_read_b64_tr_b16): within each group of 16 lanes, lane 4a + b receives
// element b of the 8-byte runs addressed by lanes a, a + 4, a + 8, a + 12.
// Lane (r', c) addressing token 4c + r'/4 at dims 16 nn + 4 (r' % 4) .. + 3
// thus hands lane (r, c) V[4c .. 4c+3][16 nn + r]: the A operand (V^T) of
// the P.V MFMA for a tile covering dims 16 nn .. 16 nn + 15, with no
// register permutes.  The output of such tiles lies transposed: lane (r, c)
// holds dims 16 nn + 4c + i of column r in acc[nn][i].
template <int kFmt>
constexpr bool wide_transposed() { return kFmt == kFmtBf16; }

template <int D, int kFmt>
struct WideLayout {
  static constexpr int kRowBytes = D * Tile<D, kFmt>::kBits / 8;       // one token row of one head
  // padded rows: K rows (read 16 bytes a lane, a row per lane) 4 banks apart; V
  // rows for transpose reads (16 lanes read 4 rows x 32 bytes) 8 banks apart
  static constexpr int kStrideK = kRowBytes + 16;
  static constexpr int kStrideV = kRowBytes + (wide_transposed<kFmt>() ? 32 : 16);
  static constexpr int kVOff = kBlockTokens * kStrideK;                // V rows follow the K rows
  static constexpr int kBuf = kVOff + kBlockTokens * kStrideV;         // K then V of one block
  static constexpr int kPiecesPerRow = kRowBytes / 16;
  static constexpr int kPieces = 2 * kBlockTokens * kPiecesPerRow;     // 16-byte pieces per block, K and V
  static constexpr int kThreads = 64 * kWideTiles;
  static constexpr int kPiecesPerThread = (kPieces + kThreads - 1) / kThreads;
};

// The register layout of load_block, read from a block staged in LDS.
template <int D, int kFmt>
__device__ __forceinline__ void load_block_lds(BlockRegs<D, kFmt>& br, const uint8_t* buf, int r, int c) {
  using T = Tile<D, kFmt>;
  using L = WideLayout<D, kFmt>;
  constexpr int kKOff = (D / 4) * T::kBits / 8, kVOffR = T::kE * T::kBits / 8;
  load_words<T::kKWords>(buf + r * L::kStrideK + kKOff * c, br.k);
#pragma unroll
  for (int e = 0; e < 4; ++e)
    load_words<T::kVWords>(buf + L::kVOff + (4 * c + e) * L::kStrideV + kVOffR * r, br.v[e]);
}

typedef short lds_short4_t __attribute__((ext_vector_type(4)));

// A bf16 block's K registers (load_block_lds) and its P.V operands by
// transpose reads, in the transposed tile layout; tokens at or past `valid`
// get V = 0 (their slots may hold NaN).
template <int D>
__device__ __forceinline__ void load_block_lds_tr(BlockRegs<D, kFmtBf16>& br, VOperands<D, kFmtBf16>& vo,
                                                  const uint8_t* buf, int valid, int r, int c) {
  using T = Tile<D, kFmtBf16>;
  using L = WideLayout<D, kFmtBf16>;
  load_words<T::kKWords>(buf + r * L::kStrideK + (D / 4) * 2 * c, br.k);
  const uint8_t* vrow = buf + L::kVOff + (4 * c + (r >> 2)) * L::kStrideV + 8 * (r & 3);
#pragma unroll
  for (int nn = 0; nn < T::kE; ++nn) {
    typedef __attribute__((address_space(3))) lds_short4_t* lds_ptr;
    vo.v[nn] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_ptr)(vrow + 32 * nn));
  }
  if (valid < kBlockTokens) {
#pragma unroll
    for (int nn = 0; nn < T::kE; ++nn)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (4 * c + i >= valid) vo.v[nn][i] = 0;
  }
}

// Fold two consecutive blocks (32 tokens) of a bf16 cache into two tiles
// of columns at once: one running-max update per 32 tokens instead of two,
// and the P.V products as 16x16x32 MFMAs whose K index k = 8c + j runs
// over tokens 4c + j of the first block (j < 4) and 4c + j - 4 of the
// second, which is how the lane's P values and both blocks' V operands
// already lie.  valid1 = 0 when the second block is past the run (its
// operands must still be in range; they are masked whole).  The wave raises
// its issue priority while it issues its MFMA bursts, so the SIMD's other
// wave (of the other workgroup) fills the matrix core's gaps with its
// vector work instead of competing for the matrix core (2% on a prefill chunk).
template <int D>
__device__ __forceinline__ void step_pair_cols2(HeadState<D, kFmtBf16>& ha, HeadState<D, kFmtBf16>& hb,
                                                const BlockRegs<D, kFmtBf16>& b0, const BlockRegs<D, kFmtBf16>& b1,
                                                const VOperands<D, kFmtBf16>& v0, const VOperands<D, kFmtBf16>& v1,
                                                int valid0, int valid1, int cva0, int cva1, int cvb0, int cvb1,
                                                float sc, int c) {
  using H = HeadState<D, kFmtBf16>;
  f32x4_t sa0 = {0.0f, 0.0f, 0.0f, 0.0f}, sb0 = sa0, sa1 = sa0, sb1 = sa0;
  __builtin_amdgcn_s_setprio(1);
#pragma unroll
  for (int st = 0; st < Tile<D, kFmtBf16>::kKSteps; ++st) {
    const bf16x8_t k0 = H::k_operand(b0, st), k1 = H::k_operand(b1, st);
    sa0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k0, ha.qop[st], sa0, 0, 0, 0);
    sb0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k0, hb.qop[st], sb0, 0, 0, 0);
    sa1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k1, ha.qop[st], sa1, 0, 0, 0);
    sb1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k1, hb.qop[st], sb1, 0, 0, 0);
  }
  __builtin_amdgcn_s_setprio(0);
  float xa[8], xb[8];
  ha.rel_logits(sa0, sc, xa);
  ha.rel_logits(sa1, sc, xa + 4);
  hb.rel_logits(sb0, sc, xb);
  hb.rel_logits(sb1, sc, xb + 4);
  // one wave-uniform test for the context end and both tiles' horizons in both blocks
  if (valid0 < kBlockTokens || valid1 < kBlockTokens ||
      __ballot(cva0 < kBlockTokens || cva1 < kBlockTokens || cvb0 < kBlockTokens || cvb1 < kBlockTokens) != 0) {
    H::hide_tokens(xa, min(valid0, cva0), c);
    H::hide_tokens(xa + 4, min(valid1, cva1), c);
    H::hide_tokens(xb, min(valid0, cvb0), c);
    H::hide_tokens(xb + 4, min(valid1, cvb1), c);
  }
  ha.template fold<8>(xa);
  hb.template fold<8>(xb);
  const short4_t pa0 = ha.probs(xa, 1.0f), pa1 = ha.probs(xa + 4, 1.0f);
  const short4_t pb0 = hb.probs(xb, 1.0f), pb1 = hb.probs(xb + 4, 1.0f);
  const bf16x8_t pa = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(pa0, pa1, 0, 1, 2, 3, 4, 5, 6, 7));
  const bf16x8_t pb = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(pb0, pb1, 0, 1, 2, 3, 4, 5, 6, 7));
  __builtin_amdgcn_s_setprio(1);
#pragma unroll
  for (int nn = 0; nn < Tile<D, kFmtBf16>::kE; ++nn) {
    const bf16x8_t v = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(v0.v[nn], v1.v[nn], 0, 1, 2, 3, 4, 5, 6, 7));
    ha.acc[nn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(v, pa, ha.acc[nn], 0, 0, 0);
    hb.acc[nn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(v, pb, hb.acc[nn], 0, 0, 0);
  }
  __builtin_amdgcn_s_setprio(0);
}

template <int D, int kFmt>
__global__ __launch_bounds__(64 * kWideTiles, 2) void attend_wide_kernel(PlannedArgs a) {   // two workgroups per CU
  constexpr int kTiles = 2;
  using L = WideLayout<D, kFmt>;
  extern __shared__ __align__(16) uint8_t s_wide[];          // block buffers, then the waves' result stages
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int r = lane & 15, c = lane >> 4;
  // Workgroup b runs on XCD b mod 8.  Logical workgroup j = (KV head, group)
  // in head-major order goes to XCD j / per_xcd, so the groups of one
  // segment and head (consecutive j) share an XCD and its L2: they read the
  // same blocks at about the same time, and the memory serves each once.
  const int n = a.num_wide_groups * a.num_kv_heads;
  const int per_xcd = (n + 7) / 8;
  const int j = (int)(blockIdx.x % 8) * per_xcd + (int)(blockIdx.x / 8);
  if (j >= n) return;                                        // (every wave of the workgroup)
  const int g = j / a.num_wide_groups;
  const PlanWideGroup grp = a.wide[j % a.num_wide_groups];
  const int nitems = clampi(grp.nitems, 0, kWideTiles);
  if (nitems == 0) return;                                   // (every wave of the workgroup)
  const int k0 = clampi(grp.item0, 0, a.num_items - 1);
  const PlanItem first = a.items[k0];
  const int seq = clampi(first.seq, 0, a.num_seqs - 1);
  const int lo = max(grp.blk_lo, 0), hi = min(grp.blk_hi, a.max_blocks_per_seq);
  const bool has_item = wave < nitems;
  const PlanItem it = a.items[clampi(grp.item0 + min(wave, nitems - 1), 0, a.num_items - 1)];
  const int it_hi = min(it.blk_hi, hi);
  const int ncols = has_item ? min(it.ncols, 16 * kTiles) : 0;
  const int G = a.num_q_heads / a.num_kv_heads;
  const int32_t* table = a.block_tables + (int64_t)seq * a.max_blocks_per_seq;
  const uint8_t* kbase = reinterpret_cast<const uint8_t*>(a.k_cache);
  const uint8_t* vbase = reinterpret_cast<const uint8_t*>(a.v_cache);
  float* stage = reinterpret_cast<float*>(s_wide + wide_block_bufs<kFmt>() * L::kBuf) + wave * kStageRows * D;

  // this wave's columns and query rows
  PlanColumn cols[kTiles];
  load_item_columns<kTiles>(a, it.col0, r, cols);
  int horizon[kTiles];
  int64_t row[kTiles];
  HeadState<D, kFmt> hs[kTiles];
#pragma unroll
  for (int t = 0; t < kTiles; ++t) {
    const bool live = 16 * t + r < ncols;
    horizon[t] = live ? cols[t].horizon : 0;
    row[t] = live ? (int64_t)clampi(cols[t].q_row, 0, a.num_q_tokens - 1) * a.num_q_heads + (int64_t)g * G +
                        clampi(cols[t].j, 0, G - 1)
                  : 0;
    hs[t].begin_row(reinterpret_cast<const uint16_t*>(a.q), live ? row[t] : -1, c);
  }
  const bool second = ncols > 16;

  // physical ids and scales of 64 blocks at a time (lane j: block idbase + j), in every wave
  int idbase = lo, my_blk = 0;
  float my_ks = 1.0f, my_vs = 1.0f;
  auto load_ids = [&]() {
    my_blk = clampi(table[clampi(idbase + lane, 0, a.max_blocks_per_seq - 1)], 0, a.num_blocks - 1);
    if constexpr (kFmt != kFmtBf16) {
      my_ks = a.k_scale[(int64_t)my_blk * a.num_kv_heads + g];
      my_vs = a.v_scale[(int64_t)my_blk * a.num_kv_heads + g];
      asm volatile("" : "+v"(my_ks), "+v"(my_vs));
    }
    asm volatile("" : "+v"(my_blk));
  };
  load_ids();

  // This thread's 16-byte pieces of a block (piece tid + k * threads): K
  // rows first, then V rows.  Threads past the pieces load piece 0 and drop
  // it, so every wave issues the same loads per block.
  constexpr int kPP = L::kPiecesPerThread;
  bool loader[kPP];
  int64_t src_off[kPP];   // byte offset of the piece in a block's K (or V) rows of one head
  int lds_off[kPP];
  bool is_v[kPP];
#pragma unroll
  for (int k = 0; k < kPP; ++k) {
    const int piece = tid + k * L::kThreads;
    loader[k] = piece < L::kPieces;
    const int half = loader[k] && piece >= L::kPieces / 2 ? 1 : 0;
    const int pidx = loader[k] ? piece - half * (L::kPieces / 2) : 0;
    const int prow = pidx / L::kPiecesPerRow, pcol = pidx % L::kPiecesPerRow;
    is_v[k] = half != 0;
    src_off[k] = (int64_t)prow * L::kRowBytes + pcol * 16;
    lds_off[k] = half ? L::kVOff + prow * L::kStrideV + pcol * 16 : prow * L::kStrideK + pcol * 16;
  }
  // A block's pieces, with its scales taken while its id is in the window
  // (the window may move on before the block is folded in).
  struct Pieces {
    uint4 v[kPP];
    float ks, vs;
  };
  auto load_piece = [&](int i) {
    if (i - idbase >= 64) {
      idbase += 64;
      load_ids();
    }
    const int64_t blk = __builtin_amdgcn_readlane(my_blk, i - idbase);
    const int64_t head0 = (blk * a.num_kv_heads + g) * kBlockTokens * L::kRowBytes;
    Pieces pc;
#pragma unroll
    for (int k = 0; k < kPP; ++k)
      pc.v[k] = *reinterpret_cast<const uint4*>((is_v[k] ? vbase : kbase) + head0 + src_off[k]);
    pc.ks = pc.vs = 1.0f;
    if constexpr (kFmt != kFmtBf16) {
      pc.ks = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(my_ks), i - idbase));
      pc.vs = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(my_vs), i - idbase));
    }
    return pc;
  };
  auto store_pieces = [&](uint8_t* buf, const Pieces& pc) {
#pragma unroll
    for (int k = 0; k < kPP; ++k)
      if (loader[k]) *reinterpret_cast<uint4*>(buf + lds_off[k]) = pc.v[k];
  };
  auto lds_barrier = [&]() {
    __builtin_amdgcn_s_waitcnt(0xc07f);      // this wave's LDS writes and reads are done (lgkmcnt(0))
    __builtin_amdgcn_s_barrier();
  };

  if constexpr (kFmt == kFmtBf16) {
    // bf16: blocks go in pairs (step_pair_cols2), kAheadPairs pairs in
    // flight per thread, two LDS buffers of a pair each.  Step p issues the
    // loads of pair p + kAheadPairs, writes pair p + 1 (loaded kAheadPairs - 1
    // steps ago) to the other buffer, and folds pair p in from LDS (the
    // writes drain while it computes).  Past the run's end the loads fetch
    // copies of its last block, so every step issues the same loads.
    constexpr int kAheadPairs = 2;
    auto pbuf = [&](int p) { return s_wide + (p & 1) * 2 * L::kBuf; };
    const int npairs = (hi - lo + 1) / 2;
    if (lo < hi) {
      Pieces ring[kAheadPairs][2];
      auto load_pair = [&](Pieces* pr, int p) {
        pr[0] = load_piece(min(lo + 2 * p, hi - 1));
        pr[1] = load_piece(min(lo + 2 * p + 1, hi - 1));
      };
      auto store_pair = [&](int p, const Pieces* pr) {
        store_pieces(pbuf(p), pr[0]);
        store_pieces(pbuf(p) + L::kBuf, pr[1]);
      };
#pragma unroll
      for (int k = 0; k < kAheadPairs; ++k) load_pair(ring[k], k);
      store_pair(0, ring[0]);
      lds_barrier();
      for (int p0 = 0; p0 < npairs; p0 += kAheadPairs) {
#pragma unroll
        for (int k = 0; k < kAheadPairs; ++k) {
          const int p = p0 + k, i = lo + 2 * p;
          load_pair(ring[k], p + kAheadPairs);
          if (p + 1 < npairs) store_pair(p + 1, ring[(k + 1) % kAheadPairs]);
          if (p < npairs && has_item && i < it_hi) {
            const int t0 = i * kBlockTokens;
            const bool two = i + 1 < it_hi;           // (it_hi <= hi)
            const int valid0 = min(kBlockTokens, it.kv_len - t0);
            const int valid1 = two ? min(kBlockTokens, it.kv_len - t0 - kBlockTokens) : 0;
            BlockRegs<D, kFmt> b0, b1;
            VOperands<D, kFmt> v0, v1;
            load_block_lds_tr<D>(b0, v0, pbuf(p), valid0, r, c);
            load_block_lds_tr<D>(b1, v1, pbuf(p) + L::kBuf, valid1, r, c);
            if (second) {
              step_pair_cols2(hs[0], hs[1], b0, b1, v0, v1, valid0, valid1, horizon[0] - t0,
                              horizon[0] - t0 - kBlockTokens, horizon[1] - t0, horizon[1] - t0 - kBlockTokens,
                              a.scale_log2, c);
            } else {
              hs[0].step_cols(b0, v0, valid0, horizon[0] - t0, a.scale_log2, 1.0f, c);
              if (two) hs[0].step_cols(b1, v1, valid1, horizon[0] - t0 - kBlockTokens, a.scale_log2, 1.0f, c);
            }
          }
          lds_barrier();
        }
      }
    }
  } else {
    // kAhead blocks in flight per thread (a ring of pieces), two LDS buffers.
    // Step i folds block i in from LDS, having issued the load of block
    // i + kAhead, and writes block i + 1 (loaded kAhead - 1 steps ago) to the
    // other buffer.  Every step issues exactly one load (past the run's end a
    // copy of its last block) so the waits before the writes leave the later
    // loads in flight.
    constexpr int kAhead = kWideAhead;
    auto buf = [&](int i) { return s_wide + ((i - lo) & 1) * L::kBuf; };
    if (lo < hi) {
      Pieces ring[kAhead];
#pragma unroll
      for (int k = 0; k < kAhead; ++k) ring[k] = load_piece(min(lo + k, hi - 1));
      store_pieces(buf(lo), ring[0]);
      lds_barrier();
      for (int i0 = lo; i0 < hi; i0 += kAhead) {
#pragma unroll
        for (int k = 0; k < kAhead; ++k) {
          const int i = i0 + k;
          const float ks = ring[k].ks, vs = ring[k].vs;   // block i's, before the slot is reloaded
          ring[k] = load_piece(min(i + kAhead, hi - 1));
          if (i < hi && has_item && i < it_hi) {
            BlockRegs<D, kFmt> br;
            load_block_lds<D, kFmt>(br, buf(i), r, c);
            const int t0 = i * kBlockTokens;
            const int valid = min(kBlockTokens, it.kv_len - t0);
            const VOperands<D, kFmt> vo = make_voperands<D, kFmt>(br, valid, c);
            if (second)
              step_cols2(hs[0], hs[1], br, vo, valid, horizon[0] - t0, horizon[1] - t0, a.scale_log2 * ks, vs, c);
            else
              hs[0].step_cols(br, vo, valid, horizon[0] - t0, a.scale_log2 * ks, vs, c);
          }
          if (i + 1 < hi) store_pieces(buf(i + 1), ring[(k + 1) % kAhead]);
          lds_barrier();
        }
      }
    }
  }
  if (!has_item || ncols <= 0) return;
  store_item_tiles<D, kFmt, kTiles, wide_transposed<kFmt>()>(a, it, hs, row, ncols, second, g, lane, stage);
}

// out = sum_k 2^(m_k - M) acc_k / sum_k 2^(m_k - M) l_k over a merge row's
// records (M = max_k m_k; records whose column saw no token have m = -inf
// and weigh nothing).  One thread per (KV head, 4-wide chunk) of the row.
constexpr int kMergeThreads = 256;

template <int D>
__global__ __launch_bounds__(kMergeThreads) void attend_planned_merge_kernel(PlannedArgs a) {
  constexpr int kChunks = D / 4;
  const int t = blockIdx.y * kMergeThreads + threadIdx.x;
  const int g = t / kChunks, ch = t % kChunks;
  if (g >= a.num_kv_heads) return;
  const PlanMergeRow mr = a.rows[blockIdx.x];
  const int G = a.num_q_heads / a.num_kv_heads;
  const int e0 = clampi(mr.e0, 0, a.num_merge_entries), e1 = clampi(mr.e0 + mr.n, e0, a.num_merge_entries);
  float M = -INFINITY, den = 0.0f;
  float4 num = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  constexpr int kBatch = 8;                                     // records whose loads are in flight together
  for (int e = e0; e < e1; e += kBatch) {
    float mv[kBatch], lv[kBatch];
    float4 av[kBatch];
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      mv[k] = -INFINITY;
      lv[k] = 0.0f;
      av[k] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
      if (e + k < e1) {
        // the three loads go out together; an empty record's l and acc are
        // dropped by selection afterwards rather than by a branch on m that
        // would wait for m before issuing them
        const int64_t wr = (int64_t)g * a.num_records + clampi(a.entries[e + k], 0, a.num_records - 1);
        const float m = a.ws_m[wr];
        const float l = a.ws_l[wr];
        const float4 acc = reinterpret_cast<const float4*>(a.ws_acc + wr * D)[ch];
        const bool seen = m != -INFINITY;
        mv[k] = m;
        lv[k] = seen ? l : 0.0f;
        av[k] = seen ? acc : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
      }
    }
    float Mn = M;
#pragma unroll
    for (int k = 0; k < kBatch; ++k) Mn = fmaxf(Mn, mv[k]);
    if (Mn == -INFINITY) continue;                              // nothing seen yet
    const float sc = __builtin_amdgcn_exp2f(M - Mn);            // 0 while M is -inf
    den *= sc;
    num.x *= sc; num.y *= sc; num.z *= sc; num.w *= sc;
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      const float wt = __builtin_amdgcn_exp2f(mv[k] - Mn);      // 0 for empty records
      den += wt * lv[k];
      num.x += wt * av[k].x; num.y += wt * av[k].y; num.z += wt * av[k].z; num.w += wt * av[k].w;
    }
    M = Mn;
  }
  const float inv = den > 0.0f ? 1.0f / den : 0.0f;
  const int64_t orow = (int64_t)clampi(mr.q_row, 0, a.num_q_tokens - 1) * a.num_q_heads + (int64_t)g * G +
                       clampi(mr.j, 0, G - 1);
  const uint2 packed = make_uint2(f32_to_bf16_bits_rne(num.x * inv) | (f32_to_bf16_bits_rne(num.y * inv) << 16),
                                  f32_to_bf16_bits_rne(num.z * inv) | (f32_to_bf16_bits_rne(num.w * inv) << 16));
  *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(a.out) + orow * D + 4 * ch) = packed;
}

}  // namespace

hipError_t launch_attend_planned(const PlannedArgs& a_in, hipStream_t stream) {
  PlannedArgs a = a_in;
  const dim3 grid(a.num_wgs, a.head_groups);
  const dim3 block(64 * a.waves_per_wg);
  const int f = a.cache_dtype == PA_DTYPE_FP8_E4M3 ? kFmtFp8 : (a.cache_dtype == PA_DTYPE_INT4 ? kFmtInt4 : kFmtBf16);
  const int tiles = a.max_item_columns > 16 ? 2 : 1;
  // the outbox: up to two record entries per wave, the workgroup within
  // 158 KB of LDS (about 2048 waves over the device: 8 waves per CU)
  const size_t entry = (size_t)(a.head_dim == 128 ? (tiles == 2 ? box_entry_words<128, 2>() : box_entry_words<128, 1>())
                                                  : (tiles == 2 ? box_entry_words<64, 2>() : box_entry_words<64, 1>())) *
                       sizeof(float);
  const size_t stage_bytes = (size_t)kStageRows * a.head_dim * sizeof(float);
  const size_t budget = ((size_t)158 << 10) / (size_t)(a.waves_per_wg < 8 ? 8 : a.waves_per_wg);   // per wave
  size_t entries = budget / entry;
  if (entries > 2) entries = 2;
  a.box_entries = (int32_t)entries;
  const size_t per_wave = entries * entry > stage_bytes ? entries * entry : stage_bytes;
  const size_t lds = (size_t)a.waves_per_wg * per_wave;
#define PA_LAUNCH(D_, F_, T_) hipLaunchKernelGGL((attend_planned_kernel<D_, F_, T_>), grid, block, lds, stream, a)
#define PA_LAUNCH_T(D_, F_) do { if (tiles == 2) PA_LAUNCH(D_, F_, 2); else PA_LAUNCH(D_, F_, 1); } while (0)
  if (a.head_dim == 128) {
    if (f == kFmtFp8) PA_LAUNCH_T(128, kFmtFp8);
    else if (f == kFmtInt4) PA_LAUNCH_T(128, kFmtInt4);
    else PA_LAUNCH_T(128, kFmtBf16);
  } else {
    if (f == kFmtFp8) PA_LAUNCH_T(64, kFmtFp8);
    else PA_LAUNCH_T(64, kFmtBf16);
  }
#undef PA_LAUNCH_T
#undef PA_LAUNCH
  return hipGetLastError();
}

// LDS of a wide workgroup: two block buffers, then a result stage per wave.
template <int D, int kFmt>
size_t wide_lds_bytes() {
  return wide_block_bufs<kFmt>() * (size_t)WideLayout<D, kFmt>::kBuf +
         (size_t)kWideTiles * kStageRows * D * sizeof(float);
}

hipError_t launch_attend_wide(const PlannedArgs& a, hipStream_t stream) {
  const int n = a.num_wide_groups * a.num_kv_heads;
  const dim3 grid((n + 7) / 8 * 8);           // XCD-ordered (attend_wide_kernel); extra workgroups exit
  const dim3 block(64 * kWideTiles);
  const int f = a.cache_dtype == PA_DTYPE_FP8_E4M3 ? kFmtFp8 : (a.cache_dtype == PA_DTYPE_INT4 ? kFmtInt4 : kFmtBf16);
#define PA_LAUNCH(D_, F_) \
  hipLaunchKernelGGL((attend_wide_kernel<D_, F_>), grid, block, (wide_lds_bytes<D_, F_>()), stream, a)
  if (a.head_dim == 128) {
    if (f == kFmtFp8) PA_LAUNCH(128, kFmtFp8);
    else if (f == kFmtInt4) PA_LAUNCH(128, kFmtInt4);
    else PA_LAUNCH(128, kFmtBf16);
  } else {
    if (f == kFmtFp8) PA_LAUNCH(64, kFmtFp8);
    else PA_LAUNCH(64, kFmtBf16);
  }
#undef PA_LAUNCH
  return hipGetLastError();
}

hipError_t launch_attend_planned_merge(const PlannedArgs& a, hipStream_t stream) {
  const int per_row = a.num_kv_heads * (a.head_dim / 4);
  const dim3 grid(a.num_merge_rows, (per_row + kMergeThreads - 1) / kMergeThreads);
  if (a.head_dim == 128)
    hipLaunchKernelGGL((attend_planned_merge_kernel<128>), grid, dim3(kMergeThreads), 0, stream, a);
  else
    hipLaunchKernelGGL((attend_planned_merge_kernel<64>), grid, dim3(kMergeThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace pa
