// Paged decode on the matrix cores (gfx950 MFMA), bf16 query with a bf16,
// e4m3 or int4 KV cache.
//
// What is computed is the attention of "系统级优化…" section 3.1 for one
// query token per sequence, over K/V gathered page by page through the block
// table (section 2.3), with the online-softmax tiling idea of section 3.2
// (the running-max rescale that page omits is applied exactly).
//
// One wave owns one KV head and applies each 16-token K/V block it loads to
// all G query heads of that head's group at once: the query heads are the N
// dimension of the MFMAs, so a block is read from HBM once per group.
//
// The register layout of a block, the two MFMA contractions and the online
// softmax are in mfma_tile.h.
//
// Two work splits (see DecodeArgs): a partition grid, and a balanced split
// in which every workgroup takes an equal slice of all (sequence, block)
// units, so no compute unit idles at the end of the launch.
#include "mfma_tile.h"
#include "pa_device.h"
#include "pa_internal.h"

namespace pa {
namespace {

constexpr int kPartWaves = 4;
constexpr int kPartThreads = 64 * kPartWaves;

__device__ __forceinline__ int clamp_context(const DecodeArgs& a, int b) {
  const int ctx = a.context_lens[b];
  return ctx < 0 ? 0 : min(min(ctx, a.max_context_len), a.max_blocks_per_seq * kBlockTokens);
}

// ---------------------------------------------------------------------------
// Partition grid: one workgroup of 4 waves per (group of 4 consecutive
// partitions, KV head, sequence); wave w folds in partition 4 * group + w
// (up to 32 blocks of 16 tokens) and the waves merge their partitions by
// log-sum-exp in LDS, so one partial record (or the output, when the group
// covers the whole sequence) leaves per group of 4 partitions.

template <int D, int kFmt>
__global__ __launch_bounds__(kPartThreads) void decode_mfma_kernel(DecodeArgs a) {
  using T = Tile<D, kFmt>;
  constexpr int kE = T::kE;
  __shared__ float lds_m[kPartWaves][16];
  __shared__ float lds_l[kPartWaves][16];
  __shared__ f32x4_t lds_acc[kPartWaves][kE][64];

  const int grp = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r = lane & 15, c = lane >> 4;
  const int G = a.num_q_heads / a.num_kv_heads;
  const int P = a.partition_tokens;

  const int ctx = clamp_context(a, b);
  const int ngroups = (ctx + kPartWaves * P - 1) / (kPartWaves * P);
  const int64_t head0 = (int64_t)b * a.num_q_heads + (int64_t)g * G;
  uint16_t* out = reinterpret_cast<uint16_t*>(a.out);
  if (ctx == 0) {
    if (grp == 0)
      for (int i = threadIdx.x; i < G * D; i += kPartThreads) out[head0 * D + i] = 0;
    return;
  }
  if (grp >= ngroups) return;                           // (every wave of the workgroup)
  const int t0 = (grp * kPartWaves + wave) * P;         // this wave's partition
  const int n = max(0, min(P, ctx - t0));
  const int nw = (n + kBlockTokens - 1) / kBlockTokens; // its blocks (<= 32)

  HeadState<D, kFmt> hs;
  hs.begin(reinterpret_cast<const uint16_t*>(a.q), head0, G, r, c);
  // physical ids (and fp8/int4 scales) of this wave's blocks: lane j holds block j
  int my_blk = 0;
  float my_ks = 1.0f, my_vs = 1.0f;
  if (lane < nw) {
    my_blk = clamp_block(a.block_tables[(int64_t)b * a.max_blocks_per_seq + t0 / kBlockTokens + lane], a.num_blocks);
    if constexpr (kFmt != kFmtBf16) {
      my_ks = a.k_scale[(int64_t)my_blk * a.num_kv_heads + g];
      my_vs = a.v_scale[(int64_t)my_blk * a.num_kv_heads + g];
    }
  }
  const uint8_t* kbase = reinterpret_cast<const uint8_t*>(a.k_cache);
  const uint8_t* vbase = reinterpret_cast<const uint8_t*>(a.v_cache);
  auto step = [&](const BlockRegs<D, kFmt>& br, int i) {
    float sc = a.scale_log2, vs = 1.0f;
    if constexpr (kFmt != kFmtBf16) {
      sc *= __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(my_ks), i));
      vs = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(my_vs), i));
    }
    const int valid = min(kBlockTokens, n - i * kBlockTokens);
    hs.step(br, valid, sc, vs, c);
  };

  // software pipeline: the next block's loads are in flight while this one computes
  BlockRegs<D, kFmt> b0, b1;
  if (nw > 0) load_block<D, kFmt>(b0, kbase, vbase, __builtin_amdgcn_readlane(my_blk, 0), a.num_kv_heads, g, r, c);
  for (int i = 0; i < nw; i += 2) {
    if (i + 1 < nw)
      load_block<D, kFmt>(b1, kbase, vbase, __builtin_amdgcn_readlane(my_blk, i + 1), a.num_kv_heads, g, r, c);
    step(b0, i);
    if (i + 1 < nw) {
      if (i + 2 < nw)
        load_block<D, kFmt>(b0, kbase, vbase, __builtin_amdgcn_readlane(my_blk, i + 2), a.num_kv_heads, g, r, c);
      step(b1, i + 1);
    }
  }

  // ---- wave totals, then the 4 partitions' log-sum-exp merge through LDS
  const float lw = hs.total_l();
  if (c == 0) {
    lds_m[wave][r] = hs.m;
    lds_l[wave][r] = lw;
  }
  hs.settle();
#pragma unroll
  for (int t = 0; t < kE; ++t) lds_acc[wave][t][lane] = hs.acc[t];
  __syncthreads();
  if (wave != 0) return;

  float mw[kPartWaves], M = -INFINITY;
#pragma unroll
  for (int w = 0; w < kPartWaves; ++w) {
    mw[w] = lds_m[w][r];
    M = fmaxf(M, mw[w]);
  }
  float L = 0.0f, wt[kPartWaves];
#pragma unroll
  for (int w = 0; w < kPartWaves; ++w) {
    wt[w] = mw[w] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(mw[w] - M);   // partitions past the context weigh nothing
    L += wt[w] * lds_l[w][r];
  }
  float o[4 * kE];
#pragma unroll
  for (int nn = 0; nn < kE; ++nn) {
    f32x4_t v = lds_acc[0][nn][lane] * wt[0];
#pragma unroll
    for (int w = 1; w < kPartWaves; ++w) v += lds_acc[w][nn][lane] * wt[w];
#pragma unroll
    for (int j = 0; j < 4; ++j) o[kE * j + nn] = v[j];
  }
  if (r >= G) return;
  const int64_t row = head0 + r;
  const int d0 = (D / 4) * c;
  if (ngroups == 1) {
    store_bf16_run<D>(out + row * D, d0, o, 1.0f / L);
  } else {
    const int64_t wr = row * a.num_recs + grp;
    store_f32_run<D>(a.ws_acc + wr * D, d0, o);
    if (c == 0) {
      a.ws_m[wr] = M;
      a.ws_l[wr] = L;
    }
  }
}

// ---------------------------------------------------------------------------
// Balanced split.  Units are (sequence, 16-token block) pairs laid end to end
// in sequence order; sequence b owns units [start[b], start[b+1]).  Workgroup
// x takes units [floor(x*U/n), floor((x+1)*U/n)) (n = min(num_wgs, U)); wave w of
// workgroup (x, y) handles KV head y*waves + w over that slice.

// n = min(workgroups, U) slices, so none is empty; slice x covers units
// [floor(x*U/n), floor((x+1)*U/n)): sizes differ by at most one.
__device__ __forceinline__ int num_slices(int U, int num_wgs) { return min(U, num_wgs); }
__device__ __forceinline__ int slice_begin(int x, int U, int n) { return (int)((int64_t)x * U / n); }
// The slice holding unit u: the largest x with slice_begin(x) <= u.
__device__ __forceinline__ int slice_of(int u, int U, int n) {
  return (int)(((int64_t)(u + 1) * n + U - 1) / U) - 1;
}

static_assert(kBalancedStageRows == kStageRows, "one staging pass: the same rows on host and device");

struct UnitIds {
  int b, i, blk;       // lane j: the (sequence, logical block, physical block) of unit base + j
  float ks, vs;        // e4m3/int4: that block's scales for this wave's head
};

__device__ __forceinline__ int find_sequence(const int* start, int num_seqs, int u) {
  // largest b with start[b] <= u (start is non-decreasing; start[num_seqs] > u)
  int lo = 0, hi = num_seqs - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (start[mid] <= u) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

// Table entries (and block scales) of 64 units, one per lane, waited for
// here: a register holding a load still in flight cannot be copied without a
// wait, and the compiler copies these ids across loop iterations.  One or
// two waits per 64 units.
template <bool kScaled>
__device__ __forceinline__ UnitIds unit_ids(const DecodeArgs& a, const int* start, int base, int u1, int g, int lane) {
  UnitIds id{0, 0, 0, 1.0f, 1.0f};
  const int u = base + lane;
  if (u < u1) {
    id.b = find_sequence(start, a.num_seqs, u);
    id.i = u - start[id.b];
    id.blk = clamp_block(a.block_tables[(int64_t)id.b * a.max_blocks_per_seq + id.i], a.num_blocks);
    if constexpr (kScaled) {
      id.ks = a.k_scale[(int64_t)id.blk * a.num_kv_heads + g];
      id.vs = a.v_scale[(int64_t)id.blk * a.num_kv_heads + g];
    }
  }
  asm volatile("" : "+v"(id.blk));
  return id;
}

template <int D, int kFmt>
struct Pending {
  // bf16 caches: the query rows of the unit's sequence come with every unit
  // (load_query; used when the unit starts the sequence).  e4m3/int4 blocks
  // are small enough that those four extra loads per unit cost more than
  // loading the query when a sequence starts.
  static constexpr bool kQueryInFetch = kFmt == kFmtBf16;
  BlockRegs<D, kFmt> regs;
  uint4 q[kQueryInFetch ? D / 32 : 1];
  int64_t blk;
  int b, i, ctx;
  float ks, vs;
  bool live;                // false: a fetch past the slice's end (a copy of its last unit, folded in as a no-op)
  bool starts;              // first unit of its sequence in this slice
  int off;                  // appending: slot of the sequence's newest token in this block, else -1
  bool row_staged;          // ... and that token's K/V runs sit in the staging registers
};

// e4m3/int4 caches: registers for the newest token's bf16 runs, filled in
// fetch() when a unit holds that token.  One set serves both units in
// flight: when the other unit still holds it (two sequences ending one unit
// apart) the unit loads at consume time instead and waits there.
template <int D>
struct Staging {
  uint32_t nk[D / 8];       // K run (lane r == off) as bf16 pairs
  uint32_t nv[D / 32];      // V run (lane group c == off / 4)
  bool row_busy = false;
};

// bf16 cache: a block's registers, where the lanes that hold the newest
// token's K run (r == off) and V run (token 4c+e == off) read it from the new
// rows kn, vn instead of the cache slot (written later in the same launch).
// off = -1: a plain block load.
template <int D>
__device__ __forceinline__ void load_block_with_row(BlockRegs<D, kFmtBf16>& br, const uint8_t* kbase,
                                                    const uint8_t* vbase, int64_t blk, int num_kv_heads, int g, int r,
                                                    int c, int off, const uint16_t* kn, const uint16_t* vn) {
  using T = Tile<D, kFmtBf16>;
  const int64_t head_base = (blk * num_kv_heads + g) * kBlockTokens;
  const uint8_t* kp = r == off ? reinterpret_cast<const uint8_t*>(kn + (D / 4) * c)
                               : kbase + T::bytes((head_base + r) * D + (D / 4) * c);
  load_words<T::kKWords>(kp, br.k);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const uint8_t* vp = 4 * c + e == off ? reinterpret_cast<const uint8_t*>(vn + T::kE * r)
                                         : vbase + T::bytes((head_base + 4 * c + e) * D + T::kE * r);
    load_words<T::kVWords>(vp, br.v[e]);
  }
}

template <int D, int kFmt>
// (int4: at least three waves per SIMD, see kBalancedMaxWavesInt4)
__global__ __launch_bounds__(64 * kBalancedMaxWaves, kFmt == kFmtInt4 ? 3 : 1) void decode_mfma_balanced_kernel(
    DecodeArgs a) {
  constexpr int kE = Tile<D, kFmt>::kE;
  extern __shared__ int s_dyn[];                 // start[B + 1], ctx[B], then per wave kStageRows x D floats
  __shared__ int s_wave_tot[kBalancedMaxWaves];
  int* s_start = s_dyn;
  int* s_ctx = s_dyn + a.num_seqs + 1;

  const int x = blockIdx.x, y = blockIdx.y;
  // (the wave index in a scalar register: the KV head and every address
  // derived from it are then wave-uniform to the compiler too)
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int r = lane & 15, c = lane >> 4;
  const int W = a.waves_per_wg;
  const int B = a.num_seqs;
  const int G = a.num_q_heads / a.num_kv_heads;

  // ---- unit prefix over the sequences (every workgroup computes it)
  int carry = 0;
  for (int base = 0; base < B; base += W * 64) {
    const int b = base + tid;
    int nb = 0;
    if (b < B) {
      const int ctx = clamp_context(a, b);
      s_ctx[b] = ctx;
      nb = (ctx + kBlockTokens - 1) / kBlockTokens;
    }
    int v = nb;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int t = __shfl_up(v, off, 64);
      if (lane >= off) v += t;
    }
    if (lane == 63) s_wave_tot[wave] = v;
    __syncthreads();
    int before = 0, total = 0;
    for (int w = 0; w < W; ++w) {
      const int t = s_wave_tot[w];
      before += (w < wave) ? t : 0;
      total += t;
    }
    if (b < B) s_start[b] = carry + before + v - nb;
    carry += total;
    __syncthreads();
  }
  if (tid == 0) s_start[B] = carry;
  __syncthreads();
  const int U = carry;
  const int ns = num_slices(U, a.num_wgs);               // workgroups x >= ns have no slice
  const int u0 = x < ns ? slice_begin(x, U, ns) : U, u1 = x < ns ? slice_begin(x + 1, U, ns) : U;
  if (x == 0 && y == 0)
    for (int b = tid; b <= B; b += W * 64) a.ws_seq_start[b] = s_start[b];

  const int g = y * W + wave;
  if (g >= a.num_kv_heads) return;
  uint16_t* out = reinterpret_cast<uint16_t*>(a.out);
  // empty sequences own no unit: workgroup 0 writes their zero rows (64
  // lengths per look, then the wave writes the rows of each empty one)
  if (x == 0) {
    for (int b0 = 0; b0 < B; b0 += 64) {
      unsigned long long empty = __ballot(b0 + lane < B && s_ctx[b0 + lane] == 0);
      while (empty) {
        const int b = b0 + __builtin_ctzll(empty);
        empty &= empty - 1;
        for (int i = lane; i < G * D; i += 64) out[((int64_t)b * a.num_q_heads + (int64_t)g * G) * D + i] = 0;
      }
    }
  }
  if (u0 >= u1) return;

  const uint16_t* q = reinterpret_cast<const uint16_t*>(a.q);
  const uint8_t* kbase = reinterpret_cast<const uint8_t*>(a.k_cache);
  const uint8_t* vbase = reinterpret_cast<const uint8_t*>(a.v_cache);
  const int d0 = (D / 4) * c;

  HeadState<D, kFmt> hs;
  int cur_b = -1;
  // The G rows a wave finishes are consecutive in `out` and in the
  // workspace, but each lane holds a 16-byte-strided run of one row; stores
  // straight from those registers would split every cache line over many
  // requests.  The rows go through this wave's LDS outbox instead and leave
  // as whole 16-byte pieces, consecutive lanes writing consecutive pieces.
  // They leave after the loop (or when the outbox is full), not when the
  // sequence ends: a store is counted with the loads in vmcnt, so a store
  // issued inside the loop would make the next unit's wait also wait for
  // the store to complete.  Entry: 4 header words (row index or byte
  // offset, low and high word; kind 1 = final bf16 rows, 0 = partial rows,
  // 2 = the newest token's bf16 K and V rows for the cache), then G rows of
  // D bf16 (final, normalised), or m[G], l[G] (padded to 4 words) and G rows
  // of D floats (partial), or the K row and the V row (D bf16 each).
  uint32_t* box = reinterpret_cast<uint32_t*>(s_dyn + balanced_stage_offset_words(a.num_seqs)) + wave * a.out_words;
  // (int4 stores its rows when each sequence ends: its loop is bound by
  // vector work, not by the loads a store would delay, and the outbox
  // writes cost it 1-4%)
  constexpr bool kDeferRows = kFmt != kFmtInt4;
  const int ml_words = (2 * G + 3) & ~3;
  int box_used = 0, box_n = 0;   // words and entries in the outbox (wave-uniform)
  auto flush = [&]() __attribute__((always_inline)) {
    if (box_n == 0) return;
    wave_lds_sync();                         // every lane's entry writes are visible
    const int ll = fresh(lane);
    int off = 0;
    for (int k = 0; k < box_n; ++k) {
      const uint32_t* e = box + off;
      const uint32_t lo = __builtin_amdgcn_readfirstlane(e[0]), hi = __builtin_amdgcn_readfirstlane(e[1]);
      const uint32_t kind = __builtin_amdgcn_readfirstlane(e[2]);
      const int64_t row0 = (int64_t)(((uint64_t)hi << 32) | lo);
      if (kind == 2) {
        // the newest token's K and V rows, D bf16 each, at byte offset row0 of both caches
        const uint4* src = reinterpret_cast<const uint4*>(e + 4);
        uint8_t* base = ll < D / 8 ? reinterpret_cast<uint8_t*>(const_cast<void*>(a.k_cache))
                                   : reinterpret_cast<uint8_t*>(const_cast<void*>(a.v_cache));
        if (ll < D / 4) reinterpret_cast<uint4*>(base + row0)[ll % (D / 8)] = src[ll];
        off += 4 + D;
      } else if (kind == 1) {
        const uint4* src = reinterpret_cast<const uint4*>(e + 4);
        uint4* dst = reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(a.out) + row0 * D);
        for (int pc = ll; pc < G * D / 8; pc += 64) dst[pc] = src[pc];
        off += 4 + G * D / 2;
      } else {
        const float* ml = reinterpret_cast<const float*>(e + 4);
        if (ll < G) {
          (a.ws_m + row0)[ll] = ml[ll];
          (a.ws_l + row0)[ll] = ml[G + ll];
        }
        const float4* src = reinterpret_cast<const float4*>(e + 4 + ml_words);
        float4* dst = reinterpret_cast<float4*>(a.ws_acc + row0 * D);
        for (int pc = ll; pc < G * D / 4; pc += 64) dst[pc] = src[pc];
        off += 4 + ml_words + G * D;
      }
    }
    box_n = 0;
    box_used = 0;
    wave_lds_sync();                         // every read of the entries is done before they are rewritten
  };
  auto finish = [&](int b) __attribute__((always_inline)) {
    const float L = hs.total_l();
    float o[4 * kE];
    hs.unpack(o);
    const int64_t row0 = (int64_t)b * a.num_q_heads + (int64_t)g * G;   // rows row0 .. row0+G-1
    // (read into scalar registers: the row addresses below are then a scalar
    // base plus a lane offset, with nothing per lane to keep across the loop)
    const int sb = __builtin_amdgcn_readfirstlane(s_start[b]), se = __builtin_amdgcn_readfirstlane(s_start[b + 1]);
    const bool whole = sb >= u0 && se <= u1;
    const int slot = sb < u0 ? 0 : 1;
    const int64_t wr0 = ((int64_t)x * 2 + slot) * a.num_q_heads + (int64_t)g * G;
    const int words = whole ? 4 + G * D / 2 : 4 + ml_words + G * D;
    if (kDeferRows && words <= a.out_words) {
      if (box_used + words > a.out_words) flush();
      uint32_t* e = box + box_used;
      const int64_t ri = whole ? row0 : wr0;
      if (lane == 0) *reinterpret_cast<uint4*>(e) = make_uint4((uint32_t)ri, (uint32_t)((uint64_t)ri >> 32), whole ? 1u : 0u, 0u);
      if (whole) {
        if (r < G) store_bf16_run<D>(reinterpret_cast<uint16_t*>(e + 4) + r * D, d0, o, 1.0f / L);
      } else {
        float* ml = reinterpret_cast<float*>(e + 4);
        if (c == 0 && r < G) {
          ml[r] = hs.m;
          ml[G + r] = L;
        }
        if (r < G) store_f32_run<D>(reinterpret_cast<float*>(e + 4 + ml_words) + r * D, d0, o);
      }
      box_used += words;
      ++box_n;
      return;
    }
    // rows stored now (not deferred, or too large for the outbox: a group
    // of many query heads), kStageRows rows per pass through the outbox's space
    if constexpr (kDeferRows) flush();
    float* stage = reinterpret_cast<float*>(box);
    // (lane offsets taken fresh here, so the compiler keeps no per-lane
    // address pairs alive across the loop for these rare stores)
    const int lr = fresh(r), ll = fresh(lane);
    if (!whole && c == 0 && r < G) {
      (a.ws_m + wr0)[lr] = hs.m;
      (a.ws_l + wr0)[lr] = L;
    }
    for (int rr = 0; rr < G; rr += kStageRows) {
      const int nr = min(kStageRows, G - rr);
      const bool mine = r >= rr && r < rr + nr;
      wave_lds_sync();                       // the previous pass's reads are done
      if (whole) {
        if (mine) store_bf16_run<D>(reinterpret_cast<uint16_t*>(stage) + (r - rr) * D, d0, o, 1.0f / L);
        wave_lds_sync();
        const uint4* src = reinterpret_cast<const uint4*>(stage);
        uint4* dst = reinterpret_cast<uint4*>(out + (row0 + rr) * D);
        for (int pc = ll; pc < nr * D / 8; pc += 64) dst[pc] = src[pc];
      } else {
        if (mine) store_f32_run<D>(stage + (r - rr) * D, d0, o);
        wave_lds_sync();
        const float4* src = reinterpret_cast<const float4*>(stage);
        float4* dst = reinterpret_cast<float4*>(a.ws_acc + (wr0 + rr) * D);
        for (int pc = ll; pc < nr * D / 4; pc += 64) dst[pc] = src[pc];
      }
    }
    if constexpr (kDeferRows) wave_lds_sync();   // the last pass's reads are done before the outbox is reused
  };

  // Table entries of the current 64-unit chunk.
  int base = u0;
  UnitIds cur = unit_ids<(kFmt != kFmtBf16)>(a, s_start, base, u1, g, lane);

  // Vector memory operations complete in issue order and are waited for by
  // a count the compiler fixes per program point, taking the path with the
  // fewest operations issued after the awaited one.  So everything a unit
  // needs is loaded in fetch() (a load issued at consume time, after the
  // other unit's block, would make this wait for that block), and fetch()
  // issues the same loads on every path: for bf16 the query rows of the
  // unit's sequence come with every unit (cache hits after its first), not
  // only with the unit that starts the sequence.  The e4m3/int4 paths take
  // their query (and new-token runs) once per sequence instead.
  constexpr bool kScaled = kFmt != kFmtBf16;
  Staging<D> st;
  int fetched_b = -1;
  auto q_row = [&](int b) { return (int64_t)b * a.num_q_heads + (int64_t)g * G; };
  auto new_k = [&](int b) { return reinterpret_cast<const uint16_t*>(a.k_new) + ((int64_t)b * a.num_kv_heads + g) * D; };
  auto new_v = [&](int b) { return reinterpret_cast<const uint16_t*>(a.v_new) + ((int64_t)b * a.num_kv_heads + g) * D; };
  // e4m3/int4: the newest token's runs as the splice quantizes them (lane
  // r == off: K elements d0 .. d0+D/4-1; lane group off/4: V elements (D/16)*r ..)
  auto load_new_runs = [&](int b, uint32_t* nk, uint32_t* nv) {
    load_words<D / 8>(reinterpret_cast<const uint8_t*>(new_k(b) + d0), nk);
    load_words<D / 32>(reinterpret_cast<const uint8_t*>(new_v(b) + (D / 16) * r), nv);
  };
  auto fetch = [&](Pending<D, kFmt>& p, int u) {
    p.live = u < u1;
    u = min(u, u1 - 1);
    if (u - base >= 64) {
      base += 64;
      cur = unit_ids<(kFmt != kFmtBf16)>(a, s_start, base, u1, g, lane);
    }
    const int j = u - base;
    p.b = __builtin_amdgcn_readlane(cur.b, j);
    p.i = __builtin_amdgcn_readlane(cur.i, j);
    p.blk = __builtin_amdgcn_readlane(cur.blk, j);
    p.ctx = s_ctx[p.b];
    p.starts = p.b != fetched_b;
    fetched_b = p.b;
    if constexpr (Pending<D, kFmt>::kQueryInFetch) load_query<D>(q, q_row(p.b), G, r, c, p.q);
    // appending: the sequence's last block holds its newest token
    p.off = p.live && a.append && (p.i + 1) * kBlockTokens >= p.ctx ? (p.ctx - 1) % kBlockTokens : -1;
    p.row_staged = false;
    if constexpr (kScaled) {
      if (p.off >= 0 && !st.row_busy) {
        st.row_busy = p.row_staged = true;
        load_new_runs(p.b, st.nk, st.nv);
      }
      // the block's loads go out before the wait for its scales (which
      // were loaded after the table entries, one round trip later)
      load_block<D, kFmt>(p.regs, kbase, vbase, p.blk, a.num_kv_heads, g, r, c);
      p.ks = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(cur.ks), j));
      p.vs = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(cur.vs), j));
    } else {
      p.ks = p.vs = 1.0f;
      load_block_with_row<D>(p.regs, kbase, vbase, p.blk, a.num_kv_heads, g, r, c, p.off, new_k(p.b), new_v(p.b));
    }
  };
  // Appending: the newest token's K/V row goes into its slot in the cache
  // (the wave that reads a block is the only reader of that slot in this
  // launch) and, for e4m3/int4, into the block this wave holds.
  auto splice = [&](Pending<D, kFmt>& p, const uint32_t* nk, const uint32_t* nv) {
    using T = Tile<D, kFmt>;
    const int64_t head_base = (p.blk * a.num_kv_heads + g) * kBlockTokens;
    uint8_t* kw = const_cast<uint8_t*>(kbase);
    uint8_t* vw = const_cast<uint8_t*>(vbase);
    if constexpr (!kScaled) {
      // the registers already hold the new row (load_block_with_row); it
      // goes to the cache with the finished rows after the loop
      if constexpr (kDeferRows) {
        constexpr int words = 4 + D;
        if (words <= a.out_words) {
          if (box_used + words > a.out_words) flush();
          uint32_t* e = box + box_used;
          const int64_t rb = T::bytes((head_base + p.off) * D);   // the row's byte offset, the same in both caches
          if (lane == 0) *reinterpret_cast<uint4*>(e) = make_uint4((uint32_t)rb, (uint32_t)((uint64_t)rb >> 32), 2u, 0u);
          if (r == p.off) {
#pragma unroll
            for (int w = 0; w < T::kKWords; ++w) e[4 + c * T::kKWords + w] = p.regs.k[w];
          }
#pragma unroll
          for (int ee = 0; ee < 4; ++ee)
            if (4 * c + ee == p.off) {
#pragma unroll
              for (int w = 0; w < T::kVWords; ++w) e[4 + D / 2 + r * T::kVWords + w] = p.regs.v[ee][w];
            }
          box_used += words;
          ++box_n;
          return;
        }
      }
      if (r == p.off) store_words<T::kKWords>(kw + T::bytes((head_base + r) * D + d0), p.regs.k);
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (4 * c + e == p.off) store_words<T::kVWords>(vw + T::bytes((head_base + p.off) * D + T::kE * r), p.regs.v[e]);
    } else {
      if (r == p.off) {
        uint32_t words[T::kKWords];
        if constexpr (kFmt == kFmtFp8) quantize_bf16_words<D / 4>(nk, p.ks, words);
        else quantize_bf16_words_int4<D / 4>(nk, p.ks, words);
#pragma unroll
        for (int w = 0; w < T::kKWords; ++w) p.regs.k[w] = words[w];
        store_words<T::kKWords>(kw + T::bytes((head_base + r) * D + d0), words);
      }
      uint32_t words[T::kVWords];
      if constexpr (kFmt == kFmtFp8) quantize_bf16_words<D / 16>(nv, p.vs, words);
      else quantize_bf16_words_int4<D / 16>(nv, p.vs, words);
      // token 4c + ee of this lane's V rows is the new one (by selection: no register indexing)
#pragma unroll
      for (int ee = 0; ee < 4; ++ee) {
        const bool hit = 4 * c + ee == p.off;
#pragma unroll
        for (int w = 0; w < T::kVWords; ++w) p.regs.v[ee][w] = hit ? words[w] : p.regs.v[ee][w];
      }
      if (c == p.off / 4) store_words<T::kVWords>(vw + T::bytes((head_base + p.off) * D + T::kE * r), words);
    }
  };
  auto consume = [&](Pending<D, kFmt>& p) {
    if (p.starts) {
      if (cur_b >= 0) finish(cur_b);
      cur_b = p.b;
      if constexpr (Pending<D, kFmt>::kQueryInFetch) {
        hs.begin_loaded(p.q, G, r);
      } else {
        // load the query now and wait here: this drains the other unit's
        // block too, once per sequence start
        uint4 qw[D / 32];
        load_query<D>(q, q_row(p.b), G, r, c, qw);
#pragma unroll
        for (int i = 0; i < D / 32; ++i) {
          uint32_t x = qw[i].x, y = qw[i].y, z = qw[i].z, w = qw[i].w;
          asm volatile("" : "+v"(x), "+v"(y), "+v"(z), "+v"(w));
          qw[i] = make_uint4(x, y, z, w);
        }
        hs.begin_loaded(qw, G, r);
      }
    }
    if (p.off >= 0) {
      if (!kScaled || p.row_staged) {
        splice(p, st.nk, st.nv);
        st.row_busy = false;
      } else {
        uint32_t nk[D / 8], nv[D / 32];
        load_new_runs(p.b, nk, nv);
#pragma unroll
        for (int w = 0; w < D / 8; ++w) asm volatile("" : "+v"(nk[w]));
#pragma unroll
        for (int w = 0; w < D / 32; ++w) asm volatile("" : "+v"(nv[w]));
        splice(p, nk, nv);
      }
    }
    // a dead unit repeats one of the sequence's units with no token valid:
    // the running max, sum and accumulator stay as they are
    const int valid = p.live ? min(kBlockTokens, p.ctx - p.i * kBlockTokens) : 0;
    hs.step(p.regs, valid, a.scale_log2 * p.ks, p.vs, c);
  };

  // Two units in flight.  The loop body is straight-line (one exit, at the
  // top; past the slice's end fetch() takes a dead copy of the last unit,
  // whose lines are cached and whose consume changes nothing), so on every
  // path the wait before a consume leaves the other unit's loads in flight.
  Pending<D, kFmt> p0, p1;
  fetch(p0, u0);
  for (int u = u0; u < u1; u += 2) {
    fetch(p1, u + 1);
    consume(p0);
    fetch(p0, u + 2);
    consume(p1);
  }
  finish(cur_b);
  if constexpr (kDeferRows) flush();
}

// Merge for the balanced split.  Sequence b's units are covered by slices
// w_first..w_last; its partial sits in slot 1 of w_first (it began inside
// that slice) and in slot 0 of every later one.
//   out = sum_w 2^(m_w - M) acc_w / sum_w 2^(m_w - M) l_w,  M = max_w m_w,
// taken in one pass with a running maximum, eight partials per round so
// their loads are in flight together.  Grid (sequence, chunk group): each thread
// owns one 4-wide chunk of one query head's output row.
constexpr int kMergeThreads = 256;

template <int D>
__global__ __launch_bounds__(kMergeThreads) void decode_merge_balanced_kernel(DecodeArgs a) {
  constexpr int kChunks = D / 4;                       // float4 chunks per output row
  const int b = blockIdx.x;
  const int it = blockIdx.y * kMergeThreads + threadIdx.x;
  if (it >= a.num_q_heads * kChunks) return;
  const int U = a.ws_seq_start[a.num_seqs];
  const int s = a.ws_seq_start[b], e = a.ws_seq_start[b + 1];
  if (s == e) return;                                  // empty: zero row written by the decode kernel
  const int ns = num_slices(U, a.num_wgs);
  const int wf = slice_of(s, U, ns), wl = slice_of(e - 1, U, ns);
  if (wf == wl) return;                                // written whole by its slice
  const int n = wl - wf + 1;
  const int h = it / kChunks, ch = it % kChunks;
  float M = -INFINITY, den = 0.0f;
  float4 num = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  constexpr int kBatch = 8;                            // partial rows whose loads are in flight together
  for (int w0 = 0; w0 < n; w0 += kBatch) {
    float mv[kBatch], lv[kBatch];
    float4 av[kBatch];
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      const int w = wf + w0 + k;
      if (w0 + k < n) {
        const int64_t row = ((int64_t)w * 2 + (w == wf ? 1 : 0)) * a.num_q_heads + h;
        mv[k] = a.ws_m[row];
        lv[k] = a.ws_l[row];
        av[k] = reinterpret_cast<const float4*>(a.ws_acc + row * D)[ch];
      } else {
        mv[k] = -INFINITY;
        lv[k] = 0.0f;
        av[k] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
      }
    }
    float Mn = M;
#pragma unroll
    for (int k = 0; k < kBatch; ++k) Mn = fmaxf(Mn, mv[k]);
    const float sc = __builtin_amdgcn_exp2f(M - Mn);          // 0 while M is still -inf
    den *= sc;
    num.x *= sc; num.y *= sc; num.z *= sc; num.w *= sc;
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      const float wt = __builtin_amdgcn_exp2f(mv[k] - Mn);    // 0 for the padding entries
      den += wt * lv[k];
      num.x += wt * av[k].x; num.y += wt * av[k].y; num.z += wt * av[k].z; num.w += wt * av[k].w;
    }
    M = Mn;
  }
  const float inv = 1.0f / den;
  const uint2 packed = make_uint2(f32_to_bf16_bits_rne(num.x * inv) | (f32_to_bf16_bits_rne(num.y * inv) << 16),
                                  f32_to_bf16_bits_rne(num.z * inv) | (f32_to_bf16_bits_rne(num.w * inv) << 16));
  *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(a.out) + ((int64_t)b * a.num_q_heads + h) * D + 4 * ch) =
      packed;
}

}  // namespace

namespace {

int kv_format(pa_dtype cache_dtype) {
  return cache_dtype == PA_DTYPE_FP8_E4M3 ? kFmtFp8 : (cache_dtype == PA_DTYPE_INT4 ? kFmtInt4 : kFmtBf16);
}

}  // namespace

hipError_t launch_decode_mfma(const DecodeArgs& a, hipStream_t stream) {
  const dim3 grid(a.num_recs, a.num_kv_heads, a.num_seqs);   // a record per group of kPartWaves partitions
  const int f = kv_format(a.cache_dtype);
#define PA_LAUNCH(D_, F_) hipLaunchKernelGGL((decode_mfma_kernel<D_, F_>), grid, dim3(kPartThreads), 0, stream, a)
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

hipError_t launch_decode_mfma_balanced(const DecodeArgs& a, hipStream_t stream) {
  const dim3 grid(a.num_wgs, a.head_groups);
  const dim3 block(64 * a.waves_per_wg);
  const size_t lds = ((size_t)balanced_stage_offset_words(a.num_seqs) + (size_t)a.waves_per_wg * a.out_words) *
                    sizeof(int);
  const int f = kv_format(a.cache_dtype);
#define PA_LAUNCH(D_, F_) hipLaunchKernelGGL((decode_mfma_balanced_kernel<D_, F_>), grid, block, lds, stream, a)
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

hipError_t launch_decode_merge_balanced(const DecodeArgs& a, hipStream_t stream) {
  const dim3 grid(a.num_seqs, (a.num_q_heads * (a.head_dim / 4) + kMergeThreads - 1) / kMergeThreads);
  if (a.head_dim == 128)
    hipLaunchKernelGGL((decode_merge_balanced_kernel<128>), grid, dim3(kMergeThreads), 0, stream, a);
  else
    hipLaunchKernelGGL((decode_merge_balanced_kernel<64>), grid, dim3(kMergeThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace pa
