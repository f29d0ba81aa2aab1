// Paged decode on the matrix cores (gfx950 MFMA), bf16 query with a bf16 or
// e4m3 KV cache.
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
// Partition grid: one workgroup of 4 waves per (partition, KV head, sequence);
// wave w takes the partition's blocks w, w+4, ... and the waves merge in LDS.

template <int D, int kFmt>
__global__ __launch_bounds__(kPartThreads) void decode_mfma_kernel(DecodeArgs a) {
  using T = Tile<D, kFmt>;
  constexpr int kE = T::kE;
  __shared__ float lds_m[kPartWaves][16];
  __shared__ float lds_l[kPartWaves][16];
  __shared__ f32x4_t lds_acc[kPartWaves][kE][64];

  const int part = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r = lane & 15, c = lane >> 4;
  const int G = a.num_q_heads / a.num_kv_heads;
  const int P = a.partition_tokens;

  const int ctx = clamp_context(a, b);
  const int nparts = (ctx + P - 1) / P;
  const int64_t head0 = (int64_t)b * a.num_q_heads + (int64_t)g * G;
  uint16_t* out = reinterpret_cast<uint16_t*>(a.out);
  if (ctx == 0) {
    if (part == 0)
      for (int i = threadIdx.x; i < G * D; i += kPartThreads) out[head0 * D + i] = 0;
    return;
  }
  const int t0 = part * P;
  if (t0 >= ctx) return;
  const int n = min(P, ctx - t0);
  const int nblk = (n + kBlockTokens - 1) / kBlockTokens;
  const int nw = wave < nblk ? (nblk - wave + kPartWaves - 1) / kPartWaves : 0;   // blocks of this wave

  HeadState<D, kFmt> hs;
  hs.begin(reinterpret_cast<const uint16_t*>(a.q), head0, G, r, c);
  // physical ids (and fp8 scales) of this wave's blocks: lane j holds block j
  int my_blk = 0;
  float my_ks = 1.0f, my_vs = 1.0f;
  if (lane < nw) {
    my_blk = clamp_block(
        a.block_tables[(int64_t)b * a.max_blocks_per_seq + t0 / kBlockTokens + wave + kPartWaves * lane],
        a.num_blocks);
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
    const int valid = min(kBlockTokens, n - (wave + kPartWaves * i) * kBlockTokens);
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

  // ---- wave totals, then the 4-wave merge through LDS
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
    wt[w] = __builtin_amdgcn_exp2f(mw[w] - M);   // waves without blocks have m = -inf -> 0
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
  if (nparts == 1) {
    store_bf16_run<D>(out + row * D, d0, o, 1.0f / L);
  } else {
    const int64_t wr = row * a.num_parts + part;
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

struct UnitIds {
  int b, i, blk;       // lane j: the (sequence, logical block, physical block) of unit base + j
  float ks, vs;        // fp8 block scales of that unit for this wave's head
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

template <bool kScaled>
__device__ __forceinline__ UnitIds unit_ids(const DecodeArgs& a, const int* start, int base, int u1, int g,
                                            int lane) {
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
  return id;
}

template <int D, int kFmt>
struct Pending {
  BlockRegs<D, kFmt> regs;
  int64_t blk;
  int b, i;
  float ks, vs;
  int off;                  // appending: slot of the sequence's newest token in this block, else -1
  uint32_t nk[D / 8];       // its K run (lane r == off) as bf16 pairs
  uint32_t nv[D / 32];      // its V run (lane group c == off / 4) as bf16 pairs
};

template <int D, int kFmt>
__global__ __launch_bounds__(64 * kBalancedMaxWaves) void decode_mfma_balanced_kernel(DecodeArgs a) {
  constexpr int kE = Tile<D, kFmt>::kE;
  extern __shared__ int s_dyn[];                 // start[B + 1], then ctx[B]
  __shared__ int s_wave_tot[kBalancedMaxWaves];
  int* s_start = s_dyn;
  int* s_ctx = s_dyn + a.num_seqs + 1;

  const int x = blockIdx.x, y = blockIdx.y;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
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
  // empty sequences own no unit: workgroup 0 writes their zero rows
  if (x == 0) {
    for (int b = 0; b < B; ++b)
      if (s_ctx[b] == 0)
        for (int i = lane; i < G * D; i += 64) out[((int64_t)b * a.num_q_heads + (int64_t)g * G) * D + i] = 0;
  }
  if (u0 >= u1) return;

  const uint16_t* q = reinterpret_cast<const uint16_t*>(a.q);
  const uint8_t* kbase = reinterpret_cast<const uint8_t*>(a.k_cache);
  const uint8_t* vbase = reinterpret_cast<const uint8_t*>(a.v_cache);
  const int d0 = (D / 4) * c;

  HeadState<D, kFmt> hs;
  int cur_b = -1;
  auto finish = [&](int b) {
    const float L = hs.total_l();
    float o[4 * kE];
    hs.unpack(o);
    if (r >= G) return;
    const int64_t row = (int64_t)b * a.num_q_heads + (int64_t)g * G + r;
    const bool whole = s_start[b] >= u0 && s_start[b + 1] <= u1;
    if (whole) {
      store_bf16_run<D>(out + row * D, d0, o, 1.0f / L);
    } else {
      const int slot = s_start[b] < u0 ? 0 : 1;
      const int64_t wr = ((int64_t)x * 2 + slot) * a.num_q_heads + (int64_t)g * G + r;
      store_f32_run<D>(a.ws_acc + wr * D, d0, o);
      if (c == 0) {
        a.ws_m[wr] = hs.m;
        a.ws_l[wr] = L;
      }
    }
  };

  // ids of the current 64-unit chunk and of the next one (kept one chunk ahead)
  int base = u0;
  UnitIds cur = unit_ids<(kFmt != kFmtBf16)>(a, s_start, base, u1, g, lane);
  UnitIds nxt = unit_ids<(kFmt != kFmtBf16)>(a, s_start, base + 64, u1, g, lane);
  auto fetch = [&](Pending<D, kFmt>& p, int u) {
    if (u - base >= 64) {
      base += 64;
      cur = nxt;
      nxt = unit_ids<(kFmt != kFmtBf16)>(a, s_start, base + 64, u1, g, lane);
    }
    const int j = u - base;
    p.b = __builtin_amdgcn_readlane(cur.b, j);
    p.i = __builtin_amdgcn_readlane(cur.i, j);
    p.blk = __builtin_amdgcn_readlane(cur.blk, j);
    if constexpr (kFmt != kFmtBf16) {
      p.ks = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(cur.ks), j));
      p.vs = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(cur.vs), j));
    } else {
      p.ks = p.vs = 1.0f;
    }
    p.off = -1;
    if (a.append) {
      const int ctx = s_ctx[p.b];
      if ((p.i + 1) * kBlockTokens >= ctx) {          // the sequence's last block holds its newest token
        p.off = (ctx - 1) % kBlockTokens;
        // every lane loads its runs of the new row; only lane r == off (K) and
        // lane group off/4 (V) use them
        const int64_t row = ((int64_t)p.b * a.num_kv_heads + g) * D;
        load_words<D / 8>(reinterpret_cast<const uint8_t*>(reinterpret_cast<const uint16_t*>(a.k_new) + row + d0),
                          p.nk);
        load_words<D / 32>(reinterpret_cast<const uint8_t*>(reinterpret_cast<const uint16_t*>(a.v_new) + row +
                                                            (D / 16) * r),
                           p.nv);
      }
    }
    load_block<D, kFmt>(p.regs, kbase, vbase, p.blk, a.num_kv_heads, g, r, c);
  };
  // Appending: put the newest token's K/V row into the block this wave holds
  // and into its slot in the cache (the wave that reads a block is the only
  // reader of that slot in this launch).
  auto splice = [&](Pending<D, kFmt>& p) {
    using T = Tile<D, kFmt>;
    const int64_t head_base = (p.blk * a.num_kv_heads + g) * kBlockTokens;
    uint8_t* kw = const_cast<uint8_t*>(kbase);
    uint8_t* vw = const_cast<uint8_t*>(vbase);
    if (r == p.off) {
      uint32_t words[T::kKWords];
      if constexpr (kFmt == kFmtFp8) quantize_bf16_words<D / 4>(p.nk, p.ks, words);
      else if constexpr (kFmt == kFmtInt4) quantize_bf16_words_int4<D / 4>(p.nk, p.ks, words);
      else
#pragma unroll
        for (int w = 0; w < T::kKWords; ++w) words[w] = p.nk[w];
#pragma unroll
      for (int w = 0; w < T::kKWords; ++w) p.regs.k[w] = words[w];
      store_words<T::kKWords>(kw + T::bytes((head_base + r) * D + d0), words);
    }
    uint32_t words[T::kVWords];
    if constexpr (kFmt == kFmtFp8) quantize_bf16_words<D / 16>(p.nv, p.vs, words);
    else if constexpr (kFmt == kFmtInt4) quantize_bf16_words_int4<D / 16>(p.nv, p.vs, words);
    else
#pragma unroll
      for (int w = 0; w < T::kVWords; ++w) words[w] = p.nv[w];
    // token 4c + ee of this lane's V rows is the new one (by selection: no register indexing)
#pragma unroll
    for (int ee = 0; ee < 4; ++ee) {
      const bool hit = 4 * c + ee == p.off;
#pragma unroll
      for (int w = 0; w < T::kVWords; ++w) p.regs.v[ee][w] = hit ? words[w] : p.regs.v[ee][w];
    }
    if (c == p.off / 4) store_words<T::kVWords>(vw + T::bytes((head_base + p.off) * D + T::kE * r), words);
  };
  auto consume = [&](Pending<D, kFmt>& p) {
    if (p.b != cur_b) {
      if (cur_b >= 0) finish(cur_b);
      cur_b = p.b;
      hs.begin(q, (int64_t)p.b * a.num_q_heads + (int64_t)g * G, G, r, c);
    }
    if (p.off >= 0) splice(p);
    const int valid = min(kBlockTokens, s_ctx[p.b] - p.i * kBlockTokens);
    hs.step(p.regs, valid, a.scale_log2 * p.ks, p.vs, c);
  };

  Pending<D, kFmt> p0, p1;
  fetch(p0, u0);
  for (int u = u0; u < u1; u += 2) {
    if (u + 1 < u1) fetch(p1, u + 1);
    consume(p0);
    if (u + 1 < u1) {
      if (u + 2 < u1) fetch(p0, u + 2);
      consume(p1);
    }
  }
  finish(cur_b);
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
  const dim3 grid(a.num_parts, a.num_kv_heads, a.num_seqs);
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
  const size_t lds = (2 * (size_t)a.num_seqs + 1) * sizeof(int);
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
