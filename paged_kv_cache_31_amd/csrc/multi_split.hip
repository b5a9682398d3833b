// Causal multi-query attention over the paged cache with a balanced split of the keys, for
// gfx950: the speculative-verification shape (a few new tokens per sequence) whose query rows
// per (sequence, KV head) fill one to four MFMA tiles.
//
// What is computed is pa_decode_multi's attention (row i of sequence b, at logical position
// p = L_b - T_b + i, attends to tokens 0 .. p; youngju.dev guide, speculative-decoding figure;
// magi page, "投機的デコードとの相互作用").  The work is laid out like the single-query decode's
// balanced split-KV:
//  * The (sequence, KV head, logical block) space of the sequences with rows is flattened and cut
//    into equal chunks, one per wave, and a launch is one workgroup of eight waves per resident
//    slot, so every CU streams the same number of bytes however ragged the batch is.
//  * A wave takes all MT row tiles (16 (token, group member) rows each) of a head at once: every
//    K/V step is loaded once, with non-temporal loads, and multiplied into each tile.  Giving the
//    tiles of a chunk to different waves instead (the second one reading the blocks from the
//    cache) was measured 30% slower: a CU then keeps half as many independent HBM streams.  Two
//    16-bit tiles at head_dim 128 fit a wave's registers with the stepper's rolling schedule;
//    only heads of three or four tiles take two waves per chunk, two tiles each.
//  * A wave walks its chunk piece by piece (a piece = the part of one sequence head inside the
//    chunk), with each query column masked at its own causal end.  A piece that is a whole
//    sequence head is normalised and written.  Cut pieces are merged by log-sum-exp in chunk
//    order inside the workgroup; a head cut at a workgroup boundary is published with
//    device-coherent stores and the last workgroup to arrive (per-boundary counter) merges it.
//  * A column that sees no key in a piece keeps max -inf and exp-sum 0, and every merge treats
//    such a part as empty; a row that sees no key at all (before the context) is zero.
#include <limits.h>

#include "device_common.hpp"
#include "pa_internal.hpp"
#include "stepper.hpp"

namespace pa {

namespace {

struct SplitMeta {
  int b, kvh, j0, j1, nblk;
  int s0;   // flattened index of the sequence head's first block
};

// One log-sum-exp step over running (m, l) and a part (pm, pl): the weights of both, with an
// all-empty pair (both maxima -inf) giving weights 0 instead of NaN.
__device__ __forceinline__ void lse_weights(float m, float pm, float& M_, float& x, float& y) {
  M_ = fmaxf(m, pm);
  const float r = M_ == -INFINITY ? 0.0f : M_;
  x = fast_exp2(m - r);
  y = fast_exp2(pm - r);
}

// Query-row geometry of one tile of a sequence head: row r = 16 * tile + col is (token i =
// r / G, member g = r % G); columns past the last row repeat it and write nothing.
struct TileRows {
  int i, g;
  int end_lane, end_lo, end_hi;   // causal ends: this column, the tile's first and last row
  bool real, any;                 // this column is a row; the tile has rows
  __device__ __forceinline__ TileRows(int tile, int col, int T, int G, int L) {
    const int rows = T * G;
    any = 16 * tile < rows;
    const int r_hi = min(16 * tile + 15, rows - 1);
    real = any && 16 * tile + col <= r_hi;
    const int r = real ? 16 * tile + col : max(r_hi, 0);
    i = r / G;
    g = r - i * G;
    auto end_of = [&](int ii) { return min(max(L - T + ii + 1, 0), L); };
    end_lane = end_of(i);
    end_lo = end_of((16 * tile) / G);
    end_hi = end_of(max(r_hi, 0) / G);
  }
};

template <int QT, int NT>
__device__ __forceinline__ void store_row(void* out, size_t row, int D, int grp, float l,
                                          const f32x4 (&acc)[NT]) {
  typedef typename Mfma<QT>::elem E;
  const float inv = l > 0.0f ? 1.0f / l : 0.0f;     // no key: a zero row
  E* o = reinterpret_cast<E*>(out) + row * D + 4 * grp;
#pragma unroll
  for (int t = 0; t < NT; ++t)
    *reinterpret_cast<uint2*>(o + 16 * t) =
        make_uint2(pack2<QT>(acc[t][0] * inv, acc[t][1] * inv),
                   pack2<QT>(acc[t][2] * inv, acc[t][3] * inv));
}

// Two waves walking one chunk (two tiles each) read the same blocks; the second finds them in
// L2 only while the first is not far ahead.  Each wave posts the flattened position of the step
// it is about to load in LDS and waits (bounded: pacing never decides a result) while its
// partner is more than kPaceLag blocks behind; a wave that is done posts INT_MAX.  A wave only
// waits for a partner behind it, which is then not waiting, so the pair always moves on.
// The pairs are two waves of two tiles each (heads of three or four row tiles).  For them
// lockstep and allowed lags of 2 and 8 blocks measured the same within noise (64 x 128-8192
// bf16 tokens with 8 drafts: 262.4-263.8 us; 4 x 32768 bf16 tokens with 8 drafts:
// 125.9-126.6 us), so the pair walks in lockstep.
constexpr int kPaceLag = 0;
constexpr int kPaceSpins = 2048;
struct PairPace {
  int* post;          // this workgroup's positions, one per wave
  int me, partner;
  int base;           // flattened position of logical block 0 of the piece's head
  __device__ __forceinline__ void operator()(int blk) const {
    const int p = base + blk;
    if ((threadIdx.x & 63) == 0)
      __hip_atomic_store(post + me, p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    for (int i = 0; i < kPaceSpins; ++i) {
      const int q = __hip_atomic_load(post + partner, __ATOMIC_RELAXED,
                                      __HIP_MEMORY_SCOPE_WORKGROUP);
      if (q >= p - kPaceLag) break;
      __builtin_amdgcn_s_sleep(1);
    }
  }
};

constexpr int kSplitMergeDirect = 16;   // parts merged with one round of loads per thread
constexpr int kSplitMergeStage = 16;    // parts staged in LDS per batch beyond that

}  // namespace

// Merges all published parts of sequence head (b, kvh) (workgroups c0..c1; c0 holds it in its
// slot 1 unless the head starts exactly at its range) and writes its rows.  Every thread of the
// workgroup calls it.
template <int D, int QT, int TT>
__device__ void merge_split_published(const MultiArgs& a, int b, int kvh, int s0, int c0, int c1,
                                      int WGB, float (&sm_mw)[kSplitMergeStage][16 * TT],
                                      float (&sm_ml)[kSplitMergeStage][16 * TT],
                                      float (&sm_hm)[16 * TT], float (&sm_hl)[16 * TT]) {
  typedef typename Mfma<QT>::elem E;
  constexpr int R = 16 * TT;
  constexpr int NTH = 64 * kWaves;
  constexpr int EPT = (R * D / 4 + NTH - 1) / NTH;
  const int tid = threadIdx.x;
  const int G = a.group, Hq = a.num_q_heads;
  const int q0 = a.query_start[b];
  const int T = min(max(a.query_start[b + 1] - q0, 0), a.max_query_len);
  const int rows = T * G;
  const int first_slot = s0 != c0 * WGB ? 1 : 0;
  const int nparts = c1 - c0 + 1;
  auto part_of = [&](int pi, int r) -> size_t {
    const int cc = c0 + pi;
    return (((size_t)cc * 2 + (pi == 0 ? first_slot : 0)) * TT + r / 16) * 16 + (r & 15);
  };
  auto out_row = [&](int r) -> long long {      // -1: no row of out
    const long long n = (long long)q0 + r / G;
    return r < rows && n >= 0 && n < a.total_queries ? n * Hq + kvh * G + r % G : -1;
  };

  if (nparts <= kSplitMergeDirect) {
#pragma unroll
    for (int x = 0; x < EPT; ++x) {
      const int e = (tid + x * NTH) * 4;
      if (e >= R * D) break;
      const int r = e / D, d = e - r * D;
      const long long orow = out_row(r);
      if (orow < 0) continue;
      f32x2 ml[kSplitMergeDirect];
      f32x4 part[kSplitMergeDirect];
#pragma unroll
      for (int k = 0; k < kSplitMergeDirect; ++k)
        if (k < nparts) {
          const size_t p = part_of(k, r);
          ml[k] = load_coherent2(a.ws_ml + p * 2);
          part[k] = load_coherent4(a.ws_acc + p * D + d);
        }
      float M_ = -INFINITY;
#pragma unroll
      for (int k = 0; k < kSplitMergeDirect; ++k)
        if (k < nparts) M_ = fmaxf(M_, ml[k][0]);
      const float Mr = M_ == -INFINITY ? 0.0f : M_;
      float Ls = 0.0f;
      f32x4 o = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int k = 0; k < kSplitMergeDirect; ++k)
        if (k < nparts) {
          const float w = fast_exp2(ml[k][0] - Mr);
          Ls += w * ml[k][1];
          o += w * part[k];
        }
      const float inv = Ls > 0.0f ? 1.0f / Ls : 0.0f;
      *reinterpret_cast<uint2*>(reinterpret_cast<E*>(a.out) + orow * D + d) =
          make_uint2(pack2<QT>(o[0] * inv, o[1] * inv), pack2<QT>(o[2] * inv, o[3] * inv));
    }
    return;
  }

  // many parts: batches whose (max, exp-sum) pairs are staged in LDS with one round of loads
  f32x4 o[EPT];
#pragma unroll
  for (int x = 0; x < EPT; ++x) o[x] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  for (int r = tid; r < R; r += NTH) {
    sm_hm[r] = -INFINITY;
    sm_hl[r] = 0.0f;
  }
  for (int pb = 0; pb < nparts; pb += kSplitMergeStage) {
    const int n = min(kSplitMergeStage, nparts - pb);
    __syncthreads();
    for (int t = tid; t < n * R; t += NTH) {
      const f32x2 ml = load_coherent2(a.ws_ml + part_of(pb + t / R, t % R) * 2);
      sm_mw[t / R][t % R] = ml[0];
      sm_ml[t / R][t % R] = ml[1];
    }
    __syncthreads();
    for (int r = tid; r < R; r += NTH) {
      float M_ = sm_hm[r];
      for (int k = 0; k < n; ++k) M_ = fmaxf(M_, sm_mw[k][r]);
      const float Mr = M_ == -INFINITY ? 0.0f : M_;
      const float sc = fast_exp2(sm_hm[r] - Mr);
      float Ls = sm_hl[r] * sc;
      for (int k = 0; k < n; ++k) {
        const float w = fast_exp2(sm_mw[k][r] - Mr);
        sm_mw[k][r] = w;
        Ls += w * sm_ml[k][r];
      }
      sm_ml[0][r] = sc;             // rescale of what is accumulated (read below)
      sm_hm[r] = M_;
      sm_hl[r] = Ls;
    }
    __syncthreads();
#pragma unroll
    for (int x = 0; x < EPT; ++x) {
      const int e = (tid + x * NTH) * 4;
      if (e >= R * D) break;
      const int r = e / D, d = e - r * D;
      f32x4 acc_b = o[x] * sm_ml[0][r];
      for (int k = 0; k < n; ++k)
        acc_b += sm_mw[k][r] * load_coherent4(a.ws_acc + part_of(pb + k, r) * D + d);
      o[x] = acc_b;
    }
  }
  __syncthreads();
#pragma unroll
  for (int x = 0; x < EPT; ++x) {
    const int e = (tid + x * NTH) * 4;
    if (e >= R * D) break;
    const int r = e / D, d = e - r * D;
    const long long orow = out_row(r);
    if (orow < 0) continue;
    const float inv = sm_hl[r] > 0.0f ? 1.0f / sm_hl[r] : 0.0f;
    *reinterpret_cast<uint2*>(reinterpret_cast<E*>(a.out) + orow * D + d) =
        make_uint2(pack2<QT>(o[x][0] * inv, o[x][1] * inv),
                   pack2<QT>(o[x][2] * inv, o[x][3] * inv));
  }
}

template <int D, int QT, int KVT, int MT, int RT>
__global__ __launch_bounds__(64 * kWaves, 8 / kWaves) void multi_split_kernel(MultiArgs a) {
  // RT waves share a chunk (one of them loads a block from HBM, the others find it in the
  // cache, so only then are the loads cached), each holding MT of the head's TT row tiles
  typedef Stepper<D, QT, KVT, RT == 1, true> St;
  typedef typename St::V8 V8;
  typedef typename St::E E;
  constexpr int NC = St::NC;
  constexpr int NT = St::NT;
  constexpr int NTH = 64 * kWaves;
  constexpr int KW = kWaves / RT;                   // chunks per workgroup
  constexpr int TT = MT * RT;                       // row tiles per head
  static_assert(RT == 1 || RT == 2, "waves per chunk");

  __shared__ int sm_wave_sum[kWaves];
  __shared__ int sm_start_b[KW], sm_start_off[KW];
  __shared__ SplitMeta sm_meta[kWaves][2];          // [wave][first cut piece / last cut piece]
  __shared__ float sm_pm[kWaves][MT][16], sm_pl[kWaves][MT][16];
  __shared__ f32x4 sm_pacc[kWaves][MT][NT][64];     // one piece per wave
  __shared__ int sm_last[2];
  __shared__ int sm_post[kWaves];                   // pacing of the waves sharing a chunk
  __shared__ float sm_mw[kSplitMergeStage][16 * TT], sm_ml[kSplitMergeStage][16 * TT];
  __shared__ float sm_hm[16 * TT], sm_hl[16 * TT];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = uniform(tid >> 6);
  const int col = lane & 15, grp = lane >> 4;
  const int B = a.batch, Hkv = a.num_kv_heads, Hq = a.num_q_heads, G = a.group;
  const int cap = a.len_cap, Tcap = a.max_query_len;
  auto len_of = [&](int b) { return clamp_len(a.context_lens[b], cap); };
  auto rows_of = [&](int b) { return min(max(a.query_start[b + 1] - a.query_start[b], 0), Tcap); };

  // ---- 1. Flattened block space of the sequences with rows, and this workgroup's chunk
  // starts.  Sequence b contributes Hkv * blocks(L_b) when it has rows.
  const int per = (B + NTH - 1) / NTH;
  const int b_lo = tid * per;
  int tot = 0;
  for (int i = 0; i < per; ++i) {
    const int b = b_lo + i;
    if (b < B && rows_of(b) > 0) tot += Hkv * blocks_of(len_of(b));
  }
  int incl = tot;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int v = __shfl_up(incl, o);
    if (lane >= o) incl += v;
  }
  if (lane == 63) sm_wave_sum[wave] = incl;
  __syncthreads();
  int before = 0, W = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    const int v = sm_wave_sum[w];
    before += w < wave ? v : 0;
    W += v;
  }
  int Cw = (W + a.total_lanes - 1) / a.total_lanes;
  Cw = max(2, (Cw + 1) & ~1);
  const int nch = (W + Cw - 1) / Cw;
  const int c_first = blockIdx.x * KW;
  {
    int run = before + incl - tot;
    for (int i = 0; i < per; ++i) {
      const int b = b_lo + i;
      if (b >= B) break;
      const int T = rows_of(b);
      if (T == 0) continue;
      const int L = len_of(b);
      const int nb = Hkv * blocks_of(L);
#pragma unroll
      for (int w = 0; w < KW; ++w) {
        const long start = (long)(c_first + w) * Cw;
        if (start >= run && start < run + nb) {
          sm_start_b[w] = b;
          sm_start_off[w] = (int)(start - run);
        }
      }
      if (nb == 0 && blockIdx.x == 0) {           // no cached token: the rows are zeros
        const int q0 = a.query_start[b];
        for (int t = 0; t < T; ++t) {
          const long long n = (long long)q0 + t;
          if (n < 0 || n >= a.total_queries) continue;
          uint4* o = reinterpret_cast<uint4*>(reinterpret_cast<E*>(a.out) + n * Hq * D);
          for (int k = 0; k < Hq * D / 8; ++k) o[k] = make_uint4(0u, 0u, 0u, 0u);
        }
      }
      run += nb;
    }
  }
  if (tid < 2 * kWaves) sm_meta[tid >> 1][tid & 1].b = -1;
  if (tid < kWaves) sm_post[tid] = INT_MIN / 2;     // not started: wait for a partner's first post
  __syncthreads();

  // ---- 2. This wave's chunk, piece by piece, all row tiles of a head at once.  A chunk's
  // first piece, if cut and not also its last, is parked in the wave's LDS slot; its last cut
  // piece stays in registers for the merge.
  const int cl = wave / RT, rt = wave - cl * RT;    // chunk of the workgroup; tiles rt*MT + u
  const int c = c_first + cl;
  const St st(a, lane);
  const int a0 = c * Cw;
  const int a1 = min(a0 + Cw, W);
  int b = 0, L = 0, T = 0, nblk = 0, kvh = 0, j = 0;
  int pos = a0;
  bool more = false;
  if (c < nch) {
    b = uniform(sm_start_b[cl]);
    L = len_of(b);
    T = rows_of(b);
    nblk = blocks_of(L);
    const int off = uniform(sm_start_off[cl]);
    kvh = off / nblk;
    j = off - kvh * nblk;
    more = true;
  }
  float m_run[MT], l_run[MT];
  f32x4 acc[MT][NT];
  bool keep = false;                                // registers hold the last cut piece
  for (int piece = 0; more; ++piece) {
    const int j0 = j;
    const int j1 = min(nblk, j0 + (a1 - pos));
    const bool last = pos + (j1 - j0) >= a1;
    const int q0 = a.query_start[b];
    V8 qB[MT][NC];
    int end_lane[MT];
    int end_lo = INT_MAX, end_hi = 0;
#pragma unroll
    for (int u = 0; u < MT; ++u) {
      const TileRows tr(rt * MT + u, col, T, G, L);
      const long long n = (long long)q0 + tr.i;
      const bool row_ok = tr.real && n >= 0 && n < a.total_queries;
      st.load_q(qB[u], row_ok ? reinterpret_cast<const E*>(a.q) +
                                    ((size_t)n * Hq + kvh * G + tr.g) * D
                              : nullptr);
      end_lane[u] = tr.any ? tr.end_lane : 0;       // a tile without rows sees nothing
      if (tr.any) {
        end_lo = min(end_lo, tr.end_lo);
        end_hi = max(end_hi, tr.end_hi);
      }
#pragma unroll
      for (int t = 0; t < NT; ++t) acc[u][t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
      m_run[u] = -INFINITY;
      l_run[u] = 0.0f;
    }
    // Blocks past the last causal end hold no key of these rows.  The ends are also clipped
    // to the piece: a piece may stop after an odd number of blocks inside the head, and the
    // last step then repeats that block as its second half, which only the end masks.
    const int jt = min(j1, blocks_of(end_hi));
    const int tend = kBlock * jt;
#pragma unroll
    for (int u = 0; u < MT; ++u) end_lane[u] = min(end_lane[u], tend);
    if (j0 < jt) {
      const int32_t* trow = a.block_tables + (size_t)b * a.max_blocks_per_seq;
      constexpr bool ROLL = KVT != DT_FP8 && D == 128 && MT == 2;
      if constexpr (RT == 2)
        st.template walk_tiles<MT, PairPace, ROLL>(qB, trow, kvh, j0, jt, end_lane,
                                                   min(end_lo, tend), min(end_hi, tend), m_run,
                                                   l_run, acc,
                                                   PairPace{sm_post, wave, wave ^ 1, pos - j0});
      else
        st.template walk_tiles<MT, NoPace, ROLL>(qB, trow, kvh, j0, jt, end_lane,
                                                 min(end_lo, tend), min(end_hi, tend), m_run,
                                                 l_run, acc);
    }
#pragma unroll
    for (int u = 0; u < MT; ++u) l_run[u] = sum_across_rows(l_run[u]);

    if (j0 == 0 && j1 == nblk) {
#pragma unroll
      for (int u = 0; u < MT; ++u) {
        const TileRows tr(rt * MT + u, col, T, G, L);
        const long long n = (long long)q0 + tr.i;
        if (tr.real && n >= 0 && n < a.total_queries)
          store_row<QT, NT>(a.out, (size_t)n * Hq + kvh * G + tr.g, D, grp, l_run[u], acc[u]);
      }
    } else if (!last) {                             // the first piece, cut: park it
      if (lane == 0) sm_meta[wave][0] = SplitMeta{b, kvh, j0, j1, nblk, pos - j0};
#pragma unroll
      for (int u = 0; u < MT; ++u) {
        if (grp == 0) {
          sm_pm[wave][u][col] = m_run[u];
          sm_pl[wave][u][col] = l_run[u];
        }
#pragma unroll
        for (int t = 0; t < NT; ++t) sm_pacc[wave][u][t][lane] = acc[u][t];
      }
    } else {
      if (lane == 0) sm_meta[wave][1] = SplitMeta{b, kvh, j0, j1, nblk, pos - j0};
      keep = true;
    }

    pos += j1 - j0;
    if (last) break;
    // next piece: the next KV head, else the next sequence with rows and cached tokens (one
    // exists while pos < a1 <= W; the bound on b only keeps the walk inside the arrays)
    if (++kvh == Hkv) {
      kvh = 0;
      L = 0;
      T = 0;
      while ((L == 0 || T == 0) && b + 1 < B) {
        ++b;
        L = len_of(b);
        T = rows_of(b);
      }
      if (L == 0 || T == 0) break;
      nblk = blocks_of(L);
    }
    j = 0;
  }
  if constexpr (RT == 2) {                          // done: the partner never waits for this wave
    if (lane == 0) __hip_atomic_store(sm_post + wave, INT_MAX, __ATOMIC_RELAXED,
                                      __HIP_MEMORY_SCOPE_WORKGROUP);
  }
  __syncthreads();

  // ---- 3. Merge the cut pieces.  Slots are ordered by tile set (rt), then chunk, then first
  // / last: slot 2c (of tile set rt) is the first cut piece of the chunk's wave (parked in
  // LDS), slot 2c+1 its last (in its registers).  In slot order the pieces of one (sequence
  // head, tile set) are consecutive and form a group; every tile set has the same groups (its
  // waves walked the same pieces).  Only a group's last piece can be a first piece (a first
  // piece that is not also the chunk's last ends its head), so after each wave takes its
  // parked piece back into registers and parks its last piece instead, every piece of a group
  // but the last is in LDS.
  constexpr int NS = 2 * kWaves;
  static_assert(NS <= 64, "one slot per lane");
  auto wave_of = [&](int x) { return ((x % (2 * KW)) >> 1) * RT + x / (2 * KW); };
  SplitMeta mt{-1, 0, 0, 0, 0, 0};
  const int my_rt = lane < NS ? lane / (2 * KW) : -1;
  if (lane < NS) mt = sm_meta[wave_of(lane)][lane & 1];
  const bool used = lane < NS && mt.b >= 0;
  const uint64_t used_mask = __ballot(used);
  const uint64_t before_me = used_mask & ((1ull << lane) - 1ull);
  const int prev = before_me ? 63 - __clzll((long long)before_me) : lane;
  const int prev_b = __shfl(mt.b, prev), prev_kvh = __shfl(mt.kvh, prev);
  const int prev_rt = __shfl(my_rt, prev);
  const uint64_t start_mask = __ballot(
      used && (prev == lane || prev_b != mt.b || prev_kvh != mt.kvh || prev_rt != my_rt));
  const int ngroups = __popcll(start_mask);
  const int gid = __popcll(start_mask & ((2ull << lane) - 1ull)) - 1;

  struct Group {
    uint64_t slots;
    int b, kvh, j0, j1, nblk, s0, last, rt;
    bool whole;
  };
  auto group = [&](int g) {
    Group r;
    r.slots = __ballot(used && gid == g);
    const int f = __builtin_ctzll(r.slots), l = 63 - __builtin_clzll(r.slots);
    r.b = __builtin_amdgcn_readlane(mt.b, f);
    r.kvh = __builtin_amdgcn_readlane(mt.kvh, f);
    r.j0 = __builtin_amdgcn_readlane(mt.j0, f);
    r.j1 = __builtin_amdgcn_readlane(mt.j1, l);
    r.nblk = __builtin_amdgcn_readlane(mt.nblk, f);
    r.s0 = __builtin_amdgcn_readlane(mt.s0, f);
    r.last = l;
    r.rt = f / (2 * KW);
    r.whole = r.j0 == 0 && r.j1 == r.nblk;
    return r;
  };

  // swap: the parked first piece into registers, the last piece into the slot (a wave's own
  // slot only, and one wave's LDS accesses stay in order, so no barrier between the two)
  const bool has_first = sm_meta[wave][0].b >= 0;
  float fm[MT], fl[MT];
  f32x4 facc[MT][NT];
  if (has_first) {
#pragma unroll
    for (int u = 0; u < MT; ++u) {
      fm[u] = sm_pm[wave][u][col];
      fl[u] = sm_pl[wave][u][col];
#pragma unroll
      for (int t = 0; t < NT; ++t) facc[u][t] = sm_pacc[wave][u][t][lane];
    }
  }
  if (keep) {
#pragma unroll
    for (int u = 0; u < MT; ++u) {
      if (grp == 0) {
        sm_pm[wave][u][col] = m_run[u];
        sm_pl[wave][u][col] = l_run[u];
      }
#pragma unroll
      for (int t = 0; t < NT; ++t) sm_pacc[wave][u][t][lane] = acc[u][t];
    }
  }
  __syncthreads();

  const int WGB = KW * Cw;                          // blocks per workgroup range
  for (int g = 0; g < ngroups; ++g) {
    const Group gr = group(g);
    // slot 1: the head starts strictly inside this workgroup's range; slot 0: at or before
    const int wslot = gr.s0 > (int)blockIdx.x * WGB ? 1 : 0;
    if (gr.last & 1) {
      // Every piece of the group is parked: all waves merge it, each a share of the (tile,
      // 16-dim block) pairs, with weights from one pass over the pieces' maxima, so that all
      // LDS reads of a pair are issued at once.
      for (int x = wave; x < MT * NT; x += kWaves) {
        const int u = x / NT, t = x - u * NT;
        float M_ = -INFINITY;
#pragma unroll
        for (int k = 0; k < NS; ++k)
          if ((gr.slots >> k) & 1) M_ = fmaxf(M_, sm_pm[wave_of(k)][u][col]);
        const float Mr = M_ == -INFINITY ? 0.0f : M_;
        float gl = 0.0f;
        f32x4 go = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int k = 0; k < NS; ++k)
          if ((gr.slots >> k) & 1) {
            const float w = fast_exp2(sm_pm[wave_of(k)][u][col] - Mr);
            gl += w * sm_pl[wave_of(k)][u][col];
            go += w * sm_pacc[wave_of(k)][u][t][lane];
          }
        if (gr.whole) {
          const TileRows tr(gr.rt * MT + u, col, rows_of(gr.b), G, len_of(gr.b));
          const long long n = (long long)a.query_start[gr.b] + tr.i;
          if (tr.real && n >= 0 && n < a.total_queries) {
            const float inv = gl > 0.0f ? 1.0f / gl : 0.0f;
            E* o = reinterpret_cast<E*>(a.out) + ((size_t)n * Hq + gr.kvh * G + tr.g) * D +
                   16 * t + 4 * grp;
            *reinterpret_cast<uint2*>(o) = make_uint2(pack2<QT>(go[0] * inv, go[1] * inv),
                                                      pack2<QT>(go[2] * inv, go[3] * inv));
          }
        } else {
          const size_t ps = (((size_t)blockIdx.x * 2 + wslot) * TT + gr.rt * MT + u) * 16 + col;
          store_coherent(a.ws_acc + ps * D + 16 * t + 4 * grp, go);
          if (t == 0 && grp == 0) {
            store_coherent(a.ws_ml + ps * 2, M_);
            store_coherent(a.ws_ml + ps * 2 + 1, gl);
          }
        }
      }
      continue;
    }
    // The group ends with a first piece, held in the registers of the wave that walked it:
    // that wave merges the group.
    if (wave_of(gr.last) != wave) continue;
#pragma unroll
    for (int u = 0; u < MT; ++u) {
      float gm = -INFINITY, gl = 0.0f;
      f32x4 go[NT];
#pragma unroll
      for (int t = 0; t < NT; ++t) go[t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
      uint64_t rest = gr.slots;
      while (rest) {
        const int k = __builtin_ctzll(rest);
        rest &= rest - 1;
        float pm, pl;
        f32x4 pa[NT];
        if (k == gr.last) {                         // this wave's first piece, in registers
          pm = fm[u];
          pl = fl[u];
#pragma unroll
          for (int t = 0; t < NT; ++t) pa[t] = facc[u][t];
        } else {                                    // a last piece, parked
          const int wk = wave_of(k);
          pm = sm_pm[wk][u][col];
          pl = sm_pl[wk][u][col];
#pragma unroll
          for (int t = 0; t < NT; ++t) pa[t] = sm_pacc[wk][u][t][lane];
        }
        float M_, x, y;
        lse_weights(gm, pm, M_, x, y);
        gl = gl * x + pl * y;
#pragma unroll
        for (int t = 0; t < NT; ++t) go[t] = go[t] * x + pa[t] * y;
        gm = M_;
      }
      if (gr.whole) {
        const TileRows tr(gr.rt * MT + u, col, rows_of(gr.b), G, len_of(gr.b));
        const long long n = (long long)a.query_start[gr.b] + tr.i;
        if (tr.real && n >= 0 && n < a.total_queries)
          store_row<QT, NT>(a.out, (size_t)n * Hq + gr.kvh * G + tr.g, D, grp, gl, go);
      } else {
        const size_t ps = (((size_t)blockIdx.x * 2 + wslot) * TT + gr.rt * MT + u) * 16 + col;
#pragma unroll
        for (int t = 0; t < NT; ++t) store_coherent(a.ws_acc + ps * D + 16 * t + 4 * grp, go[t]);
        if (grp == 0) {
          store_coherent(a.ws_ml + ps * 2, gm);
          store_coherent(a.ws_ml + ps * 2 + 1, gl);
        }
      }
    }
  }

  // the cut heads this workgroup publishes (at most two: the first and last group of a tile
  // set; the other sets' groups are the same heads)
  const int ngt = ngroups / RT;
  int npub = 0, pb_b[2] = {0, 0}, pb_kvh[2] = {0, 0}, pb_s0[2] = {0, 0};
  int pb_c0[2] = {0, 0}, pb_c1[2] = {0, 0};
#pragma unroll
  for (int x = 0; x < 2; ++x) {
    if (x >= ngt) break;
    const Group gr = group(x == 0 ? 0 : ngt - 1);
    if (gr.whole) continue;
    const int c0 = gr.s0 / WGB, c1 = (gr.s0 + gr.nblk - 1) / WGB;
#pragma unroll
    for (int y = 0; y < 2; ++y)
      if (y == npub) {
        pb_b[y] = gr.b;
        pb_kvh[y] = gr.kvh;
        pb_s0[y] = gr.s0;
        pb_c0[y] = c0;
        pb_c1[y] = c1;
      }
    ++npub;
  }
  if (npub == 0) return;

  wait_memory_ops();
  __syncthreads();
  if (tid == 0 || (tid == 64 && npub > 1)) {
    const int x = tid == 0 ? 0 : 1;
    const int c0 = x == 0 ? pb_c0[0] : pb_c0[1], c1 = x == 0 ? pb_c1[0] : pb_c1[1];
    sm_last[x] = __hip_atomic_fetch_add(a.ws_cnt + c1, 1, __ATOMIC_RELAXED,
                                        __HIP_MEMORY_SCOPE_AGENT) == c1 - c0;
  }
  __syncthreads();
  for (int x = 0; x < npub; ++x) {
    if (!sm_last[x]) continue;
    const int c1 = x == 0 ? pb_c1[0] : pb_c1[1];
    merge_split_published<D, QT, TT>(a, x == 0 ? pb_b[0] : pb_b[1], x == 0 ? pb_kvh[0] : pb_kvh[1],
                                     x == 0 ? pb_s0[0] : pb_s0[1], x == 0 ? pb_c0[0] : pb_c0[1],
                                     c1, WGB, sm_mw, sm_ml, sm_hm, sm_hl);
    if (tid == 0)                                   // ready for the next call
      __hip_atomic_store(a.ws_cnt + c1, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// The instances: one tile per head (MT 1, RT 1); two tiles in one wave (MT 2); three or four
// tiles (three laid out as four) in two paced waves of two (MT 2, RT 2).
template <int D, int QT, int KVT>
static hipError_t launch_split_t(const MultiArgs& a, hipStream_t stream) {
  const dim3 block(64 * kWaves);
  if (a.split_rt == 1)
    hipLaunchKernelGGL((multi_split_kernel<D, QT, KVT, 1, 1>),
                       dim3((unsigned)(a.total_lanes / kWaves)), block, 0, stream, a);
  else if (a.split_rt == 2)
    hipLaunchKernelGGL((multi_split_kernel<D, QT, KVT, 2, 1>),
                       dim3((unsigned)(a.total_lanes / kWaves)), block, 0, stream, a);
  else if (a.split_rt == 4)
    hipLaunchKernelGGL((multi_split_kernel<D, QT, KVT, 2, 2>),
                       dim3((unsigned)(a.total_lanes / (kWaves / 2))), block, 0, stream, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

template <int D, int QT, int KVT>
static int split_occupancy_t(int rt) {
  int n = 0;
  hipError_t e = hipErrorInvalidValue;
  if (rt == 1)
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, multi_split_kernel<D, QT, KVT, 1, 1>,
                                                     64 * kWaves, 0);
  else if (rt == 2)
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, multi_split_kernel<D, QT, KVT, 2, 1>,
                                                     64 * kWaves, 0);
  else if (rt == 4)
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, multi_split_kernel<D, QT, KVT, 2, 2>,
                                                     64 * kWaves, 0);
  return e == hipSuccess ? n : 0;
}

template <int D>
static hipError_t launch_split_d(const MultiArgs& a, int q_dtype, int kv_dtype,
                                 hipStream_t stream) {
  if (q_dtype == DT_F16 && kv_dtype == DT_F16) return launch_split_t<D, DT_F16, DT_F16>(a, stream);
  if (q_dtype == DT_BF16 && kv_dtype == DT_BF16)
    return launch_split_t<D, DT_BF16, DT_BF16>(a, stream);
  if (q_dtype == DT_BF16 && kv_dtype == DT_FP8) return launch_split_t<D, DT_BF16, DT_FP8>(a, stream);
  if (q_dtype == DT_F16 && kv_dtype == DT_FP8) return launch_split_t<D, DT_F16, DT_FP8>(a, stream);
  return hipErrorInvalidValue;
}

template <int D>
static int split_occupancy_d(int q_dtype, int kv_dtype, int rt) {
  if (q_dtype == DT_F16 && kv_dtype == DT_F16) return split_occupancy_t<D, DT_F16, DT_F16>(rt);
  if (q_dtype == DT_BF16 && kv_dtype == DT_BF16) return split_occupancy_t<D, DT_BF16, DT_BF16>(rt);
  if (q_dtype == DT_BF16 && kv_dtype == DT_FP8) return split_occupancy_t<D, DT_BF16, DT_FP8>(rt);
  if (q_dtype == DT_F16 && kv_dtype == DT_FP8) return split_occupancy_t<D, DT_F16, DT_FP8>(rt);
  return 0;
}

int multi_split_workgroups_per_cu(int head_dim, int q_dtype, int kv_dtype, int rt) {
  return head_dim == 64 ? split_occupancy_d<64>(q_dtype, kv_dtype, rt)
                        : split_occupancy_d<128>(q_dtype, kv_dtype, rt);
}

hipError_t launch_multi_split(const MultiArgs& a, int head_dim, int q_dtype, int kv_dtype,
                              hipStream_t stream) {
  if (head_dim == 64) return launch_split_d<64>(a, q_dtype, kv_dtype, stream);
  if (head_dim == 128) return launch_split_d<128>(a, q_dtype, kv_dtype, stream);
  return hipErrorInvalidValue;
}

}  // namespace pa
