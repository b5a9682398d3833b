// Paged decode attention for gfx950: one query token per sequence attends over its KV history,
// which lives in scattered 16-token physical blocks reached through a block table.
//
// What is computed (per sequence b, query head h, KV head kvh = h / group):
//   out[b][h] = softmax(scale * q[b][h] . K^T) . V over the first L_b logical tokens, gathered
//   through block_tables[b] (kasblo.com, "PagedAttentionはKV Cacheをblockで管理する"; youngju.dev
//   guide, block-table figure), with an online (running max / running sum) softmax
//   (babushkai.com "GPU推論の内部構造", FlashAttention section) and grouped-query heads sharing one
//   KV head (Scaling Book note, "生成スループット/レイテンシ改善のテクニック").
//
// Design for CDNA4.  Decode attention streams every K/V byte once at about one flop per byte
// (Scaling Book note, "Attention のボトルネック"), so the kernel is HBM-bound and is built around
// keeping enough 16-byte loads in flight on every CU, whatever the length mix of the batch.
//
//  * Balanced split-KV.  The (sequence, KV head, logical block) space is flattened into W blocks
//    and cut into equal chunks, one per wave, so every wave streams the same number of bytes
//    regardless of how ragged the batch is, and a launch is about one wave per resident slot
//    (no empty workgroups).  A workgroup is eight waves and fills its CU: the waves of one
//    workgroup start together and progress at the same rate, while two workgroups sharing a CU
//    were measured to finish far apart (the later one starts its stream later and streams
//    slower), leaving a tail.  Each workgroup finds its waves' chunk starts with a prefix scan
//    of the context lengths.  A wave walks its chunk piece by piece (a piece = the part of one
//    (sequence, KV head) inside the chunk): a piece that is a whole sequence head is normalised
//    and written out; a cut piece keeps its running max, exp-sum and unnormalised output.
//  * Log-sum-exp merge in two levels, inside this one kernel.  The eight waves of a workgroup
//    own eight consecutive chunks; their cut pieces meet in LDS, the pieces of one sequence head
//    are merged in chunk order (the waves take different heads at once), and a sequence head
//    that ends inside the workgroup is written out there.  A piece cut at a
//    workgroup boundary is published to the workspace with device-coherent stores, and an atomic
//    counter per boundary elects the last workgroup to arrive, which reads all parts of that
//    sequence head back with device-coherent loads, merges them in logical order and resets the
//    counter.  (A device-scope fence would write back or invalidate the whole L2 of the XCD,
//    which costs far more than the merge itself.)  Nothing depends on the physical block ids, so
//    results are identical for any block placement.
//  * Shared prefixes (opt-in).  Sequences whose block tables start with the same physical blocks
//    (a prefix cache shares blocks this way: youngju.dev guide, PagedAttention "主な特性"; Scaling
//    Book note, "プレフィックスキャッシュ") are grouped by prefix_kernel, which runs first and reads
//    each shared block once per tile of up to 16/group members (their query heads fill the 16
//    columns of an MFMA tile) instead of once per sequence.  It leaves every member's partial
//    results (running max, exp-sum, unnormalised output) over the shared blocks in the
//    workspace; decode_kernel then covers only each member's own blocks and folds the partial
//    results in with the same log-sum-exp rule before normalising.
//  * Matrix cores make the arithmetic nearly free: one 16x16x32 MFMA covers 16 tokens x 32 dims
//    for up to 16 query columns, leaving only the softmax on the vector ALUs.
//    QK: S^T = K . Q^T with the K tile (token-major) loaded straight into the A operand: lane
//    (row r = lane%16, group g = lane/16) reads 16 contiguous bytes of token row r.  The rows of a
//    step's two MFMAs are assigned so that the result layout (lane holds column lane%16, rows
//    4g..4g+3) is exactly the B operand of the P.V product.
//    PV: O^T = V^T . P^T.  V tiles are dim-major ([d][16 tokens]), so the A operand (row d, 8
//    consecutive tokens) is one 16-byte load.  P goes in as a bf16 hi/lo pair (two MFMAs), keeping
//    ~16 significant bits of each weight; fp16 P is used as is.
//  * fp8 (OCP e4m3fn) tiles are widened exactly to the MFMA type in registers; the K block scale
//    multiplies the scores, the V block scale the weights.
//  * A step is 32 tokens (two blocks); the loads of the next step are in flight while a step is
//    computed, and the block ids of the step after are fetched with scalar loads meanwhile.  K/V
//    loads are non-temporal: each byte is read once per launch.
#include <limits.h>

#include <type_traits>

#include "device_common.hpp"
#include "pa_internal.hpp"
#include "stepper.hpp"

namespace pa {

// Leading blocks of sequence b that prefix_kernel covers (0 when shared prefixes are off).  The
// plan never takes the block holding a sequence's last token and never more than
// kMaxSharedBlocks, so at least one block is left; the clamp only keeps indexing in range
// (the prefix parts read for a sequence then stay within its prefix_parts).
__device__ __forceinline__ int skip_of(const DecodeArgs& a, int b, int nblk) {
  if (!a.ws_skip) return 0;
  const int s = a.ws_skip[b];
  return max(0, min(min(s, nblk - 1), kMaxSharedBlocks));
}

// A cut piece parked in LDS for the workgroup-level merge.
struct PieceMeta {
  int b, kvh, j0, j1, nblk, skip;
  int s0;   // flattened index of the sequence head's first block (after the skipped ones)
};

// Published parts a merging workgroup stages in LDS at once (more are folded in batches).
constexpr int kMergeStage = 64;

// Parts (partial results over kUnitBlocks shared blocks each) that cover `skip` shared blocks.
__device__ __forceinline__ int prefix_parts(int skip) { return (skip + kUnitBlocks - 1) / kUnitBlocks; }

// Folds the prefix partial results of query row `row` (written by prefix_kernel) into a running
// (m, l, acc) whose tile t holds this lane's column at dims 16 * (t0 + tstride * t) + 4 * grp.
template <int D, int NTL>
__device__ __forceinline__ void fold_prefix(const DecodeArgs& a, size_t row, int nparts, int grp,
                                            int t0, int tstride, float& m, float& l,
                                            f32x4 (&acc)[NTL]) {
  for (int k = 0; k < nparts; ++k) {
    const size_t part = row * a.prefix_parts + k;
    const float pm = a.gp_ml[part * 2], pl = a.gp_ml[part * 2 + 1];
    const float M_ = fmaxf(pm, m);
    const float x = fast_exp2(pm - M_), y = fast_exp2(m - M_);
    l = pl * x + l * y;
    m = M_;
#pragma unroll
    for (int t = 0; t < NTL; ++t) {
      const f32x4 p =
          *reinterpret_cast<const f32x4*>(a.gp_acc + part * D + 16 * (t0 + tstride * t) + 4 * grp);
      acc[t] = p * x + acc[t] * y;
    }
  }
}

// Stores the K row of the new token of sequence b, KV head kvh (k_new [B][Hkv][D]) into offset
// off of physical block blk, one wave (the row is contiguous in the token-major K tile).  Its V
// element goes in with the stepper's read of the block (VAppend).  A block id outside the pool
// skips the store, as pa_kv_append skips such a slot (the stepper reads block 0 instead).
template <int D, int KVT>
__device__ __forceinline__ void append_token(const DecodeArgs& a, int b, int kvh, int blk, int off,
                                             int lane) {
  constexpr int EB = KVT == DT_FP8 ? 1 : 2;
  if ((unsigned)blk >= (unsigned)a.num_blocks) return;
  const size_t row = ((size_t)b * a.num_kv_heads + kvh) * D * EB;
  const size_t tile = ((size_t)blk * a.num_kv_heads + kvh) * kBlock * D * EB;
  uint8_t* kc = reinterpret_cast<uint8_t*>(const_cast<void*>(a.k_cache));
  if (lane < D * EB / 16)
    *reinterpret_cast<uint4*>(kc + tile + (size_t)off * D * EB + 16 * lane) =
        *reinterpret_cast<const uint4*>(a.k_new + row + 16 * lane);
}

// Parts merged with one round of loads per thread (more are staged through LDS in batches).
constexpr int kMergeDirect = 16;

// Merges all parts of sequence head (b, kvh) and writes its normalised output rows: the prefix
// partial results (if any shared blocks were skipped), then the parts published by workgroups
// c0..c1 (workgroup c0 holds it in its slot 0 only if the head starts exactly at its range).
// Called by every thread of the workgroup.
template <int D, int QT>
__device__ __forceinline__ void merge_published(const DecodeArgs& a, int b, int kvh, int skip,
                                                int s0, int c0,
                                int c1, int WGB, float (&sm_mw)[kMergeStage][16],
                                float (&sm_ml)[kMergeStage][16], float* sm_hm, float* sm_hl) {
  typedef typename Mfma<QT>::elem E;
  const int tid = threadIdx.x, nthr = blockDim.x;
  const int G = a.group;
  const int first_slot = s0 != c0 * WGB ? 1 : 0;
  const int npre = skip > 0 ? prefix_parts(skip) : 0;
  const size_t row0 = (size_t)b * a.num_q_heads + kvh * G;
  // part pi of head g: a prefix partial result (pi < npre) or a published part
  auto published = [&](int pi, int g) -> size_t {
    const int cc = c0 + pi - npre;
    return ((size_t)cc * 2 + (cc == c0 ? first_slot : 0)) * G + g;
  };
  // Both kinds of parts live in the workspace: address them from one base (a select between
  // two base pointers here makes the compiler keep them in scratch memory).
  const ptrdiff_t gp_ml_off = npre > 0 ? a.gp_ml - a.ws_ml : 0;
  const ptrdiff_t gp_acc_off = npre > 0 ? a.gp_acc - a.ws_acc : 0;
  auto load_ml = [&](int pi, int g) {
    const ptrdiff_t off = pi < npre
                              ? gp_ml_off + (ptrdiff_t)((row0 + g) * a.prefix_parts + pi) * 2
                              : (ptrdiff_t)published(pi, g) * 2;
    return load_coherent2(a.ws_ml + off);
  };
  auto load_acc = [&](int pi, int g, int d) {
    const ptrdiff_t off = pi < npre
                              ? gp_acc_off + (ptrdiff_t)((row0 + g) * a.prefix_parts + pi) * D
                              : (ptrdiff_t)published(pi, g) * D;
    return load_coherent4(a.ws_acc + off + d);
  };
  const int nparts = npre + c1 - c0 + 1;
  E* rows = reinterpret_cast<E*>(a.out) + row0 * D;
  constexpr int EPT = 16 * D / 4 / (64 * kWaves) > 0 ? 16 * D / 4 / (64 * kWaves) : 1;

  if (nparts <= kMergeDirect) {
    // each thread loads every part's (max, exp-sum) for its head and its four output columns
    // at once and merges them on its own
#pragma unroll
    for (int x = 0; x < EPT; ++x) {
      const int e = (tid + x * nthr) * 4;
      if (e >= G * D) break;
      const int g = e / D, d = e - g * D;
      f32x2 ml[kMergeDirect];
      f32x4 part[kMergeDirect];
#pragma unroll
      for (int k = 0; k < kMergeDirect; ++k)
        if (k < nparts) {
          ml[k] = load_ml(k, g);
          part[k] = load_acc(k, g, d);
        }
      float M_ = -INFINITY;
#pragma unroll
      for (int k = 0; k < kMergeDirect; ++k)
        if (k < nparts) M_ = fmaxf(M_, ml[k][0]);
      float Ls = 0.0f;
      f32x4 o = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int k = 0; k < kMergeDirect; ++k)
        if (k < nparts) {
          const float w = fast_exp2(ml[k][0] - M_);
          Ls += w * ml[k][1];
          o += w * part[k];
        }
      *reinterpret_cast<uint2*>(rows + e) =
          make_uint2(pack2<QT>(o[0] / Ls, o[1] / Ls), pack2<QT>(o[2] / Ls, o[3] / Ls));
    }
    return;
  }

  // Many parts: batches of up to kMergeStage; their (max, exp-sum) pairs are staged in LDS with
  // one round of loads, then every thread loads all its output columns of the batch at once.
  f32x4 o[EPT];
#pragma unroll
  for (int x = 0; x < EPT; ++x) o[x] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  if (tid < 16) {
    sm_hm[tid] = -INFINITY;
    sm_hl[tid] = 0.0f;
  }
  for (int pb = 0; pb < nparts; pb += kMergeStage) {
    const int n = min(kMergeStage, nparts - pb);
    __syncthreads();
    for (int t = tid; t < n * G; t += nthr) {
      const f32x2 ml = load_ml(pb + t / G, t % G);
      sm_mw[t / G][t % G] = ml[0];
      sm_ml[t / G][t % G] = ml[1];
    }
    __syncthreads();
    // per head: new running max; rescale of what is already accumulated
    if (tid < G) {
      float M_ = sm_hm[tid];
      for (int k = 0; k < n; ++k) M_ = fmaxf(M_, sm_mw[k][tid]);
      const float r = M_ == sm_hm[tid] ? 1.0f : fast_exp2(sm_hm[tid] - M_);
      float Ls = sm_hl[tid] * r;
      for (int k = 0; k < n; ++k) {
        const float w = fast_exp2(sm_mw[k][tid] - M_);
        sm_mw[k][tid] = w;
        Ls += w * sm_ml[k][tid];
      }
      sm_ml[0][tid] = r;          // rescale factor for this batch (read below)
      sm_hm[tid] = M_;
      sm_hl[tid] = Ls;
    }
    __syncthreads();
#pragma unroll
    for (int x = 0; x < EPT; ++x) {
      const int e = (tid + x * nthr) * 4;
      if (e >= G * D) break;
      const int g = e / D, d = e - g * D;
      f32x4 acc_b = o[x] * sm_ml[0][g];
      f32x4 part[kMergeStage / 4];
      for (int k0 = 0; k0 < n; k0 += kMergeStage / 4) {
        const int m = min(kMergeStage / 4, n - k0);
#pragma unroll
        for (int k = 0; k < kMergeStage / 4; ++k)
          if (k < m) part[k] = load_acc(pb + k0 + k, g, d);
#pragma unroll
        for (int k = 0; k < kMergeStage / 4; ++k)
          if (k < m) acc_b += sm_mw[k0 + k][g] * part[k];
      }
      o[x] = acc_b;
    }
  }
  __syncthreads();
#pragma unroll
  for (int x = 0; x < EPT; ++x) {
    const int e = (tid + x * nthr) * 4;
    if (e >= G * D) break;
    const int g = e / D;
    const float Ls = sm_hl[g];
    *reinterpret_cast<uint2*>(rows + e) =
        make_uint2(pack2<QT>(o[x][0] / Ls, o[x][1] / Ls), pack2<QT>(o[x][2] / Ls, o[x][3] / Ls));
  }
}

template <int D, int QT, int KVT, bool HEADS>
__global__ __launch_bounds__(64 * kWaves, 8 / kWaves) void decode_kernel(DecodeArgs a) {
  typedef Stepper<D, QT, KVT> St;
  typedef typename St::V8 V8;
  typedef typename St::E E;
  constexpr int NC = St::NC;
  constexpr int NT = St::NT;

  __shared__ int sm_wave_sum[kWaves];
  __shared__ int sm_start_b[kWaves], sm_start_off[kWaves], sm_start_L[kWaves];
  __shared__ int sm_start_skip[kWaves];
  __shared__ PieceMeta sm_meta[kWaves][2];          // [wave][first / last cut piece]
  __shared__ float sm_pm[kWaves][2][16], sm_pl[kWaves][2][16];
  __shared__ f32x4 sm_pacc[kWaves][2][NT][64];
  __shared__ int sm_last[2];
  __shared__ float sm_mw[kMergeStage][16], sm_ml[kMergeStage][16];   // staged parts: m, l
  __shared__ float sm_hm[16], sm_hl[16];                              // per head: max, exp-sum

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = uniform(tid >> 6);
  const int col = lane & 15, grp = lane >> 4;
  const int B = a.batch, Hkv = a.num_kv_heads, Hq = a.num_q_heads, G = a.group;
  const int cap = a.len_cap;

  if constexpr (HEADS) {
    // ---- Short heads (at most 2 * WPH blocks each): WPH waves per sequence head, wave k of a
    // head taking its blocks [skip + 2k, skip + 2k + 2) as one step; the pieces of a head meet
    // in LDS and its waves write it, each a share of the 16-dim tiles.  No scan of the lengths,
    // nothing crosses workgroups.  A launch of its own instance, whose LDS is one piece per
    // wave (a launch costs more the more LDS its workgroups take).
    __shared__ float hm_pm[kWaves][16], hm_pl[kWaves][16];
    __shared__ f32x4 hm_pacc[kWaves][NT][64];
    const int WPH = a.head_mode;
    const int hl = wave / WPH, k = wave - hl * WPH;
    const int h = uniform(blockIdx.x * (kWaves / WPH) + hl);
    int b = 0, kvh = 0, L = 0, nblk = 0, sk = 0;
    if (h < B * Hkv) {
      b = h / Hkv;
      kvh = h - b * Hkv;
      L = clamp_len(a.context_lens[b], cap);
      nblk = blocks_of(L);
      sk = skip_of(a, b, nblk);
    }
    const int j0 = min(sk + 2 * k, nblk), j1 = min(nblk, j0 + 2);
    const int h0 = kvh * G;
    float m_run = -INFINITY, l_run = 0.0f;
    f32x4 acc[NT];
#pragma unroll
    for (int i = 0; i < NT; ++i) acc[i] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    if (j0 < j1) {
      const St st(a, lane);
      const int32_t* trow = a.block_tables + (size_t)b * a.max_blocks_per_seq;
      const int end_tok = j1 == nblk ? L : kBlock * j1;
      const bool append = a.k_new != nullptr && j1 == nblk;
      if (append) append_token<D, KVT>(a, b, kvh, trow[(L - 1) / kBlock], (L - 1) % kBlock, lane);
      V8 qB[NC];
      st.load_q(qB, col < G ? reinterpret_cast<const E*>(a.q) + ((size_t)b * Hq + h0 + col) * D
                            : nullptr);
      if (append && (unsigned)trow[(L - 1) / kBlock] < (unsigned)a.num_blocks) {
        constexpr int EB = KVT == DT_FP8 ? 1 : 2;
        VAppend ap;
        ap.vnew = a.v_new + ((size_t)b * Hkv + kvh) * D * EB;
        ap.blk = (L - 1) / kBlock;
        ap.off = (L - 1) % kBlock;
        st.run_append(qB, trow, kvh, j0, j1, end_tok, m_run, l_run, acc, true, ap);
      } else {
        st.run(qB, trow, kvh, j0, j1, end_tok, 0, 1, m_run, l_run, acc);
      }
      l_run = sum_across_rows(l_run);
    }
    const size_t row = (size_t)b * Hq + h0 + col;
    E* out = reinterpret_cast<E*>(a.out) + row * D + 4 * grp;
    if (WPH == 1) {
      if (h < B * Hkv && col < G) {
        if (nblk == 0) {
#pragma unroll
          for (int i = 0; i < NT; ++i) *reinterpret_cast<uint2*>(out + 16 * i) = make_uint2(0u, 0u);
        } else {
          if (sk > 0) fold_prefix<D>(a, row, prefix_parts(sk), grp, 0, 1, m_run, l_run, acc);
#pragma unroll
          for (int i = 0; i < NT; ++i)
            *reinterpret_cast<uint2*>(out + 16 * i) =
                make_uint2(pack2<QT>(acc[i][0] / l_run, acc[i][1] / l_run),
                           pack2<QT>(acc[i][2] / l_run, acc[i][3] / l_run));
        }
      }
      return;
    }
    if (grp == 0) {
      hm_pm[wave][col] = m_run;
      hm_pl[wave][col] = l_run;
    }
#pragma unroll
    for (int i = 0; i < NT; ++i) hm_pacc[wave][i][lane] = acc[i];
    __syncthreads();
    if (h >= B * Hkv || col >= G) return;
    const int w0 = hl * WPH;
    for (int t = k; t < NT; t += WPH) {
      if (nblk == 0) {
        *reinterpret_cast<uint2*>(out + 16 * t) = make_uint2(0u, 0u);
        continue;
      }
      // piece 0 has tokens (skip_of leaves at least one block), so the maximum is finite
      float M_ = hm_pm[w0][col];
      for (int i = 1; i < WPH; ++i) M_ = fmaxf(M_, hm_pm[w0 + i][col]);
      float gl = 0.0f;
      f32x4 go[1] = {f32x4{0.0f, 0.0f, 0.0f, 0.0f}};
      for (int i = 0; i < WPH; ++i) {
        const float w = fast_exp2(hm_pm[w0 + i][col] - M_);
        gl += w * hm_pl[w0 + i][col];
        go[0] += w * hm_pacc[w0 + i][t][lane];
      }
      if (sk > 0) fold_prefix<D>(a, row, prefix_parts(sk), grp, t, 1, M_, gl, go);
      *reinterpret_cast<uint2*>(out + 16 * t) =
          make_uint2(pack2<QT>(go[0][0] / gl, go[0][1] / gl), pack2<QT>(go[0][2] / gl, go[0][3] / gl));
    }
    return;
  }

  // ---- 1. Flattened block space and this workgroup's chunk starts.  A sequence head (b, kvh)
  // takes its blocks [skip_b, blocks(L_b)) there.  Thread t owns sequences [t*per, t*per + per);
  // W = sum_b Hkv * (blocks(L_b) - skip_b).
  const int per = (B + 255) >> 8;
  const int b_lo = tid * per;
  int tot = 0;
  for (int i = 0; i < per; ++i) {
    const int b = b_lo + i;
    if (b < B) {
      const int nblk = blocks_of(clamp_len(a.context_lens[b], cap));
      tot += Hkv * (nblk - skip_of(a, b, nblk));
    }
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
  int Cw = a.chunk_blocks;
  if (Cw == 0) {
    Cw = (W + a.total_waves - 1) / a.total_waves;
    Cw = max(2, (Cw + 1) & ~1);
  }
  const int nch = (W + Cw - 1) / Cw;
  const int c_first = blockIdx.x * kWaves;
  {
    int run = before + incl - tot;                // blocks before this thread's first sequence
    for (int i = 0; i < per; ++i) {
      const int b = b_lo + i;
      if (b >= B) break;
      const int L = clamp_len(a.context_lens[b], cap);
      const int nblk = blocks_of(L);
      const int sk = skip_of(a, b, nblk);
      const int nb = Hkv * (nblk - sk);
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const long start = (long)(c_first + w) * Cw;
        if (start >= run && start < run + nb) {
          sm_start_b[w] = b;
          sm_start_off[w] = (int)(start - run);
          sm_start_L[w] = L;
          sm_start_skip[w] = sk;
        }
      }
      if (nb == 0 && blockIdx.x == 0) {           // no tokens: the output rows are zeros
        uint4* o = reinterpret_cast<uint4*>(reinterpret_cast<E*>(a.out) + (size_t)b * Hq * D);
        for (int k = 0; k < Hq * D / 8; ++k) o[k] = make_uint4(0u, 0u, 0u, 0u);
      }
      run += nb;
    }
  }
  if (tid < 2 * kWaves) sm_meta[tid >> 1][tid & 1].b = -1;
  __syncthreads();

  const int c = c_first + wave;

  // ---- 2. This wave's chunk [a0, a1) of the flattened space, piece by piece.
  const St st(a, lane);
  const int a0 = c * Cw;
  const int a1 = min(a0 + Cw, W);
  int b = 0, L = 0, nblk = 0, sk = 0, kvh = 0, j = 0;
  int pos = a0;                                     // flattened index of the next block
  bool more = false;
  if (c < nch) {
    b = uniform(sm_start_b[wave]);
    L = uniform(sm_start_L[wave]);
    sk = uniform(sm_start_skip[wave]);
    nblk = blocks_of(L);
    const int off = uniform(sm_start_off[wave]);
    kvh = off / (nblk - sk);
    j = sk + off - kvh * (nblk - sk);
    more = true;
  }
  for (int piece = 0; more; ++piece) {
    const int j0 = j;
    const int j1 = min(nblk, j0 + (a1 - pos));
    const int end_tok = j1 == nblk ? L : kBlock * j1;   // tokens at or past end_tok are masked
    const int h0 = kvh * G;

    const int32_t* trow = a.block_tables + (size_t)b * a.max_blocks_per_seq;

    // Fused append: the piece that holds the sequence head's last block (no other wave reads
    // it in this launch) appends token L-1 of this KV head: its K row is stored before the
    // loads; its V element goes into the registers of the block's V tile, which the stepper's
    // append instance stores back whole.
    const bool append = a.k_new != nullptr && j1 == nblk;
    if (append) append_token<D, KVT>(a, b, kvh, trow[(L - 1) / kBlock], (L - 1) % kBlock, lane);

    V8 qB[NC];
    st.load_q(qB, col < G ? reinterpret_cast<const E*>(a.q) + ((size_t)b * Hq + h0 + col) * D
                          : nullptr);
    float m_run = -INFINITY, l_run = 0.0f;
    f32x4 acc[NT];
#pragma unroll
    for (int i = 0; i < NT; ++i) acc[i] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    if (append && (unsigned)trow[(L - 1) / kBlock] < (unsigned)a.num_blocks) {
      constexpr int EB = KVT == DT_FP8 ? 1 : 2;
      VAppend ap;
      ap.vnew = a.v_new + ((size_t)b * Hkv + kvh) * D * EB;
      ap.blk = (L - 1) / kBlock;
      ap.off = (L - 1) % kBlock;
      st.run_append(qB, trow, kvh, j0, j1, end_tok, m_run, l_run, acc, true, ap);
    } else {
      st.run(qB, trow, kvh, j0, j1, end_tok, 0, 1, m_run, l_run, acc);
    }

    // ---- finish the piece: whole sequence head -> output; cut piece -> LDS slot
    l_run = sum_across_rows(l_run);
    if (j0 == sk && j1 == nblk) {
      if (col < G) {
        const size_t row = (size_t)b * Hq + h0 + col;
        if (sk > 0) fold_prefix<D>(a, row, prefix_parts(sk), grp, 0, 1, m_run, l_run, acc);
        E* out = reinterpret_cast<E*>(a.out) + row * D + 4 * grp;
#pragma unroll
        for (int i = 0; i < NT; ++i)
          *reinterpret_cast<uint2*>(out + 16 * i) =
              make_uint2(pack2<QT>(acc[i][0] / l_run, acc[i][1] / l_run),
                         pack2<QT>(acc[i][2] / l_run, acc[i][3] / l_run));
      }
    } else {
      const int sl = piece == 0 ? 0 : 1;          // only a chunk's first and last can be cut
      if (lane == 0) sm_meta[wave][sl] = PieceMeta{b, kvh, j0, j1, nblk, sk, pos - (j0 - sk)};
      if (grp == 0) {
        sm_pm[wave][sl][col] = m_run;
        sm_pl[wave][sl][col] = l_run;
      }
#pragma unroll
      for (int i = 0; i < NT; ++i) sm_pacc[wave][sl][i][lane] = acc[i];
    }

    pos += j1 - j0;
    if (pos >= a1) break;
    // next piece: the next KV head of this sequence, else the next sequence with tokens
    if (++kvh == Hkv) {
      // pos < a1 <= W guarantees a later sequence with tokens; the bound on b only keeps the
      // walk inside the lengths array should they change while the kernel runs
      kvh = 0;
      L = 0;
      while (L == 0 && b + 1 < B) L = clamp_len(a.context_lens[++b], cap);
      if (L == 0) break;
      nblk = blocks_of(L);
      sk = skip_of(a, b, nblk);
    }
    j = sk;
  }
  __syncthreads();

  // ---- 3. Merge the cut pieces of the workgroup's chunks.  The slots (each wave's first and
  // last piece, in chunk order) of one sequence head are consecutive among the used slots and
  // form a group.  The waves take (group, 16-dim tile) pairs in turn, so even a workgroup whose
  // chunks all belong to one long head merges with every wave.  A group that covers all blocks
  // of its sequence head is written out.  A group cut at the workgroup boundary (at most two:
  // the first group, continuing from before the range, and the last, running past its end) is
  // published; then, after one wait and one round of arrival counts for both, the last
  // workgroup to publish a part of a sequence head merges all of them.
  const int WGB = kWaves * Cw;                      // blocks per workgroup range
  constexpr int NS = 2 * kWaves;                    // slots
  static_assert(NS <= 64, "one slot per lane");
  PieceMeta mt{-1, 0, 0, 0, 0, 0, 0};
  if (lane < NS) mt = sm_meta[lane >> 1][lane & 1];
  const bool used = lane < NS && mt.b >= 0;
  const uint64_t used_mask = __ballot(used);
  const uint64_t before_me = used_mask & ((1ull << lane) - 1ull);
  const int prev = before_me ? 63 - __clzll((long long)before_me) : lane;
  const int prev_b = __shfl(mt.b, prev), prev_kvh = __shfl(mt.kvh, prev);
  const uint64_t start_mask =
      __ballot(used && (prev == lane || prev_b != mt.b || prev_kvh != mt.kvh));
  const int ngroups = __popcll(start_mask);
  // group index of this lane's slot (lane 63: the shift gives 0 and the mask all ones)
  const int gid = __popcll(start_mask & ((2ull << lane) - 1ull)) - 1;

  struct Group {
    uint64_t slots;
    int b, kvh, j0, j1, nblk, skip, s0;
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
    r.skip = __builtin_amdgcn_readlane(mt.skip, f);
    r.s0 = __builtin_amdgcn_readlane(mt.s0, f);
    r.whole = r.j0 == r.skip && r.j1 == r.nblk;
    return r;
  };

  // With one or two groups (long heads), (group, 16-dim tile) pairs are spread over the waves,
  // so that every wave merges: a pair's weights come from one pass over the group's maxima,
  // and its LDS reads are then issued at once.  With more, each wave merges whole groups
  // (weights and slot search once per group, the next slot's reads in flight); spreading
  // pairs there was measured slower (mixed batch, 204 -> 210 us: the prefix fold and the
  // group search are then repeated per tile).
  if (ngroups <= 2) {
    for (int x = wave; x < ngroups * NT; x += kWaves) {
      const int g = x / NT, t = x - g * NT;
      const Group gr = group(g);
      float gm = -INFINITY;
#pragma unroll
      for (int k = 0; k < NS; ++k)
        if ((gr.slots >> k) & 1) gm = fmaxf(gm, sm_pm[k >> 1][k & 1][col]);
      float gl = 0.0f;
      f32x4 go[1] = {f32x4{0.0f, 0.0f, 0.0f, 0.0f}};
#pragma unroll
      for (int k = 0; k < NS; ++k)
        if ((gr.slots >> k) & 1) {
          const float w = fast_exp2(sm_pm[k >> 1][k & 1][col] - gm);
          gl += w * sm_pl[k >> 1][k & 1][col];
          go[0] += w * sm_pacc[k >> 1][k & 1][t][lane];
        }
      if (col >= G) continue;
      if (gr.whole) {
        const size_t row = (size_t)gr.b * Hq + gr.kvh * G + col;
        if (gr.skip > 0) fold_prefix<D>(a, row, prefix_parts(gr.skip), grp, t, 1, gm, gl, go);
        E* out = reinterpret_cast<E*>(a.out) + row * D + 16 * t + 4 * grp;
        *reinterpret_cast<uint2*>(out) = make_uint2(pack2<QT>(go[0][0] / gl, go[0][1] / gl),
                                                    pack2<QT>(go[0][2] / gl, go[0][3] / gl));
      } else {
        // slot 1 holds the group whose sequence head starts strictly inside this workgroup's
        // range (it runs past the end); slot 0 the one that started at or before the range start
        const int wslot = gr.s0 > (int)blockIdx.x * WGB ? 1 : 0;
        const size_t ps = ((size_t)blockIdx.x * 2 + wslot) * G + col;
        store_coherent(a.ws_acc + ps * D + 16 * t + 4 * grp, go[0]);   // device-coherent stores
        if (t == 0 && grp == 0) {
          store_coherent(a.ws_ml + ps * 2, gm);
          store_coherent(a.ws_ml + ps * 2 + 1, gl);
        }
      }
    }
  } else {
    for (int g = wave; g < ngroups; g += kWaves) {
      const Group gr = group(g);
      // log-sum-exp over the group's slots in chunk order; the next slot's LDS reads are issued
      // before the current one is folded in (the last round reads its own slot again)
      uint64_t rest = gr.slots;
      int k = __builtin_ctzll(rest);
      rest &= rest - 1;
      float pm = sm_pm[k >> 1][k & 1][col], pl = sm_pl[k >> 1][k & 1][col];
      f32x4 pa[NT];
#pragma unroll
      for (int t = 0; t < NT; ++t) pa[t] = sm_pacc[k >> 1][k & 1][t][lane];
      float gm = -INFINITY, gl = 0.0f;
      f32x4 go[NT];
#pragma unroll
      for (int t = 0; t < NT; ++t) go[t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
      for (;;) {
        const bool more = rest != 0;
        const int kn = more ? __builtin_ctzll(rest) : k;
        const float pmn = sm_pm[kn >> 1][kn & 1][col], pln = sm_pl[kn >> 1][kn & 1][col];
        f32x4 pan[NT];
#pragma unroll
        for (int t = 0; t < NT; ++t) pan[t] = sm_pacc[kn >> 1][kn & 1][t][lane];
        const float M_ = fmaxf(gm, pm);
        const float x = fast_exp2(gm - M_), y = fast_exp2(pm - M_);
        gl = gl * x + pl * y;
#pragma unroll
        for (int t = 0; t < NT; ++t) go[t] = go[t] * x + pa[t] * y;
        gm = M_;
        if (!more) break;
        rest &= rest - 1;
        k = kn;
        pm = pmn;
        pl = pln;
#pragma unroll
        for (int t = 0; t < NT; ++t) pa[t] = pan[t];
      }
      if (col >= G) continue;
      if (gr.whole) {
        const size_t row = (size_t)gr.b * Hq + gr.kvh * G + col;
        if (gr.skip > 0) fold_prefix<D>(a, row, prefix_parts(gr.skip), grp, 0, 1, gm, gl, go);
        E* out = reinterpret_cast<E*>(a.out) + row * D + 4 * grp;
#pragma unroll
        for (int t = 0; t < NT; ++t)
          *reinterpret_cast<uint2*>(out + 16 * t) =
              make_uint2(pack2<QT>(go[t][0] / gl, go[t][1] / gl),
                         pack2<QT>(go[t][2] / gl, go[t][3] / gl));
      } else {
        // slot 1 holds the group whose sequence head starts strictly inside this workgroup's
        // range (it runs past the end); slot 0 the one that started at or before the range start
        const int wslot = gr.s0 > (int)blockIdx.x * WGB ? 1 : 0;
        const size_t ps = ((size_t)blockIdx.x * 2 + wslot) * G + col;
#pragma unroll
        for (int t = 0; t < NT; ++t)                 // device-coherent stores
          store_coherent(a.ws_acc + ps * D + 16 * t + 4 * grp, go[t]);
        if (grp == 0) {
          store_coherent(a.ws_ml + ps * 2, gm);
          store_coherent(a.ws_ml + ps * 2 + 1, gl);
        }
      }
    }
  }

  // the cut groups this workgroup publishes (at most two), field by field in registers
  int npub = 0, pb_b[2] = {0, 0}, pb_kvh[2] = {0, 0}, pb_skip[2] = {0, 0}, pb_s0[2] = {0, 0};
  int pb_c0[2] = {0, 0}, pb_c1[2] = {0, 0};
#pragma unroll
  for (int x = 0; x < 2; ++x) {
    if (x >= ngroups) break;
    const Group gr = group(x == 0 ? 0 : ngroups - 1);
    if (gr.whole) continue;
    const int c0 = gr.s0 / WGB, c1 = (gr.s0 + (gr.nblk - gr.skip) - 1) / WGB;
#pragma unroll
    for (int y = 0; y < 2; ++y)
      if (y == npub) {
        pb_b[y] = gr.b;
        pb_kvh[y] = gr.kvh;
        pb_skip[y] = gr.skip;
        pb_s0[y] = gr.s0;
        pb_c0[y] = c0;
        pb_c1[y] = c1;
      }
    ++npub;
  }
  if (npub == 0) return;

  // Wait for the published parts to complete, then count them: the counter of a sequence head
  // sits at the last workgroup range it touches, and its last arrival merges.
  wait_memory_ops();
  __syncthreads();
  // both counts in flight at once, from two waves
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
    merge_published<D, QT>(a, x == 0 ? pb_b[0] : pb_b[1], x == 0 ? pb_kvh[0] : pb_kvh[1],
                           x == 0 ? pb_skip[0] : pb_skip[1], x == 0 ? pb_s0[0] : pb_s0[1],
                           x == 0 ? pb_c0[0] : pb_c0[1], c1, WGB, sm_mw, sm_ml, sm_hm, sm_hl);
    if (tid == 0)                                   // ready for the next call
      __hip_atomic_store(a.ws_cnt + c1, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// ---- Shared prefixes.
//
// prefix_kernel groups the sequences whose block tables start with the same physical block,
// finds how many leading entries every member shares with the group's first sequence (its
// leader), and lays each group out as tiles of up to 16/group members in sequence order.  The
// shared length stops before the block that holds a member's last token, so every sequence
// keeps at least one block of its own, and is capped at kMaxSharedBlocks.  Every workgroup
// makes this plan in its own LDS (it depends only on the lengths and tables, so all agree);
// workgroup 0 also writes each sequence's skipped block count for decode_kernel.  Then the
// workgroups take the units: the shared blocks [32k, min(p, 32k + 32)) of one KV head for the
// members of one tile (column r*group + g = query head g of member r), read once.  The waves
// take the unit's 32-token steps in turn and merge in LDS; the unnormalised result and its
// (max, exp-sum) are left for decode_kernel as part k of each member's query rows.

// Exclusive prefix sum over the workgroup's threads (in thread order); `total` gets the sum.
template <int NTH>
__device__ __forceinline__ int block_scan(int v, int* sm, int& total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int incl = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(incl, o);
    if (lane >= o) incl += t;
  }
  if (lane == 63) sm[w] = incl;
  __syncthreads();
  int before = 0;
  total = 0;
#pragma unroll
  for (int i = 0; i < NTH / 64; ++i) {
    const int x = sm[i];
    before += i < w ? x : 0;
    total += x;
  }
  __syncthreads();
  return before + incl - v;
}

// REUSE: the instance for calls that reuse a saved plan (shared_prefixes 2), which declares
// none of the planning arrays: a launch costs more the more LDS its workgroups take.
template <int D, int QT, int KVT, bool REUSE>
__global__ __launch_bounds__(64 * kWaves, 8 / kWaves) void prefix_kernel(DecodeArgs a) {
  typedef Stepper<D, QT, KVT, false> St;
  typedef typename St::V8 V8;
  typedef typename St::E E;
  constexpr int NC = St::NC;
  constexpr int NT = St::NT;
  constexpr int TPW = (NT + kWaves - 1) / kWaves;   // tiles w, w + kWaves, ... of wave w
  constexpr int NTH = 64 * kWaves;
  constexpr int HS = 2048;                          // hash slots: at least twice the batch
  constexpr int PER = kPlanMaxBatch / NTH;          // sequences per thread
  constexpr int SPT = HS / NTH;                     // hash slots per thread
  static_assert(HS >= 2 * kPlanMaxBatch && kPlanMaxBatch % NTH == 0 && HS % NTH == 0, "plan");

  __shared__ int h_key[HS], h_lead[HS], h_cnt[HS], h_p[HS];
  __shared__ int h_mbase[HS];                       // per slot: the group's first member
  __shared__ int s_full[kPlanMaxBatch], s_slot[kPlanMaxBatch];
  __shared__ int s_off[kPlanMaxBatch], s_mslot[kPlanMaxBatch], s_mseq[kPlanMaxBatch];
  __shared__ int s_mlist[kPlanMaxBatch];            // members, group by group, in sequence order
  __shared__ int s_ubase[kPlanMaxBatch];            // per leader: the group's first unit
  __shared__ int s_scan[NTH / 64];
  __shared__ float sm_m[kWaves][16], sm_l[kWaves][16];
  __shared__ uint32_t sm_bad;                       // members a reused unit record drops
  __shared__ f32x4 sm_acc[kWaves][NT][64];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = uniform(tid >> 6);
  const int col = lane & 15, grp = lane >> 4;
  const int B = a.batch, MB = a.max_blocks_per_seq, Hq = a.num_q_heads, Hkv = a.num_kv_heads;
  const int G = a.group, S = 16 / G;

  // The plan (phases 1-3) depends only on the lengths and tables; a call that reuses the one a
  // planning call saved goes straight to the units.
  int U = 0;
  if constexpr (REUSE) {
    // The saved plan is taken only if the header carries this call's signature (descriptor and
    // workspace layout) and a unit count the layout can hold; otherwise (another kind of call
    // wrote over it, or none planned) the call runs with no shared blocks: no units, and
    // workgroup 0 sets every skip count to 0 before decode_kernel reads them.
    const int u0 = a.plan_units[0], s1 = a.plan_units[1], s2 = a.plan_units[2];
    const int umax = plan_tiles_of(B) * Hkv * a.prefix_parts;
    const bool valid = s1 == a.plan_sig && s2 == ~a.plan_sig && u0 >= 0 && u0 <= umax;
    U = valid ? uniform(u0) : 0;
    if (!valid && blockIdx.x == 0)
      for (int b = tid; b < B; b += NTH) a.ws_skip[b] = 0;
  } else {
    // ---- 1. Candidates: two or more whole blocks before the one with the last token, hashed by
    // their first physical block.  A group's leader is its smallest sequence index.
#pragma unroll
    for (int x = 0; x < SPT; ++x) {
      h_key[tid * SPT + x] = -1;
      h_lead[tid * SPT + x] = INT_MAX;
      h_cnt[tid * SPT + x] = 0;
      h_p[tid * SPT + x] = INT_MAX;
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < PER; ++q) {
      const int b = tid * PER + q;
      int slot = -1, full = 0;
      if (b < B) {
        const int L = clamp_len(a.context_lens[b], a.len_cap);
        const int key = a.block_tables[(size_t)b * MB];
        full = L > 0 ? min((L - 1) / kBlock, kMaxSharedBlocks) : 0;
        if (full >= 2 && (unsigned)key < (unsigned)a.num_blocks) {
          unsigned h = ((unsigned)key * 2654435761u) >> 21;
          for (;;) {                                  // ends: fewer keys than slots
            const int prev = atomicCAS(&h_key[h], -1, key);
            if (prev == -1 || prev == key) break;
            h = (h + 1) & (HS - 1);
          }
          slot = (int)h;
          atomicMin(&h_lead[slot], b);
          atomicAdd(&h_cnt[slot], 1);
        }
      }
      s_full[b] = full;
      s_slot[b] = slot;
    }
    __syncthreads();

    // ---- 2. Shared length of a group: the first table entry where a member differs from the
    // leader, at most the shorter of their whole-block counts.  A wave compares 8 members at a
    // time, 64 consecutive entries of each row per round (one coalesced load per row), and stops
    // at a member's first difference.
    int cmpb[PER], csum = 0;
#pragma unroll
    for (int q = 0; q < PER; ++q) {
      const int b = tid * PER + q, slot = s_slot[b];
      cmpb[q] = 0;
      if (slot >= 0 && h_cnt[slot] >= 2) {
        const int lead = h_lead[slot];
        const int cmp = min(s_full[b], s_full[lead]);
        atomicMin(&h_p[slot], cmp);
        if (b != lead && cmp > 1) cmpb[q] = cmp;
      }
      csum += cmpb[q] > 0;
    }
    int ncmp;
    {
      int pos = block_scan<NTH>(csum, s_scan, ncmp);
#pragma unroll
      for (int q = 0; q < PER; ++q)
        if (cmpb[q] > 0) {
          s_off[pos] = tid * PER + q;                 // members to compare, in sequence order
          s_mseq[pos] = cmpb[q];                      // and their comparison lengths
          ++pos;
        }
    }
    __syncthreads();
    for (int k0 = wave * 8; k0 < ncmp; k0 += kWaves * 8) {
      int mb[8], len[8], first[8];
      const int32_t* rm[8];
      const int32_t* rl[8];
#pragma unroll
      for (int v = 0; v < 8; ++v) {
        const int k = k0 + v;
        mb[v] = k < ncmp ? s_off[k] : -1;
        len[v] = k < ncmp ? s_mseq[k] : 0;
        first[v] = INT_MAX;
        const int lead = mb[v] >= 0 ? h_lead[s_slot[mb[v]]] : 0;
        rm[v] = a.block_tables + (size_t)(mb[v] >= 0 ? mb[v] : 0) * MB;
        rl[v] = a.block_tables + (size_t)lead * MB;
      }
      for (int j0 = 1;; j0 += 64) {
        const int j = j0 + lane;
        int x[8], y[8];
        bool live = false;
#pragma unroll
        for (int v = 0; v < 8; ++v) {
          // unconditional loads (clamped into the row), so that they are all in flight at once
          const int jc = min(j, max(len[v] - 1, 0));
          x[v] = rm[v][jc];
          y[v] = rl[v][jc];
        }
#pragma unroll
        for (int v = 0; v < 8; ++v) {
          const bool act = first[v] == INT_MAX && j0 < len[v];
          const unsigned long long diff = __ballot(act && j < len[v] && x[v] != y[v]);
          if (diff) first[v] = j0 + __ffsll((long long)diff) - 1;
          live |= first[v] == INT_MAX && j0 + 64 < len[v];
        }
        if (!live) break;
      }
      if (lane == 0) {
#pragma unroll
        for (int v = 0; v < 8; ++v)
          if (first[v] != INT_MAX) atomicMin(&h_p[s_slot[mb[v]]], first[v]);
      }
    }
    __syncthreads();

    // ---- 3. Members (of groups of two or more sharing two or more blocks), listed in sequence
    // order; a member's rank is the number of members of its group before it.
    int mem[PER], msum = 0;
#pragma unroll
    for (int q = 0; q < PER; ++q) {
      const int slot = s_slot[tid * PER + q];
      mem[q] = slot >= 0 && h_cnt[slot] >= 2 && h_p[slot] >= 2;
      msum += mem[q];
    }
    int nmem;
    {
      int pos = block_scan<NTH>(msum, s_scan, nmem);
#pragma unroll
      for (int q = 0; q < PER; ++q)
        if (mem[q]) {
          s_mslot[pos] = s_slot[tid * PER + q];
          s_mseq[pos] = tid * PER + q;
          ++pos;
        }
    }
    // Groups are numbered in the order of their leaders (hash slots may differ between
    // workgroups; leaders do not): each group's first member and first unit, by prefix sums over
    // the sequences.
    int mc[PER], uc[PER], ms = 0, us = 0;
#pragma unroll
    for (int q = 0; q < PER; ++q) {
      const int b = tid * PER + q, slot = s_slot[b];
      const bool leader = mem[q] && h_lead[slot] == b;
      const int cnt = leader ? h_cnt[slot] : 0;
      mc[q] = cnt;
      uc[q] = leader ? (cnt + S - 1) / S * Hkv * prefix_parts(h_p[slot]) : 0;
      ms += mc[q];
      us += uc[q];
    }
    {
      int mb = block_scan<NTH>(ms, s_scan, nmem);
      int ub = block_scan<NTH>(us, s_scan, U);
#pragma unroll
      for (int q = 0; q < PER; ++q) {
        const int b = tid * PER + q;
        if (mc[q] > 0) {
          h_mbase[s_slot[b]] = mb;
          h_key[s_slot[b]] = 0;                       // rank counter of the member list below
        }
        s_ubase[b] = ub;
        mb += mc[q];
        ub += uc[q];
      }
    }
    __syncthreads();
    // member ranks within their groups: the first wave walks the members in sequence order, 64
    // at a time, one ballot per distinct group in the round
    if (wave == 0) {
      for (int i0 = 0; i0 < nmem; i0 += 64) {
        const int i = i0 + lane;
        const int slot = i < nmem ? s_mslot[i] : -1;
        uint64_t todo = __ballot(slot >= 0);
        while (todo) {
          const int sl = __builtin_amdgcn_readlane(slot, __builtin_ctzll(todo));
          const uint64_t same = __ballot(slot == sl);
          const int base = h_key[sl];
          if (slot == sl) s_mlist[h_mbase[sl] + base + __popcll(same & ((1ull << lane) - 1ull))] =
              s_mseq[i];
          if (lane == 0) h_key[sl] = base + __popcll(same);
          todo &= ~same;
        }
      }
    }
    if (blockIdx.x == 0) {                            // shared blocks each sequence skips
#pragma unroll
      for (int q = 0; q < PER; ++q) {
        const int b = tid * PER + q, slot = s_slot[b];
        if (b < B) a.ws_skip[b] = mem[q] ? h_p[slot] : 0;
      }
      if (tid == 0) {
        a.plan_units[0] = U;
        a.plan_units[1] = a.plan_sig;
        a.plan_units[2] = ~a.plan_sig;
      }
    }
    __syncthreads();
  }

  // ---- 4. The units.
  const St st(a, lane);
  const int r = col / G, g = col - r * G;
  for (int u = blockIdx.x; u < U; u += gridDim.x) {
    int* rec = a.plan_units + kUnitHead + (size_t)u * kUnitRec;
    int lead, kvh, k, j0, j1, member;
    if constexpr (REUSE) {
      // clamped into range: the records are workspace contents this call did not write
      lead = min(max(uniform(rec[0]), 0), B - 1);
      j1 = min(max(uniform(rec[2]), 0), min(MB, kMaxSharedBlocks));
      j0 = min(max(uniform(rec[1]), 0), j1);
      kvh = min(max(uniform(rec[3]), 0), Hkv - 1);
      k = min(max(uniform(rec[4]), 0), a.prefix_parts - 1);
      member = r < S ? rec[kUnitMembers + r] : -1;
      if (member >= B) member = -1;
      // The saved plan is checked against this call's tables and lengths: a member whose table
      // entries over [j0, j1) differ from the leader's, or whose length no longer leaves it a
      // block past j1, is dropped (bit r of sm_bad): its skip count goes to 0, so that
      // decode_kernel reads its whole head, and its parts are not written.  Every unit of a
      // member checks its own range, and the unit ending at the member's skip count checks the
      // length, so a member keeps its skip count only if every shared block still matches.
      // The loads are issued here and used after the unit's steps.
      if (wave == 0) {
        uint32_t bad = 0;
        const int32_t* tl = a.block_tables + (size_t)lead * MB;
        for (int e = lane; e < S * kUnitBlocks; e += 64) {
          const int rr = e / kUnitBlocks, j = j0 + (e - rr * kUnitBlocks);
          const int mb = rec[kUnitMembers + rr];
          if (mb < 0 || mb >= B) continue;
          bool ok = j >= j1 || a.block_tables[(size_t)mb * MB + j] == tl[j];
          if (e == rr * kUnitBlocks) ok = ok && clamp_len(a.context_lens[mb], a.len_cap) > kBlock * j1;
          if (!ok) bad |= 1u << rr;
        }
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) bad |= __shfl_xor(bad, o);
        if (lane == 0) sm_bad = bad;
        if (lane < S && ((bad >> lane) & 1)) {
          const int mb = rec[kUnitMembers + lane];
          if (mb >= 0 && mb < B) a.ws_skip[mb] = 0;
        }
      }
    } else {
      int lo = 0, hi = kPlanMaxBatch - 1;           // the leader whose group's units contain u
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (s_ubase[mid] <= u) lo = mid; else hi = mid - 1;
      }
      const int s = s_slot[lo], p = h_p[s], cnt = h_cnt[s];
      const int ks = prefix_parts(p);
      const int uu = u - s_ubase[lo];
      const int tile = uu / (Hkv * ks), rem = uu - tile * (Hkv * ks);
      lead = lo;
      kvh = rem / ks;
      k = rem - kvh * ks;
      j0 = k * kUnitBlocks;
      j1 = min(p, j0 + kUnitBlocks);
      const int mi = tile * S + r;                  // this column's member within the group
      member = r < S && mi < cnt ? s_mlist[h_mbase[s] + mi] : -1;
      if (wave == 0 && lane < 16) {                 // save the unit for calls that reuse the plan
        const int ml = tile * S + lane;
        rec[kUnitMembers + lane] = lane < S && ml < cnt ? s_mlist[h_mbase[s] + ml] : -1;
        if (lane == 0) {
          rec[0] = lead;
          rec[1] = j0;
          rec[2] = j1;
          rec[3] = kvh;
          rec[4] = k;
        }
      }
    }
    const size_t row = (size_t)member * Hq + kvh * G + g;

    V8 qB[NC];
    st.load_q(qB, member >= 0 ? reinterpret_cast<const E*>(a.q) + row * D : nullptr);
    float m_run = -INFINITY, l_run = 0.0f;
    f32x4 acc[NT];
#pragma unroll
    for (int i = 0; i < NT; ++i) acc[i] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    st.run(qB, a.block_tables + (size_t)lead * MB, kvh, j0, j1, kBlock * j1, wave, kWaves, m_run,
           l_run, acc);
    l_run = sum_across_rows(l_run);

    if (grp == 0) {
      sm_m[wave][col] = m_run;
      sm_l[wave][col] = l_run;
    }
#pragma unroll
    for (int i = 0; i < NT; ++i) sm_acc[wave][i][lane] = acc[i];
    __syncthreads();
    // wave 0 has a step whenever the unit has blocks, so the maximum is finite; waves without
    // steps weigh 0 (an empty unit, possible only from a clamped record, gives zeros)
    float M_ = sm_m[0][col];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) M_ = fmaxf(M_, sm_m[w][col]);
    const float M_ref = M_ == -INFINITY ? 0.0f : M_;
    float wt[kWaves], L_ = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      wt[w] = fast_exp2(sm_m[w][col] - M_ref);
      L_ += wt[w] * sm_l[w][col];
    }
    if (member >= 0 && !(REUSE && ((sm_bad >> r) & 1))) {
      const size_t part = row * a.prefix_parts + k;
#pragma unroll
      for (int tt = 0; tt < TPW; ++tt) {
        const int ti = wave + kWaves * tt;
        if (ti >= NT) break;
        f32x4 o = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int w = 0; w < kWaves; ++w) o += sm_acc[w][ti][lane] * wt[w];
        *reinterpret_cast<f32x4*>(a.gp_acc + part * D + 16 * ti + 4 * grp) = o;
      }
      if (wave == 0 && grp == 0) {
        a.gp_ml[part * 2] = M_;
        a.gp_ml[part * 2 + 1] = L_;
      }
    }
    __syncthreads();                                // LDS is reused by the next unit
  }
}

template <int D, int QT, int KVT>
static hipError_t launch_t(const DecodeArgs& a, int prefix_wgs, hipStream_t stream) {
  if (a.ws_skip) {
    if (a.plan_reuse)
      hipLaunchKernelGGL((prefix_kernel<D, QT, KVT, true>), dim3(prefix_wgs), dim3(64 * kWaves),
                         0, stream, a);
    else
      hipLaunchKernelGGL((prefix_kernel<D, QT, KVT, false>), dim3(prefix_wgs), dim3(64 * kWaves),
                         0, stream, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (a.head_mode > 0)
    hipLaunchKernelGGL((decode_kernel<D, QT, KVT, true>), dim3(a.total_waves / kWaves),
                       dim3(64 * kWaves), 0, stream, a);
  else
    hipLaunchKernelGGL((decode_kernel<D, QT, KVT, false>), dim3(a.total_waves / kWaves),
                       dim3(64 * kWaves), 0, stream, a);
  return hipGetLastError();
}

template <int D, int QT, int KVT>
static int occupancy_t() {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, decode_kernel<D, QT, KVT, false>, 64 * kWaves,
                                                   0)
      != hipSuccess)
    return 0;
  return n;
}

template <int D>
static hipError_t launch_d(const DecodeArgs& a, int q_dtype, int kv_dtype, int prefix_wgs,
                           hipStream_t stream) {
  if (q_dtype == DT_F16 && kv_dtype == DT_F16)
    return launch_t<D, DT_F16, DT_F16>(a, prefix_wgs, stream);
  if (q_dtype == DT_BF16 && kv_dtype == DT_BF16)
    return launch_t<D, DT_BF16, DT_BF16>(a, prefix_wgs, stream);
  if (q_dtype == DT_BF16 && kv_dtype == DT_FP8)
    return launch_t<D, DT_BF16, DT_FP8>(a, prefix_wgs, stream);
  if (q_dtype == DT_F16 && kv_dtype == DT_FP8)
    return launch_t<D, DT_F16, DT_FP8>(a, prefix_wgs, stream);
  return hipErrorInvalidValue;
}

template <int D>
static int occupancy_d(int q_dtype, int kv_dtype) {
  if (q_dtype == DT_F16 && kv_dtype == DT_F16) return occupancy_t<D, DT_F16, DT_F16>();
  if (q_dtype == DT_BF16 && kv_dtype == DT_BF16) return occupancy_t<D, DT_BF16, DT_BF16>();
  if (q_dtype == DT_BF16 && kv_dtype == DT_FP8) return occupancy_t<D, DT_BF16, DT_FP8>();
  if (q_dtype == DT_F16 && kv_dtype == DT_FP8) return occupancy_t<D, DT_F16, DT_FP8>();
  return 0;
}

int decode_workgroups_per_cu(int head_dim, int q_dtype, int kv_dtype) {
  return head_dim == 64 ? occupancy_d<64>(q_dtype, kv_dtype)
                        : occupancy_d<128>(q_dtype, kv_dtype);
}

hipError_t launch_decode(const DecodeArgs& a, int head_dim, int q_dtype, int kv_dtype,
                         int prefix_wgs, hipStream_t stream) {
  if (head_dim == 64) return launch_d<64>(a, q_dtype, kv_dtype, prefix_wgs, stream);
  if (head_dim == 128) return launch_d<128>(a, q_dtype, kv_dtype, prefix_wgs, stream);
  return hipErrorInvalidValue;
}

}  // namespace pa
