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
//    (no empty workgroups).  Each workgroup finds its waves' chunk starts with a prefix scan of
//    the context lengths.  A wave walks its chunk piece by piece (a piece = the part of one
//    (sequence, KV head) inside the chunk): a piece that is a whole sequence head is normalised
//    and written out; a cut piece keeps its running max, exp-sum and unnormalised output.
//  * Log-sum-exp merge in two levels, inside this one kernel.  The four waves of a workgroup own
//    four consecutive chunks; their cut pieces meet in LDS and are merged in chunk order, so a
//    sequence head that ends inside the workgroup is written out there.  A piece cut at a
//    workgroup boundary is published to the workspace with device-coherent stores, and an atomic
//    counter per boundary elects the last workgroup to arrive, which reads all parts of that
//    sequence head back with device-coherent loads, merges them in logical order and resets the
//    counter.  (A device-scope fence would write back or invalidate the whole L2 of the XCD,
//    which costs far more than the merge itself.)  Nothing depends on the physical
//    block ids, so results are identical for any block placement.
//  * Matrix cores make the arithmetic nearly free: one 16x16x32 MFMA covers 16 tokens x 32 dims
//    for up to 16 query heads of a group, leaving only the softmax on the vector ALUs.
//    QK: S^T = K . Q^T with the K tile (token-major) loaded straight into the A operand: lane
//    (row r = lane%16, group g = lane/16) reads 16 contiguous bytes of token row r.  The rows of a
//    step's two MFMAs are assigned so that the result layout (lane holds head lane%16, rows
//    4g..4g+3) is exactly the B operand of the P.V product.
//    PV: O^T = V^T . P^T.  V tiles are dim-major ([d][16 tokens]), so the A operand (row d, 8
//    consecutive tokens) is one 16-byte load.  P goes in as a bf16 hi/lo pair (two MFMAs), keeping
//    ~16 significant bits of each weight; fp16 P is used as is.
//  * fp8 (OCP e4m3fn) tiles are widened exactly to the MFMA type in registers; the K block scale
//    multiplies the scores, the V block scale the weights.
//  * A step is 32 tokens (two blocks); the loads of step s+1 are in flight while step s is
//    computed, and the block ids of step s+2 are fetched with scalar loads meanwhile.  K/V loads
//    are non-temporal: each byte is read once per launch.
#include <type_traits>

#include "device_common.hpp"
#include "pa_internal.hpp"

namespace pa {

template <int D, bool FP8> struct StepRegs;
template <int D> struct StepRegs<D, false> {
  uint4 k[2][D / 32];   // per 16-token row set m: one 16-byte load per 32-dim chunk
  uint4 v[D / 16];      // per 16-dim tile: 8 tokens x 16-bit
};
template <int D> struct StepRegs<D, true> {
  uint4 k[2][D / 64];   // one 16-byte load covers two 32-dim chunks of 8 codes
  uint2 v[D / 16];      // 8 tokens x 1 byte
  float ks, vs;         // block scales of this lane's block
};

template <typename V8>
__device__ __forceinline__ V8 zero_vec8() {
  return __builtin_bit_cast(V8, make_uint4(0u, 0u, 0u, 0u));
}

template <int QT>
__device__ __forceinline__ uint32_t pack2(float x, float y) {
  typedef typename Mfma<QT>::elem E;
  E a = (E)x, b = (E)y;
  uint16_t ua, ub;
  __builtin_memcpy(&ua, &a, 2);
  __builtin_memcpy(&ub, &b, 2);
  return (uint32_t)ua | ((uint32_t)ub << 16);
}

__device__ __forceinline__ int clamp_len(int L, int cap) { return L < 0 ? 0 : (L > cap ? cap : L); }
__device__ __forceinline__ int blocks_of(int L) { return (L + kBlock - 1) / kBlock; }
__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

// Published parts a merging workgroup stages in LDS at once (more are folded in batches).
constexpr int kMergeStage = 64;

// A cut piece parked in LDS for the workgroup-level merge.
struct PieceMeta {
  int b, kvh, j0, j1, nblk, s0;   // s0: flattened index of the sequence head's first block
};

template <int D, int QT, int KVT>
__global__ __launch_bounds__(256, 2) void decode_kernel(DecodeArgs a) {
  typedef Mfma<QT> M;
  typedef typename M::vec8 V8;
  typedef typename M::elem E;
  constexpr bool FP8 = KVT == DT_FP8;
  constexpr bool SPLIT_P = QT == DT_BF16;
  constexpr int EB = FP8 ? 1 : 2;                 // bytes per cache element
  constexpr int NC = D / 32;                      // 32-dim chunks (QK)
  constexpr int NT = D / 16;                      // 16-dim tiles (PV)
  constexpr int KL = FP8 ? NC / 2 : NC;           // K loads per row set
  constexpr int TILE = kBlock * D * EB;           // bytes of one (block, kv head) tile

  static_assert(NT % kWaves == 0, "the merge phase gives each wave NT/4 tiles");
  constexpr int TPW = NT / kWaves;

  __shared__ int sm_wave_sum[kWaves];
  __shared__ int sm_start_b[kWaves], sm_start_off[kWaves];
  __shared__ PieceMeta sm_meta[kWaves][2];          // [wave][first / last cut piece]
  __shared__ float sm_pm[kWaves][2][16], sm_pl[kWaves][2][16];
  __shared__ f32x4 sm_pacc[kWaves][2][NT][64];
  __shared__ int sm_last;
  __shared__ int sm_start_L[kWaves];
  __shared__ float sm_mw[kMergeStage][16], sm_ml[kMergeStage][16];   // published parts: m, l
  __shared__ float sm_hm[16], sm_hl[16];                              // per head: max, exp-sum

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = uniform(tid >> 6);
  const int col = lane & 15, grp = lane >> 4;
  const int B = a.batch, Hkv = a.num_kv_heads, Hq = a.num_q_heads, G = a.group;
  const int cap = a.len_cap;

  // ---- 1. Flattened block space and this workgroup's chunk starts.
  // Thread t owns sequences [t*per, t*per + per); W = sum_b Hkv * blocks(L_b).
  const int per = (B + 255) >> 8;
  const int b_lo = tid * per;
  int tot = 0;
  for (int i = 0; i < per; ++i) {
    const int b = b_lo + i;
    if (b < B) tot += Hkv * blocks_of(clamp_len(a.context_lens[b], cap));
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
      const int nb = Hkv * blocks_of(clamp_len(a.context_lens[b], cap));
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const long start = (long)(c_first + w) * Cw;
        if (start >= run && start < run + nb) {
          sm_start_b[w] = b;
          sm_start_off[w] = (int)(start - run);
          sm_start_L[w] = clamp_len(a.context_lens[b], cap);
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
  const uint8_t* kc = reinterpret_cast<const uint8_t*>(a.k_cache);
  const uint8_t* vc = reinterpret_cast<const uint8_t*>(a.v_cache);
  // K row r = col of MFMA m holds token 16*(r/8) + 8*((r/4)%2) + 4*m + r%4 of the step; its block
  // is r/8.  Result row 4*grp+i of MFMA m is then token tb + 4*m + i with
  // tb = 16*(grp/2) + 8*(grp%2), which is exactly the token order the PV operands use.
  const int k_lane_off = (8 * ((col >> 2) & 1) + (col & 3)) * D * EB + 16 * grp;
  const int v_lane_off = (col * kBlock + 8 * (grp & 1)) * EB;
  const bool k_hi = col >= 8;
  const bool v_hi = grp >= 2;
  const int tb_lane = 16 * (grp >> 1) + 8 * (grp & 1);

  const int a0 = c * Cw;
  const int a1 = min(a0 + Cw, W);
  int b = 0, L = 0, nblk = 0, kvh = 0, j = 0;
  if (c < nch) {
    b = uniform(sm_start_b[wave]);
    L = uniform(sm_start_L[wave]);
    nblk = blocks_of(L);
    const int off = uniform(sm_start_off[wave]);
    kvh = off / nblk;
    j = off - kvh * nblk;
  }
  int pos = a0;
  for (int piece = 0; c < nch; ++piece) {
    const int j0 = j;
    const int j1 = min(nblk, j0 + (a1 - pos));
    const int end_tok = j1 == nblk ? L : kBlock * j1;   // tokens at or past end_tok are masked
    const int nsteps = (j1 - j0 + 1) >> 1;
    const int32_t* trow = a.block_tables + (size_t)b * a.max_blocks_per_seq;
    const int h0 = kvh * G;

    // Q^T as the B operand of the QK product: lane (head col, group grp) holds 8 dims per
    // chunk.  fp8 tiles pair chunks (2c, 2c+1) in one 16-byte load, which permutes which dims a
    // lane holds for each chunk; Q is loaded with the same permutation.
    V8 qB[NC];
    {
      const E* qrow = reinterpret_cast<const E*>(a.q) + ((size_t)b * Hq + h0 + col) * D;
#pragma unroll
      for (int cc = 0; cc < NC; ++cc) {
        const int d0 = FP8 ? 64 * (cc >> 1) + 16 * grp + 8 * (cc & 1) : 32 * cc + 8 * grp;
        qB[cc] = col < G ? as_vec8<V8>(*reinterpret_cast<const uint4*>(qrow + d0))
                         : zero_vec8<V8>();
      }
    }

    float m_run = -INFINITY, l_run = 0.0f;
    f32x4 acc[NT];
#pragma unroll
    for (int i = 0; i < NT; ++i) acc[i] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    // Block ids of a step: logical blocks j0+2s and j0+2s+1 (the second one repeats the first
    // when the piece ends after one block; its tokens are masked).  Ids outside the pool read
    // block 0.
    auto ids_of = [&](int s, int& p0, int& p1) {
      s = min(s, nsteps - 1);
      const int jb = j0 + 2 * s;
      const int jb1 = jb + 1 < j1 ? jb + 1 : jb;
      const int i0 = trow[jb], i1 = trow[jb1];
      p0 = (unsigned)i0 < (unsigned)a.num_blocks ? i0 : 0;
      p1 = (unsigned)i1 < (unsigned)a.num_blocks ? i1 : 0;
    };
    int nid0, nid1;
    ids_of(0, nid0, nid1);

    auto issue = [&](StepRegs<D, FP8>& r, int s) {
      const int pb0 = nid0, pb1 = nid1;
      ids_of(s + 1, nid0, nid1);                   // prefetch the next step's block ids
      const int kb = k_hi ? pb1 : pb0;
      const int vb = v_hi ? pb1 : pb0;
      const uint8_t* kp = kc + ((size_t)kb * Hkv + kvh) * TILE + k_lane_off;
      const uint8_t* vp = vc + ((size_t)vb * Hkv + kvh) * TILE + v_lane_off;
#pragma unroll
      for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int cc = 0; cc < KL; ++cc) r.k[m][cc] = load_stream16(kp + m * 4 * D * EB + cc * 64);
#pragma unroll
      for (int i = 0; i < NT; ++i) {
        if constexpr (FP8)
          r.v[i] = load_stream8(vp + i * 16 * kBlock * EB);
        else
          r.v[i] = load_stream16(vp + i * 16 * kBlock * EB);
      }
      if constexpr (FP8) {
        r.ks = a.k_scale[(size_t)vb * Hkv + kvh];
        r.vs = a.v_scale[(size_t)vb * Hkv + kvh];
      }
    };

    auto compute = [&](StepRegs<D, FP8>& r, int s) {
      const int t0 = kBlock * (j0 + 2 * s);
      const int tb = t0 + tb_lane;
      const bool partial = t0 + kStepTokens > end_tok;     // wave-uniform

      // scores of 8 tokens (tb + jj) for head col
      f32x4 S[2];
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        S[m] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int cc = 0; cc < NC; ++cc) {
          V8 kA;
          if constexpr (FP8) {
            const uint4 w = r.k[m][cc >> 1];
            kA = (cc & 1) ? fp8x8_to_vec8<QT>(w.z, w.w) : fp8x8_to_vec8<QT>(w.x, w.y);
          } else {
            kA = as_vec8<V8>(r.k[m][cc]);
          }
          S[m] = M::mma(kA, qB[cc], S[m]);
        }
      }
      float qs = a.qk_scale_log2;
      if constexpr (FP8) qs *= r.ks;
      float sc[8];
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) sc[jj] = S[jj >> 2][jj & 3] * qs;
      int nval = 8;
      if (partial) {
        nval = min(max(end_tok - tb, 0), 8);
#pragma unroll
        for (int jj = 0; jj < 8; ++jj)
          if (jj >= nval) sc[jj] = -INFINITY;
      }
      float mx = sc[0];
#pragma unroll
      for (int jj = 1; jj < 8; ++jj) mx = fmaxf(mx, sc[jj]);
      mx = max_across_rows(mx);
      const float m_new = fmaxf(m_run, mx);
      const float alpha = fast_exp2(m_run - m_new);
      float pr[8], psum = 0.0f;
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        pr[jj] = fast_exp2(sc[jj] - m_new);
        psum += pr[jj];
      }
      l_run = l_run * alpha + psum;
      m_run = m_new;
#pragma unroll
      for (int i = 0; i < NT; ++i) acc[i] *= alpha;
      if constexpr (FP8) {
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) pr[jj] *= r.vs;
      }

      // P^T as the B operand: this lane's 8 weights, in token order.
      uint4 hi_bits, lo_bits;
      {
        uint32_t h[4], l[4];
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          h[w] = pack2<QT>(pr[2 * w], pr[2 * w + 1]);
          if constexpr (SPLIT_P) {
            const V8 hv = as_vec8<V8>(make_uint4(h[w], 0u, 0u, 0u));
            l[w] = pack2<QT>(pr[2 * w] - (float)hv[0], pr[2 * w + 1] - (float)hv[1]);
          }
        }
        hi_bits = make_uint4(h[0], h[1], h[2], h[3]);
        if constexpr (SPLIT_P) lo_bits = make_uint4(l[0], l[1], l[2], l[3]);
      }
      const V8 pHi = as_vec8<V8>(hi_bits);
      V8 pLo;
      if constexpr (SPLIT_P) pLo = as_vec8<V8>(lo_bits);

      // Masked tokens get weight 0, but their cache slots may hold anything (NaN included), so
      // their V elements are zeroed before the product.
      uint32_t vm[4] = {~0u, ~0u, ~0u, ~0u};
      if (partial) {
        if constexpr (FP8) {
          vm[0] = nval >= 4 ? ~0u : (nval <= 0 ? 0u : (1u << (8 * nval)) - 1u);
          vm[1] = nval >= 8 ? ~0u : (nval <= 4 ? 0u : (1u << (8 * (nval - 4))) - 1u);
        } else {
#pragma unroll
          for (int w = 0; w < 4; ++w)
            vm[w] = (2 * w < nval ? 0x0000FFFFu : 0u) | (2 * w + 1 < nval ? 0xFFFF0000u : 0u);
        }
      }
#pragma unroll
      for (int i = 0; i < NT; ++i) {
        V8 vA;
        if constexpr (FP8) {
          vA = fp8x8_to_vec8<QT>(r.v[i].x & vm[0], r.v[i].y & vm[1]);
        } else {
          const uint4 u = r.v[i];
          vA = as_vec8<V8>(make_uint4(u.x & vm[0], u.y & vm[1], u.z & vm[2], u.w & vm[3]));
        }
        acc[i] = M::mma(vA, pHi, acc[i]);
        if constexpr (SPLIT_P) acc[i] = M::mma(vA, pLo, acc[i]);
      }
    };

    {
      // The steady-state loop issues the next step's loads unconditionally (the tail is
      // peeled), so the loads of step s+1 stay in flight while step s is computed.
      StepRegs<D, FP8> r0, r1;
      int s = 0, rest = nsteps - 1;
      issue(r0, 0);
      for (; rest >= 2; rest -= 2, s += 2) {
        issue(r1, s + 1);
        compute(r0, s);
        issue(r0, s + 2);
        compute(r1, s + 1);
      }
      if (rest == 1) {
        issue(r1, s + 1);
        compute(r0, s);
        compute(r1, s + 1);
      } else {
        compute(r0, s);
      }
    }

    // ---- finish the piece: whole sequence head -> output; cut piece -> LDS slot
    l_run = sum_across_rows(l_run);
    if (j0 == 0 && j1 == nblk) {
      if (col < G) {
        E* out = reinterpret_cast<E*>(a.out) + ((size_t)b * Hq + h0 + col) * D + 4 * grp;
#pragma unroll
        for (int i = 0; i < NT; ++i)
          *reinterpret_cast<uint2*>(out + 16 * i) =
              make_uint2(pack2<QT>(acc[i][0] / l_run, acc[i][1] / l_run),
                         pack2<QT>(acc[i][2] / l_run, acc[i][3] / l_run));
      }
    } else {
      const int sl = piece == 0 ? 0 : 1;          // only a chunk's first and last can be cut
      if (lane == 0) sm_meta[wave][sl] = PieceMeta{b, kvh, j0, j1, nblk, pos - j0};
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
    j = 0;
    if (++kvh == Hkv) {
      // pos < a1 <= W guarantees a later sequence with tokens; the bound on b only keeps the
      // walk inside the lengths array should they change while the kernel runs
      kvh = 0;
      L = 0;
      while (L == 0 && b + 1 < B) L = clamp_len(a.context_lens[++b], cap);
      if (L == 0) break;
      nblk = blocks_of(L);
    }
  }
  __syncthreads();

  // ---- 3. Merge the cut pieces of the four chunks, in chunk order.  Each wave now handles
  // tiles wave, wave+4, ... of every piece.  A group of parts of one sequence head that covers
  // all its blocks is written out; a group cut at the workgroup boundary is published and the
  // last workgroup to publish a part of that sequence head merges all of them.
  const int WGB = kWaves * Cw;                      // blocks per workgroup range
  int gb = -1, gkvh = 0, gj0 = 0, gj1 = 0, gnblk = 0, gs0 = 0;
  float gm = -INFINITY, gl = 0.0f;
  f32x4 go[TPW];

  auto merge_published = [&](int c0, int c1) {
    // parts of sequence head (gb, gkvh) published by workgroups c0..c1; workgroup c0 holds it as
    // its first group (slot 0) only if the sequence head starts exactly at its range.  Batches of
    // up to kMergeStage parts: their (max, exp-sum) pairs are staged in LDS with one round of
    // loads, then every thread loads all its output columns of the batch at once.
    const int first_slot = gs0 != c0 * WGB ? 1 : 0;
    auto slot_of = [&](int cc, int g) {
      return ((size_t)cc * 2 + (cc == c0 ? first_slot : 0)) * G + g;
    };
    E* rows = reinterpret_cast<E*>(a.out) + ((size_t)gb * Hq + gkvh * G) * D;
    constexpr int EPT = 16 * D / 4 / (64 * kWaves);          // float4 columns per thread (G=16)
    f32x4 o[EPT > 0 ? EPT : 1];
#pragma unroll
    for (int x = 0; x < (EPT > 0 ? EPT : 1); ++x) o[x] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    if (tid < 16) { sm_hm[tid] = -INFINITY; sm_hl[tid] = 0.0f; }
    for (int cb = c0; cb <= c1; cb += kMergeStage) {
      const int n = min(kMergeStage, c1 - cb + 1);
      __syncthreads();
      for (int t = tid; t < n * G; t += blockDim.x) {
        const size_t sl = slot_of(cb + t / G, t % G);
        sm_mw[t / G][t % G] = load_coherent(a.ws_ml + sl * 2);
        sm_ml[t / G][t % G] = load_coherent(a.ws_ml + sl * 2 + 1);
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
      for (int x = 0; x < (EPT > 0 ? EPT : 1); ++x) {
        const int e = (tid + x * blockDim.x) * 4;
        if (e >= G * D) break;
        const int g = e / D, d = e - g * D;
        f32x4 acc_b = o[x] * sm_ml[0][g];
        f32x4 part[kMergeStage / 4];
        for (int k0 = 0; k0 < n; k0 += kMergeStage / 4) {
          const int m = min(kMergeStage / 4, n - k0);
#pragma unroll
          for (int k = 0; k < kMergeStage / 4; ++k)
            if (k < m) part[k] = load_coherent4(a.ws_acc + slot_of(cb + k0 + k, g) * D + d);
#pragma unroll
          for (int k = 0; k < kMergeStage / 4; ++k)
            if (k < m) acc_b += sm_mw[k0 + k][g] * part[k];
        }
        o[x] = acc_b;
      }
    }
    __syncthreads();
#pragma unroll
    for (int x = 0; x < (EPT > 0 ? EPT : 1); ++x) {
      const int e = (tid + x * blockDim.x) * 4;
      if (e >= G * D) break;
      const int g = e / D;
      const float Ls = sm_hl[g];
      *reinterpret_cast<uint2*>(rows + e) =
          make_uint2(pack2<QT>(o[x][0] / Ls, o[x][1] / Ls), pack2<QT>(o[x][2] / Ls, o[x][3] / Ls));
    }
  };

  auto emit = [&]() {
    if (gj0 == 0 && gj1 == gnblk) {
      if (col < G) {
        E* out = reinterpret_cast<E*>(a.out) + ((size_t)gb * Hq + gkvh * G + col) * D + 4 * grp;
#pragma unroll
        for (int t = 0; t < TPW; ++t)
          *reinterpret_cast<uint2*>(out + 16 * (wave + kWaves * t)) =
              make_uint2(pack2<QT>(go[t][0] / gl, go[t][1] / gl),
                         pack2<QT>(go[t][2] / gl, go[t][3] / gl));
      }
    } else {
      // slot 1 holds the group whose sequence head starts strictly inside this workgroup's
      // range (it runs past the end); slot 0 the one that started at or before the range start
      const int wslot = gs0 > (int)blockIdx.x * WGB ? 1 : 0;
      const size_t ps = ((size_t)blockIdx.x * 2 + wslot) * G + col;
      // publish with device-coherent stores, wait for them to complete, then count the part;
      // the counter's last arrival reads the parts back with device-coherent loads
      if (col < G) {
#pragma unroll
        for (int t = 0; t < TPW; ++t)
          store_coherent(a.ws_acc + ps * D + 16 * (wave + kWaves * t) + 4 * grp, go[t]);
        if (wave == 0 && grp == 0) {
          store_coherent(a.ws_ml + ps * 2, gm);
          store_coherent(a.ws_ml + ps * 2 + 1, gl);
        }
      }
      wait_memory_ops();
      __syncthreads();
      const int c0 = gs0 / WGB, c1 = (gs0 + gnblk - 1) / WGB;
      if (tid == 0)
        sm_last = __hip_atomic_fetch_add(a.ws_cnt + c1, 1, __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_AGENT) == c1 - c0;
      __syncthreads();
      if (sm_last) {
        merge_published(c0, c1);
        if (tid == 0)                                 // ready for the next call
          __hip_atomic_store(a.ws_cnt + c1, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  };

  for (int k = 0; k < 2 * kWaves; ++k) {
    const PieceMeta mt = sm_meta[k >> 1][k & 1];
    if (mt.b < 0) continue;
    const float pm = sm_pm[k >> 1][k & 1][col], pl = sm_pl[k >> 1][k & 1][col];
    if (mt.b == gb && mt.kvh == gkvh) {
      const float M_ = fmaxf(gm, pm);
      const float x = fast_exp2(gm - M_), y = fast_exp2(pm - M_);
      gl = gl * x + pl * y;
#pragma unroll
      for (int t = 0; t < TPW; ++t)
        go[t] = go[t] * x + sm_pacc[k >> 1][k & 1][wave + kWaves * t][lane] * y;
      gm = M_;
      gj1 = mt.j1;
    } else {
      if (gb >= 0) emit();
      gb = mt.b;
      gkvh = mt.kvh;
      gj0 = mt.j0;
      gj1 = mt.j1;
      gnblk = mt.nblk;
      gs0 = mt.s0;
      gm = pm;
      gl = pl;
#pragma unroll
      for (int t = 0; t < TPW; ++t) go[t] = sm_pacc[k >> 1][k & 1][wave + kWaves * t][lane];
    }
  }
  if (gb >= 0) emit();
}

template <int D, int QT, int KVT>
static hipError_t launch_t(const DecodeArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL((decode_kernel<D, QT, KVT>), dim3(a.total_waves / kWaves), dim3(64 * kWaves),
                     0, stream, a);
  return hipGetLastError();
}

template <int D, int QT, int KVT>
static int occupancy_t() {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, decode_kernel<D, QT, KVT>, 64 * kWaves, 0)
      != hipSuccess)
    return 0;
  return n;
}

template <int D>
static hipError_t launch_d(const DecodeArgs& a, int q_dtype, int kv_dtype, hipStream_t stream) {
  if (q_dtype == DT_F16 && kv_dtype == DT_F16) return launch_t<D, DT_F16, DT_F16>(a, stream);
  if (q_dtype == DT_BF16 && kv_dtype == DT_BF16) return launch_t<D, DT_BF16, DT_BF16>(a, stream);
  if (q_dtype == DT_BF16 && kv_dtype == DT_FP8) return launch_t<D, DT_BF16, DT_FP8>(a, stream);
  if (q_dtype == DT_F16 && kv_dtype == DT_FP8) return launch_t<D, DT_F16, DT_FP8>(a, stream);
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
                         hipStream_t stream) {
  if (head_dim == 64) return launch_d<64>(a, q_dtype, kv_dtype, stream);
  if (head_dim == 128) return launch_d<128>(a, q_dtype, kv_dtype, stream);
  return hipErrorInvalidValue;
}

}  // namespace pa
