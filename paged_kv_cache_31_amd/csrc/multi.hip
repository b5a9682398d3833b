// Causal attention of several new query tokens per sequence over the paged cache, for gfx950.
//
// What is computed: sequence b brings T_b query tokens (rows query_start[b] ..
// query_start[b+1]-1 of q), the last T_b of its L_b = context_lens[b] cached tokens.  Row i sits
// at logical position p = L_b - T_b + i and attends, per query head h (KV head h / group), to the
// tokens 0 .. p gathered through block_tables[b].  This is the target model's one-pass check of
// K draft tokens (youngju.dev guide, speculative-decoding figure; magi page, "投機的デコードとの
// 相互作用") and a chunk of a long prompt against the cache built so far (magi page, "Prefill-
// Decode 分離 — chunked prefill と disaggregation").  Rows before the context (p < 0) see no
// token and are zero, as an empty context is in the single-query decode.
//
// Design for CDNA4.  With T_b * group query rows per (sequence, KV head) the MFMA tiles fill
// up: a row tile is 16 (token, group member) pairs, one MFMA column each, and the same K/V
// streaming core as the single-query decode runs with a causal window per column.  A wave
// handles one item (sequence, KV head, key partition, row tile).  The tiles of one (sequence,
// KV head, partition) are consecutive items, so they share workgroups, and consecutive logical
// workgroups are placed on one XCD (the hardware deals workgroups to the eight XCDs in turn), so
// the re-reads of a K/V block by the tiles of one head hit that XCD's L2 rather than HBM; K/V
// loads are therefore cached, not streamed.  This kernel serves calls with a fixed key
// partition: each tile's keys are cut into partitions whose partial results (running max,
// exp-sum, unnormalised output) go to the workspace and are merged by log-sum-exp in a second
// kernel; with one partition the kernel normalises and writes the output itself.  Without a
// fixed partition, heads of few rows take the balanced split (multi_split_kernel) and larger
// ones chunk_kernel below.
#include <type_traits>

#include "device_common.hpp"
#include "pa_internal.hpp"
#include "stepper.hpp"

namespace pa {

template <int D, int QT, int KVT>
__global__ __launch_bounds__(64 * kMultiWaves, 2) void multi_kernel(MultiArgs a) {
  typedef Stepper<D, QT, KVT, false, true> St;
  typedef typename St::V8 V8;
  typedef typename St::E E;
  constexpr int NC = D / 32;
  constexpr int NT = D / 16;
  const int lane = threadIdx.x & 63;
  const int wave = uniform(threadIdx.x >> 6);

  // logical workgroup: consecutive ones on one XCD (gridDim.x is a multiple of 8)
  const int per_xcd = gridDim.x / 8;
  const int lwg = (blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
  const long long item = (long long)lwg * kMultiWaves + wave;
  if (item >= a.total_items) return;
  const int TPB = a.tiles_per_head, NP = a.num_parts, Hkv = a.num_kv_heads, G = a.group;
  const int tile = (int)(item % TPB);
  long long rest = item / TPB;
  const int part = (int)(rest % NP);
  rest /= NP;
  const int kvh = (int)(rest % Hkv);
  const int b = (int)(rest / Hkv);

  const int q0 = a.query_start[b];
  const int T = min(max(a.query_start[b + 1] - q0, 0), a.max_query_len);
  const int L = clamp_len(a.context_lens[b], a.len_cap);
  const int rows = T * G;
  if (16 * tile >= rows) return;

  // this lane's column: row r = (token i, member g); columns past the last row repeat it
  const int col = lane & 15, grp = lane >> 4;
  const int r_hi = min(16 * tile + 15, rows - 1);
  const bool real = 16 * tile + col <= r_hi;
  const int r = real ? 16 * tile + col : r_hi;
  const int i = r / G, g = r - i * G;
  auto end_of = [&](int ii) { return min(max(L - T + ii + 1, 0), L); };
  const int end_lane = end_of(i);
  const int end_lo = end_of((16 * tile) / G);          // first row of the tile: smallest window
  const int end_hi = end_of(r_hi / G);                 // last row: largest window
  const int nblk = blocks_of(end_hi);
  const int j0 = part * a.part_blocks;
  const int j1 = min(j0 + a.part_blocks, nblk);
  // keys from 16 * j1 on belong to later partitions; a partition of an odd number of blocks
  // ends with a step whose second block repeats its first, and those slots must be masked too
  const int cap = kBlock * j1;
  const long long n = (long long)q0 + i;               // query row of q and out
  const bool row_ok = real && n >= 0 && n < a.total_queries;
  const size_t row = (size_t)n * a.num_q_heads + kvh * G + g;

  St st(a, lane);
  V8 qB[NC];
  st.load_q(qB, row_ok ? reinterpret_cast<const E*>(a.q) + row * D : nullptr);
  float m_run = -INFINITY, l_run = 0.0f;
  f32x4 acc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) acc[t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  if (j0 < j1)
    st.walk_rows(qB, a.block_tables + (size_t)b * a.max_blocks_per_seq, kvh, j0, j1,
                 min(end_lane, cap), min(end_lo, cap), min(end_hi, cap), m_run, l_run, acc);
  l_run = sum_across_rows(l_run);
  if (!row_ok) return;

  if (NP == 1) {
    // a row without keys (before the context) has l = 0 and acc = 0: output zeros
    const float l = l_run > 0.0f ? l_run : 1.0f;
    E* out = reinterpret_cast<E*>(a.out) + row * D + 4 * grp;
#pragma unroll
    for (int t = 0; t < NT; ++t)
      *reinterpret_cast<uint2*>(out + 16 * t) =
          make_uint2(pack2<QT>(acc[t][0] / l, acc[t][1] / l),
                     pack2<QT>(acc[t][2] / l, acc[t][3] / l));
  } else {
    const size_t pi = row * NP + part;
    if (grp == 0) {
      a.ws_ml[2 * pi] = m_run;
      a.ws_ml[2 * pi + 1] = l_run;
    }
#pragma unroll
    for (int t = 0; t < NT; ++t)
      *reinterpret_cast<f32x4*>(a.ws_acc + pi * D + 16 * t + 4 * grp) = acc[t];
  }
}

// Merges the num_parts partial results of each output row (sequence b, query token i, query
// head h) by log-sum-exp and writes the normalised output.  D/DPL lanes take a row (DPL dims
// each): with few partitions, 16 dims a lane and 64/(D/16) rows a wave, so that one round of
// waves covers a large batch; with many, 2 dims a lane, so that the partitions of a row are
// split over more lanes.  Every partition of a row's tile was written by multi_kernel or
// chunk_kernel (an empty one as max -inf, sum 0, output 0: it adds exactly 0).
template <int D, int QT, int DPL>
__global__ __launch_bounds__(256) void multi_merge_kernel(MultiArgs a) {
  typedef typename Mfma<QT>::elem E;
  static_assert(DPL == 2 || DPL == 16, "dims per lane");
  constexpr int LPR = D / DPL;                         // lanes per row
  constexpr int RPW = 64 / LPR > 0 ? 64 / LPR : 1;     // rows per wave
  const int lane = threadIdx.x & 63;
  const int sub = lane / LPR, slice = lane % LPR;      // row of the wave, DPL-dim slice
  const long long w = (long long)blockIdx.x * 4 + uniform(threadIdx.x >> 6);
  const int Hq = a.num_q_heads;
  const long long per_seq = (long long)a.max_query_len * Hq;
  const long long rr = w * RPW + sub;
  if (sub >= RPW || rr >= (long long)a.batch * per_seq) return;
  const int b = (int)(rr / per_seq);
  const int rem = (int)(rr - (long long)b * per_seq);
  const int i = rem / Hq, h = rem - i * Hq;
  const int q0 = a.query_start[b];
  const int T = min(max(a.query_start[b + 1] - q0, 0), a.max_query_len);
  if (i >= T) return;
  const long long n = (long long)q0 + i;
  if (n < 0 || n >= a.total_queries) return;
  const size_t row = (size_t)n * Hq + h;
  const int NP = a.num_parts;
  const float* ml = a.ws_ml + row * NP * 2;
  const float* pacc = a.ws_acc + row * NP * D + DPL * slice;

  float M = -INFINITY;
  for (int p = 0; p < NP; ++p) M = fmaxf(M, ml[2 * p]);
  float o[DPL];
#pragma unroll
  for (int k = 0; k < DPL; ++k) o[k] = 0.0f;
  float den = 1.0f;
  if (M != -INFINITY) {
    den = 0.0f;
#pragma unroll 4
    for (int p = 0; p < NP; ++p) {
      const float wt = fast_exp2(ml[2 * p] - M);
      den += wt * ml[2 * p + 1];
      if constexpr (DPL == 2) {
        const float2 x = *reinterpret_cast<const float2*>(pacc + (size_t)p * D);
        o[0] += wt * x.x;
        o[1] += wt * x.y;
      } else {
        const f32x4* x = reinterpret_cast<const f32x4*>(pacc + (size_t)p * D);
#pragma unroll
        for (int k = 0; k < DPL / 4; ++k) {
          const f32x4 v = x[k];
#pragma unroll
          for (int e = 0; e < 4; ++e) o[4 * k + e] += wt * v[e];
        }
      }
    }
  }
  E* out = reinterpret_cast<E*>(a.out) + row * D + DPL * slice;
  if constexpr (DPL == 2) {
    *reinterpret_cast<uint32_t*>(out) = pack2<QT>(o[0] / den, o[1] / den);
  } else {
#pragma unroll
    for (int k = 0; k < DPL; k += 8)
      *reinterpret_cast<uint4*>(out + k) =
          make_uint4(pack2<QT>(o[k] / den, o[k + 1] / den), pack2<QT>(o[k + 2] / den, o[k + 3] / den),
                     pack2<QT>(o[k + 4] / den, o[k + 5] / den),
                     pack2<QT>(o[k + 6] / den, o[k + 7] / den));
  }
}

// Partitions up to which the merge gives a lane 16 dims of a row (else 2).
constexpr int kMergeWideParts = 4;

template <int D, int QT>
static hipError_t launch_merge(const MultiArgs& a, hipStream_t stream) {
  const long long rows = (long long)a.batch * a.max_query_len * a.num_q_heads;
  if (a.num_parts <= kMergeWideParts) {
    constexpr int RPW = 64 / (D / 16);
    const long long wgs = ((rows + RPW - 1) / RPW + 3) / 4;
    if (wgs > 0)
      hipLaunchKernelGGL((multi_merge_kernel<D, QT, 16>), dim3((unsigned)wgs), dim3(256), 0,
                         stream, a);
  } else {
    constexpr int RPW = 64 / (D / 2) > 0 ? 64 / (D / 2) : 1;
    const long long wgs = ((rows + RPW - 1) / RPW + 3) / 4;
    if (wgs > 0)
      hipLaunchKernelGGL((multi_merge_kernel<D, QT, 2>), dim3((unsigned)wgs), dim3(256), 0,
                         stream, a);
  }
  return hipGetLastError();
}

// ---- Many query rows per (sequence, KV head): prefill chunks, verification of several drafts.
//
// A workgroup of W waves takes 16 * TPW * W consecutive rows of one head (TPW 16-column MFMA
// tiles per wave) and walks the keys of one partition of them in 32-token steps.  Each step's K
// and V tiles are loaded from HBM once per workgroup into one of three or four LDS buffers (16-bit
// caches in the 8-wave shape: straight into LDS, three steps ahead; otherwise every thread a few
// 16-byte words through registers, two steps ahead, fp8 widened on the way); the waves read their
// MFMA operands from LDS, so the tiles of a head share every load.  Per step a wave issues 8 MFMAs
// per tile for the scores and 8 (fp16) or 16 (bf16: P as a hi/lo pair) per tile for P.V.  Operand
// layouts are those of the streaming core: K token rows in the A operand in the order that makes
// the score layout the P^T operand, V^T as the A operand of P.V (the LDS V tile is dim-major, 32
// tokens per dimension row; rows padded to 96 bytes when staged through registers).  V elements of
// tokens at or past the context end are zeroed (when staged, or after the read on the direct
// path), so garbage in the last block's unused slots never reaches the products.  With several
// key partitions (taken when the blocks of rows alone are
// too few to fill the GPU) the unnormalised result and its (max, exp-sum) go to the workspace
// for multi_merge_kernel, as in multi_kernel.
template <int D, int W, int EB>
struct ChunkLds {
  // Bank model (measured on gfx950 with the LDS bank-conflict counter): a 128-bit read serves
  // 16 lanes a cycle from 64 four-byte banks, the lanes with equal bit 5 and equal parity of bits
  // 2-4 of the lane id; a 128-bit store serves 8 consecutive lanes a cycle from 32 banks.
  // K token rows are unpadded; their 16-byte chunks are permuted per row (kswz) so that the 16
  // rows one operand read touches (rows 0-3, 8-11, 16-19, 24-27 of the step) fall on distinct
  // banks.  With 2*D-byte rows, rows r and r + 16 would otherwise share banks.  V dimension rows
  // take 96 bytes (64 of data): with 80 the operand reads and the 16-bit staging stores both
  // met two-way conflicts (a third of the kernel's LDS cycles on a prefill chunk).  LDS always holds
  // 16-bit elements (fp8 codes are widened, exactly, when staged); the fp8 block scales of the
  // step (K then V, for its two blocks) follow the V tile.
  static constexpr int KSTRIDE = 2 * D;                      // bytes per K token row
  static constexpr int VSTRIDE = 2 * kStepTokens + 32;       // bytes per V dimension row
  static constexpr int KBYTES = kStepTokens * KSTRIDE;
  static constexpr int SCALES = KBYTES + D * VSTRIDE;        // 4 floats: k0, k1, v0, v1
  static constexpr int BUF = SCALES + 16;
  static constexpr int WORDS = 2 * kBlock * D * EB / 16;     // 16-byte words of K (or V) a step
  static constexpr int PER_THREAD = (WORDS + 64 * W - 1) / (64 * W);
  static_assert(WORDS % (64 * W) == 0 || WORDS < 64 * W, "whole words per thread");
};

// chunk index of 16-byte chunk c of K token row r in LDS
template <int D>
__device__ __forceinline__ int kswz(int r, int c) {
  if constexpr (D == 128) return c ^ ((r & 3) | (((r >> 3) & 3) << 2));
  else return c ^ (((r >> 1) & 1) | (((r >> 3) & 3) << 1));   // 8 chunks; rows alternate halves
}

// Tiles loaded straight into LDS (16-bit caches): V dimension rows are unpadded (64 bytes: a
// load writes 16 consecutive bytes per lane, so padding would cost loads), and the rows with
// bit 2 set hold their two blocks swapped, which keeps the operand reads on distinct banks.
constexpr int kDirectVRow = 2 * kStepTokens;
__device__ __forceinline__ int vswz(int d, int c) { return c ^ (2 * ((d >> 2) & 1)); }

// s_waitcnt that waits until at most N vector memory operations of this wave are outstanding
// (and nothing else)
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

// One 16-byte load per lane straight into LDS (global_load_lds_dwordx4): lane i writes
// dst + 16 i, dst being wave-uniform.  (A function of its own: called from a generic lambda, the
// builtin kept the host compiler from emitting the kernel's launch stub.)
__device__ __forceinline__ void lds_load16(const uint8_t* src, uint8_t* dst) {
  __builtin_amdgcn_global_load_lds(src, dst, 16, 0, 0);
}

// Workgroup barrier for loads straight into LDS: each wave first waits until its own loads up
// to the one N operations back have landed, so that once every wave has arrived those steps are
// whole in LDS.  (__syncthreads would wait for every load in flight: its release fence covers
// the loads that write LDS.)  LDS reads before the barrier have been consumed by then; the
// signal fences keep the compiler from moving memory operations across it.
template <int N>
__device__ __forceinline__ void direct_barrier() {
  wait_vm<N>();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

template <int D, int QT, int KVT, int W, int TPW, int BUFS>
__global__ __launch_bounds__(64 * W, 8 / W) void chunk_kernel(MultiArgs a) {
  typedef Mfma<QT> M;
  typedef typename M::vec8 V8;
  typedef typename M::elem E;
  constexpr bool FP8 = KVT == DT_FP8;
  constexpr int EB = FP8 ? 1 : 2;                            // bytes per cache element
  typedef ChunkLds<D, W, EB> Lay;
  // bf16 P as a hi/lo pair: rounding it once was measured 20% faster on a 512-token prefill
  // chunk but misses the 2e-3 tolerance on short contexts
  constexpr bool SPLIT_P = QT == DT_BF16;
  constexpr int NC = D / 32;
  constexpr int NT = D / 16;
  constexpr int TB = kBlock * D * EB;                        // bytes of one (block, head) tile
  constexpr int NTHR = 64 * W;
  constexpr int PT = Lay::PER_THREAD;
  constexpr int ROWS_W = 16 * TPW;                           // rows per wave
  constexpr int ROWS_G = ROWS_W * W;                         // rows per workgroup
  static_assert(BUFS == 3 || (BUFS == 4 && W == 8), "LDS step buffers");
  // 16-bit caches in the ping-pong shape load their tiles straight into LDS (four buffers of
  // their own, declared with that loop); the others stage through registers into `lds`
  constexpr bool DIRECT = W == 8 && !FP8;
  __shared__ __attribute__((aligned(16))) uint8_t lds[DIRECT ? 16 : BUFS * Lay::BUF];

  const int tid = threadIdx.x, lane = tid & 63, wave = uniform(tid >> 6);
  const int col = lane & 15, grp = lane >> 4;
  const int per_xcd = gridDim.x / 8;
  const int lwg = (blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
  if ((long long)lwg >= a.total_items) return;               // whole workgroup
  const int Hkv = a.num_kv_heads, G = a.group, RBH = a.row_blocks, NP = a.num_parts;
  const int rb = lwg % RBH;
  const int part = (lwg / RBH) % NP;
  const int kvh = (lwg / RBH / NP) % Hkv;
  const int b = lwg / RBH / NP / Hkv;

  const int q0 = a.query_start[b];
  const int T = min(max(a.query_start[b + 1] - q0, 0), a.max_query_len);
  const int L = clamp_len(a.context_lens[b], a.len_cap);
  const int rows = T * G;
  const int r0 = rb * ROWS_G;
  if (r0 >= rows) return;                                    // whole workgroup
  const int r_last = min(r0 + ROWS_G - 1, rows - 1);
  auto window = [&](int ii) { return min(max(L - T + ii + 1, 0), L); };
  const int nblk_all = blocks_of(window(r_last / G));
  const int j0 = part * a.part_blocks;                       // this partition's blocks [j0, j1)
  const int j1 = min(j0 + a.part_blocks, nblk_all);
  const int cap = kBlock * j1;                               // later keys belong to other parts
  auto end_of = [&](int ii) { return min(window(ii), cap); };
  const int s0 = j0 >> 1;                                    // j0 is even
  const int nsteps = j1 > j0 ? ((j1 - j0 + 1) >> 1) : 0;
  const int se_ = s0 + nsteps;                               // steps [s0, se_)

  // this wave's rows: TPW tiles of 16 columns; columns past the last row repeat it
  const int rw0 = r0 + ROWS_W * wave;
  const bool has_rows = rw0 <= r_last;
  const int rw_last = has_rows ? min(rw0 + ROWS_W - 1, r_last) : r_last;
  const int end_lo = end_of(min(rw0, r_last) / G);
  const int end_hi = end_of(rw_last / G);
  int end_lane[TPW];
  bool real[TPW];
  size_t orow[TPW];
  V8 qB[TPW][NC];
#pragma unroll
  for (int u = 0; u < TPW; ++u) {
    const int rr = rw0 + 16 * u + col;
    real[u] = has_rows && rr <= rw_last;
    const int r = real[u] ? rr : rw_last;
    const int i = r / G, g = r - i * G;
    end_lane[u] = end_of(i);
    const long long n = (long long)q0 + i;
    real[u] = real[u] && n >= 0 && n < a.total_queries;
    orow[u] = (size_t)(real[u] ? n : 0) * a.num_q_heads + kvh * G + g;
    const E* qrow = reinterpret_cast<const E*>(a.q) + orow[u] * D;
#pragma unroll
    for (int cc = 0; cc < NC; ++cc)
      qB[u][cc] = real[u] ? as_vec8<V8>(*reinterpret_cast<const uint4*>(qrow + 32 * cc + 8 * grp))
                          : zero_vec8<V8>();
  }
  float m_run[TPW], l_run[TPW];
  f32x4 acc[TPW][NT];
#pragma unroll
  for (int u = 0; u < TPW; ++u) {
    m_run[u] = -INFINITY;
    l_run[u] = 0.0f;
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[u][t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  }

  // ---- staging: this thread's words of a step's K and V tiles
  const int32_t* trow = a.block_tables + (size_t)b * a.max_blocks_per_seq;
  const uint8_t* kc = reinterpret_cast<const uint8_t*>(a.k_cache);
  const uint8_t* vc = reinterpret_cast<const uint8_t*>(a.v_cache);
  static_assert(PT >= 1 && PT <= 4, "one to four staged words per thread");
  struct Words {                                             // a step's words between load and store
    uint4 k0, v0, k1, v1, k2, v2, k3, v3;
    float sk0, sk1, sv0, sv1;                                // fp8: the two blocks' scales
  };
  Words wa, wb;
  auto fetch_word = [&](int idx, int p0, int p1, uint4& kx, uint4& vx) {
    const int o = 16 * idx, blk = o / TB, off = o - blk * TB;
    const size_t tile = ((size_t)(blk ? p1 : p0) * Hkv + kvh) * TB + off;
    kx = *reinterpret_cast<const uint4*>(kc + tile);
    vx = *reinterpret_cast<const uint4*>(vc + tile);
  };
  // Every fetch issues the same loads whatever the step (a step past the range reloads the last
  // one; threads past the step's words reload a word), so that the count of loads in flight is
  // the same on every path and the wait before staging a step leaves the later steps' loads in
  // flight instead of draining them all.
  // the physical blocks of step s (a step past the range: the last one's; an empty range: a
  // block its table holds)
  struct StepIds {
    int p0, p1;
  };
  auto ids_of = [&](int s) {
    s = max(min(s, se_ - 1), 0);
    const int jb0 = 2 * s, jb1 = 2 * s + 1 < j1 ? 2 * s + 1 : 2 * s;
    return StepIds{trow[jb0], trow[jb1]};
  };
  auto fetch_ids = [&](StepIds id, Words& w) {
    const int p0 = (unsigned)id.p0 < (unsigned)a.num_blocks ? id.p0 : 0;
    const int p1 = (unsigned)id.p1 < (unsigned)a.num_blocks ? id.p1 : 0;
    if constexpr (FP8) {
      w.sk0 = a.k_scale[(size_t)p0 * Hkv + kvh];
      w.sk1 = a.k_scale[(size_t)p1 * Hkv + kvh];
      w.sv0 = a.v_scale[(size_t)p0 * Hkv + kvh];
      w.sv1 = a.v_scale[(size_t)p1 * Hkv + kvh];
    }
    const int t0w = Lay::WORDS < NTHR ? tid % Lay::WORDS : tid;
    fetch_word(t0w, p0, p1, w.k0, w.v0);
    if constexpr (PT > 1) fetch_word(tid + NTHR, p0, p1, w.k1, w.v1);
    if constexpr (PT > 2) fetch_word(tid + 2 * NTHR, p0, p1, w.k2, w.v2);
    if constexpr (PT > 3) fetch_word(tid + 3 * NTHR, p0, p1, w.k3, w.v3);
  };
  auto fetch = [&](int s, Words& w) { fetch_ids(ids_of(s), w); };
  // The block ids of steps s and s + 1 (lanes 0-3: step s's two blocks, then step s + 1's), read
  // by one vector load two iterations before their use, so that its wait falls in order behind
  // the K/V loads.  Scalar loads of them at their use left the table's latency in the loop, and
  // scalar loads issued early are waited on by the next barrier (they share its wait counter
  // with LDS operations).
  auto ids_vec = [&](int s) {
    const int ss = max(min(s + ((lane >> 1) & 1), se_ - 1), 0);
    const int jb = 2 * ss + (lane & 1);
    return trow[jb < j1 ? jb : 2 * ss];
  };
  auto ids_step = [&](int ids, int k) {   // step k (0 or 1) of an ids_vec load
    return StepIds{__builtin_amdgcn_readlane(ids, 2 * k), __builtin_amdgcn_readlane(ids, 2 * k + 1)};
  };
  // V halves of 8 tokens starting at token tv of the step: tokens at or past the end zeroed
  auto keep_v = [&](uint4 x, int t0, int tv) {
    const int valid = L - (t0 + tv);
    if (valid < 8) {
      auto keep = [&](int k) {
        return (2 * k < valid ? 0x0000FFFFu : 0u) | (2 * k + 1 < valid ? 0xFFFF0000u : 0u);
      };
      x.x &= keep(0);
      x.y &= keep(1);
      x.z &= keep(2);
      x.w &= keep(3);
    }
    return x;
  };
  auto widen16 = [&](uint32_t w0, uint32_t w1) {
    return __builtin_bit_cast(uint4, fp8x8_to_vec8<QT>(w0, w1));
  };
  auto stage_word8 = [&](int idx, int t0, uint8_t* kb, uint8_t* vb, uint4 kx, uint4 vx) {
    const int o = 16 * idx, blk = o / TB, off = o - blk * TB;
    // K: 16 codes of one token row (dims cb .. cb + 15) -> two 16-byte chunks of 16-bit values
    const int tok = off / D, cb = off - tok * D;
    const int row = kBlock * blk + tok;
    // Each store writes one half per thread: the first half where bit 2 of idx is clear, the
    // second where it is set, so that the 8 threads one store cycle serves cover all 32 banks.
    const int sw = (idx >> 2) & 1;
    uint8_t* kr = kb + row * Lay::KSTRIDE;
    *reinterpret_cast<uint4*>(kr + 16 * kswz<D>(row, cb / 8 + sw)) =
        widen16(sw ? kx.z : kx.x, sw ? kx.w : kx.y);
    *reinterpret_cast<uint4*>(kr + 16 * kswz<D>(row, cb / 8 + 1 - sw)) =
        widen16(sw ? kx.x : kx.z, sw ? kx.y : kx.w);
    // V: one dimension row of the block (16 tokens) -> its two 8-token halves
    const int d = off / 16, tv = kBlock * blk;
    uint8_t* vr = vb + d * Lay::VSTRIDE + 2 * tv;
    *reinterpret_cast<uint4*>(vr + 16 * sw) =
        keep_v(widen16(sw ? vx.z : vx.x, sw ? vx.w : vx.y), t0, tv + 8 * sw);
    *reinterpret_cast<uint4*>(vr + 16 - 16 * sw) =
        keep_v(widen16(sw ? vx.x : vx.z, sw ? vx.y : vx.w), t0, tv + 8 - 8 * sw);
  };
  auto stage_word = [&](int idx, int t0, uint8_t* kb, uint8_t* vb, uint4 kx, uint4 vx) {
    if constexpr (FP8) {
      stage_word8(idx, t0, kb, vb, kx, vx);
      return;
    }
    const int o = 16 * idx, blk = o / TB, off = o - blk * TB;
    // K tile: token rows of 2*D bytes
    const int tok = off / (2 * D), cb = off - tok * (2 * D);
    const int row = kBlock * blk + tok;
    *reinterpret_cast<uint4*>(kb + row * Lay::KSTRIDE + 16 * kswz<D>(row, cb / 16)) = kx;
    // V tile: dimension rows of 16 tokens (32 bytes); this word holds 8 of them
    const int d = off / 32, h = (off / 16) & 1;
    const int tv = kBlock * blk + 8 * h;
    *reinterpret_cast<uint4*>(vb + d * Lay::VSTRIDE + 2 * tv) = keep_v(vx, t0, tv);
  };
  auto stage = [&](int s, int buf, const Words& w) {
    uint8_t* kb = lds + buf * Lay::BUF;
    uint8_t* vb = kb + Lay::KBYTES;
    const int t0 = kStepTokens * s;
    if constexpr (FP8) {
      if (tid == 0)
        *reinterpret_cast<float4*>(kb + Lay::SCALES) = make_float4(w.sk0, w.sk1, w.sv0, w.sv1);
    }
    if (Lay::WORDS < NTHR && tid >= Lay::WORDS) return;     // a step has fewer words than threads
    stage_word(tid, t0, kb, vb, w.k0, w.v0);
    if constexpr (PT > 1) stage_word(tid + NTHR, t0, kb, vb, w.k1, w.v1);
    if constexpr (PT > 2) stage_word(tid + 2 * NTHR, t0, kb, vb, w.k2, w.v2);
    if constexpr (PT > 3) stage_word(tid + 3 * NTHR, t0, kb, vb, w.k3, w.v3);
  };

  // ---- products of one step for this wave's tiles
  const int krow0 = 16 * (col >> 3) + 8 * ((col >> 2) & 1) + (col & 3);
  const int vchunk = vswz(col, grp);                      // (row 16 t + col: same bit 2)
  const float qs = a.qk_scale_log2;
  // scores of step s (unscaled) for this wave's tiles, from LDS buffer buf
  // the ping-pong shape issues all LDS operand reads of a product block before its MFMAs
  // (measured: prefill chunk 231.3 -> 228.8 us)
  constexpr bool PRE = W == 8;
  auto scores_at = [&](const uint8_t* kb, f32x4 (&S)[TPW][2]) {
#pragma unroll
    for (int u = 0; u < TPW; ++u)
#pragma unroll
      for (int m = 0; m < 2; ++m) S[u][m] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    auto kop = [&](int m, int cc) {
      const int row = krow0 + 4 * m;
      // one vector load (a uint4 read is split into dwords and merged again late, which drops
      // what tells the compiler which LDS buffer it reads)
      return *reinterpret_cast<const V8*>(kb + row * Lay::KSTRIDE + 16 * kswz<D>(row, 4 * cc + grp));
    };
    V8 kAll[PRE ? 2 : 1][PRE ? NC : 1];
    if constexpr (PRE) {
#pragma unroll
      for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int cc = 0; cc < NC; ++cc) kAll[m][cc] = kop(m, cc);
    }
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int cc = 0; cc < NC; ++cc) {
        const V8 kA = PRE ? kAll[PRE ? m : 0][PRE ? cc : 0] : kop(m, cc);
#pragma unroll
        for (int u = 0; u < TPW; ++u) S[u][m] = M::mma(kA, qB[u][cc], S[u][m]);
      }
    if constexpr (PRE) {                          // all LDS reads, then the products
      __builtin_amdgcn_sched_group_barrier(0x100, 2 * NC, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 2 * NC * TPW, 0);
    }
  };
  auto scores = [&](int buf, f32x4 (&S)[TPW][2]) { scores_at(lds + buf * Lay::BUF, S); };
  // online softmax of step s's scores (LDS buffer buf holds the step): rescales the
  // accumulators and gives the weights as the P^T operands of P.V
  auto softmax = [&](int s, int buf, f32x4 (&S)[TPW][2], V8 (&pHi)[TPW], V8 (&pLo)[TPW]) {
    const int t0 = kStepTokens * s;
    // fp8: this lane's 8 tokens lie in block grp / 2 of the step; its K scale multiplies the
    // scores, its V scale the weights (after their sum is taken)
    float ksc = 1.0f, vsc = 1.0f;
    if constexpr (FP8) {
      const float* scl = reinterpret_cast<const float*>(lds + buf * Lay::BUF + Lay::SCALES);
      ksc = scl[grp >> 1];
      vsc = scl[2 + (grp >> 1)];
    }
    const bool partial = t0 + kStepTokens > end_lo;          // wave-uniform
    const int tb = t0 + 8 * grp;
    // headroom of the reference max: weights below 2^8 (bf16 hi/lo and fp16 P hold them);
    // fp16 P over an fp8 cache carries the V block scale too, so there the weights stay <= 1
    constexpr float kLazy = QT == DT_F16 && FP8 ? 0.0f : 8.0f;

    // Scores stay unscaled until the exponent: the largest scaled score is the scaled largest
    // (or smallest, for a negative scale) raw one, and exp2(fma(s, scale, -m)) saves a pass.
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
      // masked in place: a copy of the scores would cost a move per register on every step
      if constexpr (FP8) {
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) S[u][jj >> 2][jj & 3] *= ksc;
      }
      const float masked = qs >= 0.0f ? -INFINITY : INFINITY;
      if (partial) {
        const int nval = min(max(end_lane[u] - tb, 0), 8);
#pragma unroll
        for (int jj = 0; jj < 8; ++jj)
          if (jj >= nval) S[u][jj >> 2][jj & 3] = masked;
      }
      float sc[8];
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) sc[jj] = S[u][jj >> 2][jj & 3];
      // the lane's largest scaled score (the smallest raw one for a negative scale)
      float mx = sc[0];
      if (qs >= 0.0f) {
#pragma unroll
        for (int jj = 1; jj < 8; ++jj) mx = fmaxf(mx, sc[jj]);
      } else {
#pragma unroll
        for (int jj = 1; jj < 8; ++jj) mx = fminf(mx, sc[jj]);
      }
      // A row's reference max moves only when a score exceeds it by more than kLazy (log2
      // units), so weights stay below 2^kLazy; a step that moves no reference in the wave needs
      // no reduction across the row's lanes and no rescale.
      float alpha = 1.0f;
      if (__any(mx * qs > m_run[u] + kLazy)) {
        const float mr = qs >= 0.0f ? max_across_rows(mx) : -max_across_rows(-mx);
        const float m_new = fmaxf(m_run[u], mr * qs);
        const float m_ref = m_new == -INFINITY ? 0.0f : m_new;
        alpha = fast_exp2(m_run[u] - m_ref);
        m_run[u] = m_new;
        if (__any(alpha != 1.0f)) {
#pragma unroll
          for (int t = 0; t < NT; ++t) acc[u][t] *= alpha;
        }
      }
      const float m_ref = m_run[u] == -INFINITY ? 0.0f : m_run[u];
      float pr[8];
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) pr[jj] = fast_exp2(__builtin_fmaf(sc[jj], qs, -m_ref));
      if (partial) {                              // a zero scale makes the masked exponents NaN
        const int nval = min(max(end_lane[u] - tb, 0), 8);
#pragma unroll
        for (int jj = 0; jj < 8; ++jj)
          if (jj >= nval) pr[jj] = 0.0f;
      }
      float psum = pr[0];
#pragma unroll
      for (int jj = 1; jj < 8; ++jj) psum += pr[jj];
      l_run[u] = l_run[u] * alpha + psum;
      if constexpr (FP8) {
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) pr[jj] *= vsc;
      }
      uint32_t h[4], lo[4];
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        h[w] = pack2<QT>(pr[2 * w], pr[2 * w + 1]);
        if constexpr (SPLIT_P) lo[w] = bf16_lo2(pr[2 * w], pr[2 * w + 1], h[w]);
      }
      pHi[u] = as_vec8<V8>(make_uint4(h[0], h[1], h[2], h[3]));
      if constexpr (SPLIT_P) pLo[u] = as_vec8<V8>(make_uint4(lo[0], lo[1], lo[2], lo[3]));
    }
  };
  // the P.V products of a step whose weights softmax() gave, V from LDS buffer buf
  // (tiles loaded straight into LDS keep whatever the cache holds past the context end, so the
  // step holding it zeroes those V elements after reading them)
  auto pv_at = [&](const uint8_t* vb, int t0, const V8 (&pHi)[TPW], const V8 (&pLo)[TPW]) {
    auto vraw = [&](int t) {          // whole-vector loads, as kop's
      if constexpr (DIRECT)
        return *reinterpret_cast<const u32x4*>(vb + (16 * t + col) * kDirectVRow + 16 * vchunk);
      else
        return *reinterpret_cast<const u32x4*>(vb + (16 * t + col) * Lay::VSTRIDE + 16 * grp);
    };
    auto vop = [&](int t) { return __builtin_bit_cast(V8, vraw(t)); };
    V8 vAll[PRE ? NT : 1];
    if constexpr (PRE) {
      u32x4 raw[NT];
#pragma unroll
      for (int t = 0; t < NT; ++t) raw[t] = vraw(t);
      if (DIRECT && t0 + kStepTokens > L) {             // (selects: no divergent branch)
        const int valid = L - (t0 + 8 * grp);
        auto keep = [&](int k) {
          return (2 * k < valid ? 0x0000FFFFu : 0u) | (2 * k + 1 < valid ? 0xFFFF0000u : 0u);
        };
        const u32x4 km = {keep(0), keep(1), keep(2), keep(3)};
#pragma unroll
        for (int t = 0; t < NT; ++t) raw[t] &= km;
      }
#pragma unroll
      for (int t = 0; t < NT; ++t) vAll[t] = __builtin_bit_cast(V8, raw[t]);
    }
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const V8 vA = PRE ? vAll[PRE ? t : 0] : vop(t);
#pragma unroll
      for (int u = 0; u < TPW; ++u) {
        acc[u][t] = M::mma(vA, pHi[u], acc[u][t]);
        if constexpr (SPLIT_P) acc[u][t] = M::mma(vA, pLo[u], acc[u][t]);
      }
    }
    if constexpr (PRE) {                          // all LDS reads, then the products
      __builtin_amdgcn_sched_group_barrier(0x100, NT, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, NT * TPW * (SPLIT_P ? 2 : 1), 0);
    }
  };
  auto pv = [&](int buf, const V8 (&pHi)[TPW], const V8 (&pLo)[TPW]) {
    pv_at(lds + buf * Lay::BUF + Lay::KBYTES, 0, pHi, pLo);
  };
  auto softmax_pv = [&](int s, int buf, f32x4 (&S)[TPW][2]) {
    V8 pHi[TPW], pLo[TPW];
    softmax(s, buf, S, pHi, pLo);
    pv(buf, pHi, pLo);
  };

  const int se = s0 + nsteps;
  auto active = [&](int s) { return has_rows && kStepTokens * s < end_hi; };
  if constexpr (DIRECT) {
    // The ping-pong schedule below with the tiles loaded straight into LDS
    // (global_load_lds_dwordx4: each lane writes 16 bytes, consecutive in lane order, at a
    // wave-uniform LDS address): no register staging and no LDS stores.  Four buffers, each an
    // LDS array of its own so that the compiler can tell them apart (a read of one buffer then
    // waits for none of the loads into the others); the loop is unrolled by four so that every
    // buffer index is known.  Step s + 3 is loaded at the middle barrier of iteration s, into
    // the buffer step s - 1 left (its last readers ran before that barrier), and must have
    // landed by the middle barrier of iteration s + 2 (the first group reads it after that one).
    // Every step's loads are issued whatever the step (past the range: the last step again), so
    // that the count of vector memory operations behind a step's loads is fixed: one step's
    // (NSEG per wave) per iteration.
    constexpr int KBY = kStepTokens * 2 * D;                 // K tile of a step, then V
    constexpr int DBUF = 2 * KBY;
    constexpr int NSEG = D / 64;                             // 1 KiB segments per wave and step
    static_assert(DBUF == 8 * NSEG * 1024 && D * kDirectVRow == KBY, "direct layout");
    __shared__ __attribute__((aligned(16))) uint8_t db0[DBUF], db1[DBUF], db2[DBUF], db3[DBUF];
    auto bufp = [&](auto bc) -> uint8_t* {
      constexpr int B = decltype(bc)::value & 3;
      return B == 0 ? db0 : B == 1 ? db1 : B == 2 ? db2 : db3;
    };
    // waves 0-3 load the K tile (token rows, chunks permuted by kswz), waves 4-7 the V tile
    // (dimension rows, chunks permuted by vswz); per lane and segment: the block of the step
    // and the byte offset inside its (block, head) tile
    const bool dk = wave < 4;
    const uint8_t* dsrc = dk ? kc : vc;
    const int dl0 = (dk ? 0 : KBY) + 1024 * NSEG * (wave & 3);
    int dofs[NSEG], dblk[NSEG];
#pragma unroll
    for (int j = 0; j < NSEG; ++j) {
      const int o = 1024 * (NSEG * (wave & 3) + j) + 16 * lane;
      if (dk) {
        const int row = o / (2 * D), c = kswz<D>(row, (o % (2 * D)) / 16);   // kswz: an involution
        dblk[j] = row / kBlock;
        dofs[j] = (row % kBlock) * 2 * D + 16 * c;
      } else {
        const int d = o / kDirectVRow, c = vswz(d, (o % kDirectVRow) / 16);
        dblk[j] = c >> 1;
        dofs[j] = d * 2 * kBlock + 16 * (c & 1);
      }
    }
    auto load_step = [&](StepIds id, auto bc) {
      constexpr int B = decltype(bc)::value & 3;
      const int p0 = (unsigned)id.p0 < (unsigned)a.num_blocks ? id.p0 : 0;
      const int p1 = (unsigned)id.p1 < (unsigned)a.num_blocks ? id.p1 : 0;
#pragma unroll
      for (int j = 0; j < NSEG; ++j) {
        const uint8_t* src = dsrc + ((size_t)(dblk[j] ? p1 : p0) * Hkv + kvh) * TB + dofs[j];
        lds_load16(src, bufp(bc) + dl0 + 1024 * j);
      }
    };
    typedef std::integral_constant<int, 0> B0;
    typedef std::integral_constant<int, 1> B1;
    typedef std::integral_constant<int, 2> B2;
    typedef std::integral_constant<int, 3> B3;
    const bool lead = wave < W / 2;
    // The partition's block ids go to LDS first (the plan keeps partitions of this kernel within
    // kDirectMaxBlocks): read from there, they cost no vector load in the loop, whose result the
    // compiler would wait for together with every tile load issued before it.
    __shared__ int dids[kDirectMaxBlocks];
    // (the launch rejects longer partitions; the bound keeps the copy inside the table anyway)
    for (int k = tid; k < min(j1 - j0, kDirectMaxBlocks); k += NTHR) dids[k] = trow[j0 + k];
    __syncthreads();
    auto ids_at = [&](int s) {            // a step past the range: the last one's
      const int ss = max(min(s, se_ - 1), s0);
      const int jb = min(2 * ss - j0, kDirectMaxBlocks - 2);
      return StepIds{dids[jb], dids[2 * ss + 1 < j1 ? jb + 1 : jb]};
    };
    f32x4 S[TPW][2];
    V8 pHi[TPW], pLo[TPW];
    // the middle barrier of iteration s: step s + 1 in LDS; then step s + 3's loads (its block
    // ids read at the start of the iteration)
    auto middle = [&](auto bc, StepIds id) {
      constexpr int B = decltype(bc)::value;
      direct_barrier<NSEG>();
      load_step(id, std::integral_constant<int, B + 3>());
    };
    // The loop starts three iterations early, which only load steps s0 .. s0 + 2: with every
    // load issued from inside the loop, the compiler keeps track of which buffer each one fills
    // across the loop's back edge (loads issued before the loop made it wait for all of them at
    // the first reads of every pass).  Step s lives in buffer (s - s0) % 4.
    auto run = [&](auto iteration) {
      for (int s = s0 - 3; s < se;) {
        iteration(s, B1());
        if (++s >= se) break;
        iteration(s, B2());
        if (++s >= se) break;
        iteration(s, B3());
        if (++s >= se) break;
        iteration(s, B0());
        ++s;
      }
    };
    auto on = [&](int s) { return s >= s0 && s < se && active(s); };
    if (lead) {
      run([&](int s, auto bc) {
        constexpr int B = decltype(bc)::value;
        const StepIds id = ids_at(s + 3);
        if (on(s)) softmax(s, 0, S, pHi, pLo);
        middle(bc, id);
        if (on(s)) pv_at(bufp(bc) + KBY, kStepTokens * s, pHi, pLo);
        if (on(s + 1)) scores_at(bufp(std::integral_constant<int, B + 1>()), S);
        direct_barrier<63>();
      });
    } else {
      run([&](int s, auto bc) {
        constexpr int B = decltype(bc)::value;
        const StepIds id = ids_at(s + 3);
        if (on(s - 1))
          pv_at(bufp(std::integral_constant<int, B + 3>()) + KBY, kStepTokens * (s - 1), pHi, pLo);
        if (on(s)) scores_at(bufp(bc), S);
        middle(bc, id);
        if (on(s)) softmax(s, 0, S, pHi, pLo);
        direct_barrier<63>();
      });
    }
    wait_vm<0>();                                            // no load into LDS left in flight
    if (!lead && se > s0 && active(se - 1)) {
      const int bl = (se - 1 - s0) & 3;
      const uint8_t* vb = (bl == 0 ? db0 : bl == 1 ? db1 : bl == 2 ? db2 : db3) + KBY;
      pv_at(vb, kStepTokens * (se - 1), pHi, pLo);
    }
  } else if constexpr (W == 8) {
    // Ping-pong (four buffers, step s in buffer (s - s0) % 4).  Waves w and w + 4 share a
    // SIMD; the second group (waves 4-7) runs half a step behind the first, so that on every
    // SIMD one wave is in its softmax (vector ALU) while the other issues matrix products.
    // Iteration s, phase 1 -- first group: softmax(s); second: P.V(s - 1), scores(s).  Phase 2
    // -- first: P.V(s), scores(s + 1); second: softmax(s).  A barrier ends each phase.
    // Every second iteration (s - s0 even), phase 2 also stores steps s + 2 and s + 3 into the
    // buffers of s - 2 and s - 1 (their last reader, the second group's P.V(s - 1), ran in
    // phase 1) and loads steps s + 4 and s + 5 into the registers just stored.  A store waits
    // for every load issued before it (the compiler counts loop-carried loads conservatively),
    // so the loads get two iterations to land only if none is issued between them and their
    // store: storing one step per iteration, they had one (measured: with the stores and loads
    // skipped, 229 -> 187 us).
    static_assert(BUFS == 4, "the ping-pong schedule takes four buffers");

    const bool lead = wave < W / 2;
    auto buf_of = [&](int s) { return (s - s0) & 3; };
    fetch(s0, wa);
    fetch(s0 + 1, wb);
    if (s0 < se) stage(s0, 0, wa);
    if (s0 + 1 < se) stage(s0 + 1, 1, wb);
    fetch(s0 + 2, wa);
    fetch(s0 + 3, wb);
    __syncthreads();
    // The two groups run separate loops with the same barriers (two per step), so that each
    // keeps only its own registers live across them.
    f32x4 S[TPW][2];
    V8 pHi[TPW], pLo[TPW];
    int ids = ids_vec(s0 + 4);
    auto tail = [&](int s, bool store) {          // phase 2's stores and loads, its barrier
      if (store) {
        if (s + 2 < se) stage(s + 2, buf_of(s + 2), wa);
        if (s + 3 < se) stage(s + 3, buf_of(s + 3), wb);
        fetch_ids(ids_step(ids, 0), wa);
        fetch_ids(ids_step(ids, 1), wb);
        ids = ids_vec(s + 6);
      }
      __syncthreads();
    };
    if (lead) {
      if (s0 < se && active(s0)) scores(0, S);
      auto iteration = [&](int s, bool store) {
        if (active(s)) softmax(s, buf_of(s), S, pHi, pLo);
        __syncthreads();
        if (active(s)) pv(buf_of(s), pHi, pLo);
        if (s + 1 < se && active(s + 1)) scores(buf_of(s + 1), S);
        tail(s, store);
      };
      for (int s = s0; s < se;) {
        iteration(s, true);
        if (++s >= se) break;
        iteration(s, false);
        ++s;
      }
    } else {
      auto iteration = [&](int s, bool store) {
        if (s > s0 && active(s - 1)) pv(buf_of(s - 1), pHi, pLo);
        if (active(s)) scores(buf_of(s), S);
        __syncthreads();
        if (active(s)) softmax(s, buf_of(s), S, pHi, pLo);
        tail(s, store);
      };
      for (int s = s0; s < se;) {
        iteration(s, true);
        if (++s >= se) break;
        iteration(s, false);
        ++s;
      }
      if (se > s0 && active(se - 1)) pv(buf_of(se - 1), pHi, pLo);
    }
  } else if constexpr (BUFS == 3) {
    // Software pipeline (step s in buffer (s - s0) % 3): iteration s issues the score products
    // of step s + 1 before the softmax and P.V products of step s, so the matrix cores have
    // independent work while the softmax runs; it then stores step s + 2 into the buffer step
    // s - 1 has left and loads step s + 4 into the registers step s + 2 has left (two register
    // sets; the loop is unrolled by two so each keeps its registers).  A wave whose rows see
    // none of a step's keys skips its products.
    auto buf_of = [&](int s) { return (s - s0) % 3; };
    fetch(s0, wa);
    fetch(s0 + 1, wb);
    if (s0 < se) stage(s0, 0, wa);
    fetch(s0 + 2, wa);
    if (s0 + 1 < se) stage(s0 + 1, 1, wb);
    fetch(s0 + 3, wb);
    __syncthreads();
    f32x4 Sa[TPW][2], Sb[TPW][2];
    if (s0 < se && active(s0)) scores(0, Sa);
    // (the block ids stay scalar loads at their use here: read ahead by a vector load, their
    // wait drained every load in flight, 191 -> 234 us for 128-row heads)
    auto iteration = [&](int s, f32x4 (&Sc)[TPW][2], f32x4 (&Sn)[TPW][2], Words& w) {
      if (s + 1 < se && active(s + 1)) scores(buf_of(s + 1), Sn);
      if (active(s)) softmax_pv(s, buf_of(s), Sc);
      if (s + 2 < se) stage(s + 2, buf_of(s + 2), w);
      fetch(s + 4, w);
      __syncthreads();
    };
    for (int s = s0; s < se;) {
      iteration(s, Sa, Sb, wa);
      if (++s >= se) break;
      iteration(s, Sb, Sa, wb);
      ++s;
    }
  }

#pragma unroll
  for (int u = 0; u < TPW; ++u) {
    const float lsum = sum_across_rows(l_run[u]);
    if (!real[u]) continue;
    if (NP == 1) {
      // a row without keys (before the context) has l = 0 and acc = 0: output zeros
      const float l = lsum > 0.0f ? lsum : 1.0f;
      E* out = reinterpret_cast<E*>(a.out) + orow[u] * D + 4 * grp;
#pragma unroll
      for (int t = 0; t < NT; ++t)
        *reinterpret_cast<uint2*>(out + 16 * t) =
            make_uint2(pack2<QT>(acc[u][t][0] / l, acc[u][t][1] / l),
                       pack2<QT>(acc[u][t][2] / l, acc[u][t][3] / l));
    } else {
      const size_t pi = orow[u] * NP + part;
      if (grp == 0) {
        a.ws_ml[2 * pi] = m_run[u];
        a.ws_ml[2 * pi + 1] = lsum;
      }
#pragma unroll
      for (int t = 0; t < NT; ++t)
        *reinterpret_cast<f32x4*>(a.ws_acc + pi * D + 16 * t + 4 * grp) = acc[u][t];
    }
  }
}

template <int D, int QT, int KVT, int W, int TPW, int BUFS>
static hipError_t launch_chunk(const MultiArgs& a, hipStream_t stream) {
  const long long wgs = (a.total_items + 7) / 8 * 8;
  hipLaunchKernelGGL((chunk_kernel<D, QT, KVT, W, TPW, BUFS>), dim3((unsigned)wgs), dim3(64 * W),
                     0, stream, a);
  return hipGetLastError();
}

template <int D, int QT, int KVT>
static hipError_t launch_multi_t(const MultiArgs& a, hipStream_t stream) {
  if (a.row_blocks > 0) {   // with one key partition the chunk kernel writes the rows itself
    // the 16-bit ping-pong instance holds a partition's block ids in LDS
    if (a.chunk_waves == kChunkPingPong.waves && KVT != DT_FP8 && a.part_blocks > kDirectMaxBlocks)
      return hipErrorInvalidValue;
    const hipError_t e =
        a.chunk_waves == kChunkPingPong.waves
            ? launch_chunk<D, QT, KVT, kChunkPingPong.waves, kChunkPingPong.tiles, 4>(a, stream)
            : launch_chunk<D, QT, KVT, kChunkWide.waves, kChunkWide.tiles, 3>(a, stream);
    if (e != hipSuccess || a.num_parts <= 1) return e;
    return launch_merge<D, QT>(a, stream);
  }
  long long wgs = (a.total_items + kMultiWaves - 1) / kMultiWaves;
  wgs = (wgs + 7) / 8 * 8;
  if (wgs > 0) {
    hipLaunchKernelGGL((multi_kernel<D, QT, KVT>), dim3((unsigned)wgs), dim3(64 * kMultiWaves),
                       0, stream, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (a.num_parts > 1) return launch_merge<D, QT>(a, stream);
  return hipSuccess;
}

template <int D>
static hipError_t launch_multi_d(const MultiArgs& a, int q_dtype, int kv_dtype,
                                 hipStream_t stream) {
  if (q_dtype == DT_F16 && kv_dtype == DT_F16) return launch_multi_t<D, DT_F16, DT_F16>(a, stream);
  if (q_dtype == DT_BF16 && kv_dtype == DT_BF16)
    return launch_multi_t<D, DT_BF16, DT_BF16>(a, stream);
  if (q_dtype == DT_BF16 && kv_dtype == DT_FP8) return launch_multi_t<D, DT_BF16, DT_FP8>(a, stream);
  if (q_dtype == DT_F16 && kv_dtype == DT_FP8) return launch_multi_t<D, DT_F16, DT_FP8>(a, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_multi(const MultiArgs& a, int head_dim, int q_dtype, int kv_dtype,
                        hipStream_t stream) {
  if (head_dim == 64) return launch_multi_d<64>(a, q_dtype, kv_dtype, stream);
  if (head_dim == 128) return launch_multi_d<128>(a, q_dtype, kv_dtype, stream);
  return hipErrorInvalidValue;
}

}  // namespace pa
