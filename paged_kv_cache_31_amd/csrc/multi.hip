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
// loads are therefore cached, not streamed.  Long contexts with few rows (speculative
// verification) are split into key partitions whose partial results (running max, exp-sum,
// unnormalised output) go to the workspace and are merged by log-sum-exp in a second kernel;
// with one partition the kernel normalises and writes the output itself.
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
    st.walk_rows(qB, a.block_tables + (size_t)b * a.max_blocks_per_seq, kvh, j0, j1, end_lane,
                 end_lo, end_hi, m_run, l_run, acc);
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

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

// One wave per (sequence b, query token i, query head h): merges the num_parts partial results
// of that row by log-sum-exp and writes the normalised output.  Every partition of a row's tile
// was written by multi_kernel (an empty one as max -inf, sum 0, output 0).
template <int D, int QT>
__global__ __launch_bounds__(256) void multi_merge_kernel(MultiArgs a) {
  typedef typename Mfma<QT>::elem E;
  constexpr int DPL = D / 64;                          // dims per lane
  const int lane = threadIdx.x & 63;
  const long long w = (long long)blockIdx.x * 4 + uniform(threadIdx.x >> 6);
  const int Hq = a.num_q_heads;
  const long long per_seq = (long long)a.max_query_len * Hq;
  if (w >= (long long)a.batch * per_seq) return;
  const int b = (int)(w / per_seq);
  const int rem = (int)(w - (long long)b * per_seq);
  const int i = rem / Hq, h = rem - i * Hq;
  const int q0 = a.query_start[b];
  const int T = min(max(a.query_start[b + 1] - q0, 0), a.max_query_len);
  if (i >= T) return;
  const long long n = (long long)q0 + i;
  if (n < 0 || n >= a.total_queries) return;
  const size_t row = (size_t)n * Hq + h;
  const int NP = a.num_parts;
  const float* ml = a.ws_ml + row * NP * 2;
  const float* pacc = a.ws_acc + row * NP * D;

  float M = -INFINITY;
  for (int p = lane; p < NP; p += 64) M = fmaxf(M, ml[2 * p]);
  M = wave_max(M);
  float o[DPL];
#pragma unroll
  for (int k = 0; k < DPL; ++k) o[k] = 0.0f;
  float den = 1.0f;
  if (M != -INFINITY) {
    float s = 0.0f;
    for (int p = lane; p < NP; p += 64) s += fast_exp2(ml[2 * p] - M) * ml[2 * p + 1];
    den = wave_sum(s);
    for (int p = 0; p < NP; ++p) {
      const float wt = fast_exp2(ml[2 * p] - M);
      if (wt == 0.0f) continue;                        // partitions without keys
#pragma unroll
      for (int k = 0; k < DPL; ++k) o[k] += wt * pacc[(size_t)p * D + lane * DPL + k];
    }
  }
  E* out = reinterpret_cast<E*>(a.out) + row * D + lane * DPL;
  if constexpr (DPL == 2) {
    *reinterpret_cast<uint32_t*>(out) = pack2<QT>(o[0] / den, o[1] / den);
  } else {
    out[0] = (E)(o[0] / den);
  }
}

template <int D, int QT, int KVT>
static hipError_t launch_multi_t(const MultiArgs& a, hipStream_t stream) {
  long long wgs = (a.total_items + kMultiWaves - 1) / kMultiWaves;
  wgs = (wgs + 7) / 8 * 8;
  if (wgs > 0) {
    hipLaunchKernelGGL((multi_kernel<D, QT, KVT>), dim3((unsigned)wgs), dim3(64 * kMultiWaves),
                       0, stream, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (a.num_parts > 1) {
    const long long waves = (long long)a.batch * a.max_query_len * a.num_q_heads;
    const long long mwgs = (waves + 3) / 4;
    if (mwgs > 0) {
      hipLaunchKernelGGL((multi_merge_kernel<D, QT>), dim3((unsigned)mwgs), dim3(256), 0, stream,
                         a);
      return hipGetLastError();
    }
  }
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
