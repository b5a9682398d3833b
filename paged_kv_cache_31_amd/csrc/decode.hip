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
// keeping enough 16-byte loads in flight.  The matrix cores are used because they make the
// arithmetic nearly free, not because the work is a large GEMM: one 16x16x32 MFMA covers 16
// tokens x 32 dims for up to 16 query heads of a group, so the vector ALUs are left with the
// softmax only.
//
//  * Workgroup = 4 waves = one (key partition, KV head, sequence).  The partition's tokens are cut
//    into 32-token steps (two blocks); wave w takes steps w, w+4, ...  Partials of the 4 waves are
//    merged through LDS; partials of several partitions go to the workspace and are merged by
//    log-sum-exp in merge_kernel.  Reduction order depends only on logical token positions.
//  * QK: S^T = K . Q^T.  The K tile (token-major) is loaded straight into the MFMA A operand:
//    lane (row r = lane%16, group g = lane/16) reads 16 contiguous bytes of token row r, so each
//    instruction fetches 64 contiguous bytes of 16 token rows.  Rows of the two MFMAs of a step are
//    assigned so that the result layout (lane holds head lane%16, rows 4g..4g+3) is directly the
//    B operand of the P.V product -- no shuffles between QK and PV.
//  * PV: O^T = V^T . P^T.  V tiles are stored dim-major ([d][16 tokens]), so the A operand (row d,
//    8 consecutive tokens) is one 16-byte load and an instruction fetches 2 x 512 contiguous bytes.
//    P is fed as a bf16 hi/lo pair (two MFMAs) so the weights keep ~16 significant bits; fp16 P is
//    used as is.
//  * fp8 (OCP e4m3fn) tiles are widened exactly to the MFMA type in registers; the K block scale
//    multiplies the scores and the V block scale the weights.
//  * Double-buffered steps: the loads of step s+4 are issued before step s is computed.
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

template <int D, int QT, int KVT>
__global__ __launch_bounds__(256, 2) void decode_partition_kernel(DecodeArgs a) {
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

  __shared__ int sm_tab[kMaxPartition / kBlock];
  __shared__ float sm_m[kWaves][16];
  __shared__ float sm_l[kWaves][16];
  __shared__ f32x4 sm_acc[kWaves][NT][64];

  const int p = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
  const int col = lane & 15, grp = lane >> 4;
  const int G = a.group, Hq = a.num_q_heads, Hkv = a.num_kv_heads;
  const int h0 = kvh * G;

  int L = a.context_lens[b];
  L = L < 0 ? 0 : (L > a.len_cap ? a.len_cap : L);
  const int P = a.partition;
  const int start = p * P;
  if (L == 0) {
    // No tokens: the output is defined as zeros (written once, by partition 0).
    if (p == 0) {
      E* o = reinterpret_cast<E*>(a.out) + ((size_t)b * Hq + h0) * D;
      for (int e = tid; e < G * D; e += blockDim.x) o[e] = (E)0.0f;
    }
    return;
  }
  if (start >= L) return;
  const int end = min(start + P, L);
  const int np_b = (L + P - 1) / P;
  const int nsteps = (end - start + kStepTokens - 1) / kStepTokens;
  const int nblk_seq = (L + kBlock - 1) / kBlock;
  const int blk0 = start / kBlock;

  // Stage this partition's block ids in LDS.  Entries past the sequence's last block (the second
  // block of a final half-step) reuse the partition's first block, so no unread table entry is
  // ever dereferenced; ids outside the pool read block 0.
  const int32_t* trow = a.block_tables + (size_t)b * a.max_blocks_per_seq;
  for (int e = tid; e < 2 * nsteps; e += blockDim.x) {
    const int lb = blk0 + e;
    const int id = trow[lb < nblk_seq ? lb : blk0];
    sm_tab[e] = (unsigned)id < (unsigned)a.num_blocks ? id : 0;
  }

  // Q^T as the B operand of the QK product: lane (head col, group grp) holds 8 dims per chunk.
  // fp8 tiles pair chunks (2c, 2c+1) in one 16-byte load, which permutes which dims a lane holds
  // for each chunk; Q is loaded with the same permutation.
  V8 qB[NC];
  {
    const E* qrow = reinterpret_cast<const E*>(a.q) + ((size_t)b * Hq + h0 + col) * D;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int d0 = FP8 ? 64 * (c >> 1) + 16 * grp + 8 * (c & 1) : 32 * c + 8 * grp;
      qB[c] = col < G ? as_vec8<V8>(*reinterpret_cast<const uint4*>(qrow + d0)) : zero_vec8<V8>();
    }
  }
  __syncthreads();

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

  float m_run = -INFINITY, l_run = 0.0f;
  f32x4 acc[NT];
#pragma unroll
  for (int i = 0; i < NT; ++i) acc[i] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  auto issue = [&](StepRegs<D, FP8>& r, int s) {
    const int pb0 = sm_tab[2 * s], pb1 = sm_tab[2 * s + 1];
    const int kb = k_hi ? pb1 : pb0;
    const int vb = v_hi ? pb1 : pb0;
    const uint8_t* kp = kc + ((size_t)kb * Hkv + kvh) * TILE + k_lane_off;
    const uint8_t* vp = vc + ((size_t)vb * Hkv + kvh) * TILE + v_lane_off;
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int c = 0; c < KL; ++c)
        r.k[m][c] = *reinterpret_cast<const uint4*>(kp + m * 4 * D * EB + c * 64);
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      if constexpr (FP8)
        r.v[i] = *reinterpret_cast<const uint2*>(vp + i * 16 * kBlock * EB);
      else
        r.v[i] = *reinterpret_cast<const uint4*>(vp + i * 16 * kBlock * EB);
    }
    if constexpr (FP8) {
      r.ks = a.k_scale[(size_t)vb * Hkv + kvh];
      r.vs = a.v_scale[(size_t)vb * Hkv + kvh];
    }
  };

  auto compute = [&](StepRegs<D, FP8>& r, int s) {
    const int t0 = start + kStepTokens * s;
    const int tb = t0 + tb_lane;
    const bool partial = t0 + kStepTokens > L;     // wave-uniform

    // scores of 8 tokens (tb + j) for head col
    f32x4 S[2];
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      S[m] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        V8 kA;
        if constexpr (FP8) {
          const uint4 w = r.k[m][c >> 1];
          kA = (c & 1) ? fp8x8_to_vec8<QT>(w.z, w.w) : fp8x8_to_vec8<QT>(w.x, w.y);
        } else {
          kA = as_vec8<V8>(r.k[m][c]);
        }
        S[m] = M::mma(kA, qB[c], S[m]);
      }
    }
    float qs = a.qk_scale_log2;
    if constexpr (FP8) qs *= r.ks;
    float sc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) sc[j] = S[j >> 2][j & 3] * qs;
    int nval = 8;
    if (partial) {
      nval = min(max(L - tb, 0), 8);
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (j >= nval) sc[j] = -INFINITY;
    }
    float mx = sc[0];
#pragma unroll
    for (int j = 1; j < 8; ++j) mx = fmaxf(mx, sc[j]);
    mx = max_across_rows(mx);
    const float m_new = fmaxf(m_run, mx);
    const float alpha = fast_exp2(m_run - m_new);
    float pr[8], psum = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      pr[j] = fast_exp2(sc[j] - m_new);
      psum += pr[j];
    }
    l_run = l_run * alpha + psum;
    m_run = m_new;
#pragma unroll
    for (int i = 0; i < NT; ++i) acc[i] *= alpha;
    if constexpr (FP8) {
#pragma unroll
      for (int j = 0; j < 8; ++j) pr[j] *= r.vs;
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

    // Masked tokens contribute weight 0, but their cache slots may hold anything (NaN
    // included), so their V elements are zeroed before the product.
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
    // Steps of this wave: wave, wave+4, ...  The steady-state loop issues the next step's loads
    // unconditionally (the tail is peeled), so the loads of step s+4 stay in flight while step s
    // is computed.
    StepRegs<D, FP8> r0, r1;
    int s = wave;
    if (s < nsteps) {
      int rest = (nsteps - 1 - s) / kWaves;   // steps after the first one
      issue(r0, s);
      for (; rest >= 2; rest -= 2, s += 2 * kWaves) {
        issue(r1, s + kWaves);
        compute(r0, s);
        issue(r0, s + 2 * kWaves);
        compute(r1, s + kWaves);
      }
      if (rest == 1) {
        issue(r1, s + kWaves);
        compute(r0, s);
        compute(r1, s + kWaves);
      } else {
        compute(r0, s);
      }
    }
  }

  // Merge the four waves' partials of this partition.
  l_run = sum_across_rows(l_run);
  if (grp == 0) {
    sm_m[wave][col] = m_run;
    sm_l[wave][col] = l_run;
  }
#pragma unroll
  for (int i = 0; i < NT; ++i) sm_acc[wave][i][lane] = acc[i];
  __syncthreads();

  float wgt[kWaves], M_ = -INFINITY;
#pragma unroll
  for (int v = 0; v < kWaves; ++v) {
    wgt[v] = sm_m[v][col];
    M_ = fmaxf(M_, wgt[v]);
  }
  float Ls = 0.0f;
#pragma unroll
  for (int v = 0; v < kWaves; ++v) {
    wgt[v] = wgt[v] == -INFINITY ? 0.0f : fast_exp2(wgt[v] - M_);
    Ls += wgt[v] * sm_l[v][col];
  }
  const int h = h0 + col;
  for (int i = wave; i < NT; i += kWaves) {
    f32x4 o = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int v = 0; v < kWaves; ++v) o += wgt[v] * sm_acc[v][i][lane];
    if (col < G) {
      const int d = 16 * i + 4 * grp;
      if (np_b == 1) {
        E* out = reinterpret_cast<E*>(a.out) + ((size_t)b * Hq + h) * D + d;
        *reinterpret_cast<uint2*>(out) =
            make_uint2(pack2<QT>(o[0] / Ls, o[1] / Ls), pack2<QT>(o[2] / Ls, o[3] / Ls));
      } else {
        float* w = a.ws_acc + (((size_t)b * Hq + h) * a.np_max + p) * D + d;
        *reinterpret_cast<f32x4*>(w) = o;
      }
    }
  }
  if (np_b > 1 && wave == 0 && grp == 0 && col < G) {
    float* ml = a.ws_ml + (((size_t)b * Hq + h) * a.np_max + p) * 2;
    ml[0] = M_;
    ml[1] = Ls;
  }
}

// Log-sum-exp merge of the key partitions of one (sequence, query head):
//   out = sum_j 2^(m_j - M) acc_j / sum_j 2^(m_j - M) l_j,  M = max_j m_j  (m in log2 units).
template <int D, int QT>
__global__ __launch_bounds__(64) void merge_kernel(DecodeArgs a) {
  typedef typename Mfma<QT>::elem E;
  constexpr int PER = D / 64;
  const int h = blockIdx.x, b = blockIdx.y, lane = threadIdx.x;
  int L = a.context_lens[b];
  L = L < 0 ? 0 : (L > a.len_cap ? a.len_cap : L);
  const int P = a.partition;
  if (L <= P) return;   // a single partition wrote its output directly
  const int np = (L + P - 1) / P;
  const size_t row = ((size_t)b * a.num_q_heads + h) * a.np_max;
  float M_ = -INFINITY;
  for (int j = 0; j < np; ++j) M_ = fmaxf(M_, a.ws_ml[(row + j) * 2]);
  float o[PER], Ls = 0.0f;
#pragma unroll
  for (int e = 0; e < PER; ++e) o[e] = 0.0f;
  for (int j = 0; j < np; ++j) {
    const float w = fast_exp2(a.ws_ml[(row + j) * 2] - M_);
    Ls += w * a.ws_ml[(row + j) * 2 + 1];
    const float* src = a.ws_acc + (row + j) * D + lane * PER;
#pragma unroll
    for (int e = 0; e < PER; ++e) o[e] += w * src[e];
  }
  E* out = reinterpret_cast<E*>(a.out) + ((size_t)b * a.num_q_heads + h) * D + lane * PER;
#pragma unroll
  for (int e = 0; e < PER; ++e) out[e] = (E)(o[e] / Ls);
}

template <int D, int QT, int KVT>
static hipError_t launch_t(const DecodeArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL((decode_partition_kernel<D, QT, KVT>),
                     dim3(a.np_max, a.num_kv_heads, a.batch), dim3(64 * kWaves), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.np_max == 1) return e;
  hipLaunchKernelGGL((merge_kernel<D, QT>), dim3(a.num_q_heads, a.batch), dim3(64), 0, stream, a);
  return hipGetLastError();
}

template <int D>
static hipError_t launch_d(const DecodeArgs& a, int q_dtype, int kv_dtype, hipStream_t stream) {
  if (q_dtype == DT_F16 && kv_dtype == DT_F16) return launch_t<D, DT_F16, DT_F16>(a, stream);
  if (q_dtype == DT_BF16 && kv_dtype == DT_BF16) return launch_t<D, DT_BF16, DT_BF16>(a, stream);
  if (q_dtype == DT_BF16 && kv_dtype == DT_FP8) return launch_t<D, DT_BF16, DT_FP8>(a, stream);
  if (q_dtype == DT_F16 && kv_dtype == DT_FP8) return launch_t<D, DT_F16, DT_FP8>(a, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_decode(const DecodeArgs& a, int head_dim, int q_dtype, int kv_dtype,
                         hipStream_t stream) {
  if (head_dim == 64) return launch_d<64>(a, q_dtype, kv_dtype, stream);
  if (head_dim == 128) return launch_d<128>(a, q_dtype, kv_dtype, stream);
  return hipErrorInvalidValue;
}

}  // namespace pa
