// The K/V streaming core of the attention kernels: block-table walk, MFMA products and online
// softmax for one wave, shared by decode_kernel, prefix_kernel and multi_kernel.
#pragma once

#include "device_common.hpp"
#include "pa_internal.hpp"

namespace pa {

template <int D, bool FP8> struct StepRegs;
template <int D> struct StepRegs<D, false> {
  uint4 k[2][D / 32];   // per 16-token row set m: one 16-byte load per 32-dim chunk
  uint4 v[D / 16];      // per 16-dim tile: 8 tokens x 16-bit
  int pb0, pb1;         // physical blocks of the step
};
template <int D> struct StepRegs<D, true> {
  uint4 k[2][D / 64];   // one 16-byte load covers two 32-dim chunks of 8 codes
  uint2 v[D / 16];      // 8 tokens x 1 byte
  float ks, vs;         // block scales of this lane's block
  int pb0, pb1;
};

// A token appended by the launch that reads its block (no other wave reads that block in the
// launch).  Its V element is written into the wave's registers of the block's V tile, which is
// then stored back whole: a dim-major tile holds one element of a token per 16-token row, so
// storing the element alone would leave every cache line of the tile partly written, and later
// reads of partly written lines were measured to be far slower than of whole ones.
struct VAppend {
  const uint8_t* vnew = nullptr;   // the head's new V row (head_dim elements); nullptr: none
  int blk = -1;                    // logical block of the new token
  int off = 0;                     // its slot in the block
};

// Pacing hook of the walk, called with a step's first logical block before its loads are
// issued (the default does nothing).
struct NoPace {
  __device__ __forceinline__ void operator()(int) const {}
};

template <typename V8>
__device__ __forceinline__ V8 zero_vec8() {
  return __builtin_bit_cast(V8, make_uint4(0u, 0u, 0u, 0u));
}

// Two floats rounded (to nearest even) to the 16-bit element type, x in the low half: one
// packed conversion (two scalar ones and the packing cost five instructions).
template <int QT>
__device__ __forceinline__ uint32_t pack2(float x, float y) {
  typedef typename Mfma<QT>::elem E;
  typedef E E2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{x, y}, E2));
}

// The low part of a bf16 hi/lo pair: hi = pack2(x, y), and x - hi, y - hi rounded again, so
// that hi + lo carries about 16 significant bits of each weight.
__device__ __forceinline__ uint32_t bf16_lo2(float x, float y, uint32_t hi) {
  return pack2<DT_BF16>(x - __builtin_bit_cast(float, hi << 16),
                        y - __builtin_bit_cast(float, hi & 0xFFFF0000u));
}

__device__ __forceinline__ int clamp_len(int L, int cap) { return L < 0 ? 0 : (L > cap ? cap : L); }
__device__ __forceinline__ int blocks_of(int L) { return (L + kBlock - 1) / kBlock; }
__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

// The streaming core shared by decode_kernel, prefix_kernel and multi_kernel: one wave, one
// query column per lane column (lane%16), online softmax over a range of logical blocks of one
// table row.  K/V loads are non-temporal (STREAM) where each byte is read once per launch, and
// cached where several workgroups read the same blocks.  ROWS: each column has its own causal
// window (walk_rows), so a column may see no key at all in a range.
template <int D, int QT, int KVT, bool STREAM = true, bool ROWS = false>
struct Stepper {
  typedef Mfma<QT> M;
  typedef typename M::vec8 V8;
  typedef typename M::elem E;
  static constexpr bool FP8 = KVT == DT_FP8;
  static constexpr bool SPLIT_P = QT == DT_BF16;
  static constexpr int EB = FP8 ? 1 : 2;          // bytes per cache element
  static constexpr int NC = D / 32;               // 32-dim chunks (QK)
  static constexpr int NT = D / 16;               // 16-dim tiles (PV)
  static constexpr int KL = FP8 ? NC / 2 : NC;    // K loads per row set
  static constexpr int TILE = kBlock * D * EB;    // bytes of one (block, kv head) tile

  const uint8_t* kc;
  const uint8_t* vc;
  const float* ksc;
  const float* vsc;
  int Hkv, num_blocks;
  float qk_scale_log2;
  int col, grp, k_lane_off, v_lane_off, tb_lane;
  bool k_hi, v_hi;

  template <class Args>
  __device__ __forceinline__ Stepper(const Args& a, int lane)
      : kc(reinterpret_cast<const uint8_t*>(a.k_cache)),
        vc(reinterpret_cast<const uint8_t*>(a.v_cache)),
        ksc(a.k_scale), vsc(a.v_scale), Hkv(a.num_kv_heads), num_blocks(a.num_blocks),
        qk_scale_log2(a.qk_scale_log2) {
    col = lane & 15;
    grp = lane >> 4;
    // K row r = col of MFMA m holds token 16*(r/8) + 8*((r/4)%2) + 4*m + r%4 of the step; its
    // block is r/8.  Result row 4*grp+i of MFMA m is then token tb + 4*m + i with
    // tb = 16*(grp/2) + 8*(grp%2), which is exactly the token order the PV operands use.
    k_lane_off = (8 * ((col >> 2) & 1) + (col & 3)) * D * EB + 16 * grp;
    v_lane_off = (col * kBlock + 8 * (grp & 1)) * EB;
    k_hi = col >= 8;
    v_hi = grp >= 2;
    tb_lane = 16 * (grp >> 1) + 8 * (grp & 1);
  }

  static __device__ __forceinline__ uint4 load16(const uint8_t* p) {
    if constexpr (STREAM) return load_stream16(p);
    else return *reinterpret_cast<const uint4*>(p);
  }
  static __device__ __forceinline__ uint2 load8(const uint8_t* p) {
    if constexpr (STREAM) return load_stream8(p);
    else return *reinterpret_cast<const uint2*>(p);
  }

  // Q^T as the B operand of the QK product for this lane's query row (nullptr: zeros).  Lane
  // (column col, group grp) holds 8 dims per chunk; fp8 tiles pair chunks (2c, 2c+1) in one
  // 16-byte load, which permutes which dims a lane holds for each chunk, and Q follows suit.
  __device__ __forceinline__ void load_q(V8 (&qB)[NC], const E* qrow) const {
#pragma unroll
    for (int cc = 0; cc < NC; ++cc) {
      const int d0 = FP8 ? 64 * (cc >> 1) + 16 * grp + 8 * (cc & 1) : 32 * cc + 8 * grp;
      qB[cc] = qrow ? as_vec8<V8>(*reinterpret_cast<const uint4*>(qrow + d0)) : zero_vec8<V8>();
    }
  }

  // The single-tile form of the walk's per-tile arguments (copies the compiler keeps in the
  // same registers).
  struct Tile1 {
    V8 q[1][NC];
    int e[1];
    float m[1], l[1];
    f32x4 acc[1][NT];
    __device__ __forceinline__ Tile1(const V8 (&qB)[NC], int end, float m0, float l0,
                                     const f32x4 (&a0)[NT]) {
#pragma unroll
      for (int c = 0; c < NC; ++c) q[0][c] = qB[c];
      e[0] = end;
      m[0] = m0;
      l[0] = l0;
#pragma unroll
      for (int i = 0; i < NT; ++i) acc[0][i] = a0[i];
    }
    __device__ __forceinline__ void back(float& m0, float& l0, f32x4 (&a0)[NT]) const {
      m0 = m[0];
      l0 = l[0];
#pragma unroll
      for (int i = 0; i < NT; ++i) a0[i] = acc[0][i];
    }
  };

  // Online-softmax attention over logical blocks [j0, j1) of table row trow for KV head kvh
  // (tokens at or past end_tok are masked), taking the steps s_first, s_first + stride, ... of
  // the range, into the running (m_run, l_run, acc).
  // wait_stores: this wave's earlier stores write a block the run reads in its last step.  The
  // loads of a run's third and later steps are issued after the first step's wait on the memory
  // counter, which in-order completion makes cover those older stores; a run of one or two
  // steps waits for them explicitly before its first load.
  __device__ __forceinline__ void run(const V8 (&qB)[NC], const int32_t* trow, int kvh, int j0,
                                      int j1, int end_tok, int s_first, int stride,
                                      float& m_run, float& l_run, f32x4 (&acc)[NT],
                                      bool wait_stores = false) const {
    Tile1 t(qB, end_tok, m_run, l_run, acc);
    walk<false, 1>(t.q, trow, kvh, j0, j1, t.e, end_tok, end_tok, s_first, stride, t.m, t.l,
                   t.acc, wait_stores, VAppend());
    t.back(m_run, l_run, acc);
  }
  // The same with a token appended to one of the range's blocks (a separate instance, so that
  // the plain loop carries none of the append's registers).
  __device__ __forceinline__ void run_append(const V8 (&qB)[NC], const int32_t* trow, int kvh,
                                             int j0, int j1, int end_tok, float& m_run,
                                             float& l_run, f32x4 (&acc)[NT], bool wait_stores,
                                             VAppend ap) const {
    Tile1 t(qB, end_tok, m_run, l_run, acc);
    walk<true, 1>(t.q, trow, kvh, j0, j1, t.e, end_tok, end_tok, 0, 1, t.m, t.l, t.acc,
                  wait_stores, ap);
    t.back(m_run, l_run, acc);
  }

  // The same walk with a window per query column: this lane's column sees tokens below
  // end_lane; end_lo (wave-uniform) is the smallest such end over the wave's columns and end_v
  // (wave-uniform) the largest, past which V slots may hold anything.
  __device__ __forceinline__ void walk_rows(const V8 (&qB)[NC], const int32_t* trow, int kvh,
                                            int j0, int j1, int end_lane, int end_lo, int end_v,
                                            float& m_run, float& l_run,
                                            f32x4 (&acc)[NT]) const {
    Tile1 t(qB, end_lane, m_run, l_run, acc);
    walk<false, 1>(t.q, trow, kvh, j0, j1, t.e, end_lo, end_v, 0, 1, t.m, t.l, t.acc, false,
                   VAppend());
    t.back(m_run, l_run, acc);
  }
  // Several column tiles per wave: tile u's columns take qB[u] and their windows end_lane[u];
  // every K/V step is loaded once and multiplied into all MT tiles.  end_lo and end_v bound the
  // windows of all tiles.
  // ROLL: one register set instead of two; the next step's K is loaded as soon as this step's
  // scores are taken, its V as soon as this step's P.V is done (16-bit K/V, no append).
  template <int MT, class Pace = NoPace, bool ROLL = false>
  __device__ __forceinline__ void walk_tiles(const V8 (&qB)[MT][NC], const int32_t* trow,
                                             int kvh, int j0, int j1, const int (&end_lane)[MT],
                                             int end_lo, int end_v, float (&m_run)[MT],
                                             float (&l_run)[MT], f32x4 (&acc)[MT][NT],
                                             Pace pace = Pace()) const {
    walk<false, MT, Pace, ROLL>(qB, trow, kvh, j0, j1, end_lane, end_lo, end_v, 0, 1, m_run,
                                l_run, acc, false, VAppend(), pace);
  }

  template <bool APP, int MT, class Pace = NoPace, bool ROLL = false>
  __device__ __forceinline__ void walk(const V8 (&qB)[MT][NC], const int32_t* trow, int kvh,
                                       int j0, int j1, const int (&end_tok)[MT], int end_lo,
                                       int end_v, int s_first, int stride, float (&m_run)[MT],
                                       float (&l_run)[MT], f32x4 (&acc)[MT][NT],
                                       bool wait_stores, VAppend ap, Pace pace = Pace()) const {
    static_assert(!APP || MT == 1, "the append instance takes one tile");
    static_assert(!ROLL || (!APP && !FP8), "the rolling schedule takes 16-bit K/V, no append");
    const int nsteps = (j1 - j0 + 1) >> 1;
    if (s_first >= nsteps) return;

    // Block ids of a step: logical blocks j0+2s and j0+2s+1 (the second one repeats the first
    // when the range ends after one block; its tokens are masked).  Ids outside the pool read
    // block 0.
    auto ids_of = [&](int s, int& p0, int& p1) {
      s = min(s, nsteps - 1);
      const int jb = j0 + 2 * s;
      const int jb1 = jb + 1 < j1 ? jb + 1 : jb;
      const int i0 = trow[jb], i1 = trow[jb1];
      p0 = (unsigned)i0 < (unsigned)num_blocks ? i0 : 0;
      p1 = (unsigned)i1 < (unsigned)num_blocks ? i1 : 0;
    };
    int nid0, nid1;
    ids_of(s_first, nid0, nid1);
    if (wait_stores && nsteps - s_first <= 2 * stride) wait_memory_ops();

    // the appended token's V element for each of this lane's 16-dim tiles (dim 16i + col),
    // packed PK to a register
    constexpr int PK = FP8 ? 4 : 2;
    uint32_t vn[(NT + PK - 1) / PK];
    if constexpr (APP) {
#pragma unroll
      for (int i = 0; i < (NT + PK - 1) / PK; ++i) vn[i] = 0u;
#pragma unroll
      for (int i = 0; i < NT; ++i)
        vn[i / PK] |= (FP8 ? (uint32_t)ap.vnew[16 * i + col]
                           : (uint32_t)reinterpret_cast<const uint16_t*>(ap.vnew)[16 * i + col])
                      << (32 / PK * (i % PK));
    }

    auto issue = [&](StepRegs<D, FP8>& r, int s) {
      pace(j0 + 2 * min(s, nsteps - 1));
      const int pb0 = nid0, pb1 = nid1;
      if constexpr (APP) {
        r.pb0 = pb0;
        r.pb1 = pb1;
      }
      ids_of(s + stride, nid0, nid1);              // prefetch the next step's block ids
      const int kb = k_hi ? pb1 : pb0;
      const int vb = v_hi ? pb1 : pb0;
      const uint8_t* kp = kc + ((size_t)kb * Hkv + kvh) * TILE + k_lane_off;
      const uint8_t* vp = vc + ((size_t)vb * Hkv + kvh) * TILE + v_lane_off;
#pragma unroll
      for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int cc = 0; cc < KL; ++cc) r.k[m][cc] = load16(kp + m * 4 * D * EB + cc * 64);
#pragma unroll
      for (int i = 0; i < NT; ++i) {
        if constexpr (FP8)
          r.v[i] = load8(vp + i * 16 * kBlock * EB);
        else
          r.v[i] = load16(vp + i * 16 * kBlock * EB);
      }
      if constexpr (FP8) {
        r.ks = ksc[(size_t)vb * Hkv + kvh];
        r.vs = vsc[(size_t)vb * Hkv + kvh];
      }
    };

    // the rolling schedule's halves of issue(): K with the pacing and the id prefetch, then V
    const uint8_t* roll_vp = nullptr;
    auto issue_k = [&](StepRegs<D, FP8>& r, int s) {
      pace(j0 + 2 * min(s, nsteps - 1));
      const int pb0 = nid0, pb1 = nid1;
      ids_of(s + stride, nid0, nid1);
      const int kb = k_hi ? pb1 : pb0;
      const int vb = v_hi ? pb1 : pb0;
      const uint8_t* kp = kc + ((size_t)kb * Hkv + kvh) * TILE + k_lane_off;
      roll_vp = vc + ((size_t)vb * Hkv + kvh) * TILE + v_lane_off;
#pragma unroll
      for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int cc = 0; cc < KL; ++cc) r.k[m][cc] = load16(kp + m * 4 * D * EB + cc * 64);
    };
    auto issue_v = [&](StepRegs<D, FP8>& r) {
#pragma unroll
      for (int i = 0; i < NT; ++i) {
        if constexpr (FP8)
          r.v[i] = load8(roll_vp + i * 16 * kBlock * EB);
        else
          r.v[i] = load16(roll_vp + i * 16 * kBlock * EB);
      }
    };

    // nxt >= 0 (rolling schedule only): the step whose loads go into r's registers as they free
    auto compute = [&](StepRegs<D, FP8>& r, int s, int nxt) {
      const int t0 = kBlock * (j0 + 2 * s);
      const int tb = t0 + tb_lane;
      const bool partial = t0 + kStepTokens > (ROWS ? end_lo : end_tok[0]);   // wave-uniform

      // the appended token: into the registers of its block's V tile, then the tile back whole
      if constexpr (APP) {
        const int bj = ap.blk - (j0 + 2 * s);                          // wave-uniform
        if (bj == 0 || bj == 1) {
          const bool mine = (grp >> 1) == bj;
          if (mine && (grp & 1) == (ap.off >> 3)) {
            const int e = ap.off & 7;
#pragma unroll
            for (int i = 0; i < NT; ++i) {
              const uint32_t val = (vn[i / PK] >> (32 / PK * (i % PK))) & (FP8 ? 0xFFu : 0xFFFFu);
              if constexpr (FP8) {
                const int sh = 8 * (e & 3);
                const uint32_t m8 = ~(0xFFu << sh), b8 = val << sh;
                if (e < 4) r.v[i].x = (r.v[i].x & m8) | b8;
                else r.v[i].y = (r.v[i].y & m8) | b8;
              } else {
                const int sh = 16 * (e & 1);
                const uint32_t m16 = ~(0xFFFFu << sh), b16 = val << sh;
                if ((e >> 1) == 0) r.v[i].x = (r.v[i].x & m16) | b16;
                else if ((e >> 1) == 1) r.v[i].y = (r.v[i].y & m16) | b16;
                else if ((e >> 1) == 2) r.v[i].z = (r.v[i].z & m16) | b16;
                else r.v[i].w = (r.v[i].w & m16) | b16;
              }
            }
          }
          if (mine) {
            uint8_t* vp = const_cast<uint8_t*>(vc) +
                          ((size_t)(bj ? r.pb1 : r.pb0) * Hkv + kvh) * TILE + v_lane_off;
#pragma unroll
            for (int i = 0; i < NT; ++i) {
              if constexpr (FP8)
                *reinterpret_cast<uint2*>(vp + i * 16 * kBlock * EB) = r.v[i];
              else
                *reinterpret_cast<uint4*>(vp + i * 16 * kBlock * EB) = r.v[i];
            }
          }
        }
      }

      // scores of 8 tokens (tb + jj) for column col of every tile; each K operand is widened
      // once and multiplied into all tiles
      f32x4 S[MT][2];
#pragma unroll
      for (int m = 0; m < 2; ++m) {
#pragma unroll
        for (int u = 0; u < MT; ++u) S[u][m] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int cc = 0; cc < NC; ++cc) {
          V8 kA;
          if constexpr (FP8) {
            const uint4 w = r.k[m][cc >> 1];
            kA = (cc & 1) ? fp8x8_to_vec8<QT>(w.z, w.w) : fp8x8_to_vec8<QT>(w.x, w.y);
          } else {
            kA = as_vec8<V8>(r.k[m][cc]);
          }
#pragma unroll
          for (int u = 0; u < MT; ++u) S[u][m] = M::mma(kA, qB[u][cc], S[u][m]);
        }
      }
      if constexpr (ROLL) {
        if (nxt >= 0) issue_k(r, nxt);
      }
      float qs = qk_scale_log2;
      if constexpr (FP8) qs *= r.ks;

      // per tile: online softmax, rescale, and P^T as the B operand (this lane's 8 weights in
      // token order; bf16 P as a hi/lo pair)
      V8 pHi[MT], pLo[MT];
#pragma unroll
      for (int u = 0; u < MT; ++u) {
        float sc[8];
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) sc[jj] = S[u][jj >> 2][jj & 3] * qs;
        if (partial) {
          const int nval = min(max(end_tok[u] - tb, 0), 8);
#pragma unroll
          for (int jj = 0; jj < 8; ++jj)
            if (jj >= nval) sc[jj] = -INFINITY;
        }
        float mx = sc[0];
#pragma unroll
        for (int jj = 1; jj < 8; ++jj) mx = fmaxf(mx, sc[jj]);
        mx = max_across_rows(mx);
        const float m_new = fmaxf(m_run[u], mx);
        // a column that has seen no key yet keeps m = -inf; its weights and rescale are then 0
        const float m_ref = ROWS && m_new == -INFINITY ? 0.0f : m_new;
        const float alpha = fast_exp2(m_run[u] - m_ref);
        float pr[8];
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) pr[jj] = fast_exp2(sc[jj] - m_ref);
        float psum = pr[0];
#pragma unroll
        for (int jj = 1; jj < 8; ++jj) psum += pr[jj];
        l_run[u] = l_run[u] * alpha + psum;
        m_run[u] = m_new;
        // once the running maxima settle, most steps leave them unchanged (alpha = 1 exactly,
        // and the rescale would change no bit); with two tiles the branch costs the fp8
        // instance registers it cannot spare (measured: fp8 verification 60.7 -> 66.4 us)
        if (MT > 1 || __any(alpha != 1.0f)) {
#pragma unroll
          for (int i = 0; i < NT; ++i) acc[u][i] *= alpha;
        }
        if constexpr (FP8) {
#pragma unroll
          for (int jj = 0; jj < 8; ++jj) pr[jj] *= r.vs;
        }
        uint32_t h[4], l[4];
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          h[w] = pack2<QT>(pr[2 * w], pr[2 * w + 1]);
          if constexpr (SPLIT_P) l[w] = bf16_lo2(pr[2 * w], pr[2 * w + 1], h[w]);
        }
        pHi[u] = as_vec8<V8>(make_uint4(h[0], h[1], h[2], h[3]));
        if constexpr (SPLIT_P) pLo[u] = as_vec8<V8>(make_uint4(l[0], l[1], l[2], l[3]));
      }

      // Masked tokens get weight 0, but slots at or past end_v may hold anything (NaN
      // included), so their V elements are zeroed before the product (each V operand is
      // widened once and multiplied into all tiles).
      uint32_t vm[4] = {~0u, ~0u, ~0u, ~0u};
      if (partial) {
        const int nval_v = min(max((ROWS ? end_v : end_tok[0]) - tb, 0), 8);
        if constexpr (FP8) {
          vm[0] = nval_v >= 4 ? ~0u : (nval_v <= 0 ? 0u : (1u << (8 * nval_v)) - 1u);
          vm[1] = nval_v >= 8 ? ~0u : (nval_v <= 4 ? 0u : (1u << (8 * (nval_v - 4))) - 1u);
        } else {
#pragma unroll
          for (int w = 0; w < 4; ++w)
            vm[w] = (2 * w < nval_v ? 0x0000FFFFu : 0u) | (2 * w + 1 < nval_v ? 0xFFFF0000u : 0u);
        }
      }
#pragma unroll
      for (int i = 0; i < NT; ++i) {
        V8 vA;
        if constexpr (FP8) {
          vA = fp8x8_to_vec8<QT>(r.v[i].x & vm[0], r.v[i].y & vm[1]);
        } else {
          const uint4 u4 = r.v[i];
          vA = as_vec8<V8>(make_uint4(u4.x & vm[0], u4.y & vm[1], u4.z & vm[2], u4.w & vm[3]));
        }
#pragma unroll
        for (int u = 0; u < MT; ++u) {
          acc[u][i] = M::mma(vA, pHi[u], acc[u][i]);
          if constexpr (SPLIT_P) acc[u][i] = M::mma(vA, pLo[u], acc[u][i]);
        }
      }
      if constexpr (ROLL) {
        if (nxt >= 0) issue_v(r);
      }
    };


    // The steady-state loop issues the next step's loads unconditionally (the tail is peeled),
    // so the loads of one step stay in flight while the previous step is computed.
    if constexpr (ROLL) {
      StepRegs<D, FP8> r;
      issue(r, s_first);
      for (int s = s_first; s < nsteps; s += stride)
        compute(r, s, s + stride < nsteps ? s + stride : -1);
      return;
    }
    StepRegs<D, FP8> r0, r1;
    int s = s_first, rest = (nsteps - 1 - s_first) / stride;
    issue(r0, s);
    for (; rest >= 2; rest -= 2, s += 2 * stride) {
      issue(r1, s + stride);
      compute(r0, s, -1);
      issue(r0, s + 2 * stride);
      compute(r1, s + stride, -1);
    }
    if (rest == 1) {
      issue(r1, s + stride);
      compute(r0, s, -1);
      compute(r1, s + stride, -1);
    } else {
      compute(r0, s, -1);
    }
  }
};

}  // namespace pa
