// Device-side helpers for the gfx950 paged-attention kernels: vector types, MFMA wrappers,
// fp8 (OCP e4m3fn) widening and wave-level cross-lane reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

enum : int { DT_F16 = 0, DT_BF16 = 1, DT_FP8 = 2 };

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2;

// Element type fed to the matrix cores: the query's 16-bit type.
template <int QT> struct Mfma;

template <> struct Mfma<DT_BF16> {
  typedef __bf16 elem;
  typedef bf16x8 vec8;
  // D = A(16x32) * B(32x16) + C.  Lane l holds A[l%16][8*(l/16)+i], B[8*(l/16)+i][l%16] and
  // C[4*(l/16)+i][l%16].
  static __device__ __forceinline__ f32x4 mma(vec8 a, vec8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  // Two fp8 codes (the low or high 16 bits of w) widened exactly.
  template <bool HI>
  static __device__ __forceinline__ bf16x2 from_fp8x2(uint32_t w) {
    return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI);
  }
};

template <> struct Mfma<DT_F16> {
  typedef _Float16 elem;
  typedef f16x8 vec8;
  static __device__ __forceinline__ f32x4 mma(vec8 a, vec8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
  template <bool HI>
  static __device__ __forceinline__ f16x2 from_fp8x2(uint32_t w) {
    return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, HI);
  }
};

template <typename V8>
__device__ __forceinline__ V8 as_vec8(uint4 u) {
  return __builtin_bit_cast(V8, u);
}

// Eight fp8 codes (two dwords) -> eight 16-bit MFMA elements, exactly.
template <int QT>
__device__ __forceinline__ typename Mfma<QT>::vec8 fp8x8_to_vec8(uint32_t w0, uint32_t w1) {
  typedef typename Mfma<QT>::vec8 V8;
  auto a = Mfma<QT>::template from_fp8x2<false>(w0);
  auto b = Mfma<QT>::template from_fp8x2<true>(w0);
  auto c = Mfma<QT>::template from_fp8x2<false>(w1);
  auto d = Mfma<QT>::template from_fp8x2<true>(w1);
  V8 r;
  r[0] = a[0]; r[1] = a[1]; r[2] = b[0]; r[3] = b[1];
  r[4] = c[0]; r[5] = c[1]; r[6] = d[0]; r[7] = d[1];
  return r;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Device-coherent stores and loads (agent-scope relaxed atomics: the L2 is bypassed for
// visibility across XCDs) for results one workgroup publishes and another reads in the same
// kernel, without a whole-L2 writeback or invalidate.
typedef __attribute__((ext_vector_type(2))) float f32x2;
__device__ __forceinline__ void store_coherent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_coherent(float* p, f32x4 v) {
  uint64_t* q = reinterpret_cast<uint64_t*>(p);
  __hip_atomic_store(q, __builtin_bit_cast(uint64_t, f32x2{v[0], v[1]}), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
  __hip_atomic_store(q + 1, __builtin_bit_cast(uint64_t, f32x2{v[2], v[3]}), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_coherent(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ f32x2 load_coherent2(const float* p) {
  uint64_t* q = reinterpret_cast<uint64_t*>(const_cast<float*>(p));
  return __builtin_bit_cast(f32x2,
                            __hip_atomic_load(q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
}
__device__ __forceinline__ f32x4 load_coherent4(const float* p) {
  uint64_t* q = reinterpret_cast<uint64_t*>(const_cast<float*>(p));
  const f32x2 a = __builtin_bit_cast(
      f32x2, __hip_atomic_load(q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
  const f32x2 b = __builtin_bit_cast(
      f32x2, __hip_atomic_load(q + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
  return f32x4{a[0], a[1], b[0], b[1]};
}
// Streaming loads of K/V tiles: every byte is read once per launch, so they are marked
// non-temporal (measured ~13% more gather bandwidth than plain loads on MI355X).
typedef __attribute__((ext_vector_type(4))) unsigned u32x4;
typedef __attribute__((ext_vector_type(2))) unsigned u32x2;
__device__ __forceinline__ uint4 load_stream16(const void* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ uint2 load_stream8(const void* p) {
  const u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
  return make_uint2(v[0], v[1]);
}

// Wait until this wave's memory operations have completed (stores acknowledged).
__device__ __forceinline__ void wait_memory_ops() { __builtin_amdgcn_s_waitcnt(0); }

// Butterfly over the four 16-lane rows of a wave (lanes l, l^16, l^32, l^48) with the gfx950
// lane-swap instructions, which stay in the vector ALU (a cross-lane shuffle would go through
// the LDS crossbar).  Swapping a value with itself, v_permlane16_swap returns the even row of
// each row pair in its first result and the odd row in its second (v_permlane32_swap: the lower
// and upper halves), so combining the two results gives every lane the same pairwise result.
__device__ __forceinline__ float max_across_rows(float x) {
  const uint32_t u = __float_as_uint(x);
  const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const uint32_t w = __float_as_uint(x);
  const auto b = __builtin_amdgcn_permlane32_swap(w, w, false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float sum_across_rows(float x) {
  const uint32_t u = __float_as_uint(x);
  const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const uint32_t w = __float_as_uint(x);
  const auto b = __builtin_amdgcn_permlane32_swap(w, w, false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

}  // namespace pa
