// KV append: scatter each new token's K and V rows into its slot of the paged cache.
//
// A generation step stores the new token's K/V projection (Scaling Book note, "Transformer 推論の
// 基礎: Prefill と Generation"); in the paged cache the token occupies offset slot%16 of physical
// block slot/16 (kasblo.com, "blockはrequestの成長に合わせて割り当てる").  K tiles are token-major,
// so a token's K row for one head is one contiguous run copied in 16-byte vectors; V tiles are
// dim-major, so the token's V row lands as one element in each of head_dim rows of 16.
//
// One workgroup per (token, KV head) and one thread per head dimension: every thread issues its
// loads before its stores, so the whole append costs about one memory round trip.  The copy moves
// raw bytes, so it is exact for every dtype.
#include <type_traits>

#include "pa_internal.hpp"

namespace pa {

template <int EB>
__global__ __launch_bounds__(128) void append_kernel(AppendArgs a) {
  typedef typename std::conditional<EB == 2, uint16_t, uint8_t>::type E;
  const int i = blockIdx.x, h = blockIdx.y, t = threadIdx.x;   // t < head_dim
  const int H = a.num_kv_heads, D = a.head_dim;
  const int kvecs = D * EB / 16;                                 // 16-byte pieces of a K row
  const size_t row = (size_t)i * H + h;

  const E v = reinterpret_cast<const E*>(a.v_new)[row * D + t];
  uint4 k = make_uint4(0u, 0u, 0u, 0u);
  if (t < kvecs) k = reinterpret_cast<const uint4*>(a.k_new)[row * kvecs + t];

  const int64_t s = a.slots[i];
  if (s < 0 || s >= a.num_slots) return;                 // padding token / outside the pool
  const int64_t blk = s >> 4;
  const int off = (int)(s & 15);
  const size_t tile = (size_t)blk * H + h;
  // K: token-major tile, the row is contiguous
  if (t < kvecs)
    reinterpret_cast<uint4*>(a.k_cache + (tile * kBlock + off) * D * EB)[t] = k;
  // V: dim-major tile, element t goes to row t, column off
  reinterpret_cast<E*>(a.v_cache)[(tile * D + t) * kBlock + off] = v;
}

// ---- The append of a decode step taken out of the decode launch (pa_decode_append with many
// appends per decode wave): token L-1 of every sequence, its slot read from the block table, one
// workgroup per (sequence, KV head) and one thread per dimension as in append_kernel.
template <int EB>
__global__ __launch_bounds__(128) void append_last_kernel(LastAppendArgs a) {
  typedef typename std::conditional<EB == 2, uint16_t, uint8_t>::type E;
  const int b = blockIdx.x, h = blockIdx.y, t = threadIdx.x;   // t < head_dim
  const int H = a.num_kv_heads, D = a.head_dim;
  const int kvecs = D * EB / 16;
  const size_t row = (size_t)b * H + h;

  const E v = reinterpret_cast<const E*>(a.v_new)[row * D + t];
  uint4 k = make_uint4(0u, 0u, 0u, 0u);
  if (t < kvecs) k = reinterpret_cast<const uint4*>(a.k_new)[row * kvecs + t];

  const int L = min(max(a.context_lens[b], 0), a.len_cap);
  if (L == 0) return;                                     // no token: nothing appended
  const int blk = a.block_tables[(size_t)b * a.max_blocks_per_seq + (L - 1) / kBlock];
  if ((unsigned)blk >= (unsigned)a.num_blocks) return;   // outside the pool: skipped
  const int off = (L - 1) % kBlock;
  const size_t tile = (size_t)blk * H + h;
  if (t < kvecs)
    reinterpret_cast<uint4*>(a.k_cache + (tile * kBlock + off) * D * EB)[t] = k;
  reinterpret_cast<E*>(a.v_cache)[(tile * D + t) * kBlock + off] = v;
}

hipError_t launch_append_last(const LastAppendArgs& a, int batch, int elem_bytes,
                              hipStream_t stream) {
  const dim3 grid(batch, a.num_kv_heads);
  if (elem_bytes == 2)
    hipLaunchKernelGGL(append_last_kernel<2>, grid, dim3(a.head_dim), 0, stream, a);
  else
    hipLaunchKernelGGL(append_last_kernel<1>, grid, dim3(a.head_dim), 0, stream, a);
  return hipGetLastError();
}

// ---- Quantising append into an fp8 (OCP e4m3fn) cache with per-(block, KV head) scales.
//
// The fp8 KV cache stores value = code * scale (design.babushkai.com "GPU推論の内部構造", KV-cache
// and quantisation sections).  How a block's scale is chosen is not given there; this follows
// one reading: with the first-token policy, a token written at offset 0 of its block first sets
// that block's scale to fp32(max |x|) / 448 (1 if the maximum is 0), per KV head and separately
// for K and V (quant_scale_kernel); then every token is encoded as
// e4m3fn(clamp(fp32(x) / scale, +-448)) with round-to-nearest-even (quant_append_kernel).  A
// token later in a block uses the block's scale as it stands and saturates if it is larger.

template <typename S>
__device__ __forceinline__ float widen(S x) {
  return (float)x;                                  // exact: 16-bit values fit in fp32
}

template <typename S>
__global__ __launch_bounds__(64) void quant_scale_kernel(QuantAppendArgs a) {
  const int i = blockIdx.x, h = blockIdx.y, lane = threadIdx.x;
  const int64_t s = a.slots[i];
  if (s < 0 || s >= a.num_slots || (s & 15) != 0) return;   // only a block's first token
  const int H = a.num_kv_heads, D = a.head_dim;
  const S* kn = reinterpret_cast<const S*>(a.k_new) + ((size_t)i * H + h) * D;
  const S* vn = reinterpret_cast<const S*>(a.v_new) + ((size_t)i * H + h) * D;
  // A compare-and-select skips NaN elements of either kind (fmaxf would let a signalling NaN
  // through as a quiet one), so the running maxima stay numbers.
  float km = 0.0f, vm = 0.0f;
  for (int d = lane; d < D; d += 64) {
    const float xk = fabsf(widen(kn[d])), xv = fabsf(widen(vn[d]));
    km = xk > km ? xk : km;
    vm = xv > vm ? xv : vm;
  }
  for (int o = 32; o > 0; o >>= 1) {
    km = fmaxf(km, __shfl_xor(km, o));
    vm = fmaxf(vm, __shfl_xor(vm, o));
  }
  if (lane == 0) {
    const size_t at = (size_t)(s >> 4) * H + h;
    a.k_scale[at] = km == 0.0f ? 1.0f : km / 448.0f;
    a.v_scale[at] = vm == 0.0f ? 1.0f : vm / 448.0f;
  }
}

// e4m3fn code of y: saturate at 448, round to nearest even (the hardware conversion on the
// magnitude), keep the sign (so -0 and values that round to zero from below give 0x80), NaN 0x7F.
__device__ __forceinline__ uint8_t e4m3fn_code(float y) {
  if (y != y) return 0x7F;
  const float m = fminf(fabsf(y), 448.0f);
  const uint32_t c = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(m, m, 0, false) & 0x7Fu;
  return (uint8_t)(c | (__builtin_signbitf(y) ? 0x80u : 0u));
}

template <typename S>
__global__ __launch_bounds__(128) void quant_append_kernel(QuantAppendArgs a) {
  const int i = blockIdx.x, h = blockIdx.y, t = threadIdx.x;   // t < head_dim
  const int H = a.num_kv_heads, D = a.head_dim;
  const size_t row = ((size_t)i * H + h) * D;
  const float xk = widen(reinterpret_cast<const S*>(a.k_new)[row + t]);
  const float xv = widen(reinterpret_cast<const S*>(a.v_new)[row + t]);
  const int64_t s = a.slots[i];
  if (s < 0 || s >= a.num_slots) return;
  const int off = (int)(s & 15);
  const size_t tile = (size_t)(s >> 4) * H + h;
  const uint8_t ck = e4m3fn_code(xk / a.k_scale[tile]);   // IEEE fp32 division
  const uint8_t cv = e4m3fn_code(xv / a.v_scale[tile]);
  a.k_cache[(tile * kBlock + off) * D + t] = ck;
  a.v_cache[(tile * D + t) * kBlock + off] = cv;
}

hipError_t launch_append_quant(const QuantAppendArgs& a, int num_tokens, bool bf16_src,
                               bool first_token_scale, hipStream_t stream) {
  const dim3 grid(num_tokens, a.num_kv_heads);
  if (first_token_scale) {
    if (bf16_src)
      hipLaunchKernelGGL(quant_scale_kernel<__bf16>, grid, dim3(64), 0, stream, a);
    else
      hipLaunchKernelGGL(quant_scale_kernel<_Float16>, grid, dim3(64), 0, stream, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (bf16_src)
    hipLaunchKernelGGL(quant_append_kernel<__bf16>, grid, dim3(a.head_dim), 0, stream, a);
  else
    hipLaunchKernelGGL(quant_append_kernel<_Float16>, grid, dim3(a.head_dim), 0, stream, a);
  return hipGetLastError();
}

// Copy-on-write copies: workgroup (pair i, KV head h) copies the K and V tiles of block
// pairs[i][0] into block pairs[i][1] with 16-byte loads and stores, and the fp8 scales with
// them.  Many small workgroups, each thread with one word per pool, keep the reads and writes
// of the copy interleaved across the chip (measured faster than fewer workgroups moving 16 KiB
// chunks with all loads issued before the stores).  Pairs whose blocks lie outside the pool,
// or that copy a block onto itself, are skipped.
__global__ __launch_bounds__(256) void copy_blocks_kernel(CopyArgs a) {
  const int i = blockIdx.x, h = blockIdx.y;
  const int src = a.pairs[2 * i], dst = a.pairs[2 * i + 1];
  if ((unsigned)src >= (unsigned)a.num_blocks || (unsigned)dst >= (unsigned)a.num_blocks ||
      src == dst)
    return;
  const size_t so = ((size_t)src * a.num_kv_heads + h) * a.tile_bytes;
  const size_t dof = ((size_t)dst * a.num_kv_heads + h) * a.tile_bytes;
  const int n16 = a.tile_bytes / 16;
  for (int e = threadIdx.x; e < n16; e += blockDim.x) {
    const uint4 kx = *reinterpret_cast<const uint4*>(a.k_cache + so + 16 * (size_t)e);
    const uint4 vx = *reinterpret_cast<const uint4*>(a.v_cache + so + 16 * (size_t)e);
    *reinterpret_cast<uint4*>(a.k_cache + dof + 16 * (size_t)e) = kx;
    *reinterpret_cast<uint4*>(a.v_cache + dof + 16 * (size_t)e) = vx;
  }
  if (a.k_scale && threadIdx.x == 0) {
    a.k_scale[(size_t)dst * a.num_kv_heads + h] = a.k_scale[(size_t)src * a.num_kv_heads + h];
    a.v_scale[(size_t)dst * a.num_kv_heads + h] = a.v_scale[(size_t)src * a.num_kv_heads + h];
  }
}

hipError_t launch_copy_blocks(const CopyArgs& a, int n, hipStream_t stream) {
  hipLaunchKernelGGL(copy_blocks_kernel, dim3(n, a.num_kv_heads), dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_append(const AppendArgs& a, int num_tokens, int elem_bytes, hipStream_t stream) {
  const dim3 grid(num_tokens, a.num_kv_heads), block(a.head_dim);
  if (elem_bytes == 2)
    hipLaunchKernelGGL(append_kernel<2>, grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL(append_kernel<1>, grid, block, 0, stream, a);
  return hipGetLastError();
}

}  // namespace pa
