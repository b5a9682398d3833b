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

hipError_t launch_append(const AppendArgs& a, int num_tokens, int elem_bytes, hipStream_t stream) {
  const dim3 grid(num_tokens, a.num_kv_heads), block(a.head_dim);
  if (elem_bytes == 2)
    hipLaunchKernelGGL(append_kernel<2>, grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL(append_kernel<1>, grid, block, 0, stream, a);
  return hipGetLastError();
}

}  // namespace pa
