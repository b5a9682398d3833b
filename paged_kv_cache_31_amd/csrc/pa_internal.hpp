// Internal launch interface between the C ABI (pa_api.hip) and the kernel translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pa {

constexpr int kBlock = 16;          // tokens per physical KV block
constexpr int kStepTokens = 32;     // tokens one wave consumes per step (two blocks)
constexpr int kWaves = 4;           // waves per decode workgroup
constexpr int kMaxPartition = 4096; // largest key partition (block ids staged in LDS)

struct AppendArgs {
  const uint8_t* k_new;
  const uint8_t* v_new;
  const int64_t* slots;
  uint8_t* k_cache;
  uint8_t* v_cache;
  int64_t num_slots;   // num_blocks * 16: slots at or beyond this are skipped
  int num_kv_heads;
  int head_dim;
};

struct DecodeArgs {
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const float* k_scale;
  const float* v_scale;
  const int32_t* block_tables;
  const int32_t* context_lens;
  void* out;
  float* ws_acc;        // [batch][num_q_heads][np_max][head_dim]
  float* ws_ml;         // [batch][num_q_heads][np_max][2]: running max (log2 units), exp-sum
  int batch;
  int num_q_heads;
  int num_kv_heads;
  int group;            // num_q_heads / num_kv_heads, 1..16
  int num_blocks;
  int max_blocks_per_seq;
  int len_cap;          // context lengths are clamped to [0, len_cap]
  int partition;        // key-partition length in tokens (multiple of 32)
  int np_max;           // partitions launched per (sequence, kv head)
  float qk_scale_log2;  // scale * log2(e)
};

// Workspace split: acc floats first, then (m, l) pairs, each 256-byte aligned.
inline size_t ws_acc_bytes(int batch, int hq, int np_max, int head_dim) {
  size_t b = (size_t)batch * hq * np_max * head_dim * sizeof(float);
  return (b + 255) & ~(size_t)255;
}
inline size_t ws_ml_bytes(int batch, int hq, int np_max) {
  size_t b = (size_t)batch * hq * np_max * 2 * sizeof(float);
  return (b + 255) & ~(size_t)255;
}

hipError_t launch_append(const AppendArgs& a, int num_tokens, int elem_bytes, hipStream_t stream);
hipError_t launch_decode(const DecodeArgs& a, int head_dim, int q_dtype, int kv_dtype,
                         hipStream_t stream);

}  // namespace pa
