// Internal launch interface between the C ABI (pa_api.hip) and the kernel translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pa {

constexpr int kBlock = 16;          // tokens per physical KV block
constexpr int kStepTokens = 32;     // tokens one wave consumes per step (two blocks)
constexpr int kWaves = 4;           // waves per decode workgroup
constexpr int kMaxPartition = 65536; // largest fixed key partition (tokens)

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
  int* ws_cnt;          // [kMaxWorkgroups] arrival counters, zero between calls
  float* ws_acc;        // [workgroups][2][group][head_dim]: unnormalised output of a cut group
  float* ws_ml;         // [workgroups][2][group][2]: running max (log2 units), exp-sum
  int batch;
  int num_q_heads;
  int num_kv_heads;
  int group;            // num_q_heads / num_kv_heads, 1..16
  int num_blocks;
  int max_blocks_per_seq;
  int len_cap;          // context lengths are clamped to [0, len_cap]
  int chunk_blocks;     // fixed chunk length in blocks (even), or 0: balanced over total_waves
  int total_waves;      // waves launched (4 per workgroup); chunk c is wave c's
  float qk_scale_log2;  // scale * log2(e)
};

// Workspace: a fixed region of arrival counters (so that their place never depends on the
// descriptor and a workspace zero-filled once stays valid for every call), then two published
// partial results per workgroup; each part 256-byte aligned.
constexpr long kMaxWorkgroups = 65536;
struct WorkspaceLayout {
  size_t acc, ml, total;
};
inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
inline WorkspaceLayout workspace_layout(int group, int head_dim, long workgroups) {
  WorkspaceLayout w;
  w.acc = align256((size_t)kMaxWorkgroups * sizeof(int));
  w.ml = w.acc + align256((size_t)workgroups * 2 * group * head_dim * sizeof(float));
  w.total = w.ml + align256((size_t)workgroups * 2 * group * 2 * sizeof(float));
  return w;
}

// Waves launched by the balanced mode never exceed this (a workspace bound known without a GPU).
constexpr long kMaxWaves = 8192;

hipError_t launch_append(const AppendArgs& a, int num_tokens, int elem_bytes, hipStream_t stream);
hipError_t launch_decode(const DecodeArgs& a, int head_dim, int q_dtype, int kv_dtype,
                         hipStream_t stream);
// Resident decode workgroups per CU for this kernel instance (0 if the query fails).
int decode_workgroups_per_cu(int head_dim, int q_dtype, int kv_dtype);

}  // namespace pa
