// C ABI of the paged decode-attention library (declared in include/pa.h): host-side argument
// validation, the split-KV partition choice, workspace sizing and kernel dispatch.  Nothing here
// reads device memory or synchronises.
#include <stdint.h>

#include <map>
#include <mutex>
#include <tuple>

#include "pa.h"
#include "pa_internal.hpp"

#define PA_EXPORT extern "C" __attribute__((visibility("default")))

// Bytes of the static scratch behind pa_decode_noalloc, per GPU (see include/pa.h).
#ifndef PA_NOALLOC_SCRATCH_BYTES
#define PA_NOALLOC_SCRATCH_BYTES (64u << 20)
#endif

// Balanced mode launches this many waves per resident wave slot.
#ifndef PA_WAVE_ROUNDS
#define PA_WAVE_ROUNDS 1
#endif

namespace {

thread_local int32_t g_last_hip_error = 0;

bool aligned(const void* p, uintptr_t n) { return (reinterpret_cast<uintptr_t>(p) % n) == 0; }

pa_status check_cache(const pa_cache_desc* c) {
  if (!c) return PA_ERR_INVALID_ARG;
  if (c->num_blocks <= 0 || c->num_kv_heads <= 0 || c->head_dim <= 0 || c->block_size <= 0)
    return PA_ERR_INVALID_ARG;
  if (c->kv_dtype < PA_F16 || c->kv_dtype > PA_FP8_E4M3) return PA_ERR_INVALID_ARG;
  if (c->block_size != pa::kBlock) return PA_ERR_UNSUPPORTED;
  if (c->num_kv_heads > 65535) return PA_ERR_UNSUPPORTED;   // launch grid limit
  if (c->head_dim != 64 && c->head_dim != 128) return PA_ERR_UNSUPPORTED;
  return PA_OK;
}

int64_t blocks_upper(const pa_decode_desc* d);
int64_t chunk_capacity(const pa_decode_desc* d);

pa_status check_decode_desc(const pa_decode_desc* d) {
  if (!d) return PA_ERR_INVALID_ARG;
  pa_status s = check_cache(&d->cache);
  if (s != PA_OK) return s;
  if (d->batch <= 0 || d->num_q_heads <= 0 || d->max_blocks_per_seq <= 0 ||
      d->max_context_len < 0 || d->partition_tokens < 0)
    return PA_ERR_INVALID_ARG;
  if (d->num_q_heads % d->cache.num_kv_heads != 0) return PA_ERR_INVALID_ARG;
  if (d->batch > 65535 || d->num_q_heads > 65535) return PA_ERR_UNSUPPORTED;   // grid y/z limits
  const int group = d->num_q_heads / d->cache.num_kv_heads;
  if (group > 16) return PA_ERR_UNSUPPORTED;
  if (d->partition_tokens != 0 &&
      (d->partition_tokens % pa::kBlock != 0 || d->partition_tokens > pa::kMaxPartition))
    return PA_ERR_INVALID_ARG;
  if (blocks_upper(d) >= INT32_MAX) return PA_ERR_UNSUPPORTED;   // flattened index is 32-bit
  if (chunk_capacity(d) > pa::kMaxWorkgroups * pa::kWaves) return PA_ERR_UNSUPPORTED;
  if (d->shared_prefixes < 0 || d->shared_prefixes > 2) return PA_ERR_INVALID_ARG;
  if (d->q_dtype != PA_F16 && d->q_dtype != PA_BF16) return PA_ERR_UNSUPPORTED;
  const int kv = d->cache.kv_dtype;
  if (kv != PA_FP8_E4M3 && kv != d->q_dtype) return PA_ERR_UNSUPPORTED;
  return PA_OK;
}

// Longest context the launch covers.
int len_cap(const pa_decode_desc* d) {
  const int64_t table_cap = (int64_t)d->max_blocks_per_seq * pa::kBlock;
  int64_t cap = d->max_context_len > 0 ? d->max_context_len : table_cap;
  if (cap > table_cap) cap = table_cap;
  if (cap > INT32_MAX) cap = INT32_MAX;
  return (int)cap;
}

// Longest context a multi-query launch covers (same rule as len_cap).
int multi_len_cap(const pa_multi_desc* d) {
  const int64_t table_cap = (int64_t)d->max_blocks_per_seq * pa::kBlock;
  int64_t cap = d->max_context_len > 0 ? d->max_context_len : table_cap;
  if (cap > table_cap) cap = table_cap;
  if (cap > INT32_MAX) cap = INT32_MAX;
  return (int)cap;
}

// Resident multi_split_kernel workgroups on the current device, cached per device and instance.
int64_t resident_split_wgs(const pa_multi_desc* d, int rt) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  static std::mutex mu;
  static std::map<std::tuple<int, int, int, int, int>, int64_t> cache;
  const auto key = std::make_tuple(dev, (int)d->cache.head_dim, (int)d->q_dtype,
                                   (int)d->cache.kv_dtype, rt);
  std::lock_guard<std::mutex> lock(mu);
  auto it = cache.find(key);
  if (it != cache.end()) return it->second;
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    cus = 0;
  const int per_cu = pa::multi_split_workgroups_per_cu(d->cache.head_dim, d->q_dtype,
                                                       d->cache.kv_dtype, rt);
  const int64_t wgs = (int64_t)(cus > 0 ? cus : 1) * (per_cu > 0 ? per_cu : 1);
  cache[key] = wgs;
  return wgs;
}

pa::MultiPlan multi_plan_of(const pa_multi_desc* d) {
  return pa::multi_plan(d->batch, d->cache.num_kv_heads, d->num_q_heads / d->cache.num_kv_heads,
                        d->max_query_len, multi_len_cap(d), d->partition_tokens,
                        d->cache.head_dim, d->cache.kv_dtype == PA_FP8_E4M3);
}

// Upper bound of the flattened (sequence, KV head, block) space.
int64_t blocks_upper(const pa_decode_desc* d) {
  return (int64_t)d->batch * d->cache.num_kv_heads * ((len_cap(d) + pa::kBlock - 1) / pa::kBlock);
}

// Chunks (= waves) the workspace must hold.  Fixed partitions: every chunk of the upper bound.
// Balanced mode: one chunk per launched wave, at most kMaxWaves and never more than the space
// has two-block chunks.
int64_t chunk_capacity(const pa_decode_desc* d) {
  const int64_t W = blocks_upper(d);
  int64_t n;
  if (d->partition_tokens > 0) {
    const int64_t cw = d->partition_tokens / pa::kBlock;
    n = (W + cw - 1) / cw;
  } else {
    n = (W + 1) / 2;
    if (n > pa::kMaxWaves) n = pa::kMaxWaves;
  }
  if (n < 1) n = 1;
  return (n + pa::kWaves - 1) / pa::kWaves * pa::kWaves;
}

// Shared prefixes are planned when asked for, when a tile holds at least two members
// (group <= 8) and when the batch fits one planning workgroup.
bool sharing_active(const pa_decode_desc* d) {
  return d->shared_prefixes != 0 && d->num_q_heads / d->cache.num_kv_heads <= 8 &&
         d->batch <= pa::kPlanMaxBatch;
}

pa::WorkspaceLayout layout_of(const pa_decode_desc* d) {
  const bool share = sharing_active(d);
  return pa::workspace_layout(d->num_q_heads / d->cache.num_kv_heads, d->cache.head_dim,
                              chunk_capacity(d) / pa::kWaves, d->batch, d->num_q_heads,
                              share ? pa::prefix_parts_of(d->max_blocks_per_seq) : 0);
}

size_t workspace_bytes_of(const pa_decode_desc* d) { return layout_of(d).total; }

// Signature of a shared-prefix plan: the descriptor fields and the workspace layout it was made
// for (FNV-1a over them).  A call reusing a plan takes it only if it finds its own signature.
int32_t plan_signature(const pa_decode_desc* d, const pa::WorkspaceLayout& w) {
  const uint64_t fields[] = {(uint64_t)d->batch, (uint64_t)d->num_q_heads,
                             (uint64_t)d->cache.num_kv_heads, (uint64_t)d->cache.head_dim,
                             (uint64_t)d->cache.kv_dtype, (uint64_t)d->q_dtype,
                             (uint64_t)d->cache.num_blocks, (uint64_t)d->max_blocks_per_seq,
                             (uint64_t)len_cap(d), (uint64_t)d->partition_tokens,
                             (uint64_t)w.plan, (uint64_t)w.gp_acc, (uint64_t)w.units,
                             (uint64_t)w.total};
  uint32_t h = 2166136261u;
  for (uint64_t f : fields)
    for (int i = 0; i < 8; ++i) {
      h ^= (uint32_t)((f >> (8 * i)) & 0xFF);
      h *= 16777619u;
    }
  return (int32_t)h;
}

// Resident decode waves on the current device for this kernel instance, cached per device.
int64_t resident_waves(const pa_decode_desc* d) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  static std::mutex mu;
  static std::map<std::tuple<int, int, int, int>, int64_t> cache;
  const auto key = std::make_tuple(dev, (int)d->cache.head_dim, (int)d->q_dtype,
                                   (int)d->cache.kv_dtype);
  std::lock_guard<std::mutex> lock(mu);
  auto it = cache.find(key);
  if (it != cache.end()) return it->second;
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    cus = 0;
  const int per_cu = pa::decode_workgroups_per_cu(d->cache.head_dim, d->q_dtype,
                                                  d->cache.kv_dtype);
  const int64_t waves = (int64_t)(cus > 0 ? cus : 1) * (per_cu > 0 ? per_cu : 1) * pa::kWaves;
  cache[key] = waves;
  return waves;
}

}  // namespace

PA_EXPORT const char* pa_status_string(pa_status s) {
  switch (s) {
    case PA_OK: return "ok";
    case PA_ERR_INVALID_ARG: return "invalid argument";
    case PA_ERR_UNSUPPORTED: return "unsupported configuration";
    case PA_ERR_WORKSPACE: return "workspace missing or too small";
    case PA_ERR_HIP: return "HIP launch failed";
    case PA_ERR_OUT_OF_BLOCKS: return "no free block in the pool";
  }
  return "unknown status";
}

PA_EXPORT int32_t pa_last_hip_error(void) { return g_last_hip_error; }

PA_EXPORT pa_status pa_kv_append(const pa_cache_desc* cache, int32_t num_tokens,
                                 const void* k_new, const void* v_new,
                                 const int64_t* slot_mapping, void* k_cache, void* v_cache,
                                 void* stream) {
  pa_status s = check_cache(cache);
  if (s != PA_OK) return s;
  if (num_tokens < 0) return PA_ERR_INVALID_ARG;
  if (num_tokens == 0) return PA_OK;
  if (!k_new || !v_new || !slot_mapping || !k_cache || !v_cache) return PA_ERR_INVALID_ARG;
  if (!aligned(k_new, 16) || !aligned(v_new, 16) || !aligned(k_cache, 16) ||
      !aligned(v_cache, 16) || !aligned(slot_mapping, 8))
    return PA_ERR_INVALID_ARG;
  pa::AppendArgs a;
  a.k_new = static_cast<const uint8_t*>(k_new);
  a.v_new = static_cast<const uint8_t*>(v_new);
  a.slots = slot_mapping;
  a.k_cache = static_cast<uint8_t*>(k_cache);
  a.v_cache = static_cast<uint8_t*>(v_cache);
  a.num_slots = (int64_t)cache->num_blocks * pa::kBlock;
  a.num_kv_heads = cache->num_kv_heads;
  a.head_dim = cache->head_dim;
  const int eb = cache->kv_dtype == PA_FP8_E4M3 ? 1 : 2;
  hipError_t e = pa::launch_append(a, num_tokens, eb, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) {
    g_last_hip_error = (int32_t)e;
    return PA_ERR_HIP;
  }
  return PA_OK;
}

PA_EXPORT pa_status pa_kv_append_quant(const pa_cache_desc* cache, int32_t num_tokens,
                                       int32_t src_dtype, const void* k_new, const void* v_new,
                                       const int64_t* slot_mapping, void* k_cache, void* v_cache,
                                       float* k_scale, float* v_scale, int32_t scale_policy,
                                       void* stream) {
  pa_status s = check_cache(cache);
  if (s != PA_OK) return s;
  if (num_tokens < 0) return PA_ERR_INVALID_ARG;
  if (scale_policy != PA_SCALE_KEEP && scale_policy != PA_SCALE_FIRST_TOKEN)
    return PA_ERR_INVALID_ARG;
  if (src_dtype != PA_F16 && src_dtype != PA_BF16) return PA_ERR_UNSUPPORTED;
  if (cache->kv_dtype != PA_FP8_E4M3) return PA_ERR_UNSUPPORTED;
  if (num_tokens == 0) return PA_OK;
  if (!k_new || !v_new || !slot_mapping || !k_cache || !v_cache || !k_scale || !v_scale)
    return PA_ERR_INVALID_ARG;
  if (!aligned(k_new, 16) || !aligned(v_new, 16) || !aligned(k_cache, 16) ||
      !aligned(v_cache, 16) || !aligned(slot_mapping, 8) || !aligned(k_scale, 4) ||
      !aligned(v_scale, 4))
    return PA_ERR_INVALID_ARG;
  pa::QuantAppendArgs a;
  a.k_new = static_cast<const uint8_t*>(k_new);
  a.v_new = static_cast<const uint8_t*>(v_new);
  a.slots = slot_mapping;
  a.k_cache = static_cast<uint8_t*>(k_cache);
  a.v_cache = static_cast<uint8_t*>(v_cache);
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.num_slots = (int64_t)cache->num_blocks * pa::kBlock;
  a.num_kv_heads = cache->num_kv_heads;
  a.head_dim = cache->head_dim;
  hipError_t e = pa::launch_append_quant(a, num_tokens, src_dtype == PA_BF16,
                                         scale_policy == PA_SCALE_FIRST_TOKEN,
                                         static_cast<hipStream_t>(stream));
  if (e != hipSuccess) {
    g_last_hip_error = (int32_t)e;
    return PA_ERR_HIP;
  }
  return PA_OK;
}

namespace {

pa_status check_multi_desc(const pa_multi_desc* d) {
  if (!d) return PA_ERR_INVALID_ARG;
  pa_status s = check_cache(&d->cache);
  if (s != PA_OK) return s;
  if (d->batch <= 0 || d->num_q_heads <= 0 || d->max_blocks_per_seq <= 0 ||
      d->max_context_len < 0 || d->partition_tokens < 0 || d->total_queries < 0 ||
      d->max_query_len <= 0)
    return PA_ERR_INVALID_ARG;
  if (d->num_q_heads % d->cache.num_kv_heads != 0) return PA_ERR_INVALID_ARG;
  if (d->partition_tokens != 0 &&
      (d->partition_tokens % pa::kBlock != 0 || d->partition_tokens > pa::kMaxPartition))
    return PA_ERR_INVALID_ARG;
  if (d->q_dtype != PA_F16 && d->q_dtype != PA_BF16) return PA_ERR_UNSUPPORTED;
  const int kv = d->cache.kv_dtype;
  if (kv != PA_FP8_E4M3 && kv != d->q_dtype) return PA_ERR_UNSUPPORTED;
  // grid sizes: items of the attention kernel and rows of the merge, 4 waves per workgroup
  const pa::MultiPlan p = multi_plan_of(d);
  if (p.split_rt > 0 && (int64_t)d->batch * d->cache.num_kv_heads *
                                ((multi_len_cap(d) + pa::kBlock - 1) / pa::kBlock) >= INT32_MAX)
    return PA_ERR_UNSUPPORTED;   // the balanced split indexes the flattened block space in 32 bits
  if (p.items > (1LL << 32) || (long long)d->batch * d->max_query_len * d->num_q_heads > (1LL << 32))
    return PA_ERR_UNSUPPORTED;
  if (p.row_blocks > 0 && p.items > (1LL << 31) - 8) return PA_ERR_UNSUPPORTED;  // one per workgroup
  return PA_OK;
}

}  // namespace

PA_EXPORT size_t pa_decode_multi_workspace_size(const pa_multi_desc* desc) {
  if (check_multi_desc(desc) != PA_OK) return 0;
  return pa::multi_workspace_bytes(multi_plan_of(desc), desc->total_queries, desc->num_q_heads,
                                   desc->cache.head_dim);
}

PA_EXPORT pa_status pa_decode_multi(const pa_multi_desc* desc, const void* q,
                                    const int32_t* query_start, const void* k_cache,
                                    const void* v_cache, const float* k_scale,
                                    const float* v_scale, const int32_t* block_tables,
                                    const int32_t* context_lens, float scale, void* out,
                                    void* workspace, size_t workspace_bytes, void* stream) {
  pa_status s = check_multi_desc(desc);
  if (s != PA_OK) return s;
  if (!query_start || !k_cache || !v_cache || !block_tables || !context_lens)
    return PA_ERR_INVALID_ARG;
  if (desc->total_queries > 0 && (!q || !out || !aligned(q, 16) || !aligned(out, 16)))
    return PA_ERR_INVALID_ARG;
  if (!aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(block_tables, 4) ||
      !aligned(context_lens, 4) || !aligned(query_start, 4))
    return PA_ERR_INVALID_ARG;
  const bool fp8 = desc->cache.kv_dtype == PA_FP8_E4M3;
  if (fp8 && (!k_scale || !v_scale || !aligned(k_scale, 4) || !aligned(v_scale, 4)))
    return PA_ERR_INVALID_ARG;
  if (!fp8 && (k_scale || v_scale)) return PA_ERR_INVALID_ARG;
  const pa::MultiPlan p = multi_plan_of(desc);
  const size_t need = pa::multi_workspace_bytes(p, desc->total_queries, desc->num_q_heads,
                                                desc->cache.head_dim);
  if (desc->total_queries == 0) return PA_OK;                // no rows: nothing to do
  if (need > 0 && (!workspace || workspace_bytes < need || !aligned(workspace, 16)))
    return PA_ERR_WORKSPACE;

  pa::MultiArgs a;
  a.q = q;
  a.query_start = query_start;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.out = out;
  a.split_rt = p.split_rt;
  a.total_lanes = 0;
  a.ws_cnt = nullptr;
  if (p.split_rt > 0) {
    const pa::SplitLayout lay = pa::split_layout(p, desc->cache.head_dim);
    int64_t wgs = resident_split_wgs(desc, p.split_rt);
    if (wgs > p.split_wgs) wgs = p.split_wgs;
    a.total_lanes = (int)(wgs * (pa::kWaves / p.split_waves));
    a.ws_cnt = static_cast<int*>(workspace);
    a.ws_acc = reinterpret_cast<float*>(static_cast<char*>(workspace) + lay.acc);
    a.ws_ml = reinterpret_cast<float*>(static_cast<char*>(workspace) + lay.ml);
  } else if (need > 0) {
    const pa::PartsLayout lay =
        pa::parts_layout(p, desc->total_queries, desc->num_q_heads, desc->cache.head_dim);
    a.ws_acc = reinterpret_cast<float*>(static_cast<char*>(workspace) + lay.acc);
    a.ws_ml = reinterpret_cast<float*>(static_cast<char*>(workspace) + lay.ml);
  } else {
    a.ws_acc = a.ws_ml = nullptr;
  }
  a.batch = desc->batch;
  a.num_q_heads = desc->num_q_heads;
  a.num_kv_heads = desc->cache.num_kv_heads;
  a.group = desc->num_q_heads / desc->cache.num_kv_heads;
  a.num_blocks = desc->cache.num_blocks;
  a.max_blocks_per_seq = desc->max_blocks_per_seq;
  a.len_cap = multi_len_cap(desc);
  a.total_queries = desc->total_queries;
  a.max_query_len = desc->max_query_len;
  a.tiles_per_head = p.tiles_per_head;
  a.num_parts = p.num_parts;
  a.part_blocks = p.part_blocks;
  a.total_items = p.items;
  a.row_blocks = p.row_blocks;
  a.chunk_waves = p.chunk_waves;
  a.qk_scale_log2 = scale * 1.4426950408889634f;
  hipError_t e =
      p.split_rt > 0
          ? pa::launch_multi_split(a, desc->cache.head_dim, desc->q_dtype, desc->cache.kv_dtype,
                                   static_cast<hipStream_t>(stream))
          : pa::launch_multi(a, desc->cache.head_dim, desc->q_dtype, desc->cache.kv_dtype,
                             static_cast<hipStream_t>(stream));
  if (e != hipSuccess) {
    g_last_hip_error = (int32_t)e;
    return PA_ERR_HIP;
  }
  return PA_OK;
}

PA_EXPORT pa_status pa_copy_blocks(const pa_cache_desc* cache, int32_t num_pairs,
                                   const int32_t* pairs, void* k_cache, void* v_cache,
                                   float* k_scale, float* v_scale, void* stream) {
  pa_status s = check_cache(cache);
  if (s != PA_OK) return s;
  if (num_pairs < 0) return PA_ERR_INVALID_ARG;
  if (num_pairs == 0) return PA_OK;
  if (num_pairs > INT32_MAX / 2) return PA_ERR_UNSUPPORTED;
  if (!pairs || !k_cache || !v_cache || !aligned(pairs, 4) || !aligned(k_cache, 16) ||
      !aligned(v_cache, 16))
    return PA_ERR_INVALID_ARG;
  const bool fp8 = cache->kv_dtype == PA_FP8_E4M3;
  if (fp8 && (!k_scale || !v_scale || !aligned(k_scale, 4) || !aligned(v_scale, 4)))
    return PA_ERR_INVALID_ARG;
  if (!fp8 && (k_scale || v_scale)) return PA_ERR_INVALID_ARG;
  pa::CopyArgs a;
  a.pairs = pairs;
  a.k_cache = static_cast<uint8_t*>(k_cache);
  a.v_cache = static_cast<uint8_t*>(v_cache);
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.num_blocks = cache->num_blocks;
  a.num_kv_heads = cache->num_kv_heads;
  a.tile_bytes = pa::kBlock * cache->head_dim * (fp8 ? 1 : 2);
  hipError_t e = pa::launch_copy_blocks(a, num_pairs, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) {
    g_last_hip_error = (int32_t)e;
    return PA_ERR_HIP;
  }
  return PA_OK;
}

PA_EXPORT size_t pa_decode_workspace_size(const pa_decode_desc* desc) {
  if (check_decode_desc(desc) != PA_OK) return 0;
  return workspace_bytes_of(desc);
}

namespace {

// pa_decode, and with k_new/v_new set, pa_decode_append.
// Host-visible checks of a decode call's descriptor and pointers (the workspace aside).
pa_status check_decode_args(const pa_decode_desc* desc, const void* q, const void* k_cache,
                            const void* v_cache, const float* k_scale, const float* v_scale,
                            const int32_t* block_tables, const int32_t* context_lens,
                            const void* out) {
  pa_status s = check_decode_desc(desc);
  if (s != PA_OK) return s;
  if (!q || !k_cache || !v_cache || !block_tables || !context_lens || !out)
    return PA_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(out, 16) ||
      !aligned(block_tables, 4) || !aligned(context_lens, 4))
    return PA_ERR_INVALID_ARG;
  const bool fp8 = desc->cache.kv_dtype == PA_FP8_E4M3;
  if (fp8 && (!k_scale || !v_scale || !aligned(k_scale, 4) || !aligned(v_scale, 4)))
    return PA_ERR_INVALID_ARG;
  if (!fp8 && (k_scale || v_scale)) return PA_ERR_INVALID_ARG;
  return PA_OK;
}

pa_status decode_impl(const pa_decode_desc* desc, const void* q, const void* k_new,
                      const void* v_new, const void* k_cache, const void* v_cache,
                      const float* k_scale, const float* v_scale, const int32_t* block_tables,
                      const int32_t* context_lens, float scale, void* out, void* workspace,
                      size_t workspace_bytes, void* stream) {
  pa_status s = check_decode_args(desc, q, k_cache, v_cache, k_scale, v_scale, block_tables,
                                  context_lens, out);
  if (s != PA_OK) return s;
  const bool fp8 = desc->cache.kv_dtype == PA_FP8_E4M3;

  const size_t need = workspace_bytes_of(desc);
  if (!workspace || workspace_bytes < need || !aligned(workspace, 16)) return PA_ERR_WORKSPACE;

  const int64_t cap_chunks = chunk_capacity(desc);
  int64_t waves = cap_chunks;
  // Short heads: WPH waves per head, one step each, when every head fits the resident waves.
  const int64_t heads = (int64_t)desc->batch * desc->cache.num_kv_heads;
  const int max_blocks = (len_cap(desc) + pa::kBlock - 1) / pa::kBlock;
  int wph = 1;
  while (2 * wph < max_blocks) wph *= 2;
  const bool head_mode = desc->partition_tokens == 0 && max_blocks <= pa::kHeadModeBlocks &&
                         heads * wph <= resident_waves(desc);
  if (head_mode) {
    waves = (heads * wph + pa::kWaves - 1) / pa::kWaves * pa::kWaves;
    if (waves < pa::kWaves) waves = pa::kWaves;
  } else if (desc->partition_tokens == 0) {
    const int64_t resident = resident_waves(desc) * PA_WAVE_ROUNDS;
    if (resident > 0 && resident < waves) waves = resident / pa::kWaves * pa::kWaves;
    if (waves < pa::kWaves) waves = pa::kWaves;
  }
  const pa::WorkspaceLayout lay = layout_of(desc);
  char* ws = static_cast<char*>(workspace);
  const bool share = sharing_active(desc);

  pa::DecodeArgs a;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.k_new = static_cast<const uint8_t*>(k_new);
  a.v_new = static_cast<const uint8_t*>(v_new);
  a.out = out;
  a.ws_cnt = reinterpret_cast<int*>(ws);
  a.ws_acc = reinterpret_cast<float*>(ws + lay.acc);
  a.ws_ml = reinterpret_cast<float*>(ws + lay.ml);
  a.ws_skip = share ? reinterpret_cast<int*>(ws + lay.plan) : nullptr;
  a.gp_acc = share ? reinterpret_cast<float*>(ws + lay.gp_acc) : nullptr;
  a.gp_ml = share ? reinterpret_cast<float*>(ws + lay.gp_ml) : nullptr;
  a.prefix_parts = share ? pa::prefix_parts_of(desc->max_blocks_per_seq) : 0;
  a.plan_units = share ? reinterpret_cast<int*>(ws + lay.units) : nullptr;
  a.plan_reuse = share && desc->shared_prefixes == 2 ? 1 : 0;
  a.plan_sig = share ? plan_signature(desc, lay) : 0;
  a.batch = desc->batch;
  a.num_q_heads = desc->num_q_heads;
  a.num_kv_heads = desc->cache.num_kv_heads;
  a.group = desc->num_q_heads / desc->cache.num_kv_heads;
  a.num_blocks = desc->cache.num_blocks;
  a.max_blocks_per_seq = desc->max_blocks_per_seq;
  a.len_cap = len_cap(desc);
  a.chunk_blocks = desc->partition_tokens / pa::kBlock;
  a.total_waves = (int)waves;
  a.head_mode = head_mode ? wph : 0;
  a.qk_scale_log2 = scale * 1.4426950408889634f;

  // prefix workgroups: one per resident slot, never more than the plan can have units
  int64_t prefix_wgs = 0;
  if (share) {
    const int64_t units =
        (int64_t)pa::plan_tiles_of(desc->batch) * a.num_kv_heads * a.prefix_parts;
    prefix_wgs = resident_waves(desc) / pa::kWaves;
    if (prefix_wgs < 1) prefix_wgs = 1;
    if (prefix_wgs > units) prefix_wgs = units;
  }
  // The append goes into the decode launch (the wave that reads a head's last block writes the
  // token there) unless the batch has at least one append per launched wave: then waves append
  // to several short heads each, and the stores stall their streams more than a launch of its
  // own costs (measured: 256 sequences x 8 KV heads on 2048 waves, 232.7 us fused against
  // 224.2 us with the separate append; 512 appends on 2048 waves, fused equal or faster).
  hipError_t e = hipSuccess;
  if (k_new && !head_mode && heads >= waves) {
    pa::LastAppendArgs ap;
    ap.k_new = a.k_new;
    ap.v_new = a.v_new;
    ap.block_tables = block_tables;
    ap.context_lens = context_lens;
    ap.k_cache = static_cast<uint8_t*>(const_cast<void*>(k_cache));
    ap.v_cache = static_cast<uint8_t*>(const_cast<void*>(v_cache));
    ap.num_blocks = desc->cache.num_blocks;
    ap.num_kv_heads = desc->cache.num_kv_heads;
    ap.head_dim = desc->cache.head_dim;
    ap.max_blocks_per_seq = desc->max_blocks_per_seq;
    ap.len_cap = a.len_cap;
    e = pa::launch_append_last(ap, desc->batch, fp8 ? 1 : 2, static_cast<hipStream_t>(stream));
    a.k_new = a.v_new = nullptr;
  }
  if (e == hipSuccess)
    e = pa::launch_decode(a, desc->cache.head_dim, desc->q_dtype, desc->cache.kv_dtype,
                          (int)prefix_wgs, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) {
    g_last_hip_error = (int32_t)e;
    return PA_ERR_HIP;
  }
  return PA_OK;
}

}  // namespace

PA_EXPORT pa_status pa_decode(const pa_decode_desc* desc, const void* q, const void* k_cache,
                              const void* v_cache, const float* k_scale, const float* v_scale,
                              const int32_t* block_tables, const int32_t* context_lens,
                              float scale, void* out, void* workspace, size_t workspace_bytes,
                              void* stream) {
  return decode_impl(desc, q, nullptr, nullptr, k_cache, v_cache, k_scale, v_scale,
                     block_tables, context_lens, scale, out, workspace, workspace_bytes, stream);
}

PA_EXPORT pa_status pa_decode_append(const pa_decode_desc* desc, const void* q,
                                     const void* k_new, const void* v_new, void* k_cache,
                                     void* v_cache, const float* k_scale, const float* v_scale,
                                     const int32_t* block_tables, const int32_t* context_lens,
                                     float scale, void* out, void* workspace,
                                     size_t workspace_bytes, void* stream) {
  if (!k_new || !v_new || !aligned(k_new, 16) || !aligned(v_new, 16)) return PA_ERR_INVALID_ARG;
  return decode_impl(desc, q, k_new, v_new, k_cache, v_cache, k_scale, v_scale, block_tables,
                     context_lens, scale, out, workspace, workspace_bytes, stream);
}

// ---- pa_decode_noalloc: pa_decode with the library's own scratch, for callers that cannot
// allocate device memory.  The scratch is a static device array; each GPU the library runs on
// holds its own copy (PA_NOALLOC_SCRATCH_BYTES) until the process ends.  In host code its name
// stands for a host-side symbol, so its device address on each GPU is taken once with
// hipGetSymbolAddress and only that address is ever passed on.
static __device__ __align__(256) uint8_t scratch[PA_NOALLOC_SCRATCH_BYTES];

namespace {

// Zero-fills n 32-bit words (the arrival counters of a fresh scratch).
__global__ void clear_words_kernel(uint32_t* p, int n) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x)
    p[i] = 0u;
}

std::mutex g_scratch_mu;
std::map<int, void*> g_scratch;   // device -> the device address of `scratch` there

// The scratch of the current device; its first use on a device also enqueues, on `stream`, the
// clearing of the arrival counters (the decode kernels leave them at zero after every call).
pa_status scratch_of_current_device(hipStream_t stream, void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    g_last_hip_error = (int32_t)e;
    return PA_ERR_HIP;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  auto it = g_scratch.find(dev);
  if (it != g_scratch.end()) {
    *ptr = it->second;
    return PA_OK;
  }
  void* p = nullptr;
  e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
  if (e != hipSuccess || p == nullptr) {
    g_last_hip_error = (int32_t)(e != hipSuccess ? e : hipErrorInvalidSymbol);
    return PA_ERR_HIP;
  }
  const int words = (int)(pa::kMaxWorkgroups * sizeof(int) / sizeof(uint32_t));
  hipLaunchKernelGGL(clear_words_kernel, dim3(64), dim3(256), 0, stream,
                     static_cast<uint32_t*>(p), words);
  e = hipGetLastError();
  if (e != hipSuccess) {
    g_last_hip_error = (int32_t)e;
    return PA_ERR_HIP;
  }
  g_scratch[dev] = p;
  *ptr = p;
  return PA_OK;
}

}  // namespace

PA_EXPORT pa_status pa_decode_noalloc(const pa_decode_desc* desc, const void* q,
                                      const void* k_cache, const void* v_cache,
                                      const float* k_scale, const float* v_scale,
                                      const int32_t* block_tables, const int32_t* context_lens,
                                      float scale, void* out, void* stream) {
  pa_status s = check_decode_args(desc, q, k_cache, v_cache, k_scale, v_scale, block_tables,
                                  context_lens, out);
  if (s != PA_OK) return s;
  if (workspace_bytes_of(desc) > (size_t)PA_NOALLOC_SCRATCH_BYTES) return PA_ERR_UNSUPPORTED;
  void* ws = nullptr;
  s = scratch_of_current_device(static_cast<hipStream_t>(stream), &ws);
  if (s != PA_OK) return s;
  return decode_impl(desc, q, nullptr, nullptr, k_cache, v_cache, k_scale, v_scale,
                     block_tables, context_lens, scale, out, ws, PA_NOALLOC_SCRATCH_BYTES,
                     stream);
}

// ---- HIP graphs of whole steps.  The entry points above enqueue kernels only (no allocation,
// no memset, no synchronisation), so a step of several of them can be captured once and
// replayed with a single launch.
struct pa_graph {
  hipGraph_t graph;
  hipGraphExec_t exec;
};

PA_EXPORT pa_status pa_graph_begin(void* stream) {
  if (!stream) return PA_ERR_INVALID_ARG;   // the legacy null stream cannot be captured
  const hipError_t e = hipStreamBeginCapture(static_cast<hipStream_t>(stream),
                                             hipStreamCaptureModeThreadLocal);
  if (e != hipSuccess) {
    g_last_hip_error = (int32_t)e;
    return PA_ERR_HIP;
  }
  return PA_OK;
}

PA_EXPORT pa_status pa_graph_end(void* stream, pa_graph** graph) {
  if (!stream || !graph) return PA_ERR_INVALID_ARG;
  *graph = nullptr;
  hipGraph_t g = nullptr;
  hipError_t e = hipStreamEndCapture(static_cast<hipStream_t>(stream), &g);
  if (e != hipSuccess) {
    g_last_hip_error = (int32_t)e;
    return PA_ERR_HIP;
  }
  hipGraphExec_t x = nullptr;
  e = hipGraphInstantiate(&x, g, nullptr, nullptr, 0);
  if (e != hipSuccess) {
    (void)hipGraphDestroy(g);
    g_last_hip_error = (int32_t)e;
    return PA_ERR_HIP;
  }
  *graph = new pa_graph{g, x};
  return PA_OK;
}

PA_EXPORT pa_status pa_graph_launch(const pa_graph* graph, void* stream) {
  if (!graph) return PA_ERR_INVALID_ARG;
  const hipError_t e = hipGraphLaunch(graph->exec, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) {
    g_last_hip_error = (int32_t)e;
    return PA_ERR_HIP;
  }
  return PA_OK;
}

PA_EXPORT pa_status pa_graph_destroy(pa_graph* graph) {
  if (!graph) return PA_OK;
  (void)hipGraphExecDestroy(graph->exec);
  (void)hipGraphDestroy(graph->graph);
  delete graph;
  return PA_OK;
}
