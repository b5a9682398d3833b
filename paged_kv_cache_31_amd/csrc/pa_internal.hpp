// Internal launch interface between the C ABI (pa_api.hip) and the kernel translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pa {

constexpr int kBlock = 16;          // tokens per physical KV block
constexpr int kStepTokens = 32;     // tokens one wave consumes per step (two blocks)
#ifndef PA_WG_WAVES
#define PA_WG_WAVES 8
#endif
constexpr int kWaves = PA_WG_WAVES;  // waves per decode workgroup (4: two per CU, 8: one per CU)
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

// The append of a decode step (token L-1 of every sequence, slots from the block tables).
struct LastAppendArgs {
  const uint8_t* k_new;        // [batch][num_kv_heads][head_dim]
  const uint8_t* v_new;
  const int32_t* block_tables;
  const int32_t* context_lens;
  uint8_t* k_cache;
  uint8_t* v_cache;
  int num_blocks;
  int num_kv_heads;
  int head_dim;
  int max_blocks_per_seq;
  int len_cap;
};

struct QuantAppendArgs {
  const uint8_t* k_new;  // [T][num_kv_heads][head_dim] 16-bit
  const uint8_t* v_new;
  const int64_t* slots;
  uint8_t* k_cache;      // fp8 pools
  uint8_t* v_cache;
  float* k_scale;        // [num_blocks][num_kv_heads]
  float* v_scale;
  int64_t num_slots;
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
  const uint8_t* k_new;   // fused append: [batch][num_kv_heads][head_dim] (null: decode only)
  const uint8_t* v_new;
  void* out;
  int* ws_cnt;          // [kMaxWorkgroups] arrival counters, zero between calls
  float* ws_acc;        // [workgroups][2][group][head_dim]: unnormalised output of a cut group
  float* ws_ml;         // [workgroups][2][group][2]: running max (log2 units), exp-sum
  // Shared-prefix plan and prefix partial results (all null when shared prefixes are off).
  int* ws_skip;         // [batch]: leading blocks of each sequence the prefix kernel covers
  float* gp_acc;        // [batch * num_q_heads][prefix_parts][head_dim]: unnormalised output
  float* gp_ml;         // [batch * num_q_heads][prefix_parts][2]: running max (log2), exp-sum
  int prefix_parts;     // partial results per query row: ceil(min(table width, 256) / 16)
  // The plan's units, saved by a planning call for calls that reuse it (the layers of one step
  // read the same tables): [0] the unit count, then kUnitRec ints per unit from kUnitHead on.
  int* plan_units;
  int plan_reuse;       // 1: take the saved units instead of planning (and keep ws_skip)
  int plan_sig;         // signature of the descriptor and workspace layout: a planning call
                        // saves it beside the unit count, a reusing call takes the saved plan
                        // only if it finds its own there (else it runs without shared blocks)
  int batch;
  int num_q_heads;
  int num_kv_heads;
  int group;            // num_q_heads / num_kv_heads, 1..16
  int num_blocks;
  int max_blocks_per_seq;
  int len_cap;          // context lengths are clamped to [0, len_cap]
  int chunk_blocks;     // fixed chunk length in blocks, or 0: balanced over total_waves
  int total_waves;      // waves launched (kWaves per workgroup); chunk c is wave c's
  int head_mode;        // 0, or WPH (1, 2, 4 or 8): short heads, WPH waves per sequence head
                        // in head order, each wave one step of its head (no scan, nothing
                        // crosses workgroups)
  float qk_scale_log2;  // scale * log2(e)
};

// Head mode: with no fixed partition and every head at most 2 * kWaves blocks, when the heads
// fit the resident waves at WPH = (blocks / 2 rounded up to a power of two) waves each.
constexpr int kHeadModeBlocks = 2 * kWaves;

// Shared prefixes.  Sequences whose block tables start with the same physical blocks are
// grouped; each group is cut into tiles of up to 16/group members (one MFMA column per query
// head of a member), and a tile's shared blocks are read in units of kUnitBlocks blocks per KV
// head.
constexpr int kPlanMaxBatch = 1024;   // groups are formed for batches up to this size
constexpr int kUnitBlocks = 32;       // shared blocks one prefix workgroup reads per unit
constexpr int kMaxSharedBlocks = 256; // longest shared prefix taken (blocks)

// Groups have at least two members and tiles at least two columns of members, so a batch of n
// sequences makes at most floor(2n/3) tiles (groups of three, two tiles each, are the worst case).
__host__ __device__ inline int plan_tiles_of(int batch) {
  return 2 * batch / 3 > 0 ? 2 * batch / 3 : 1;
}
// A saved unit: lead sequence, shared blocks [j0, j1), KV head, part index, then the member
// sequence of each of the 16 tile slots (-1: none).
constexpr int kUnitRec = 24;
constexpr int kUnitMembers = 8;       // offset of the member slots in a record
constexpr int kUnitHead = 64;         // ints before the first record: the count, the signature
                                      // and its complement, padding
inline int prefix_parts_of(int max_blocks_per_seq) {
  const int m = max_blocks_per_seq < kMaxSharedBlocks ? max_blocks_per_seq : kMaxSharedBlocks;
  return (m + kUnitBlocks - 1) / kUnitBlocks;
}

// Workspace: a fixed region of arrival counters (so that their place never depends on the
// descriptor and a workspace zero-filled once stays valid for every call), then two published
// partial results per workgroup; with shared prefixes, each sequence's skipped block count, the
// prefix partial results and the saved units follow.  Each part is 256-byte aligned.
constexpr long kMaxWorkgroups = 65536;
struct WorkspaceLayout {
  size_t acc, ml, plan, gp_acc, gp_ml, units, total;
};
inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
inline WorkspaceLayout workspace_layout(int group, int head_dim, long workgroups, int batch = 0,
                                        int num_q_heads = 0, int prefix_parts = 0) {
  WorkspaceLayout w;
  w.acc = align256((size_t)kMaxWorkgroups * sizeof(int));
  w.ml = w.acc + align256((size_t)workgroups * 2 * group * head_dim * sizeof(float));
  w.plan = w.ml + align256((size_t)workgroups * 2 * group * 2 * sizeof(float));
  w.gp_acc = w.gp_ml = w.units = w.total = w.plan;
  if (prefix_parts > 0) {
    const size_t rows = (size_t)batch * num_q_heads * prefix_parts;
    const size_t units = (size_t)plan_tiles_of(batch) * (num_q_heads / group) * prefix_parts;
    w.gp_acc = w.plan + align256((size_t)batch * sizeof(int));
    w.gp_ml = w.gp_acc + align256(rows * head_dim * sizeof(float));
    w.units = w.gp_ml + align256(rows * 2 * sizeof(float));
    w.total = w.units + align256((kUnitHead + units * kUnitRec) * sizeof(int));
  }
  return w;
}

// Waves launched by the balanced mode never exceed this (a workspace bound known without a GPU).
constexpr long kMaxWaves = 8192;

// Several query tokens per sequence (pa_decode_multi).  The query rows of one (sequence, KV
// head) are (token i, group member g) pairs in the order i * group + g, cut into tiles of 16
// (one MFMA column each); each tile's keys are cut into partitions of part_blocks blocks.  An
// item is one (sequence, KV head, partition, tile), handled by one wave.
struct MultiArgs {
  const void* q;               // [total_queries][num_q_heads][head_dim]
  const int32_t* query_start;  // [batch + 1]: rows of sequence b are query_start[b] ..
  const void* k_cache;
  const void* v_cache;
  const float* k_scale;
  const float* v_scale;
  const int32_t* block_tables;
  const int32_t* context_lens;
  void* out;                   // [total_queries][num_q_heads][head_dim]
  float* ws_acc;               // [total_queries * num_q_heads][num_parts][head_dim] (num_parts > 1)
  float* ws_ml;                // [total_queries * num_q_heads][num_parts][2]: max (log2), exp-sum
  int batch;
  int num_q_heads;
  int num_kv_heads;
  int group;
  int num_blocks;
  int max_blocks_per_seq;
  int len_cap;                 // context lengths are clamped to [0, len_cap]
  int total_queries;
  int max_query_len;           // query counts are clamped to [0, max_query_len]
  int tiles_per_head;          // ceil(max_query_len * group / 16)
  int num_parts;
  int part_blocks;             // blocks per key partition (even unless partition_tokens fixes it)
  long long total_items;
  int row_blocks;              // > 0: chunk_kernel, this many row blocks per head
  int chunk_waves;             // chunk_kernel: waves per workgroup (kChunkWide or kChunkPingPong)
  // Balanced split (multi_split_kernel): split_rt > 0 row tiles per head.
  int split_rt;
  int total_lanes;             // chunks of the flattened block space
  int* ws_cnt;                 // [kMaxWorkgroups] arrival counters, zero between calls
  float qk_scale_log2;
};

constexpr int kMultiWaves = 4;             // waves per multi_kernel workgroup
constexpr long kMultiTargetWaves = 4096;   // waves the automatic partition aims for (multi_kernel)
constexpr int kMultiMinPartBlocks = 16;    // automatic partitions are at least 256 tokens

// Heads with more query rows than multi_split_kernel takes (more than four MFMA tiles) go to
// chunk_kernel: a workgroup takes a block of rows of one head and stages each K/V step once in
// LDS for all of them: 128 rows (4 waves x 2 tiles), or for heads of at least 256 rows (prefill
// chunks) 256 rows in 8 waves whose two halves ping-pong between softmax and matrix products.
struct ChunkShape {
  int waves, tiles;            // waves per workgroup, 16-column tiles per wave
};
constexpr ChunkShape kChunkWide = {4, 2};
constexpr ChunkShape kChunkPingPong = {8, 2};
constexpr int kCUs = 256;                   // compute units of an MI355X
constexpr int kChunkMinPartBlocks = 32;
// chunk_kernel over 16-bit caches in the ping-pong shape holds its partition's block ids in LDS:
// its partitions are at most this many blocks (32768 tokens)
constexpr int kDirectMaxBlocks = 2048;     // chunk_kernel's own key partitions: 512+ tokens

struct MultiPlan {
  int tiles_per_head, num_parts, part_blocks;
  long long items;             // waves (multi_kernel) or workgroups (chunk_kernel)
  int row_blocks;              // > 0: chunk_kernel, this many row blocks per head
  int chunk_waves;             // chunk_kernel: waves per workgroup
  int split_rt;                // > 0: multi_split_kernel with this many row tiles per head
  int split_waves;             // multi_split_kernel: waves per chunk
  long long split_wgs;         // multi_split_kernel: most workgroups a launch may use
};

// multi_split_kernel takes heads of up to four row tiles: one or two in one wave, three or
// four (three laid out as four) in two paced waves of two.  Two 16-bit tiles at head_dim 128
// fit a wave's registers only with the stepper's rolling schedule (one K/V register set).  A
// launch is one workgroup per resident slot, at most kMaxSplitWorkgroups (a workspace bound
// known without a GPU: twice the 256 CUs of an MI355X).
constexpr int kSplitMaxTiles = 4;
inline int split_chunk_waves(int tiles) { return tiles > 2 ? 2 : 1; }
constexpr long kMaxSplitWorkgroups = 512;

// Key partitions for `base` independent units so that about `target` units run, each at least
// min_part_blocks blocks long; part_blocks is even unless partition_tokens fixes it.
inline void multi_parts(MultiPlan& p, long long base, long long target, long long maxblk,
                        int partition_tokens, int min_part_blocks = kMultiMinPartBlocks,
                        long long max_part_blocks = 0) {
  long long pb;
  if (partition_tokens > 0) {
    pb = partition_tokens / kBlock;
  } else {
    long long np = (target + base - 1) / (base > 0 ? base : 1);
    const long long np_max = (maxblk + min_part_blocks - 1) / min_part_blocks;
    if (np > np_max) np = np_max;
    if (np < 1) np = 1;
    pb = (maxblk + np - 1) / np;
    pb += pb & 1;
    if (pb < 2) pb = 2;
    if (max_part_blocks > 0 && pb > max_part_blocks) pb = max_part_blocks;   // even
  }
  long long np = (maxblk + pb - 1) / pb;
  if (np < 1) np = 1;
  p.part_blocks = (int)pb;
  p.num_parts = (int)np;
}

// A pure function of the descriptor, so the workspace size is known without a GPU.
inline MultiPlan multi_plan(int batch, int num_kv_heads, int group, int max_query_len,
                            int len_cap, int partition_tokens, int head_dim, bool fp8_kv) {
  MultiPlan p;
  const long long rows = (long long)max_query_len * group;
  const long long maxblk = ((long long)len_cap + kBlock - 1) / kBlock;
  p.tiles_per_head = (int)((rows + 15) / 16);
  p.row_blocks = 0;
  p.chunk_waves = 0;
  p.split_rt = 0;
  p.split_waves = 0;
  p.split_wgs = 0;
  if (partition_tokens == 0 && p.tiles_per_head <= kSplitMaxTiles) {
    // balanced split: equal chunks of the block space, at least two blocks each, so the space
    // never needs more than half its blocks in chunks
    p.split_rt = p.tiles_per_head == 3 ? 4 : p.tiles_per_head;   // 1, 2 or 4 tiles
    p.split_waves = split_chunk_waves(p.split_rt);
    const long long lanes_max = ((long long)batch * num_kv_heads * maxblk + 1) / 2;
    const long long per_wg = kWaves / p.split_waves;
    long long wgs = (lanes_max + per_wg - 1) / per_wg;
    if (wgs > kMaxSplitWorkgroups) wgs = kMaxSplitWorkgroups;
    p.split_wgs = wgs < 1 ? 1 : wgs;
    p.num_parts = 1;
    p.part_blocks = (int)(maxblk + (maxblk & 1));
    p.items = 0;
    return p;
  }
  if (partition_tokens == 0) {   // more than 64 rows (fewer took the split above)
    const ChunkShape sh =
        rows >= 16 * kChunkPingPong.waves * kChunkPingPong.tiles ? kChunkPingPong : kChunkWide;
    const int block_rows = 16 * sh.waves * sh.tiles;
    p.chunk_waves = sh.waves;
    p.row_blocks = (int)((rows + block_rows - 1) / block_rows);
    // Too few row blocks to fill the chip (a small batch of long prompts): the keys are cut
    // into partitions as well, merged afterwards like multi_kernel's.
    const long long wgs = (long long)batch * num_kv_heads * p.row_blocks;
    const bool direct = sh.waves == kChunkPingPong.waves && !fp8_kv;
    multi_parts(p, wgs, (long long)kCUs * (8 / sh.waves), maxblk, 0, kChunkMinPartBlocks,
                direct ? kDirectMaxBlocks : 0);
    p.items = wgs * p.num_parts;
    return p;
  }
  multi_parts(p, (long long)batch * num_kv_heads * (p.tiles_per_head > 0 ? p.tiles_per_head : 1),
              kMultiTargetWaves, maxblk, partition_tokens);
  p.items = (long long)batch * num_kv_heads * p.num_parts * p.tiles_per_head;
  return p;
}
// Balanced split workspace: the arrival counters (the same fixed region as the decode's), then
// two published parts per (workgroup, row tile): an fp32 output row per column and its max and
// exp-sum.
struct SplitLayout {
  size_t acc, ml, total;
};
inline SplitLayout split_layout(const MultiPlan& p, int head_dim) {
  SplitLayout w;
  const size_t cols = (size_t)p.split_wgs * 2 * p.split_rt * 16;
  w.acc = align256((size_t)kMaxWorkgroups * sizeof(int));
  w.ml = w.acc + align256(cols * head_dim * sizeof(float));
  w.total = w.ml + align256(cols * 2 * sizeof(float));
  return w;
}
// Fixed partitions: the same counter region first (left untouched, so one zero-filled
// workspace serves every call on a stream), then per (query row, head, partition) an fp32
// output row and its max and exp-sum.
struct PartsLayout {
  size_t acc, ml, total;
};
inline PartsLayout parts_layout(const MultiPlan& p, int total_queries, int num_q_heads,
                                int head_dim) {
  PartsLayout w;
  const size_t rows = (size_t)total_queries * num_q_heads * p.num_parts;
  w.acc = align256((size_t)kMaxWorkgroups * sizeof(int));
  w.ml = w.acc + align256(rows * head_dim * sizeof(float));
  w.total = w.ml + align256(rows * 2 * sizeof(float));
  return w;
}
inline size_t multi_workspace_bytes(const MultiPlan& p, int total_queries, int num_q_heads,
                                    int head_dim) {
  if (p.split_rt > 0) return split_layout(p, head_dim).total;
  if (p.num_parts <= 1) return 0;
  return parts_layout(p, total_queries, num_q_heads, head_dim).total;
}

struct CopyArgs {
  const int32_t* pairs;   // [n][2] (source block, target block), device
  uint8_t* k_cache;
  uint8_t* v_cache;
  float* k_scale;         // fp8 caches only (else null)
  float* v_scale;
  int num_blocks;
  int num_kv_heads;
  int tile_bytes;         // 16 * head_dim * element bytes
};
hipError_t launch_copy_blocks(const CopyArgs& a, int n, hipStream_t stream);

hipError_t launch_append(const AppendArgs& a, int num_tokens, int elem_bytes, hipStream_t stream);
hipError_t launch_append_last(const LastAppendArgs& a, int batch, int elem_bytes,
                              hipStream_t stream);
hipError_t launch_append_quant(const QuantAppendArgs& a, int num_tokens, bool bf16_src,
                               bool first_token_scale, hipStream_t stream);
// Enqueues the decode; with a.ws_skip set, the prefix kernel runs first (prefix_wgs workgroups).
hipError_t launch_decode(const DecodeArgs& a, int head_dim, int q_dtype, int kv_dtype,
                         int prefix_wgs, hipStream_t stream);
// Enqueues multi_kernel and, with more than one partition, the merge.
hipError_t launch_multi(const MultiArgs& a, int head_dim, int q_dtype, int kv_dtype,
                        hipStream_t stream);
// Enqueues multi_split_kernel (a.split_rt row tiles per head, a.total_lanes chunks).
hipError_t launch_multi_split(const MultiArgs& a, int head_dim, int q_dtype, int kv_dtype,
                              hipStream_t stream);
// Resident multi_split_kernel workgroups per CU for this instance (0 if the query fails).
int multi_split_workgroups_per_cu(int head_dim, int q_dtype, int kv_dtype, int rt);
// Resident decode workgroups per CU for this kernel instance (0 if the query fails).
int decode_workgroups_per_cu(int head_dim, int q_dtype, int kv_dtype);

}  // namespace pa
