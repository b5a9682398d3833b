/*
 * pa.h -- paged decode attention for AMD Instinct MI355X (gfx950): the C ABI.
 *
 * Two operations on a PagedAttention KV cache, as the pages state the problem:
 *
 *  - pa_kv_append: each generation step stores the new token's K and V rows in the cache
 *    (Scaling Book note on notes.yuuk.io, "Transformer 推論の基礎: Prefill と Generation"; the
 *    youngju.dev serving guide's KV-cache module).  In the paged cache the token goes to one slot
 *    of a fixed-size block (kasblo.com vLLM explainer, "blockはrequestの成長に合わせて割り当てる").
 *
 *  - pa_decode: single-query attention of each sequence's new query over all of its cached
 *    tokens, reading K/V through a per-sequence block table that maps logical blocks to
 *    scattered physical blocks (kasblo.com, "PagedAttentionはKV Cacheをblockで管理する";
 *    youngju.dev guide, PagedAttention block-table figure), with grouped-query heads
 *    (Scaling Book note, "生成スループット/レイテンシ改善のテクニック") and an online softmax
 *    (babushkai.com "GPU推論の内部構造", FlashAttention section).  The keys of the whole batch
 *    are split into chunks of equal length, one per GPU wave, whatever the mix of context
 *    lengths; a sequence cut between chunks has its partial results merged by log-sum-exp.
 *
 * Cache layout (one "tile" = one physical block of one KV head, contiguous in memory):
 *   k_cache  [num_blocks][num_kv_heads][16][head_dim]   token-major: a token's K row is contiguous
 *   v_cache  [num_blocks][num_kv_heads][head_dim][16]   dim-major: one dimension's 16 token values
 *                                                         are contiguous
 *   slot s   = physical_block * 16 + offset_in_block
 *   fp8 caches store OCP e4m3fn codes; the real value is code * scale[block][kv_head], with one
 *   fp32 scale per (physical block, KV head), separate arrays for K and V.
 *
 * Query head h reads KV head h / (num_q_heads / num_kv_heads).
 *
 * Ownership and execution: every data pointer of the attention and cache calls is a device
 * pointer owned by the caller, and the library never allocates or frees device memory.  Its own
 * state is a thread-local copy of the last HIP error, a per-device cache of the compute-unit
 * count and kernel occupancy, and the host objects the caller creates and destroys explicitly
 * (pa_block_pool, pa_graph).  Calls only enqueue work on `stream` (a hipStream_t; NULL = the default stream)
 * and return without synchronising; the caller orders and synchronises.
 *
 * Errors: conditions the host can see (null pointers, non-positive sizes, unsupported shapes or
 * dtype pairs, misaligned pointers, a short workspace) return a status before anything is
 * launched.  Device-resident values are a caller contract that is not checked on the host (the
 * Python binding's check=True validates it on host copies, for tests); the kernels clamp them
 * so that nothing is ever read or written outside the described arrays:
 *   - a slot outside [0, num_blocks*16) is skipped by pa_kv_append;
 *   - a context length is clamped to [0, min(max_context_len, max_blocks_per_seq*16)];
 *   - a block-table entry outside [0, num_blocks) reads physical block 0 instead
 *     (the result is then unspecified but the call stays in bounds).
 */
#ifndef PA_H
#define PA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum pa_status {
  PA_OK = 0,
  PA_ERR_INVALID_ARG = 1,  /* null pointer, non-positive size, misaligned pointer */
  PA_ERR_UNSUPPORTED = 2,  /* head_dim, block_size, head grouping or dtype pair not implemented */
  PA_ERR_WORKSPACE = 3,    /* workspace NULL or smaller than pa_decode_workspace_size() */
  PA_ERR_HIP = 4,          /* a kernel launch failed; pa_last_hip_error() has the hipError_t */
  PA_ERR_OUT_OF_BLOCKS = 5 /* the block pool has too few free blocks (nothing was changed) */
} pa_status;

typedef enum pa_dtype {
  PA_F16 = 0,              /* IEEE binary16 */
  PA_BF16 = 1,             /* bfloat16 */
  PA_FP8_E4M3 = 2          /* OCP fp8 e4m3fn (bias 7, max 448, no infinities) -- caches only */
} pa_dtype;

/* Geometry of the paged K/V pools, shared by both calls. */
typedef struct pa_cache_desc {
  int32_t num_blocks;      /* physical blocks in each pool, > 0 */
  int32_t num_kv_heads;    /* KV heads per token, > 0 */
  int32_t head_dim;        /* 64 or 128 */
  int32_t block_size;      /* tokens per block; must be 16 */
  int32_t kv_dtype;        /* pa_dtype of the cache elements */
} pa_cache_desc;

typedef struct pa_decode_desc {
  pa_cache_desc cache;
  int32_t batch;              /* sequences, > 0 */
  int32_t num_q_heads;        /* multiple of num_kv_heads with a group size of 1..16 */
  int32_t max_blocks_per_seq; /* row length (stride) of block_tables, > 0 */
  int32_t max_context_len;    /* host-side upper bound on context_lens; sizes the launch without
                                 reading device memory.  0 = max_blocks_per_seq * 16. */
  int32_t partition_tokens;   /* split-KV chunk length in tokens, a multiple of the 16-token
                                 block in [16, 65536]; 0 = chunks of equal length balanced over
                                 the GPU's resident waves (the default, best for ragged batches) */
  int32_t q_dtype;            /* PA_F16 or PA_BF16; the output has the same dtype */
  int32_t shared_prefixes;    /* 0, 1 or 2.  1: sequences whose block tables start with the same
                                 physical blocks (a prefix cache shares blocks this way: youngju.dev
                                 LLM inference guide, PagedAttention "主な特性" and its prefix-
                                 caching example; Scaling Book note, "プレフィックスキャッシュ") read
                                 those blocks once per group of up to 16/group sequences instead of
                                 once each.  Taken when group <= 8 and batch <= 1024, else ignored.
                                 The result is the same attention up to rounding order.
                                 2: the same, reusing the grouping that the last call with 1 left in
                                 this workspace instead of planning again: for the layers of one
                                 step, and for later steps while the batch keeps its sequences.
                                 The reusing call checks the saved grouping against its own
                                 block_tables and context_lens: a member whose shared entries
                                 now differ from its leader's, or whose length no longer leaves
                                 it a block past the shared ones, reads its whole head instead
                                 (sequences that came to share blocks since the plan are read
                                 unshared until a call with 1 plans again).  With tables and
                                 lengths unchanged the results are bitwise those of a call with
                                 1.  The planning call saves a signature of its descriptor and
                                 workspace layout with the plan; a reusing call that finds
                                 another signature there (a workspace no planning call has
                                 written, another descriptor, or scratch of another call written
                                 over it) reads no shared blocks and gives the unshared results.
                                 Saved plan entries are clamped into range before use, so even a
                                 workspace overwritten in a way the signature misses is never
                                 read or written out of bounds. */
} pa_decode_desc;

typedef struct pa_multi_desc {
  pa_cache_desc cache;
  int32_t batch;              /* sequences, > 0 */
  int32_t num_q_heads;        /* a multiple of num_kv_heads (any group size) */
  int32_t max_blocks_per_seq; /* row length (stride) of block_tables, > 0 */
  int32_t max_context_len;    /* host-side bound on context_lens, as in pa_decode_desc (0: table) */
  int32_t total_queries;      /* rows of q and out, >= 0 */
  int32_t max_query_len;      /* host-side bound on query_start[b+1] - query_start[b], > 0 */
  int32_t partition_tokens;   /* key partition per row tile, a multiple of the 16-token block in
                                 [16, 65536]; 0 = chosen from the shape (see pa_decode_multi) */
  int32_t q_dtype;            /* PA_F16 or PA_BF16; the output has the same dtype */
} pa_multi_desc;

/*
 * pa_kv_append -- write num_tokens new K/V rows into their cache slots.
 *
 *   k_new, v_new  [num_tokens][num_kv_heads][head_dim] elements of cache->kv_dtype, 16-byte
 *                 aligned.  For an fp8 cache they are codes already quantised with the scale of
 *                 the block they go to; the bytes are copied unchanged.
 *   slot_mapping  [num_tokens] int64, 8-byte aligned: token i goes to offset slot%16 of physical
 *                 block slot/16 for every KV head.  A negative slot skips the token (padding).
 *   k_cache, v_cache  the pools described above, updated in place, 16-byte aligned.
 *
 * The copy is exact.  Two tokens with the same slot in one call race (caller error).
 * num_tokens == 0 is a no-op that returns PA_OK.
 */
pa_status pa_kv_append(const pa_cache_desc* cache, int32_t num_tokens,
                       const void* k_new, const void* v_new, const int64_t* slot_mapping,
                       void* k_cache, void* v_cache, void* stream);

/* Scale policies of pa_kv_append_quant. */
typedef enum pa_scale_policy {
  PA_SCALE_KEEP = 0,        /* quantise with the block's stored scale */
  PA_SCALE_FIRST_TOKEN = 1  /* a token written at offset 0 of its block first sets its scale */
} pa_scale_policy;

/*
 * pa_kv_append_quant -- write num_tokens new K/V rows given in 16 bits into an fp8 (e4m3fn)
 * cache, quantising them with the per-(block, KV head) scales (value = code * scale: the FP8 KV
 * cache of design.babushkai.com "GPU推論の内部構造", KV-cache and quantisation sections).
 *
 *   src_dtype     PA_F16 or PA_BF16: the dtype of k_new, v_new [num_tokens][num_kv_heads][head_dim]
 *   slot_mapping  as pa_kv_append (negative or outside the pool: skipped)
 *   k_cache, v_cache  fp8 pools (cache->kv_dtype must be PA_FP8_E4M3), updated in place
 *   k_scale, v_scale  [num_blocks][num_kv_heads] fp32, read, and written under
 *                 PA_SCALE_FIRST_TOKEN
 *   scale_policy  PA_SCALE_KEEP: every row uses its block's stored scale.
 *                 PA_SCALE_FIRST_TOKEN: first, each token of this call at offset 0 of its block
 *                 sets that block's scale, per KV head and separately for K and V, to
 *                 fp32(max |x|) / 448 (1 if the maximum is 0; NaN elements are ignored);
 *                 then all rows are quantised (a token later in a block uses the block's scale
 *                 as it stands and saturates if it is larger).
 *
 * Each element becomes e4m3fn(clamp(fp32(x) / fp32(scale), +-448)): IEEE fp32 division, round to
 * nearest even, sign kept (0x80 for values that round to zero from below), NaN -> 0x7F.  The
 * pages leave the scale policy open; this is one plain reading.  Two tokens with the same slot,
 * or two offset-0 tokens of one block, in one call race (caller error).  Two kernels are
 * enqueued under PA_SCALE_FIRST_TOKEN, one under PA_SCALE_KEEP.
 */
pa_status pa_kv_append_quant(const pa_cache_desc* cache, int32_t num_tokens, int32_t src_dtype,
                             const void* k_new, const void* v_new, const int64_t* slot_mapping,
                             void* k_cache, void* v_cache, float* k_scale, float* v_scale,
                             int32_t scale_policy, void* stream);

/*
 * pa_decode -- out[b][h] = softmax(scale * q[b][h] . K_b^T) . V_b for every sequence b and query
 * head h, where K_b, V_b are the first context_lens[b] tokens of sequence b gathered through
 * block_tables[b] from the KV head of h's group (times the block scales for fp8 caches).
 *
 *   q             [batch][num_q_heads][head_dim] of q_dtype, 16-byte aligned
 *   k_cache, v_cache  pools as above, 16-byte aligned
 *   k_scale, v_scale  [num_blocks][num_kv_heads] fp32 for fp8 caches, 4-byte aligned; must be
 *                 NULL for f16/bf16 caches
 *   block_tables  [batch][max_blocks_per_seq] int32: logical block j of sequence b lives in
 *                 physical block block_tables[b][j]; only j < ceil(context_lens[b]/16) is read
 *   context_lens  [batch] int32, tokens to attend over (including the token appended this step)
 *   scale         softmax scale, usually 1/sqrt(head_dim)
 *   out           [batch][num_q_heads][head_dim] of q_dtype, 16-byte aligned, written (rounded to
 *                 nearest even from fp32); a sequence with context length 0 gets zeros
 *   workspace     device scratch of at least pa_decode_workspace_size(desc) bytes, 16-byte
 *                 aligned (never NULL), zero-filled once before its first use.  Its first
 *                 256 KiB hold arrival counters that every call leaves at zero again, so one
 *                 workspace serves any later call whatever its descriptor; the rest is scratch.
 *                 Calls that share a workspace must not overlap (same stream, or synchronised).
 *
 * Supported pairs (q_dtype, kv_dtype): (F16, F16), (BF16, BF16), (BF16, FP8_E4M3),
 * (F16, FP8_E4M3).  Accumulation is fp32.  Results depend only on logical token positions and
 * on the context lengths of the batch (which set the chunk boundaries), so the same data behind
 * any physical block placement gives bit-identical output (with shared_prefixes 0).  One kernel
 * is enqueued; with shared prefixes taken, a prefix kernel runs before it.
 *
 * Shared prefixes: the sequences whose first block-table entries are equal form a group; the
 * shared length of a group is the number of leading entries every member has in common with the
 * group's first sequence, stops before the block that holds any member's last token and is at
 * most 256 blocks; groups sharing fewer than two blocks are not used.  The shared
 * blocks' partial softmax results are merged into each member's own with the log-sum-exp rule.
 * Results then also depend on the grouping (not on which member gets which MFMA column).
 */
pa_status pa_decode(const pa_decode_desc* desc, const void* q, const void* k_cache,
                    const void* v_cache, const float* k_scale, const float* v_scale,
                    const int32_t* block_tables, const int32_t* context_lens, float scale,
                    void* out, void* workspace, size_t workspace_bytes, void* stream);

/*
 * pa_decode_multi -- causal attention of several new query tokens per sequence over the paged
 * cache: the target model's one-pass check of draft tokens in speculative decoding (youngju.dev
 * guide, speculative-decoding figure; magi-web "Inference Batching", "投機的デコードとの相互作用")
 * and a chunk of a long prompt against the cache built so far (magi-web, "Prefill-Decode 分離 —
 * chunked prefill と disaggregation").
 *
 *   q             [total_queries][num_q_heads][head_dim] of q_dtype, 16-byte aligned
 *   query_start   [batch + 1] int32 (device): sequence b owns rows query_start[b] ..
 *                 query_start[b+1] - 1, T_b of them (clamped to [0, max_query_len]); rows no
 *                 sequence owns are left untouched in out
 *   context_lens  [batch] int32 (device): L_b counts every cached token including the T_b new
 *                 ones, which must already be in the cache (pa_kv_append with their slots)
 *   out           [total_queries][num_q_heads][head_dim] of q_dtype
 *   other arguments as pa_decode
 *
 * Row i of sequence b sits at position p = L_b - T_b + i and gets
 * softmax(scale * q . K[0..p]^T) . V[0..p] with query head h reading KV head h / group; a row
 * with p < 0 sees no token and is zero.  fp32 accumulation; within 2e-3 absolute + 2e-3 relative
 * of the exact result, and the same bits on every call with the same inputs.
 *
 * With partition_tokens 0, heads of at most 64 query rows (T_b * group) get the decode's
 * balanced split-KV: equal chunks of the batch's (sequence, KV head, block) space, each walked
 * by one wave holding the head's 16-row tiles (two waves of two tiles for 33-64 rows), partial
 * results merged by log-sum-exp inside the kernel.  Larger heads take a kernel that
 * stages K/V in LDS for blocks of rows; when those blocks are too few to fill the GPU (a small
 * batch of long contexts) it also cuts the keys into partitions of at least 512 tokens, merged
 * by a second kernel.  A fixed partition_tokens cuts every row tile's keys into partitions
 * merged by a second kernel.
 *
 * The workspace (pa_decode_multi_workspace_size bytes, 16-byte aligned; none when the size is
 * 0) follows pa_decode's contract: zero-filled once before its first use, its first 256 KiB are
 * arrival counters that every call leaves at zero, the rest is scratch; one workspace may serve
 * pa_decode and pa_decode_multi calls alike.  Calls sharing a workspace must not overlap.  A
 * call with total_queries 0 does nothing and needs no workspace.
 */
pa_status pa_decode_multi(const pa_multi_desc* desc, const void* q, const int32_t* query_start,
                          const void* k_cache, const void* v_cache, const float* k_scale,
                          const float* v_scale, const int32_t* block_tables,
                          const int32_t* context_lens, float scale, void* out, void* workspace,
                          size_t workspace_bytes, void* stream);

/* Workspace bytes pa_decode_multi needs for desc (0 if none or if desc is invalid). */
size_t pa_decode_multi_workspace_size(const pa_multi_desc* desc);

/*
 * pa_decode_append -- one whole decode step in one launch: for every sequence b with
 * L_b = context_lens[b] > 0 (clamped as in pa_decode), store the new token's K/V row into
 * token L_b - 1 of the sequence (offset (L_b-1) % 16 of physical block
 * block_tables[b][(L_b-1) / 16], for every KV head), then compute pa_decode over the L_b tokens.
 * It is pa_kv_append with that slot for each sequence followed by pa_decode (each generation
 * step appends the new token's K/V before attending: Scaling Book note, "Transformer 推論の基礎:
 * Prefill と Generation"; youngju.dev guide, KV-cache module), without the second launch and its
 * gap (design.babushkai.com "GPU推論の内部構造": the per-launch cost of decode steps).
 *
 *   k_new, v_new  [batch][num_kv_heads][head_dim] of kv_dtype, 16-byte aligned (fp8: codes
 *                 already quantised with the scale of their block; copied unchanged)
 *   other arguments as pa_decode; k_cache and v_cache are updated in place.
 *
 * The block that receives a sequence's new token must not be read by another sequence of the
 * same call (a block that is appended to is owned by one sequence; shared blocks are copied
 * before they are written).  A block id outside the pool skips that store.  Output equals
 * pa_kv_append + pa_decode bit for bit.
 */
pa_status pa_decode_append(const pa_decode_desc* desc, const void* q, const void* k_new,
                           const void* v_new, void* k_cache, void* v_cache,
                           const float* k_scale, const float* v_scale,
                           const int32_t* block_tables, const int32_t* context_lens, float scale,
                           void* out, void* workspace, size_t workspace_bytes, void* stream);

/*
 * pa_decode_noalloc -- pa_decode without a workspace argument, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  The library keeps its own scratch, a static device array of 64 MiB
 * (PA_NOALLOC_SCRATCH_BYTES) on every GPU it runs on, held until the process ends; it calls no
 * hipMalloc, hipFree or other allocating routine.  Arguments, results and errors are those of
 * pa_decode, plus: a descriptor whose workspace (pa_decode_workspace_size) exceeds 64 MiB returns
 * PA_ERR_UNSUPPORTED before anything is launched (every decode descriptor without shared prefixes
 * needs at most about 17 MiB; shared prefixes add batch * num_q_heads * P * (head_dim + 2) * 4
 * bytes).  The first call on a device also enqueues on `stream` a small kernel that clears the
 * scratch's arrival counters.  Every call on one GPU shares that GPU's scratch, which keeps the
 * last call's contents: calls that overlap on one GPU (other streams, other threads) race, so the
 * caller serialises them.  shared_prefixes 2 reuses a plan that the last pa_decode_noalloc call
 * with 1 left in the scratch, under the rules of pa_decode_desc.
 */
pa_status pa_decode_noalloc(const pa_decode_desc* desc, const void* q, const void* k_cache,
                            const void* v_cache, const float* k_scale, const float* v_scale,
                            const int32_t* block_tables, const int32_t* context_lens,
                            float scale, void* out, void* stream);

/* Bytes of workspace pa_decode needs for this descriptor, or 0 if the descriptor is invalid
 * (pa_decode reports why).  It depends only on the descriptor, not on the GPU:
 * 262144 + workgroups * 2 * group * (head_dim + 2) * 4 bytes (each part rounded up to 256),
 * where workgroups = ceil(chunks / 8): at most 1024 when partition_tokens is 0, else the
 * chunks of partition_tokens / 16 blocks that cover batch * num_kv_heads *
 * ceil(max_context_len / 16) blocks.  Shared prefixes, when taken, add batch * 4 bytes of
 * per-sequence counts and batch * num_q_heads * P * (head_dim + 2) * 4 bytes of partial results
 * with P = ceil(min(max_blocks_per_seq, 256) / 32) (each part rounded up to 256). */
size_t pa_decode_workspace_size(const pa_decode_desc* desc);

/* A static, human-readable name for a status code. */
const char* pa_status_string(pa_status status);

/* The hipError_t of the last failed launch on the calling thread (0 if none). */
int32_t pa_last_hip_error(void);

/*
 * Block sharing and copy-on-write (kasblo.com vLLM explainer, "blockはrequestの成長に合わせて
 * 割り当てる" and "block共有とAutomatic Prefix Caching"): a request takes blocks from a pool of
 * reusable physical blocks as it grows and gives back, when it ends, the blocks only it uses;
 * every block has a reference count (the sequences referring to it), so that sequences forked
 * for parallel sampling or sharing a prefix hold its content once, and a shared block is
 * duplicated only when one of them writes into it.
 *
 * pa_block_pool is a host-side object (one per cache; thread-safe).  A block is free when its
 * count is 0.  Every call validates all its arguments before changing anything; PA_ERR_INVALID_ARG
 * (bad id, sharing or writing a free block, releasing a block more often than it is referred to)
 * and PA_ERR_OUT_OF_BLOCKS (the pool is short: the caller's scheduler preempts) leave the pool
 * unchanged.  Which free block an allocation returns is unspecified (the most recently freed
 * first).
 *
 * pa_pool_create     a pool of num_blocks free blocks (> 0) in *pool.
 * pa_pool_destroy    frees the pool (NULL: no-op).
 * pa_pool_free_blocks, pa_pool_refcount   the free count / a block's count (-1: bad argument).
 * pa_pool_alloc      n blocks, each now referred to once, into blocks[n]; all or nothing.
 * pa_pool_share      one more reference to each listed block (all must be in use): a fork, a
 *                    reused prefix.
 * pa_pool_release    one reference fewer per listed occurrence; a block reaching 0 is free again.
 * pa_pool_write      before writing into `block`: if it is referred to once, *target = block and
 *                    *needs_copy = 0; otherwise the caller's reference moves to a newly allocated
 *                    block *target (count 1), *needs_copy = 1, and the caller must copy block's
 *                    content into it (pa_copy_blocks) before writing.
 * pa_pool_slot_for   the slot of token `pos` of a sequence whose block table (host memory) holds
 *                    *num_blocks entries of max_blocks: a token at the start of a block after the
 *                    last opens a new block (appended to the table); a token in a shared block
 *                    gets a private copy of it (the table entry is replaced and *copy_src,
 *                    *copy_dst name the copy to make; both are -1 when no copy is needed).
 *                    Tokens go in order: pos / 16 must be at most *num_blocks.
 *
 * pa_copy_blocks     for each of num_pairs (source, target) pairs in `pairs` (device memory,
 *                    int32 [num_pairs][2]), copies the K and V tiles of every KV head, and for fp8
 *                    caches the K and V scales, from block source to block target.  Targets must
 *                    be distinct and must not be sources of other pairs in the same call (copy-on-
 *                    write targets are fresh blocks, so this holds).  Pairs with a block outside
 *                    the pool or source == target are skipped.  The copy is exact.
 */
typedef struct pa_block_pool pa_block_pool;
pa_status pa_pool_create(int32_t num_blocks, pa_block_pool** pool);
pa_status pa_pool_destroy(pa_block_pool* pool);
int32_t pa_pool_free_blocks(pa_block_pool* pool);
int32_t pa_pool_refcount(pa_block_pool* pool, int32_t block);
pa_status pa_pool_alloc(pa_block_pool* pool, int32_t n, int32_t* blocks);
pa_status pa_pool_share(pa_block_pool* pool, int32_t n, const int32_t* blocks);
pa_status pa_pool_release(pa_block_pool* pool, int32_t n, const int32_t* blocks);
pa_status pa_pool_write(pa_block_pool* pool, int32_t block, int32_t* target, int32_t* needs_copy);
pa_status pa_pool_slot_for(pa_block_pool* pool, int32_t* table, int32_t* num_blocks,
                           int32_t max_blocks, int32_t pos, int64_t* slot, int32_t* copy_src,
                           int32_t* copy_dst);
pa_status pa_copy_blocks(const pa_cache_desc* cache, int32_t num_pairs, const int32_t* pairs,
                         void* k_cache, void* v_cache, float* k_scale, float* v_scale,
                         void* stream);

/*
 * HIP graphs of whole steps: launching one kernel per layer and call costs a few microseconds
 * each, which a decode step of many layers pays again and again (design.babushkai.com
 * "GPU推論の内部構造": the per-launch overhead of decode and CUDA graphs as its remedy).  Every
 * entry point above only enqueues kernels on the given stream (no allocation, no memset, no
 * synchronisation), so a step made of any sequence of them, for example pa_decode_append for
 * every layer, can be captured once and replayed with one launch.
 *
 * pa_graph_begin  starts capturing the calls made on `stream` (not the null stream) by this
 *                 thread (hipStreamCaptureModeThreadLocal).  Call each entry point once outside
 *                 the capture first on this device, so that its one-time device queries are done.
 * pa_graph_end    ends the capture and instantiates the graph into *graph (NULL on failure).
 * pa_graph_launch replays the captured step on `stream` with the pointers, sizes and scalars
 *                 it was captured with; the buffers they point to are read and written afresh
 *                 each time, so updating the data in place between replays is how a later step
 *                 runs (new tokens, queries, lengths and tables in the same buffers).
 * pa_graph_destroy frees the graph (NULL: no-op).
 * A failure of a HIP call returns PA_ERR_HIP (see pa_last_hip_error).
 */
typedef struct pa_graph pa_graph;
pa_status pa_graph_begin(void* stream);
pa_status pa_graph_end(void* stream, pa_graph** graph);
pa_status pa_graph_launch(const pa_graph* graph, void* stream);
pa_status pa_graph_destroy(pa_graph* graph);

#ifdef __cplusplus
}
#endif

#endif /* PA_H */
