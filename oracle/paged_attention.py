"""fp64 CPU oracle for single-query attention over a paged KV cache.

TEST INFRASTRUCTURE.  Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may
import or run this module.  It shares no code with the HIP library and imports nothing from it.

What is computed, and where the pages state it:

* kv_append -- each generation step stores the new token's K/V projection in the cache
  (Scaling Book note on notes.yuuk.io, "Transformer 推論の基礎: Prefill と Generation"; the
  youngju.dev guide's KV-cache module concatenates the new K, V onto the cache before attending).
  In the paged form the token goes to slot (physical_block * 16 + offset) of its block
  (kasblo.com, "blockはrequestの成長に合わせて割り当てる").
* gather -- a sequence's logical block j lives in physical block block_table[j]; the attention
  kernel reads K/V through that table (kasblo.com, "PagedAttentionはKV Cacheをblockで管理する";
  youngju.dev guide, PagedAttention block-table figure).  Only the first ceil(L/16) blocks are
  read, and only the first L tokens of them.
* attend -- scores = q . K^T * scale, softmax over the keys, weights . V (youngju.dev guide,
  KV-cache attention module; scale is passed in, the configs use 1/sqrt(head_dim)).
  GQA: query head h reads KV head h // (Hq / Hkv) (Scaling Book note, "生成スループット/レイテンシ
  改善のテクニック": groups of query heads share one KV head).
* decode_multi -- several new query tokens per sequence in one pass, each attending causally
  to every cached token up to and including its own position: the target model's verification
  of K draft tokens in one forward pass (youngju.dev guide, speculative-decoding figure; magi
  page, "投機的デコードとの相互作用") and a chunk of a long prompt processed against the cache
  built so far (magi page, "Prefill-Decode 分離 — chunked prefill と disaggregation").  The T
  new tokens are the last T of the sequence's context_lens tokens (already in the cache).
* decode_split -- the same attention evaluated over fixed key partitions and merged by
  log-sum-exp; used only to pin the merge algebra the GPU's split-KV path relies on.  The pages
  give online softmax without spelling out a split (babushkai.com "GPU推論の内部構造",
  FlashAttention section); partitions start at logical token 0.

Cache layout (shared contract, see include/pa.h):
  K pool [NB][Hkv][16][D] (token-major tile), V pool [NB][Hkv][D][16] (dim-major tile),
  raw storage bits; fp8 values are code * scale[block][kv_head].

Every function here is pinned by tests/test_oracle.py against something other than itself:
brute-force flat-address loops on tiny inputs, torch's scaled_dot_product_attention on
contiguous per-sequence arrays, softmax normalisation, the L=1 and needle special cases, the
two-token closed form, the pages' block-table examples and torch's own dtype decoders.
"""

from __future__ import annotations

import numpy as np

from .formats import e4m3fn_encode, to_f64

BLOCK = 16


def kv_append(k_cache: np.ndarray, v_cache: np.ndarray, k_new: np.ndarray, v_new: np.ndarray,
              slot_mapping: np.ndarray):
    """Scatter each new token's K/V rows into its slot; negative slots are skipped.

    Raw bits are copied, so the result is exact.  Tokens are applied in order, so with a
    duplicated slot the last token wins.  Returns new arrays; the inputs are not modified.
    """
    k = k_cache.copy()
    v = v_cache.copy()
    for i, s in enumerate(np.asarray(slot_mapping, dtype=np.int64)):
        if s < 0:
            continue
        blk, off = divmod(int(s), BLOCK)
        k[blk, :, off, :] = k_new[i]
        v[blk, :, :, off] = v_new[i]
    return k, v


SCALE_KEEP = 0          # quantise with the block's stored scale
SCALE_FIRST_TOKEN = 1   # a token written at offset 0 of its block first sets that block's scale


def kv_append_quant(k_cache, v_cache, k_scale, v_scale, k_new, v_new, src_dtype, slot_mapping,
                    policy):
    """Append 16-bit K/V rows into an fp8 e4m3fn cache with per-(block, KV head) scales.

    The fp8 KV cache stores value = code * scale (babushkai.com "GPU推論の内部構造", KV-cache and
    quantisation sections).  The pages do not say how a block's scale is chosen or what happens
    when later tokens outgrow it; the reading taken here:
      * policy SCALE_FIRST_TOKEN: every token of this call written at offset 0 of its block
        first sets that block's scale, per KV head and separately for K and V, to
        fp32(max |x|) / fp32(448) in fp32 (1 if the maximum is 0; NaN elements are ignored);
      * then every token is encoded as e4m3fn(clamp(fp32(x) / fp32(scale), +-448)), the division
        in fp32 and the rounding to nearest even (a token later in a block uses the block's
        scale as it stands, saturating if it is larger).
    Tokens are applied in order (a duplicated slot: the last one wins).  Returns new arrays.
    """
    k, v = k_cache.copy(), v_cache.copy()
    ks, vs = k_scale.copy(), v_scale.copy()
    with np.errstate(invalid="ignore"):                  # NaN payloads stay NaN
        xk = to_f64(k_new, src_dtype).astype(np.float32)   # exact: 16-bit values fit in fp32
        xv = to_f64(v_new, src_dtype).astype(np.float32)
    slots = np.asarray(slot_mapping, dtype=np.int64)

    def first_scale(row):
        with np.errstate(invalid="ignore"):
            m = np.float32(np.nanmax(np.abs(row))) if not np.all(np.isnan(row)) else np.float32(0)
        return np.float32(1.0) if m == 0 else np.float32(m / np.float32(448.0))

    if policy == SCALE_FIRST_TOKEN:
        for i, s in enumerate(slots):
            if s >= 0 and s % BLOCK == 0:
                blk = int(s) // BLOCK
                for h in range(k.shape[1]):
                    ks[blk, h] = first_scale(xk[i, h])
                    vs[blk, h] = first_scale(xv[i, h])
    for i, s in enumerate(slots):
        if s < 0:
            continue
        blk, off = divmod(int(s), BLOCK)
        for h in range(k.shape[1]):
            with np.errstate(over="ignore", invalid="ignore"):   # inf and NaN are encoded too
                k[blk, h, off, :] = e4m3fn_encode(xk[i, h] / ks[blk, h])
                v[blk, h, :, off] = e4m3fn_encode(xv[i, h] / vs[blk, h])
    return k, v, ks, vs


def gather(k_cache, v_cache, kv_dtype, table_row, length, kvh, k_scale=None, v_scale=None):
    """Logical-order K and V of one sequence and KV head, as float64 [L][D]."""
    length = int(length)
    nb = -(-length // BLOCK)
    ids = np.asarray(table_row[:nb], dtype=np.int64)
    k_tiles = k_cache[ids, kvh]                          # [nb][16][D]
    v_tiles = v_cache[ids, kvh].transpose(0, 2, 1)       # [nb][D][16] -> [nb][16][D]
    D = k_tiles.shape[-1]
    k = to_f64(k_tiles.reshape(nb * BLOCK, D)[:length], kv_dtype)
    v = to_f64(v_tiles.reshape(nb * BLOCK, D)[:length], kv_dtype)
    if kv_dtype == "fp8_e4m3":
        blk_of_tok = ids[np.arange(length) // BLOCK]
        k = k * np.asarray(k_scale, dtype=np.float64)[blk_of_tok, kvh][:, None]
        v = v * np.asarray(v_scale, dtype=np.float64)[blk_of_tok, kvh][:, None]
    return k, v


def attend(q_rows: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float):
    """softmax(scale * q_rows . k^T) . v for one KV head; returns (out [G][D], weights [G][L])."""
    G, D = q_rows.shape
    if k.shape[0] == 0:
        return np.zeros((G, D)), np.zeros((G, 0))
    s = (q_rows @ k.T) * scale
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    w = e / e.sum(axis=1, keepdims=True)
    return w @ v, w


def _q_f64(q, q_dtype):
    return to_f64(q, q_dtype)


def decode(q, k_cache, v_cache, block_tables, context_lens, scale, q_dtype, kv_dtype,
           k_scale=None, v_scale=None, return_weights=False):
    """Attention output [B][Hq][D] (float64, unrounded) for every sequence and query head."""
    qf = _q_f64(q, q_dtype)
    B, Hq, D = qf.shape
    Hkv = k_cache.shape[1]
    G = Hq // Hkv
    sc = float(np.float32(scale))
    out = np.zeros((B, Hq, D))
    weights = {}
    for b in range(B):
        for kvh in range(Hkv):
            k, v = gather(k_cache, v_cache, kv_dtype, block_tables[b], context_lens[b], kvh,
                          k_scale, v_scale)
            o, w = attend(qf[b, kvh * G:(kvh + 1) * G], k, v, sc)
            out[b, kvh * G:(kvh + 1) * G] = o
            if return_weights:
                weights[(b, kvh)] = w
    return (out, weights) if return_weights else out


def decode_multi(q, query_start, k_cache, v_cache, block_tables, context_lens, scale, q_dtype,
                 kv_dtype, k_scale=None, v_scale=None):
    """Causal attention of several query tokens per sequence over its paged cache.

    q holds [N][Hq][D] query rows; sequence b owns rows query_start[b] .. query_start[b+1]-1,
    T_b of them, and context_lens[b] = L_b counts every cached token including those T_b.
    Row i of sequence b sits at logical position p = L_b - T_b + i and attends to the tokens
    0 .. p, i.e. the first min(max(p + 1, 0), L_b) of the sequence (none when p < 0: zeros, as for
    an empty context).  Returns [N][Hq][D] float64.
    """
    qf = _q_f64(q, q_dtype)
    N, Hq, D = qf.shape
    Hkv = k_cache.shape[1]
    G = Hq // Hkv
    sc = float(np.float32(scale))
    qs = np.asarray(query_start, dtype=np.int64)
    out = np.zeros((N, Hq, D))
    for b in range(len(qs) - 1):
        T = int(qs[b + 1] - qs[b])
        L = int(context_lens[b])
        for kvh in range(Hkv):
            k, v = gather(k_cache, v_cache, kv_dtype, block_tables[b], L, kvh, k_scale, v_scale)
            for i in range(T):
                n = min(max(L - T + i + 1, 0), L)
                row = int(qs[b]) + i
                o, _ = attend(qf[row, kvh * G:(kvh + 1) * G], k[:n], v[:n], sc)
                out[row, kvh * G:(kvh + 1) * G] = o
    return out


def decode_split(q, k_cache, v_cache, block_tables, context_lens, scale, q_dtype, kv_dtype,
                 partition_tokens, k_scale=None, v_scale=None):
    """Same result as decode(), computed per key partition and merged by log-sum-exp.

    Partition j covers logical tokens [j*P, min((j+1)*P, L)).  Each yields its max score m_j,
    its exp-sum l_j and its normalised output o_j; the merge takes M = max_j m_j and returns
    sum_j e^(m_j - M) l_j o_j / sum_j e^(m_j - M) l_j.
    """
    qf = _q_f64(q, q_dtype)
    B, Hq, D = qf.shape
    Hkv = k_cache.shape[1]
    G = Hq // Hkv
    sc = float(np.float32(scale))
    P = int(partition_tokens)
    out = np.zeros((B, Hq, D))
    for b in range(B):
        L = int(context_lens[b])
        if L == 0:
            continue
        for kvh in range(Hkv):
            k, v = gather(k_cache, v_cache, kv_dtype, block_tables[b], L, kvh, k_scale, v_scale)
            qg = qf[b, kvh * G:(kvh + 1) * G]
            ms, ls, os_ = [], [], []
            for lo in range(0, L, P):
                s = (qg @ k[lo:lo + P].T) * sc
                m = s.max(axis=1)
                e = np.exp(s - m[:, None])
                ms.append(m)
                ls.append(e.sum(axis=1))
                os_.append((e @ v[lo:lo + P]) / ls[-1][:, None])
            ms, ls, os_ = np.array(ms), np.array(ls), np.array(os_)   # [NP][G], [NP][G], [NP][G][D]
            M = ms.max(axis=0)
            a = np.exp(ms - M) * ls
            out[b, kvh * G:(kvh + 1) * G] = (a[:, :, None] * os_).sum(axis=0) / a.sum(axis=0)[:, None]
    return out
