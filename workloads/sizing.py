"""KV-cache sizing and the algorithmic byte model of one decode step.

The sizing formulas restate the block arithmetic of the vLLM/PagedAttention explainer
(kasblo.com, "KV Cacheの容量をtokenから計算する"): raw K/V payload per token is
2 * layers * kv_heads * head_dim * bytes, a block holds block_size tokens, a sequence of N tokens
occupies ceil(N / block_size) blocks, and only the tail of the last block is wasted.

The byte model counts what one paged decode step must move at minimum: every valid K/V element
once, the fp8 block scales of the blocks read, the query and output rows, and the block-table
entries walked.  Partial-tile over-read and split-KV workspace traffic are deliberately not
counted; they are overhead charged to the kernel.
"""

from __future__ import annotations

import numpy as np

BLOCK_SIZE = 16  # tokens per physical KV block (the pages' default)

ELEM_BYTES = {"f16": 2, "bf16": 2, "fp8_e4m3": 1}


def kv_bytes_per_token(layers: int, kv_heads: int, head_dim: int, elem_bytes: int) -> int:
    """m_token = 2 * L * H_kv * d_h * b (K and V)."""
    return 2 * layers * kv_heads * head_dim * elem_bytes


def n_blocks(num_tokens: int, block_size: int = BLOCK_SIZE) -> int:
    """n_blocks = ceil(N / B)."""
    return -(-int(num_tokens) // block_size)


def m_block(m_token: int, block_size: int = BLOCK_SIZE) -> int:
    """m_block = B * m_token."""
    return block_size * m_token


def m_alloc(num_tokens: int, m_token: int, block_size: int = BLOCK_SIZE) -> int:
    """M_alloc = ceil(N / B) * B * m_token."""
    return n_blocks(num_tokens, block_size) * block_size * m_token


def m_waste(num_tokens: int, m_token: int, block_size: int = BLOCK_SIZE) -> int:
    """M_waste = (ceil(N / B) * B - N) * m_token; never more than (B - 1) tokens."""
    return (n_blocks(num_tokens, block_size) * block_size - int(num_tokens)) * m_token


def decode_bytes(context_lens, num_q_heads: int, num_kv_heads: int, head_dim: int,
                 q_dtype: str, kv_dtype: str, unique_tokens: int | None = None) -> int:
    """Algorithmic HBM bytes of one decode call over the given context lengths.

    unique_tokens, when given, replaces sum(context_lens) for the K/V term: blocks that several
    sequences share through their block tables are then counted once.
    """
    lens = np.asarray(context_lens, dtype=np.int64)
    e_kv = ELEM_BYTES[kv_dtype]
    e_q = ELEM_BYTES[q_dtype]
    tokens = int(lens.sum()) if unique_tokens is None else int(unique_tokens)
    blocks = int(sum(n_blocks(x) for x in lens))
    kv = tokens * num_kv_heads * head_dim * e_kv * 2
    scales = blocks * num_kv_heads * 4 * 2 if kv_dtype == "fp8_e4m3" else 0
    q_and_out = 2 * len(lens) * num_q_heads * head_dim * e_q
    tables = blocks * 4 + 4 * len(lens)
    return kv + scales + q_and_out + tables


def append_bytes(num_tokens: int, num_kv_heads: int, head_dim: int, kv_dtype: str) -> int:
    """Bytes of one append: read the new K and V rows, write them into the cache, read slots."""
    row = num_kv_heads * head_dim * ELEM_BYTES[kv_dtype]
    return num_tokens * (2 * row * 2 + 8)


def visible_keys(context_lens, query_lens) -> int:
    """Keys seen summed over query rows: row i of a sequence with L cached tokens, the last T of
    them new, sees min(max(L - T + i + 1, 0), L) of them (causal over the cache)."""
    total = 0
    for L, T in zip(np.asarray(context_lens, dtype=np.int64), np.asarray(query_lens, dtype=np.int64)):
        i = np.arange(int(T))
        total += int(np.clip(L - T + i + 1, 0, L).sum())
    return total


def multi_bytes(context_lens, query_lens, num_q_heads: int, num_kv_heads: int, head_dim: int,
                q_dtype: str, kv_dtype: str) -> int:
    """Algorithmic HBM bytes of one multi-query call: every K/V element of each sequence once
    (however many rows see it), the fp8 block scales, every query and output row once, the
    block-table entries and the query start offsets."""
    lens = np.asarray(context_lens, dtype=np.int64)
    rows = int(np.asarray(query_lens, dtype=np.int64).sum())
    e_q = ELEM_BYTES[q_dtype]
    single = decode_bytes(lens, num_q_heads, num_kv_heads, head_dim, q_dtype, kv_dtype)
    single -= 2 * len(lens) * num_q_heads * head_dim * e_q
    return single + 2 * rows * num_q_heads * head_dim * e_q + 4 * (len(lens) + 1)


def multi_flops(context_lens, query_lens, num_q_heads: int, head_dim: int) -> int:
    """Algorithmic flops of one multi-query call: per query head and visible key, a head_dim dot
    product for the score and a head_dim multiply-add into the output (2 * 2 * head_dim)."""
    return 4 * head_dim * num_q_heads * visible_keys(context_lens, query_lens)
