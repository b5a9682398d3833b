"""The device-side contract of the library's calls, checked on the host.

The kernels read block tables, context lengths, slots and query offsets from device memory and
do not validate them on the hot path (they only clamp them so that nothing is read or written
out of bounds).  These functions spell the contract out for host copies of those arrays; the
binding runs them when a call is made with check=True (a test aid: it copies the arrays to the
host and so synchronises).  Each raises ContractError naming the first violation.

The contract follows the paged cache as the pages describe it: a sequence reaches logical block
j through entry j of its block table, which must name a physical block of the pool (kasblo.com
vLLM explainer, "PagedAttentionはKV Cacheをblockで管理する"); a block being written belongs to one
sequence, shared blocks being copied before a write (same page, "block共有とAutomatic Prefix
Caching").
"""

from __future__ import annotations

import numpy as np

BLOCK = 16


class ContractError(ValueError):
    """A device-resident argument breaks the documented contract of a call."""


def _as(a, dtype):
    return np.asarray(a).astype(dtype, copy=False)


def check_tables(block_tables, context_lens, num_blocks: int, max_context_len: int = 0):
    """Every length L_b lies in [0, min(max_blocks_per_seq * 16, max_context_len or that)], and
    the first ceil(L_b / 16) entries of row b name blocks of the pool [0, num_blocks)."""
    tables = _as(block_tables, np.int64)
    lens = _as(context_lens, np.int64)
    if tables.ndim != 2 or lens.shape != (tables.shape[0],):
        raise ContractError(f"block_tables {tables.shape} and context_lens {lens.shape} disagree")
    cap = tables.shape[1] * BLOCK
    if max_context_len > 0:
        cap = min(cap, int(max_context_len))
    for b, L in enumerate(lens):
        if L < 0 or L > cap:
            raise ContractError(f"context_lens[{b}] = {L} is outside [0, {cap}]")
        nb = -(-int(L) // BLOCK)
        row = tables[b, :nb]
        bad = np.nonzero((row < 0) | (row >= num_blocks))[0]
        if len(bad):
            j = int(bad[0])
            raise ContractError(f"block_tables[{b}][{j}] = {int(row[j])} is not a block of the "
                                f"pool [0, {num_blocks})")


def check_slots(slot_mapping, num_blocks: int):
    """Slots are below num_blocks * 16 (a negative slot skips its token) and no slot appears
    twice in one append."""
    slots = _as(slot_mapping, np.int64)
    if slots.ndim != 1:
        raise ContractError(f"slot_mapping must be one-dimensional, got {slots.shape}")
    over = np.nonzero(slots >= num_blocks * BLOCK)[0]
    if len(over):
        i = int(over[0])
        raise ContractError(f"slot_mapping[{i}] = {int(slots[i])} is past the pool "
                            f"({num_blocks} blocks of {BLOCK})")
    live = slots[slots >= 0]
    uniq, counts = np.unique(live, return_counts=True)
    if (counts > 1).any():
        s = int(uniq[np.argmax(counts > 1)])
        raise ContractError(f"slot {s} appears {int(counts.max())} times in one append")


def check_decode_append(block_tables, context_lens, num_blocks: int, max_context_len: int = 0):
    """check_tables, and the block that receives sequence b's new token (entry (L_b - 1) / 16)
    is read by no other sequence of the call: a block being written belongs to one sequence."""
    check_tables(block_tables, context_lens, num_blocks, max_context_len)
    tables = _as(block_tables, np.int64)
    lens = _as(context_lens, np.int64)
    readers: dict = {}
    for b, L in enumerate(lens):
        for p in tables[b, :-(-int(L) // BLOCK)]:
            readers.setdefault(int(p), set()).add(b)
    for b, L in enumerate(lens):
        if L <= 0:
            continue
        p = int(tables[b, (int(L) - 1) // BLOCK])
        others = readers[p] - {b}
        if others:
            raise ContractError(f"sequence {b} appends into block {p}, which sequence "
                                f"{min(others)} also reads in this call")


def check_multi(query_start, block_tables, context_lens, num_blocks: int, total_queries: int,
                max_query_len: int, max_context_len: int = 0):
    """check_tables, and the query rows: query_start is non-decreasing from >= 0 to at most
    total_queries, and every sequence has at most max_query_len rows."""
    check_tables(block_tables, context_lens, num_blocks, max_context_len)
    qs = _as(query_start, np.int64)
    B = _as(context_lens, np.int64).shape[0]
    if qs.shape != (B + 1,):
        raise ContractError(f"query_start must hold batch + 1 = {B + 1} offsets, got {qs.shape}")
    if qs[0] < 0 or qs[-1] > total_queries:
        raise ContractError(f"query_start runs from {int(qs[0])} to {int(qs[-1])}, outside "
                            f"[0, {total_queries}]")
    T = np.diff(qs)
    if (T < 0).any():
        b = int(np.argmax(T < 0))
        raise ContractError(f"query_start decreases at sequence {b}")
    if (T > max_query_len).any():
        b = int(np.argmax(T > max_query_len))
        raise ContractError(f"sequence {b} has {int(T[b])} query rows, more than "
                            f"max_query_len = {max_query_len}")


def check_copy_pairs(pairs, num_blocks: int):
    """Copy targets are distinct and no target is the source of another pair (pairs naming a
    block outside the pool, or a block onto itself, are skipped by the kernel)."""
    pr = _as(pairs, np.int64).reshape(-1, 2)
    ok = (pr >= 0).all(axis=1) & (pr < num_blocks).all(axis=1) & (pr[:, 0] != pr[:, 1])
    src, dst = pr[ok, 0], pr[ok, 1]
    uniq, counts = np.unique(dst, return_counts=True)
    if (counts > 1).any():
        raise ContractError(f"block {int(uniq[np.argmax(counts > 1)])} is the target of "
                            f"{int(counts.max())} copies")
    both = np.intersect1d(src, dst)
    if len(both):
        raise ContractError(f"block {int(both[0])} is both a source and a target")
