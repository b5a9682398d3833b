"""Block sharing in the paged cache: reference counts, copy-on-write and the block copy.

TEST INFRASTRUCTURE.  Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may
import or run this module.  It shares no code with the HIP library.

What the kasblo.com vLLM explainer states (sections "blockはrequestの成長に合わせて割り当てる"
and "block共有とAutomatic Prefix Caching"):
  * a request takes the blocks its prefill needs from a pool of reusable physical blocks, adds a
    free block whenever decoding has filled its current one, and gives back, when it ends, the
    blocks only it uses; freed blocks are reused by later requests;
  * every physical block carries a reference count, the number of sequences referring to it, so
    that several sequences (parallel sampling, a common prefix) can hold the same content once;
  * a shared block is duplicated only when one of its sequences has to change its content
    (copy-on-write).

Which physical block an allocation returns is not fixed by the pages; the model therefore does
not choose ids.  It is told the library's choice and checks that it is allowed (free, distinct,
in the pool), then tracks the counts, so a test can compare every count after every operation.
"""

from __future__ import annotations

import numpy as np


class BlockPoolModel:
    """Reference counts of num_blocks physical blocks; a block with count 0 is free."""

    def __init__(self, num_blocks: int):
        self.ref = np.zeros(int(num_blocks), dtype=np.int64)

    @property
    def num_blocks(self) -> int:
        return len(self.ref)

    def free_count(self) -> int:
        return int((self.ref == 0).sum())

    def take(self, ids) -> None:
        """A new allocation: each id must be a free block of the pool, all distinct; each now
        has one referring sequence."""
        ids = [int(i) for i in ids]
        assert len(set(ids)) == len(ids), "an allocation returned a block twice"
        for i in ids:
            assert 0 <= i < self.num_blocks, f"block {i} outside the pool"
            assert self.ref[i] == 0, f"block {i} handed out while in use"
        for i in ids:
            self.ref[i] = 1

    def share(self, ids) -> None:
        """More sequences refer to blocks already in use (a fork, a reused prefix)."""
        ids = [int(i) for i in ids]
        for i in ids:
            assert self.ref[i] >= 1, f"sharing free block {i}"
        for i in ids:
            self.ref[i] += 1

    def release(self, ids) -> None:
        """Sequences stop referring to blocks (a request ends); a block whose count reaches 0
        goes back to the pool."""
        ids = [int(i) for i in ids]
        need = {}
        for i in ids:
            need[i] = need.get(i, 0) + 1
        for i, n in need.items():
            assert self.ref[i] >= n, f"releasing block {i} more often than it is referred to"
        for i, n in need.items():
            self.ref[i] -= n

    def write(self, block: int, new_block: int) -> bool:
        """A sequence is about to write into `block`.  If it is the only sequence referring to
        it, it writes in place (new_block must equal block; returns False).  Otherwise it gets
        `new_block`, a free block that receives a copy of the content, and lets go of its
        reference to the shared one (returns True: a copy is needed)."""
        block, new_block = int(block), int(new_block)
        assert self.ref[block] >= 1, f"writing into free block {block}"
        if self.ref[block] == 1:
            assert new_block == block, "a block only one sequence uses must not be copied"
            return False
        assert new_block != block and self.ref[new_block] == 0, "copy target must be free"
        self.ref[block] -= 1
        self.ref[new_block] = 1
        return True


def copy_blocks(k_cache, v_cache, k_scale, v_scale, pairs):
    """The copy of copy-on-write: for each (src, dst) pair in order, physical block dst gets the
    K tile, the V tile and (fp8 caches) the K and V scales of block src, for every KV head.
    Returns new arrays; scales may be None."""
    k, v = k_cache.copy(), v_cache.copy()
    ks = None if k_scale is None else k_scale.copy()
    vs = None if v_scale is None else v_scale.copy()
    for src, dst in np.asarray(pairs, dtype=np.int64).reshape(-1, 2):
        k[dst] = k[src]
        v[dst] = v[src]
        if ks is not None:
            ks[dst] = ks[src]
            vs[dst] = vs[src]
    return k, v, ks, vs
