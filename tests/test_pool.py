"""The library's host-side block pool (pa_pool_*) against oracle.BlockPoolModel, on the CPU.

Every operation is mirrored into the model with the ids the library chose; the model checks
that each choice is allowed (kasblo.com vLLM explainer: blocks come from a pool of free blocks,
carry reference counts, and a shared block is copied before it is written), and all counts are
compared after every step.  Refused calls must leave the pool unchanged."""

import threading

import numpy as np
import pytest

import oracle
import paged_kv_cache_31_amd as pa

BLOCK = 16


def counts(pool, nb):
    return np.array([pool.refcount(b) for b in range(nb)])


def status_of(fn, *args):
    try:
        fn(*args)
    except pa.PaError as e:
        return e.status
    return pa.PA_OK


def test_random_operations_match_the_model():
    rng = np.random.default_rng(5)
    NB = 48
    pool, model = pa.BlockPool(NB), oracle.BlockPoolModel(NB)
    for step in range(3000):
        used = np.nonzero(model.ref)[0]
        op = rng.integers(0, 4)
        if op == 0:
            n = int(rng.integers(0, 6))
            if n > model.free_count():
                assert status_of(pool.alloc, n) == pa.PA_ERR_OUT_OF_BLOCKS
            else:
                model.take(pool.alloc(n))
        elif op == 1 and len(used):
            ids = rng.choice(used, size=int(rng.integers(1, 4)))
            pool.share(ids)
            model.share(ids)
        elif op == 2 and len(used):
            ids = rng.choice(used, size=int(rng.integers(1, 4)))
            ok = all(model.ref[i] >= (ids == i).sum() for i in set(ids.tolist()))
            if ok:
                pool.release(ids)
                model.release(ids)
            else:
                assert status_of(pool.release, ids) == pa.PA_ERR_INVALID_ARG
        elif op == 3 and len(used):
            b = int(rng.choice(used))
            if model.ref[b] > 1 and model.free_count() == 0:
                assert status_of(pool.write, b) == pa.PA_ERR_OUT_OF_BLOCKS
            else:
                target, copy = pool.write(b)
                assert model.write(b, target) == copy
        assert np.array_equal(counts(pool, NB), model.ref), f"step {step}"
        assert pool.free_blocks() == model.free_count()


def test_refusals_change_nothing():
    NB = 6
    pool = pa.BlockPool(NB)
    a = pool.alloc(4)
    pool.share(a[:1])
    before = counts(pool, NB)
    assert status_of(pool.alloc, 3) == pa.PA_ERR_OUT_OF_BLOCKS
    assert status_of(pool.share, [a[1], 5]) == pa.PA_ERR_INVALID_ARG     # 5 is free
    assert status_of(pool.share, [NB]) == pa.PA_ERR_INVALID_ARG
    assert status_of(pool.release, [a[2], a[2]]) == pa.PA_ERR_INVALID_ARG
    assert status_of(pool.release, [-1]) == pa.PA_ERR_INVALID_ARG
    assert status_of(pool.write, 5) == pa.PA_ERR_INVALID_ARG
    pool.alloc(2)                                                      # pool now empty
    before = counts(pool, NB)
    assert status_of(pool.write, a[0]) == pa.PA_ERR_OUT_OF_BLOCKS       # shared, no free block
    t = list(a[:1])
    assert status_of(pool.slot_for, t, 16, 4) == pa.PA_ERR_OUT_OF_BLOCKS
    assert status_of(pool.slot_for, t, 40, 4) == pa.PA_ERR_INVALID_ARG  # skips a block
    assert status_of(pool.slot_for, t, 5, 1) == pa.PA_ERR_OUT_OF_BLOCKS  # a[0] shared, pool empty
    assert np.array_equal(counts(pool, NB), before) and t == a[:1]
    assert pool.refcount(NB) == -1


def test_lifecycle_of_a_request():
    """Prefill of 100 tokens takes 7 blocks, decode fills them to 112 and opens an eighth at
    token 113 (position 112), and the end of the request returns them all."""
    pool = pa.BlockPool(20)
    table, slots = [], []
    for pos in range(100):
        slot, copy = pool.slot_for(table, pos, 16)
        assert copy is None
        slots.append(slot)
    assert len(table) == 7 and pool.free_blocks() == 13
    for pos in range(100, 112):
        slots.append(pool.slot_for(table, pos, 16)[0])
    assert len(table) == 7
    slots.append(pool.slot_for(table, 112, 16)[0])
    assert len(table) == 8
    assert slots == [table[p // BLOCK] * BLOCK + p % BLOCK for p in range(113)]
    pool.release(table)
    assert pool.free_blocks() == 20


def test_fork_then_copy_on_write_through_slot_for():
    pool, model = pa.BlockPool(16), oracle.BlockPoolModel(16)
    parent = []
    for pos in range(40):                         # 3 blocks, the last holds tokens 32..39
        pool.slot_for(parent, pos, 8)
    model.take(parent)
    children = [list(parent) for _ in range(2)]
    for c in children:
        pool.share(c)
        model.share(c)
    shared_last = parent[2]
    for c in children:                            # each child writes token 40 into a copy
        slot, copy = pool.slot_for(c, 40, 8)
        assert copy is not None and copy[0] == shared_last and c[2] == copy[1]
        assert slot == copy[1] * BLOCK + 8
        assert model.write(shared_last, copy[1])
    slot, copy = pool.slot_for(parent, 40, 8)     # the parent is now its only user
    assert copy is None and slot == shared_last * BLOCK + 8
    assert not model.write(shared_last, shared_last)
    assert np.array_equal(counts(pool, 16), model.ref)
    assert children[0][:2] == children[1][:2] == parent[:2]       # the prefix stays shared
    assert len({children[0][2], children[1][2], parent[2]}) == 3


def test_threads_share_one_pool():
    NB = 256
    pool = pa.BlockPool(NB)
    errors = []

    def worker(seed):
        rng = np.random.default_rng(seed)
        try:
            for _ in range(400):
                got = pool.alloc(int(rng.integers(1, 4)))
                pool.share(got)
                pool.release(got)
                pool.release(got)
        except Exception as e:   # noqa: BLE001 - reported below
            errors.append(e)

    threads = [threading.Thread(target=worker, args=(s,)) for s in range(8)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors and pool.free_blocks() == NB
    assert (counts(pool, NB) == 0).all()
