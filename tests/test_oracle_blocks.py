"""Pins of oracle.blocks: the block copy against flat-address loops and against decoding, the
reference-count model against the kasblo explainer's lifecycle (the 100-token example in
tests/golden/pages_sizing.json) and its copy-on-write rule, and the model's refusal of every
decision the pages rule out."""

import json
import os

import numpy as np
import pytest

import oracle
from cpu_cases import Case

BLOCK = 16


def _pool(rng, NB=9, H=2, D=8, fp8=False):
    if fp8:
        k = rng.integers(0, 256, (NB, H, BLOCK, D), dtype=np.uint8)
        v = rng.integers(0, 256, (NB, H, D, BLOCK), dtype=np.uint8)
        ks = rng.uniform(0.1, 1, (NB, H)).astype(np.float32)
        vs = rng.uniform(0.1, 1, (NB, H)).astype(np.float32)
        return k, v, ks, vs
    k = rng.integers(0, 1 << 16, (NB, H, BLOCK, D), dtype=np.uint16)
    v = rng.integers(0, 1 << 16, (NB, H, D, BLOCK), dtype=np.uint16)
    return k, v, None, None


@pytest.mark.parametrize("fp8", [False, True])
def test_copy_matches_flat_address_loops(fp8):
    rng = np.random.default_rng(1)
    k, v, ks, vs = _pool(rng, fp8=fp8)
    pairs = [(3, 0), (5, 7), (0, 8), (2, 2)]          # a later pair reads an earlier result
    got = oracle.copy_blocks(k, v, ks, vs, pairs)
    NB, H, _, D = k.shape
    kf, vf = k.reshape(-1).copy(), v.reshape(-1).copy()
    ksf = None if ks is None else ks.reshape(-1).copy()
    vsf = None if vs is None else vs.reshape(-1).copy()
    tile = BLOCK * D
    for src, dst in pairs:
        for h in range(H):
            for e in range(tile):
                kf[(dst * H + h) * tile + e] = kf[(src * H + h) * tile + e]
                vf[(dst * H + h) * tile + e] = vf[(src * H + h) * tile + e]
            if ksf is not None:
                ksf[dst * H + h] = ksf[src * H + h]
                vsf[dst * H + h] = vsf[src * H + h]
    assert np.array_equal(got[0].reshape(-1), kf) and np.array_equal(got[1].reshape(-1), vf)
    if fp8:
        assert np.array_equal(got[2].reshape(-1), ksf) and np.array_equal(got[3].reshape(-1), vsf)
    assert np.array_equal(got[0][1], k[1])             # blocks not named stay as they were


@pytest.mark.parametrize("kv", ["bf16", "fp8_e4m3"])
def test_decode_through_the_copies_is_unchanged(kv):
    """A sequence whose table points at copies of its blocks attends to the same values."""
    rng = np.random.default_rng(2)
    case = Case(rng, [40, 70], Hkv=2, G=2, D=16, kv_dtype=kv)
    args = case.oracle_args()
    before = oracle.decode(**args)
    free = sorted(set(range(case.NB)) - set(case.tables[:, :5].reshape(-1).tolist()))
    pairs = [(int(case.tables[1, j]), free[j]) for j in range(5)]
    k, v, ks, vs = oracle.copy_blocks(case.k_cache, case.v_cache, case.k_scale, case.v_scale,
                                      pairs)
    tables = case.tables.copy()
    tables[1, :5] = free[:5]
    args.update(k_cache=k, v_cache=v, k_scale=ks, v_scale=vs, block_tables=tables)
    assert np.array_equal(oracle.decode(**args), before)


def test_lifecycle_of_the_100_token_example(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "pages_sizing.json")))["kasblo_100_tokens"]
    m = oracle.BlockPoolModel(64)
    blocks = list(range(g["n_blocks"]))                # prefill of 100 tokens
    m.take(blocks)
    assert m.free_count() == 64 - 7
    for length in range(101, g["capacity_tokens"] + 1):
        assert length <= BLOCK * len(blocks)           # decode fills the 12 spare slots
    m.take([7])                                        # token 113 needs an eighth block
    blocks.append(7)
    assert m.free_count() == 64 - 8
    m.release(blocks)                                  # the request ends
    assert m.free_count() == 64 and (m.ref == 0).all()
    m.take([3, 9])                                     # freed blocks are reused
    assert m.ref[3] == 1 and m.ref[9] == 1


def test_parallel_sampling_fork_and_copy_on_write():
    m = oracle.BlockPoolModel(16)
    parent = [4, 5, 6]
    m.take(parent)
    children = [list(parent) for _ in range(3)]
    for c in children:
        m.share(c)
    assert list(m.ref[parent]) == [4, 4, 4]
    # every sequence appends into the shared last block: the first three get copies
    assert m.write(6, 10) and m.write(6, 11) and m.write(6, 12)
    assert not m.write(6, 6)                           # the last one left writes in place
    assert list(m.ref[[4, 5, 6, 10, 11, 12]]) == [4, 4, 1, 1, 1, 1]
    assert m.free_count() == 16 - 6


def test_model_refuses_what_the_pages_rule_out():
    m = oracle.BlockPoolModel(8)
    m.take([1, 2])
    with pytest.raises(AssertionError):
        m.take([2])                                    # in use
    with pytest.raises(AssertionError):
        m.take([3, 3])                                 # twice in one allocation
    with pytest.raises(AssertionError):
        m.take([8])                                    # outside the pool
    with pytest.raises(AssertionError):
        m.share([5])                                   # free
    with pytest.raises(AssertionError):
        m.release([1, 1])                              # more often than referred to
    m.share([1])
    with pytest.raises(AssertionError):
        m.write(1, 1)                                  # shared: must be copied
    with pytest.raises(AssertionError):
        m.write(1, 2)                                  # copy target in use
    with pytest.raises(AssertionError):
        m.write(2, 4)                                  # sole user: no copy
    assert list(m.ref[:4]) == [0, 2, 1, 0]             # refused calls changed nothing
