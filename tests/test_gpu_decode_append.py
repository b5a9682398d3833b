"""pa_decode_append (the append and the decode of one step in one launch) on the GPU: the caches
it leaves are bit-exact against the oracle's append, and its output equals pa_kv_append followed
by pa_decode bit for bit, and the oracle within tolerance."""

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_31_amd as pa
import workloads
from gpu_util import Dev, assert_close, host_bits, oracle_after_append
from workloads.generate import Spec

pytestmark = pytest.mark.gpu

LENS = (1, 15, 16, 17, 31, 32, 33, 100, 511, 512, 513, 1000, 2049, 0)

CASES = [
    # (q dtype, kv dtype, kv heads, group, head_dim, partition, shared prefix (sharing, tokens))
    ("bf16", "bf16", 2, 8, 128, 0, None),
    ("bf16", "bf16", 2, 4, 64, 128, None),
    ("f16", "f16", 4, 1, 128, 0, None),
    ("bf16", "fp8_e4m3", 2, 8, 128, 0, None),
    ("f16", "fp8_e4m3", 2, 4, 128, 512, None),
    ("bf16", "bf16", 2, 4, 128, 0, (6, 256)),
]


def _fused(dev, P, share):
    wl = dev.wl
    pa.pa_decode_append(dev.q, dev.k_new, dev.v_new, dev.k_cache, dev.v_cache, dev.tables,
                        dev.lens, float(wl.scale), dev.out, k_scale=dev.k_scale,
                        v_scale=dev.v_scale, max_context_len=wl.max_context_len,
                        partition_tokens=P, shared_prefixes=share)
    torch.cuda.synchronize()
    return host_bits(dev.out)


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[0]}-{c[1]}-kv{c[2]}g{c[3]}d{c[4]}"
                         f"-P{c[5]}-{'share' if c[6] else 'private'}")
def test_fused_equals_append_then_decode(case):
    qd, kvd, hkv, g, d, P, prefix = case
    # with a shared prefix every length is at least 1, so each new token goes to a block of its
    # own sequence (a block being appended to is not shared: the contract of the fused call)
    lens = LENS if prefix is None else tuple(max(1, x) for x in LENS)
    spec = Spec("fused", len(lens), hkv * g, hkv, d, qd, kvd, ("list", lens), pool=("times", 2),
                seed=81 + CASES.index(case), prefix=prefix)
    wl = workloads.make(spec)
    share = prefix is not None
    fused = Dev(wl)
    out_fused = _fused(fused, P, share)
    ref, k_ref, v_ref = oracle_after_append(wl)
    assert np.array_equal(host_bits(fused.k_cache), k_ref)
    assert np.array_equal(host_bits(fused.v_cache), v_ref)
    split = Dev(wl)
    split.append()
    out_split = split.decode(partition_tokens=P, shared_prefixes=share)
    assert np.array_equal(out_fused, out_split)
    # the edge lengths start at 0 and 1 (counted rounding-limited relief)
    assert_close(out_fused, ref, qd, label=f"fused {case}", relief=True)


@pytest.mark.parametrize("kvd", ["bf16", "fp8_e4m3"])
def test_dense_appends(kvd):
    """64 short sequences x 8 KV heads: one append per launched wave or more, so the step's
    append runs as a launch of its own before the decode; the caches and the output must be
    the same as in every other case."""
    rng = np.random.default_rng(89)
    lens = tuple(int(x) for x in rng.integers(1, 40, size=64))
    spec = Spec("dense", 64, 32, 8, 128, "bf16", kvd, ("list", lens), pool=("times", 2),
                seed=89)
    wl = workloads.make(spec)
    fused = Dev(wl)
    out_fused = _fused(fused, 0, False)
    ref, k_ref, v_ref = oracle_after_append(wl)
    assert np.array_equal(host_bits(fused.k_cache), k_ref)
    assert np.array_equal(host_bits(fused.v_cache), v_ref)
    split = Dev(wl)
    split.append()
    assert np.array_equal(out_fused, split.decode())
    # contexts of 1 to 39 tokens (counted rounding-limited relief)
    assert_close(out_fused, ref, "bf16", label=f"dense appends {kvd}", relief=True)


def test_block_outside_the_pool_is_not_written():
    spec = Spec("oob", 3, 8, 2, 128, "bf16", "bf16", ("list", (40, 17, 5)), pool=("times", 2),
                seed=88)
    wl = workloads.make(spec)
    dev = Dev(wl)
    tables = wl.block_tables.copy()
    tables[1, 1] = wl.num_blocks + 3                # token 16 of sequence 1 lives "outside"
    dev.tables = torch.from_numpy(tables).cuda()
    before_k, before_v = host_bits(dev.k_cache), host_bits(dev.v_cache)
    _fused(dev, 0, False)
    k_after, v_after = host_bits(dev.k_cache), host_bits(dev.v_cache)
    # sequences 0 and 2 wrote their slots; sequence 1 wrote nothing
    slots = wl.slot_mapping.copy()
    slots[1] = -1
    k_ref, v_ref = oracle.kv_append(before_k, before_v, wl.k_new, wl.v_new, slots)
    assert np.array_equal(k_after, k_ref) and np.array_equal(v_after, v_ref)


@pytest.mark.parametrize("name", workloads.spec_names())
def test_full_size_fused_step(name):
    """Each workload at full size as the benchmark runs a step: one pa_decode_append call."""
    wl = workloads.make(name)
    dev = Dev(wl)
    out = _fused(dev, wl.spec.partition_tokens, wl.spec.prefix is not None)
    ref, k_ref, v_ref = oracle_after_append(wl)
    assert np.array_equal(host_bits(dev.k_cache), k_ref)
    assert np.array_equal(host_bits(dev.v_cache), v_ref)
    assert_close(out, ref, wl.spec.q_dtype, label=f"{name} fused")
