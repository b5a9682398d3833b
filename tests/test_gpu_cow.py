"""pa_copy_blocks against oracle.copy_blocks (bit-exact), and parallel sampling end to end:
prompts forked into several samples share their blocks, each sample's first write into a shared
block goes to a private copy (kasblo.com vLLM explainer, "block共有とAutomatic Prefix Caching"),
and every decode step is checked against the oracle run on the same operations."""

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_31_amd as pa
import workloads
from gpu_util import assert_close, dev_bits, host_bits

pytestmark = pytest.mark.gpu
BLOCK = 16


@pytest.mark.parametrize("kv,D", [("bf16", 128), ("f16", 64), ("fp8_e4m3", 128), ("fp8_e4m3", 64)])
def test_copy_blocks_bit_exact(kv, D):
    rng = np.random.default_rng(300 + D)
    NB, H = 300, 4
    if kv == "fp8_e4m3":
        k = rng.integers(0, 256, (NB, H, BLOCK, D), dtype=np.uint8)
        v = rng.integers(0, 256, (NB, H, D, BLOCK), dtype=np.uint8)
        ks = rng.uniform(0.01, 1, (NB, H)).astype(np.float32)
        vs = rng.uniform(0.01, 1, (NB, H)).astype(np.float32)
    else:
        k = rng.integers(0, 1 << 16, (NB, H, BLOCK, D), dtype=np.uint16)
        v = rng.integers(0, 1 << 16, (NB, H, D, BLOCK), dtype=np.uint16)
        ks = vs = None
    perm = rng.permutation(NB)
    pairs = np.stack([perm[:100], perm[100:200]], axis=1).astype(np.int32)   # targets fresh
    skipped = np.array([[5, NB], [NB + 3, 7], [-1, 9], [11, 11]], dtype=np.int32)
    all_pairs = np.concatenate([pairs[:50], skipped, pairs[50:]])
    kd, vd = dev_bits(k, kv), dev_bits(v, kv)
    ksd = None if ks is None else torch.from_numpy(ks).cuda()
    vsd = None if vs is None else torch.from_numpy(vs).cuda()
    pa.pa_copy_blocks(torch.from_numpy(all_pairs).cuda(), kd, vd, ksd, vsd)
    torch.cuda.synchronize()
    rk, rv, rks, rvs = oracle.copy_blocks(k, v, ks, vs, pairs)
    assert np.array_equal(host_bits(kd), rk) and np.array_equal(host_bits(vd), rv)
    if ks is not None:
        assert np.array_equal(ksd.cpu().numpy(), rks) and np.array_equal(vsd.cpu().numpy(), rvs)


@pytest.mark.parametrize("kv,q", [("bf16", "bf16"), ("f16", "f16")])
def test_parallel_sampling_with_copy_on_write(kv, q):
    rng = np.random.default_rng(310)
    NB, Hkv, G, D, MB = 160, 2, 4, 128, 32
    Hq = Hkv * G
    prompts, samples, steps = (40, 300, 16), 3, 6
    pool, model = pa.BlockPool(NB), oracle.BlockPoolModel(NB)
    k = workloads.storage_bits(rng.standard_normal((NB, Hkv, BLOCK, D)), kv)
    v = workloads.storage_bits(rng.standard_normal((NB, Hkv, D, BLOCK)), kv)
    kd, vd = dev_bits(k, kv), dev_bits(v, kv)

    # prefill: every prompt token's slot from the pool, rows appended by the library
    tables, lens, pre_slots = [], [], []
    for L in prompts:
        t = []
        for pos in range(L):
            pre_slots.append(pool.slot_for(t, pos, MB)[0])
        model.take(t)
        tables.append(t)
        lens.append(L)
    T = len(pre_slots)
    kn = workloads.storage_bits(rng.standard_normal((T, Hkv, D)), kv)
    vn = workloads.storage_bits(rng.standard_normal((T, Hkv, D)), kv)
    pa.pa_kv_append(dev_bits(kn, kv), dev_bits(vn, kv), torch.tensor(pre_slots).cuda(), kd, vd)
    k, v = oracle.kv_append(k, v, kn, vn, np.array(pre_slots))

    # fork: samples - 1 more sequences per prompt share its blocks
    for p in range(len(prompts)):
        for _ in range(samples - 1):
            child = list(tables[p])
            pool.share(child)
            model.share(child)
            tables.append(child)
            lens.append(lens[p])
    B = len(tables)
    assert np.array_equal(np.array([pool.refcount(b) for b in range(NB)]), model.ref)

    for step in range(steps):
        pairs, slots = [], []
        for b in range(B):
            slot, copy = pool.slot_for(tables[b], lens[b], MB)
            if copy is not None:
                assert model.write(copy[0], copy[1])
                pairs.append(copy)
            elif lens[b] % BLOCK == 0:
                model.take([tables[b][-1]])
            else:
                assert not model.write(tables[b][lens[b] // BLOCK], tables[b][lens[b] // BLOCK])
            slots.append(slot)
            lens[b] += 1
        assert np.array_equal(np.array([pool.refcount(b) for b in range(NB)]), model.ref)
        if pairs:
            pa.pa_copy_blocks(torch.tensor(pairs, dtype=torch.int32).cuda(), kd, vd)
            k, v, _, _ = oracle.copy_blocks(k, v, None, None, pairs)
        kn = workloads.storage_bits(rng.standard_normal((B, Hkv, D)), kv)
        vn = workloads.storage_bits(rng.standard_normal((B, Hkv, D)), kv)
        qb = workloads.storage_bits(rng.standard_normal((B, Hq, D)), q)
        tab = np.zeros((B, MB), dtype=np.int32)
        for b in range(B):
            tab[b, :len(tables[b])] = tables[b]
        ln = np.array(lens, dtype=np.int32)
        qd = dev_bits(qb, q)
        out = torch.empty_like(qd)
        pa.pa_decode_append(qd, dev_bits(kn, kv), dev_bits(vn, kv), kd, vd,
                            torch.from_numpy(tab).cuda(), torch.from_numpy(ln).cuda(),
                            float(1 / np.sqrt(D)), out)
        torch.cuda.synchronize()
        k, v = oracle.kv_append(k, v, kn, vn, np.array(slots))
        assert np.array_equal(host_bits(kd), k) and np.array_equal(host_bits(vd), v), step
        ref = oracle.decode(qb, k, v, tab, ln, np.float32(1 / np.sqrt(D)), q, kv)
        assert_close(host_bits(out), ref, q, f"step {step}")

    # the samples of one prompt still share its full blocks
    for p in range(len(prompts)):
        full = prompts[p] // BLOCK
        fam = [tables[p]] + tables[len(prompts) + p * (samples - 1):
                                   len(prompts) + (p + 1) * (samples - 1)]
        for t in fam[1:]:
            assert t[:full] == fam[0][:full]
    for t in tables:
        pool.release(t)
        model.release(t)
    assert pool.free_blocks() == NB == model.free_count()
