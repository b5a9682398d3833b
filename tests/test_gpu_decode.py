"""pa_decode on the GPU against the fp64 oracle, plus the exact special cases and the bitwise
invariants (placement, prefix sharing, determinism)."""

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_31_amd as pa
import workloads
from cpu_cases import round_bits, torch_decode
from gpu_util import Dev, assert_close, dev_bits, host_bits, oracle_after_append
from workloads.generate import Spec

pytestmark = pytest.mark.gpu
BLOCK = 16

EDGE_LENS = (1, 15, 16, 17, 31, 32, 33, 63, 64, 65, 100, 511, 512, 513, 1000, 2049)

CASES = [
    # (q dtype, kv dtype, kv heads, group, head_dim, lengths, partition)
    ("bf16", "bf16", 2, 8, 128, EDGE_LENS, 0),
    ("bf16", "bf16", 2, 8, 128, EDGE_LENS, 32),
    ("bf16", "bf16", 2, 8, 128, EDGE_LENS, 128),
    ("bf16", "bf16", 2, 8, 128, EDGE_LENS, 1024),
    ("bf16", "bf16", 3, 4, 64, EDGE_LENS, 0),
    ("bf16", "bf16", 2, 1, 128, EDGE_LENS[:12], 64),
    ("bf16", "bf16", 2, 3, 128, EDGE_LENS[:12], 0),
    ("bf16", "bf16", 1, 16, 128, EDGE_LENS[:12], 96),
    ("bf16", "bf16", 2, 2, 64, EDGE_LENS[:12], 4096),
    ("f16", "f16", 4, 1, 128, EDGE_LENS, 0),
    ("f16", "f16", 2, 4, 128, EDGE_LENS, 64),
    ("f16", "f16", 2, 8, 64, EDGE_LENS[:12], 160),
    ("bf16", "fp8_e4m3", 2, 8, 128, EDGE_LENS, 0),
    ("bf16", "fp8_e4m3", 2, 8, 128, EDGE_LENS, 96),
    ("bf16", "fp8_e4m3", 2, 4, 64, EDGE_LENS[:12], 32),
    ("f16", "fp8_e4m3", 2, 4, 128, EDGE_LENS, 512),
    ("f16", "fp8_e4m3", 2, 2, 64, EDGE_LENS[:12], 0),
    # partitions of an odd number of blocks (any multiple of 16 tokens)
    ("bf16", "bf16", 2, 8, 128, EDGE_LENS, 48),
    ("bf16", "fp8_e4m3", 2, 4, 128, EDGE_LENS, 16),
    ("f16", "f16", 2, 4, 64, EDGE_LENS[:12], 80),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[0]}-{c[1]}-kv{c[2]}g{c[3]}d{c[4]}"
                         f"-n{len(c[5])}-P{c[6]}")
def test_decode_parity_small(case):
    qd, kvd, hkv, g, d, lens, P = case
    spec = Spec("small", len(lens), hkv * g, hkv, d, qd, kvd, ("list", lens), pool=("times", 2),
                seed=31 + CASES.index(case))
    wl = workloads.make(spec)
    dev = Dev(wl)
    dev.append()
    out = dev.decode(partition_tokens=P)
    ref, _, _ = oracle_after_append(wl)
    # length 1 returns one V row; for an fp8 cache that is a code times its fp32 block scale,
    # which bf16 cannot always hold within the bound (counted as rounding-limited)
    assert_close(out, ref, qd, label=str(case[:5]) + f" P={P}", relief=kvd == "fp8_e4m3")


def _needle_setup(kv_dtype, q_dtype, t_stars, L, D=128, G=4, Hkv=2):
    spec = Spec("needle", len(t_stars), Hkv * G, Hkv, D, q_dtype, kv_dtype,
                ("list", (L,) * len(t_stars)), pool=("times", 2), seed=41)
    wl = workloads.make(spec)
    k_ref, v_ref = oracle.kv_append(wl.k_cache, wl.v_cache, wl.k_new, wl.v_new, wl.slot_mapping)
    q = np.zeros_like(wl.q)
    q[:, :, 0] = round_bits(np.array([1.0]), q_dtype)[0]
    k = np.zeros_like(k_ref)
    k_scale = None if wl.k_scale is None else wl.k_scale.copy()
    v_scale = None if wl.v_scale is None else wl.v_scale.copy()
    expect = np.zeros(wl.q.shape, dtype=np.float64)
    for b, t in enumerate(t_stars):
        blk = int(wl.block_tables[b, t // BLOCK])
        if kv_dtype == "fp8_e4m3":
            k[blk, :, t % BLOCK, 0] = 0x7E                       # 448
            k_scale[blk, :] = 2.0                                 # 448 * 2 / sqrt(128) ~ 79
            v_scale[blk, :] = 1.0                                 # needle value exact in bf16
        else:
            k[blk, :, t % BLOCK, 0] = round_bits(np.array([576.0]), kv_dtype)[0]  # 576/sqrt(128)
        for h in range(Hkv * G):
            expect[b, h] = torch_decode(v_ref[blk, h // G, :, t % BLOCK], kv_dtype)
            if kv_dtype == "fp8_e4m3":
                expect[b, h] *= v_scale[blk, h // G]
    return wl, q, k, v_ref, k_scale, v_scale, expect


@pytest.mark.parametrize("kv_dtype,q_dtype", [("bf16", "bf16"), ("f16", "f16"),
                                               ("fp8_e4m3", "bf16")])
@pytest.mark.parametrize("P", [0, 48, 128, 512])
def test_needle_bit_exact(kv_dtype, q_dtype, P):
    """One key dominates by e^-50 or more: the output must be exactly that token's V row, through
    the block table, the in-workgroup merge and the split-KV merge."""
    L = 1100
    t_stars = (0, 15, 16, 31, 32, 33, 511, 512, 1023, 1024, 1098, L - 1)
    wl, q, k, v, ks, vs, expect = _needle_setup(kv_dtype, q_dtype, t_stars, L)
    dev = Dev(wl)
    dev.q = dev_bits(q, q_dtype)
    dev.k_cache = dev_bits(k, kv_dtype)
    dev.v_cache = dev_bits(v, kv_dtype)
    if ks is not None:
        dev.k_scale = torch.from_numpy(ks).cuda()
        dev.v_scale = torch.from_numpy(vs).cuda()
    out = oracle.to_f64(dev.decode(partition_tokens=P), q_dtype)
    mism = np.argwhere(out != expect)
    assert len(mism) == 0, f"{len(mism)} mismatches, first {mism[:4].tolist()}"


@pytest.mark.parametrize("kv_dtype,q_dtype", [("bf16", "bf16"), ("f16", "f16"),
                                               ("fp8_e4m3", "bf16")])
@pytest.mark.parametrize("lens", [(1, 17, 300, 600), (64, 64, 64, 64, 64, 64, 64, 64),
                                  (33, 0, 1, 800, 100)])
def test_small_ragged_batches(kv_dtype, q_dtype, lens):
    """Small ragged batches (2 KV heads, a few hundred to a few thousand keys): chunks of two
    blocks holding pieces of several sequence heads, empty sequences, a head cut across
    workgroups; decode alone and with the append fused in."""
    spec = Spec("small_ragged", len(lens), 8, 2, 128, q_dtype, kv_dtype, ("list", lens),
                pool=("times", 2), seed=43)
    wl = workloads.make(spec)
    dev = Dev(wl)
    dev.append()
    ref, k_ref, v_ref = oracle_after_append(wl)
    # contexts of 1 and 0 tokens: an fp8 code times its scale (counted rounding-limited relief)
    assert_close(dev.decode(partition_tokens=0), ref, q_dtype, f"small ragged {lens}",
                 relief=kv_dtype == "fp8_e4m3")
    fused = Dev(wl)
    pa.pa_decode_append(fused.q, fused.k_new, fused.v_new, fused.k_cache, fused.v_cache,
                        fused.tables, fused.lens, float(wl.scale), fused.out,
                        k_scale=fused.k_scale, v_scale=fused.v_scale,
                        max_context_len=wl.max_context_len)
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(fused.k_cache), k_ref)
    assert np.array_equal(host_bits(fused.v_cache), v_ref)
    assert np.array_equal(host_bits(fused.out), dev.decode(partition_tokens=0))


@pytest.mark.parametrize("kv_dtype,q_dtype", [("bf16", "bf16"), ("fp8_e4m3", "bf16"),
                                               ("f16", "f16")])
@pytest.mark.parametrize("scale", [0.0, -0.09])
@pytest.mark.parametrize("P", [0, 64])
def test_zero_and_negative_scale(kv_dtype, q_dtype, scale, P):
    """A zero softmax scale gives every visible key the same weight (the output is the mean of
    V), a negative one weights the smallest scores most; ragged lengths put masked slots in the
    last step of most heads.  Balanced split and fixed partitions."""
    lens = (1, 17, 300, 600, 33, 0, 129)
    spec = Spec("scales", len(lens), 8, 2, 128, q_dtype, kv_dtype, ("list", lens),
                pool=("times", 2), seed=47)
    wl = workloads.make(spec)
    wl.scale = scale
    dev = Dev(wl)
    dev.append()
    ref, _, _ = oracle_after_append(wl)
    assert_close(dev.decode(partition_tokens=P), ref, q_dtype, f"scale {scale} P{P}",
                 relief=True)


@pytest.mark.parametrize("kv_dtype,q_dtype", [("bf16", "bf16"), ("f16", "f16")])
def test_length_one_returns_v_exactly(kv_dtype, q_dtype):
    spec = Spec("one", 5, 16, 2, 128, q_dtype, kv_dtype, ("list", (1,) * 5), pool=("times", 2),
                seed=43)
    wl = workloads.make(spec)
    dev = Dev(wl)
    dev.append()
    out = dev.decode()
    for b in range(5):
        for h in range(16):
            assert np.array_equal(out[b, h], wl.v_new[b, h // 8])


def test_length_zero_gives_zeros():
    spec = Spec("zero", 4, 8, 2, 128, "bf16", "bf16", ("list", (0, 40, 0, 700)),
                pool=("times", 2), seed=44)
    wl = workloads.make(spec)
    dev = Dev(wl)
    dev.out.fill_(float("nan"))
    dev.append()
    out = dev.decode(partition_tokens=256)
    assert (out[0] == 0).all() and (out[2] == 0).all()
    ref, _, _ = oracle_after_append(wl)
    assert_close(out, ref, "bf16", "zero-length batch")


# Heads of at most 16 blocks that fit the resident waves take the head mode: 1, 2, 4 or 8
# waves per sequence head (blocks / 2 rounded up to a power of two), one 32-token step each,
# the pieces of a head merged in LDS.  Lengths by waves per head, each set with an empty
# sequence, single tokens and block edges.
SHORT_LENS = {1: (1, 0, 32, 20, 17), 2: (33, 64, 0, 1, 50), 4: (100, 7, 128, 0, 65, 16),
              8: (256, 1, 0, 129, 200, 17, 240, 255)}


@pytest.mark.parametrize("q_dtype,kv_dtype,hkv,g,d", [("bf16", "bf16", 2, 8, 128),
                                                      ("f16", "f16", 4, 1, 64),
                                                      ("bf16", "fp8_e4m3", 2, 4, 128),
                                                      ("f16", "fp8_e4m3", 1, 16, 64)])
@pytest.mark.parametrize("wph", [1, 2, 4, 8])
def test_short_heads(q_dtype, kv_dtype, hkv, g, d, wph):
    """Short heads: decode and the fused step against the oracle; rows of an empty sequence are
    zeros; the fused append leaves the caches of the separate append and the same output."""
    lens = SHORT_LENS[wph]
    spec = Spec("short", len(lens), hkv * g, hkv, d, q_dtype, kv_dtype, ("list", lens),
                pool=("times", 2), seed=50 + wph)
    wl = workloads.make(spec)
    assert wl.max_context_len <= 16 * 2 * wph
    dev = Dev(wl)
    dev.out.fill_(float("nan"))
    dev.append()
    out = dev.decode(partition_tokens=0)
    ref, k_ref, v_ref = oracle_after_append(wl)
    assert_close(out, ref, q_dtype, f"short heads wph={wph}", relief=kv_dtype == "fp8_e4m3")
    for b in np.flatnonzero(wl.context_lens == 0):
        assert (out[b] == 0).all()
    fused = Dev(wl)
    fused.out.fill_(float("nan"))
    pa.pa_decode_append(fused.q, fused.k_new, fused.v_new, fused.k_cache, fused.v_cache,
                        fused.tables, fused.lens, float(wl.scale), fused.out,
                        k_scale=fused.k_scale, v_scale=fused.v_scale,
                        max_context_len=wl.max_context_len)
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(fused.k_cache), k_ref)
    assert np.array_equal(host_bits(fused.v_cache), v_ref)
    assert np.array_equal(host_bits(fused.out), out)


@pytest.mark.parametrize("kv_dtype,q_dtype", [("bf16", "bf16"), ("fp8_e4m3", "bf16")])
def test_short_heads_needle_bit_exact(kv_dtype, q_dtype):
    """The needle through the head mode's LDS merge (8 waves per head)."""
    L = 250
    t_stars = (0, 15, 16, 31, 32, 33, 100, 127, 128, 200, L - 1)
    wl, q, k, v, ks, vs, expect = _needle_setup(kv_dtype, q_dtype, t_stars, L)
    dev = Dev(wl)
    dev.q = dev_bits(q, q_dtype)
    dev.k_cache = dev_bits(k, kv_dtype)
    dev.v_cache = dev_bits(v, kv_dtype)
    if ks is not None:
        dev.k_scale = torch.from_numpy(ks).cuda()
        dev.v_scale = torch.from_numpy(vs).cuda()
    out = oracle.to_f64(dev.decode(partition_tokens=0), q_dtype)
    mism = np.argwhere(out != expect)
    assert len(mism) == 0, f"{len(mism)} mismatches, first {mism[:4].tolist()}"


def test_short_heads_with_shared_prefix():
    """Head mode with shared prefixes: members skip the shared blocks and fold the prefix parts
    in; the same call without sharing reads the prefix per sequence."""
    spec = Spec("short_prefix", 10, 16, 2, 128, "bf16", "bf16",
                ("list", (40, 3, 120, 0, 77, 17, 150, 96, 1, 60)), prefix=(5, 64),
                pool=("times", 2), seed=58)
    wl = workloads.make(spec)
    assert wl.max_context_len <= 256 and len(wl.sharing) == 5
    dev = Dev(wl)
    dev.append()
    ref, _, _ = oracle_after_append(wl)
    planned = dev.decode(partition_tokens=0, shared_prefixes=True)
    assert_close(planned, ref, "bf16", "short heads, shared prefix")
    unshared = dev.decode(partition_tokens=0)
    assert_close(unshared, ref, "bf16", "short heads, prefix read per sequence")


def _relocate(wl, seed):
    """Same logical K/V, every used block moved to a fresh random physical block."""
    rng = np.random.default_rng(seed)
    NB = wl.num_blocks
    perm = rng.permutation(NB)
    k = np.empty_like(wl.k_cache)
    v = np.empty_like(wl.v_cache)
    k[perm] = wl.k_cache
    v[perm] = wl.v_cache
    tables = perm[wl.block_tables].astype(np.int32)
    slots = np.where(wl.slot_mapping >= 0,
                     perm[wl.slot_mapping // BLOCK] * BLOCK + wl.slot_mapping % BLOCK, -1)
    ks = vs = None
    if wl.k_scale is not None:
        ks = np.empty_like(wl.k_scale)
        vs = np.empty_like(wl.v_scale)
        ks[perm] = wl.k_scale
        vs[perm] = wl.v_scale
    return k, v, tables, slots.astype(np.int64), ks, vs


@pytest.mark.parametrize("kv_dtype,q_dtype", [("bf16", "bf16"), ("fp8_e4m3", "bf16"),
                                               ("f16", "f16")])
def test_physical_placement_is_bitwise_invisible(kv_dtype, q_dtype):
    spec = Spec("perm", 8, 16, 2, 128, q_dtype, kv_dtype,
                ("list", (1, 17, 100, 511, 513, 1500, 33, 64)), pool=("times", 2), seed=45)
    wl = workloads.make(spec)
    outs = []
    for seed in (None, 1, 2):
        dev = Dev(wl)
        if seed is not None:
            k, v, tables, slots, ks, vs = _relocate(wl, seed)
            dev.k_cache, dev.v_cache = dev_bits(k, kv_dtype), dev_bits(v, kv_dtype)
            dev.tables = torch.from_numpy(tables).cuda()
            dev.slots = torch.from_numpy(slots).cuda()
            if ks is not None:
                dev.k_scale, dev.v_scale = torch.from_numpy(ks).cuda(), torch.from_numpy(vs).cuda()
        dev.append()
        outs.append(dev.decode(partition_tokens=128))
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[0], outs[2])


def test_shared_prefix_equals_private_copies_bitwise():
    spec = Spec("prefix", 12, 16, 2, 128, "bf16", "bf16", ("lognormal", 100.0, 1.0, 3000),
                prefix=(4, 256), pool=("times", 2), seed=46)
    wl = workloads.make(spec)
    shared = Dev(wl)
    shared.append()
    out_shared = shared.decode(partition_tokens=128)
    # private copies: each sharing sequence gets its own copy of the prefix blocks
    nb_pre = wl.prefix_blocks
    extra = len(wl.sharing) * nb_pre
    NB = wl.num_blocks
    k = np.concatenate([wl.k_cache, np.zeros((extra,) + wl.k_cache.shape[1:], wl.k_cache.dtype)])
    v = np.concatenate([wl.v_cache, np.zeros((extra,) + wl.v_cache.shape[1:], wl.v_cache.dtype)])
    tables = wl.block_tables.copy()
    for i, b in enumerate(wl.sharing):
        for j in range(nb_pre):
            new = NB + i * nb_pre + j
            k[new] = wl.k_cache[wl.block_tables[b, j]]
            v[new] = wl.v_cache[wl.block_tables[b, j]]
            tables[b, j] = new
    assert len(np.unique(tables[wl.sharing, :nb_pre])) == extra
    private = Dev(wl)
    private.k_cache, private.v_cache = dev_bits(k, "bf16"), dev_bits(v, "bf16")
    private.tables = torch.from_numpy(tables).cuda()
    private.append()
    out_private = private.decode(partition_tokens=128)
    assert np.array_equal(out_shared, out_private)
    ref, _, _ = oracle_after_append(wl)
    assert_close(out_shared, ref, "bf16", "prefix sharing")


def test_repeat_runs_bitwise_identical():
    wl = workloads.make(Spec("det", 16, 32, 4, 128, "bf16", "bf16", ("uniform", 1, 3000),
                             pool=("times", 2), seed=47))
    dev = Dev(wl)
    dev.append()
    first = dev.decode()
    for _ in range(3):
        assert np.array_equal(dev.decode(), first)


def test_context_lengths_are_clamped_to_the_launch():
    wl = workloads.make(Spec("clamp", 4, 8, 2, 128, "bf16", "bf16", ("list", (640, 300, 90, 64)),
                             pool=("times", 2), seed=48))
    dev = Dev(wl)
    dev.append()
    # the host hint says 256 tokens: every sequence is attended over at most 256 tokens
    out = dev.decode(partition_tokens=128, max_context_len=256)
    k, v = oracle.kv_append(wl.k_cache, wl.v_cache, wl.k_new, wl.v_new, wl.slot_mapping)
    lens = np.minimum(wl.context_lens, 256)
    ref = oracle.decode(wl.q, k, v, wl.block_tables, lens, wl.scale, "bf16", "bf16")
    assert_close(out, ref, "bf16", "hint clamp")
    # a device length beyond the table row is clamped to the row (640 = 40 full blocks)
    dev.lens = torch.tensor([10_000, 300, 90, 64], dtype=torch.int32, device="cuda")
    out = dev.decode(partition_tokens=128, max_context_len=0)
    ref = oracle.decode(wl.q, k, v, wl.block_tables, wl.context_lens, wl.scale, "bf16", "bf16")
    assert_close(out, ref, "bf16", "table clamp")


def test_short_workspace_is_rejected():
    wl = workloads.make(Spec("ws", 2, 8, 2, 128, "bf16", "bf16", ("list", (600, 10)),
                             pool=("times", 2), seed=49))
    dev = Dev(wl)
    small = torch.empty(64, dtype=torch.uint8, device="cuda")
    with pytest.raises(pa.PaError) as e:
        pa.pa_decode(dev.q, dev.k_cache, dev.v_cache, dev.tables, dev.lens, float(wl.scale),
                     dev.out, partition_tokens=128, workspace=small)
    assert e.value.status == pa.PA_ERR_WORKSPACE


@pytest.mark.parametrize("name", workloads.spec_names())
def test_full_size_workload(name):
    """Each workload at full size, in the launch configuration the benchmark times (shared
    prefixes on for the workload with a shared prefix, and off as well): the append is bit-exact
    over the whole pool and every output element is within tolerance."""
    wl = workloads.make(name)
    dev = Dev(wl)
    dev.append()
    torch.cuda.synchronize()
    ref, k_ref, v_ref = oracle_after_append(wl)
    assert np.array_equal(host_bits(dev.k_cache), k_ref)
    assert np.array_equal(host_bits(dev.v_cache), v_ref)
    for share in ((False, True) if wl.spec.prefix is not None else (False,)):
        out = dev.decode(shared_prefixes=share)
        assert_close(out, ref, wl.spec.q_dtype, label=f"{name} shared_prefixes={share}")
