"""pa_decode with shared_prefixes on, against the fp64 oracle.

Sequences whose block tables start with the same physical blocks share those blocks' K/V (the
youngju.dev guide, PagedAttention "主な特性", and the Scaling Book note, "プレフィックスキャッシュ").
The oracle gathers every sequence through its own table row, so it knows nothing of the grouping;
these cases build tables with groups of every shape the plan distinguishes (shared length odd or
capped, a member that diverges early, identical rows, members whose last token sits right after
the shared part, tiles of 1..16 columns, batches where the plan is skipped) and check that the
result is the same attention within tolerance, and bitwise equal to the unshared path where the
plan is not taken."""

import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import Dev, assert_close, dev_bits, host_bits
from workloads.generate import Spec

pytestmark = pytest.mark.gpu
BLOCK = 16


def _setup(q_dtype, kv_dtype, hkv, g, d, lens, seed):
    spec = Spec("share", len(lens), hkv * g, hkv, d, q_dtype, kv_dtype, ("list", tuple(lens)),
                pool=("times", 2), seed=seed)
    wl = workloads.make(spec)
    k, v = oracle.kv_append(wl.k_cache, wl.v_cache, wl.k_new, wl.v_new, wl.slot_mapping)
    return wl, k, v


def _share(tables, leader, members, nblocks):
    for b in members:
        tables[b, :nblocks] = tables[leader, :nblocks]


def _run(wl, k, v, tables, label, P=0, share=True, lens=None):
    s = wl.spec
    lens = wl.context_lens if lens is None else np.asarray(lens, dtype=np.int32)
    dev = Dev(wl)
    dev.k_cache, dev.v_cache = dev_bits(k, s.kv_dtype), dev_bits(v, s.kv_dtype)
    dev.tables = torch.from_numpy(np.ascontiguousarray(tables)).cuda()
    dev.lens = torch.from_numpy(lens).cuda()
    out = dev.decode(partition_tokens=P, max_context_len=0, shared_prefixes=share)
    ref = oracle.decode(wl.q, k, v, tables, lens, wl.scale, s.q_dtype, s.kv_dtype, wl.k_scale,
                        wl.v_scale)
    assert_close(out, ref, s.q_dtype, label)
    return out


LENS = (700, 1500, 1201, 977, 33, 1300, 48, 49, 2000, 640, 641, 1100, 0, 17, 900, 1024)

GROUPED = [
    # (q dtype, kv dtype, kv heads, group, head_dim, partition)
    ("bf16", "bf16", 2, 8, 128, 0),
    ("bf16", "bf16", 2, 4, 128, 0),
    ("bf16", "bf16", 2, 4, 128, 64),
    ("bf16", "bf16", 2, 2, 64, 0),
    ("bf16", "bf16", 4, 1, 128, 0),
    ("bf16", "bf16", 2, 3, 128, 0),
    ("f16", "f16", 2, 4, 128, 0),
    ("f16", "f16", 2, 8, 64, 512),
    ("bf16", "fp8_e4m3", 2, 4, 128, 0),
    ("f16", "fp8_e4m3", 2, 8, 128, 128),
]


@pytest.mark.parametrize("case", GROUPED, ids=lambda c: f"{c[0]}-{c[1]}-kv{c[2]}g{c[3]}d{c[4]}"
                         f"-P{c[5]}")
def test_groups_of_every_shape(case):
    qd, kvd, hkv, g, d, P = case
    wl, k, v = _setup(qd, kvd, hkv, g, d, LENS, seed=61 + GROUPED.index(case))
    t = wl.block_tables.copy()
    # group A, leader 1 (94 blocks): 2, 3, 5, 8, 11, 14 share 40 blocks, but 11 diverges at
    # block 33 -> a shared length of 33 (odd) for the whole group
    _share(t, 1, (2, 3, 5, 8, 11, 14), 40)
    t[11, 33:40] = t[9, 33:40]
    # group B: 9 and 10 share all their blocks; 9 has 640 tokens (40 whole blocks), so the last
    # one is its own and the shared length is 39
    _share(t, 9, (10,), 40)
    # group C: shortest usable group, 48 and 49 tokens share 2 blocks
    _share(t, 6, (7,), 3)
    # not a group: 17 tokens share one block with 4 (33 tokens); 15 shares only its first block
    _share(t, 4, (13,), 1)
    _share(t, 0, (15,), 1)
    _run(wl, k, v, t, f"groups {case}", P=P)


def test_shared_length_is_capped_and_members_keep_their_last_block():
    # 0 and 1 have identical rows of 313 blocks and 2 (4097 tokens) shares 257: the shared part
    # stops at 256 blocks, so 2 keeps the block of its last token.  3 (4096 tokens) and 4 (300)
    # share 19 blocks, of which 4 keeps the last one: 18 are shared.
    lens = (5000, 5000, 4097, 4096, 300)
    wl, k, v = _setup("bf16", "bf16", 2, 4, 128, lens, seed=71)
    t = wl.block_tables.copy()
    _share(t, 0, (1,), 313)
    _share(t, 0, (2,), 257)
    _share(t, 3, (4,), 19)
    _run(wl, k, v, t, "cap 256")


def test_many_members_fill_several_tiles():
    # group of 1 (MHA): 16 members per tile -> tiles of 16, 16, 8; a second group of 3
    lens = [800 + 37 * i for i in range(44)]
    wl, k, v = _setup("bf16", "bf16", 2, 1, 128, lens, seed=72)
    t = wl.block_tables.copy()
    _share(t, 3, [b for b in range(40) if b != 3], 48)
    _share(t, 40, (41, 42), 20)
    _run(wl, k, v, t, "tiles of 16")
    # group of 8: two members per tile -> 4 tiles for 7 members
    lens = [500 + 11 * i for i in range(9)]
    wl, k, v = _setup("bf16", "bf16", 2, 8, 128, lens, seed=73)
    t = wl.block_tables.copy()
    _share(t, 0, range(1, 7), 30)
    _run(wl, k, v, t, "tiles of 2")


def test_repeat_runs_bitwise_identical_with_sharing():
    wl, k, v = _setup("bf16", "bf16", 2, 4, 128, LENS, seed=74)
    t = wl.block_tables.copy()
    _share(t, 1, (2, 3, 5, 8, 11, 14), 40)
    first = _run(wl, k, v, t, "repeat")
    for _ in range(3):
        assert np.array_equal(_run(wl, k, v, t, "repeat"), first)


@pytest.mark.parametrize("g,batch", [(16, 8), (4, 1100)])
def test_plan_not_taken_is_the_unshared_path(g, batch):
    """group 16 (one member per tile) and batches over 1024 are run without a plan: bitwise the
    same output as with shared_prefixes off."""
    rng = np.random.default_rng(75)
    lens = rng.integers(40, 400 if batch > 100 else 2000, size=batch)
    wl, k, v = _setup("bf16", "bf16", 1, g, 128, lens, seed=75)
    t = wl.block_tables.copy()
    _share(t, 0, range(1, batch // 2), 2)
    on = _run(wl, k, v, t, f"g{g} b{batch} on", share=True)
    off = _run(wl, k, v, t, f"g{g} b{batch} off", share=False)
    assert np.array_equal(on, off)


def _abi_decode(dev, mode, ws, partition=0):
    """pa_decode through the C ABI itself (none of the binding's bookkeeping), with
    shared_prefixes = mode and the given workspace."""
    import ctypes

    import paged_kv_cache_31_amd as pa

    def ptr(t):
        return None if t is None else ctypes.c_void_p(t.data_ptr())

    desc = pa.decode_desc(dev.q, dev.k_cache, dev.tables, 0, partition, mode)
    st = pa.lib().pa_decode(ctypes.byref(desc), ptr(dev.q), ptr(dev.k_cache), ptr(dev.v_cache),
                            ptr(dev.k_scale), ptr(dev.v_scale), ptr(dev.tables), ptr(dev.lens),
                            ctypes.c_float(float(dev.wl.scale)), ptr(dev.out), ptr(ws),
                            ctypes.c_size_t(ws.numel()),
                            ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == pa.PA_OK, pa.status_string(st)
    torch.cuda.synchronize()
    return host_bits(dev.out)


def _layer(wl, k, v, tables):
    s = wl.spec
    dev = Dev(wl)
    dev.k_cache, dev.v_cache = dev_bits(k, s.kv_dtype), dev_bits(v, s.kv_dtype)
    dev.tables = torch.from_numpy(np.ascontiguousarray(tables)).cuda()
    return dev


def _grouped_tables(wl):
    t = wl.block_tables.copy()
    _share(t, 1, (2, 3, 5, 8, 11, 14), 40)
    t[11, 33:40] = t[9, 33:40]
    _share(t, 9, (10,), 40)
    _share(t, 6, (7,), 3)
    return t


def _workspace(dev, extra=0):
    import paged_kv_cache_31_amd as pa
    need = max(pa.pa_decode_workspace_size(pa.decode_desc(dev.q, dev.k_cache, dev.tables, 0, P, 1))
               for P in (0, 128))
    return pa.new_workspace(max(need, extra), dev.q.device)


@pytest.mark.parametrize("kvd", ["bf16", "fp8_e4m3"])
def test_layers_reuse_the_plan(kvd):
    """The layers of one step read the same tables and lengths: the first call plans the groups
    (shared_prefixes 1), the next ones reuse its saved units (2) with their own queries and K/V
    (another layer's cache), and give bitwise what a planning call gives.  Through the C ABI, so
    that the reusing calls really take the saved plan."""
    import copy
    wl0, k0, v0 = _setup("bf16", kvd, 2, 4, 128, LENS, seed=76)
    # another layer over the same blocks: other queries, K with its sign bits flipped, V
    # reversed along the head dimension (unused, poisoned blocks stay poisoned)
    wl1 = copy.copy(wl0)
    wl1.q = _setup("bf16", kvd, 2, 4, 128, LENS, seed=77)[0].q
    sign = np.uint8(0x80) if kvd == "fp8_e4m3" else np.uint16(0x8000)
    k1 = k0 ^ sign
    v1 = np.ascontiguousarray(v0[:, :, ::-1, :])
    t = _grouped_tables(wl0)
    dev0, dev1 = _layer(wl0, k0, v0, t), _layer(wl1, k1, v1, t)
    ws = _workspace(dev0)
    first = _abi_decode(dev0, 1, ws)
    reused = _abi_decode(dev1, 2, ws)
    again = _abi_decode(dev0, 2, ws)
    assert np.array_equal(again, first)
    planned = _abi_decode(dev1, 1, ws)
    assert np.array_equal(reused, planned)
    s = wl1.spec
    ref = oracle.decode(wl1.q, k1, v1, t, wl1.context_lens, wl1.scale, s.q_dtype, s.kv_dtype,
                        wl1.k_scale, wl1.v_scale)
    assert_close(reused, ref, s.q_dtype, f"layer 1 reuses ({kvd})")
    # with sharing on, the plan is really taken: the result differs from the unshared path
    off = _abi_decode(dev1, 0, _workspace(dev1))
    assert not np.array_equal(reused, off)


def test_reuse_on_a_fresh_workspace_is_the_unshared_path():
    """shared_prefixes 2 on a zero-filled workspace that no planning call has written reads no
    shared blocks: bitwise the output with shared prefixes off."""
    wl, k, v = _setup("bf16", "bf16", 2, 4, 128, LENS, seed=78)
    t = wl.block_tables.copy()
    _share(t, 1, (2, 3, 5, 8, 11, 14), 40)
    dev = _layer(wl, k, v, t)
    off = _abi_decode(dev, 0, _workspace(dev))
    assert np.array_equal(_abi_decode(dev, 2, _workspace(dev)), off)


def test_reuse_after_the_workspace_was_overwritten():
    """A reusing call whose workspace another call has written since the planning call (here:
    pa_decode_multi, whose scratch overlaps the saved plan, and then random bytes over all of
    the workspace but its arrival counters) finds a foreign signature and runs unshared; a
    changed descriptor (another max_context_len) is refused the same way.  Through the C ABI:
    the kernels alone must keep every access in bounds and the result right."""
    import ctypes

    import paged_kv_cache_31_amd as pa
    wl, k, v = _setup("bf16", "bf16", 2, 4, 128, LENS, seed=79)
    t = _grouped_tables(wl)
    dev = _layer(wl, k, v, t)
    s = wl.spec
    ref = oracle.decode(wl.q, k, v, t, wl.context_lens, wl.scale, s.q_dtype, s.kv_dtype)
    # a multi-query problem over the same cache: 4 rows per sequence, fixed partitions of 32
    T = np.minimum(4, wl.context_lens).astype(np.int64)
    qs = np.concatenate([[0], np.cumsum(T)]).astype(np.int32)
    N = int(qs[-1])
    qm = dev_bits(workloads.storage_bits(np.random.default_rng(5).standard_normal(
        (N, s.num_q_heads, s.head_dim)), "bf16"), "bf16")
    om = torch.empty_like(qm)
    mdesc = pa.multi_desc(qm, dev.k_cache, dev.tables, 4, 0, 32)
    need_m = pa.pa_decode_multi_workspace_size(mdesc)
    ws = _workspace(dev, need_m)
    planned = _abi_decode(dev, 1, ws)
    off = _abi_decode(dev, 0, _workspace(dev))
    assert not np.array_equal(planned, off)
    qsd = torch.from_numpy(qs).cuda()

    def p(x):
        return ctypes.c_void_p(x.data_ptr())
    st = pa.lib().pa_decode_multi(ctypes.byref(mdesc), p(qm), p(qsd), p(dev.k_cache),
                                  p(dev.v_cache), None, None, p(dev.tables), p(dev.lens),
                                  ctypes.c_float(float(wl.scale)), p(om), p(ws),
                                  ctypes.c_size_t(ws.numel()),
                                  ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == pa.PA_OK
    torch.cuda.synchronize()
    got = _abi_decode(dev, 2, ws)
    assert np.array_equal(got, off) or np.array_equal(got, planned)
    assert_close(got, ref, s.q_dtype, "reuse after pa_decode_multi")
    # random bytes over everything after the counters: the signature is foreign
    _abi_decode(dev, 1, ws)
    g = torch.Generator(device="cuda").manual_seed(7)
    ws[65536 * 4:] = torch.randint(0, 256, (ws.numel() - 65536 * 4,), dtype=torch.uint8,
                                   device="cuda", generator=g)
    assert np.array_equal(_abi_decode(dev, 2, ws), off)
    # a planning call, then a reuse with another descriptor (fixed partitions of 128 tokens):
    # the signature differs, so the call runs unshared
    _abi_decode(dev, 1, ws)
    assert np.array_equal(_abi_decode(dev, 2, ws, partition=128),
                          _abi_decode(dev, 0, _workspace(dev), partition=128))


def test_binding_plans_again_after_another_call():
    """The binding's prepared calls keep the plan only while nothing else used the workspace:
    planning call, reusing call (takes the plan), a multi-query call on the same workspace,
    then the reusing call plans again (bitwise the planning output)."""
    import paged_kv_cache_31_amd as pa
    wl, k, v = _setup("bf16", "bf16", 2, 4, 128, LENS, seed=80)
    t = _grouped_tables(wl)
    dev = _layer(wl, k, v, t)
    s = wl.spec
    T = np.minimum(2, wl.context_lens).astype(np.int64)
    qs = torch.from_numpy(np.concatenate([[0], np.cumsum(T)]).astype(np.int32)).cuda()
    qm = dev.q[:0].new_empty((int(T.sum()), s.num_q_heads, s.head_dim)).fill_(0.5)
    om = torch.empty_like(qm)
    mdesc = pa.multi_desc(qm, dev.k_cache, dev.tables, 2, 0, 32)
    ws = _workspace(dev, pa.pa_decode_multi_workspace_size(mdesc))
    outs = [torch.empty_like(dev.out) for _ in range(3)]

    def call(mode, out):
        return pa.DecodeCall(dev.q, dev.k_cache, dev.v_cache, dev.tables, dev.lens,
                             float(wl.scale), out, workspace=ws, shared_prefixes=mode)
    plan, reuse_a, reuse_b = call(1, outs[0]), call(2, outs[1]), call(2, outs[2])
    multi = pa.MultiCall(qm, qs, dev.k_cache, dev.v_cache, dev.tables, dev.lens, float(wl.scale),
                         om, 2, partition_tokens=32, workspace=ws)
    plan()
    reuse_a()
    multi()
    reuse_b()
    torch.cuda.synchronize()
    assert reuse_a.reused and not reuse_b.reused
    first = host_bits(outs[0])
    assert np.array_equal(host_bits(outs[1]), first)
    assert np.array_equal(host_bits(outs[2]), first)


@pytest.mark.parametrize("change", ["member_block", "member_length", "leader_row", "none"])
def test_reuse_checks_the_saved_plan(change):
    """A reusing call (shared_prefixes 2) checks the saved plan against its own tables and
    lengths: a member whose shared entries now differ from its leader's, or whose length no
    longer leaves it a block past the shared ones, reads its whole head instead.  After each
    change the result is the attention over the changed tables (oracle), and with no change it
    is bitwise the planning call's.  Through the C ABI."""
    wl, k, v = _setup("bf16", "bf16", 2, 4, 128, LENS, seed=79)
    t = _grouped_tables(wl)
    dev = _layer(wl, k, v, t)
    ws = _workspace(dev)
    planned = _abi_decode(dev, 1, ws)
    t2, lens2 = t.copy(), wl.context_lens.copy()
    if change == "member_block":          # member 3 now holds another sequence's block at 10
        t2[3, 10] = t[0, 10]
    elif change == "member_length":       # member 8 (2000 tokens) shrinks inside the shared part
        lens2[8] = 100
    elif change == "leader_row":          # the leader's slot now holds another request's blocks
        t2[1, :40] = t[0, :40]
    dev.tables = torch.from_numpy(np.ascontiguousarray(t2)).cuda()
    dev.lens = torch.from_numpy(lens2).cuda()
    reused = _abi_decode(dev, 2, ws)
    s = wl.spec
    ref = oracle.decode(wl.q, k, v, t2, lens2, wl.scale, s.q_dtype, s.kv_dtype)
    assert_close(reused, ref, s.q_dtype, f"reuse after {change}")
    if change == "none":
        assert np.array_equal(reused, planned)
    else:                                 # and a fresh plan of the changed tables agrees
        fresh = _abi_decode(dev, 1, _workspace(dev))
        assert_close(fresh, ref, s.q_dtype, f"planning after {change}")
