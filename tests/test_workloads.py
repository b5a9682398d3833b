"""The seeded generators: determinism, shapes, block placement and the appended token's slot."""

import numpy as np
import pytest

import workloads as W
from workloads.generate import Spec

BLOCK = 16


def test_deterministic():
    a = W.make("tiny_b4_h8kv2_d64_bf16")
    b = W.make("tiny_b4_h8kv2_d64_bf16")
    for f in ("q", "k_cache", "v_cache", "k_new", "v_new", "block_tables", "slot_mapping"):
        assert np.array_equal(getattr(a, f), getattr(b, f)), f
    c = W.make("tiny_b4_h8kv2_d64_bf16", seed=11)
    assert not np.array_equal(a.q, c.q)


def test_tiny_shapes_and_lengths():
    wl = W.make("tiny_b4_h8kv2_d64_bf16")
    assert wl.num_blocks == 64
    assert list(wl.context_lens) == [1, 17, 33, 100]
    assert wl.k_cache.shape == (64, 2, 16, 64) and wl.v_cache.shape == (64, 2, 64, 16)
    assert wl.q.shape == (4, 8, 64) and wl.k_new.shape == (4, 2, 64)
    assert float(wl.scale) == 0.125


def test_blocks_distinct_and_slots_point_at_last_token():
    wl = W.make("tiny_b4_h8kv2_d64_bf16")
    used = []
    for b, L in enumerate(wl.context_lens):
        nb = -(-int(L) // BLOCK)
        used.extend(wl.block_tables[b, :nb])
        s = wl.slot_mapping[b]
        assert s // BLOCK == wl.block_tables[b, (L - 1) // BLOCK] and s % BLOCK == (L - 1) % BLOCK
    assert len(set(used)) == len(used) == 13


def test_poison_everywhere_unread():
    wl = W.make("tiny_b4_h8kv2_d64_bf16")
    used = set()
    for b, L in enumerate(wl.context_lens):
        nb = -(-int(L) // BLOCK)
        used.update(int(x) for x in wl.block_tables[b, :nb])
        # table entries past the last block point at unused blocks
        assert not (set(int(x) for x in wl.block_tables[b, nb:]) & used)
    unused = [i for i in range(wl.num_blocks) if i not in used]
    assert (wl.k_cache[unused] == 0x7FC0).all() and (wl.v_cache[unused] == 0x7FC0).all()
    for b, L in enumerate(wl.context_lens):       # pre-append slot and tail are poisoned
        blk = wl.block_tables[b, (L - 1) // BLOCK]
        assert (wl.k_cache[blk, :, (L - 1) % BLOCK:, :] == 0x7FC0).all()
        assert (wl.v_cache[blk, :, :, (L - 1) % BLOCK:] == 0x7FC0).all()


def test_prefix_sharing_structure():
    spec = W.SPECS["mixed_b256_h32kv8_d128_bf16_lognorm600_prefix1024"].replace(
        batch=16, prefix=(4, 64), lengths=("lognormal", 60.0, 1.0, 300), num_q_heads=4,
        num_kv_heads=2, head_dim=16)
    wl = W.make(spec)
    assert len(wl.sharing) == 4 and wl.prefix_blocks == 4
    rows = wl.block_tables[wl.sharing, :4]
    assert (rows == rows[0]).all()                      # same physical prefix blocks
    assert (wl.context_lens[wl.sharing] > 64).all()
    others = [b for b in range(16) if b not in set(wl.sharing)]
    for b in others:
        nb = -(-int(wl.context_lens[b]) // BLOCK)
        assert not set(wl.block_tables[b, :nb]) & set(rows[0])
    assert wl.unique_tokens == int(wl.context_lens.sum()) - 3 * 64


def test_fp8_scales_are_tile_amax_over_448():
    spec = W.SPECS["tiny_b4_h8kv2_d64_bf16"].replace(kv_dtype="fp8_e4m3")
    wl = W.make(spec)
    import torch
    blk = int(wl.block_tables[3, 0])      # a full block of the 100-token sequence
    codes = torch.from_numpy(wl.k_cache[blk]).view(torch.float8_e4m3fn).float()
    amax_codes = codes.abs().amax(dim=(1, 2))
    assert torch.all(amax_codes == 448)    # the largest |value| maps onto the largest code
    assert np.isfinite(wl.k_scale[blk]).all() and (wl.k_scale[blk] > 0).all()


@pytest.mark.parametrize("name", ["gqa_b64_h64kv8_d128_bf16_l128to8192",
                                  "mixed_b256_h32kv8_d128_bf16_lognorm600_prefix1024"])
def test_length_distributions(name):
    spec = W.SPECS[name].replace(num_kv_heads=1, num_q_heads=1, head_dim=8)
    wl = W.make(spec, poison=False)
    L = wl.context_lens
    if name.startswith("gqa"):
        assert L.min() >= 128 and L.max() <= 8192
    else:
        assert L.min() >= 1 and L.max() <= 16384
        assert 300 < np.median(L[[b for b in range(256) if b not in set(wl.sharing)]]) < 1200
