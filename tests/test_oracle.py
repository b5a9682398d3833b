"""Pins for the fp64 oracle, each against something other than the oracle itself (CPU only)."""

import json
import math
import os
import struct

import numpy as np
import pytest
import torch

import oracle
import workloads
from cpu_cases import Case, round_bits, torch_decode
from workloads.generate import Spec

BLOCK = 16


# ---------------------------------------------------------------- dtype decoders vs torch / numpy

def test_bf16_decoder_matches_torch_all_patterns():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(oracle.bf16_to_f64(bits), ref)


def test_f16_decoder_matches_torch_all_patterns():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.float16).to(torch.float64).numpy()
    np.testing.assert_array_equal(oracle.f16_to_f64(bits), ref)


def test_e4m3fn_table_matches_torch_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    np.testing.assert_array_equal(oracle.e4m3fn_to_f64(codes), ref)


def test_e4m3fn_special_values():
    t = oracle.E4M3FN_TABLE
    assert t[0x7E] == 448.0 and t[0xFE] == -448.0          # largest finite
    assert t[0x01] == 2.0**-9                               # smallest subnormal
    assert t[0x08] == 2.0**-6                               # smallest normal
    assert t[0x38] == 1.0 and t[0xB8] == -1.0
    assert np.isnan(t[0x7F]) and np.isnan(t[0xFF])          # the only NaNs, no infinities
    assert np.isfinite(np.delete(t, [0x7F, 0xFF])).all()


# ---------------------------------------------------------------- attention vs library SDPA

@pytest.mark.parametrize("kv_dtype,q_dtype", [("bf16", "bf16"), ("f16", "f16"),
                                               ("fp8_e4m3", "bf16")])
@pytest.mark.parametrize("G", [1, 3])
def test_decode_matches_sdpa_on_contiguous_arrays(kv_dtype, q_dtype, G):
    rng = np.random.default_rng(10 + G)
    case = Case(rng, [1, 15, 16, 17, 33, 70, 0], Hkv=2, G=G, D=16, kv_dtype=kv_dtype,
                q_dtype=q_dtype)
    got = oracle.decode(**case.oracle_args())
    np.testing.assert_allclose(got, case.sdpa(), rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("names,lens,pool", [(("Req1", "Req2"), (20, 32), 4),
                                             (("A", "B"), (40, 17), 10)])
def test_pages_block_table_examples(golden_dir, names, lens, pool):
    """The pages' concrete logical->physical maps (each figure in its own pool)."""
    g = json.load(open(os.path.join(golden_dir, "pages_block_tables.json")))
    tables = [g["tables"][n] for n in names]
    rng = np.random.default_rng(7)
    case = Case(rng, lens, Hkv=2, G=2, D=8, pool_blocks=pool, tables=tables)
    got = oracle.decode(**case.oracle_args())
    np.testing.assert_allclose(got, case.sdpa(), rtol=1e-12, atol=1e-13)
    # logical block 1 of the first request sits in its listed physical block
    phys = tables[0][1]
    assert np.array_equal(torch_decode(case.k_cache[phys, 0, 0], "bf16"), case.K[0][0][16])
    assert np.array_equal(torch_decode(case.k_cache[tables[1][0], 1, 5], "bf16"), case.K[1][1][5])


def test_permutation_invariance_bitwise():
    """Same logical K/V behind different physical placements gives bit-identical results."""
    lens = [5, 16, 47, 64]
    outs = []
    for perm_seed in range(3):
        rng = np.random.default_rng(99)           # same logical values every time
        case = Case(rng, lens, Hkv=2, G=2, D=8)
        # re-place the same logical data with another permutation
        prng = np.random.default_rng(1000 + perm_seed)
        nblk = [-(-L // BLOCK) for L in lens]
        perm = prng.permutation(case.NB)
        k2 = np.full_like(case.k_cache, 0x7FC0)
        v2 = np.full_like(case.v_cache, 0x7FC0)
        t2 = np.zeros_like(case.tables)
        c = 0
        for b, n in enumerate(nblk):
            for j in range(n):
                src, dst = case.tables[b, j], perm[c]
                k2[dst] = case.k_cache[src]
                v2[dst] = case.v_cache[src]
                t2[b, j] = dst
                c += 1
        args = case.oracle_args()
        args.update(k_cache=k2, v_cache=v2, block_tables=t2)
        outs.append(oracle.decode(**args))
        np.testing.assert_allclose(outs[-1], case.sdpa(), rtol=1e-12, atol=1e-13)
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[0], outs[2])


# ---------------------------------------------------------------- brute force, flat addresses

def _scalar(bits, dtype):
    bits = int(bits)
    if dtype == "bf16":
        return struct.unpack("<f", struct.pack("<I", bits << 16))[0]
    if dtype == "f16":
        return struct.unpack("<e", struct.pack("<H", bits))[0]
    return float(torch.tensor([bits], dtype=torch.uint8).view(torch.float8_e4m3fn)
                 .to(torch.float64)[0])


def _brute(wl):
    """Explicit loops over flat pool addresses; token L-1 is read from the new-token rows
    (the cache holds L-1 tokens, the new one is concatenated, as in the contiguous module)."""
    s = wl.spec
    B, Hq, Hkv, D = s.batch, s.num_q_heads, s.num_kv_heads, s.head_dim
    G = Hq // Hkv
    kf, vf = wl.k_cache.reshape(-1), wl.v_cache.reshape(-1)
    sc = float(wl.scale)
    out = np.zeros((B, Hq, D))
    for b in range(B):
        L = int(wl.context_lens[b])
        for h in range(Hq):
            kvh = h // G
            qv = [_scalar(wl.q[b, h, d], s.q_dtype) for d in range(D)]
            keys, vals = [], []
            for t in range(L):
                blk = int(wl.block_tables[b, t // BLOCK])
                off = t % BLOCK
                ksc = float(wl.k_scale[blk, kvh]) if wl.k_scale is not None else 1.0
                vsc = float(wl.v_scale[blk, kvh]) if wl.v_scale is not None else 1.0
                if t == L - 1:
                    krow = [_scalar(wl.k_new[b, kvh, d], s.kv_dtype) * ksc for d in range(D)]
                    vrow = [_scalar(wl.v_new[b, kvh, d], s.kv_dtype) * vsc for d in range(D)]
                else:
                    krow = [_scalar(kf[((blk * Hkv + kvh) * BLOCK + off) * D + d], s.kv_dtype) * ksc
                            for d in range(D)]
                    vrow = [_scalar(vf[((blk * Hkv + kvh) * D + d) * BLOCK + off], s.kv_dtype) * vsc
                            for d in range(D)]
                keys.append(krow)
                vals.append(vrow)
            if L == 0:
                continue
            scores = [sc * math.fsum(qv[d] * k[d] for d in range(D)) for k in keys]
            mx = max(scores)
            e = [math.exp(x - mx) for x in scores]
            tot = math.fsum(e)
            for d in range(D):
                out[b, h, d] = math.fsum(e[t] / tot * vals[t][d] for t in range(L))
    return out


@pytest.mark.parametrize("kv_dtype,q_dtype,G,D", [("bf16", "bf16", 3, 8), ("f16", "f16", 1, 16),
                                                   ("fp8_e4m3", "bf16", 2, 8)])
def test_append_then_decode_matches_brute_force(kv_dtype, q_dtype, G, D):
    spec = Spec("brute", 3, 2 * G, 2, D, q_dtype, kv_dtype, ("list", (1, 18, 40)),
                pool=("times", 2), seed=5)
    wl = workloads.make(spec)
    k, v = oracle.kv_append(wl.k_cache, wl.v_cache, wl.k_new, wl.v_new, wl.slot_mapping)
    got = oracle.decode(wl.q, k, v, wl.block_tables, wl.context_lens, wl.scale, q_dtype, kv_dtype,
                        wl.k_scale, wl.v_scale)
    np.testing.assert_allclose(got, _brute(wl), rtol=1e-12, atol=1e-13)


# ---------------------------------------------------------------- invariants and special cases

def _tiny(seed=3, lens=(1, 17, 33, 100), G=4, D=64, kv="bf16"):
    spec = Spec("t", len(lens), 2 * G, 2, D, "bf16", kv, ("list", tuple(lens)),
                pool=("times", 2), seed=seed)
    wl = workloads.make(spec)
    k, v = oracle.kv_append(wl.k_cache, wl.v_cache, wl.k_new, wl.v_new, wl.slot_mapping)
    return wl, k, v


def test_softmax_weights_sum_to_one():
    wl, k, v = _tiny()
    _, w = oracle.decode(wl.q, k, v, wl.block_tables, wl.context_lens, wl.scale, "bf16", "bf16",
                         return_weights=True)
    for (b, kvh), ww in w.items():
        assert ww.shape[1] == wl.context_lens[b]
        np.testing.assert_allclose(ww.sum(axis=1), 1.0, rtol=0, atol=1e-12)
        assert (ww >= 0).all()


def test_length_one_returns_v_exactly():
    wl, k, v = _tiny(lens=(1, 1, 1))
    out = oracle.decode(wl.q, k, v, wl.block_tables, wl.context_lens, wl.scale, "bf16", "bf16")
    for b in range(3):
        for h in range(wl.spec.num_q_heads):
            kvh = h // wl.group
            expect = torch_decode(wl.v_new[b, kvh], "bf16")
            assert np.array_equal(out[b, h], expect)


def test_length_zero_gives_zeros():
    wl, k, v = _tiny(lens=(0, 5))
    out = oracle.decode(wl.q, k, v, wl.block_tables, wl.context_lens, wl.scale, "bf16", "bf16")
    assert np.array_equal(out[0], np.zeros_like(out[0]))
    assert np.abs(out[1]).sum() > 0


def test_gqa_equals_mha_with_repeated_kv_heads():
    wl, k, v = _tiny(G=4, D=16, lens=(3, 29, 50))
    out = oracle.decode(wl.q, k, v, wl.block_tables, wl.context_lens, wl.scale, "bf16", "bf16")
    k_rep = np.repeat(k, wl.group, axis=1)
    v_rep = np.repeat(v, wl.group, axis=1)
    out_mha = oracle.decode(wl.q, k_rep, v_rep, wl.block_tables, wl.context_lens, wl.scale,
                            "bf16", "bf16")
    np.testing.assert_allclose(out, out_mha, rtol=1e-13, atol=1e-15)   # BLAS order may differ
    # and the head mapping is contiguous groups: head h reads kv head h // G
    shuffled = k.copy()
    shuffled[:, [0, 1]] = shuffled[:, [1, 0]]
    out_sw = oracle.decode(wl.q, shuffled, v, wl.block_tables, wl.context_lens, wl.scale,
                           "bf16", "bf16")
    assert not np.allclose(out_sw, out)


@pytest.mark.parametrize("t_star", [0, 15, 16, 31, 63, 99])
def test_needle_returns_v_of_needle(t_star):
    """q = e0 for every head, every K row zero except k[t*] = c e0 with c*scale >= 50."""
    L = 100
    wl, k, v = _tiny(lens=(L,), G=4, D=64)
    one = round_bits(np.array([1.0]), "bf16")[0]
    c = round_bits(np.array([576.0]), "bf16")[0]        # 576 / 8 = 72 >= 50
    q = np.zeros_like(wl.q)
    q[:, :, 0] = one
    k[:] = 0
    blk = int(wl.block_tables[0, t_star // BLOCK])
    k[blk, :, t_star % BLOCK, 0] = c
    out = oracle.decode(q, k, v, wl.block_tables, wl.context_lens, wl.scale, "bf16", "bf16")
    for h in range(wl.spec.num_q_heads):
        expect = torch_decode(v[blk, h // wl.group, :, t_star % BLOCK], "bf16")
        np.testing.assert_allclose(out[0, h], expect, rtol=1e-14, atol=1e-20)


def test_two_token_closed_form():
    wl, k, v = _tiny(lens=(2,), G=1, D=16)
    out = oracle.decode(wl.q, k, v, wl.block_tables, wl.context_lens, wl.scale, "bf16", "bf16")
    blk = int(wl.block_tables[0, 0])
    for h in range(wl.spec.num_q_heads):
        q = torch_decode(wl.q[0, h], "bf16")
        k0 = torch_decode(k[blk, h, 0], "bf16")
        k1 = torch_decode(k[blk, h, 1], "bf16")
        v0 = torch_decode(v[blk, h, :, 0], "bf16")
        v1 = torch_decode(v[blk, h, :, 1], "bf16")
        delta = float(wl.scale) * (q @ k1 - q @ k0)
        expect = (v0 + math.exp(delta) * v1) / (1 + math.exp(delta))
        np.testing.assert_allclose(out[0, h], expect, rtol=1e-13, atol=1e-15)


@pytest.mark.parametrize("P", [16, 32, 48, 512])
def test_split_lse_merge_equals_single_pass(P):
    wl, k, v = _tiny(lens=(1, 17, 33, 100, 700), G=2, D=16)
    args = (wl.q, k, v, wl.block_tables, wl.context_lens, wl.scale, "bf16", "bf16")
    np.testing.assert_allclose(oracle.decode_split(*args, P), oracle.decode(*args),
                               rtol=1e-12, atol=1e-14)


def test_split_lse_merge_fp8():
    spec = workloads.SPECS["tiny_b4_h8kv2_d64_bf16"].replace(kv_dtype="fp8_e4m3",
                                                             lengths=("list", (1, 40, 300, 513)))
    wl = workloads.make(spec)
    k, v = oracle.kv_append(wl.k_cache, wl.v_cache, wl.k_new, wl.v_new, wl.slot_mapping)
    args = (wl.q, k, v, wl.block_tables, wl.context_lens, wl.scale, "bf16", "fp8_e4m3")
    np.testing.assert_allclose(
        oracle.decode_split(*args, 64, k_scale=wl.k_scale, v_scale=wl.v_scale),
        oracle.decode(*args, k_scale=wl.k_scale, v_scale=wl.v_scale), rtol=1e-12, atol=1e-14)


# ---------------------------------------------------------------- append

def test_append_writes_exactly_the_slots():
    wl = workloads.make(Spec("a", 5, 4, 2, 16, "bf16", "bf16", ("list", (1, 16, 17, 32, 50)),
                             pool=("times", 2), seed=8))
    slots = wl.slot_mapping.copy()
    slots[2] = -1                                      # a padding token: skipped
    k, v = oracle.kv_append(wl.k_cache, wl.v_cache, wl.k_new, wl.v_new, slots)
    NB, Hkv, _, D = wl.k_cache.shape
    written_k = np.zeros(k.size, dtype=bool)
    written_v = np.zeros(v.size, dtype=bool)
    kf, vf = k.reshape(-1), v.reshape(-1)
    for i, s in enumerate(slots):
        if s < 0:
            continue
        blk, off = int(s) // BLOCK, int(s) % BLOCK
        for h in range(Hkv):
            for d in range(D):
                a = ((blk * Hkv + h) * BLOCK + off) * D + d
                assert kf[a] == wl.k_new[i, h, d]
                written_k[a] = True
                a = ((blk * Hkv + h) * D + d) * BLOCK + off
                assert vf[a] == wl.v_new[i, h, d]
                written_v[a] = True
    assert np.array_equal(kf[~written_k], wl.k_cache.reshape(-1)[~written_k])
    assert np.array_equal(vf[~written_v], wl.v_cache.reshape(-1)[~written_v])
    assert written_k.sum() == 4 * Hkv * D
    # the skipped token's slot still holds the poison it had before
    s2 = wl.slot_mapping[2]
    assert np.isnan(torch_decode(k[s2 // BLOCK, :, s2 % BLOCK], "bf16")).all()


def test_append_duplicate_slot_last_wins():
    wl = workloads.make(Spec("d", 2, 2, 1, 8, "bf16", "bf16", ("list", (3, 3)),
                             pool=("fixed", 4), seed=9))
    slots = np.array([5, 5], dtype=np.int64)
    k, v = oracle.kv_append(wl.k_cache, wl.v_cache, wl.k_new, wl.v_new, slots)
    assert np.array_equal(k[0, :, 5], wl.k_new[1]) and np.array_equal(v[0, :, :, 5], wl.v_new[1])
