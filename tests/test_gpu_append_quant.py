"""pa_kv_append_quant against the oracle: fp8 e4m3fn codes and per-(block, KV head) scales
bit-exact, then decode over the caches it wrote within the attention tolerance.

The fp8 cache keeps value = code * scale per block and KV head (babushkai.com "GPU推論の内部構造",
KV-cache and quantisation sections).  The oracle encodes with its own e4m3fn table search and
takes the scale policy's reading step by step; the library converts with the hardware's fp8
conversion, so every 16-bit source value is run through both."""

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_31_amd as pa
import workloads
from gpu_util import assert_close, dev_bits, host_bits
from workloads.generate import Spec

pytestmark = pytest.mark.gpu
BLOCK = 16
TORCH16 = {"bf16": torch.bfloat16, "f16": torch.float16}


def _bits16(x: np.ndarray, dtype: str) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(TORCH16[dtype])
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def _quant_both(k_cache, v_cache, k_scale, v_scale, k_new, v_new, src, slots, first,
                oracle_slots=None):
    """Run the library and the oracle on the same inputs; return both results."""
    kc, vc = dev_bits(k_cache, "fp8_e4m3"), dev_bits(v_cache, "fp8_e4m3")
    ks, vs = torch.from_numpy(k_scale.copy()).cuda(), torch.from_numpy(v_scale.copy()).cuda()
    pa.pa_kv_append_quant(dev_bits(k_new, src), dev_bits(v_new, src),
                          torch.from_numpy(np.asarray(slots, dtype=np.int64)).cuda(), kc, vc, ks,
                          vs, first_token_scale=first)
    torch.cuda.synchronize()
    got = (host_bits(kc), host_bits(vc), ks.cpu().numpy(), vs.cpu().numpy())
    policy = oracle.SCALE_FIRST_TOKEN if first else oracle.SCALE_KEEP
    ref = oracle.kv_append_quant(k_cache, v_cache, k_scale, v_scale, k_new, v_new, src,
                                 slots if oracle_slots is None else oracle_slots, policy)
    return got, ref


def _assert_same(got, ref, label):
    for name, g, r in zip(("k codes", "v codes", "k scales", "v scales"), got, ref):
        if g.dtype == np.float32:
            same = (g.view(np.uint32) == r.view(np.uint32)) | (np.isnan(g) & np.isnan(r))
        else:
            same = g == r
        bad = np.argwhere(~same)
        assert bad.size == 0, (f"{label}: {name} differ at {len(bad)} places, first "
                               f"{tuple(bad[0])}: {g[tuple(bad[0])]} vs {r[tuple(bad[0])]}")


@pytest.mark.parametrize("src", ["bf16", "f16"])
@pytest.mark.parametrize("scales", ["one", "random"])
def test_every_16bit_value(src, scales):
    """All 65536 source bit patterns (NaNs, infinities, subnormals, both zeros) in K and, in
    another order, in V; scale 1 checks the encoder alone, random scales its fp32 division."""
    rng = np.random.default_rng(81)
    Hkv, D, T, NB = 2, 128, 256, 24
    k_new = np.arange(65536, dtype=np.uint32).astype(np.uint16).reshape(T, Hkv, D)
    v_new = rng.permutation(65536).astype(np.uint16).reshape(T, Hkv, D)
    slots = rng.permutation(NB * BLOCK)[:T].astype(np.int64)
    k_cache = rng.integers(0, 256, (NB, Hkv, BLOCK, D), dtype=np.uint8)
    v_cache = rng.integers(0, 256, (NB, Hkv, D, BLOCK), dtype=np.uint8)
    if scales == "one":
        k_scale = np.ones((NB, Hkv), np.float32)
        v_scale = np.ones((NB, Hkv), np.float32)
    else:
        k_scale = (2.0 ** rng.uniform(-12, 12, (NB, Hkv))).astype(np.float32)
        v_scale = (2.0 ** rng.uniform(-12, 12, (NB, Hkv))).astype(np.float32)
    got, ref = _quant_both(k_cache, v_cache, k_scale, v_scale, k_new, v_new, src, slots, False)
    _assert_same(got, ref, f"{src} {scales}")


def _prefill_runs(rng, NB, runs):
    """Slots of several sequences' runs of tokens: (first block, start offset, tokens) each,
    over distinct blocks, in order."""
    slots = []
    for blk, off, n in runs:
        assert blk + (off + n - 1) // BLOCK < NB
        slots.extend(blk * BLOCK + off + np.arange(n))
    return np.asarray(slots, dtype=np.int64)


@pytest.mark.parametrize("src", ["bf16", "f16"])
def test_first_token_sets_the_scale(src):
    """Prefill-like runs that start at offset 0 of a block or in the middle of one: a token at
    offset 0 sets its block's scale from its own amax, later tokens use that scale and saturate
    when they are larger; NaN elements (quiet and signalling) do not count towards the amax, an
    all-zero token gives scale 1; skipped slots (-1) leave everything as it was."""
    rng = np.random.default_rng(82)
    Hkv, D, NB = 4, 128, 40
    runs = [(0, 0, 40), (3, 5, 27), (6, 0, 16), (7, 0, 1), (9, 15, 2), (12, 0, 100)]
    slots = _prefill_runs(rng, NB, runs)
    T = len(slots)
    mag = 2.0 ** rng.uniform(-6, 6, (T, Hkv, 1))                # tokens of very different size
    k = (rng.standard_normal((T, Hkv, D)) * mag).astype(np.float32)
    v = (rng.standard_normal((T, Hkv, D)) * mag * 0.5).astype(np.float32)
    k[40 + 27] = 0.0                                             # all-zero first token of block 6
    k_new, v_new = _bits16(k, src), _bits16(v, src)
    qnan, snan = (0x7FC0, 0x7F81) if src == "bf16" else (0x7E00, 0x7C01)
    k_new[0, 1, 5] = qnan                                        # NaNs inside first tokens
    v_new[0, 2, 7] = snan | 0x8000
    k_new[40 + 27 + 16, 0, :] = snan                             # block 7: all NaN -> scale 1
    k_new[3, 0, 9] = qnan                                        # NaN in a later token
    inf = 0x7F80 if src == "bf16" else 0x7C00
    v_new[5, 3, 0] = inf                                         # inf in a later token: saturates
    slots[[10, 50]] = -1
    k_cache = rng.integers(0, 256, (NB, Hkv, BLOCK, D), dtype=np.uint8)
    v_cache = rng.integers(0, 256, (NB, Hkv, D, BLOCK), dtype=np.uint8)
    k_scale = rng.uniform(0.01, 1.0, (NB, Hkv)).astype(np.float32)
    v_scale = rng.uniform(0.01, 1.0, (NB, Hkv)).astype(np.float32)
    for first in (True, False):
        got, ref = _quant_both(k_cache, v_cache, k_scale, v_scale, k_new, v_new, src, slots,
                               first)
        _assert_same(got, ref, f"{src} first={first}")
    # the reading itself, spelled out for three blocks: block 0 head 1 holds a NaN in its first
    # token, block 6 head 0 an all-zero first token, block 7 head 0 an all-NaN one
    got, _ = _quant_both(k_cache, v_cache, k_scale, v_scale, k_new, v_new, src, slots, True)
    kx = oracle.to_f64(k_new[0, 1], src).astype(np.float32)
    assert got[2][0, 1] == np.float32(np.nanmax(np.abs(kx)) / np.float32(448))
    assert got[2][6, 0] == 1.0 and got[2][7, 0] == 1.0


def test_slots_outside_the_pool_are_skipped():
    rng = np.random.default_rng(83)
    Hkv, D, NB = 2, 64, 8
    slots = np.array([0, 1, NB * BLOCK, 17, NB * BLOCK + 16, 32], dtype=np.int64)
    T = len(slots)
    k_new = _bits16(rng.standard_normal((T, Hkv, D)), "bf16")
    v_new = _bits16(rng.standard_normal((T, Hkv, D)), "bf16")
    k_cache = rng.integers(0, 256, (NB, Hkv, BLOCK, D), dtype=np.uint8)
    v_cache = rng.integers(0, 256, (NB, Hkv, D, BLOCK), dtype=np.uint8)
    ones = np.ones((NB, Hkv), np.float32)
    oracle_slots = np.where(slots >= NB * BLOCK, -1, slots)
    got, ref = _quant_both(k_cache, v_cache, ones, ones, k_new, v_new, "bf16", slots, True,
                           oracle_slots=oracle_slots)
    _assert_same(got, ref, "outside the pool")


@pytest.mark.parametrize("src", ["bf16", "f16"])
@pytest.mark.parametrize("first", [True, False])
def test_decode_after_quantised_append(src, first):
    """One decode step of an fp8 serving batch: the new tokens arrive in 16 bits, are quantised
    into the cache, and the decode reads them back with the scales the append left."""
    spec = Spec("quant_decode", 12, 16, 4, 128, "bf16", "fp8_e4m3",
                ("list", (1, 16, 17, 32, 33, 100, 250, 257, 700, 1024, 1025, 1601)),
                seed=84)
    wl = workloads.make(spec)
    rng = np.random.default_rng(85)
    B, Hkv, D = spec.batch, spec.num_kv_heads, spec.head_dim
    k_new = _bits16(rng.standard_normal((B, Hkv, D)) * 1.5, src)
    v_new = _bits16(rng.standard_normal((B, Hkv, D)), src)
    (kc, vc, ks, vs), (rk, rv, rks, rvs) = _quant_both(
        wl.k_cache, wl.v_cache, wl.k_scale, wl.v_scale, k_new, v_new, src, wl.slot_mapping,
        first)
    _assert_same((kc, vc, ks, vs), (rk, rv, rks, rvs), f"append {src} first={first}")
    q = dev_bits(wl.q, spec.q_dtype)
    out = torch.empty_like(q)
    pa.pa_decode(q, dev_bits(kc, "fp8_e4m3"), dev_bits(vc, "fp8_e4m3"),
                 torch.from_numpy(wl.block_tables).cuda(), torch.from_numpy(wl.context_lens).cuda(),
                 float(wl.scale), out, k_scale=torch.from_numpy(ks).cuda(),
                 v_scale=torch.from_numpy(vs).cuda(), max_context_len=wl.max_context_len)
    torch.cuda.synchronize()
    ref = oracle.decode(wl.q, rk, rv, wl.block_tables, wl.context_lens, wl.scale, spec.q_dtype,
                        spec.kv_dtype, rks, rvs)
    # contexts of 1 and 16 tokens: outputs of one or a few rows (counted rounding-limited relief)
    assert_close(host_bits(out), ref, spec.q_dtype, f"decode {src} first={first}", relief=True)
