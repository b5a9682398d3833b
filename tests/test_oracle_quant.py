"""Pins for the oracle's fp8 quantisation (e4m3fn encoding and the quantising append), each
against something other than the oracle itself: torch's float8_e4m3fn conversion, the format's
own round trip, hand-derived ties and saturation cases, and the scale reading."""

import numpy as np
import torch

import oracle
from oracle.formats import E4M3FN_TABLE


def _torch_codes(y32: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(y32, dtype=np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_encode_matches_torch_on_every_bf16_value_in_range():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    x = oracle.bf16_to_f64(bits).astype(np.float32)
    keep = np.isfinite(x) & (np.abs(x) <= 448)
    y = x[keep]
    assert np.array_equal(oracle.e4m3fn_encode(y), _torch_codes(y))


def test_encode_matches_torch_on_random_fp32_and_midpoints():
    rng = np.random.default_rng(5)
    y = (rng.standard_normal(200_000) * np.exp2(rng.integers(-12, 9, 200_000))).astype(np.float32)
    y = np.clip(y, -448, 448)
    finite = E4M3FN_TABLE[np.isfinite(E4M3FN_TABLE)]
    grid = np.unique(finite)
    mids = ((grid[1:] + grid[:-1]) / 2).astype(np.float32)      # exact halfway points
    y = np.concatenate([y, mids, -mids])
    assert np.array_equal(oracle.e4m3fn_encode(y), _torch_codes(y))


def test_round_trip_of_every_finite_code():
    codes = np.array([c for c in range(256) if np.isfinite(E4M3FN_TABLE[c])], dtype=np.uint8)
    values = E4M3FN_TABLE[codes].astype(np.float32)
    assert np.array_equal(oracle.e4m3fn_encode(values), codes)


def test_ties_saturation_and_special_values():
    cases = [
        (1.0625, 0x38),      # halfway between 1 (m=0) and 1.125 (m=1): even -> 1
        (1.1875, 0x3A),      # halfway between 1.125 (m=1) and 1.25 (m=2): even -> 1.25
        (432.0, 0x7E),       # halfway between 416 and 448: even mantissa is 448's
        (500.0, 0x7E), (1e30, 0x7E), (float("inf"), 0x7E), (-1e30, 0xFE),  # saturate
        (2.0**-9, 0x01), (2.0**-10, 0x00), (3 * 2.0**-10, 0x02),           # subnormals
        (-0.0, 0x80), (-1e-6, 0x80), (0.0, 0x00), (float("nan"), 0x7F),
    ]
    y = np.array([c[0] for c in cases], dtype=np.float32)
    assert oracle.e4m3fn_encode(y).tolist() == [c[1] for c in cases]


def _setup(nb=4, hkv=2, d=8, seed=0):
    rng = np.random.default_rng(seed)
    k = rng.integers(0, 256, (nb, hkv, 16, d), dtype=np.uint8)
    v = rng.integers(0, 256, (nb, hkv, d, 16), dtype=np.uint8)
    ks = np.full((nb, hkv), 0.5, np.float32)
    vs = np.full((nb, hkv), 0.25, np.float32)
    return k, v, ks, vs


def _bf16_bits(x):
    return (torch.tensor(x, dtype=torch.float32).to(torch.bfloat16).view(torch.int16).numpy()
            .view(np.uint16))


def test_first_token_sets_the_scale_and_its_largest_element_encodes_to_448():
    k, v, ks, vs = _setup()
    rng = np.random.default_rng(1)
    xk = rng.standard_normal((2, 2, 8)) * 3
    xv = rng.standard_normal((2, 2, 8))
    kn, vn = _bf16_bits(xk), _bf16_bits(xv)
    slots = np.array([2 * 16 + 0, 2 * 16 + 5])       # block 2: offset 0, then offset 5
    k2, v2, ks2, vs2 = oracle.kv_append_quant(k, v, ks, vs, kn, vn, "bf16", slots,
                                              oracle.SCALE_FIRST_TOKEN)
    xk0 = oracle.bf16_to_f64(kn).astype(np.float32)
    for h in range(2):
        amax = np.abs(xk0[0, h]).max()
        assert ks2[2, h] == np.float32(amax) / np.float32(448)
        arg = np.abs(xk0[0, h]).argmax()
        assert k2[2, h, 0, arg] & 0x7F == 0x7E            # +-448
        # the token at offset 5 used the new scale of its block
        assert np.array_equal(k2[2, h, 5], oracle.e4m3fn_encode(xk0[1, h] / ks2[2, h]))
    # other blocks untouched, scales included
    for blk in (0, 1, 3):
        assert np.array_equal(k2[blk], k[blk]) and ks2[blk].tolist() == ks[blk].tolist()
    # dequantised rows stay within half an e4m3 step (2**-4 relative, 2**-10 absolute below the
    # normals) of the input saturated at 448 * scale
    sc = ks2[2][:, None].astype(np.float64)
    want = np.clip(xk0[1], -448 * sc, 448 * sc)
    deq = E4M3FN_TABLE[k2[2, :, 5]] * sc
    assert np.all(np.abs(deq - want) <= 2.0**-4 * np.abs(want) + sc * 2.0**-10)


def test_keep_policy_uses_the_stored_scale_and_saturates():
    k, v, ks, vs = _setup()
    xk = np.zeros((1, 2, 8)); xk[0, 0, 3] = 1000.0; xk[0, 1, 1] = -0.3
    xv = np.ones((1, 2, 8))
    kn, vn = _bf16_bits(xk), _bf16_bits(xv)
    k2, v2, ks2, vs2 = oracle.kv_append_quant(k, v, ks, vs, kn, vn, "bf16", np.array([16]),
                                              oracle.SCALE_KEEP)
    assert ks2.tolist() == ks.tolist() and vs2.tolist() == vs.tolist()
    assert k2[1, 0, 0, 3] == 0x7E                         # 1000 / 0.5 saturates at 448
    assert k2[1, 1, 0, 1] == oracle.e4m3fn_encode(np.float32(-0.30078125) / np.float32(0.5))
    assert np.all(v2[1, :, :, 0] == oracle.e4m3fn_encode(np.float32(1) / np.float32(0.25)))


def test_zero_token_gets_scale_one_and_negative_slots_are_skipped():
    k, v, ks, vs = _setup()
    kn = _bf16_bits(np.zeros((2, 2, 8)))
    k2, v2, ks2, vs2 = oracle.kv_append_quant(k, v, ks, vs, kn, kn, "bf16", np.array([48, -1]),
                                              oracle.SCALE_FIRST_TOKEN)
    assert ks2[3].tolist() == [1.0, 1.0] and np.all(k2[3, :, 0] == 0)
    assert np.array_equal(k2[:3], k[:3])
