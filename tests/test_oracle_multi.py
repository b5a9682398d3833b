"""Pins of oracle.decode_multi: several query tokens per sequence, causal over the paged cache.

Each query token attends to the cached tokens up to and including its own position, the new
tokens being the last T of the context (the verification pass of speculative decoding, youngju.dev
guide, speculative-decoding figure; chunked prefill, magi page, "Prefill-Decode 分離").  The pins
check it against things other than itself: torch's scaled_dot_product_attention with an explicit
bottom-right causal mask on contiguous per-sequence arrays built by the test-side scatter; the
single-query decode (itself pinned) with the context cut at each row's position; the invariance
of a row to every token after its position; and the degenerate shapes."""

import numpy as np
import pytest
import torch

import oracle
from cpu_cases import Case, round_bits


def _queries(rng, case, T):
    qs = np.concatenate([[0], np.cumsum(T)]).astype(np.int32)
    bits = round_bits(rng.standard_normal((int(qs[-1]), case.Hq, case.D)), case.q_dtype)
    return qs, bits


def _sdpa_multi(case, qs, q_bits):
    """torch SDPA per (sequence, head) with mask[i][t] = t <= L - T + i (float64)."""
    from cpu_cases import torch_decode
    qf = torch_decode(q_bits, case.q_dtype)
    out = np.zeros(qf.shape)
    for b in range(case.B):
        T, L = int(qs[b + 1] - qs[b]), int(case.lens[b])
        if T == 0 or L == 0:
            continue
        mask = np.tril(np.ones((T, L), dtype=bool), k=L - T)
        live = mask.any(axis=1)                       # rows before the context: no keys
        for h in range(case.Hq):
            kvh = h // case.G
            q = torch.from_numpy(qf[qs[b]:qs[b + 1], h]).view(1, 1, T, case.D)
            k = torch.from_numpy(case.K[b][kvh]).view(1, 1, L, case.D)
            v = torch.from_numpy(case.V[b][kvh]).view(1, 1, L, case.D)
            o = torch.nn.functional.scaled_dot_product_attention(
                q, k, v, attn_mask=torch.from_numpy(mask), scale=float(case.scale))
            o = o.view(T, case.D).numpy()
            out[qs[b]:qs[b + 1], h] = np.where(live[:, None], o, 0.0)
    return out


def _multi(case, qs, q_bits):
    a = case.oracle_args()
    a.pop("q")
    return oracle.decode_multi(q_bits, qs, **a)


@pytest.mark.parametrize("kv_dtype,q_dtype,G", [("bf16", "bf16", 1), ("bf16", "bf16", 3),
                                                ("f16", "f16", 2), ("fp8_e4m3", "bf16", 4)])
def test_multi_matches_masked_sdpa(kv_dtype, q_dtype, G):
    rng = np.random.default_rng(30 + G)
    lens = [1, 4, 17, 33, 40, 70, 16]
    T = [1, 4, 5, 16, 33, 3, 0]
    case = Case(rng, lens, Hkv=2, G=G, D=16, kv_dtype=kv_dtype, q_dtype=q_dtype)
    qs, q_bits = _queries(rng, case, T)
    np.testing.assert_allclose(_multi(case, qs, q_bits), _sdpa_multi(case, qs, q_bits),
                               rtol=1e-12, atol=1e-13)


def test_each_row_is_the_single_query_decode_at_its_position():
    """Row i of sequence b equals decode() of that query over the first L - T + i + 1 tokens."""
    rng = np.random.default_rng(41)
    lens, T = [20, 49, 64, 100], [3, 8, 16, 7]
    case = Case(rng, lens, Hkv=2, G=2, D=8)
    qs, q_bits = _queries(rng, case, T)
    got = _multi(case, qs, q_bits)
    a = case.oracle_args()
    for b in range(case.B):
        for i in range(T[b]):
            a["q"] = q_bits[qs[b] + i][None]
            a["block_tables"] = case.tables[b:b + 1]
            a["context_lens"] = np.array([lens[b] - T[b] + i + 1], dtype=np.int32)
            ref = oracle.decode(**a)[0]
            np.testing.assert_array_equal(got[qs[b] + i], ref)


def test_a_row_ignores_every_later_token():
    """Overwriting the K/V of positions after row i changes no row up to i and does change the
    rows after it."""
    rng = np.random.default_rng(42)
    lens, T = [50], [10]
    case = Case(rng, lens, Hkv=1, G=2, D=8)
    qs, q_bits = _queries(rng, case, T)
    base = _multi(case, qs, q_bits)
    p_cut = 44                                  # rows 0..4 sit at positions 40..44
    for t in range(p_cut + 1, 50):
        blk, off = int(case.tables[0, t // 16]), t % 16
        case.k_cache[blk, 0, off] = round_bits(rng.standard_normal(8) * 3, "bf16")
        case.v_cache[blk, 0, :, off] = round_bits(rng.standard_normal(8) * 3, "bf16")
    after = _multi(case, qs, q_bits)
    np.testing.assert_array_equal(after[:5], base[:5])
    assert np.all(np.abs(after[5:] - base[5:]).max(axis=(1, 2)) > 0)


def test_last_row_is_the_full_context_and_one_token_rows_are_decode():
    rng = np.random.default_rng(43)
    lens, T = [33, 5, 80], [1, 1, 1]
    case = Case(rng, lens, Hkv=2, G=3, D=16)
    qs, q_bits = _queries(rng, case, T)
    a = case.oracle_args()
    a["q"] = q_bits
    np.testing.assert_array_equal(_multi(case, qs, q_bits), oracle.decode(**a))


def test_rows_before_the_context_are_zero_and_empty_sequences_have_no_rows():
    rng = np.random.default_rng(44)
    lens, T = [3, 0, 20], [5, 2, 0]
    case = Case(rng, lens, Hkv=1, G=2, D=8)
    qs, q_bits = _queries(rng, case, T)
    got = _multi(case, qs, q_bits)
    assert np.all(got[0:2] == 0)                 # positions -2, -1 of a 3-token context
    assert np.all(got[2] != 0)                   # position 0 sees token 0: returns V[0]
    np.testing.assert_array_equal(got[2, 0], case.V[0][0][0])
    assert np.all(got[5:7] == 0)                 # a sequence with no cached tokens
    assert got.shape[0] == 7
