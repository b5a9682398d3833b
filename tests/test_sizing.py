"""The byte model's sizing helpers against the pages' worked examples (tests/golden)."""

import json
import os

import numpy as np

import workloads as W


def _g(golden_dir):
    return json.load(open(os.path.join(golden_dir, "pages_sizing.json")))


def test_kasblo_100_token_example(golden_dir):
    ex = _g(golden_dir)["kasblo_100_tokens"]
    m_tok = W.kv_bytes_per_token(ex["layers"], ex["kv_heads"], ex["head_dim"], ex["elem_bytes"])
    assert m_tok == ex["m_token"]
    assert W.m_block(m_tok, ex["block_size"]) == ex["m_block"]
    assert W.n_blocks(ex["tokens"], ex["block_size"]) == ex["n_blocks"]
    assert W.m_alloc(ex["tokens"], m_tok) == ex["capacity_tokens"] * m_tok
    assert W.m_waste(ex["tokens"], m_tok) == ex["waste_tokens"] * m_tok


def test_llama3_70b_bytes_per_token(golden_dir):
    ex = _g(golden_dir)["babushkai_llama3_70b"]
    m = W.kv_bytes_per_token(ex["layers"], ex["kv_heads"], ex["head_dim"], ex["elem_bytes"])
    assert m == ex["m_token"]
    assert round(m / 1024) == ex["printed_kb"]


def test_tail_waste_never_reaches_a_block(golden_dir):
    ex = _g(golden_dir)["tail_bound"]
    worst = max(W.m_waste(n, 1, ex["block_size"]) for n in range(1, 1000))
    assert worst == ex["max_waste_tokens"]


def test_decode_bytes_counts_each_part():
    lens = np.array([16, 17])
    # K+V: 33 tokens * 2 heads * 8 dims * 2 B * 2; q+out: 2*2 seqs*4 heads*8*2; tables: 3 blocks*4 + 2*4
    expect = 33 * 2 * 8 * 2 * 2 + 2 * 2 * 4 * 8 * 2 + 3 * 4 + 8
    assert W.decode_bytes(lens, 4, 2, 8, "bf16", "bf16") == expect
    # fp8 halves K/V and adds one fp32 scale per block and head for K and V
    expect8 = 33 * 2 * 8 * 1 * 2 + 3 * 2 * 4 * 2 + 2 * 2 * 4 * 8 * 2 + 3 * 4 + 8
    assert W.decode_bytes(lens, 4, 2, 8, "bf16", "fp8_e4m3") == expect8
    assert W.append_bytes(2, 2, 8, "bf16") == 2 * (2 * 32 * 2 + 8)


def test_multi_query_counts():
    """Visible keys counted one row at a time, and the multi-query bytes part by part."""
    lens, T = np.array([16, 17, 3]), np.array([4, 1, 5])
    brute = 0
    for L, t in zip(lens, T):
        for i in range(t):
            brute += sum(1 for key in range(L) if key <= L - t + i)
    assert W.visible_keys(lens, T) == brute == (13 + 14 + 15 + 16) + 17 + (0 + 0 + 1 + 2 + 3)
    assert W.multi_flops(lens, T, 4, 8) == 4 * 8 * 4 * brute
    # K+V once per sequence; q+out per row (10 rows); tables; query starts (B + 1)
    expect = 36 * 2 * 8 * 2 * 2 + 2 * 10 * 4 * 8 * 2 + (1 + 2 + 1) * 4 + 3 * 4 + 4 * 4
    assert W.multi_bytes(lens, T, 4, 2, 8, "bf16", "bf16") == expect
    # one query per sequence: the single-query decode's bytes plus the query start offsets
    assert (W.multi_bytes(lens, [1, 1, 1], 4, 2, 8, "bf16", "fp8_e4m3")
            == W.decode_bytes(lens, 4, 2, 8, "bf16", "fp8_e4m3") + 16)
