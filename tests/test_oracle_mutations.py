"""Plant plausible mistakes in the oracle (on the CPU) and check that its pins catch each one."""

import numpy as np
import pytest

import oracle.paged_attention as pa
import test_oracle as T

BLOCK = 16
_orig_gather, _orig_attend, _orig_append = pa.gather, pa.attend, pa.kv_append


def gather_v_token_major(k_cache, v_cache, kv_dtype, table_row, length, kvh, k_scale=None,
                         v_scale=None):
    # mistake: reads the V tile as if it were token-major like K
    k, _ = _orig_gather(k_cache, v_cache, kv_dtype, table_row, length, kvh, k_scale, v_scale)
    nb = -(-int(length) // BLOCK)
    ids = np.asarray(table_row[:nb], dtype=np.int64)
    D = k_cache.shape[-1]
    v = pa.to_f64(v_cache[ids, kvh].reshape(nb * BLOCK, D)[:length], kv_dtype)
    if kv_dtype == "fp8_e4m3":
        v = v * np.asarray(v_scale, dtype=np.float64)[ids[np.arange(length) // BLOCK], kvh][:, None]
    return k, v


def gather_drops_last_token(k_cache, v_cache, kv_dtype, table_row, length, kvh, k_scale=None,
                            v_scale=None):
    return _orig_gather(k_cache, v_cache, kv_dtype, table_row, max(int(length) - 1, 1), kvh,
                        k_scale, v_scale)


def gather_no_fp8_scale(k_cache, v_cache, kv_dtype, table_row, length, kvh, k_scale=None,
                        v_scale=None):
    if k_scale is not None:
        v_scale = np.ones_like(v_scale)
    return _orig_gather(k_cache, v_cache, kv_dtype, table_row, length, kvh, k_scale, v_scale)


def gather_ignores_table(k_cache, v_cache, kv_dtype, table_row, length, kvh, k_scale=None,
                         v_scale=None):
    nb = -(-int(length) // BLOCK)
    return _orig_gather(k_cache, v_cache, kv_dtype, np.sort(table_row[:nb]), length, kvh,
                        k_scale, v_scale)


def attend_no_scale(q_rows, k, v, scale):
    return _orig_attend(q_rows, k, v, 1.0)


def attend_wrong_axis(q_rows, k, v, scale):
    if k.shape[0] == 0:
        return _orig_attend(q_rows, k, v, scale)
    s = (q_rows @ k.T) * scale
    e = np.exp(s - s.max(axis=0, keepdims=True))
    w = e / e.sum(axis=0, keepdims=True)
    return w @ v, w


def append_v_token_major(k_cache, v_cache, k_new, v_new, slot_mapping):
    k, v = _orig_append(k_cache, v_cache, k_new, v_new, np.full_like(slot_mapping, -1))
    for i, s in enumerate(slot_mapping):
        if s < 0:
            continue
        blk, off = divmod(int(s), BLOCK)
        k[blk, :, off, :] = k_new[i]
        v.reshape(v.shape[0], v.shape[1], BLOCK, -1)[blk, :, off, :] = v_new[i]
    return k, v


MUTATIONS = {
    "gather: V read token-major": ("gather", gather_v_token_major),
    "gather: last token dropped": ("gather", gather_drops_last_token),
    "gather: fp8 V scale ignored": ("gather", gather_no_fp8_scale),
    "gather: block table order ignored": ("gather", gather_ignores_table),
    "attend: scale dropped": ("attend", attend_no_scale),
    "attend: softmax over queries": ("attend", attend_wrong_axis),
    "append: V written token-major": ("kv_append", append_v_token_major),
}

PINS = [
    lambda: T.test_decode_matches_sdpa_on_contiguous_arrays("bf16", "bf16", 3),
    lambda: T.test_decode_matches_sdpa_on_contiguous_arrays("fp8_e4m3", "bf16", 3),
    lambda: T.test_append_then_decode_matches_brute_force("bf16", "bf16", 3, 8),
    lambda: T.test_append_writes_exactly_the_slots(),
    lambda: T.test_two_token_closed_form(),
]


@pytest.mark.parametrize("name", list(MUTATIONS))
def test_pins_catch_planted_mistake(name, monkeypatch):
    attr, fn = MUTATIONS[name]
    monkeypatch.setattr(pa, attr, fn)
    monkeypatch.setattr(T.oracle, attr, fn)
    caught = 0
    for pin in PINS:
        try:
            pin()
        except AssertionError:
            caught += 1
    assert caught >= 1, f"no pin caught: {name}"


def test_unmutated_pins_pass():
    for pin in PINS:
        pin()
