"""Plant plausible mistakes in the oracle (on the CPU) and check that its pins catch each one."""

import os

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


# ---- fp8 quantisation: planted mistakes in the encoder and in the quantising append.

import oracle as O  # noqa: E402
import oracle.formats as F  # noqa: E402
import test_oracle_quant as Q  # noqa: E402

_orig_encode, _orig_quant = F.e4m3fn_encode, pa.kv_append_quant


def _encode_with(rounder):
    def enc(y):
        y = np.asarray(y, dtype=np.float64)
        nan, neg = np.isnan(y), np.signbit(y)
        a = np.minimum(np.abs(np.where(nan, 0.0, y)), 448.0)
        _, ex = np.frexp(a)
        q = np.exp2(np.maximum(ex - 1.0, -6.0) - 3.0)
        r = rounder(a / q) * q
        codes = np.vectorize(lambda v: F._E4M3FN_CODE_OF[float(v)], otypes=[np.uint8])(r)
        codes = np.where(neg, codes | 0x80, codes).astype(np.uint8)
        return np.where(nan, np.uint8(0x7F), codes).astype(np.uint8)
    return enc


def quant_scale_without_448(k_cache, v_cache, k_scale, v_scale, k_new, v_new, src_dtype, slots,
                            policy):
    k, v, ks, vs = _orig_quant(k_cache, v_cache, k_scale, v_scale, k_new, v_new, src_dtype, slots,
                               policy)
    if policy == O.SCALE_FIRST_TOKEN:             # mistake: scale = amax (codes then tiny)
        x = O.to_f64(k_new, src_dtype)
        for i, s in enumerate(slots):
            if s >= 0 and s % BLOCK == 0:
                for h in range(k.shape[1]):
                    ks[s // BLOCK, h] = np.float32(np.abs(x[i, h]).max() or 1.0)
                    k[s // BLOCK, h, s % BLOCK] = F.e4m3fn_encode(x[i, h] / ks[s // BLOCK, h])
    return k, v, ks, vs


def quant_v_scale_from_k(k_cache, v_cache, k_scale, v_scale, k_new, v_new, src_dtype, slots,
                         policy):
    return _orig_quant(k_cache, v_cache, k_scale, v_scale, k_new, k_new, src_dtype, slots, policy)


QUANT_MUTATIONS = {
    "encode: rounds toward zero": ("encode", _encode_with(np.trunc)),
    "encode: ties away from zero": ("encode", _encode_with(lambda m: np.floor(m + 0.5))),
    "quant append: scale is amax, not amax / 448": ("quant", quant_scale_without_448),
    "quant append: V quantised from K": ("quant", quant_v_scale_from_k),
}

QUANT_PINS = [
    Q.test_encode_matches_torch_on_every_bf16_value_in_range,
    Q.test_encode_matches_torch_on_random_fp32_and_midpoints,
    Q.test_ties_saturation_and_special_values,
    Q.test_first_token_sets_the_scale_and_its_largest_element_encodes_to_448,
    Q.test_keep_policy_uses_the_stored_scale_and_saturates,
]


@pytest.mark.parametrize("name", list(QUANT_MUTATIONS))
def test_quant_pins_catch_planted_mistake(name, monkeypatch):
    kind, fn = QUANT_MUTATIONS[name]
    if kind == "encode":
        for mod in (F, pa, O):
            monkeypatch.setattr(mod, "e4m3fn_encode", fn)
    else:
        for mod in (pa, O):
            monkeypatch.setattr(mod, "kv_append_quant", fn)
    caught = 0
    for pin in QUANT_PINS:
        try:
            pin()
        except AssertionError:
            caught += 1
    assert caught >= 1, f"no pin caught: {name}"


# ---- several query tokens per sequence: planted mistakes in the causal window and row mapping.
import test_oracle_multi as M  # noqa: E402

_orig_multi = pa.decode_multi


def _multi_with(n_of=lambda L, T, i: min(max(L - T + i + 1, 0), L),
                row_of=lambda qs, b, i: int(qs[b]) + i):
    def multi(q, query_start, k_cache, v_cache, block_tables, context_lens, scale, q_dtype,
              kv_dtype, k_scale=None, v_scale=None):
        qf = pa._q_f64(q, q_dtype)
        N, Hq, D = qf.shape
        Hkv = k_cache.shape[1]
        G = Hq // Hkv
        qs = np.asarray(query_start, dtype=np.int64)
        out = np.zeros((N, Hq, D))
        for b in range(len(qs) - 1):
            T, L = int(qs[b + 1] - qs[b]), int(context_lens[b])
            for kvh in range(Hkv):
                k, v = pa.gather(k_cache, v_cache, kv_dtype, block_tables[b], L, kvh, k_scale,
                                 v_scale)
                for i in range(T):
                    n = n_of(L, T, i)
                    o, _ = pa.attend(qf[row_of(qs, b, i), kvh * G:(kvh + 1) * G], k[:n], v[:n],
                                     float(np.float32(scale)))
                    out[int(qs[b]) + i, kvh * G:(kvh + 1) * G] = o
        return out
    return multi


MULTI_MUTATIONS = {
    "multi: a row misses its own token": _multi_with(n_of=lambda L, T, i: max(L - T + i, 0)),
    "multi: mask aligned to the first key": _multi_with(n_of=lambda L, T, i: min(i + 1, L)),
    "multi: no causal mask": _multi_with(n_of=lambda L, T, i: L),
    "multi: rows of a sequence reversed":
        _multi_with(row_of=lambda qs, b, i: int(qs[b + 1]) - 1 - i),
}

MULTI_PINS = [
    lambda: M.test_multi_matches_masked_sdpa("bf16", "bf16", 3),
    M.test_each_row_is_the_single_query_decode_at_its_position,
    M.test_a_row_ignores_every_later_token,
    M.test_rows_before_the_context_are_zero_and_empty_sequences_have_no_rows,
]


@pytest.mark.parametrize("name", list(MULTI_MUTATIONS))
def test_multi_pins_catch_planted_mistake(name, monkeypatch):
    monkeypatch.setattr(pa, "decode_multi", MULTI_MUTATIONS[name])
    monkeypatch.setattr(M.oracle, "decode_multi", MULTI_MUTATIONS[name])
    caught = 0
    for pin in MULTI_PINS:
        try:
            pin()
        except AssertionError:
            caught += 1
    assert caught >= 1, f"no pin caught: {name}"


def test_multi_unmutated_copy_passes(monkeypatch):
    monkeypatch.setattr(M.oracle, "decode_multi", _multi_with())
    for pin in MULTI_PINS:
        pin()


# ---- block sharing: planted mistakes in the copy and in the reference-count model.
import oracle.blocks as OB  # noqa: E402
import test_oracle_blocks as TB  # noqa: E402

_orig_copy = OB.copy_blocks


def copy_without_v(k_cache, v_cache, k_scale, v_scale, pairs):
    k, _, ks, vs = _orig_copy(k_cache, v_cache, k_scale, v_scale, pairs)
    return k, v_cache.copy(), ks, vs


def copy_without_scales(k_cache, v_cache, k_scale, v_scale, pairs):
    k, v, _, _ = _orig_copy(k_cache, v_cache, k_scale, v_scale, pairs)
    return k, v, None if k_scale is None else k_scale.copy(), None if v_scale is None else v_scale.copy()


def copy_reversed(k_cache, v_cache, k_scale, v_scale, pairs):
    return _orig_copy(k_cache, v_cache, k_scale, v_scale,
                      [(d, s) for s, d in np.asarray(pairs).reshape(-1, 2)])


class WriteKeepsOldReference(OB.BlockPoolModel):
    def write(self, block, new_block):
        if self.ref[block] == 1:
            assert new_block == block
            return False
        self.ref[new_block] = 1                        # mistake: the shared block keeps its count
        return True


class ReleaseIgnoresCounts(OB.BlockPoolModel):
    def release(self, ids):
        for i in ids:                                  # mistake: any release frees the block
            assert self.ref[int(i)] >= 1
            self.ref[int(i)] = 0


BLOCK_MUTATIONS = {
    "copy: V not copied": ("copy_blocks", copy_without_v),
    "copy: fp8 scales not copied": ("copy_blocks", copy_without_scales),
    "copy: source and target swapped": ("copy_blocks", copy_reversed),
    "model: copy-on-write keeps the old reference": ("BlockPoolModel", WriteKeepsOldReference),
    "model: release frees a still-shared block": ("BlockPoolModel", ReleaseIgnoresCounts),
}

BLOCK_PINS = [
    lambda: TB.test_copy_matches_flat_address_loops(True),
    lambda: TB.test_decode_through_the_copies_is_unchanged("bf16"),
    TB.test_parallel_sampling_fork_and_copy_on_write,
    lambda: TB.test_lifecycle_of_the_100_token_example(
        os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")),
    TB.test_model_refuses_what_the_pages_rule_out,
]


@pytest.mark.parametrize("name", list(BLOCK_MUTATIONS))
def test_block_pins_catch_planted_mistake(name, monkeypatch):
    attr, fn = BLOCK_MUTATIONS[name]
    monkeypatch.setattr(OB, attr, fn)
    monkeypatch.setattr(TB.oracle, attr, fn)
    caught = 0
    for pin in BLOCK_PINS:
        try:
            pin()
        except (AssertionError, pytest.fail.Exception):   # a refusal that did not happen
            caught += 1
    assert caught >= 1, f"no pin caught: {name}"


def test_block_pins_pass_unmutated():
    for pin in BLOCK_PINS:
        pin()
