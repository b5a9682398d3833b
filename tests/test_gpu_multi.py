"""pa_decode_multi against the oracle: several query tokens per sequence, causal over the paged
cache (speculative verification: youngju.dev guide, speculative-decoding figure; chunked
prefill: magi page, "Prefill-Decode 分離").

The cases cover draft lengths 1..8 with every group size the row tiling distinguishes (tiles
holding several tokens, one token, part of a token), prefill chunks of 512, sequences without
queries or with more queries than cached tokens (rows before the context are zero), fixed key
partitions from 32 tokens (many partitions merged) to the whole context, fp16, bf16 and fp8
caches, head_dim 64 and 128; rows that no sequence owns must be left as they were."""

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_31_amd as pa
import workloads
from gpu_util import assert_close, dev_bits, host_bits
from workloads.generate import Spec

pytestmark = pytest.mark.gpu
SENTINEL = {"bf16": 0x7FA5, "f16": 0x7E5A}   # NaN payloads no kernel writes


class Multi:
    """A multi-query problem: a seeded paged cache (every context token stored) plus query rows."""

    def __init__(self, q_dtype, kv_dtype, hkv, g, d, lens, T, seed, spare_rows=0):
        spec = Spec("multi", len(lens), hkv * g, hkv, d, q_dtype, kv_dtype, ("list", tuple(lens)),
                    pool=("times", 2), seed=seed)
        self.wl = wl = workloads.make(spec)
        self.spec = spec
        self.k, self.v = oracle.kv_append(wl.k_cache, wl.v_cache, wl.k_new, wl.v_new,
                                          wl.slot_mapping)
        self.T = np.asarray(T, dtype=np.int64)
        self.qs = np.concatenate([[0], np.cumsum(self.T)]).astype(np.int32)
        self.N = int(self.qs[-1]) + spare_rows
        rng = np.random.default_rng(seed + 1000)
        self.q = workloads.storage_bits(rng.standard_normal((self.N, hkv * g, d)), q_dtype)
        self.max_q = max(1, int(self.T.max(initial=0)))

    def run(self, partition_tokens=0, max_query_len=None, max_context_len=0):
        s, wl = self.spec, self.wl
        q = dev_bits(self.q, s.q_dtype)
        out = torch.full_like(q, 0).view(torch.int16).fill_(SENTINEL[s.q_dtype]).view(q.dtype)
        pa.pa_decode_multi(q, torch.from_numpy(self.qs).cuda(), dev_bits(self.k, s.kv_dtype),
                           dev_bits(self.v, s.kv_dtype), torch.from_numpy(wl.block_tables).cuda(),
                           torch.from_numpy(wl.context_lens).cuda(), float(wl.scale), out,
                           self.max_q if max_query_len is None else max_query_len,
                           k_scale=None if wl.k_scale is None else torch.from_numpy(wl.k_scale).cuda(),
                           v_scale=None if wl.v_scale is None else torch.from_numpy(wl.v_scale).cuda(),
                           max_context_len=max_context_len, partition_tokens=partition_tokens)
        torch.cuda.synchronize()
        return host_bits(out)

    def reference(self):
        s, wl = self.spec, self.wl
        return oracle.decode_multi(self.q[:self.qs[-1]], self.qs, self.k, self.v, wl.block_tables,
                                   wl.context_lens, wl.scale, s.q_dtype, s.kv_dtype, wl.k_scale,
                                   wl.v_scale)

    def check(self, got, label, ref=None, relief=False):
        n = int(self.qs[-1])
        ref = self.reference() if ref is None else ref
        assert_close(got[:n], ref, self.spec.q_dtype, label, relief=relief)
        assert np.all(got[n:] == SENTINEL[self.spec.q_dtype]), f"{label}: unowned rows written"


LENS = (1, 2, 5, 16, 17, 33, 64, 100, 257, 700, 1023, 2049)
# The small shapes put query rows at the very start of a context, where a row sees one to a few
# keys and its output is an average of that many N(0,1) values: bf16 cannot then always hold the
# result within 2e-3 + 2e-3 |ref|, so those comparisons allow the counted rounding-limited
# elements (see gpu_util.assert_close).  Full-size batches are compared without it.
SHORT_WINDOWS = True
DRAFT = (1, 2, 5, 4, 8, 3, 0, 8, 7, 4, 6, 5)       # 2 queries with a 1-token context; one empty

VERIFY = [
    # (q dtype, kv dtype, kv heads, group, head_dim)
    ("bf16", "bf16", 2, 8, 128),
    ("bf16", "bf16", 4, 1, 128),
    ("bf16", "bf16", 2, 4, 64),
    ("bf16", "bf16", 2, 3, 128),
    ("bf16", "bf16", 1, 16, 128),
    ("bf16", "bf16", 1, 32, 64),
    ("f16", "f16", 2, 8, 128),
    ("bf16", "fp8_e4m3", 2, 8, 128),
    ("f16", "fp8_e4m3", 2, 4, 64),
]


@pytest.mark.parametrize("case", VERIFY, ids=lambda c: f"{c[0]}-{c[1]}-kv{c[2]}g{c[3]}d{c[4]}")
@pytest.mark.parametrize("P", [0, 32, 48, 256])
def test_speculative_verification(case, P):
    qd, kvd, hkv, g, d = case
    m = Multi(qd, kvd, hkv, g, d, LENS, DRAFT, seed=90 + VERIFY.index(case), spare_rows=3)
    m.check(m.run(partition_tokens=P), f"verify {case} P{P}", relief=SHORT_WINDOWS)


@pytest.mark.parametrize("qd,kvd,g,P", [("bf16", "bf16", 4, 0), ("bf16", "bf16", 4, 512),
                                        ("f16", "f16", 1, 0), ("bf16", "fp8_e4m3", 8, 0),
                                        ("bf16", "bf16", 4, 80)])
def test_prefill_chunks_of_512(qd, kvd, g, P):
    """Chunks of 512 tokens: the first chunk of a prompt (the chunk is the whole context), later
    chunks of long prompts, and a short last chunk."""
    lens, T = (512, 1100, 2048, 1700), (512, 512, 512, 188)
    m = Multi(qd, kvd, 2, g, 128, lens, T, seed=100)
    m.check(m.run(partition_tokens=P), f"prefill g{g} P{P}", relief=SHORT_WINDOWS)


CHUNK = [
    # (q dtype, kv heads, group, head_dim, context lengths, new tokens): 128+ rows per head take
    # the LDS-staged path; lengths end inside blocks, so the last step holds unused slots
    ("bf16", 2, 1, 64, (200, 531, 130), (200, 131, 130)),
    ("f16", 2, 3, 128, (700, 77, 1025), (130, 77, 50)),
    ("bf16", 1, 8, 128, (40, 1000, 333), (40, 17, 300)),
    ("bf16", 2, 4, 64, (20, 600, 5), (64, 35, 32)),          # more queries than context
    ("f16", 2, 16, 128, (300, 45, 1000), (9, 3, 5)),         # a partial second row block
]


@pytest.mark.parametrize("case", CHUNK, ids=lambda c: f"{c[0]}-kv{c[1]}g{c[2]}d{c[3]}")
@pytest.mark.parametrize("fp8", [False, True], ids=["16bit", "fp8"])
def test_prefill_chunk_shapes(case, fp8):
    """The same shapes over a 16-bit cache and over an fp8 one (codes widened when staged,
    block scales applied per lane)."""
    qd, hkv, g, d, lens, T = case
    kv = "fp8_e4m3" if fp8 else qd
    m = Multi(qd, kv, hkv, g, d, lens, T, seed=110 + CHUNK.index(case), spare_rows=2)
    m.check(m.run(), f"chunk {case} {kv}", relief=SHORT_WINDOWS)


SPLIT = [
    # (q dtype, kv dtype, kv heads, group, head_dim, most draft tokens): heads of at most four
    # row tiles take the balanced split (every tile of a head in one wave, or two tiles in each
    # of two waves sharing a chunk)
    ("bf16", "fp8_e4m3", 2, 8, 128, 4),      # two full tiles over fp8 codes
    ("f16", "fp8_e4m3", 2, 4, 128, 8),
    ("bf16", "bf16", 2, 8, 128, 2),          # one tile of 16-bit K/V
    ("bf16", "bf16", 2, 8, 128, 4),          # two 16-bit tiles at head_dim 128: rolling loads
    ("f16", "f16", 2, 3, 128, 8),            # the same with a partial second tile
    ("f16", "f16", 4, 1, 128, 8),            # one tile, several tokens in it
    ("f16", "f16", 2, 16, 64, 2),            # two tiles at head_dim 64
    ("bf16", "bf16", 2, 3, 64, 8),           # a partial second tile
    ("bf16", "fp8_e4m3", 2, 8, 128, 8),      # four fp8 tiles: two waves of two tiles
    ("bf16", "bf16", 2, 8, 128, 8),          # four 16-bit tiles at head_dim 128
    ("f16", "f16", 2, 6, 128, 8),            # three 16-bit tiles, the last partial
    ("f16", "f16", 2, 8, 64, 6),             # three tiles at head_dim 64 (the fourth empty)
    ("bf16", "bf16", 2, 16, 64, 4),          # four tiles at head_dim 64
    ("f16", "fp8_e4m3", 2, 5, 128, 8),       # three fp8 tiles, the last partial
]


@pytest.mark.parametrize("case", SPLIT, ids=lambda c: f"{c[0]}-{c[1]}-kv{c[2]}g{c[3]}d{c[4]}t{c[5]}")
def test_balanced_split_shapes(case):
    """Ragged contexts of 1..2049 tokens cut into chunks of every alignment (pieces ending after
    an odd number of blocks, heads cut inside and across workgroups), sequences without rows or
    with more rows than cached tokens; rows no sequence owns stay untouched."""
    qd, kvd, hkv, g, d, tmax = case
    T = tuple(min(t, tmax) for t in DRAFT)
    m = Multi(qd, kvd, hkv, g, d, LENS, T, seed=120 + SPLIT.index(case), spare_rows=3)
    m.check(m.run(), f"split {case}", relief=SHORT_WINDOWS)


def _set_v(m, b, kvh, tokens, value):
    """Store `value` in every dimension of V for the given tokens of sequence b, KV head kvh."""
    bits = workloads.storage_bits(np.array([value]), m.spec.kv_dtype)[0]
    for t in tokens:
        blk = m.wl.block_tables[b, t // 16]
        m.v[blk, kvh, :, t % 16] = bits


def test_chunk_rows_with_long_windows():
    """bf16 prefill chunks whose rows see 189..1200 keys (no row in its first few keys): the
    strict bound, no relief."""
    m = Multi("bf16", "bf16", 2, 4, 128, (700, 1200), (512, 512), seed=109)
    m.check(m.run(), "long windows")


@pytest.mark.parametrize("value", [70000.0, 65280.0, -65280.0])
def test_chunk_large_v_values(value):
    """V elements of magnitude 65280 and 70144, far outside N(0,1), in every dimension of four
    tokens of one head: the products keep their precision at any magnitude.  Outputs near the
    large values are large, where the output format itself can miss the bound (relief)."""
    m = Multi("bf16", "bf16", 2, 4, 128, (1500, 900), (600, 300), seed=111)
    _set_v(m, 0, 1, (3, 700, 1201, 1499), value)
    got = m.run()
    assert np.isfinite(oracle.to_f64(got[:int(m.qs[-1])], "bf16")).all()
    m.check(got, f"large V {value}", relief=True)


SCALE_CASES = [
    # (q dtype, kv dtype, group, context lengths, new tokens, partition): the ping-pong chunk
    # shape (512 rows a head), the four-wave one (128), the balanced split (a few rows) and
    # fixed partitions, each with masked slots in the last steps
    ("bf16", "bf16", 4, (700, 1200), (512, 512), 0),
    ("bf16", "bf16", 4, (700, 333), (32, 32), 0),
    ("f16", "fp8_e4m3", 4, (700, 333), (32, 32), 0),
    ("bf16", "bf16", 8, LENS, DRAFT, 0),
    ("bf16", "fp8_e4m3", 8, LENS, DRAFT, 48),
]


@pytest.mark.parametrize("case", SCALE_CASES, ids=lambda c: f"{c[0]}-{c[1]}-g{c[2]}-P{c[5]}-T{max(c[4])}")
@pytest.mark.parametrize("scale", [0.0, -0.09])
def test_zero_and_negative_scale(case, scale):
    """A zero softmax scale weights every visible key alike (the output is the mean of V); a
    negative one weights the smallest scores most."""
    qd, kvd, g, lens, T, P = case
    m = Multi(qd, kvd, 2, g, 128, lens, T, seed=112 + SCALE_CASES.index(case))
    m.wl.scale = scale
    m.check(m.run(partition_tokens=P), f"scale {scale} {case}", relief=True)


@pytest.mark.parametrize("qd,kvd,T", [("bf16", "bf16", 64), ("bf16", "bf16", 32),
                                      ("f16", "fp8_e4m3", 64), ("bf16", "fp8_e4m3", 24)])
def test_chunk_rows_with_key_partitions(qd, kvd, T):
    """One long and one short prompt: too few blocks of rows to fill the GPU, so the keys are cut
    into partitions too (merged afterwards); the short prompt's later partitions see no key of
    its rows.  Every row, both row-block shapes."""
    m = Multi(qd, kvd, 2, 4, 128, (6000, 700), (T, T), seed=116)
    m.check(m.run(), f"key partitions {qd} {kvd} T{T}")


def test_chunk_partition_cap_long_context():
    """A 35000-token bf16 prompt with 1024 new rows per head: 256 blocks of rows, so the plan keeps
    one key partition, and the 16-bit chunk kernel's cap (2048 blocks, the partition's block ids
    held in LDS) cuts the 2188 blocks in two, merged afterwards.  Sampled rows (every KV head,
    first and last rows included) against the oracle; row i attends the first 33977 + i tokens."""
    L, T, G, hkv = 35000, 1024, 8, 8
    m = Multi("bf16", "bf16", hkv, G, 128, (L,), (T,), seed=117)
    got = m.run()
    wl, s = m.wl, m.spec
    rng = np.random.default_rng(117)
    rows = sorted({0, 1, 512, T - 2, T - 1} | set(int(r) for r in rng.integers(0, T, 11)))
    qf = oracle.to_f64(m.q[rows], s.q_dtype)                       # [rows][Hq][D]
    ref = np.zeros((len(rows), hkv * G, 128))
    for kvh in range(hkv):
        k, v = oracle.gather(m.k, m.v, s.kv_dtype, wl.block_tables[0], L, kvh)
        for r, i in enumerate(rows):
            n = L - T + i + 1
            ref[r, kvh * G:(kvh + 1) * G], _ = oracle.attend(qf[r, kvh * G:(kvh + 1) * G],
                                                            k[:n], v[:n], float(np.float32(wl.scale)))
    assert_close(got[rows], ref, s.q_dtype, "partition cap, sampled rows")


def test_more_queries_than_context_and_loose_bounds():
    """Rows before the context are zero; host bounds larger than needed change nothing."""
    m = Multi("bf16", "bf16", 2, 4, 128, (3, 1, 40), (6, 4, 2), seed=101, spare_rows=2)
    ref = m.reference()
    assert np.all(ref[0:3] == 0) and np.all(ref[6:9] == 0)
    m.check(m.run(), "tight", ref, relief=SHORT_WINDOWS)
    m.check(m.run(max_query_len=64, max_context_len=4096), "loose", ref,
            relief=SHORT_WINDOWS)


def test_repeat_runs_bitwise_identical():
    m = Multi("bf16", "bf16", 2, 8, 128, LENS, DRAFT, seed=102)
    first = m.run(partition_tokens=64)
    for _ in range(2):
        assert np.array_equal(m.run(partition_tokens=64), first)


def test_full_size_verification_batch():
    """64 sequences of 128..8192 tokens, GQA 64/8, 4 draft tokens each: every row."""
    rng = np.random.default_rng(103)
    lens = rng.integers(128, 8192, size=64, endpoint=True)
    m = Multi("bf16", "bf16", 8, 8, 128, lens, [4] * 64, seed=103)
    m.check(m.run(), "full-size verification")


def test_full_size_prefill_chunk():
    """4 prompts whose last 512-token chunk runs against 4096 cached tokens: every row."""
    m = Multi("bf16", "bf16", 8, 4, 128, [4608] * 4, [512] * 4, seed=104)
    m.check(m.run(), "full-size prefill chunk")


def test_full_size_fp8_verification():
    """4 sequences of 32768 fp8 tokens, GQA 64/8, 4 draft tokens each: two row tiles per head in
    one wave; every row."""
    m = Multi("bf16", "fp8_e4m3", 8, 8, 128, [32768] * 4, [4] * 4, seed=105)
    m.check(m.run(), "full-size fp8 verification")


@pytest.mark.parametrize("kvd", ["bf16", "fp8_e4m3"])
def test_full_size_wide_verification(kvd):
    """4 sequences of 32768 tokens, GQA 64/8, 8 draft tokens each: four row tiles per head in
    two waves a chunk; every row."""
    m = Multi("bf16", kvd, 8, 8, 128, [32768] * 4, [8] * 4, seed=108)
    m.check(m.run(), f"full-size wide verification {kvd}")


@pytest.mark.parametrize("kvd,T", [("fp8_e4m3", 4), ("bf16", 2), ("bf16", 4), ("fp8_e4m3", 6),
                                   ("bf16", 8)])
def test_full_size_one_head_over_many_workgroups(kvd, T):
    """One KV head of 65536 tokens: two-block chunks, so its parts come from hundreds of
    workgroups and are merged in LDS-staged batches; every row."""
    m = Multi("bf16", kvd, 1, 8, 128, [65536], [T], seed=106)
    m.check(m.run(), f"one head {kvd} T{T}")


def test_one_workspace_serves_every_entry_point():
    """The binding's workspace of a stream is shared by all calls on it: a fixed-partition call
    (partial results after the counter region) must leave the arrival counters of the balanced
    split and of pa_decode at zero, call after call, in any order."""
    m = Multi("bf16", "fp8_e4m3", 2, 8, 128, LENS, [min(t, 4) for t in DRAFT], seed=107,
              spare_rows=2)
    ref = m.reference()
    wl, s = m.wl, m.spec
    ks, vs = torch.from_numpy(wl.k_scale).cuda(), torch.from_numpy(wl.v_scale).cuda()
    # single-query decode of each sequence's last row: the multi-query row at position L - 1
    has = [b for b in range(s.batch) if m.T[b] > 0]
    last = np.array([int(m.qs[b + 1]) - 1 for b in has])
    qd = dev_bits(np.ascontiguousarray(m.q[last]), s.q_dtype)
    kd, vd = dev_bits(m.k, s.kv_dtype), dev_bits(m.v, s.kv_dtype)
    tables = torch.from_numpy(np.ascontiguousarray(wl.block_tables[has])).cuda()
    lens = torch.from_numpy(np.ascontiguousarray(wl.context_lens[has])).cuda()
    for order in ((32, 0, "decode"), ("decode", 32, 0), (0, "decode", 32)):
        for step in order:
            if step == "decode":
                out = torch.empty_like(qd)
                pa.pa_decode(qd, kd, vd, tables, lens, float(wl.scale), out, k_scale=ks,
                             v_scale=vs)
                torch.cuda.synchronize()
                assert_close(host_bits(out), ref[last], s.q_dtype, f"decode after {order}",
                             relief=SHORT_WINDOWS)
            else:
                m.check(m.run(partition_tokens=step), f"multi P{step} in {order}", ref,
                        relief=SHORT_WINDOWS)


RANDOM = [
    # (seed, q dtype, kv dtype, kv heads, group, head_dim, batch, longest context, most drafts)
    (200, "bf16", "bf16", 2, 8, 128, 40, 3000, 2),
    (201, "f16", "fp8_e4m3", 1, 4, 128, 60, 2500, 8),
    (202, "bf16", "bf16", 3, 2, 64, 90, 1200, 8),
    (203, "f16", "f16", 2, 1, 128, 30, 4000, 16),
    (204, "bf16", "fp8_e4m3", 2, 16, 64, 25, 2000, 2),
    (205, "bf16", "bf16", 1, 8, 128, 700, 120, 4),     # several sequences per scanning thread
    (206, "bf16", "bf16", 2, 16, 64, 50, 3000, 4),     # heads of one to four tiles
    (208, "bf16", "bf16", 2, 8, 128, 50, 3000, 8),
    (207, "f16", "fp8_e4m3", 2, 8, 128, 50, 3000, 8),
]


@pytest.mark.parametrize("case", RANDOM, ids=lambda c: f"seed{c[0]}")
def test_random_split_batches(case):
    """Random batches for the balanced split: lengths from 0 (no cached token) to the bound,
    draft counts from 0 (no rows) to the bound, so heads of one to four tiles, empty sequences
    and rows before the context all occur in one call."""
    seed, qd, kvd, hkv, g, d, B, lmax, tmax = case
    rng = np.random.default_rng(seed)
    lens = rng.integers(0, lmax + 1, size=B)
    lens[rng.random(B) < 0.1] = 0
    T = rng.integers(0, tmax + 1, size=B)
    m = Multi(qd, kvd, hkv, g, d, [int(x) for x in lens], [int(x) for x in T], seed=seed,
              spare_rows=2)
    m.check(m.run(), f"random {case}", relief=SHORT_WINDOWS)
