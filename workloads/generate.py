"""Seeded generators for the paged decode-attention workloads.

Every workload is a batch of sequences whose K/V history lives in a pool of 16-token physical
blocks, reached through per-sequence block tables with the blocks scattered by a seeded
permutation (the logical-block -> physical-block mapping of the PagedAttention explainers: the
youngju.dev serving guide, "PagedAttention" memory-layout figure, and kasblo.com,
"PagedAttentionはKV Cacheをblockで管理する").

Context lengths count the token appended this step (a decode step first appends the new token's
K/V, then attends over all of them).  The generator therefore returns the pool *before* the
append, with the slot of token L-1 poisoned, plus that token's K/V rows and its slot.

Values: Q, K, V ~ N(0, 1) in float32, rounded once to the storage dtype (round-to-nearest-even).
fp8 e4m3 caches get one fp32 scale per (physical block, kv_head) for K and for V, equal to the
tile's amax / 448 over its valid tokens (1.0 for an all-zero tile); codes are RNE of value/scale.

With poison=True every byte the decode must not read is NaN: slots past the end of each
sequence's last block, all unused blocks, the pre-append slot, the scales of unused blocks, and
block-table entries past a sequence's last block point at unused (poisoned) blocks.
"""

from __future__ import annotations

import dataclasses
import math
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

from .sizing import BLOCK_SIZE

FP8_MAX = 448.0
NAN_BITS = {"bf16": 0x7FC0, "f16": 0x7E00, "fp8_e4m3": 0x7F}
TORCH_DTYPE = {"bf16": torch.bfloat16, "f16": torch.float16, "fp8_e4m3": torch.float8_e4m3fn}
BITS_DTYPE = {"bf16": np.uint16, "f16": np.uint16, "fp8_e4m3": np.uint8}


@dataclasses.dataclass(frozen=True)
class Spec:
    """Shape and distribution of one workload."""

    name: str
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    q_dtype: str
    kv_dtype: str
    lengths: tuple            # ("list", (..)) | ("fixed", L) | ("uniform", lo, hi) | ("lognormal", median, sigma, cap)
    pool: tuple = ("times", 2)  # ("fixed", num_blocks) | ("times", k): k x the unique blocks needed
    prefix: tuple | None = None  # (num_sharing_sequences, prefix_tokens), prefix block-aligned
    partition_tokens: int = 0    # split-KV partition the workload prescribes (0: library's choice)
    seed: int = 0

    def replace(self, **kw) -> "Spec":
        return dataclasses.replace(self, **kw)


SPECS: dict[str, Spec] = {
    s.name: s
    for s in [
        # Small case: GQA group 4, head_dim 64, pool of 64 blocks; lengths cover L=1, a fresh block
        # (17, 33) and a 7-block sequence (100 tokens).
        Spec("tiny_b4_h8kv2_d64_bf16", 4, 8, 2, 64, "bf16", "bf16",
             ("list", (1, 17, 33, 100)), pool=("fixed", 64), seed=0),
        # 7B-style multi-head attention layer, fp16.
        Spec("mha_b16_h32_d128_f16_l2048", 16, 32, 32, 128, "f16", "f16",
             ("fixed", 2048), seed=1),
        # 70B-style GQA layer (group 8), ragged uniform lengths.
        Spec("gqa_b64_h64kv8_d128_bf16_l128to8192", 64, 64, 8, 128, "bf16", "bf16",
             ("uniform", 128, 8192), seed=2),
        # Mixed serving batch: lognormal lengths, a quarter of the batch shares a 1024-token prefix.
        Spec("mixed_b256_h32kv8_d128_bf16_lognorm600_prefix1024", 256, 32, 8, 128, "bf16", "bf16",
             ("lognormal", 600.0, 1.0, 16384), prefix=(64, 1024), seed=3),
        # Long context with fp8 e4m3 K/V and 512-token split-KV partitions.
        Spec("long_b4_h64kv8_d128_fp8_l32768_split512", 4, 64, 8, 128, "bf16", "fp8_e4m3",
             ("fixed", 32768), partition_tokens=512, seed=4),
    ]
}


def spec_names() -> list[str]:
    return list(SPECS)


@dataclasses.dataclass
class Workload:
    spec: Spec
    seed: int
    num_blocks: int
    context_lens: np.ndarray      # [B] int32, post-append lengths
    block_tables: np.ndarray      # [B][max_blocks_per_seq] int32
    q: np.ndarray                 # [B][Hq][D] raw bits of q_dtype
    k_cache: np.ndarray           # [NB][Hkv][16][D] raw bits, pre-append
    v_cache: np.ndarray           # [NB][Hkv][D][16] raw bits, pre-append
    k_scale: np.ndarray | None    # [NB][Hkv] float32 (fp8 only)
    v_scale: np.ndarray | None
    k_new: np.ndarray             # [B][Hkv][D] raw bits of token L-1
    v_new: np.ndarray
    slot_mapping: np.ndarray      # [B] int64, -1 where L == 0
    scale: np.float32             # 1/sqrt(head_dim) rounded to fp32
    sharing: np.ndarray           # indices of sequences that share the prefix (may be empty)
    prefix_blocks: int            # physical blocks shared by them
    unique_tokens: int            # K/V tokens stored once (shared prefix counted once)

    @property
    def batch(self) -> int:
        return self.spec.batch

    @property
    def group(self) -> int:
        return self.spec.num_q_heads // self.spec.num_kv_heads

    @property
    def max_blocks_per_seq(self) -> int:
        return self.block_tables.shape[1]

    @property
    def max_context_len(self) -> int:
        return int(self.context_lens.max()) if len(self.context_lens) else 0


def _derive(seed: int, stream: int, chunk: int = 0) -> int:
    return (seed * 1_000_003 + stream * 10_007 + chunk * 7_919 + 12_345) % (2**62)


def storage_bits(x: torch.Tensor | np.ndarray, dtype: str) -> np.ndarray:
    """Round float32 values to the storage dtype (RNE) and return the raw bits."""
    t = torch.as_tensor(np.asarray(x, dtype=np.float32))
    if dtype == "fp8_e4m3":
        t = t.clamp(-FP8_MAX, FP8_MAX)
    bits = t.to(TORCH_DTYPE[dtype])
    if dtype == "fp8_e4m3":
        return bits.view(torch.uint8).numpy().copy()
    return bits.view(torch.int16).numpy().view(np.uint16).copy()


def _lengths(spec: Spec, rng: np.random.Generator) -> np.ndarray:
    kind = spec.lengths[0]
    if kind == "list":
        lens = np.array(spec.lengths[1], dtype=np.int64)
        assert len(lens) == spec.batch
    elif kind == "fixed":
        lens = np.full(spec.batch, spec.lengths[1], dtype=np.int64)
    elif kind == "uniform":
        lo, hi = spec.lengths[1], spec.lengths[2]
        lens = rng.integers(lo, hi, size=spec.batch, endpoint=True)
    elif kind == "lognormal":
        median, sigma, cap = spec.lengths[1:]
        x = rng.lognormal(mean=math.log(median), sigma=sigma, size=spec.batch)
        lens = np.clip(np.rint(x), 1, cap).astype(np.int64)
    else:
        raise ValueError(f"unknown length kind {kind!r}")
    return lens


def _draw_tiles(seed: int, stream: int, n: int, tile_shape: tuple, chunk_blocks: int = 256):
    """n tiles of N(0,1) float32, drawn in independently seeded chunks (thread-count invariant)."""
    out = torch.empty((n,) + tile_shape, dtype=torch.float32)
    chunks = [(c, c * chunk_blocks, min(n, (c + 1) * chunk_blocks))
              for c in range(-(-n // chunk_blocks))]

    def work(item):
        c, lo, hi = item
        g = torch.Generator().manual_seed(_derive(seed, stream, c))
        out[lo:hi] = torch.randn((hi - lo,) + tile_shape, generator=g, dtype=torch.float32)

    workers = max(1, min(8, os.cpu_count() or 1))
    with ThreadPoolExecutor(workers) as ex:
        list(ex.map(work, chunks))
    return out


def _quantize_tiles(x: torch.Tensor, valid_mask: torch.Tensor, dtype: str):
    """Round tiles to dtype; for fp8 also return the per-(tile, head) fp32 scales."""
    if dtype != "fp8_e4m3":
        bits = x.to(TORCH_DTYPE[dtype]).view(torch.int16)
        return bits.numpy().view(np.uint16), None
    amax = (x.abs() * valid_mask).amax(dim=(2, 3))                    # [n][Hkv]
    scale = torch.where(amax > 0, amax / FP8_MAX, torch.ones_like(amax)).to(torch.float32)
    q = (x / scale[:, :, None, None]).clamp(-FP8_MAX, FP8_MAX).to(torch.float8_e4m3fn)
    return q.view(torch.uint8).numpy(), scale.numpy()


def make(spec: Spec | str, seed: int | None = None, poison: bool = True,
         extra_table_cols: int = 0) -> Workload:
    """Build one seeded workload (see the module docstring for the conventions)."""
    if isinstance(spec, str):
        spec = SPECS[spec]
    seed = spec.seed if seed is None else seed
    B, Hq, Hkv, D = spec.batch, spec.num_q_heads, spec.num_kv_heads, spec.head_dim
    assert Hq % Hkv == 0
    rng = np.random.default_rng(seed)

    # 1. lengths, 2. sharing choice
    lens = _lengths(spec, rng)
    sharing = np.zeros(0, dtype=np.int64)
    prefix_tokens = 0
    if spec.prefix is not None:
        n_share, prefix_tokens = spec.prefix
        assert prefix_tokens % BLOCK_SIZE == 0
        sharing = np.sort(rng.choice(B, size=n_share, replace=False))
        cap = spec.lengths[3] if spec.lengths[0] == "lognormal" else np.iinfo(np.int64).max
        lens[sharing] = np.minimum(prefix_tokens + lens[sharing], cap)
    prefix_blocks = prefix_tokens // BLOCK_SIZE
    nblk = -(-lens // BLOCK_SIZE)

    # Unique blocks in a fixed order: the shared prefix, then each sequence's private blocks.
    is_sharing = np.zeros(B, dtype=bool)
    is_sharing[sharing] = True
    private = nblk - np.where(is_sharing, prefix_blocks, 0)
    n_unique = int(prefix_blocks + private.sum()) if len(sharing) else int(nblk.sum())
    if not len(sharing):
        prefix_blocks = 0
    valid = np.full(n_unique, BLOCK_SIZE, dtype=np.int64)   # valid tokens per unique block
    seq_unique = []                                         # unique ids of each sequence's blocks
    cursor = prefix_blocks
    for b in range(B):
        ids = []
        if is_sharing[b]:
            ids.extend(range(prefix_blocks))
        ids.extend(range(cursor, cursor + int(private[b])))
        cursor += int(private[b])
        if ids and lens[b] % BLOCK_SIZE:
            valid[ids[-1]] = lens[b] % BLOCK_SIZE
        seq_unique.append(np.array(ids, dtype=np.int64))

    # 3. block placement
    if spec.pool[0] == "fixed":
        NB = int(spec.pool[1])
    else:
        NB = int(spec.pool[1]) * max(n_unique, 1)
    assert NB >= n_unique, "pool too small"
    perm = rng.permutation(NB)
    phys = perm[:n_unique]
    unused = perm[n_unique:]
    MB = max(1, int(nblk.max()) if B else 1) + extra_table_cols
    tables = np.zeros((B, MB), dtype=np.int32)
    for b in range(B):
        tables[b, : len(seq_unique[b])] = phys[seq_unique[b]]
        rest = MB - len(seq_unique[b])
        if rest and poison and len(unused):
            tables[b, len(seq_unique[b]):] = rng.choice(unused, size=rest)

    # 4. values
    g = torch.Generator().manual_seed(_derive(seed, 1))
    q = torch.randn((B, Hq, D), generator=g, dtype=torch.float32)
    q_bits = storage_bits(q, spec.q_dtype)

    tok = torch.arange(BLOCK_SIZE)
    valid_t = torch.from_numpy(valid)
    k_mask = (tok[None, :] < valid_t[:, None]).to(torch.float32)[:, None, :, None]  # [n][1][16][1]
    v_mask = (tok[None, :] < valid_t[:, None]).to(torch.float32)[:, None, None, :]  # [n][1][1][16]
    k_f = _draw_tiles(seed, 2, n_unique, (Hkv, BLOCK_SIZE, D))
    k_bits, k_sc = _quantize_tiles(k_f, k_mask, spec.kv_dtype)
    del k_f
    v_f = _draw_tiles(seed, 3, n_unique, (Hkv, D, BLOCK_SIZE))
    v_bits, v_sc = _quantize_tiles(v_f, v_mask, spec.kv_dtype)
    del v_f

    bits_t = BITS_DTYPE[spec.kv_dtype]
    nan = bits_t(NAN_BITS[spec.kv_dtype])
    fill = nan if poison else bits_t(0)
    k_pool = np.full((NB, Hkv, BLOCK_SIZE, D), fill, dtype=bits_t)
    v_pool = np.full((NB, Hkv, D, BLOCK_SIZE), fill, dtype=bits_t)
    if poison:
        for u in np.nonzero(valid < BLOCK_SIZE)[0]:
            k_bits[u, :, valid[u]:, :] = nan
            v_bits[u, :, :, valid[u]:] = nan
    k_pool[phys] = k_bits
    v_pool[phys] = v_bits
    del k_bits, v_bits
    k_scale = v_scale = None
    if spec.kv_dtype == "fp8_e4m3":
        k_scale = np.full((NB, Hkv), np.nan if poison else 1.0, dtype=np.float32)
        v_scale = np.full((NB, Hkv), np.nan if poison else 1.0, dtype=np.float32)
        k_scale[phys] = k_sc
        v_scale[phys] = v_sc

    # 5. the token appended this step: position L-1 of every sequence
    k_new = np.full((B, Hkv, D), nan, dtype=bits_t)
    v_new = np.full((B, Hkv, D), nan, dtype=bits_t)
    slots = np.full(B, -1, dtype=np.int64)
    for b in range(B):
        if lens[b] == 0:
            continue
        t = int(lens[b]) - 1
        blk = int(tables[b, t // BLOCK_SIZE])
        off = t % BLOCK_SIZE
        slots[b] = blk * BLOCK_SIZE + off
        k_new[b] = k_pool[blk, :, off, :]
        v_new[b] = v_pool[blk, :, :, off]
        if poison:
            k_pool[blk, :, off, :] = nan
            v_pool[blk, :, :, off] = nan

    unique_tokens = int(lens.sum()) - max(len(sharing) - 1, 0) * prefix_tokens
    return Workload(
        spec=spec, seed=seed, num_blocks=NB,
        context_lens=lens.astype(np.int32), block_tables=tables,
        q=q_bits, k_cache=k_pool, v_cache=v_pool, k_scale=k_scale, v_scale=v_scale,
        k_new=k_new, v_new=v_new, slot_mapping=slots,
        scale=np.float32(1.0 / math.sqrt(D)),
        sharing=sharing, prefix_blocks=prefix_blocks, unique_tokens=unique_tokens,
    )


# Several query tokens per sequence: (cache workload, new query tokens per sequence).
MULTI_SPECS: dict[str, tuple[Spec, int]] = {
    # Speculative verification: the GQA serving batch checks 4 draft tokens per sequence.
    "verify_b64_h64kv8_d128_bf16_l128to8192_t4": (
        Spec("verify_b64_h64kv8_d128_bf16_l128to8192_t4", 64, 64, 8, 128, "bf16", "bf16",
             ("uniform", 128, 8192), seed=2), 4),
    # Speculative verification on the long-context fp8 batch: 4 draft tokens per sequence.
    "verify_b4_h64kv8_d128_fp8_l32768_t4": (
        Spec("verify_b4_h64kv8_d128_fp8_l32768_t4", 4, 64, 8, 128, "bf16", "fp8_e4m3",
             ("fixed", 32768), seed=4), 4),
    # Chunked prefill: 4 prompts whose next 512-token chunk runs against 4096 cached tokens.
    "prefill_b4_h32kv8_d128_bf16_l4608_chunk512": (
        Spec("prefill_b4_h32kv8_d128_bf16_l4608_chunk512", 4, 32, 8, 128, "bf16", "bf16",
             ("fixed", 4608), seed=6), 512),
}


@dataclasses.dataclass
class MultiWorkload:
    wl: Workload                # the cache: context_lens count the new tokens too
    query_lens: np.ndarray      # [B] int32
    query_start: np.ndarray     # [B + 1] int32
    q: np.ndarray               # [N][Hq][D] raw bits of q_dtype
    slot_mapping: np.ndarray    # [N] int64: cache slot of each new token
    k_new: np.ndarray           # [N][Hkv][D] raw bits: the new tokens' K/V as stored
    v_new: np.ndarray


def make_multi(name: str, poison: bool = False) -> MultiWorkload:
    """A multi-query workload: every one of the context_lens tokens already in the cache, the
    last T of each sequence being the new ones; their rows (for an append) and N(0,1) queries."""
    spec, T = MULTI_SPECS[name]
    wl = make(spec, poison=False)
    B, Hq, D = spec.batch, spec.num_q_heads, spec.head_dim
    lens = wl.context_lens.astype(np.int64)
    qlens = np.minimum(lens, T).astype(np.int32)
    qs = np.concatenate([[0], np.cumsum(qlens)]).astype(np.int32)
    N = int(qs[-1])
    slots = np.empty(N, dtype=np.int64)
    for b in range(B):
        pos = lens[b] - qlens[b] + np.arange(qlens[b])
        slots[qs[b]:qs[b + 1]] = wl.block_tables[b, pos // BLOCK_SIZE].astype(np.int64) * \
            BLOCK_SIZE + pos % BLOCK_SIZE
    blk, off = slots // BLOCK_SIZE, slots % BLOCK_SIZE
    k_new = np.ascontiguousarray(wl.k_cache[blk, :, off, :])
    v_new = np.ascontiguousarray(wl.v_cache[blk, :, :, off])
    g = torch.Generator().manual_seed(_derive(wl.seed, 4))
    q = storage_bits(torch.randn((N, Hq, D), generator=g, dtype=torch.float32), spec.q_dtype)
    return MultiWorkload(wl=wl, query_lens=qlens, query_start=qs, q=q, slot_mapping=slots,
                         k_new=k_new, v_new=v_new)
