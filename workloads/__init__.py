"""Seeded synthetic inputs for paged decode attention.

This package only *makes inputs*: context lengths, block tables, Q/K/V values rounded to their
storage dtypes, fp8 block scales and the slot of the token appended each step.  It holds none of
the attention arithmetic, so the HIP library's tests, the benchmark and the fp64 oracle can all
draw from it without sharing any of the method's code.

Cache layout used by every producer and consumer (one (block, kv_head) tile each):
  K pool  [num_blocks][num_kv_heads][16][head_dim]   token-major tile
  V pool  [num_blocks][num_kv_heads][head_dim][16]   dim-major tile
"""

from .generate import (MULTI_SPECS, SPECS, MultiWorkload, Workload, make,  # noqa: F401
                       make_multi, spec_names, storage_bits)
from .sizing import (  # noqa: F401
    BLOCK_SIZE,
    append_bytes,
    decode_bytes,
    kv_bytes_per_token,
    m_alloc,
    m_block,
    m_waste,
    multi_bytes,
    multi_flops,
    n_blocks,
    visible_keys,
)
