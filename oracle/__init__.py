"""fp64 CPU oracle for paged decode attention.

TEST INFRASTRUCTURE, not part of the product: only tests/, __graft_entry__.smoke() and
bench.py's cpu_baseline leg may import, call or run anything in this package.  It is written from
the pages' definitions (see paged_attention.py for the citations), works in float64 on exactly
decoded inputs, and shares no code with the HIP library.
"""

from .blocks import BlockPoolModel, copy_blocks  # noqa: F401
from .formats import (E4M3FN_TABLE, bf16_to_f64, e4m3fn_encode, e4m3fn_to_f64,  # noqa: F401
                      f16_to_f64, to_f64)
from .paged_attention import (SCALE_FIRST_TOKEN, SCALE_KEEP, attend, decode,  # noqa: F401
                              decode_multi, decode_split, gather, kv_append, kv_append_quant)
