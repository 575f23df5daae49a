"""fp64 CPU oracles (test infrastructure only): the fused Ulysses attention
path (``oracle.py`` over ``attn_oracle.c``) and the MoE expert path with its
Combine exchange (``moe_oracle.py``, imported as ``oracle.moe_oracle``).

Only ``tests/``, the smoke check and the benchmark's CPU-baseline leg import this
package; the product library never does.
"""
from .oracle import (attn_all, attn_rows, build, dest_offset, dest_offsets, gather,  # noqa: F401
                     max_threads, permute, softmax_row, widen)
