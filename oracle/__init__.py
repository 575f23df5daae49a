"""fp64 CPU oracle for the fused Ulysses attention path (test infrastructure only).

Only ``tests/``, the smoke check and the benchmark's CPU-baseline leg import this
package; the product library never does.
"""
from .oracle import (attn_all, attn_rows, build, dest_offset, dest_offsets, gather,  # noqa: F401
                     max_threads, permute, softmax_row, widen)
