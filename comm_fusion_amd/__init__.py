"""MI355X (gfx950) Ulysses-shard attention with the post-attention All-to-All
fused into the output epilogue.

Thin ctypes binding over ``libulysses_attn.so`` (C ABI in
``include/ulysses_attn.h``).  It only marshals arguments: tensor pointers,
shapes and the current HIP stream.  Every step of the computation runs in the
library's HIP kernels; if the library is not built this package raises instead
of computing anything itself.

Names and arguments follow the C calls:
  attn_ulysses_fused(Q, K, V, rank, P, out, scale=None, stream=None)
  attn_serial(Q, K, V, rank, P, O_local, scale=None, stream=None)
  a2a_permute(O_local, rank, P, out, stream=None)
  attn_ulysses_fused_io(Xq, Xk, Xv, rank, P, out, scale=None, stream=None)
  a2a_gather(X, rank, P, X_local, stream=None)
  attn_ulysses_fused_ws(Q, K, V, rank, P, out, workspace, scale=None, stream=None)
  attn_serial_ws(Q, K, V, rank, P, O_local, workspace, scale=None, stream=None)
  attn_ulysses_fused_io_ws(Xq, Xk, Xv, rank, P, out, workspace, scale=None, stream=None)
  attn_ulysses_fused_noalloc(Q, K, V, rank, P, out, scale=None, stream=None)
      (the _ws call with its workspace in the library's fixed device scratch)
  workspace_bytes(B, S, H, d, P), workspace_count_bytes(B, S, H, d, P), key_split(B, S, H, d, P),
  stream_k_iters(B, S, H, d, P)
  new_workspace(B, S, H, d, P, device)  (a zeroed uint8 tensor, or None)
the MoE expert path with the Combine fused into Linear-2 (include/moe_combine.h):
  moe_recv_layout(topk_idx, rank, P, hidden, inter, E) -> (expert_offsets, row_slot)
  moe_experts_combine(x, row_slot, topk_w, expert_offsets, W1, W2, P, E, combine, act,
                      schedule=MOE_INTERLEAVED, experts_per_wave=4, stream=None)
  moe_experts_local(...), moe_combine_scatter(...)   (the serial form)
  moe_experts_combine_ws(..., act, workspace, schedule=..., experts_per_wave=..., stream=None),
  moe_experts_local_ws(...)   (the persistent form: one launch, a device tile queue)
  moe_workspace_bytes(P, T, hidden, inter, E, k), new_moe_workspace(x, W1, topk_w, P, E)
and, for measurement only,
  attn_ulysses_fused_trace(Q, K, V, rank, P, out, trace, scale=None, stream=None)
  epilogue_store_only(B, S, H, d, rank, P, out, stream=None)
  fused_write_counts(Q, K, V, rank, P, out, counts, workspace=None, scale=None, stream=None)
  work_units(B, S, H, d, P)
Tensors are torch tensors on the GPU: Q, K, V, O_local bfloat16
[B][S][Hl][d]; out bfloat16 with B*S*(Hl*P)*d elements, laid out
[B][P][S/P][H][d]; Xq, Xk, Xv, X bfloat16 in the sequence-partitioned layout
[B][P][S/P][H][d] (or the same bytes viewed as [B][S][H][d]).
"""
from ._binding import (UA_ERR_ALIGN, UA_ERR_HIP, UA_ERR_NULL, UA_ERR_RANK,  # noqa: F401
                       UA_ERR_SCRATCH, UA_ERR_SHAPE, UA_ERR_UNSUPPORTED, UA_ERR_WORKSPACE, UA_OK,
                       SCRATCH_BYTES, UAError,
                       a2a_gather, a2a_permute, attn_serial, attn_serial_ws, attn_ulysses_fused,
                       attn_ulysses_fused_io, attn_ulysses_fused_io_ws, attn_ulysses_fused_trace,
                       attn_ulysses_fused_noalloc, attn_ulysses_fused_ws,
                       dest_bytes, epilogue_store_only, fused_write_counts, key_split, lib, lib_path, local_bytes,
                       new_workspace, status_string, stream_k_iters, version, work_units, workspace_bytes,
                       workspace_count_bytes)
from ._moe_binding import (MOE_EXPERT_WAVE, MOE_INTERLEAVED, MOE_MAX_WAVE, MoeShape,  # noqa: F401,E402
                           moe_combine_scatter, moe_experts_combine, moe_experts_combine_ws, moe_experts_local,
                           moe_experts_local_ws, moe_recv_layout, moe_workspace_bytes, new_moe_workspace)
