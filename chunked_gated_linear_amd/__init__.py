"""Gated delta-rule linear attention for AMD Instinct MI355X (gfx950).

The work runs in hand-written HIP kernels behind a C ABI (include/lin_attn.h,
built into liblinattn.so); this package only marshals torch tensors into it.
"""

from .api import (lin_attn_chunk_bwd, lin_attn_chunk_bwd_workspace_size,  # noqa: F401
                  lin_attn_chunk_bwd_varlen, lin_attn_chunk_bwd_varlen_workspace_size,
                  lin_attn_check_inputs, lin_attn_chunk_fwd_noalloc,
                  lin_attn_chunk_fwd, lin_attn_chunk_fwd_channel,
                  lin_attn_chunk_fwd_channel_varlen,
                  lin_attn_chunk_fwd_channel_varlen_workspace_size,
                  lin_attn_chunk_fwd_channel_workspace_size,
                  lin_attn_chunk_fwd_workspace_size,
                  lin_attn_chunk_fwd_varlen, lin_attn_chunk_fwd_varlen_workspace_size,
                  lin_attn_decode_step, lin_attn_decode_step_channel, lin_attn_gate)
from ._native import LinAttnError, lib  # noqa: F401

__all__ = ["lin_attn_chunk_bwd", "lin_attn_chunk_bwd_workspace_size",
           "lin_attn_chunk_bwd_varlen", "lin_attn_chunk_bwd_varlen_workspace_size",
           "lin_attn_check_inputs", "lin_attn_chunk_fwd_noalloc",
           "lin_attn_chunk_fwd", "lin_attn_chunk_fwd_channel",
           "lin_attn_chunk_fwd_channel_varlen", "lin_attn_chunk_fwd_channel_varlen_workspace_size",
           "lin_attn_chunk_fwd_channel_workspace_size",
           "lin_attn_chunk_fwd_workspace_size",
           "lin_attn_chunk_fwd_varlen", "lin_attn_chunk_fwd_varlen_workspace_size",
           "lin_attn_decode_step", "lin_attn_decode_step_channel", "lin_attn_gate", "LinAttnError", "lib"]
