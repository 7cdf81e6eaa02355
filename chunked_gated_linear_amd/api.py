"""Python entry points with the C ABI's names.  Argument marshalling only:
every step of the computation runs in the library's HIP kernels.

Tensors are torch tensors on the GPU (PyTorch supplies device memory and the
current stream); shapes and layouts are those of include/lin_attn.h.

Streams: with stream=None the kernels run on torch's current stream.  With
stream=s every tensor a wrapper allocates (outputs and a missing workspace)
is taken from the caching allocator while s is current, so torch reuses that
memory only in s's order, after the library's kernels; tensors the caller
passes in stay the caller's to order.
"""

from __future__ import annotations

import functools

import torch

from . import _native as N

_DTYPES = {torch.bfloat16: N.LA_BF16, torch.float32: N.LA_FP32}
_GATE = {"log": N.LA_GATE_LOG, "logit": N.LA_GATE_BOUNDED_LOGIT}


def _ptr(t):
    return None if t is None else t.data_ptr()


def _need(t, name, dtype=None, shape=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _on_stream(fn):
    """Run the wrapper with `stream` (keyword) current, so that its
    allocations belong to that stream."""
    @functools.wraps(fn)
    def wrapper(*args, **kwargs):
        stream = kwargs.get("stream")
        if stream is None:
            return fn(*args, **kwargs)
        with torch.cuda.stream(stream):
            return fn(*args, **kwargs)
    return wrapper


def _stream(t, stream):
    s = stream if stream is not None else torch.cuda.current_stream(t.device)
    return s.cuda_stream


def lin_attn_chunk_fwd_workspace_size(B, T, H, Dk, Dv, dtype=torch.bfloat16):
    """Workspace bytes lin_attn_chunk_fwd needs for these sizes (0 if none)."""
    n = N.lib().lin_attn_chunk_fwd_workspace_size(B, T, H, Dk, Dv, _DTYPES[dtype])
    if n < 0:
        raise N.LinAttnError(N.LA_EINVAL, N.lib().lin_attn_last_error().decode())
    return n


@_on_stream
def lin_attn_chunk_fwd(q, k, v, gate, beta, h0=None, *, gate_mode="log", G=5.0,
                       o=None, hT=None, output_final_state=True, workspace=None,
                       stream=None, raw=False, gate_scale=None, gate_bias=None):
    """o [B,T,H,Dv] and final state hT [B,H,Dk,Dv] (None if not requested).

    `workspace` is an optional uint8 GPU tensor of at least
    lin_attn_chunk_fwd_workspace_size(...) bytes; without one, a fresh tensor
    is taken from torch's caching allocator.  raw=True calls
    lin_attn_chunk_fwd_raw: q and k as they come (L2-normalised inside the
    pass) and `beta` holding logits.  gate_scale / gate_bias (float32 [H],
    with raw=True and gate_mode="logit") call lin_attn_chunk_fwd_raw_affine:
    g = -G * sigmoid(gate_scale[h] * gate + gate_bias[h])."""
    _need(q, "q")
    if q.dtype not in _DTYPES:
        raise TypeError("q, k, v must be bfloat16 or float32")
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    _need(k, "k", q.dtype, (B, T, H, Dk))
    _need(v, "v", q.dtype, (B, T, H, Dv))
    _need(gate, "gate", torch.float32, (B, T, H))
    _need(beta, "beta", torch.float32, (B, T, H))
    if h0 is not None:
        _need(h0, "h0", torch.float32, (B, H, Dk, Dv))
    if o is None:
        o = torch.empty((B, T, H, Dv), dtype=q.dtype, device=q.device)
    _need(o, "o", q.dtype, (B, T, H, Dv))
    if hT is None and output_final_state:
        hT = torch.empty((B, H, Dk, Dv), dtype=torch.float32, device=q.device)
    if hT is not None:
        _need(hT, "hT", torch.float32, (B, H, Dk, Dv))
    nws = lin_attn_chunk_fwd_workspace_size(B, T, H, Dk, Dv, q.dtype)
    if workspace is None and nws > 0:
        workspace = torch.empty(nws, dtype=torch.uint8, device=q.device)
    if workspace is not None:
        _need(workspace, "workspace", torch.uint8)
    if _affine(gate_scale, gate_bias, raw, gate_mode, H):
        N.check(N.lib().lin_attn_chunk_fwd_raw_affine(
            _ptr(q), _ptr(k), _ptr(v), _ptr(gate), float(G), _ptr(gate_scale), _ptr(gate_bias),
            _ptr(beta), _ptr(h0), _ptr(o), _ptr(hT), B, T, H, Dk, Dv, _DTYPES[q.dtype],
            _ptr(workspace), 0 if workspace is None else workspace.numel(), _stream(q, stream)))
        return o, hT
    fn = N.lib().lin_attn_chunk_fwd_raw if raw else N.lib().lin_attn_chunk_fwd
    N.check(fn(
        _ptr(q), _ptr(k), _ptr(v), _ptr(gate), _GATE[gate_mode], float(G), _ptr(beta),
        _ptr(h0), _ptr(o), _ptr(hT), B, T, H, Dk, Dv, _DTYPES[q.dtype], _ptr(workspace),
        0 if workspace is None else workspace.numel(), _stream(q, stream)))
    return o, hT


def _affine(gate_scale, gate_bias, raw, gate_mode, H):
    """True when a per-head affine gate pre-activation is asked for (checked)."""
    if gate_scale is None and gate_bias is None:
        return False
    if not raw or gate_mode != "logit":
        raise ValueError("gate_scale / gate_bias need raw=True and gate_mode='logit'")
    for t, nm in ((gate_scale, "gate_scale"), (gate_bias, "gate_bias")):
        if t is not None:
            _need(t, nm, torch.float32, (H,))
    return True


def lin_attn_chunk_fwd_noalloc(q, k, v, gate, beta, h0=None, *, o, hT=None, gate_mode="log",
                               G=5.0, stream=None):
    """lin_attn_chunk_fwd without a workspace, for callers that cannot
    allocate: the library's own 64 MiB scratch per GPU serves it, and this
    wrapper allocates nothing either (o, and hT if wanted, come from the
    caller).  Calls on one GPU must not overlap in time."""
    _need(q, "q")
    if q.dtype not in _DTYPES:
        raise TypeError("q, k, v must be bfloat16 or float32")
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    _need(k, "k", q.dtype, (B, T, H, Dk))
    _need(v, "v", q.dtype, (B, T, H, Dv))
    _need(gate, "gate", torch.float32, (B, T, H))
    _need(beta, "beta", torch.float32, (B, T, H))
    if h0 is not None:
        _need(h0, "h0", torch.float32, (B, H, Dk, Dv))
    _need(o, "o", q.dtype, (B, T, H, Dv))
    if hT is not None:
        _need(hT, "hT", torch.float32, (B, H, Dk, Dv))
    s = (stream if stream is not None else torch.cuda.current_stream(q.device)).cuda_stream
    N.check(N.lib().lin_attn_chunk_fwd_noalloc(
        _ptr(q), _ptr(k), _ptr(v), _ptr(gate), _GATE[gate_mode], float(G), _ptr(beta),
        _ptr(h0), _ptr(o), _ptr(hT), B, T, H, Dk, Dv, _DTYPES[q.dtype], s))
    return o, hT


def lin_attn_chunk_fwd_channel_workspace_size(B, T, H, Dk, Dv, dtype=torch.bfloat16):
    """Workspace bytes lin_attn_chunk_fwd_channel needs for these sizes."""
    n = N.lib().lin_attn_chunk_fwd_channel_workspace_size(B, T, H, Dk, Dv, _DTYPES[dtype])
    if n < 0:
        raise N.LinAttnError(N.LA_EINVAL, N.lib().lin_attn_last_error().decode())
    return n


@_on_stream
def lin_attn_chunk_fwd_channel(q, k, v, gate, beta, h0=None, *, gate_mode="log", G=5.0,
                               o=None, hT=None, output_final_state=True, workspace=None,
                               stream=None):
    """lin_attn_chunk_fwd with one log-decay per key channel: gate [B,T,H,Dk]
    float32.  Returns o [B,T,H,Dv] and hT [B,H,Dk,Dv] (None if not requested).
    `workspace`: optional uint8 GPU tensor of at least
    lin_attn_chunk_fwd_channel_workspace_size(...) bytes (else one is taken
    from torch's caching allocator)."""
    _need(q, "q")
    if q.dtype not in _DTYPES:
        raise TypeError("q, k, v must be bfloat16 or float32")
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    _need(k, "k", q.dtype, (B, T, H, Dk))
    _need(v, "v", q.dtype, (B, T, H, Dv))
    _need(gate, "gate", torch.float32, (B, T, H, Dk))
    _need(beta, "beta", torch.float32, (B, T, H))
    if h0 is not None:
        _need(h0, "h0", torch.float32, (B, H, Dk, Dv))
    if o is None:
        o = torch.empty((B, T, H, Dv), dtype=q.dtype, device=q.device)
    _need(o, "o", q.dtype, (B, T, H, Dv))
    if hT is None and output_final_state:
        hT = torch.empty((B, H, Dk, Dv), dtype=torch.float32, device=q.device)
    if hT is not None:
        _need(hT, "hT", torch.float32, (B, H, Dk, Dv))
    nws = lin_attn_chunk_fwd_channel_workspace_size(B, T, H, Dk, Dv, q.dtype)
    if workspace is None and nws > 0:
        workspace = torch.empty(nws, dtype=torch.uint8, device=q.device)
    if workspace is not None:
        _need(workspace, "workspace", torch.uint8)
    N.check(N.lib().lin_attn_chunk_fwd_channel(
        _ptr(q), _ptr(k), _ptr(v), _ptr(gate), _GATE[gate_mode], float(G), _ptr(beta),
        _ptr(h0), _ptr(o), _ptr(hT), B, T, H, Dk, Dv, _DTYPES[q.dtype], _ptr(workspace),
        0 if workspace is None else workspace.numel(), _stream(q, stream)))
    return o, hT


def lin_attn_chunk_fwd_channel_varlen_workspace_size(T, nseq, H, Dk, Dv, dtype=torch.bfloat16):
    """Workspace bytes lin_attn_chunk_fwd_channel_varlen needs for these sizes."""
    n = N.lib().lin_attn_chunk_fwd_channel_varlen_workspace_size(T, nseq, H, Dk, Dv,
                                                                 _DTYPES[dtype])
    if n < 0:
        raise N.LinAttnError(N.LA_EINVAL, N.lib().lin_attn_last_error().decode())
    return n


@_on_stream
def lin_attn_chunk_fwd_channel_varlen(q, k, v, gate, beta, cu_seqlens, h0=None, *,
                                      gate_mode="log", G=5.0, o=None, hT=None,
                                      output_final_state=True, workspace=None, stream=None):
    """Per-channel gate over packed sequences: q, k [1,T,H,Dk], v [1,T,H,Dv],
    gate [1,T,H,Dk], beta [1,T,H], cu_seqlens int32 [nseq+1] on the device.
    Returns o [1,T,H,Dv] and hT [nseq,H,Dk,Dv] (None if not requested)."""
    _need(q, "q")
    if q.dtype not in _DTYPES:
        raise TypeError("q, k, v must be bfloat16 or float32")
    one, T, H, Dk = q.shape
    if one != 1:
        raise ValueError("packed sequences come as one batch entry: q is [1, T, H, Dk]")
    Dv = v.shape[-1]
    _need(k, "k", q.dtype, (1, T, H, Dk))
    _need(v, "v", q.dtype, (1, T, H, Dv))
    _need(gate, "gate", torch.float32, (1, T, H, Dk))
    _need(beta, "beta", torch.float32, (1, T, H))
    _need(cu_seqlens, "cu_seqlens", torch.int32)
    nseq = cu_seqlens.numel() - 1
    if h0 is not None:
        _need(h0, "h0", torch.float32, (nseq, H, Dk, Dv))
    if o is None:
        o = torch.empty((1, T, H, Dv), dtype=q.dtype, device=q.device)
    _need(o, "o", q.dtype, (1, T, H, Dv))
    if hT is None and output_final_state:
        hT = torch.empty((nseq, H, Dk, Dv), dtype=torch.float32, device=q.device)
    if hT is not None:
        _need(hT, "hT", torch.float32, (nseq, H, Dk, Dv))
    nws = lin_attn_chunk_fwd_channel_varlen_workspace_size(T, nseq, H, Dk, Dv, q.dtype)
    if workspace is None and nws > 0:
        workspace = torch.empty(nws, dtype=torch.uint8, device=q.device)
    N.check(N.lib().lin_attn_chunk_fwd_channel_varlen(
        _ptr(q), _ptr(k), _ptr(v), _ptr(gate), _GATE[gate_mode], float(G), _ptr(beta), _ptr(h0),
        _ptr(o), _ptr(hT), _ptr(cu_seqlens), nseq, T, H, Dk, Dv, _DTYPES[q.dtype],
        _ptr(workspace), 0 if workspace is None else workspace.numel(), _stream(q, stream)))
    return o, hT


def lin_attn_chunk_bwd_workspace_size(B, T, H, Dk, Dv, dtype=torch.bfloat16, segment_tokens=None):
    """Workspace bytes lin_attn_chunk_bwd needs for these sizes (of the
    segmented form when segment_tokens is given)."""
    if segment_tokens is None:
        n = N.lib().lin_attn_chunk_bwd_workspace_size(B, T, H, Dk, Dv, _DTYPES[dtype])
    else:
        n = N.lib().lin_attn_chunk_bwd_segmented_workspace_size(B, T, H, Dk, Dv, _DTYPES[dtype],
                                                               int(segment_tokens))
    if n < 0:
        raise N.LinAttnError(N.LA_EINVAL, N.lib().lin_attn_last_error().decode())
    return n


@_on_stream
def lin_attn_chunk_bwd(q, k, v, gate, beta, dout, h0=None, dhT=None, *, gate_mode="log",
                       G=5.0, output_dh0=True, workspace=None, stream=None, segment_tokens=None):
    """Gradients of <o, dout> + <hT, dhT> for lin_attn_chunk_fwd's inputs.

    Returns float32 tensors (dq, dk, dv, dgate, dbeta, dh0): dgate is dL/dg in
    "log" mode and dL/dx in "logit" mode; dh0 is None unless output_dh0.
    segment_tokens (a multiple of 64; bf16 inputs, d_v <= 128) selects the
    segmented form (lin_attn_chunk_bwd_segmented): the same results with a
    workspace bounded by the segment length."""
    _need(q, "q")
    if q.dtype not in _DTYPES:
        raise TypeError("q, k, v, dout must be bfloat16 or float32")
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    _need(k, "k", q.dtype, (B, T, H, Dk))
    _need(v, "v", q.dtype, (B, T, H, Dv))
    _need(dout, "dout", q.dtype, (B, T, H, Dv))
    _need(gate, "gate", torch.float32, (B, T, H))
    _need(beta, "beta", torch.float32, (B, T, H))
    if h0 is not None:
        _need(h0, "h0", torch.float32, (B, H, Dk, Dv))
    if dhT is not None:
        _need(dhT, "dhT", torch.float32, (B, H, Dk, Dv))
    f32 = dict(dtype=torch.float32, device=q.device)
    dq = torch.empty((B, T, H, Dk), **f32)
    dk = torch.empty((B, T, H, Dk), **f32)
    dv = torch.empty((B, T, H, Dv), **f32)
    dgate = torch.empty((B, T, H), **f32)
    dbeta = torch.empty((B, T, H), **f32)
    dh0 = torch.empty((B, H, Dk, Dv), **f32) if output_dh0 else None
    nws = lin_attn_chunk_bwd_workspace_size(B, T, H, Dk, Dv, q.dtype, segment_tokens)
    if workspace is None and nws > 0:
        workspace = torch.empty(nws, dtype=torch.uint8, device=q.device)
    if workspace is not None:
        _need(workspace, "workspace", torch.uint8)
    args = [_ptr(q), _ptr(k), _ptr(v), _ptr(gate), _GATE[gate_mode], float(G), _ptr(beta),
            _ptr(h0), _ptr(dout), _ptr(dhT), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dgate),
            _ptr(dbeta), _ptr(dh0), B, T, H, Dk, Dv, _DTYPES[q.dtype]]
    tail = [_ptr(workspace), 0 if workspace is None else workspace.numel(), _stream(q, stream)]
    if segment_tokens is None:
        N.check(N.lib().lin_attn_chunk_bwd(*args, *tail))
    else:
        N.check(N.lib().lin_attn_chunk_bwd_segmented(*args, int(segment_tokens), *tail))
    return dq, dk, dv, dgate, dbeta, dh0


def lin_attn_chunk_bwd_varlen_workspace_size(T, nseq, H, Dk, Dv, dtype=torch.bfloat16):
    """Workspace bytes lin_attn_chunk_bwd_varlen needs for these sizes."""
    n = N.lib().lin_attn_chunk_bwd_varlen_workspace_size(T, nseq, H, Dk, Dv, _DTYPES[dtype])
    if n < 0:
        raise N.LinAttnError(N.LA_EINVAL, N.lib().lin_attn_last_error().decode())
    return n


@_on_stream
def lin_attn_chunk_bwd_varlen(q, k, v, gate, beta, dout, cu_seqlens, h0=None, dhT=None, *,
                              gate_mode="log", G=5.0, output_dh0=True, workspace=None,
                              stream=None):
    """Gradients of <o, dout> + <hT, dhT> for lin_attn_chunk_fwd_varlen's
    inputs: packed q, k [1,T,H,Dk], v, dout [1,T,H,Dv], gate, beta [1,T,H],
    sequence s at tokens [cu[s], cu[s+1]) (cu_seqlens an int32 GPU tensor of
    nseq + 1 offsets), h0, dhT [nseq,H,Dk,Dv].  Returns float32 (dq, dk, dv,
    dgate, dbeta, dh0) as lin_attn_chunk_bwd does."""
    _need(q, "q")
    if q.dtype not in _DTYPES:
        raise TypeError("q, k, v, dout must be bfloat16 or float32")
    _, T, H, Dk = q.shape
    Dv = v.shape[-1]
    _need(k, "k", q.dtype, (1, T, H, Dk))
    _need(v, "v", q.dtype, (1, T, H, Dv))
    _need(dout, "dout", q.dtype, (1, T, H, Dv))
    _need(gate, "gate", torch.float32, (1, T, H))
    _need(beta, "beta", torch.float32, (1, T, H))
    _need(cu_seqlens, "cu_seqlens", torch.int32)
    nseq = cu_seqlens.numel() - 1
    if cu_seqlens.dim() != 1 or nseq < 0:
        raise ValueError("cu_seqlens must be a 1-D tensor of nseq + 1 offsets")
    if h0 is not None:
        _need(h0, "h0", torch.float32, (nseq, H, Dk, Dv))
    if dhT is not None:
        _need(dhT, "dhT", torch.float32, (nseq, H, Dk, Dv))
    f32 = dict(dtype=torch.float32, device=q.device)
    dq = torch.empty((1, T, H, Dk), **f32)
    dk = torch.empty((1, T, H, Dk), **f32)
    dv = torch.empty((1, T, H, Dv), **f32)
    dgate = torch.empty((1, T, H), **f32)
    dbeta = torch.empty((1, T, H), **f32)
    dh0 = torch.empty((nseq, H, Dk, Dv), **f32) if output_dh0 else None
    nws = lin_attn_chunk_bwd_varlen_workspace_size(T, nseq, H, Dk, Dv, q.dtype)
    if workspace is None and nws > 0:
        workspace = torch.empty(nws, dtype=torch.uint8, device=q.device)
    if workspace is not None:
        _need(workspace, "workspace", torch.uint8)
    N.check(N.lib().lin_attn_chunk_bwd_varlen(
        _ptr(q), _ptr(k), _ptr(v), _ptr(gate), _GATE[gate_mode], float(G), _ptr(beta),
        _ptr(h0), _ptr(dout), _ptr(dhT), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dgate),
        _ptr(dbeta), _ptr(dh0), _ptr(cu_seqlens), nseq, T, H, Dk, Dv, _DTYPES[q.dtype],
        _ptr(workspace), 0 if workspace is None else workspace.numel(), _stream(q, stream)))
    return dq, dk, dv, dgate, dbeta, dh0


def lin_attn_chunk_fwd_varlen_workspace_size(T, nseq, H, Dk, Dv, dtype=torch.bfloat16):
    """Workspace bytes lin_attn_chunk_fwd_varlen needs for these sizes."""
    n = N.lib().lin_attn_chunk_fwd_varlen_workspace_size(T, nseq, H, Dk, Dv, _DTYPES[dtype])
    if n < 0:
        raise N.LinAttnError(N.LA_EINVAL, N.lib().lin_attn_last_error().decode())
    return n


@_on_stream
def lin_attn_chunk_fwd_varlen(q, k, v, gate, beta, cu_seqlens, h0=None, *, gate_mode="log",
                              G=5.0, o=None, hT=None, output_final_state=True,
                              workspace=None, stream=None, raw=False, gate_scale=None,
                              gate_bias=None):
    """Packed sequences: q, k [1,T,H,Dk], v [1,T,H,Dv], gate, beta [1,T,H] hold
    nseq sequences back to back, sequence s at tokens [cu[s], cu[s+1]) with
    cu_seqlens an int32 GPU tensor of nseq + 1 offsets.  Returns o [1,T,H,Dv]
    and the final states hT [nseq,H,Dk,Dv] (None if not requested).  raw=True:
    q, k as they come and `beta` holding logits, and gate_scale / gate_bias
    (lin_attn_chunk_fwd_varlen_raw_affine), as in lin_attn_chunk_fwd.
    bf16 or float32 q, k, v; float32 needs no workspace."""
    _need(q, "q")
    _, T, H, Dk = q.shape
    Dv = v.shape[-1]
    _need(k, "k", q.dtype, (1, T, H, Dk))
    _need(v, "v", q.dtype, (1, T, H, Dv))
    _need(gate, "gate", torch.float32, (1, T, H))
    _need(beta, "beta", torch.float32, (1, T, H))
    _need(cu_seqlens, "cu_seqlens", torch.int32)
    nseq = cu_seqlens.numel() - 1
    if cu_seqlens.dim() != 1 or nseq < 0:
        raise ValueError("cu_seqlens must be a 1-D tensor of nseq + 1 offsets")
    if h0 is not None:
        _need(h0, "h0", torch.float32, (nseq, H, Dk, Dv))
    if o is None:
        o = torch.empty((1, T, H, Dv), dtype=q.dtype, device=q.device)
    _need(o, "o", q.dtype, (1, T, H, Dv))
    if hT is None and output_final_state:
        hT = torch.empty((nseq, H, Dk, Dv), dtype=torch.float32, device=q.device)
    if hT is not None:
        _need(hT, "hT", torch.float32, (nseq, H, Dk, Dv))
    nws = lin_attn_chunk_fwd_varlen_workspace_size(T, nseq, H, Dk, Dv, q.dtype)
    if workspace is None and nws > 0:
        workspace = torch.empty(nws, dtype=torch.uint8, device=q.device)
    if workspace is not None:
        _need(workspace, "workspace", torch.uint8)
    if _affine(gate_scale, gate_bias, raw, gate_mode, H):
        N.check(N.lib().lin_attn_chunk_fwd_varlen_raw_affine(
            _ptr(q), _ptr(k), _ptr(v), _ptr(gate), float(G), _ptr(gate_scale), _ptr(gate_bias),
            _ptr(beta), _ptr(h0), _ptr(o), _ptr(hT), _ptr(cu_seqlens), nseq, T, H, Dk, Dv,
            _DTYPES[q.dtype], _ptr(workspace), 0 if workspace is None else workspace.numel(),
            _stream(q, stream)))
        return o, hT
    fn = N.lib().lin_attn_chunk_fwd_varlen_raw if raw else N.lib().lin_attn_chunk_fwd_varlen
    N.check(fn(
        _ptr(q), _ptr(k), _ptr(v), _ptr(gate), _GATE[gate_mode], float(G), _ptr(beta),
        _ptr(h0), _ptr(o), _ptr(hT), _ptr(cu_seqlens), nseq, T, H, Dk, Dv, _DTYPES[q.dtype],
        _ptr(workspace), 0 if workspace is None else workspace.numel(), _stream(q, stream)))
    return o, hT


def _decode(fn, channel, q, k, v, gate, beta, S, gate_mode, G, o, stream):
    _need(q, "q")
    if q.dtype not in _DTYPES:
        raise TypeError("q, k, v must be bfloat16 or float32")
    B, H, Dk = q.shape
    Dv = v.shape[-1]
    _need(k, "k", q.dtype, (B, H, Dk))
    _need(v, "v", q.dtype, (B, H, Dv))
    _need(gate, "gate", torch.float32, (B, H, Dk) if channel else (B, H))
    _need(beta, "beta", torch.float32, (B, H))
    _need(S, "S", torch.float32, (B, H, Dk, Dv))
    if o is None:
        o = torch.empty((B, H, Dv), dtype=q.dtype, device=q.device)
    _need(o, "o", q.dtype, (B, H, Dv))
    N.check(fn(_ptr(q), _ptr(k), _ptr(v), _ptr(gate), _GATE[gate_mode], float(G), _ptr(beta),
               _ptr(S), _ptr(o), B, H, Dk, Dv, _DTYPES[q.dtype], _stream(q, stream)))
    return o


@_on_stream
def lin_attn_decode_step(q, k, v, gate, beta, S, *, gate_mode="log", G=5.0, o=None,
                         stream=None):
    """Advance S [B,H,Dk,Dv] by one token in place; returns o [B,H,Dv]."""
    return _decode(N.lib().lin_attn_decode_step, False, q, k, v, gate, beta, S, gate_mode, G, o,
                   stream)


@_on_stream
def lin_attn_decode_step_channel(q, k, v, gate, beta, S, *, gate_mode="log", G=5.0, o=None,
                                 stream=None):
    """lin_attn_decode_step with one log-decay per key channel: gate [B,H,Dk]."""
    return _decode(N.lib().lin_attn_decode_step_channel, True, q, k, v, gate, beta, S,
                   gate_mode, G, o, stream)


@_on_stream
def lin_attn_gate(x, G=5.0, out=None, *, stream=None):
    """g = -G * sigmoid(x), float32, same shape as x."""
    _need(x, "x", torch.float32)
    if out is None:
        out = torch.empty_like(x)
    _need(out, "out", torch.float32, tuple(x.shape))
    N.check(N.lib().lin_attn_gate(_ptr(x), float(G), _ptr(out), x.numel(), _stream(x, stream)))
    return out


@_on_stream
def lin_attn_check_inputs(q, k, v, gate, beta, h0=None, *, gate_mode="log", G=5.0,
                          stream=None):
    """Opt-in debug range check of a forward pass's inputs (blocks until done):
    raises LinAttnError with code LA_ERANGE when a q, k, v or h0 element is not
    finite, a beta lies outside [0, 1], or a gate value lies outside [-G, 0]
    (log mode) or is NaN (logit mode).  q, k [B,T,H,Dk], v [B,T,H,Dv], gate
    [B,T,H] or [B,T,H,Dk] (per-channel), beta [B,T,H], h0 [nstate,H,Dk,Dv]."""
    _need(q, "q")
    if q.dtype not in _DTYPES:
        raise TypeError("q, k, v must be bfloat16 or float32")
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    _need(k, "k", q.dtype, (B, T, H, Dk))
    _need(v, "v", q.dtype, (B, T, H, Dv))
    channel = gate.dim() == 4
    _need(gate, "gate", torch.float32, (B, T, H, Dk) if channel else (B, T, H))
    _need(beta, "beta", torch.float32, (B, T, H))
    nstate = 0
    if h0 is not None:
        _need(h0, "h0", torch.float32)
        nstate = h0.shape[0]
        if tuple(h0.shape[1:]) != (H, Dk, Dv):
            raise ValueError(f"h0 must be [nstate, {H}, {Dk}, {Dv}]")
    flags = torch.empty(1, dtype=torch.int32, device=q.device)
    N.check(N.lib().lin_attn_check_inputs(
        _ptr(q), _ptr(k), _ptr(v), _ptr(gate), _GATE[gate_mode], float(G), _ptr(beta), _ptr(h0),
        B * T, nstate, H, Dk, Dv, int(channel), _DTYPES[q.dtype], _ptr(flags),
        _stream(q, stream)))
