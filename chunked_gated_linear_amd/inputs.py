"""Seeded synthetic inputs shared by the tests, the benchmark and the oracle runs.

This module draws random numbers and shapes them into the library's layouts.
It holds none of the attention method's arithmetic: it never forms a decay, a
gate, a state update or an output.  Gate inputs are handed out as logits x (the
library's bounded-logit mode turns them into log-decays) or as constants given
by the caller.

Recipe (every draw is float32 N(0, 1) from one torch.Generator seeded with
`seed` on `device`, in this fixed order): q, k, v, x (gate logits), xb (write
strength logits), h0.  q and k are L2-normalised over the head dimension in
float32 and then cast to the element type; beta = 1 / (1 + exp(-xb)) in
float32; x = mu + std * N(0, 1); h0 = h0_std * N(0, 1) (std, not variance).
"""

from __future__ import annotations

import torch

_DT = {"bf16": torch.bfloat16, "fp32": torch.float32}


def _gen(device, seed):
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def _randn(shape, gen, device):
    return torch.randn(*shape, generator=gen, device=device, dtype=torch.float32)


def _unit(x):
    return x / torch.linalg.vector_norm(x, dim=-1, keepdim=True).clamp_min(1e-30)


def make_inputs(B, T, H, Dk, Dv, dtype="bf16", seed=0, device="cpu",
                gate_mu=0.0, gate_std=1.0, h0_std=None):
    """Chunked-forward inputs: dict(q, k, v, x, beta, h0).

    q, k [B,T,H,Dk] and v [B,T,H,Dv] in `dtype`; x, beta [B,T,H] float32;
    h0 [B,H,Dk,Dv] float32 (None when h0_std is None).
    """
    dt = _DT[dtype]
    gen = _gen(device, seed)
    q = _unit(_randn((B, T, H, Dk), gen, device)).to(dt)
    k = _unit(_randn((B, T, H, Dk), gen, device)).to(dt)
    v = _randn((B, T, H, Dv), gen, device).to(dt)
    x = gate_mu + gate_std * _randn((B, T, H), gen, device)
    beta = torch.sigmoid(_randn((B, T, H), gen, device))
    h0 = None
    if h0_std is not None:
        h0 = h0_std * _randn((B, H, Dk, Dv), gen, device)
    return {"q": q.contiguous(), "k": k.contiguous(), "v": v.contiguous(),
            "x": x.contiguous(), "beta": beta.contiguous(), "h0": h0}


def make_channel_gate(B, T, H, Dk, seed=0, device="cpu", mu=0.0, std=1.0):
    """Per-channel gate logits x [B,T,H,Dk] float32, x = mu + std * N(0, 1), from
    their own generator stream (seed + 104729), so the other inputs of the same
    seed are unchanged."""
    gen = _gen(device, seed + 104729)
    return (mu + std * _randn((B, T, H, Dk), gen, device)).contiguous()


def make_upstream_grads(B, T, H, Dk, Dv, dtype="bf16", seed=0, device="cpu", dhT=True):
    """Upstream gradients for the reverse pass: dict(dout [B,T,H,Dv] in
    `dtype`, dhT [B,H,Dk,Dv] float32 or None), N(0,1) entries."""
    gen = _gen(device, seed + 7919)
    dout = _randn((B, T, H, Dv), gen, device).to(_DT[dtype]).contiguous()
    dh = _randn((B, H, Dk, Dv), gen, device).contiguous() if dhT else None
    return {"dout": dout, "dhT": dh}


def make_decode_inputs(B, H, Dk, Dv, dtype="bf16", seed=0, device="cpu",
                       steps=1, S_std=0.02, gate_mu=0.0, gate_std=1.0):
    """Decode inputs for `steps` consecutive tokens: dict(q, k, v, x, beta, S).

    q, k [steps,B,H,Dk], v [steps,B,H,Dv] in `dtype`; x, beta [steps,B,H]
    float32; S [B,H,Dk,Dv] float32 = S_std * N(0, 1).
    """
    dt = _DT[dtype]
    gen = _gen(device, seed)
    q = _unit(_randn((steps, B, H, Dk), gen, device)).to(dt)
    k = _unit(_randn((steps, B, H, Dk), gen, device)).to(dt)
    v = _randn((steps, B, H, Dv), gen, device).to(dt)
    x = gate_mu + gate_std * _randn((steps, B, H), gen, device)
    beta = torch.sigmoid(_randn((steps, B, H), gen, device))
    S = S_std * _randn((B, H, Dk, Dv), gen, device)
    return {"q": q.contiguous(), "k": k.contiguous(), "v": v.contiguous(),
            "x": x.contiguous(), "beta": beta.contiguous(), "S": S.contiguous()}


# Named workloads.  Shapes follow the pages' context ladder (8K, 64K, 256K, 1M
# tokens) and 16-token tiles; the value distributions are the recipe above.
WORKLOADS = {
    "tiny_fp32": dict(B=1, H=2, T=256, Dk=64, Dv=64, dtype="fp32"),
    "train_8k": dict(B=4, H=16, T=8192, Dk=128, Dv=128, dtype="bf16"),
    "long_64k": dict(B=1, H=16, T=65536, Dk=128, Dv=128, dtype="bf16"),
    "long_256k": dict(B=1, H=16, T=262144, Dk=128, Dv=128, dtype="bf16"),
    "million_1m": dict(B=1, H=8, T=1048576, Dk=128, Dv=128, dtype="bf16", h0_std=0.02),
}
DECODE_WORKLOAD = dict(B=256, H=32, Dk=128, Dv=128, dtype="bf16", steps=1000)


# Packed prefill batch (serving): nseq request lengths drawn log-normally
# (median T / nseq, sigma 1), then scaled and rounded to sum to T exactly with
# every request at least one token.
VARLEN_WORKLOAD = dict(nseq=64, T=65536, H=16, Dk=128, Dv=128, dtype="bf16")


def varlen_lengths(nseq, T, seed=0):
    """Seeded request lengths (a list of nseq ints >= 1 summing to T)."""
    import numpy as np
    if nseq <= 0 or T < nseq:
        raise ValueError("need 1 <= nseq <= T")
    rng = np.random.default_rng(seed)
    w = rng.lognormal(mean=0.0, sigma=1.0, size=nseq)
    raw = 1 + (T - nseq) * w / w.sum()
    lengths = np.floor(raw).astype(np.int64)
    short = T - int(lengths.sum())
    order = np.argsort(-(raw - lengths))            # largest remainders first
    lengths[order[:short]] += 1
    return [int(x) for x in lengths]
