"""Helpers for the GPU parity tests: seeded inputs on the device, the same
values handed to the fp64 oracle on the host, and the error measure.

Error measure (per output tensor): max |x - ref| / max |ref| over the whole
tensor, compared with 1e-2 for bf16 q/k/v (fp32 state) and 1e-5 for fp32.
"""

from __future__ import annotations

import sys

import numpy as np
import torch

from chunked_gated_linear_amd import inputs as I
from oracle import c_recurrent as crec
from oracle import linattn_oracle as orc

TOL = {"fp32": 1e-5, "bf16": 1e-2}

# gate-logit distributions: x ~ N(mu, std)
REGIMES = {
    "std": (0.0, 1.0),            # g = -5 sigmoid(N(0,1)): sum of g per tile ~ -40
    "stress_minus": (-4.0, 2.0),  # as written for the 64K stress variant: sum -> 0
    "stress_plus": (4.0, 2.0),    # its stated intent: sum of g per tile -> -80
    "weak": (-8.0, 1.0),          # g ~ -0.0017: state carried over thousands of tokens
    "zero": (0.0, 1.0),           # g == 0 exactly (log mode)
    "min": (0.0, 1.0),            # g == -5 exactly (log mode)
}


def say(msg: str) -> None:
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def host(t: torch.Tensor) -> np.ndarray:
    """Device tensor -> float32 numpy (bf16 -> fp32 is exact)."""
    return t.detach().float().cpu().numpy()


def relerr(x: np.ndarray, ref: np.ndarray) -> float:
    d = np.max(np.abs(np.asarray(x, np.float64) - ref)) if ref.size else 0.0
    m = np.max(np.abs(ref)) if ref.size else 0.0
    return float(d / m) if m > 0 else float(d)


def make_case(B, T, H, Dk, Dv, dtype, regime, mode, h0_std=None, seed=0, dev="cuda"):
    """Device inputs and the oracle's view of them.

    Returns (dev_args, host_args) where dev_args feed lin_attn_chunk_fwd and
    host_args = (q, k, v, g64, beta64, h0_64) are the same values for the oracle.
    """
    mu, sd = REGIMES[regime]
    inp = I.make_inputs(B, T, H, Dk, Dv, dtype=dtype, seed=seed, device=dev,
                        gate_mu=mu, gate_std=sd, h0_std=h0_std)
    x = inp["x"]
    if regime in ("zero", "min"):
        assert mode == "log", "constant gates are given in log mode"
        gate = torch.full_like(x, 0.0 if regime == "zero" else -5.0)
        g64 = host(gate).astype(np.float64)
    elif mode == "logit":
        gate = x
        g64 = orc.bounded_gate(host(x).astype(np.float64))
    else:
        g64_exact = orc.bounded_gate(host(x).astype(np.float64))
        gate = torch.from_numpy(g64_exact.astype(np.float32)).to(dev)
        g64 = host(gate).astype(np.float64)      # the fp32 values the GPU sees
    dev_args = dict(q=inp["q"], k=inp["k"], v=inp["v"], gate=gate, beta=inp["beta"],
                    h0=inp["h0"], gate_mode=mode)
    h0 = None if inp["h0"] is None else host(inp["h0"]).astype(np.float64)
    host_args = (host(inp["q"]), host(inp["k"]), host(inp["v"]), g64,
                 host(inp["beta"]).astype(np.float64), h0)
    return dev_args, host_args


def oracle_full(host_args, workers=16):
    """(o, hT) of the whole problem from the C copy of the fp64 recurrence."""
    q, k, v, g, beta, h0 = host_args
    return crec.recurrent_fwd(q, k, v, g, beta, h0, workers=workers)


def state_bound_before(host_args, b, h, t):
    """Upper bound on |h_t|_2 (state after t tokens): |h0| + sum beta |k| |v|.
    Holds because |exp(g)(I - beta k k^T)|_2 <= 1 when g <= 0 and
    beta |k|^2 <= 2."""
    q, k, v, g, beta, h0 = host_args
    base = 0.0 if h0 is None else float(np.linalg.norm(h0[b, h], 2))
    kk = np.linalg.norm(k[b, :t, h].astype(np.float64), axis=-1)
    vv = np.linalg.norm(v[b, :t, h].astype(np.float64), axis=-1)
    return base + float(np.sum(beta[b, :t, h] * kk * vv))
