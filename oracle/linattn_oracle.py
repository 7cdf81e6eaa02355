"""Plain, slow, fp64 CPU oracle for gated delta-rule linear attention.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the package smoke check and the
benchmark's CPU-baseline leg may import or run anything in this directory.  The
product path (the HIP library and its Python binding) never calls it, shares no
code with it, and fails loudly when its own native library is missing.

What is computed, and where the pages say so
--------------------------------------------
Pages cited (by title and section):
  [DD]  "Deep Dive: The Next Generation of Ultra-Long Context Sparse MoE LLMs",
        sec. 3.2 (chunked parallelism, 16-token tiles, intra-chunk parallel /
        inter-chunk recursion) and sec. 3.3 (bounded decay, g_min = -5).
  [CT]  "Core Technologies Behind Ultra-Long-Context Sparse MoE Large Models",
        sec. 2.1 (fixed-size matrix state, per-token decay, diagonal and
        off-diagonal tiles) and sec. 2.2 (scaled-sigmoid log-decay).
  [TS]  "How Trillion-Scale Sparse MoE Models Achieve Million-Token Long
        Context", sec. 3.1 (states propagate between chunks) and sec. 3.2
        (g = g_min * sigmoid(u), exp(-g) in [1, ~148]).
  [EV]  "Evaluating Next-Gen Sparse MoE and Long-Context LLMs", sec. 2 item 2
        (incremental linear attention: a fixed-size matrix state updated token
        by token with a delta rule; new information written, old information
        diluted by a data-dependent decay) and item 3 (bounded log-decay).

The pages name the delta rule and the data-dependent decay but do not print the
update.  The reading taken here is the plain gated delta rule, per (batch,
head), with a scalar log-decay g_t and a scalar write strength beta_t:

    S_t = exp(g_t) * S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T
    o_t = S_t q_t

S_t is d_v x d_k.  Every array here stores its transpose h_t = S_t^T
(d_k rows, d_v columns), so the same update reads

    h_t = exp(g_t) (h_{t-1} - beta_t k_t (k_t^T h_{t-1})) + beta_t k_t v_t^T
    o_t = h_t^T q_t

Decay multiplies the erased old state; the new write is not decayed at its own
step; the output reads the state after the step's update; there is no query
scale.  The log-decay is the bounded parameterisation g = -G * sigmoid(x) with
G = 5 ([DD] 3.3, [CT] 2.2, [TS] 3.2, [EV] 2.3).

Functions and their pins (the tests that tie each to something other than
itself are in tests/test_oracle.py):
  bounded_gate     values printed on the pages (exp(-5) ~ 0.0067, exp(5) ~ 148,
                   g in [-5, 0]) and the sigmoid reflection identity.
  bounded_gate_affine
                   closed forms at x = 0 (g = -G sigmoid(b)) and at a scaled
                   logit (sigmoid(ln 3) = 3/4), the reflection a, b -> -a, -b,
                   and per-head broadcast checked head by head.
  recurrent_fwd    a hand-worked example, a pure-Python brute force in the
                   S orientation, closed forms (pure decay, orthogonal keys =
                   masked gated linear attention), invariants (identity step,
                   write-then-query, split invariance, linearity, norm bound).
  decode_step      equals recurrent_fwd applied one token at a time.
  prepare_inputs   unit norms, directions kept (q / |q| times |q| gives q back),
                   zero vectors kept, sigmoid values checked against closed forms.
  recurrent_fwd_varlen
                   packed sequences: a closed form at every boundary (a
                   sequence whose tokens neither write nor decay returns its own
                   h0 exactly, whatever came before it; a planted carry-over
                   fails it), equal lengths equal the batch axis, and the C
                   copy agrees on mixed lengths with empty sequences.
  chunked_fwd      equals recurrent_fwd for chunk sizes 1, 3, 16 and 32 (two
                   independent formulations of the same definition).
  recurrent_bwd    central finite differences of recurrent_fwd, element by
                   element on tiny inputs and along random directions on larger
                   ones; closed forms for pure decay (beta = 0) and for
                   mutually orthogonal keys (masked gated linear attention);
                   the zero-upstream case.
  bounded_gate_bwd central finite differences of bounded_gate.
  recurrent_fwd_channel
                   per-channel gate: equals recurrent_fwd when every channel
                   has the same g; closed forms for pure decay (beta = 0) and
                   for keys of disjoint support (masked gated linear attention
                   with a per-channel decay); write-then-query returns v
                   exactly under any per-channel decay (this fixes the order
                   decay -> erase -> write); a pure-Python brute force in the
                   S orientation; planted mistakes (decay on the value axis,
                   erase before decay, decayed write, reversed channels) fail.
  chunked_fwd_channel
                   equals recurrent_fwd_channel for chunk sizes 1, 3, 16; its
                   in-tile reciprocals stay finite at the bound.
  decode_step_channel
                   steps applied one token at a time equal recurrent_fwd_channel
                   over the same tokens.
  recurrent_fwd_channel_varlen
                   packed sequences with a per-channel gate: the boundary closed
                   form (a sequence whose tokens neither write nor decay returns
                   its own h0, and outputs h0^T q_t, exactly, whatever precedes
                   it), equal lengths equal the batch axis.
Every function is pinned; none is "parity unpinned".

Layouts (row-major, as the library uses them):
  q, k  [B, T, H, Dk]    v, o  [B, T, H, Dv]    g, beta  [B, T, H]
  h0, hT  [B, H, Dk, Dv]  (h = S^T)
Everything is computed in float64 from the exact values given.
"""

from __future__ import annotations

import multiprocessing as _mp
import os

import numpy as np

__all__ = [
    "bounded_gate",
    "recurrent_fwd",
    "decode_step",
    "chunked_fwd",
    "recurrent_fwd_heads",
    "recurrent_fwd_varlen",
    "prepare_inputs",
    "recurrent_bwd",
    "bounded_gate_bwd",
    "recurrent_fwd_channel",
    "chunked_fwd_channel",
    "decode_step_channel",
    "recurrent_fwd_channel_varlen",
]


def _f64(a):
    return np.asarray(a, dtype=np.float64)


# ----------------------------------------------------------------------------
# Bounded log-decay.  [DD] 3.3, [CT] 2.2, [TS] 3.2, [EV] 2.3: the log-decay is
# g_min * sigmoid(.) with g_min = -5, so g lies in [-5, 0] and exp(g) in
# [exp(-5), 1].
# ----------------------------------------------------------------------------
def sigmoid(x):
    """Logistic function 1 / (1 + exp(-x)) in fp64, evaluated without overflow."""
    x = _f64(x)
    out = np.empty_like(x)
    pos = x >= 0
    out[pos] = 1.0 / (1.0 + np.exp(-x[pos]))
    ex = np.exp(x[~pos])
    out[~pos] = ex / (1.0 + ex)
    return out


def bounded_gate(x, G: float = 5.0):
    """g = -G * sigmoid(x), the scaled-sigmoid log-decay ([DD] 3.3, [CT] 2.2)."""
    return -float(G) * sigmoid(x)


def bounded_gate_affine(x, a=None, b=None, G: float = 5.0):
    """g = -G * sigmoid(a_h * x + b_h): the bounded log-decay of an affine
    function of the input ([EV] 2 item 3, [CT] 2.2), with one scale a_h and one
    shift b_h per head.  x has heads on its last axis; a and b are [H] arrays
    (None: a = 1, b = 0)."""
    x = _f64(x)
    H = x.shape[-1]
    a = np.ones(H) if a is None else _f64(a).reshape(H)
    b = np.zeros(H) if b is None else _f64(b).reshape(H)
    return bounded_gate(a * x + b, G)


# ----------------------------------------------------------------------------
# Token-by-token recurrence ([EV] sec. 2 item 2: fixed-size matrix state,
# delta-rule write, data-dependent decay).  This is the definition; it is the
# oracle for every parity test.
# ----------------------------------------------------------------------------
def recurrent_fwd(q, k, v, g, beta, h0=None):
    """Run the gated delta rule over T tokens for every (batch, head).

    Returns (o [B,T,H,Dv], hT [B,H,Dk,Dv]) in float64.  h0 = None means a zero
    initial state.
    """
    q, k, v, g, beta = map(_f64, (q, k, v, g, beta))
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    h = np.zeros((B, H, Dk, Dv)) if h0 is None else _f64(h0).copy()
    o = np.empty((B, T, H, Dv))
    for t in range(T):
        kt = k[:, t]                                        # [B,H,Dk]
        vt = v[:, t]                                        # [B,H,Dv]
        a = np.exp(g[:, t])[:, :, None, None]               # decay exp(g_t)
        b = beta[:, t][:, :, None, None]                    # write strength
        kh = np.einsum("bhk,bhkv->bhv", kt, h)              # k_t^T h_{t-1}
        erased = h - b * kt[:, :, :, None] * kh[:, :, None, :]
        h = a * erased + b * kt[:, :, :, None] * vt[:, :, None, :]
        o[:, t] = np.einsum("bhk,bhkv->bhv", q[:, t], h)    # h_t^T q_t
    return o, h


def prepare_inputs(q, k, x_beta):
    """Input preparation of the raw-input forward pass: q and k L2-normalised
    over their last axis (a zero vector stays zero) and beta = sigmoid(x_beta),
    in float64.  The pages' configurations draw q and k from N(0,1) and
    normalise them per head and token; the raw entry point does this inside the
    pass."""
    q, k, x_beta = map(_f64, (q, k, x_beta))

    def unit(a):
        n = np.linalg.norm(a, axis=-1, keepdims=True)
        return np.divide(a, n, out=np.zeros_like(a), where=n > 0)

    return unit(q), unit(k), sigmoid(x_beta)


def recurrent_fwd_varlen(q, k, v, g, beta, cu_seqlens, h0=None):
    """Packed sequences, as a serving batch prefills several requests back to
    back ("Evaluating Next-Gen Sparse MoE and Long-Context LLMs", sec. 4):
    sequence s is tokens [cu[s], cu[s+1]) of the packed arrays q, k [1,T,H,Dk],
    v [1,T,H,Dv], g, beta [1,T,H].  It starts from h0[s] (zeros when h0 is
    None) and its recurrence reads no other sequence's tokens or state.

    Returns (o [1,T,H,Dv], hT [N,H,Dk,Dv]) in float64; an empty sequence has
    hT = its initial state.
    """
    q, k, v, g, beta = map(_f64, (q, k, v, g, beta))
    cu = [int(x) for x in cu_seqlens]
    _, T, H, Dk = q.shape
    Dv = v.shape[-1]
    N = len(cu) - 1
    if N < 0 or cu[0] != 0 or cu[-1] != T or any(b < a for a, b in zip(cu, cu[1:])):
        raise ValueError("cu_seqlens must run from 0 to T without decreasing")
    o = np.empty((1, T, H, Dv))
    hT = np.zeros((N, H, Dk, Dv))
    for s in range(N):
        a, b = cu[s], cu[s + 1]
        init = None if h0 is None else _f64(h0)[s:s + 1]
        if b > a:
            o_s, h_s = recurrent_fwd(q[:, a:b], k[:, a:b], v[:, a:b], g[:, a:b], beta[:, a:b], init)
            o[:, a:b] = o_s
            hT[s] = h_s[0]
        elif init is not None:
            hT[s] = init[0]
    return o, hT


def bounded_gate_bwd(x, dg, G: float = 5.0):
    """Gradient through g = -G * sigmoid(x): dx = -G * s (1 - s) * dg."""
    s = sigmoid(x)
    return -float(G) * s * (1.0 - s) * _f64(dg)


# ----------------------------------------------------------------------------
# Reverse mode of the recurrence, for training ("Core Technologies Behind
# Ultra-Long-Context Sparse MoE Large Models", sec. 2.3: the bounded decay is
# chosen for BF16 training; the pages print no backward pass, so this is the
# adjoint of recurrent_fwd, derived by hand).  With a = exp(g_t), b = beta_t,
# c = k_t^T h_{t-1} and e = h_{t-1} - b k_t c^T (the erased old state), one
# step is h_t = a e + b k_t v_t^T and o_t = h_t^T q_t.  Walking t from T-1 down
# to 0 with dh = dL/dh_t (starting from dhT):
#     dh   += q_t do_t^T                 dq_t  = h_t do_t
#     dg_t  = a <dh, e>                  dv_t  = b dh^T k_t
#     de    = a dh
#     dbeta_t = k_t^T dh v_t - (k_t^T de) . c
#     dk_t  = b dh v_t - b (de c + h_{t-1} (de^T k_t))
#     dh_{t-1} = de - b k_t (k_t^T de)
# and dh0 = dh after the last step.  States are kept every `seg` tokens and
# recomputed inside a segment, which changes nothing in the arithmetic.
# ----------------------------------------------------------------------------
def recurrent_bwd(q, k, v, g, beta, do, dhT=None, h0=None, seg: int = 64):
    """Gradients of L = <o, do> + <hT, dhT> with respect to every input.

    Returns dq [B,T,H,Dk], dk [B,T,H,Dk], dv [B,T,H,Dv], dg [B,T,H],
    dbeta [B,T,H], dh0 [B,H,Dk,Dv], all float64.  dhT = None means zero.
    """
    q, k, v, g, beta, do = map(_f64, (q, k, v, g, beta, do))
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    seg = max(1, int(seg))
    h = np.zeros((B, H, Dk, Dv)) if h0 is None else _f64(h0).copy()
    checkpoints = []
    for s0 in range(0, T, seg):                 # state before each segment
        checkpoints.append(h.copy())
        s1 = min(T, s0 + seg)
        _, h = recurrent_fwd(q[:, s0:s1], k[:, s0:s1], v[:, s0:s1], g[:, s0:s1],
                             beta[:, s0:s1], h)
    dq, dk = np.zeros_like(q), np.zeros_like(k)
    dv = np.zeros_like(v)
    dg, dbeta = np.zeros_like(g), np.zeros_like(beta)
    dh = np.zeros((B, H, Dk, Dv)) if dhT is None else _f64(dhT).copy()
    for si in range(len(checkpoints) - 1, -1, -1):
        s0 = si * seg
        s1 = min(T, s0 + seg)
        states = [checkpoints[si]]              # h_{s0-1}, h_{s0}, ..., h_{s1-1}
        for t in range(s0, s1):
            _, hn = recurrent_fwd(q[:, t:t + 1], k[:, t:t + 1], v[:, t:t + 1], g[:, t:t + 1],
                                  beta[:, t:t + 1], states[-1])
            states.append(hn)
        for t in range(s1 - 1, s0 - 1, -1):
            h_prev, h_t = states[t - s0], states[t - s0 + 1]
            kt, vt, qt, dot = k[:, t], v[:, t], q[:, t], do[:, t]
            a = np.exp(g[:, t])[:, :, None, None]
            b = beta[:, t][:, :, None, None]
            dh = dh + qt[:, :, :, None] * dot[:, :, None, :]
            dq[:, t] = np.einsum("bhkv,bhv->bhk", h_t, dot)
            c = np.einsum("bhk,bhkv->bhv", kt, h_prev)
            e = h_prev - b * kt[:, :, :, None] * c[:, :, None, :]
            dg[:, t] = a[:, :, 0, 0] * np.einsum("bhkv,bhkv->bh", dh, e)
            dv[:, t] = b[:, :, :, 0] * np.einsum("bhkv,bhk->bhv", dh, kt)
            de = a * dh
            kde = np.einsum("bhk,bhkv->bhv", kt, de)            # k_t^T de
            dbeta[:, t] = (np.einsum("bhk,bhkv,bhv->bh", kt, dh, vt)
                           - np.einsum("bhv,bhv->bh", kde, c))
            dk[:, t] = b[:, :, :, 0] * (np.einsum("bhkv,bhv->bhk", dh, vt)
                                        - np.einsum("bhkv,bhv->bhk", de, c)
                                        - np.einsum("bhkv,bhv->bhk", h_prev, kde))
            dh = de - b * kt[:, :, :, None] * kde[:, :, None, :]
    return dq, dk, dv, dg, dbeta, dh


def decode_step(q, k, v, g, beta, S):
    """One token of the same recurrence for every (batch, head).

    q, k [B,H,Dk]; v [B,H,Dv]; g, beta [B,H]; S [B,H,Dk,Dv] (the state, stored as
    h = S^T).  Returns (o [B,H,Dv], S_new); the input S is not modified.
    """
    q, k, v, g, beta, S = map(_f64, (q, k, v, g, beta, S))
    o, hT = recurrent_fwd(q[:, None], k[:, None], v[:, None], g[:, None],
                          beta[:, None], S)
    return o[:, 0], hT


# ----------------------------------------------------------------------------
# Chunked (tiled) form.  [DD] 3.2: tiles of 16 tokens, parallel inside a tile,
# recursive between tiles.  [CT] 2.1: diagonal blocks carry the in-tile
# token interactions, off-diagonal blocks the "historical state -> current
# token" flow.  [TS] 3.1: the recurrent state propagates between chunks.
#
# Derived from the recurrence (the pages do not print it).  Inside a chunk
# that starts from state H, with G_t the in-chunk running sum of g and
# gamma_t = exp(G_t), write u_t = beta_t (v_t - exp(g_t) h_{t-1}^T k_t).  Then
# h_t = exp(g_t) h_{t-1} + k_t u_t^T, and stacking the u_t of the chunk:
#     (I + A) U = diag(beta) V - diag(beta*gamma) K H,
#     A[t, s] = beta_t exp(G_t - G_s) k_t . k_s   for s < t (0 otherwise),
#     O       = diag(gamma) Q H + P U,  P[t, s] = exp(G_t - G_s) q_t . k_s, s <= t
#     H_next  = gamma_C H + K~^T U,     K~[s]   = exp(G_C - G_s) k_s.
# Only exp of a non-positive number is formed.  The triangular system is solved
# with a library solver (one step, no blocking of our own).
# ----------------------------------------------------------------------------
def chunked_fwd(q, k, v, g, beta, h0=None, chunk: int = 16):
    """Same result as recurrent_fwd, computed chunk by chunk in fp64."""
    q, k, v, g, beta = map(_f64, (q, k, v, g, beta))
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    C = int(chunk)
    # (B,T,H,.) -> (B,H,T,.)
    qh, kh, vh = (np.moveaxis(a, 2, 1) for a in (q, k, v))
    gh, bh = np.moveaxis(g, 2, 1), np.moveaxis(beta, 2, 1)
    Hs = np.zeros((B, H, Dk, Dv)) if h0 is None else _f64(h0).copy()
    o = np.empty((B, H, T, Dv))
    for c0 in range(0, T, C):
        c1 = min(T, c0 + C)
        n = c1 - c0
        Q, K, V = qh[:, :, c0:c1], kh[:, :, c0:c1], vh[:, :, c0:c1]
        beta_c = bh[:, :, c0:c1]
        Gc = np.cumsum(gh[:, :, c0:c1], axis=-1)            # in-chunk cumsum
        gam = np.exp(Gc)
        diff = Gc[..., :, None] - Gc[..., None, :]          # G_t - G_s
        lower_strict = np.tril(np.ones((n, n)), -1)
        lower_incl = np.tril(np.ones((n, n)), 0)
        dec = np.exp(np.where(lower_incl > 0, diff, -np.inf))
        KK = K @ np.swapaxes(K, -1, -2)
        QK = Q @ np.swapaxes(K, -1, -2)
        A = beta_c[..., :, None] * dec * KK * lower_strict
        P = dec * QK
        rhs = beta_c[..., None] * V - (beta_c * gam)[..., None] * (K @ Hs)
        U = np.linalg.solve(np.eye(n) + A, rhs)
        o[:, :, c0:c1] = gam[..., None] * (Q @ Hs) + P @ U
        ktil = np.exp(Gc[..., -1:] - Gc)[..., None] * K
        Hs = np.exp(Gc[..., -1])[..., None, None] * Hs + np.swapaxes(ktil, -1, -2) @ U
    return np.moveaxis(o, 1, 2), Hs


# ----------------------------------------------------------------------------
# Runner over independent (batch, head) streams on host cores.  Each stream is
# the same recurrent_fwd on a [1, T, 1, .] slice; the streams share nothing,
# so a process pool gives the same numbers as one call.
# ----------------------------------------------------------------------------
_POOL_DATA = None


def _run_one(args):
    b, h, t0, t1 = args
    q, k, v, g, beta, h0 = _POOL_DATA
    sl = (slice(b, b + 1), slice(t0, t1), slice(h, h + 1))
    init = None if h0 is None else h0[b:b + 1, h:h + 1]
    o, hT = recurrent_fwd(q[sl], k[sl], v[sl], g[sl], beta[sl], init)
    return o[0, :, 0], hT[0, 0]


def recurrent_fwd_heads(q, k, v, g, beta, h0=None, heads=None, t_range=None,
                        workers: int | None = None):
    """recurrent_fwd on selected (b, h) streams, optionally over tokens [t0, t1).

    heads: list of (b, h); default all.  t_range: (t0, t1) with h0 taken as the
    state before token t0.  Returns {(b, h): (o [t1-t0, Dv], hT [Dk, Dv])}.
    workers: processes to use (default: all cores, capped by the stream count).
    """
    global _POOL_DATA
    B, T, H, _ = np.shape(q)
    if heads is None:
        heads = [(b, h) for b in range(B) for h in range(H)]
    t0, t1 = (0, T) if t_range is None else t_range
    jobs = [(b, h, t0, t1) for (b, h) in heads]
    if workers is None:
        workers = os.cpu_count() or 1
    workers = max(1, min(int(workers), len(jobs)))
    _POOL_DATA = (q, k, v, g, beta, h0)
    try:
        if workers == 1:
            res = [_run_one(j) for j in jobs]
        else:
            ctx = _mp.get_context("fork")
            with ctx.Pool(workers) as pool:
                res = pool.map(_run_one, jobs, chunksize=1)
    finally:
        _POOL_DATA = None
    return {(b, h): r for (b, h, _, _), r in zip(jobs, res)}


# ----------------------------------------------------------------------------
# Per-channel gate.  The pages call the decay "per-token decay factors"
# ([CT] 2.1) and bound the log-decay elementwise ([DD] 3.3, [TS] 3.2); with one
# log-decay per key channel, g_t in [-G, 0]^{d_k}, the scalar exp(g_t) acting
# on S_{t-1} becomes the diagonal matrix D_t = diag(exp(g_t)) on the key side
# of S_{t-1}:
#     S_t = S_{t-1} D_t (I - beta_t k_t k_t^T) + beta_t v_t k_t^T
# i.e. in the h = S^T orientation, with d_t = D_t h_{t-1} (row c of h_{t-1}
# scaled by exp(g_t[c])):
#     h_t = d_t - beta_t k_t (k_t^T d_t) + beta_t k_t v_t^T,   o_t = h_t^T q_t.
# The decay acts first, the delta-rule erase and write then act on the decayed
# state; with all channels equal this is recurrent_fwd.
# ----------------------------------------------------------------------------
def recurrent_fwd_channel(q, k, v, g, beta, h0=None):
    """Gated delta rule with one log-decay per key channel, token by token.

    g is [B, T, H, Dk]; everything else as recurrent_fwd.  Returns
    (o [B,T,H,Dv], hT [B,H,Dk,Dv]) in float64.
    """
    q, k, v, g, beta = map(_f64, (q, k, v, g, beta))
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    h = np.zeros((B, H, Dk, Dv)) if h0 is None else _f64(h0).copy()
    o = np.empty((B, T, H, Dv))
    for t in range(T):
        kt = k[:, t]
        vt = v[:, t]
        b = beta[:, t][:, :, None, None]
        d = np.exp(g[:, t])[:, :, :, None] * h                   # D_t h_{t-1}
        kd = np.einsum("bhk,bhkv->bhv", kt, d)                  # k_t^T d_t
        h = d - b * kt[:, :, :, None] * kd[:, :, None, :] + b * kt[:, :, :, None] * vt[:, :, None, :]
        o[:, t] = np.einsum("bhk,bhkv->bhv", q[:, t], h)
    return o, h


# Chunked form of the per-channel recurrence, as the pages organise it: inside
# a 16-token tile the per-channel cumulative decay Gam_t = exp(G_t) (G_t the
# in-tile running sum of g_t, a vector) no longer factors out of the dot
# products, so the tile products take the decay into their operands -- queries
# and keys scaled by Gam_t, keys divided by Gam_s -- and the reciprocal 1/Gam_s
# appears ([CT] 2.1 and 2.3, [TS] 3.1 and 3.2: the bounded gate keeps it at most
# exp(16 G) = exp(80) in a 16-token tile, inside the float range).  Derived
# from the recurrence: with H the state entering the tile and
# u_t = beta_t (v_t - d_t^T k_t),
#     (I + A) U = diag(beta) (V - (K o Gam) H),
#     A[t, s] = beta_t (k_t o Gam_t) . (k_s / Gam_s)   (s < t),
#     O       = (Q o Gam) H + P U,   P[t, s] = (q_t o Gam_t) . (k_s / Gam_s)  (s <= t),
#     H_next  = diag(Gam_C) H + (K o (Gam_C / Gam))^T U.
def chunked_fwd_channel(q, k, v, g, beta, h0=None, chunk: int = 16):
    """Same result as recurrent_fwd_channel, tile by tile in fp64."""
    q, k, v, g, beta = map(_f64, (q, k, v, g, beta))
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    C = int(chunk)
    qh, kh, vh, gh = (np.moveaxis(a, 2, 1) for a in (q, k, v, g))   # (B,H,T,.)
    bh = np.moveaxis(beta, 2, 1)
    Hs = np.zeros((B, H, Dk, Dv)) if h0 is None else _f64(h0).copy()
    o = np.empty((B, H, T, Dv))
    for c0 in range(0, T, C):
        c1 = min(T, c0 + C)
        n = c1 - c0
        Q, K, V = qh[:, :, c0:c1], kh[:, :, c0:c1], vh[:, :, c0:c1]
        beta_c = bh[:, :, c0:c1]
        Gc = np.cumsum(gh[:, :, c0:c1], axis=2)                   # (B,H,n,Dk)
        gam = np.exp(Gc)
        inv = np.exp(-Gc)                                          # 1 / Gam_s
        Kg, Qg, Ki = K * gam, Q * gam, K * inv
        lower_strict = np.tril(np.ones((n, n)), -1)
        lower_incl = np.tril(np.ones((n, n)), 0)
        A = beta_c[..., :, None] * (Kg @ np.swapaxes(Ki, -1, -2)) * lower_strict
        P = (Qg @ np.swapaxes(Ki, -1, -2)) * lower_incl
        rhs = beta_c[..., None] * (V - Kg @ Hs)
        U = np.linalg.solve(np.eye(n) + A, rhs)
        o[:, :, c0:c1] = Qg @ Hs + P @ U
        gC = gam[:, :, -1]                                         # (B,H,Dk)
        Kd = K * (gC[:, :, None, :] * inv)
        Hs = gC[..., None] * Hs + np.swapaxes(Kd, -1, -2) @ U
    return np.moveaxis(o, 1, 2), Hs


def decode_step_channel(q, k, v, g, beta, S):
    """One token of the per-channel recurrence for every (batch, head).

    q, k [B,H,Dk]; v [B,H,Dv]; g [B,H,Dk]; beta [B,H]; S [B,H,Dk,Dv] (h = S^T).
    Returns (o [B,H,Dv], S_new); the input S is not modified.
    """
    q, k, v, g, beta, S = map(_f64, (q, k, v, g, beta, S))
    o, hT = recurrent_fwd_channel(q[:, None], k[:, None], v[:, None], g[:, None],
                                  beta[:, None], S)
    return o[:, 0], hT


def recurrent_fwd_channel_varlen(q, k, v, g, beta, cu_seqlens, h0=None):
    """Packed sequences with a per-channel gate: sequence s is tokens
    [cu[s], cu[s+1]) of q, k [1,T,H,Dk], v [1,T,H,Dv], g [1,T,H,Dk], beta [1,T,H];
    it starts from h0[s] (zeros when h0 is None) and reads nothing of another
    sequence.  Returns (o [1,T,H,Dv], hT [N,H,Dk,Dv]) in float64."""
    q, k, v, g, beta = map(_f64, (q, k, v, g, beta))
    cu = [int(x) for x in cu_seqlens]
    _, T, H, Dk = q.shape
    Dv = v.shape[-1]
    N = len(cu) - 1
    if N < 0 or cu[0] != 0 or cu[-1] != T or any(b < a for a, b in zip(cu, cu[1:])):
        raise ValueError("cu_seqlens must run from 0 to T without decreasing")
    o = np.empty((1, T, H, Dv))
    hT = np.zeros((N, H, Dk, Dv))
    for s in range(N):
        a, b = cu[s], cu[s + 1]
        init = None if h0 is None else _f64(h0)[s:s + 1]
        if b > a:
            o_s, h_s = recurrent_fwd_channel(q[:, a:b], k[:, a:b], v[:, a:b], g[:, a:b],
                                             beta[:, a:b], init)
            o[:, a:b] = o_s
            hT[s] = h_s[0]
        elif init is not None:
            hT[s] = init[0]
    return o, hT
