"""Pins for the plain-C copies of the oracle's per-channel recurrence and of
its reverse mode (oracle/recurrent.c: oracle_head_fwd_channel,
oracle_head_bwd), which serve the full-size GPU parity tests.

Each C function answers to anchors other than itself: the C adjoint to
central finite differences of the C forward (element by element on tiny
inputs, along random directions on sequences long enough to cross several of
its recomputation segments) and to the pure-decay closed form; the C
per-channel forward to every pin of the NumPy per-channel recurrence (scalar
reduction, pure decay, disjoint keys, write-then-query, the S-orientation
brute force).  Agreement with the NumPy copies is checked on top.
"""

import numpy as np
import pytest

from oracle import c_recurrent as crec
from oracle import linattn_oracle as orc

import test_oracle_channel as tch

NAMES = ("q", "k", "v", "g", "beta", "h0")


def _inputs(B, T, H, Dk, Dv, seed, gate_mu=0.0, unit=True):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, T, H, Dk))
    k = rng.standard_normal((B, T, H, Dk))
    if unit:
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, H, Dv))
    g = orc.bounded_gate(rng.normal(gate_mu, 1.0, (B, T, H)))
    beta = orc.sigmoid(rng.standard_normal((B, T, H)))
    h0 = rng.standard_normal((B, H, Dk, Dv))
    do = rng.standard_normal((B, T, H, Dv))
    dhT = rng.standard_normal((B, H, Dk, Dv))
    return [q, k, v, g, beta, h0], do, dhT


def _loss(args, do, dhT):
    o, hT = crec.recurrent_fwd(*args, workers=1)
    return float((o * do).sum() + (hT * dhT).sum())


def _rel(a, b):
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


@pytest.mark.parametrize("seed,unit", [(0, True), (1, False)])
def test_c_bwd_matches_elementwise_finite_differences(seed, unit):
    args, do, dhT = _inputs(1, 7, 2, 3, 2, seed, unit=unit)
    grads = crec.recurrent_bwd(*args[:5], do, dhT, args[5], workers=1)
    eps = 1e-6
    for i, (name, gr) in enumerate(zip(NAMES, grads)):
        fd = np.zeros_like(args[i])
        for idx in np.ndindex(args[i].shape):
            ap = [x.copy() for x in args]
            am = [x.copy() for x in args]
            ap[i][idx] += eps
            am[i][idx] -= eps
            fd[idx] = (_loss(ap, do, dhT) - _loss(am, do, dhT)) / (2 * eps)
        assert _rel(gr, fd) < 1e-6, name


@pytest.mark.parametrize("gate_mu", [0.0, -8.0])
def test_c_bwd_matches_directional_finite_differences(gate_mu):
    # 150 tokens: three recomputation segments of 64 and a ragged tail; weak
    # decay (gate_mu = -8) keeps the whole history in play
    args, do, dhT = _inputs(2, 150, 2, 8, 6, 10, gate_mu=gate_mu)
    grads = crec.recurrent_bwd(*args[:5], do, dhT, args[5])
    rng = np.random.default_rng(11)
    eps = 1e-6
    for i, name in enumerate(NAMES):
        d = rng.standard_normal(args[i].shape)
        ap = [x.copy() for x in args]
        am = [x.copy() for x in args]
        ap[i] += eps * d
        am[i] -= eps * d
        fd = (_loss(ap, do, dhT) - _loss(am, do, dhT)) / (2 * eps)
        an = float((grads[i] * d).sum())
        assert abs(an - fd) <= 1e-6 * max(1.0, abs(fd)), name


def test_c_bwd_pure_decay_closed_form():
    # beta = 0: o_t = exp(G_t) h0^T q_t, hT = exp(G_T) h0 (G_t the running sum)
    args, do, dhT = _inputs(1, 70, 2, 4, 3, 3)
    q, k, v, g, beta, h0 = args
    beta = np.zeros_like(beta)
    dq, dk, dv, dg, dbeta, dh0 = crec.recurrent_bwd(q, k, v, g, beta, do, dhT, h0)
    e = np.exp(np.cumsum(g, axis=1))
    np.testing.assert_allclose(dq, e[..., None] * np.einsum("bhkv,bthv->bthk", h0, do),
                               rtol=1e-12, atol=1e-14)
    assert np.all(dk == 0) and np.all(dv == 0)
    want_h0 = np.einsum("bth,bthk,bthv->bhkv", e, q, do) + e[:, -1][..., None, None] * dhT
    np.testing.assert_allclose(dh0, want_h0, rtol=1e-12, atol=1e-14)


def test_c_bwd_agrees_with_numpy_adjoint():
    args, do, dhT = _inputs(2, 137, 3, 8, 6, 12, gate_mu=-3.0)
    a = orc.recurrent_bwd(*args[:5], do, dhT, args[5])
    b = crec.recurrent_bwd(*args[:5], do, dhT, args[5])
    for name, x, y in zip(NAMES, a, b):
        assert _rel(y, x) < 1e-12, name


@pytest.mark.parametrize("name", sorted(tch.PINS))
def test_c_channel_pins(name):
    assert tch.PINS[name](lambda *a: crec.recurrent_fwd_channel(*a, workers=1))


def test_c_channel_agrees_with_numpy_on_a_window():
    q, k, v, g, beta, h0 = tch._inputs(2, 60, 3, 8, 6, gate="std", seed=14, h0=True)
    ro, rh = orc.recurrent_fwd_channel(q, k, v, g, beta, h0)
    co, ch = crec.recurrent_fwd_channel(q, k, v, g, beta, h0)
    assert _rel(co, ro) < 1e-12 and _rel(ch, rh) < 1e-12
    # a token window started from the state the first 25 tokens leave behind
    res = crec.recurrent_fwd_channel_c(q, k, v, g, beta, None, t_range=(0, 25))
    mid = np.stack([np.stack([res[(b, h)][1] for h in range(3)]) for b in range(2)])
    res2 = crec.recurrent_fwd_channel_c(q, k, v, g, beta, mid, t_range=(25, 60))
    ro0, _ = orc.recurrent_fwd_channel(q, k, v, g, beta, None)
    for (b, h), (ow, _) in res2.items():
        assert _rel(ow, ro0[b, 25:, h]) < 1e-12
