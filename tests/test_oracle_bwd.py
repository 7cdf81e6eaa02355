"""Pins for the oracle's reverse mode (recurrent_bwd, bounded_gate_bwd).

Anchors other than the backward code itself: central finite differences of the
forward recurrence (element by element on tiny inputs, along random directions
on larger ones), closed forms (pure decay when beta = 0; masked gated linear
attention when the keys are mutually orthogonal and h0 = 0), and zero upstream
gradients.  test_bwd_mutants_are_caught plants plausible mistakes in copies of
the backward and checks that each fails the finite-difference pin.
"""

import inspect
import textwrap

import numpy as np
import pytest

from oracle import linattn_oracle as orc

NAMES = ("q", "k", "v", "g", "beta", "h0")


def _inputs(B, T, H, Dk, Dv, seed, unit=True, gate_mu=0.0):
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
    o, hT = orc.recurrent_fwd(*args)
    return float((o * do).sum() + (hT * dhT).sum())


def _fd_elementwise(args, do, dhT, eps=1e-6):
    out = []
    for i, a in enumerate(args):
        fd = np.zeros_like(a)
        for idx in np.ndindex(a.shape):
            ap = [x.copy() for x in args]
            am = [x.copy() for x in args]
            ap[i][idx] += eps
            am[i][idx] -= eps
            fd[idx] = (_loss(ap, do, dhT) - _loss(am, do, dhT)) / (2 * eps)
        out.append(fd)
    return out


def _rel(a, b):
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


@pytest.mark.parametrize("seed,unit,seg", [(0, True, 3), (1, False, 64), (2, True, 1)])
def test_bwd_matches_elementwise_finite_differences(seed, unit, seg):
    args, do, dhT = _inputs(1, 7, 2, 3, 2, seed, unit=unit)
    grads = orc.recurrent_bwd(*args[:5], do, dhT, args[5], seg=seg)
    fds = _fd_elementwise(args, do, dhT)
    for name, gr, fd in zip(NAMES, grads, fds):
        assert _rel(gr, fd) < 1e-6, name


@pytest.mark.parametrize("gate_mu", [0.0, -8.0, 4.0])
def test_bwd_matches_directional_finite_differences(gate_mu):
    # longer sequence, several 16-token tiles and a ragged tail; weak decay
    # (gate_mu = -8) keeps the whole history in play
    args, do, dhT = _inputs(2, 37, 2, 8, 6, 10, gate_mu=gate_mu)
    grads = orc.recurrent_bwd(*args[:5], do, dhT, args[5], seg=16)
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


def test_bwd_pure_decay_closed_form():
    # beta = 0: o_t = exp(G_t) h0^T q_t and hT = exp(G_T) h0, with G_t the
    # running sum of g up to and including t
    args, do, dhT = _inputs(1, 12, 2, 4, 3, 3)
    q, k, v, g, beta, h0 = args
    beta = np.zeros_like(beta)
    dq, dk, dv, dg, dbeta, dh0 = orc.recurrent_bwd(q, k, v, g, beta, do, dhT, h0)
    G = np.cumsum(g, axis=1)                                    # [B,T,H]
    e = np.exp(G)
    np.testing.assert_allclose(dq, e[..., None] * np.einsum("bhkv,bthv->bthk", h0, do), rtol=1e-12, atol=1e-14)
    assert np.all(dk == 0) and np.all(dv == 0)
    want_h0 = np.einsum("bth,bthk,bthv->bhkv", e, q, do) + e[:, -1][..., None, None] * dhT
    np.testing.assert_allclose(dh0, want_h0, rtol=1e-12, atol=1e-14)
    # dL/dg_j = sum_{t >= j} exp(G_t) q_t^T h0 do_t + exp(G_T) <h0, dhT>
    per_t = e * np.einsum("bthk,bhkv,bthv->bth", q, h0, do)
    tail = np.flip(np.cumsum(np.flip(per_t, 1), 1), 1)
    want_g = tail + (e[:, -1] * np.einsum("bhkv,bhkv->bh", h0, dhT))[:, None]
    np.testing.assert_allclose(dg, want_g, rtol=1e-12, atol=1e-14)
    # beta enters through the write and the erase.  At beta = 0 the gradient
    # with respect to h_t is D_t = sum_{s>=t} exp(G_s - G_t) q_s do_s^T +
    # exp(G_T - G_t) dhT, and h_{t-1} = exp(G_{t-1}) h0, so
    # dbeta_t = k_t^T D_t v_t - exp(G_t) (D_t^T k_t) . (h0^T k_t)
    T = q.shape[1]
    for t in range(T):
        D = sum(np.exp(G[:, s] - G[:, t])[..., None, None] * np.einsum("bhk,bhv->bhkv", q[:, s], do[:, s])
                for s in range(t, T))
        D = D + np.exp(G[:, -1] - G[:, t])[..., None, None] * dhT
        kD = np.einsum("bhk,bhkv->bhv", k[:, t], D)
        want = (np.einsum("bhv,bhv->bh", kD, v[:, t])
                - e[:, t] * np.einsum("bhv,bhv->bh", kD, np.einsum("bhkv,bhk->bhv", h0, k[:, t])))
        np.testing.assert_allclose(dbeta[:, t], want, rtol=1e-11, atol=1e-13)


def test_bwd_orthogonal_keys_closed_form():
    # mutually orthogonal unit keys and h0 = 0: o_t = sum_{i<=t} beta_i
    # exp(G_t - G_i) (q_t . k_i) v_i, a masked matmul, for every q, v, g, beta
    B, T, H, D = 1, 6, 1, 8
    rng = np.random.default_rng(5)
    basis = np.linalg.qr(rng.standard_normal((D, D)))[0]
    k = basis[:T][None, :, None, :]
    q = rng.standard_normal((B, T, H, D))
    v = rng.standard_normal((B, T, H, 5))
    g = orc.bounded_gate(rng.standard_normal((B, T, H)))
    beta = orc.sigmoid(rng.standard_normal((B, T, H)))
    do = rng.standard_normal((B, T, H, 5))
    dq, _, dv, dg, dbeta, _ = orc.recurrent_bwd(q, k, v, g, beta, do, None, None)
    G = np.cumsum(g[0, :, 0])
    M = np.tril(np.exp(G[:, None] - G[None, :]))                 # [t, i]
    QK = q[0, :, 0] @ k[0, :, 0].T
    W = M * QK                                                   # o = W diag(beta) V
    b = beta[0, :, 0]
    V, DO = v[0, :, 0], do[0, :, 0]
    np.testing.assert_allclose(dv[0, :, 0], (W.T @ DO) * b[:, None], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(dq[0, :, 0], (M * (DO @ V.T)) * b[None, :] @ k[0, :, 0], rtol=1e-12, atol=1e-13)
    S = DO @ V.T                                                 # S[t, i] = do_t . v_i
    np.testing.assert_allclose(dbeta[0, :, 0], (W * S).sum(0), rtol=1e-12, atol=1e-13)
    # dL/dg_j = sum over (t, i) with i < j <= t of W[t,i] beta_i S[t,i]
    contrib = W * S * b[None, :]
    want = np.array([sum(contrib[t, i] for t in range(T) for i in range(T) if i < j <= t)
                     for j in range(T)])
    np.testing.assert_allclose(dg[0, :, 0], want, rtol=1e-12, atol=1e-13)


def test_bwd_zero_upstream_gives_zero():
    args, do, dhT = _inputs(1, 9, 2, 4, 3, 4)
    grads = orc.recurrent_bwd(*args[:5], np.zeros_like(do), None, args[5])
    for gr in grads:
        assert np.all(gr == 0)


def test_bounded_gate_bwd_finite_differences():
    x = np.linspace(-20, 20, 81)
    dg = np.random.default_rng(6).standard_normal(x.shape)
    eps = 1e-6
    fd = (orc.bounded_gate(x + eps) - orc.bounded_gate(x - eps)) / (2 * eps) * dg
    np.testing.assert_allclose(orc.bounded_gate_bwd(x, dg), fd, rtol=1e-7, atol=2e-9)


# ------------------------------------------------------------- mutants
MUTATIONS = {
    "dq from h_prev": ("dq[:, t] = np.einsum(\"bhkv,bhv->bhk\", h_t, dot)",
                       "dq[:, t] = np.einsum(\"bhkv,bhv->bhk\", h_prev, dot)"),
    "dg without decay": ("dg[:, t] = a[:, :, 0, 0] * np.einsum", "dg[:, t] = 1.0 * np.einsum"),
    "dv without beta": ("dv[:, t] = b[:, :, :, 0] * np.einsum", "dv[:, t] = np.einsum"),
    "dbeta sign": ("- np.einsum(\"bhv,bhv->bh\", kde, c))", "+ np.einsum(\"bhv,bhv->bh\", kde, c))"),
    "dk drops a term": ("- np.einsum(\"bhkv,bhv->bhk\", h_prev, kde))", ")"),
    "dh without erase": ("dh = de - b * kt[:, :, :, None] * kde[:, :, None, :]", "dh = de"),
    "dh before output": ("dh = dh + qt[:, :, :, None] * dot[:, :, None, :]", "dh = dh"),
}


def _mutant_bwd(kind):
    src = textwrap.dedent(inspect.getsource(orc.recurrent_bwd))
    a, b = MUTATIONS[kind]
    assert src.count(a) == 1, kind
    ns = dict(orc.__dict__)
    exec(compile(src.replace(a, b), "<mutant>", "exec"), ns)
    return ns["recurrent_bwd"]


@pytest.mark.parametrize("kind", sorted(MUTATIONS))
def test_bwd_mutants_are_caught(kind):
    bwd = _mutant_bwd(kind)
    args, do, dhT = _inputs(1, 5, 1, 3, 2, 21, unit=False)
    grads = bwd(*args[:5], do, dhT, args[5])
    fds = _fd_elementwise(args, do, dhT)
    assert any(_rel(gr, fd) > 1e-4 for gr, fd in zip(grads, fds)), kind
