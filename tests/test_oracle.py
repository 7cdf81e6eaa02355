"""Pins for the fp64 oracle: each ties it to something other than itself.

Anchors: values printed on the pages (tests/golden/gate_pins.txt), a hand-worked
example (tests/golden/hand_example.txt), a pure-Python brute force written in
the other orientation (S = h^T, explicit S (I - beta k k^T) product), closed
forms (pure decay; orthogonal keys reduce to masked gated linear attention),
and invariants (identity step, write-then-query, split invariance, linearity,
norm bound, tail padding).  test_mutants_are_caught plants plausible mistakes in
copies of the recurrence and checks that every one fails at least one pin.
"""

import math
import os

import numpy as np
import pytest

from oracle import linattn_oracle as orc

RNG = np.random.default_rng(1234)


# ---------------------------------------------------------------- fixtures
def _read_kv(path):
    out = {}
    with open(path) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            key, val = (s.strip() for s in line.split("=", 1))
            out[key] = val
    return out


def _mat_rows(s):
    return np.array([[float(x) for x in row.split()] for row in s.split("|")])


def rand_inputs(B, T, H, Dk, Dv, gate="std", seed=0, unit=True, h0=False):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, T, H, Dk))
    k = rng.standard_normal((B, T, H, Dk))
    if unit:
        q /= np.linalg.norm(q, axis=-1, keepdims=True)
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, H, Dv))
    xs = rng.standard_normal((B, T, H))
    if gate == "std":
        g = orc.bounded_gate(xs)
    elif gate == "stress_minus":      # x ~ N(-4, 2): sum of g per tile -> 0
        g = orc.bounded_gate(-4 + 2 * xs)
    elif gate == "stress_plus":       # x ~ N(+4, 2): sum of g per tile -> -80
        g = orc.bounded_gate(4 + 2 * xs)
    elif gate == "weak":              # x ~ N(-8, 1): g ~ -0.003
        g = orc.bounded_gate(-8 + xs)
    elif gate == "zero":
        g = np.zeros((B, T, H))
    elif gate == "min":
        g = np.full((B, T, H), -5.0)
    else:
        raise ValueError(gate)
    beta = orc.sigmoid(rng.standard_normal((B, T, H)))
    hh = 0.02 * rng.standard_normal((B, H, Dk, Dv)) if h0 else None
    return q, k, v, g, beta, hh


def relerr(a, b):
    return np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300)


# ------------------------------------------------------------ gate pins (P1)
def test_gate_values_printed_on_pages(golden_dir):
    pins = _read_kv(os.path.join(golden_dir, "gate_pins.txt"))
    gmin = float(pins["g_min"])
    G = -gmin
    # sigmoid(0) = 1/2 exactly, so g(0) = g_min / 2.
    assert orc.bounded_gate(np.array([0.0]), G)[0] == gmin / 2
    x = np.concatenate([[-1e4], np.linspace(-60, 60, 2001), [1e4]])
    g = orc.bounded_gate(x, G)
    assert np.all(g <= 0) and np.all(g >= gmin)
    assert np.all(np.diff(g) <= 0)                    # decreasing in x
    assert g[-1] == gmin and g[0] == 0.0              # saturates at both ends
    # printed decay range: exp(g) in about [0.0067, 1]
    assert abs(math.exp(g.min()) - float(pins["decay_min_printed"])) < 5e-5
    assert math.exp(g.max()) == float(pins["decay_max_printed"])
    # printed reciprocal range: exp(-g) in [1, about 148]
    assert abs(math.exp(-g.min()) - float(pins["recip_max_printed"])) < 0.5
    assert math.exp(-g.max()) == float(pins["recip_min_printed"])


def test_gate_reflection_identity():
    # sigmoid(x) + sigmoid(-x) = 1, so g(x) + g(-x) = -G for every x.
    x = RNG.standard_normal(1000) * 20
    for G in (5.0, 1.0, 3.5):
        np.testing.assert_allclose(orc.bounded_gate(x, G) + orc.bounded_gate(-x, G),
                                   -G, rtol=0, atol=1e-13)


def test_gate_affine_closed_forms():
    # x = 0: g = -G sigmoid(b); sigmoid(ln 3) = 3/4 exactly, so b = ln 3 gives
    # -3G/4 and a scale a = 2 at x = ln(3) / 2 gives the same logit
    G = 5.0
    a = np.array([2.0, -0.5, 3.0])
    b = np.array([math.log(3.0), 0.0, -math.log(3.0)])
    g0 = orc.bounded_gate_affine(np.zeros((1, 2, 3)), a, b, G)
    np.testing.assert_allclose(g0[0, 0], [-0.75 * G, -0.5 * G, -0.25 * G], rtol=0, atol=1e-14)
    x = np.full((1, 1, 3), math.log(3.0) / 2)
    np.testing.assert_allclose(orc.bounded_gate_affine(x, [2.0, 2.0, 2.0], None, G)[0, 0],
                               -0.75 * G, rtol=0, atol=1e-14)
    # both None is the plain bounded gate
    xr = RNG.standard_normal((2, 5, 3)) * 4
    np.testing.assert_array_equal(orc.bounded_gate_affine(xr, None, None, G), orc.bounded_gate(xr, G))


def test_gate_affine_reflection_and_heads():
    # sigmoid(z) + sigmoid(-z) = 1: flipping a and b gives -G - g
    G = 5.0
    x = RNG.standard_normal((2, 7, 4)) * 6
    a, b = RNG.standard_normal(4) * 2, RNG.standard_normal(4) * 3
    np.testing.assert_allclose(orc.bounded_gate_affine(x, a, b, G) + orc.bounded_gate_affine(x, -a, -b, G),
                               -G, rtol=0, atol=1e-13)
    # head h uses a[h], b[h] at every token and batch (T != H, so a broadcast
    # over the wrong axis cannot pass)
    g = orc.bounded_gate_affine(x, a, b, G)
    for h in range(4):
        for bb in range(2):
            for t in range(7):
                z = a[h] * x[bb, t, h] + b[h]
                assert abs(g[bb, t, h] - (-G / (1.0 + math.exp(-z)))) <= 1e-13


def test_gate_affine_mutants_are_caught():
    G = 5.0
    a, b = np.array([2.0]), np.array([math.log(3.0)])
    x0, x1 = np.zeros((1, 1, 1)), np.full((1, 1, 1), -math.log(3.0))
    wrong = {
        "swapped": lambda x: orc.bounded_gate(b * x + a, G),
        "scale_outside": lambda x: a * orc.bounded_gate(x + b, G),
        "shift_outside": lambda x: orc.bounded_gate(a * x, G) + b,
        "shift_sign": lambda x: orc.bounded_gate(a * x - b, G),
    }
    for name, f in wrong.items():
        # the right gate: -3G/4 at x = 0 and -G sigmoid(-ln 3) = -G/4 at x = -ln 3
        good = (abs(f(x0).item() + 0.75 * G) < 1e-12 and abs(f(x1).item() + 0.25 * G) < 1e-12)
        assert not good, name
    assert abs(orc.bounded_gate_affine(x0, a, b, G).item() + 0.75 * G) < 1e-12
    assert abs(orc.bounded_gate_affine(x1, a, b, G).item() + 0.25 * G) < 1e-12


# --------------------------------------------------------------- the pins
def pin_hand_example(fwd, golden_dir):
    ex = _read_kv(os.path.join(golden_dir, "hand_example.txt"))
    k, v, q = (_mat_rows(ex[n]) for n in ("k", "v", "q"))
    g = np.log(np.array([float(s) for s in ex["decay"].split()]))
    beta = np.array([float(s) for s in ex["beta"].split()])
    o, hT = fwd(q[None, :, None], k[None, :, None], v[None, :, None],
                g[None, :, None], beta[None, :, None], None)
    return (np.allclose(o[0, :, 0], _mat_rows(ex["o"]), atol=1e-14)
            and np.allclose(hT[0, 0], _mat_rows(ex["hT"]), atol=1e-14))


def brute_force_S(q, k, v, g, beta, h0):
    """Pure-Python loops, state S (d_v x d_k): S <- e^g S (I - b k k^T) + b v k^T."""
    T, Dk = len(q), len(q[0])
    Dv = len(v[0])
    S = [[h0[j][i] for j in range(Dk)] for i in range(Dv)]
    outs = []
    for t in range(T):
        e, b = math.exp(g[t]), beta[t]
        M = [[(1.0 if a == c else 0.0) - b * k[t][a] * k[t][c] for c in range(Dk)]
             for a in range(Dk)]
        SM = [[sum(S[i][a] * M[a][j] for a in range(Dk)) for j in range(Dk)]
              for i in range(Dv)]
        S = [[e * SM[i][j] + b * v[t][i] * k[t][j] for j in range(Dk)] for i in range(Dv)]
        outs.append([sum(S[i][j] * q[t][j] for j in range(Dk)) for i in range(Dv)])
    return np.array(outs), np.array(S).T


def pin_brute_force(fwd):
    ok = True
    for seed, (T, Dk, Dv), gate in [(0, (7, 3, 4), "std"), (1, (9, 4, 2), "weak"),
                                    (2, (6, 4, 4), "zero"), (3, (5, 2, 3), "stress_plus")]:
        q, k, v, g, beta, _ = rand_inputs(1, T, 1, Dk, Dv, gate, seed)
        h0 = np.random.default_rng(seed + 50).standard_normal((1, 1, Dk, Dv))
        o, hT = fwd(q, k, v, g, beta, h0)
        ob, hb = brute_force_S(q[0, :, 0].tolist(), k[0, :, 0].tolist(), v[0, :, 0].tolist(),
                               g[0, :, 0].tolist(), beta[0, :, 0].tolist(), h0[0, 0].tolist())
        ok &= np.allclose(o[0, :, 0], ob, rtol=1e-12, atol=1e-12)
        ok &= np.allclose(hT[0, 0], hb, rtol=1e-12, atol=1e-12)
    return bool(ok)


def pin_identity_step(fwd):
    # beta = 0 and g = 0: the state never changes and o_t = h0^T q_t.
    q, k, v, _, _, h0 = rand_inputs(2, 11, 3, 5, 4, seed=7, h0=True)
    z = np.zeros(q.shape[:3])
    o, hT = fwd(q, k, v, z, z, h0)
    return (np.array_equal(hT, h0)
            and np.allclose(o, np.einsum("bthk,bhkv->bthv", q, h0), rtol=1e-14, atol=1e-15))


def sparse_unit_keys(n, d, seed):
    """Keys with exactly representable unit norm: 4 entries of +-1/2 (d >= 4)."""
    rng = np.random.default_rng(seed)
    K = np.zeros((n, d))
    for i in range(n):
        idx = rng.choice(d, 4, replace=False)
        K[i, idx] = rng.choice([-0.5, 0.5], 4)
    return K


def pin_write_then_query(fwd):
    # g = 0, beta = 1, |k| = 1: after writing v under key k, querying q = k returns
    # v exactly, whatever the prior state.
    Dk, Dv, T = 8, 5, 6
    K = sparse_unit_keys(T, Dk, 3)
    rng = np.random.default_rng(9)
    V = rng.standard_normal((T, Dv))
    h0 = rng.standard_normal((1, 1, Dk, Dv))
    o, _ = fwd(K[None, :, None], K[None, :, None], V[None, :, None],
               np.zeros((1, T, 1)), np.ones((1, T, 1)), h0)
    return np.allclose(o[0, :, 0], V, rtol=0, atol=1e-13)


def pin_orthogonal_keys(fwd):
    # Orthonormal keys, h0 = 0: the erase term vanishes and the recurrence is
    # masked gated linear attention:
    #   o_t = sum_{i<=t} beta_i exp(G_t - G_i) (q_t . k_i) v_i,  G = cumsum(g).
    T, Dk, Dv = 6, 8, 3
    rng = np.random.default_rng(11)
    Kq, _ = np.linalg.qr(rng.standard_normal((Dk, Dk)))
    K = Kq[:, :T].T
    Q = rng.standard_normal((T, Dk))
    V = rng.standard_normal((T, Dv))
    g = orc.bounded_gate(rng.standard_normal(T))
    beta = orc.sigmoid(rng.standard_normal(T))
    Gc = np.cumsum(g)
    M = np.tril(np.exp(Gc[:, None] - Gc[None, :]))
    ref = (M * (Q @ K.T)) @ (beta[:, None] * V)
    o, _ = fwd(Q[None, :, None], K[None, :, None], V[None, :, None],
               g[None, :, None], beta[None, :, None], None)
    return np.allclose(o[0, :, 0], ref, rtol=1e-12, atol=1e-13)


def pin_pure_decay(fwd):
    # beta = 0: h_t = exp(G_t) h0 and o_t = exp(G_t) h0^T q_t.
    q, k, v, g, _, h0 = rand_inputs(1, 9, 2, 4, 3, gate="std", seed=13, h0=True)
    o, hT = fwd(q, k, v, g, np.zeros_like(g), h0)
    Gc = np.cumsum(g, axis=1)
    ref_o = np.exp(Gc)[..., None] * np.einsum("bthk,bhkv->bthv", q, h0)
    ref_h = np.exp(Gc[:, -1])[..., None, None] * h0
    return np.allclose(o, ref_o, rtol=1e-12, atol=1e-15) and np.allclose(hT, ref_h, rtol=1e-12)


def pin_split_invariance(fwd):
    q, k, v, g, beta, h0 = rand_inputs(2, 37, 2, 6, 5, gate="weak", seed=17, h0=True)
    o, hT = fwd(q, k, v, g, beta, h0)
    o1, h1 = fwd(q[:, :20], k[:, :20], v[:, :20], g[:, :20], beta[:, :20], h0)
    o2, h2 = fwd(q[:, 20:], k[:, 20:], v[:, 20:], g[:, 20:], beta[:, 20:], h1)
    return (np.allclose(np.concatenate([o1, o2], 1), o, rtol=1e-12, atol=1e-13)
            and np.allclose(h2, hT, rtol=1e-12, atol=1e-13))


def pin_linearity(fwd):
    # o and hT are jointly linear in (V, h0) for fixed q, k, g, beta.
    q, k, v1, g, beta, h01 = rand_inputs(1, 13, 2, 5, 4, gate="std", seed=19, h0=True)
    _, _, v2, _, _, h02 = rand_inputs(1, 13, 2, 5, 4, gate="std", seed=20, h0=True)
    a, b = 0.7, -1.9
    o, h = fwd(q, k, a * v1 + b * v2, g, beta, a * h01 + b * h02)
    oa, ha = fwd(q, k, v1, g, beta, h01)
    ob, hb = fwd(q, k, v2, g, beta, h02)
    return (np.allclose(o, a * oa + b * ob, rtol=1e-11, atol=1e-12)
            and np.allclose(h, a * ha + b * hb, rtol=1e-11, atol=1e-12))


def pin_norm_bound(fwd):
    # For g <= 0, |k| = 1 and beta in [0, 1], |exp(g)(I - beta k k^T)|_2 <= 1, so
    # |h_t|_2 <= |h0|_2 + sum_{i<=t} beta_i |v_i|: everything stays finite over
    # the whole bounded range (g = 0, g = -5, and the stress draws).
    ok = True
    for gate in ("zero", "min", "stress_plus", "stress_minus", "std"):
        q, k, v, g, beta, h0 = rand_inputs(1, 40, 2, 6, 4, gate=gate, seed=23, h0=True)
        o, hT = fwd(q, k, v, g, beta, h0)
        ok &= bool(np.all(np.isfinite(o)) and np.all(np.isfinite(hT)))
        for h in range(2):
            bound = (np.linalg.norm(h0[0, h], 2)
                     + np.sum(beta[0, :, h] * np.linalg.norm(v[0, :, h], axis=-1)))
            ok &= bool(np.linalg.norm(hT[0, h], 2) <= bound * (1 + 1e-12))
            # and each output obeys |o_t| <= |h_t|_2 |q_t| <= bound
            ok &= bool(np.all(np.linalg.norm(o[0, :, h], axis=-1) <= bound * (1 + 1e-12)))
    return ok


def pin_tail_padding(fwd):
    # Appending tokens with q = k = v = 0, g = 0, beta = 0 is an exact identity
    # step: the state is unchanged and the padded outputs are 0.
    q, k, v, g, beta, h0 = rand_inputs(1, 10, 2, 4, 3, gate="std", seed=29, h0=True)
    o, hT = fwd(q, k, v, g, beta, h0)
    pad = lambda a: np.concatenate([a, np.zeros((1, 6) + a.shape[2:])], axis=1)
    op, hp = fwd(pad(q), pad(k), pad(v), pad(g), pad(beta), h0)
    return np.array_equal(hp, hT) and np.array_equal(op[:, :10], o) and not np.any(op[:, 10:])


PINS = {
    "hand_example": pin_hand_example,
    "brute_force": pin_brute_force,
    "identity_step": pin_identity_step,
    "write_then_query": pin_write_then_query,
    "orthogonal_keys": pin_orthogonal_keys,
    "pure_decay": pin_pure_decay,
    "split_invariance": pin_split_invariance,
    "linearity": pin_linearity,
    "norm_bound": pin_norm_bound,
    "tail_padding": pin_tail_padding,
}


def run_pin(name, fwd, golden_dir):
    f = PINS[name]
    return f(fwd, golden_dir) if name == "hand_example" else f(fwd)


@pytest.mark.parametrize("name", sorted(PINS))
def test_recurrent_pins(name, golden_dir):
    assert run_pin(name, orc.recurrent_fwd, golden_dir)


@pytest.mark.parametrize("name", sorted(PINS))
def test_c_recurrent_pins(name, golden_dir):
    # The plain-C copy of the recurrence (used for long sequences) answers to
    # the same pins as the NumPy one.
    from oracle import c_recurrent
    fwd = lambda *a: c_recurrent.recurrent_fwd(*a, workers=2)
    assert run_pin(name, fwd, golden_dir)


def test_c_recurrent_matches_numpy_on_windows():
    from oracle import c_recurrent
    q, k, v, g, beta, h0 = rand_inputs(2, 50, 3, 16, 8, gate="weak", seed=43, h0=True)
    o, hT = orc.recurrent_fwd(q, k, v, g, beta, h0)
    _, hmid = orc.recurrent_fwd(q[:, :20], k[:, :20], v[:, :20], g[:, :20], beta[:, :20], h0)
    res = c_recurrent.recurrent_fwd_c(q, k, v, g, beta, hmid, heads=[(0, 1), (1, 2)],
                                      t_range=(20, 50), workers=2)
    for (b, h), (ob, hb) in res.items():
        np.testing.assert_allclose(ob, o[b, 20:, h], rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(hb, hT[b, h], rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("chunk", [1, 3, 16, 32])
def test_chunked_pins(chunk, golden_dir):
    fwd = lambda *a: orc.chunked_fwd(*a, chunk=chunk)
    for name in ("hand_example", "brute_force", "orthogonal_keys", "write_then_query"):
        assert run_pin(name, fwd, golden_dir), name


@pytest.mark.parametrize("gate", ["std", "stress_minus", "stress_plus", "weak", "zero", "min"])
@pytest.mark.parametrize("chunk", [1, 3, 16, 32])
def test_chunked_equals_recurrent(gate, chunk):
    # T = 100 leaves a ragged tail for every chunk size but 1.
    q, k, v, g, beta, h0 = rand_inputs(2, 100, 3, 8, 6, gate=gate, seed=31, h0=True)
    o_r, h_r = orc.recurrent_fwd(q, k, v, g, beta, h0)
    o_c, h_c = orc.chunked_fwd(q, k, v, g, beta, h0, chunk=chunk)
    assert relerr(o_c, o_r) < 1e-12
    assert relerr(h_c, h_r) < 1e-12


def test_decode_equals_forward():
    q, k, v, g, beta, h0 = rand_inputs(3, 12, 2, 5, 4, gate="std", seed=37, h0=True)
    o_f, h_f = orc.recurrent_fwd(q, k, v, g, beta, h0)
    S = h0.copy()
    for t in range(12):
        o_t, S_new = orc.decode_step(q[:, t], k[:, t], v[:, t], g[:, t], beta[:, t], S)
        assert np.allclose(o_t, o_f[:, t], rtol=1e-12, atol=1e-14)
        S = S_new
    assert np.allclose(S, h_f, rtol=1e-12, atol=1e-14)
    # decode never mutates its input state
    S0 = h0.copy()
    orc.decode_step(q[:, 0], k[:, 0], v[:, 0], g[:, 0], beta[:, 0], S0)
    assert np.array_equal(S0, h0)


def test_heads_runner_matches_vectorised():
    q, k, v, g, beta, h0 = rand_inputs(2, 30, 3, 6, 5, gate="std", seed=41, h0=True)
    o, hT = orc.recurrent_fwd(q, k, v, g, beta, h0)
    res = orc.recurrent_fwd_heads(q, k, v, g, beta, h0, workers=2)
    for (b, h), (ob, hb) in res.items():
        np.testing.assert_array_equal(ob, o[b, :, h])
        np.testing.assert_array_equal(hb, hT[b, h])
    # a token window started from the true state reproduces that window
    _, hmid = orc.recurrent_fwd(q[:, :11], k[:, :11], v[:, :11], g[:, :11], beta[:, :11], h0)
    res = orc.recurrent_fwd_heads(q, k, v, g, beta, hmid, heads=[(1, 2)], t_range=(11, 30),
                                  workers=1)
    np.testing.assert_allclose(res[(1, 2)][0], o[1, 11:, 2], rtol=1e-12, atol=1e-14)


# ------------------------------------------------------------- mutants
def _mutant(kind):
    def fwd(q, k, v, g, beta, h0=None):
        B, T, H, Dk = q.shape
        Dv = v.shape[-1]
        h = np.zeros((B, H, Dk, Dv)) if h0 is None else np.array(h0, dtype=float)
        o = np.empty((B, T, H, Dv))
        for t in range(T):
            kt, vt, qt = k[:, t], v[:, t], q[:, t]
            a = np.exp(-g[:, t] if kind == "gate_sign" else g[:, t])[:, :, None, None]
            if kind == "no_decay":
                a = np.ones_like(a)
            b = beta[:, t][:, :, None, None]
            kh = np.einsum("bhk,bhkv->bhv", kt, h)
            outer_kk = kt[:, :, :, None] * kh[:, :, None, :]
            write = kt[:, :, :, None] * vt[:, :, None, :]
            if kind == "transposed_write":
                write = np.swapaxes(write, -1, -2)
            prev = h
            if kind == "decay_after_write":
                h = a * (h - b * outer_kk + b * write)
            elif kind == "erase_without_beta":
                h = a * (h - outer_kk) + b * write
            elif kind == "erase_sign":
                h = a * (h + b * outer_kk) + b * write
            elif kind == "erase_not_decayed":
                h = a * h - b * outer_kk + b * write
            elif kind == "write_without_beta":
                h = a * (h - b * outer_kk) + write
            else:
                h = a * (h - b * outer_kk) + b * write
            src = prev if kind == "output_pre_update" else h
            qq = kt if kind == "output_uses_key" else qt
            o[:, t] = np.einsum("bhk,bhkv->bhv", qq, src)
        return o, h
    return fwd


MUTANTS = ["gate_sign", "no_decay", "transposed_write", "decay_after_write",
           "erase_without_beta", "erase_sign", "erase_not_decayed",
           "write_without_beta", "output_pre_update", "output_uses_key"]


@pytest.mark.parametrize("kind", MUTANTS)
def test_mutants_are_caught(kind, golden_dir):
    # every pin is a function of the implementation under test, so a mutant
    # copy of the recurrence can be run through all of them
    fwd = _mutant(kind)
    failed = []
    for name in PINS:
        try:
            ok = run_pin(name, fwd, golden_dir)
        except (ValueError, IndexError):       # shape errors count as caught
            ok = False
        if not ok:
            failed.append(name)
    assert failed, f"mutant {kind} passed every pin"


def test_unmutated_control_passes_every_pin(golden_dir):
    fwd = _mutant("none")
    assert all(run_pin(name, fwd, golden_dir) for name in PINS)


def test_gate_mutants_are_caught(golden_dir):
    pins = _read_kv(os.path.join(golden_dir, "gate_pins.txt"))
    G = -float(pins["g_min"])
    x = np.array([-1e4, 0.0, 1e4])
    wrong = {
        "flipped_sigmoid": lambda x: -G * orc.sigmoid(-x),
        "softplus": lambda x: -np.logaddexp(0, x),
        "positive": lambda x: G * orc.sigmoid(x),
    }
    for name, f in wrong.items():
        g = f(x)
        good = g[1] == -G / 2 and g[2] == -G and g[0] == 0.0
        assert not good, name


# ------------------------------------------------------ packed sequences
def _varlen_case(lengths, H=2, Dk=8, Dv=6, gate="std", seed=0, h0=True):
    T = int(sum(lengths))
    q, k, v, g, beta, _ = rand_inputs(1, T, H, Dk, Dv, gate=gate, seed=seed)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    hh = 0.02 * np.random.default_rng(seed + 1).standard_normal((len(lengths), H, Dk, Dv)) if h0 else None
    return q, k, v, g, beta, cu, hh


def _carry_over_mutant(q, k, v, g, beta, cu, h0):
    """A plausible mistake: the state is not reset where a sequence begins."""
    o, hlast = orc.recurrent_fwd(q, k, v, g, beta, None if h0 is None else h0[:1])
    hT = np.stack([orc.recurrent_fwd(q[:, :b], k[:, :b], v[:, :b], g[:, :b], beta[:, :b],
                                     None if h0 is None else h0[:1])[1][0] for b in cu[1:]])
    return o, hT


def _boundary_pin(fwd):
    """Closed form at a boundary: the second sequence neither writes (beta = 0)
    nor decays (g = 0), so its outputs are h0[1]^T q_t exactly and its final
    state is h0[1], whatever the first sequence did."""
    q, k, v, g, beta, cu, h0 = _varlen_case([7, 5], gate="std", seed=3)
    g[:, 7:] = 0.0
    beta[:, 7:] = 0.0
    o, hT = fwd(q, k, v, g, beta, cu, h0)
    want = np.einsum("thk,hkv->thv", q[0, 7:], h0[1])
    return np.allclose(o[0, 7:], want, rtol=1e-13, atol=1e-15) and np.allclose(hT[1], h0[1], rtol=0, atol=0)


def test_varlen_boundary_closed_form():
    assert _boundary_pin(orc.recurrent_fwd_varlen)


def test_varlen_carry_over_mutant_is_caught():
    assert not _boundary_pin(_carry_over_mutant)


def test_varlen_equal_lengths_equal_the_batch_axis():
    N, L, H, Dk, Dv = 3, 11, 2, 8, 6
    q, k, v, g, beta, cu, h0 = _varlen_case([L] * N, H, Dk, Dv, gate="weak", seed=5)
    o, hT = orc.recurrent_fwd_varlen(q, k, v, g, beta, cu, h0)
    rs = lambda a: a.reshape((N, L) + a.shape[2:])
    ob, hb = orc.recurrent_fwd(rs(q), rs(k), rs(v), rs(g), rs(beta), h0)
    np.testing.assert_allclose(o.reshape(ob.shape), ob, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(hT, hb, rtol=1e-13, atol=1e-15)


def test_varlen_c_matches_numpy_with_empty_sequences():
    from oracle import c_recurrent
    lengths = [0, 1, 17, 0, 33, 5]
    for h0flag in (True, False):
        q, k, v, g, beta, cu, h0 = _varlen_case(lengths, 3, 16, 8, gate="weak", seed=7, h0=h0flag)
        o, hT = orc.recurrent_fwd_varlen(q, k, v, g, beta, cu, h0)
        oc, hc = c_recurrent.recurrent_fwd_varlen(q, k, v, g, beta, cu, h0, workers=2)
        np.testing.assert_allclose(oc, o, rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(hc, hT, rtol=1e-12, atol=1e-14)
        assert np.array_equal(hT[0], np.zeros_like(hT[0]) if h0 is None else h0[0])


def test_varlen_rejects_bad_offsets():
    q, k, v, g, beta, cu, h0 = _varlen_case([3, 4], seed=9)
    with pytest.raises(ValueError):
        orc.recurrent_fwd_varlen(q, k, v, g, beta, [0, 5, 4], h0)
    with pytest.raises(ValueError):
        orc.recurrent_fwd_varlen(q, k, v, g, beta, [0, 3, 6], h0)


# ------------------------------------------------------- input preparation
def test_prepare_inputs_pins():
    rng = np.random.default_rng(17)
    q = rng.standard_normal((2, 5, 3, 8)) * 7.0
    k = rng.standard_normal((2, 5, 3, 8))
    k[0, 1, 2] = 0.0                                  # a zero key stays zero
    xb = np.array([0.0, math.log(3.0), -math.log(3.0), 40.0, -40.0])
    qn, kn, b = orc.prepare_inputs(q, k, xb)
    np.testing.assert_allclose(np.linalg.norm(qn, axis=-1), 1.0, rtol=1e-14)
    np.testing.assert_allclose(qn * np.linalg.norm(q, axis=-1, keepdims=True), q, rtol=1e-13)
    assert np.all(kn[0, 1, 2] == 0.0)
    mask = np.ones(k.shape[:-1], bool)
    mask[0, 1, 2] = False
    np.testing.assert_allclose(np.linalg.norm(kn, axis=-1)[mask], 1.0, rtol=1e-14)
    # sigmoid(0) = 1/2, sigmoid(ln 3) = 3/4, sigmoid(-ln 3) = 1/4, saturation
    np.testing.assert_allclose(b[:3], [0.5, 0.75, 0.25], rtol=1e-15)
    assert b[3] == 1.0 and 0.0 < b[4] < 1e-17
