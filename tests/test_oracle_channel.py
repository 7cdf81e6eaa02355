"""Pins for the per-channel-gate oracle (recurrent_fwd_channel and its tiled
companion chunked_fwd_channel): each ties it to something other than itself.

Anchors: the scalar-gate oracle (itself pinned in test_oracle.py) when every
channel carries the same g; closed forms for pure decay (beta = 0) and for keys
of disjoint support (the erase term vanishes and the recurrence is masked gated
linear attention with a per-channel decay, a masked matmul); the delta rule's
defining property that a full-strength write under a unit key followed by a
query with that key returns the written value whatever the decay (this fixes
the order decay -> erase -> write); a pure-Python brute force written in the S
orientation with explicit matrices.  test_channel_mutants_are_caught plants
plausible mistakes in copies of the recurrence and checks that each fails at
least one pin.
"""

import math

import numpy as np
import pytest

from oracle import linattn_oracle as orc


def _inputs(B, T, H, Dk, Dv, gate="std", seed=0, h0=False):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, T, H, Dk))
    k = rng.standard_normal((B, T, H, Dk))
    q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, H, Dv))
    x = rng.standard_normal((B, T, H, Dk))
    g = {"std": orc.bounded_gate(x), "weak": orc.bounded_gate(x - 8.0),
         "min": np.full_like(x, -5.0), "zero": np.zeros_like(x),
         "split": np.where(np.arange(Dk) % 2 == 0, -5.0, 0.0) + 0 * x}[gate]
    beta = orc.sigmoid(rng.standard_normal((B, T, H)))
    hh = 0.5 * rng.standard_normal((B, H, Dk, Dv)) if h0 else None
    return q, k, v, g, beta, hh


# ------------------------------------------------------------------ the pins
def pin_scalar_reduction(fwd):
    # the same g on every channel is the scalar gate
    q, k, v, g, beta, h0 = _inputs(2, 23, 2, 8, 5, seed=1, h0=True)
    g = np.repeat(g[..., :1], 8, axis=-1)
    o, hT = fwd(q, k, v, g, beta, h0)
    ro, rh = orc.recurrent_fwd(q, k, v, g[..., 0], beta, h0)
    return max(np.abs(o - ro).max(), np.abs(hT - rh).max()) < 1e-12


def pin_pure_decay(fwd):
    # beta = 0: h_t[c, :] = exp(G_t[c]) h0[c, :], o_t = sum_c q_t[c] exp(G_t[c]) h0[c, :]
    q, k, v, g, beta, h0 = _inputs(1, 17, 2, 6, 4, seed=2, h0=True)
    beta = np.zeros_like(beta)
    o, hT = fwd(q, k, v, g, beta, h0)
    Gt = np.cumsum(g, axis=1)                                   # (B,T,H,Dk)
    ro = np.einsum("bthc,bthc,bhcv->bthv", q, np.exp(Gt), h0)
    rh = np.exp(Gt[:, -1])[..., None] * h0
    return max(np.abs(o - ro).max(), np.abs(hT - rh).max()) < 1e-12


def pin_disjoint_keys(fwd):
    # keys with pairwise disjoint supports (T <= Dk / 2, two channels each),
    # h0 = 0: k_t^T D h_{t-1} = 0, so
    #   o_t = sum_{i <= t} beta_i (sum_c q_t[c] k_i[c] exp(G_t[c] - G_i[c])) v_i
    rng = np.random.default_rng(3)
    B, T, H, Dk, Dv = 1, 6, 2, 12, 5
    q, _, v, g, beta, _ = _inputs(B, T, H, Dk, Dv, seed=3)
    perm = rng.permutation(Dk)
    k = np.zeros((B, T, H, Dk))
    for t in range(T):
        for c in perm[2 * t:2 * t + 2]:
            k[:, t, :, c] = rng.standard_normal((B, H))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    o, hT = fwd(q, k, v, g, beta, None)
    G = np.cumsum(g, axis=1)
    ro = np.zeros((B, T, H, Dv))
    rh = np.zeros((B, H, Dk, Dv))
    for t in range(T):
        for i in range(t + 1):
            w = np.einsum("bhc,bhc,bhc->bh", q[:, t], k[:, i], np.exp(G[:, t] - G[:, i]))
            ro[:, t] += (beta[:, i] * w)[..., None] * v[:, i]
    for i in range(T):
        dec = np.exp(G[:, -1] - G[:, i])                        # (B,H,Dk)
        rh += beta[:, i][..., None, None] * (dec * k[:, i])[..., None] * v[:, i][:, :, None, :]
    return max(np.abs(o - ro).max(), np.abs(hT - rh).max()) < 1e-12


def pin_write_then_query(fwd):
    # beta = 1 and a unit key that is exact in binary (four entries +-1/2):
    # querying with that key right after the write returns v exactly, from any
    # prior state and under any per-channel decay of that step
    q, k, v, g, beta, h0 = _inputs(1, 9, 2, 8, 4, seed=4, h0=True)
    key = np.array([0.5, -0.5, 0, 0.5, 0, 0, -0.5, 0])
    t = 8
    k[:, t] = key
    q[:, t] = key
    beta[:, t] = 1.0
    o, _ = fwd(q, k, v, g, beta, h0)
    return np.abs(o[:, t] - v[:, t]).max() < 1e-12


def pin_brute_force(fwd):
    # pure Python, S orientation: S_t = S_{t-1} D_t (I - b k k^T) + b v k^T
    q, k, v, g, beta, h0 = _inputs(1, 7, 1, 4, 3, seed=5, h0=True)
    Dk, Dv = 4, 3
    S = [[h0[0, 0][c][r] for c in range(Dk)] for r in range(Dv)]      # S = h^T
    outs = []
    for t in range(7):
        kt, qt, vt = list(k[0, t, 0]), list(q[0, t, 0]), list(v[0, t, 0])
        b = beta[0, t, 0]
        D = [np.exp(g[0, t, 0, c]) for c in range(Dk)]
        M = [[D[r] * ((1.0 if r == c else 0.0) - b * kt[r] * kt[c]) for c in range(Dk)]
             for r in range(Dk)]                                        # D (I - b k k^T)
        S = [[sum(S[r][j] * M[j][c] for j in range(Dk)) + b * vt[r] * kt[c]
              for c in range(Dk)] for r in range(Dv)]
        outs.append([sum(S[r][c] * qt[c] for c in range(Dk)) for r in range(Dv)])
    o, hT = fwd(q, k, v, g, beta, h0)
    e_o = np.abs(o[0, :, 0] - np.array(outs)).max()
    e_h = np.abs(hT[0, 0] - np.array(S).T).max()
    return max(e_o, e_h) < 1e-12


PINS = {"scalar_reduction": pin_scalar_reduction, "pure_decay": pin_pure_decay,
        "disjoint_keys": pin_disjoint_keys, "write_then_query": pin_write_then_query,
        "brute_force": pin_brute_force}


@pytest.mark.parametrize("name", sorted(PINS))
def test_recurrent_channel_pins(name):
    assert PINS[name](orc.recurrent_fwd_channel)


@pytest.mark.parametrize("name", sorted(PINS))
def test_chunked_channel_pins(name):
    assert PINS[name](lambda *a: orc.chunked_fwd_channel(*a, chunk=3))


@pytest.mark.parametrize("gate", ["std", "weak", "min", "zero", "split"])
@pytest.mark.parametrize("chunk", [1, 3, 16])
def test_chunked_channel_equals_recurrent(gate, chunk):
    q, k, v, g, beta, h0 = _inputs(2, 45, 2, 8, 6, gate=gate, seed=6, h0=True)
    ro, rh = orc.recurrent_fwd_channel(q, k, v, g, beta, h0)
    co, ch = orc.chunked_fwd_channel(q, k, v, g, beta, h0, chunk=chunk)
    assert np.abs(co - ro).max() <= 1e-12 * max(1.0, np.abs(ro).max())
    assert np.abs(ch - rh).max() <= 1e-12 * max(1.0, np.abs(rh).max())


def test_in_tile_reciprocal_stays_finite_at_the_bound():
    # g = -5 on every channel: across a 16-token tile the reciprocal of the
    # cumulative decay reaches exp(80) ~ 5.5e34, finite in float32 (and in
    # bfloat16, which has float32's exponent range); one token more would
    # reach exp(85), and 18 tokens exp(90) > FLT_MAX
    Gmin = 16 * -5.0
    assert np.isfinite(np.float32(np.exp(-Gmin)))
    assert np.float32(np.exp(-Gmin)) < np.finfo(np.float32).max
    assert np.exp(-18 * -5.0) > np.finfo(np.float32).max
    assert np.float32(np.exp(Gmin)) >= np.finfo(np.float32).tiny     # still a normal number
    q, k, v, g, beta, h0 = _inputs(1, 64, 2, 16, 8, gate="min", seed=7, h0=True)
    co, ch = orc.chunked_fwd_channel(q, k, v, g, beta, h0, chunk=16)
    ro, rh = orc.recurrent_fwd_channel(q, k, v, g, beta, h0)
    assert np.isfinite(co).all() and np.isfinite(ch).all()
    assert np.abs(co - ro).max() <= 1e-10 * max(1.0, np.abs(ro).max())


def _tile_operands_f32(k, g, chunk=16):
    """The per-channel in-tile operands in float32, tile by tile: keys scaled
    by the cumulative decay Gam_t and keys divided by it (Gam_s^-1), and their
    products A[t, s] = (k_t o Gam_t) . (k_s / Gam_s), s < t.  Returns the
    largest |log| of 1/Gam in any tile and whether every operand and product
    is finite."""
    k32, g32 = np.asarray(k, np.float32), np.asarray(g, np.float32)
    B, T, H, Dk = k32.shape
    worst, finite = 0.0, True
    with np.errstate(over="ignore", invalid="ignore"):
        for c0 in range(0, T, chunk):
            Gc = np.cumsum(g32[:, c0:c0 + chunk], axis=1, dtype=np.float32)
            worst = max(worst, float(-Gc.min()))
            inv = np.exp(-Gc)
            kg, ki = k32[:, c0:c0 + chunk] * np.exp(Gc), k32[:, c0:c0 + chunk] * inv
            A = np.einsum("bthc,bshc->bhts", kg, ki)
            finite &= bool(np.isfinite(inv).all() and np.isfinite(ki).all() and np.isfinite(A).all())
    return worst, finite


def test_softplus_contrast_overflows_where_the_bound_stays_finite():
    """The pages bound the log-decay so that inside a 16-token tile the
    reciprocal of the cumulative decay stays finite ("Deep Dive ...", sec. 3.2
    and 3.3; "How Trillion-Scale ...", sec. 3.2).  Contrast: the same logits
    x ~ N(mu, 1) through g = -softplus(x) (unbounded below) and through
    g = -5 sigmoid(x).  A tile's operand 1/Gam reaches exp(-sum g); float32
    overflows past ln(FLT_MAX) ~ 88.72, i.e. a mean decay above ~5.55 per
    token over 16 tokens -- just beyond the bound's 16 * 5 = 80."""
    ln_max = math.log(float(np.finfo(np.float32).max))
    assert 16 * 5.0 < ln_max < 16 * 5.6
    rng = np.random.default_rng(23)
    k = rng.standard_normal((1, 128, 2, 16))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    seen = {}
    for mu in (0.0, 2.0, 4.0, 6.0, 8.0):
        x = mu + rng.standard_normal((1, 128, 2, 16))
        sp_worst, sp_finite = _tile_operands_f32(k, -np.logaddexp(0.0, x))
        bd_worst, bd_finite = _tile_operands_f32(k, orc.bounded_gate(x, 5.0))
        seen[mu] = (sp_worst, sp_finite, bd_worst, bd_finite)
        # the bound: finite at every shift, never beyond exp(80)
        assert bd_finite and bd_worst <= 80.0 + 1e-3, (mu, bd_worst)
        # -softplus: finite exactly while every tile's summed decay stays below
        # ln(FLT_MAX) (a margin of 1 for float32 rounding of the sums)
        if sp_worst < ln_max - 1.0:
            assert sp_finite, (mu, sp_worst)
        if sp_worst > ln_max + 1.0:
            assert not sp_finite, (mu, sp_worst)
    # the contrast itself: small shifts are fine both ways, large ones
    # overflow without the bound
    assert seen[0.0][1] and seen[2.0][1]
    assert not seen[6.0][1] and not seen[8.0][1]
    # with the bound the float32 tile products agree with fp64 ones
    x = 8.0 + rng.standard_normal((1, 32, 2, 16))
    g = orc.bounded_gate(x, 5.0)
    Gc = np.cumsum(g[:, :16], axis=1)
    A64 = np.einsum("bthc,bshc->bhts", k[:, :16] * np.exp(Gc), k[:, :16] * np.exp(-Gc))
    Gc32 = np.cumsum(g[:, :16].astype(np.float32), axis=1, dtype=np.float32)
    k32 = k[:, :16].astype(np.float32)
    A32 = np.einsum("bthc,bshc->bhts", k32 * np.exp(Gc32), k32 * np.exp(-Gc32))
    low = np.tril(np.ones((16, 16)), -1).astype(bool)
    rel = np.abs(A32 - A64)[..., low] / np.maximum(np.abs(A64)[..., low], 1e-30)
    assert np.isfinite(A32).all() and np.median(rel) < 1e-4


# ------------------------------------------------------- planted mistakes
def _mutant(kind):
    def fwd(q, k, v, g, beta, h0=None):
        q, k, v, g, beta = (np.asarray(a, dtype=np.float64) for a in (q, k, v, g, beta))
        B, T, H, Dk = q.shape
        Dv = v.shape[-1]
        h = np.zeros((B, H, Dk, Dv)) if h0 is None else np.array(h0, dtype=np.float64)
        o = np.empty((B, T, H, Dv))
        for t in range(T):
            kt, vt = k[:, t], v[:, t]
            b = beta[:, t][:, :, None, None]
            a = np.exp(g[:, t])
            if kind == "reversed_channels":
                a = a[..., ::-1]
            if kind == "decay_on_values":          # decay indexed by the value axis
                d = a[:, :, None, :Dv] * h if Dv <= Dk else h
            elif kind == "erase_before_decay":     # D (I - b k k^T) h instead of (I - b k k^T) D h
                kh = np.einsum("bhk,bhkv->bhv", kt, h)
                d = a[..., None] * (h - b * kt[..., None] * kh[:, :, None, :])
                h = d + b * kt[..., None] * vt[:, :, None, :]
                o[:, t] = np.einsum("bhk,bhkv->bhv", q[:, t], h)
                continue
            else:
                d = a[..., None] * h
            kd = np.einsum("bhk,bhkv->bhv", kt, d)
            w = b * kt[..., None] * vt[:, :, None, :]
            if kind == "decayed_write":
                w = a[..., None] * w
            h = d - b * kt[..., None] * kd[:, :, None, :] + w
            o[:, t] = np.einsum("bhk,bhkv->bhv", q[:, t], h)
        return o, h
    return fwd


CHANNEL_MUTANTS = ["reversed_channels", "decay_on_values", "erase_before_decay", "decayed_write"]


@pytest.mark.parametrize("kind", CHANNEL_MUTANTS)
def test_channel_mutants_are_caught(kind):
    f = _mutant(kind)
    assert not all(p(f) for p in PINS.values()), kind


def test_unmutated_channel_control_passes_every_pin():
    f = _mutant("none")
    assert all(p(f) for p in PINS.values())


def test_decode_channel_steps_equal_the_forward():
    q, k, v, g, beta, h0 = _inputs(2, 9, 3, 8, 5, gate="std", seed=8, h0=True)
    ro, rh = orc.recurrent_fwd_channel(q, k, v, g, beta, h0)
    S = h0.copy()
    for t in range(9):
        o, S = orc.decode_step_channel(q[:, t], k[:, t], v[:, t], g[:, t], beta[:, t], S)
        assert np.abs(o - ro[:, t]).max() < 1e-12
    assert np.abs(S - rh).max() < 1e-12


def test_channel_varlen_boundary_closed_form():
    # sequence 1 neither writes (beta = 0) nor decays (g = 0): it returns its
    # own h0 and outputs h0^T q_t exactly, whatever sequence 0 left behind
    q, k, v, g, beta, _ = _inputs(1, 20, 2, 8, 5, seed=9)
    cu = [0, 12, 20]
    h0 = np.random.default_rng(9).standard_normal((2, 2, 8, 5))
    beta[:, 12:] = 0.0
    g[:, 12:] = 0.0
    o, hT = orc.recurrent_fwd_channel_varlen(q, k, v, g, beta, cu, h0)
    assert np.array_equal(hT[1], h0[1])
    ref = np.einsum("thc,hcv->thv", q[0, 12:], h0[1])
    assert np.abs(o[0, 12:] - ref).max() < 1e-12


def test_channel_varlen_equal_lengths_equal_the_batch_axis():
    q, k, v, g, beta, h0 = _inputs(3, 7, 2, 8, 5, seed=10, h0=True)
    ro, rh = orc.recurrent_fwd_channel(q, k, v, g, beta, h0)
    pk = lambda a: a.reshape((1, 3 * 7) + a.shape[2:])
    o, hT = orc.recurrent_fwd_channel_varlen(pk(q), pk(k), pk(v), pk(g), pk(beta), [0, 7, 14, 21],
                                             h0)
    assert np.abs(o.reshape(ro.shape) - ro).max() < 1e-12
    assert np.abs(hT - rh).max() < 1e-12


def test_channel_varlen_carry_over_mutant_is_caught():
    # a packed runner that carries the state across the boundary fails the
    # boundary closed form
    q, k, v, g, beta, _ = _inputs(1, 20, 2, 8, 5, seed=9)
    h0 = np.random.default_rng(9).standard_normal((2, 2, 8, 5))
    beta[:, 12:] = 0.0
    g[:, 12:] = 0.0
    _, h_first = orc.recurrent_fwd_channel(q[:, :12], k[:, :12], v[:, :12], g[:, :12],
                                           beta[:, :12], h0[0:1])
    o_bad, _ = orc.recurrent_fwd_channel(q[:, 12:], k[:, 12:], v[:, 12:], g[:, 12:],
                                         beta[:, 12:], h_first)
    ref = np.einsum("thc,hcv->thv", q[0, 12:], h0[1])
    assert np.abs(o_bad[0] - ref).max() > 1e-3
