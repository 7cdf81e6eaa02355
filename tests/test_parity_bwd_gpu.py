"""GPU parity of the reverse pass (lin_attn_chunk_bwd through the C ABI)
against the oracle's fp64 adjoint of the recurrence.

Small cases compare every gradient element; the 64K x 16-head shape compares
the last three tiles of every head (their gradients depend only on the tokens
after them and on dhT, so the oracle runs from the state the fp64 forward
recurrence reaches there).

Bars, max|x - ref| / max|ref| per gradient tensor:
  float32 inputs: 1e-5, the float32 bar of the forward pass (float32
    products on the float32 matrix cores throughout);
  bf16 inputs: 5e-5.  These run on the bf16 matrix cores with every float32
    operand split into bf16 hi + lo parts, each carrying a relative error of
    at most 2^-16 ~ 1.5e-5 (the inputs themselves enter exactly), and the
    products and sums over d_k, d_v and 16 tokens add a few of those.  The
    forward pass holds bf16 inputs to 1e-2.
"""

import numpy as np
import pytest
import torch

from chunked_gated_linear_amd import lin_attn_chunk_bwd
from chunked_gated_linear_amd import inputs as I
from oracle import c_recurrent as crec
from oracle import linattn_oracle as orc

from parity_util import host, make_case, relerr, say

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

TOL_BWD = 1e-5          # float32 inputs
TOL_BWD_BF16 = 5e-5     # bf16 inputs (split bf16 products)


def tol(dtype):
    return TOL_BWD_BF16 if dtype == "bf16" else TOL_BWD
NAMES = ("dq", "dk", "dv", "dgate", "dbeta", "dh0")


def run_bwd(a, up, out_dh0=True):
    res = lin_attn_chunk_bwd(a["q"], a["k"], a["v"], a["gate"], a["beta"], up["dout"], a["h0"],
                             up["dhT"], gate_mode=a["gate_mode"], G=5.0, output_dh0=out_dh0)
    torch.cuda.synchronize()
    return res


def oracle_grads(host_args, dev_args, up, t_range=None, h_start=None):
    q, k, v, g, beta, h0 = host_args
    do = host(up["dout"]).astype(np.float64)
    dhT = None if up["dhT"] is None else host(up["dhT"]).astype(np.float64)
    sl = slice(None) if t_range is None else slice(*t_range)
    init = h0 if t_range is None else h_start
    dq, dk, dv, dg, db, dh0 = orc.recurrent_bwd(q[:, sl], k[:, sl], v[:, sl], g[:, sl],
                                                beta[:, sl], do[:, sl], dhT, init)
    if dev_args["gate_mode"] == "logit":
        dg = orc.bounded_gate_bwd(host(dev_args["gate"]).astype(np.float64)[:, sl], dg)
    return dq, dk, dv, dg, db, dh0


CASES = [
    # dtype, Dk, Dv, B, H, T, regime, mode, h0_std, dhT
    ("fp32", 64, 32, 1, 2, 37, "std", "log", 0.02, True),
    ("fp32", 128, 128, 1, 2, 100, "weak", "logit", 0.02, True),
    ("bf16", 128, 128, 2, 2, 16 * 9 + 5, "std", "logit", None, False),
    ("bf16", 128, 128, 1, 2, 300, "weak", "logit", 0.02, True),
    ("bf16", 128, 128, 1, 2, 200, "stress_plus", "logit", 0.02, True),
    ("bf16", 128, 128, 1, 2, 200, "stress_minus", "logit", 0.02, True),
    ("bf16", 128, 64, 1, 2, 64, "zero", "log", 0.02, True),
    ("bf16", 64, 48, 1, 3, 50, "min", "log", None, True),
    ("bf16", 128, 128, 1, 1, 1, "std", "logit", 0.02, True),
    ("bf16", 128, 128, 1, 2, 16, "std", "logit", 0.02, True),
    ("bf16", 128, 256, 1, 1, 40, "weak", "logit", 0.02, True),
    # d_v / 16 even but not a multiple of 4: two slices per state block
    ("bf16", 128, 96, 1, 2, 16 * 11 + 3, "weak", "logit", 0.02, True),
    ("bf16", 64, 32, 2, 1, 77, "std", "log", None, True),
    # d_k 64 with four slices per state block
    ("bf16", 64, 128, 1, 2, 16 * 7 + 9, "weak", "logit", 0.02, True),
    ("bf16", 64, 64, 2, 1, 200, "std", "logit", None, False),
    # more state workgroups than compute units: 68 heads at d_v = 128 make
    # 272 chain workgroups of one per unit, so the launch takes two rounds;
    # 7 tiles, the last ragged (the gradient chain's empty front tile)
    ("bf16", 128, 128, 1, 68, 16 * 6 + 4, "weak", "logit", 0.02, True),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(map(str, c)))
def test_bwd_parity(case):
    dtype, Dk, Dv, B, H, T, regime, mode, h0_std, with_dhT = case
    say(f"bwd parity {case}")
    dev_args, host_args = make_case(B, T, H, Dk, Dv, dtype, regime, mode, h0_std=h0_std, seed=T)
    up = I.make_upstream_grads(B, T, H, Dk, Dv, dtype=dtype, seed=T, device="cuda", dhT=with_dhT)
    got = run_bwd(dev_args, up)
    ref = oracle_grads(host_args, dev_args, up)
    errs = {}
    for name, x, r in zip(NAMES, got, ref):
        xh = host(x)
        assert np.all(np.isfinite(xh)), name
        errs[name] = relerr(xh, r)
    say("  " + " ".join(f"{n}={e:.2e}" for n, e in errs.items()))
    for name, e in errs.items():
        assert e <= tol(dtype), f"{name}: error {e}"


def test_bwd_empty_sequence_copies_dhT():
    say("bwd T=0")
    dev_args, _ = make_case(1, 0, 2, 128, 64, "bf16", "std", "logit", h0_std=0.02, seed=3)
    up = I.make_upstream_grads(1, 0, 2, 128, 64, dtype="bf16", seed=3, device="cuda")
    dq, dk, dv, dg, db, dh0 = run_bwd(dev_args, up)
    assert dq.numel() == 0 and dg.numel() == 0
    assert torch.equal(dh0, up["dhT"])


def test_bwd_is_deterministic_and_dh0_optional():
    say("bwd determinism")
    dev_args, _ = make_case(1, 133, 2, 128, 128, "bf16", "weak", "logit", h0_std=0.02, seed=5)
    up = I.make_upstream_grads(1, 133, 2, 128, 128, dtype="bf16", seed=5, device="cuda")
    a = run_bwd(dev_args, up)
    b = run_bwd(dev_args, up, out_dh0=False)
    for x, y in zip(a[:5], b[:5]):
        assert torch.equal(x, y)
    assert b[5] is None


def test_bwd_long_64k_tail_tiles():
    # the 64K x 16-head shape: every gradient finite, and the last 3 tiles of
    # every head against the oracle started from the fp64 state at T - 48
    B, T, H, D = 1, 65536, 16, 128
    say("bwd long_64k")
    dev_args, host_args = make_case(B, T, H, D, D, "bf16", "std", "logit", seed=1002)
    up = I.make_upstream_grads(B, T, H, D, D, dtype="bf16", seed=1002, device="cuda")
    got = run_bwd(dev_args, up)
    for name, x in zip(NAMES, got):
        assert bool(torch.isfinite(x).all()), name
    t0 = T - 48
    q, k, v, g, beta, _ = host_args
    _, h_start = crec.recurrent_fwd(q[:, :t0], k[:, :t0], v[:, :t0], g[:, :t0], beta[:, :t0],
                                    None, workers=16)
    ref = oracle_grads(host_args, dev_args, up, t_range=(t0, T), h_start=h_start)
    for name, x, r in zip(NAMES[:5], got[:5], ref[:5]):
        e = relerr(host(x[:, t0:]), r)
        say(f"  {name} tail err={e:.2e}")
        assert e <= TOL_BWD_BF16, f"{name}: error {e}"


def test_bwd_graph_capture_replays():
    """The reverse pass (four launches) captured in a graph replays to the
    eager gradients, replay after replay, with eager work between replays."""
    from chunked_gated_linear_amd import lin_attn_chunk_bwd_workspace_size
    say("graph capture: reverse pass B1 H2 T600, 3 replays")
    B, T, H, D = 1, 600, 2, 128
    dev_args, _ = make_case(B, T, H, D, D, "bf16", "weak", "logit", 0.02, seed=50)
    up = I.make_upstream_grads(B, T, H, D, D, dtype="bf16", seed=50, device="cuda")
    ws = torch.empty(lin_attn_chunk_bwd_workspace_size(B, T, H, D, D), dtype=torch.uint8,
                     device="cuda")

    def work():
        return lin_attn_chunk_bwd(dev_args["q"], dev_args["k"], dev_args["v"], dev_args["gate"],
                                  dev_args["beta"], up["dout"], dev_args["h0"], up["dhT"],
                                  gate_mode="logit", G=5.0, workspace=ws)

    ref = [x.clone() for x in work()]
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=side):
            outs = work()
    torch.cuda.synchronize()
    for rep in range(3):
        for x in outs:
            x.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, x, r in zip(NAMES, outs, ref):
            assert torch.equal(x, r), (name, rep)
        run_bwd(dev_args, up)                     # eager work between replays


# ------------------------------------------------------- packed sequences
VARLEN_BWD = [
    # dtype, Dk, Dv, H, sequence lengths, gate mode
    ("bf16", 128, 128, 2, [0, 1, 17, 40, 100, 33, 64], "logit"),
    ("fp32", 64, 32, 3, [5, 0, 48, 77], "log"),
    ("bf16", 64, 96, 3, [130, 0, 7, 64, 201], "log"),
]


@pytest.mark.parametrize("case", VARLEN_BWD, ids=lambda c: f"{c[0]}-d{c[1]}x{c[2]}-n{len(c[4])}")
def test_bwd_varlen_parity(case):
    """The packed reverse pass against the oracle's adjoint run on each
    sequence alone (from its own h0 and dhT); empty sequences pass dhT to dh0."""
    from chunked_gated_linear_amd import lin_attn_chunk_bwd_varlen
    dtype, Dk, Dv, H, lengths, mode = case
    T, nseq = int(sum(lengths)), len(lengths)
    say(f"bwd varlen {case}")
    dev_args, host_args = make_case(1, T, H, Dk, Dv, dtype, "weak", mode, h0_std=None, seed=71)
    up = I.make_upstream_grads(1, T, H, Dk, Dv, dtype=dtype, seed=71, device="cuda", dhT=False)
    gen = torch.Generator(device="cuda").manual_seed(72)
    h0 = 0.02 * torch.randn((nseq, H, Dk, Dv), generator=gen, device="cuda")
    dhT = torch.randn((nseq, H, Dk, Dv), generator=gen, device="cuda")
    cu_h = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    cu = torch.tensor(cu_h, dtype=torch.int32, device="cuda")
    got = lin_attn_chunk_bwd_varlen(dev_args["q"], dev_args["k"], dev_args["v"], dev_args["gate"],
                                    dev_args["beta"], up["dout"], cu, h0, dhT, gate_mode=mode)
    torch.cuda.synchronize()
    q, k, v, g, beta, _ = host_args
    do = host(up["dout"]).astype(np.float64)
    x = host(dev_args["gate"]).astype(np.float64)
    h0_h, dhT_h = host(h0).astype(np.float64), host(dhT).astype(np.float64)
    ref = [np.zeros((1, T, H, Dk)), np.zeros((1, T, H, Dk)), np.zeros((1, T, H, Dv)),
           np.zeros((1, T, H)), np.zeros((1, T, H)), np.zeros((nseq, H, Dk, Dv))]
    for s_ in range(nseq):
        a_, b_ = cu_h[s_], cu_h[s_ + 1]
        if a_ == b_:
            ref[5][s_] = dhT_h[s_]
            continue
        sl = slice(a_, b_)
        dq, dk, dv, dg, db, dh0 = orc.recurrent_bwd(q[:, sl], k[:, sl], v[:, sl], g[:, sl],
                                                    beta[:, sl], do[:, sl], dhT_h[s_:s_ + 1],
                                                    h0_h[s_:s_ + 1])
        if mode == "logit":
            dg = orc.bounded_gate_bwd(x[:, sl], dg)
        for r_, val in zip(ref[:5], (dq, dk, dv, dg, db)):
            r_[:, sl] = val
        ref[5][s_] = dh0[0]
    errs = {}
    for name, xg, r in zip(NAMES, got, ref):
        xh = host(xg)
        assert np.all(np.isfinite(xh)), name
        errs[name] = relerr(xh, r)
    say("  " + " ".join(f"{n}={e:.2e}" for n, e in errs.items()))
    for name, e in errs.items():
        assert e <= tol(dtype), f"{name}: error {e}"
    for s_, n_ in enumerate(lengths):
        if n_ == 0:
            assert torch.equal(got[5][s_], dhT[s_])


def test_bwd_varlen_equal_lengths_match_batched_bitwise():
    """Equal lengths: the packed reverse pass reproduces the batched one bit
    for bit (the same per-tile work in the same order)."""
    from chunked_gated_linear_amd import lin_attn_chunk_bwd_varlen
    N_, L_, H = 3, 150, 2
    say("bwd varlen vs batched: 3 x 150 tokens H2 d128 bf16")
    dev_args, _ = make_case(N_, L_, H, 128, 128, "bf16", "weak", "logit", h0_std=0.02, seed=73)
    up = I.make_upstream_grads(N_, L_, H, 128, 128, dtype="bf16", seed=73, device="cuda")
    ref = run_bwd(dev_args, up)
    pk = lambda t: t.reshape((1, N_ * L_) + tuple(t.shape[2:]))
    cu = torch.tensor([0, L_, 2 * L_, 3 * L_], dtype=torch.int32, device="cuda")
    got = lin_attn_chunk_bwd_varlen(pk(dev_args["q"]), pk(dev_args["k"]), pk(dev_args["v"]),
                                    pk(dev_args["gate"]), pk(dev_args["beta"]), pk(up["dout"]), cu,
                                    dev_args["h0"], up["dhT"], gate_mode="logit")
    torch.cuda.synchronize()
    for name, x, r in zip(NAMES, got, ref):
        assert torch.equal(x.reshape(r.shape), r), name


def test_bwd_varlen_all_empty_passes_dhT():
    """A packed batch of empty sequences (T = 0): dh0 is dhT, nothing else."""
    from chunked_gated_linear_amd import lin_attn_chunk_bwd_varlen
    say("bwd varlen: 3 empty sequences")
    nseq, H, D = 3, 2, 64
    e = lambda *s_, dt=torch.bfloat16: torch.empty(s_, dtype=dt, device="cuda")
    gen = torch.Generator(device="cuda").manual_seed(74)
    dhT = torch.randn((nseq, H, D, D), generator=gen, device="cuda")
    cu = torch.zeros(nseq + 1, dtype=torch.int32, device="cuda")
    got = lin_attn_chunk_bwd_varlen(e(1, 0, H, D), e(1, 0, H, D), e(1, 0, H, D),
                                    e(1, 0, H, dt=torch.float32), e(1, 0, H, dt=torch.float32),
                                    e(1, 0, H, D), cu, None, dhT, gate_mode="logit")
    torch.cuda.synchronize()
    assert got[0].numel() == 0 and torch.equal(got[5], dhT)


# ------------------------------------------- long chains, every gradient
def _c_grads(host_args, dev_args, up, heads):
    """The C adjoint on the listed (b, h) streams; in logit mode dg is taken
    through the bounded gate to dx."""
    q, k, v, g, beta, h0 = host_args
    do = host(up["dout"]).astype(np.float64)
    dhT = None if up["dhT"] is None else host(up["dhT"]).astype(np.float64)
    res = crec.recurrent_bwd_c(q, k, v, g, beta, do, dhT, h0, heads=heads, workers=16)
    if dev_args["gate_mode"] == "logit":
        x = host(dev_args["gate"]).astype(np.float64)
        for (b, h), r in res.items():
            r = list(r)
            r[3] = orc.bounded_gate_bwd(x[b, :, h], r[3])
            res[(b, h)] = tuple(r)
    return res


def _compare_heads(got, res):
    gh = [host(x) for x in got]
    worst = dict.fromkeys(NAMES, 0.0)
    for (b, h), r in res.items():
        for i, name in enumerate(NAMES):
            x = gh[i][b, h] if name == "dh0" else gh[i][b, :, h]
            assert np.all(np.isfinite(x)), name
            worst[name] = max(worst[name], relerr(x, r[i]))
    return worst


@pytest.mark.parametrize("shape", [(1, 4096, 2, "weak", 0.02, 1005),
                                   (4, 8192, 16, "std", None, 1001)],
                         ids=["weak_4k_B1_H2", "train_8k_B4_H16"])
def test_bwd_every_gradient_long(shape):
    """Every gradient of every head against the C adjoint: a weak-decay chain
    of 256 tiles (g ~ -0.002, the state gradient carried through every tile)
    and the benchmarked training shape."""
    B, T, H, regime, h0s, seed = shape
    say(f"bwd every gradient B{B} T{T} H{H} d128 bf16 {regime}")
    dev_args, host_args = make_case(B, T, H, 128, 128, "bf16", regime, "logit", h0_std=h0s,
                                    seed=seed)
    up = I.make_upstream_grads(B, T, H, 128, 128, dtype="bf16", seed=seed, device="cuda")
    got = run_bwd(dev_args, up)
    res = _c_grads(host_args, dev_args, up, [(b, h) for b in range(B) for h in range(H)])
    worst = _compare_heads(got, res)
    say("  " + " ".join(f"{n}={e:.2e}" for n, e in worst.items()))
    for name, e in worst.items():
        assert e <= TOL_BWD_BF16, f"{name}: error {e}"


def test_bwd_train_8k_weak_sampled_heads():
    """The training shape under weak decay (the state gradient carried through
    all 512 tiles), h0 and dhT given: three heads, every gradient and dh0."""
    B, T, H = 4, 8192, 16
    say("bwd train_8k weak, heads (0,0) (1,7) (3,15)")
    dev_args, host_args = make_case(B, T, H, 128, 128, "bf16", "weak", "logit", h0_std=0.02,
                                    seed=1011)
    up = I.make_upstream_grads(B, T, H, 128, 128, dtype="bf16", seed=1011, device="cuda")
    got = run_bwd(dev_args, up)
    res = _c_grads(host_args, dev_args, up, [(0, 0), (1, 7), (3, 15)])
    worst = _compare_heads(got, res)
    say("  " + " ".join(f"{n}={e:.2e}" for n, e in worst.items()))
    for name, e in worst.items():
        assert e <= TOL_BWD_BF16, f"{name}: error {e}"


def test_bwd_varlen_weak_8k():
    """A packed training batch of 8192 tokens (five sequences, one empty)
    under weak decay with h0 and dhT: every gradient of every sequence and
    head against the C adjoint run on each sequence alone."""
    from chunked_gated_linear_amd import lin_attn_chunk_bwd_varlen
    lengths, H, D = [3000, 17, 0, 4100, 1075], 4, 128
    T, nseq = int(sum(lengths)), len(lengths)
    say(f"bwd varlen weak {nseq} seqs T{T} H{H}")
    dev_args, host_args = make_case(1, T, H, D, D, "bf16", "weak", "logit", h0_std=None,
                                    seed=1012)
    up = I.make_upstream_grads(1, T, H, D, D, dtype="bf16", seed=1012, device="cuda", dhT=False)
    gen = torch.Generator(device="cuda").manual_seed(1013)
    h0 = 0.02 * torch.randn((nseq, H, D, D), generator=gen, device="cuda")
    dhT = torch.randn((nseq, H, D, D), generator=gen, device="cuda")
    cu_h = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    cu = torch.tensor(cu_h, dtype=torch.int32, device="cuda")
    got = lin_attn_chunk_bwd_varlen(dev_args["q"], dev_args["k"], dev_args["v"], dev_args["gate"],
                                    dev_args["beta"], up["dout"], cu, h0, dhT, gate_mode="logit")
    torch.cuda.synchronize()
    q, k, v, g, beta, _ = host_args
    do = host(up["dout"]).astype(np.float64)
    x = host(dev_args["gate"]).astype(np.float64)
    h0_h, dhT_h = host(h0).astype(np.float64), host(dhT).astype(np.float64)
    gh = [host(t) for t in got]
    worst = dict.fromkeys(NAMES, 0.0)
    for s_ in range(nseq):
        a_, b_ = int(cu_h[s_]), int(cu_h[s_ + 1])
        for h in range(H):
            if a_ == b_:
                assert np.array_equal(gh[5][s_, h], host(dhT)[s_, h])
                continue
            r = list(crec.head_bwd(q[0, a_:b_, h], k[0, a_:b_, h], v[0, a_:b_, h], g[0, a_:b_, h],
                                   beta[0, a_:b_, h], do[0, a_:b_, h], dhT_h[s_, h], h0_h[s_, h]))
            r[3] = orc.bounded_gate_bwd(x[0, a_:b_, h], r[3])
            for i, name in enumerate(NAMES):
                xg = gh[i][s_, h] if name == "dh0" else gh[i][0, a_:b_, h]
                worst[name] = max(worst[name], relerr(xg, r[i]))
    say("  " + " ".join(f"{n}={e:.2e}" for n, e in worst.items()))
    for name, e in worst.items():
        assert e <= TOL_BWD_BF16, f"{name}: error {e}"


# ------------------------------------------- segmented form (bounded workspace)
SEG_CASES = [
    # Dk, Dv, B, H, T, regime, mode, h0_std, dhT, segment_tokens
    (128, 128, 2, 2, 1000, "weak", "logit", 0.02, True, 256),
    (64, 96, 1, 3, 777, "std", "log", None, True, 192),
    (128, 48, 1, 2, 130, "weak", "logit", 0.02, True, 64),
    (128, 64, 1, 2, 300, "weak", "logit", 0.02, False, 512),     # one segment
]


@pytest.mark.parametrize("case", SEG_CASES, ids=lambda c: "-".join(map(str, c)))
def test_bwd_segmented_matches_one_pass_bitwise(case):
    """Segments of whole groups of four tiles put every tile, group and stored
    state where one pass over the sequence puts them, and the carried states
    are the float32 chain states themselves: the segmented reverse pass
    reproduces lin_attn_chunk_bwd bit for bit; the first case is also held to
    the oracle's adjoint."""
    Dk, Dv, B, H, T, regime, mode, h0_std, with_dhT, L = case
    say(f"bwd segmented {case}")
    dev_args, host_args = make_case(B, T, H, Dk, Dv, "bf16", regime, mode, h0_std=h0_std, seed=T)
    up = I.make_upstream_grads(B, T, H, Dk, Dv, dtype="bf16", seed=T, device="cuda", dhT=with_dhT)
    one = run_bwd(dev_args, up)
    seg = lin_attn_chunk_bwd(dev_args["q"], dev_args["k"], dev_args["v"], dev_args["gate"],
                             dev_args["beta"], up["dout"], dev_args["h0"], up["dhT"],
                             gate_mode=dev_args["gate_mode"], G=5.0, segment_tokens=L)
    torch.cuda.synchronize()
    for name, x, y in zip(NAMES, one, seg):
        assert torch.equal(x, y), name
    if case is SEG_CASES[0]:
        ref = oracle_grads(host_args, dev_args, up)
        errs = {name: relerr(host(x), r) for name, x, r in zip(NAMES, seg, ref)}
        say("  " + " ".join(f"{n}={e:.2e}" for n, e in errs.items()))
        for name, e in errs.items():
            assert e <= TOL_BWD_BF16, f"{name}: error {e}"
