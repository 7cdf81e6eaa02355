"""GPU parity of the per-channel-gate forward (lin_attn_chunk_fwd_channel
through the C ABI) against the fp64 oracle recurrent_fwd_channel.

Error per output tensor: max |x - ref| / max |ref|.  Bars: 1e-5 for fp32
inputs (float32 throughout); 1e-2 on o and hT for bf16 inputs (the products
with the carried state run on bf16 matrix cores with a float32 state).  Gate regimes per channel: x ~ N(0,1) (sum of g per tile ~ -40),
x ~ N(-8,1) (weak decay: the state carries over thousands of tokens),
x ~ N(+4,2) and N(-4,2) (the stress variants), g = -5 and g = 0 exactly, and
channels alternating between -5 and 0.
"""

import numpy as np
import pytest
import torch

from chunked_gated_linear_amd import inputs as I
from chunked_gated_linear_amd import (lin_attn_chunk_fwd, lin_attn_chunk_fwd_channel,
                                      lin_attn_decode_step_channel)
from oracle import c_recurrent as crec
from oracle import linattn_oracle as orc

from parity_util import host, relerr, say

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

REG = {"std": (0.0, 1.0), "weak": (-8.0, 1.0), "stress_plus": (4.0, 2.0),
       "stress_minus": (-4.0, 2.0)}


def make(B, T, H, Dk, Dv, dtype, regime, mode, h0_std, seed):
    inp = I.make_inputs(B, T, H, Dk, Dv, dtype=dtype, seed=seed, device="cuda", h0_std=h0_std)
    if regime in ("zero", "min", "split"):
        assert mode == "log"
        c = torch.arange(Dk, device="cuda")
        val = {"zero": torch.zeros(Dk, device="cuda"), "min": torch.full((Dk,), -5.0, device="cuda"),
               "split": torch.where(c % 2 == 0, -5.0, 0.0)}[regime]
        gate = val.expand(B, T, H, Dk).contiguous()
        g64 = host(gate).astype(np.float64)
    else:
        mu, sd = REG[regime]
        x = I.make_channel_gate(B, T, H, Dk, seed=seed, device="cuda", mu=mu, std=sd)
        if mode == "logit":
            gate = x
            g64 = orc.bounded_gate(host(x).astype(np.float64))
        else:
            gate = torch.from_numpy(orc.bounded_gate(host(x).astype(np.float64))
                                    .astype(np.float32)).cuda()
            g64 = host(gate).astype(np.float64)
    h0 = None if inp["h0"] is None else host(inp["h0"]).astype(np.float64)
    host_args = (host(inp["q"]), host(inp["k"]), host(inp["v"]), g64,
                 host(inp["beta"]).astype(np.float64), h0)
    return inp, gate, host_args


CASES = [
    # dtype, Dk, Dv, B, H, T, regime, mode, h0_std
    ("fp32", 64, 64, 1, 2, 256, "std", "logit", None),        # the tiny workload's shape
    ("fp32", 64, 32, 2, 2, 37, "weak", "logit", 0.02),         # ragged tail, h0
    ("fp32", 128, 128, 1, 2, 160, "weak", "log", 0.02),
    ("fp32", 64, 16, 1, 3, 48, "min", "log", 0.02),            # g = -5: exp(80) at the bound
    ("fp32", 64, 48, 1, 1, 40, "zero", "log", 0.02),
    ("fp32", 128, 64, 1, 2, 70, "split", "log", 0.02),
    ("bf16", 128, 128, 1, 2, 300, "weak", "logit", 0.02),
    ("bf16", 128, 128, 2, 2, 16 * 9 + 5, "std", "logit", None),
    ("bf16", 128, 128, 1, 2, 200, "stress_plus", "logit", 0.02),
    ("bf16", 128, 128, 1, 2, 200, "stress_minus", "logit", 0.02),
    ("bf16", 64, 256, 1, 1, 33, "weak", "logit", 0.02),
    ("bf16", 128, 128, 1, 2, 1, "std", "logit", 0.02),
    ("bf16", 128, 128, 1, 2, 16, "std", "logit", 0.02),
    # bf16 records are consumed three tiles per epoch: tile counts of every
    # residue mod 3, one partial epoch, and whole epochs only
    ("bf16", 128, 128, 1, 2, 32, "weak", "logit", 0.02),       # 2 tiles
    ("bf16", 128, 128, 2, 1, 64, "std", "logit", 0.02),        # 4 tiles
    ("bf16", 128, 64, 1, 2, 80, "std", "log", 0.02),           # 5 tiles
    ("bf16", 64, 128, 1, 2, 96, "weak", "logit", None),        # 6 tiles, two whole epochs
    # at least two workgroups per compute unit: two tiles per epoch, the chain
    # forms the outputs, two workgroups share a unit
    ("bf16", 128, 128, 4, 16, 70, "weak", "logit", 0.02),
    ("bf16", 64, 128, 2, 32, 40, "std", "log", None),
    # pair path, one 16-column slice per head (the L2 prefetch lines and v rows
    # of a narrow slice) and a ragged end
    ("bf16", 128, 16, 1, 2, 100, "std", "logit", 0.02),
    ("bf16", 64, 16, 2, 3, 77, "weak", "logit", None),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(map(str, c)))
def test_channel_parity(case):
    dtype, Dk, Dv, B, H, T, regime, mode, h0_std = case
    say(f"channel {case}")
    inp, gate, host_args = make(B, T, H, Dk, Dv, dtype, regime, mode, h0_std, seed=41)
    o, hT = lin_attn_chunk_fwd_channel(inp["q"], inp["k"], inp["v"], gate, inp["beta"],
                                       inp["h0"], gate_mode=mode, G=5.0)
    torch.cuda.synchronize()
    ro, rh = orc.recurrent_fwd_channel(*host_args)
    eo, eh = relerr(host(o), ro), relerr(host(hT), rh)
    say(f"  err(o)={eo:.2e} err(hT)={eh:.2e}")
    assert np.isfinite(host(o)).all() and np.isfinite(host(hT)).all()
    tol = 1e-5 if dtype == "fp32" else 1e-2
    assert eo <= tol and eh <= tol


def test_channel_constant_gate_matches_scalar_path():
    # the same log-decay on every channel is the scalar gate: the per-channel
    # pass agrees with lin_attn_chunk_fwd (fp32) to the fp32 bar
    B, T, H, D = 1, 100, 2, 64
    inp = I.make_inputs(B, T, H, D, D, dtype="fp32", seed=43, device="cuda", gate_mu=-3.0,
                        h0_std=0.02)
    o1, h1 = lin_attn_chunk_fwd(inp["q"], inp["k"], inp["v"], inp["x"], inp["beta"], inp["h0"],
                                gate_mode="logit")
    xc = inp["x"][..., None].expand(B, T, H, D).contiguous()
    o2, h2 = lin_attn_chunk_fwd_channel(inp["q"], inp["k"], inp["v"], xc, inp["beta"],
                                        inp["h0"], gate_mode="logit")
    torch.cuda.synchronize()
    assert relerr(host(o2), host(o1).astype(np.float64)) <= 1e-5
    assert relerr(host(h2), host(h1).astype(np.float64)) <= 1e-5


def test_channel_deterministic_and_hT_optional():
    inp, gate, _ = make(1, 77, 2, 128, 64, "bf16", "std", "logit", 0.02, seed=44)
    a = lin_attn_chunk_fwd_channel(inp["q"], inp["k"], inp["v"], gate, inp["beta"], inp["h0"],
                                   gate_mode="logit")
    b = lin_attn_chunk_fwd_channel(inp["q"], inp["k"], inp["v"], gate, inp["beta"], inp["h0"],
                                   gate_mode="logit", output_final_state=False)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and b[1] is None


@pytest.mark.parametrize("regime", ["std", "weak"])
def test_channel_long_64k_every_head(regime):
    # the 64K x 16-head shape in bf16: every output of every head against the
    # C copy of the per-channel recurrence
    B, T, H, D = 1, 65536, 16, 128
    say(f"channel long_64k {regime}")
    inp, gate, host_args = make(B, T, H, D, D, "bf16", regime, "logit", None, seed=1002)
    o, hT = lin_attn_chunk_fwd_channel(inp["q"], inp["k"], inp["v"], gate, inp["beta"], None,
                                       gate_mode="logit", G=5.0)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(o.float()).all()) and bool(torch.isfinite(hT).all())
    ro, rh = crec.recurrent_fwd_channel(*host_args, workers=16)
    eo = relerr(host(o), ro)
    eh = relerr(host(hT), rh)
    say(f"  all 16 heads: err(o)={eo:.2e} err(hT)={eh:.2e}")
    assert eo <= 1e-2 and eh <= 1e-2


@pytest.mark.parametrize("B,H,T,Dk,Dv", [(2, 2, 16 * 1024 + 37, 128, 64), (1, 3, 20000, 128, 128),
                                         (1, 2, 17000, 64, 16)])
def test_channel_stretched_long_sequences(B, H, T, Dk, Dv):
    # bf16 sequences of 512 pairs or more with few heads run in stretches: the
    # state crosses each cut through the workspace; every output and the final
    # state against the C copy of the per-channel recurrence, with h0 and a
    # ragged end
    say(f"channel stretched B={B} H={H} T={T} Dk={Dk} Dv={Dv}")
    inp, gate, host_args = make(B, T, H, Dk, Dv, "bf16", "weak", "logit", 0.02, seed=1003)
    o, hT = lin_attn_chunk_fwd_channel(inp["q"], inp["k"], inp["v"], gate, inp["beta"], inp["h0"],
                                       gate_mode="logit", G=5.0)
    torch.cuda.synchronize()
    ro, rh = crec.recurrent_fwd_channel(*host_args, workers=16)
    eo, eh = relerr(host(o), ro), relerr(host(hT), rh)
    say(f"  err(o)={eo:.2e} err(hT)={eh:.2e}")
    assert eo <= 1e-2 and eh <= 1e-2


def test_channel_hT_in_place_of_h0():
    inp, gate, host_args = make(1, 70, 2, 128, 64, "fp32", "weak", "logit", 0.02, seed=45)
    h = inp["h0"].clone()
    o, hT = lin_attn_chunk_fwd_channel(inp["q"], inp["k"], inp["v"], gate, inp["beta"], h,
                                       gate_mode="logit", hT=h)
    torch.cuda.synchronize()
    ro, rh = orc.recurrent_fwd_channel(*host_args)
    assert hT.data_ptr() == h.data_ptr()
    assert relerr(host(o), ro) <= 1e-5 and relerr(host(h), rh) <= 1e-5


@pytest.mark.parametrize("dtype,Dk,Dv", [("fp32", 64, 64), ("fp32", 128, 64), ("bf16", 64, 128),
                                         ("bf16", 128, 128)])
def test_decode_channel_parity(dtype, Dk, Dv):
    # three decode steps from a random state, every output and the state
    # against the fp64 per-channel step
    B, H, steps = 3, 5, 3
    say(f"decode channel {dtype} {Dk} {Dv}")
    inp = I.make_inputs(B, steps, H, Dk, Dv, dtype=dtype, seed=46, device="cuda", h0_std=0.02)
    x = I.make_channel_gate(B, steps, H, Dk, seed=46, device="cuda")
    S = inp["h0"].clone()
    S_ref = host(S).astype(np.float64)
    tol = 1e-5 if dtype == "fp32" else 1e-2
    for t in range(steps):
        o = lin_attn_decode_step_channel(inp["q"][:, t].contiguous(), inp["k"][:, t].contiguous(),
                                         inp["v"][:, t].contiguous(), x[:, t].contiguous(),
                                         inp["beta"][:, t].contiguous(), S, gate_mode="logit")
        torch.cuda.synchronize()
        ro, S_ref = orc.decode_step_channel(host(inp["q"][:, t]), host(inp["k"][:, t]),
                                            host(inp["v"][:, t]),
                                            orc.bounded_gate(host(x[:, t]).astype(np.float64)),
                                            host(inp["beta"][:, t]), S_ref)
        assert relerr(host(o), ro) <= tol
    assert relerr(host(S), S_ref) <= 1e-5


def test_channel_prefill_hands_off_to_decode():
    # per-channel prefill of 40 tokens, then 3 decode steps from its hT: the
    # same outputs as one prefill over the 43 tokens (the oracle decides both)
    B, T1, T2, H, D = 2, 40, 3, 2, 128
    inp = I.make_inputs(B, T1 + T2, H, D, D, dtype="bf16", seed=47, device="cuda")
    x = I.make_channel_gate(B, T1 + T2, H, D, seed=47, device="cuda", mu=-3.0)
    sl = lambda a: a[:, :T1].contiguous()
    _, hT = lin_attn_chunk_fwd_channel(sl(inp["q"]), sl(inp["k"]), sl(inp["v"]), sl(x),
                                       sl(inp["beta"]), None, gate_mode="logit")
    outs = []
    for t in range(T1, T1 + T2):
        outs.append(lin_attn_decode_step_channel(
            inp["q"][:, t].contiguous(), inp["k"][:, t].contiguous(), inp["v"][:, t].contiguous(),
            x[:, t].contiguous(), inp["beta"][:, t].contiguous(), hT, gate_mode="logit"))
    torch.cuda.synchronize()
    g = orc.bounded_gate(host(x).astype(np.float64))
    ro, rh = orc.recurrent_fwd_channel(host(inp["q"]), host(inp["k"]), host(inp["v"]), g,
                                       host(inp["beta"]).astype(np.float64), None)
    got = np.stack([host(o) for o in outs], axis=1)
    assert relerr(got, ro[:, T1:]) <= 1e-2
    assert relerr(host(hT), rh) <= 1e-2


def test_channel_graph_capture_replays():
    """The per-channel forward (two launches) and decode steps captured in one
    graph replay to the eager results, replay after replay, with eager work
    and synchronisations between the replays."""
    from chunked_gated_linear_amd import lin_attn_chunk_fwd_channel_workspace_size
    say("graph capture: per-channel forward B1 H4 T3000 + 2 decode steps, 3 replays")
    inp, gate, _ = make(1, 3000, 4, 128, 128, "bf16", "weak", "logit", 0.02, seed=48)
    ws = torch.empty(lin_attn_chunk_fwd_channel_workspace_size(1, 3000, 4, 128, 128),
                     dtype=torch.uint8, device="cuda")
    o = torch.empty_like(inp["v"])
    hT = torch.empty((1, 4, 128, 128), dtype=torch.float32, device="cuda")
    d = I.make_decode_inputs(8, 4, 128, 128, dtype="bf16", seed=49, device="cuda", steps=2)
    xd = I.make_channel_gate(2, 8, 4, 128, seed=49, device="cuda")
    S0 = d["S"].clone()
    S = S0.clone()
    od = torch.empty((8, 4, 128), dtype=torch.bfloat16, device="cuda")

    def work():
        lin_attn_chunk_fwd_channel(inp["q"], inp["k"], inp["v"], gate, inp["beta"], inp["h0"],
                                   gate_mode="logit", o=o, hT=hT, workspace=ws)
        for st in range(2):
            lin_attn_decode_step_channel(d["q"][st], d["k"][st], d["v"][st], xd[st], d["beta"][st],
                                         S, gate_mode="logit", o=od)

    work()
    torch.cuda.synchronize()
    o_ref, h_ref, S_ref, od_ref = o.clone(), hT.clone(), S.clone(), od.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        S.copy_(S0)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=side):
            work()
    torch.cuda.synchronize()
    for rep in range(3):
        o.zero_()
        hT.zero_()
        S.copy_(S0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref) and torch.equal(hT, h_ref), rep
        assert torch.equal(S, S_ref) and torch.equal(od, od_ref), rep
        lin_attn_chunk_fwd_channel(inp["q"], inp["k"], inp["v"], gate, inp["beta"], None,
                                   gate_mode="logit")          # eager work between replays


def _packed(lengths, H, Dk, Dv, dtype, seed, mu=-3.0, h0_std=0.02):
    T = int(sum(lengths))
    inp = I.make_inputs(1, T, H, Dk, Dv, dtype=dtype, seed=seed, device="cuda")
    x = I.make_channel_gate(1, T, H, Dk, seed=seed, device="cuda", mu=mu)
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lengths)]), dtype=torch.int32, device="cuda")
    h0 = h0_std * torch.randn((len(lengths), H, Dk, Dv), device="cuda",
                              generator=torch.Generator("cuda").manual_seed(seed))
    return inp, x, cu, h0


@pytest.mark.parametrize("dtype,Dk,Dv,lengths", [
    ("fp32", 64, 32, [17, 0, 40, 1, 33]),
    ("bf16", 128, 128, [100, 0, 16, 5, 250, 0]),
    ("bf16", 64, 256, [48, 31]),
    ("bf16", 128, 128, [32, 80, 96, 64, 1, 47]),               # 2, 5, 6, 4, 1, 3 tiles
])
def test_channel_varlen_parity(dtype, Dk, Dv, lengths):
    from chunked_gated_linear_amd import lin_attn_chunk_fwd_channel_varlen
    say(f"channel varlen {dtype} {Dk} {Dv} {lengths}")
    H = 2
    inp, x, cu, h0 = _packed(lengths, H, Dk, Dv, dtype, seed=51)
    o, hT = lin_attn_chunk_fwd_channel_varlen(inp["q"], inp["k"], inp["v"], x, inp["beta"], cu,
                                              h0, gate_mode="logit")
    torch.cuda.synchronize()
    g = orc.bounded_gate(host(x).astype(np.float64))
    ro, rh = orc.recurrent_fwd_channel_varlen(host(inp["q"]), host(inp["k"]), host(inp["v"]), g,
                                              host(inp["beta"]).astype(np.float64),
                                              host(cu).astype(np.int64),
                                              host(h0).astype(np.float64))
    tol = 1e-5 if dtype == "fp32" else 1e-2
    eo, eh = relerr(host(o), ro), relerr(host(hT), rh)
    say(f"  err(o)={eo:.2e} err(hT)={eh:.2e}")
    assert eo <= tol and eh <= tol


def test_channel_varlen_equal_lengths_match_the_batched_call_bitwise():
    from chunked_gated_linear_amd import lin_attn_chunk_fwd_channel_varlen
    B, T, H, D = 3, 70, 2, 128
    inp = I.make_inputs(B, T, H, D, D, dtype="bf16", seed=52, device="cuda", h0_std=0.02)
    x = I.make_channel_gate(B, T, H, D, seed=52, device="cuda", mu=-3.0)
    ob, hb = lin_attn_chunk_fwd_channel(inp["q"], inp["k"], inp["v"], x, inp["beta"], inp["h0"],
                                        gate_mode="logit")
    pk = lambda a: a.reshape((1, B * T) + tuple(a.shape[2:])).contiguous()
    cu = torch.arange(0, B * T + 1, T, dtype=torch.int32, device="cuda")
    ov, hv = lin_attn_chunk_fwd_channel_varlen(pk(inp["q"]), pk(inp["k"]), pk(inp["v"]), pk(x),
                                               pk(inp["beta"]), cu, inp["h0"], gate_mode="logit")
    torch.cuda.synchronize()
    assert torch.equal(ov.reshape(ob.shape), ob) and torch.equal(hv, hb)


def test_channel_varlen_serving_batch_sampled():
    # the packed prefill workload (64 log-normal requests, 64K tokens, 16 heads)
    # with a per-channel gate: three requests of head 5 against the oracle
    from chunked_gated_linear_amd import lin_attn_chunk_fwd_channel_varlen
    vw = I.VARLEN_WORKLOAD
    lengths = I.varlen_lengths(vw["nseq"], vw["T"], seed=1006)
    say("channel varlen serving batch")
    inp, x, cu, _ = _packed(lengths, vw["H"], vw["Dk"], vw["Dv"], "bf16", seed=1006, mu=0.0)
    o, hT = lin_attn_chunk_fwd_channel_varlen(inp["q"], inp["k"], inp["v"], x, inp["beta"], cu,
                                              None, gate_mode="logit")
    torch.cuda.synchronize()
    cuh = [0] + list(np.cumsum(lengths))
    h = 5
    for s in (0, 17, 63):
        a, b = cuh[s], cuh[s + 1]
        sl = (slice(None), slice(a, b), slice(h, h + 1))
        ro, rh = orc.recurrent_fwd_channel(host(inp["q"][sl]), host(inp["k"][sl]),
                                           host(inp["v"][sl]),
                                           orc.bounded_gate(host(x[sl]).astype(np.float64)),
                                           host(inp["beta"][sl]).astype(np.float64), None)
        eo = relerr(host(o[sl]), ro)
        eh = relerr(host(hT[s:s + 1, h:h + 1]), rh)
        say(f"  request {s} ({b - a} tokens): err(o)={eo:.2e} err(hT)={eh:.2e}")
        assert eo <= 1e-2 and eh <= 1e-2
