"""Benchmark: chunked gated delta-rule linear-attention forward on one MI355X.

A step is one pass of the whole forward path (bounded gate from logits, the
in-tile cumulative decay, intra-tile products and solve, state propagation,
outputs and final state) over one batch of synthetic input resident in HBM.
Default workload: B=1, H=16, T=65536, d_k=d_v=128, bf16 q/k/v, fp32 gates and
state, 16-token tiles.  Prints ONE JSON line.

    python bench.py [--steps K] [--warmup W] [--workload long_64k]
                    [--decode-steps 1000] [--varlen-steps 20] [--no-cpu-baseline]
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "tokens/s + % bf16 MFMA peak, chunked linear-attn fwd H=16 d=128 T=64K"
PEAK_HBM = 8.0e12           # bytes/s, MI355X HBM3E
PEAK_BF16 = 2.5e15          # dense bf16 MFMA flop/s (published figure)
CHUNK = 16
CSRC = os.path.join(ROOT, "chunked_gated_linear_amd", "csrc")

# HBM traffic per call from the rocprofv3 FETCH_SIZE and WRITE_SIZE counters,
# in KiB as the counters read them (summed over the call's dispatches), for the kernels as they stood
# when the counters were taken (keyed by a hash of their sources).  A plain
# 1 GiB copy through the library reads 524319 KiB of FETCH_SIZE and 1048576 KiB
# of WRITE_SIZE, so reads are scaled by 2 and writes by 1.
FETCH_SCALE, WRITE_SCALE = 2.0, 1.0
TRAFFIC_KIB = {
    "chunk": {"sources": ("chunk_pair.hip", "la_device.h"),
              "sha256_16": "0cafb7645a20fa6c",
              # one call: the intra-tile launch and the 16 state launches of 64K x 16 heads
              "fetch": 776930, "write": 488455},
    "varlen": {"sources": ("chunk_pair.hip", "la_device.h"),
               "sha256_16": "0cafb7645a20fa6c",
               # one call on the 64-request packed batch (64K tokens, 16 heads)
               "fetch": 824922, "write": 546356},
    # the other rungs of the context ladder, one call each
    "ladder_train_8k": {"sources": ("chunk_pair.hip", "la_device.h"),
                        "sha256_16": "0cafb7645a20fa6c",
                        "fetch": 398611, "write": 254224},
    "ladder_long_256k": {"sources": ("chunk_pair.hip", "la_device.h"),
                         "sha256_16": "0cafb7645a20fa6c",
                         "fetch": 3150047, "write": 1905380},
    "ladder_million_1m": {"sources": ("chunk_pair.hip", "la_device.h"),
                          "sha256_16": "0cafb7645a20fa6c",
                          "fetch": 7724248, "write": 3823233},
    "channel": {"sources": ("chunk_channel.hip", "chunk_channel_pair.hip", "la_device.h"),
                "sha256_16": "0f24b3a4c5929fde",
                # one call at 64K x 16 heads: the pair preparation of stretch 0 and
                # the 16 stretch launches (state + next stretch's preparation)
                "fetch": 1224072, "write": 1277957},
    "channel_varlen": {"sources": ("chunk_channel.hip", "chunk_channel_pair.hip", "la_device.h"),
                       "sha256_16": "0f24b3a4c5929fde",
                       # one call on the 64-request packed batch with a per-channel
                       # gate: the 16-token preparation and state launches
                       "fetch": 1391772, "write": 1591826},
    "backward": {"sources": ("chunk_bwd_bf16.hip", "chunk_bwd_bf16_states.hip", "la_bwd_bf16.h", "la_bwd.h",
                             "la_device.h", "../build.py"),
                 "sha256_16": "5bf4829476362ab1",
                 # one call at B=4 H=16 T=8192: tile records, states + state
                 # gradients (one launch), gradients
                 "fetch": 2153326, "write": 2493887},
    "decode_channel": {"sources": ("chunk_channel.hip", "la_device.h"),
                       "sha256_16": "7fa2297eef5c7589",
                       # one step at B=256 H=32 d=128 with a per-channel gate (median of six)
                       "fetch": 267548, "write": 527096},
    "decode": {"sources": ("decode.hip", "la_device.h"),
               "sha256_16": "f8c6337c80342a66",
               # one step at B=256 H=32 d=128 (median of six dispatches)
               "fetch": 265754, "write": 526921},
}


def host_info():
    """CPU model, core count and OpenMP thread setting of the host."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            model = next((ln.split(":", 1)[1].strip() for ln in fh if ln.startswith("model name")),
                         model)
    except OSError:
        pass
    return {"nproc": os.cpu_count(), "cpu_model": model,
            "omp_num_threads": os.environ.get("OMP_NUM_THREADS")}


def source_hash(names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(CSRC, n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(which, workload=None):
    """Counter-derived HBM bytes per call, or None once the kernels changed (or
    for a workload other than the one the counters were taken on)."""
    t = TRAFFIC_KIB.get(which)
    if t is None:
        return None
    if which == "chunk" and workload != "long_64k":
        return None
    if source_hash(t["sources"]) != t["sha256_16"]:
        return None
    return int((t["fetch"] * FETCH_SCALE + t["write"] * WRITE_SCALE) * 1024)


def alg_counts(B, T, H, Dk, Dv, ebytes=2, h0=False):
    """Algorithmic flops and compulsory HBM bytes of one forward call.

    flops/token/head = 6 Dk Dv (state products K H, Q H, K^T U) +
                       2 C (3 Dk + 2 Dv) (in-tile K K^T, Q K^T, T-products, P U)
    bytes/token/head = ebytes (2 Dk + Dv) in + ebytes Dv out + 8 (gate, beta fp32)
    plus the final state (and h0 when given) once per head, fp32.
    """
    toks = B * T * H
    flops = toks * (6 * Dk * Dv + 2 * CHUNK * (3 * Dk + 2 * Dv))
    byts = toks * (ebytes * (2 * Dk + Dv) + ebytes * Dv + 8)
    byts += B * H * Dk * Dv * 4 * (2 if h0 else 1)
    return flops, byts


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="long_64k")
    ap.add_argument("--decode-steps", type=int, default=1000)
    ap.add_argument("--varlen-steps", type=int, default=20)
    ap.add_argument("--raw-steps", type=int, default=10)
    ap.add_argument("--bwd-steps", type=int, default=5)
    ap.add_argument("--bwd-1m-steps", type=int, default=0,
                    help="timed reverse passes at B=1 H=8 T=1M, in one pass and in segments "
                         "of 64K tokens (off by default: ~50 GB of device memory)")
    ap.add_argument("--channel-steps", type=int, default=5)
    ap.add_argument("--ladder-steps", type=int, default=5,
                    help="timed calls per rung of the context ladder (8K, 256K, 1M); 0 skips it")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-ceilings", action="store_true",
                    help="skip the copy and GEMM ceiling measurements")
    ap.add_argument("--cpu-tokens", type=int, default=65536,
                    help="tokens per head in the CPU-baseline sample")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="also run one state copy of this many MiB through the library "
                         "(lin_attn_chunk_fwd with T = 0): a kernel of known traffic that "
                         "calibrates the FETCH_SIZE / WRITE_SIZE counters")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(heads and batch would shard across GPUs with no exchange)",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from chunked_gated_linear_amd import inputs as I
    from chunked_gated_linear_amd import (lin_attn_chunk_fwd, lin_attn_chunk_fwd_varlen,
                                          lin_attn_chunk_fwd_varlen_workspace_size,
                                          lin_attn_chunk_fwd_workspace_size, lin_attn_decode_step)

    wl = dict(I.WORKLOADS[args.workload])
    B, H, T, Dk, Dv, dtype = wl["B"], wl["H"], wl["T"], wl["Dk"], wl["Dv"], wl["dtype"]
    h0_std = wl.get("h0_std")
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    inp = I.make_inputs(B, T, H, Dk, Dv, dtype=dtype, seed=1002, device=dev, h0_std=h0_std)
    o = torch.empty((B, T, H, Dv), dtype=inp["q"].dtype, device=dev)
    hT = torch.empty((B, H, Dk, Dv), dtype=torch.float32, device=dev)
    nws = lin_attn_chunk_fwd_workspace_size(B, T, H, Dk, Dv, inp["q"].dtype)
    ws = torch.empty(max(nws, 1), dtype=torch.uint8, device=dev)

    def step():
        lin_attn_chunk_fwd(inp["q"], inp["k"], inp["v"], inp["x"], inp["beta"], inp["h0"],
                           gate_mode="logit", G=5.0, o=o, hT=hT, workspace=ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)          # the stream the kernels run on
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    t = ms * 1e-3
    # per-call spread, in a separate pass (an event pair around each call)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    for a, b in evs:
        a.record(stream)
        step()
        b.record(stream)
    torch.cuda.synchronize()
    per_call = sorted(a.elapsed_time(b) for a, b in evs)
    ebytes = 2 if dtype == "bf16" else 4
    flops, byts = alg_counts(B, T, H, Dk, Dv, ebytes, h0_std is not None)
    tokens_per_s = B * T / t

    result = {
        "metric": METRIC,
        "value": tokens_per_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "ms_per_call_median": per_call[len(per_call) // 2],
        "ms_per_call_min": per_call[0],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic",
        "config": {"workload": args.workload, "B": B, "H": H, "T": T, "d_k": Dk, "d_v": Dv,
                   "chunk": CHUNK, "gate": "bounded logit, x ~ N(0,1), G=5",
                   "h0": "N(0,0.02)" if h0_std else "zero"},
        "mfma_pct_of_bf16_peak": 100.0 * flops / t / PEAK_BF16,
        "tflops": flops / t / 1e12,
        "roofline": {"bound": "hbm", "achieved": byts / t / 1e9, "peak": PEAK_HBM / 1e9,
                     "unit": "GB/s", "frac": byts / t / PEAK_HBM,
                     "traffic": measured_traffic("chunk", args.workload) if dtype == "bf16" else None,
                     "kernel": ("chunk_prep_kernel + chunk_state_kernel (one lin_attn_chunk_fwd call)"
                                if dtype == "bf16" else "chunk_fwd_kernel"),
                     "alg_bytes_per_launch": byts,
                     "alg_flops_per_launch": flops,
                     "attainable_frac": max(byts / PEAK_HBM, flops / PEAK_BF16) / t},
    }

    # ---- the rest of the context ladder (8K, 256K and 1M tokens; the headline
    # above is the 64K rung): one object per rung with its own roofline and a
    # CPU baseline of the oracle on a bounded sample of the same rung
    if args.ladder_steps > 0:
        from oracle import c_recurrent as crec
        from oracle import linattn_oracle as orc
        ladder = {}
        for name, seed, cpu_tok in (("train_8k", 1001, 8192), ("long_256k", 1007, 262144),
                                    ("million_1m", 1003, 262144)):
            if name == args.workload:
                continue
            lw = dict(I.WORKLOADS[name])
            lB, lH, lT, lK, lV = lw["B"], lw["H"], lw["T"], lw["Dk"], lw["Dv"]
            lh0 = lw.get("h0_std")
            lin = I.make_inputs(lB, lT, lH, lK, lV, dtype=lw["dtype"], seed=seed, device=dev,
                                h0_std=lh0)
            lo = torch.empty((lB, lT, lH, lV), dtype=lin["q"].dtype, device=dev)
            lh = torch.empty((lB, lH, lK, lV), dtype=torch.float32, device=dev)
            lws = torch.empty(max(1, lin_attn_chunk_fwd_workspace_size(lB, lT, lH, lK, lV)),
                              dtype=torch.uint8, device=dev)

            def lstep():
                lin_attn_chunk_fwd(lin["q"], lin["k"], lin["v"], lin["x"], lin["beta"], lin["h0"],
                                   gate_mode="logit", G=5.0, o=lo, hT=lh, workspace=lws)

            nsteps = args.ladder_steps if lT <= 262144 else max(2, args.ladder_steps // 2)
            lstep()
            torch.cuda.synchronize()
            e0.record(stream)
            for _ in range(nsteps):
                lstep()
            e1.record(stream)
            torch.cuda.synchronize()
            lms = e0.elapsed_time(e1) / nsteps
            lt = lms * 1e-3
            lfl, lby = alg_counts(lB, lT, lH, lK, lV, 2, lh0 is not None)
            rung = {
                "workload": (f"{name} B={lB} H={lH} T={lT} d={lK} bf16, gate x ~ N(0,1) G=5, "
                             f"h0 {'N(0,0.02)' if lh0 else 'zero'}"),
                "steps": nsteps, "ms_per_call": lms, "tokens_per_s": lB * lT / lt,
                "tflops": lfl / lt / 1e12, "mfma_pct_of_bf16_peak": 100.0 * lfl / lt / PEAK_BF16,
                "roofline": {"bound": "hbm", "achieved": lby / lt / 1e9, "peak": PEAK_HBM / 1e9,
                             "unit": "GB/s", "frac": lby / lt / PEAK_HBM,
                             "traffic": measured_traffic("ladder_" + name),
                             "alg_bytes_per_launch": lby, "alg_flops_per_launch": lfl,
                             "kernel": "chunk_prep_kernel + chunk_state_kernel (one call)",
                             "attainable_frac": max(lby / PEAK_HBM, lfl / PEAK_BF16) / lt},
            }
            if not args.no_cpu_baseline:
                S_tok = min(lT, cpu_tok)
                f = lambda x: x.detach().float().cpu().numpy()
                q_, k_, v_ = (f(lin[n_][:, :S_tok]) for n_ in ("q", "k", "v"))
                x_ = f(lin["x"][:, :S_tok]).astype(np.float64)
                b_ = f(lin["beta"][:, :S_tok]).astype(np.float64)
                h_ = None if lin["h0"] is None else f(lin["h0"]).astype(np.float64)
                workers = min(16, os.cpu_count() or 1, lB * lH)
                c0 = time.perf_counter()
                crec.recurrent_fwd_c(q_, k_, v_, orc.bounded_gate(x_), b_, h_, workers=workers)
                cs = time.perf_counter() - c0
                rung["cpu_baseline"] = {
                    "value": lB * S_tok / cs, "unit": "tokens/s", "cores": workers,
                    "kind": "oracle",
                    "sample": (f"all {lB * lH} heads, first {S_tok} of {lT} tokens (fp64 C "
                               f"recurrence, one thread per head stream), {cs:.1f} s wall")}
            ladder[name] = rung
            del lin, lo, lh, lws
        result["ladder"] = ladder

    # ---- the same workload from raw inputs (q, k normalised and beta from
    # logits inside the pass): what the fused input preparation costs
    if args.raw_steps > 0 and dtype == "bf16":
        o_raw, hT_raw = torch.empty_like(o), torch.empty_like(hT)   # o, hT stay for the parity check

        def rstep():
            lin_attn_chunk_fwd(inp["q"], inp["k"], inp["v"], inp["x"], inp["x"], inp["h0"],
                               gate_mode="logit", G=5.0, o=o_raw, hT=hT_raw, workspace=ws, raw=True)
        rstep()
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(args.raw_steps):
            rstep()
        e1.record(stream)
        torch.cuda.synchronize()
        rms = e0.elapsed_time(e1) / args.raw_steps
        result["raw_inputs"] = {"workload": f"{args.workload}, q and k unnormalised, beta as logits",
                                "ms_per_call": rms, "tokens_per_s": B * T / (rms * 1e-3),
                                "vs_prepared_call": rms / ms}
        del o_raw, hT_raw

    # ---- packed prefill batch: 64 requests of mixed lengths, 64K tokens in all
    if args.varlen_steps > 0:
        vw = I.VARLEN_WORKLOAD
        lengths = I.varlen_lengths(vw["nseq"], vw["T"], seed=1006)
        vin = I.make_inputs(1, vw["T"], vw["H"], vw["Dk"], vw["Dv"], dtype=vw["dtype"], seed=1006,
                            device=dev)
        cu = torch.tensor(np.concatenate([[0], np.cumsum(lengths)]), dtype=torch.int32, device=dev)
        ov = torch.empty((1, vw["T"], vw["H"], vw["Dv"]), dtype=vin["q"].dtype, device=dev)
        hv = torch.empty((vw["nseq"], vw["H"], vw["Dk"], vw["Dv"]), dtype=torch.float32, device=dev)
        wsv = torch.empty(lin_attn_chunk_fwd_varlen_workspace_size(vw["T"], vw["nseq"], vw["H"],
                                                                    vw["Dk"], vw["Dv"]),
                          dtype=torch.uint8, device=dev)

        def vstep():
            lin_attn_chunk_fwd_varlen(vin["q"], vin["k"], vin["v"], vin["x"], vin["beta"], cu,
                                      gate_mode="logit", G=5.0, o=ov, hT=hv, workspace=wsv)

        for _ in range(2):
            vstep()
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(args.varlen_steps):
            vstep()
        e1.record(stream)
        torch.cuda.synchronize()
        vms = e0.elapsed_time(e1) / args.varlen_steps
        vbytes = vw["T"] * vw["H"] * (2 * (2 * vw["Dk"] + vw["Dv"]) + 2 * vw["Dv"] + 8) \
            + vw["nseq"] * vw["H"] * vw["Dk"] * vw["Dv"] * 4
        result["varlen"] = {
            "workload": (f"{vw['nseq']} packed sequences, lengths {min(lengths)}..{max(lengths)} "
                         f"(log-normal), {vw['T']} tokens, H={vw['H']} d={vw['Dk']} bf16"),
            "ms_per_call": vms, "tokens_per_s": vw["T"] / (vms * 1e-3),
            "roofline": {"bound": "hbm", "achieved": vbytes / (vms * 1e-3) / 1e9,
                         "peak": PEAK_HBM / 1e9, "unit": "GB/s",
                         "frac": vbytes / (vms * 1e-3) / PEAK_HBM, "alg_bytes_per_launch": vbytes,
                         "traffic": measured_traffic("varlen"),
                         "kernel": "chunk_prep_kernel + chunk_state_kernel (packed sequences)"},
        }
        del vin, ov, hv, wsv

    # ---- per-channel gate: the headline shape with one log-decay per key
    # channel (gate logits [B,T,H,Dk] ~ N(0,1))
    if args.channel_steps > 0 and dtype == "bf16":
        from chunked_gated_linear_amd import (lin_attn_chunk_fwd_channel,
                                              lin_attn_chunk_fwd_channel_workspace_size)
        xc = I.make_channel_gate(B, T, H, Dk, seed=1002, device=dev)
        oc, hc = torch.empty_like(o), torch.empty_like(hT)
        wsc = torch.empty(lin_attn_chunk_fwd_channel_workspace_size(B, T, H, Dk, Dv),
                          dtype=torch.uint8, device=dev)

        def cstep():
            lin_attn_chunk_fwd_channel(inp["q"], inp["k"], inp["v"], xc, inp["beta"], inp["h0"],
                                       gate_mode="logit", G=5.0, o=oc, hT=hc, workspace=wsc)

        cstep()
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(args.channel_steps):
            cstep()
        e1.record(stream)
        torch.cuda.synchronize()
        cms = e0.elapsed_time(e1) / args.channel_steps
        # q, k, v, o in bf16, gate logits fp32 per channel, beta; hT (and h0) per head
        cbytes = B * T * H * (2 * (2 * Dk + Dv) + 2 * Dv + 4 * Dk + 4) \
            + B * H * Dk * Dv * 4 * (2 if h0_std is not None else 1)
        result["channel_gate"] = {
            "workload": f"{args.workload} with a per-channel gate (x [B,T,H,Dk] ~ N(0,1), G=5)",
            "ms_per_call": cms, "tokens_per_s": B * T / (cms * 1e-3),
            "roofline": {"bound": "hbm", "achieved": cbytes / (cms * 1e-3) / 1e9,
                         "peak": PEAK_HBM / 1e9, "unit": "GB/s",
                         "frac": cbytes / (cms * 1e-3) / PEAK_HBM, "alg_bytes_per_launch": cbytes,
                         "traffic": (measured_traffic("channel")
                                     if args.workload == "long_64k" else None),
                         "kernel": ("chunk_channel_prep_pair_kernel + 16 x "
                                    "chunk_fwd_channel_pair_kernel (one lin_attn_chunk_fwd_channel "
                                    "call: stretch launches, each with the next stretch's "
                                    "preparation beside the state)")},
        }
        del xc, oc, hc, wsc

    # ---- the packed prefill batch with a per-channel gate
    if args.channel_steps > 0 and args.varlen_steps > 0:
        from chunked_gated_linear_amd import (lin_attn_chunk_fwd_channel_varlen,
                                              lin_attn_chunk_fwd_channel_varlen_workspace_size)
        vw = I.VARLEN_WORKLOAD
        lengths = I.varlen_lengths(vw["nseq"], vw["T"], seed=1006)
        vin = I.make_inputs(1, vw["T"], vw["H"], vw["Dk"], vw["Dv"], dtype=vw["dtype"], seed=1006,
                            device=dev)
        xv = I.make_channel_gate(1, vw["T"], vw["H"], vw["Dk"], seed=1006, device=dev)
        cu = torch.tensor(np.concatenate([[0], np.cumsum(lengths)]), dtype=torch.int32, device=dev)
        ov = torch.empty((1, vw["T"], vw["H"], vw["Dv"]), dtype=vin["q"].dtype, device=dev)
        hv = torch.empty((vw["nseq"], vw["H"], vw["Dk"], vw["Dv"]), dtype=torch.float32, device=dev)
        wsv = torch.empty(lin_attn_chunk_fwd_channel_varlen_workspace_size(
            vw["T"], vw["nseq"], vw["H"], vw["Dk"], vw["Dv"]), dtype=torch.uint8, device=dev)

        def cvstep():
            lin_attn_chunk_fwd_channel_varlen(vin["q"], vin["k"], vin["v"], xv, vin["beta"], cu,
                                              gate_mode="logit", G=5.0, o=ov, hT=hv, workspace=wsv)

        cvstep()
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(args.channel_steps):
            cvstep()
        e1.record(stream)
        torch.cuda.synchronize()
        cvms = e0.elapsed_time(e1) / args.channel_steps
        cvbytes = vw["T"] * vw["H"] * (2 * (2 * vw["Dk"] + vw["Dv"]) + 2 * vw["Dv"] + 4 * vw["Dk"] + 4) \
            + vw["nseq"] * vw["H"] * vw["Dk"] * vw["Dv"] * 4
        result["channel_gate_varlen"] = {
            "workload": (f"{vw['nseq']} packed sequences, lengths {min(lengths)}..{max(lengths)}, "
                         f"{vw['T']} tokens, H={vw['H']} d={vw['Dk']} bf16, per-channel gate"),
            "ms_per_call": cvms, "tokens_per_s": vw["T"] / (cvms * 1e-3),
            "roofline": {"bound": "hbm", "achieved": cvbytes / (cvms * 1e-3) / 1e9,
                         "peak": PEAK_HBM / 1e9, "unit": "GB/s",
                         "frac": cvbytes / (cvms * 1e-3) / PEAK_HBM,
                         "alg_bytes_per_launch": cvbytes,
                         "traffic": measured_traffic("channel_varlen"),
                         "kernel": "chunk_channel_prep_kernel + chunk_fwd_channel_kernel (packed)"},
        }
        del vin, xv, ov, hv, wsv

    # ---- reverse pass at the training shape (B=4, H=16, T=8192, d=128): the
    # gradients of every input for an upstream dout and dhT
    if args.bwd_steps > 0:
        from chunked_gated_linear_amd import lin_attn_chunk_bwd, lin_attn_chunk_bwd_workspace_size
        bw = I.WORKLOADS["train_8k"]
        bB, bH, bT, bK, bV = bw["B"], bw["H"], bw["T"], bw["Dk"], bw["Dv"]
        bin_ = I.make_inputs(bB, bT, bH, bK, bV, dtype=bw["dtype"], seed=1001, device=dev)
        up = I.make_upstream_grads(bB, bT, bH, bK, bV, dtype=bw["dtype"], seed=1001, device=dev)
        wsb = torch.empty(lin_attn_chunk_bwd_workspace_size(bB, bT, bH, bK, bV),
                          dtype=torch.uint8, device=dev)

        def bstep():
            return lin_attn_chunk_bwd(bin_["q"], bin_["k"], bin_["v"], bin_["x"], bin_["beta"],
                                      up["dout"], None, up["dhT"], gate_mode="logit", G=5.0,
                                      workspace=wsb)

        for _ in range(2):
            bstep()
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(args.bwd_steps):
            bstep()
        e1.record(stream)
        torch.cuda.synchronize()
        bms = e0.elapsed_time(e1) / args.bwd_steps
        # inputs q, k, v, dout (bf16), x, beta; outputs dq, dk, dv (fp32),
        # dgate, dbeta; per head dhT in and dh0 out (fp32)
        per_tok = 2 * (2 * bK + 2 * bV) + 8 + 4 * (2 * bK + bV) + 8
        bbytes = bB * bT * bH * per_tok + 2 * bB * bH * bK * bV * 4
        result["backward"] = {
            "workload": (f"train_8k B={bB} H={bH} T={bT} d={bK} bf16 inputs, fp32 gradients, "
                         "dout and dhT ~ N(0,1)"),
            "ms_per_call": bms, "tokens_per_s": bB * bT / (bms * 1e-3),
            "roofline": {"bound": "hbm", "achieved": bbytes / (bms * 1e-3) / 1e9,
                         "peak": PEAK_HBM / 1e9, "unit": "GB/s",
                         "frac": bbytes / (bms * 1e-3) / PEAK_HBM, "alg_bytes_per_launch": bbytes,
                         "traffic": measured_traffic("backward"),
                         "kernel": ("bwd_prep_wave_kernel + bwd2_states_kernel + bwd2_grad_kernel "
                                    "(one lin_attn_chunk_bwd call, bf16 inputs)")},
        }
        del bin_, up, wsb

    # ---- the reverse pass at 1M tokens x 8 heads: one pass (workspace for the
    # whole sequence) and the segmented form (workspace for 64K tokens)
    if args.bwd_1m_steps > 0:
        from chunked_gated_linear_amd import lin_attn_chunk_bwd, lin_attn_chunk_bwd_workspace_size
        mw = I.WORKLOADS["million_1m"]
        mB, mH, mT, mK, mV = mw["B"], mw["H"], mw["T"], mw["Dk"], mw["Dv"]
        min_ = I.make_inputs(mB, mT, mH, mK, mV, dtype=mw["dtype"], seed=1003, device=dev,
                             h0_std=mw.get("h0_std"))
        mup = I.make_upstream_grads(mB, mT, mH, mK, mV, dtype=mw["dtype"], seed=1003, device=dev)
        per_tok = 2 * (2 * mK + 2 * mV) + 8 + 4 * (2 * mK + mV) + 8
        mbytes = mB * mT * mH * per_tok + 2 * mB * mH * mK * mV * 4
        rows = {}
        for name, seg in (("one_pass", None), ("segments_64k", 65536)):
            nws = lin_attn_chunk_bwd_workspace_size(mB, mT, mH, mK, mV, torch.bfloat16, seg)
            mws = torch.empty(nws, dtype=torch.uint8, device=dev)

            def mstep():
                return lin_attn_chunk_bwd(min_["q"], min_["k"], min_["v"], min_["x"], min_["beta"],
                                          mup["dout"], min_["h0"], mup["dhT"], gate_mode="logit",
                                          G=5.0, workspace=mws, segment_tokens=seg)

            mstep()
            torch.cuda.synchronize()
            e0.record(stream)
            for _ in range(args.bwd_1m_steps):
                mstep()
            e1.record(stream)
            torch.cuda.synchronize()
            mms = e0.elapsed_time(e1) / args.bwd_1m_steps
            rows[name] = {"ms_per_call": mms, "workspace_bytes": nws,
                          "tokens_per_s": mB * mT / (mms * 1e-3),
                          "roofline": {"bound": "hbm", "achieved": mbytes / (mms * 1e-3) / 1e9,
                                       "peak": PEAK_HBM / 1e9, "unit": "GB/s",
                                       "frac": mbytes / (mms * 1e-3) / PEAK_HBM,
                                       "alg_bytes_per_launch": mbytes}}
            del mws
            torch.cuda.empty_cache()
        result["backward_1m"] = {
            "workload": (f"million_1m B={mB} H={mH} T={mT} d={mK} bf16 inputs, fp32 gradients, "
                         "dout and dhT ~ N(0,1)"), **rows}
        del min_, mup

    # ---- optional calibration copy (reads and writes exactly copy_mib MiB)
    if args.copy_mib > 0:
        nh = args.copy_mib * 16                       # 64 KiB of fp32 state per head
        src = torch.ones((1, nh, 128, 128), dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        e16 = torch.empty((1, 0, nh, 128), dtype=torch.bfloat16, device=dev)
        e32 = torch.empty((1, 0, nh), dtype=torch.float32, device=dev)
        lin_attn_chunk_fwd(e16, e16, e16, e32, e32, src, gate_mode="logit", hT=dst)
        torch.cuda.synchronize()
        del src, dst

    # ---- decode: B=256, H=32, d=128, fresh token every step, state in place
    if args.decode_steps > 0:
        dw = I.DECODE_WORKLOAD
        dB, dH, dD = dw["B"], dw["H"], dw["Dk"]
        n = args.decode_steps
        d = I.make_decode_inputs(dB, dH, dD, dD, dtype=dw["dtype"], seed=1004, device=dev,
                                 steps=n)
        S = d["S"]
        od = torch.empty((dB, dH, dD), dtype=d["q"].dtype, device=dev)
        for s in range(min(3, n)):
            lin_attn_decode_step(d["q"][s], d["k"][s], d["v"][s], d["x"][s], d["beta"][s], S,
                                 gate_mode="logit", o=od)
        torch.cuda.synchronize()
        e0.record(stream)
        for s in range(n):
            lin_attn_decode_step(d["q"][s], d["k"][s], d["v"][s], d["x"][s], d["beta"][s], S,
                                 gate_mode="logit", o=od)
        e1.record(stream)
        torch.cuda.synchronize()
        dms = e0.elapsed_time(e1) / n
        per_head = 2 * dD * dD * 4 + 3 * dD * 2 + dD * 2 + 8
        dbytes = dB * dH * per_head
        result["decode"] = {
            "workload": f"B={dB} H={dH} d={dD} bf16, fp32 state in place, {n} steps",
            "us_per_step": dms * 1e3, "tokens_per_s": dB / (dms * 1e-3),
            "roofline": {"bound": "hbm", "achieved": dbytes / (dms * 1e-3) / 1e9,
                         "peak": PEAK_HBM / 1e9, "unit": "GB/s",
                         "frac": dbytes / (dms * 1e-3) / PEAK_HBM,
                         "traffic": measured_traffic("decode", None),
                         "alg_bytes_per_launch": dbytes, "kernel": "decode_kernel"},
        }
        del d, S

    # ---- decode with a per-channel gate: same shape, gate logits [B,H,Dk]
    if args.decode_steps > 0:
        from chunked_gated_linear_amd import lin_attn_decode_step_channel
        dw = I.DECODE_WORKLOAD
        dB, dH, dD = dw["B"], dw["H"], dw["Dk"]
        n = min(args.decode_steps, 200)
        d = I.make_decode_inputs(dB, dH, dD, dD, dtype=dw["dtype"], seed=1005, device=dev,
                                 steps=n)
        xg = I.make_channel_gate(n, dB, dH, dD, seed=1005, device=dev)   # [steps, B, H, Dk]
        S = d["S"]
        od = torch.empty((dB, dH, dD), dtype=d["q"].dtype, device=dev)
        for s_ in range(min(3, n)):
            lin_attn_decode_step_channel(d["q"][s_], d["k"][s_], d["v"][s_], xg[s_], d["beta"][s_],
                                         S, gate_mode="logit", o=od)
        torch.cuda.synchronize()
        e0.record(stream)
        for s_ in range(n):
            lin_attn_decode_step_channel(d["q"][s_], d["k"][s_], d["v"][s_], xg[s_], d["beta"][s_],
                                         S, gate_mode="logit", o=od)
        e1.record(stream)
        torch.cuda.synchronize()
        cms = e0.elapsed_time(e1) / n
        per_head = 2 * dD * dD * 4 + 3 * dD * 2 + dD * 2 + 4 * dD + 4
        cbytes = dB * dH * per_head
        result["decode_channel"] = {
            "workload": f"B={dB} H={dH} d={dD} bf16, per-channel gate, fp32 state in place, {n} steps",
            "us_per_step": cms * 1e3, "tokens_per_s": dB / (cms * 1e-3),
            "roofline": {"bound": "hbm", "achieved": cbytes / (cms * 1e-3) / 1e9,
                         "peak": PEAK_HBM / 1e9, "unit": "GB/s",
                         "frac": cbytes / (cms * 1e-3) / PEAK_HBM,
                         "alg_bytes_per_launch": cbytes,
                         "traffic": measured_traffic("decode_channel"),
                         "kernel": "decode_channel_kernel"},
        }
        del d, S, xg

    # ---- measured ceilings of this GPU beside the published peaks: a device
    # copy (reads and writes every byte once) and a large bf16 GEMM (torch's
    # library GEMM, contiguous operands)
    if not args.no_ceilings:
        nbytes = 2 << 30
        src = torch.empty(nbytes // 4, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(10):
            dst.copy_(src)
        e1.record(stream)
        torch.cuda.synchronize()
        copy_s = e0.elapsed_time(e1) / 10 * 1e-3
        del src, dst
        n = 8192
        a = torch.randn((n, n), device=dev, dtype=torch.bfloat16)
        bm = torch.randn((n, n), device=dev, dtype=torch.bfloat16)
        c = a @ bm
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(10):
            c = a @ bm
        e1.record(stream)
        torch.cuda.synchronize()
        gemm_s = e0.elapsed_time(e1) / 10 * 1e-3
        del a, bm, c
        result["ceilings"] = {
            "copy_GBps": 2 * nbytes / copy_s / 1e9, "copy_frac_of_peak": 2 * nbytes / copy_s / PEAK_HBM,
            "bf16_gemm_TFLOPs": 2 * n ** 3 / gemm_s / 1e12,
            "bf16_gemm_frac_of_peak": 2 * n ** 3 / gemm_s / PEAK_BF16,
            "what": "device copy of 2 GiB (read + write) and an 8192^3 bf16 GEMM (torch), HIP events"}

    # ---- CPU baseline: the fp64 oracle (plain C recurrence) on host cores
    if not args.no_cpu_baseline:
        from oracle import c_recurrent as crec
        from oracle import linattn_oracle as orc

        S_tok = min(T, args.cpu_tokens)
        f = lambda x: x.detach().float().cpu().numpy()
        q, k, v = f(inp["q"][:, :S_tok]), f(inp["k"][:, :S_tok]), f(inp["v"][:, :S_tok])
        x, beta = f(inp["x"][:, :S_tok]), f(inp["beta"][:, :S_tok]).astype(np.float64)
        h0 = None if inp["h0"] is None else f(inp["h0"]).astype(np.float64)
        workers = min(16, os.cpu_count() or 1, B * H)
        c0 = time.perf_counter()
        g = orc.bounded_gate(x.astype(np.float64))
        res = crec.recurrent_fwd_c(q, k, v, g, beta, h0, workers=workers)
        cpu_s = time.perf_counter() - c0
        result["cpu_baseline"] = {
            "value": B * S_tok / cpu_s, "unit": "tokens/s", "cores": workers, "kind": "oracle",
            "sample": f"all {B * H} heads, first {S_tok} of {T} tokens (fp64 C recurrence, "
                      f"one thread per head stream), {cpu_s:.1f} s wall",
            "host": host_info()}
        if S_tok == T:   # the sample is the whole workload: compare every output
            oh, hh = f(o), f(hT)
            eo = max(np.max(np.abs(oh[b, :, h] - r[0])) for (b, h), r in res.items())
            eh = max(np.max(np.abs(hh[b, h] - r[1])) for (b, h), r in res.items())
            so = max(np.max(np.abs(r[0])) for r in res.values())
            sh = max(np.max(np.abs(r[1])) for r in res.values())
            result["parity"] = {"err_o": float(eo / so), "err_hT": float(eh / sh), "tol": 1e-2}

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
