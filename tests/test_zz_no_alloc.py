"""lin_attn_chunk_fwd_noalloc through the C ABI: the library-owned scratch
gives the same outputs as lin_attn_chunk_fwd with a caller workspace, bit for
bit, on two calls in a row (the second smaller, so it reuses a buffer that
still holds the first call's records), and sizes beyond the scratch are
rejected."""

import pytest
import torch

from chunked_gated_linear_amd import _native as N
from chunked_gated_linear_amd import lin_attn_chunk_fwd, lin_attn_chunk_fwd_workspace_size

from parity_util import make_case, say

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def _noalloc(dev, o, hT):
    q = dev["q"]
    B, T, H, Dk = q.shape
    Dv = dev["v"].shape[-1]
    dt = N.LA_BF16 if q.dtype == torch.bfloat16 else N.LA_FP32
    p = lambda t: None if t is None else t.data_ptr()
    rc = N.lib().lin_attn_chunk_fwd_noalloc(
        p(q), p(dev["k"]), p(dev["v"]), p(dev["gate"]), N.LA_GATE_BOUNDED_LOGIT, 5.0,
        p(dev["beta"]), p(dev["h0"]), p(o), p(hT), B, T, H, Dk, Dv, dt,
        torch.cuda.current_stream().cuda_stream)
    return rc


def test_noalloc_matches_workspace_entry_point():
    # first call: stretched (4 stretches of whole pairs, carried state in the
    # scratch), then a smaller batched call and an fp32 call (no scratch)
    cases = [(1, 20000, 8, 128, 128, "bf16", 0.02), (2, 1000, 3, 128, 64, "bf16", None),
             (1, 300, 2, 64, 64, "fp32", 0.02)]
    for i, (B, T, H, Dk, Dv, dtype, h0s) in enumerate(cases):
        say(f"noalloc call {i}: B{B} T{T} H{H} dk{Dk} dv{Dv} {dtype}")
        dev, _ = make_case(B, T, H, Dk, Dv, dtype, "weak", "logit", h0s, seed=101 + i)
        assert lin_attn_chunk_fwd_workspace_size(B, T, H, Dk, Dv, dev["q"].dtype) <= 64 << 20
        o_ref, h_ref = lin_attn_chunk_fwd(dev["q"], dev["k"], dev["v"], dev["gate"], dev["beta"],
                                          dev["h0"], gate_mode="logit")
        o = torch.full_like(o_ref, 7.0)
        hT = torch.full_like(h_ref, 7.0)
        assert _noalloc(dev, o, hT) == N.LA_OK, N.lib().lin_attn_last_error()
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref) and torch.equal(hT, h_ref), i


def test_noalloc_rejects_sizes_beyond_the_scratch():
    say("noalloc: a size whose workspace exceeds the scratch")
    B, T, H, D = 1, 65536, 16, 128          # 218 MB of records
    assert lin_attn_chunk_fwd_workspace_size(B, T, H, D, D) > 64 << 20
    e = lambda *s, dt=torch.bfloat16: torch.empty(s, dtype=dt, device="cuda")
    dev = dict(q=e(B, T, H, D), k=e(B, T, H, D), v=e(B, T, H, D),
               gate=e(B, T, H, dt=torch.float32), beta=e(B, T, H, dt=torch.float32), h0=None)
    o = e(B, T, H, D)
    assert _noalloc(dev, o, None) == N.LA_EINVAL
    assert b"scratch" in N.lib().lin_attn_last_error()
