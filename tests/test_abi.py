"""The C ABI library loads, exports every symbol the header declares, and
rejects bad arguments on the host with the documented codes.  No call here
reaches a kernel launch, so these run without a GPU."""

import ctypes
import os
import re

import pytest

from chunked_gated_linear_amd import _native as N

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lin_attn.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(lin_attn_\w+)\s*\(", text)))


def declared_constants():
    text = open(HEADER).read()
    return {m[0]: int(m[1]) for m in re.findall(r"#define\s+(LA_\w+)\s+(\d+)", text)}


def test_library_loads_and_exports_header_symbols():
    L = N.lib()
    names = declared_functions()
    assert names == sorted(N.SIGNATURES), "binding and header disagree"
    for name in names:
        assert hasattr(L, name), name
    assert L.lin_attn_version() >= 100


def test_binding_constants_match_header():
    c = declared_constants()
    assert c["LA_OK"] == N.LA_OK and c["LA_EINVAL"] == N.LA_EINVAL
    assert c["LA_EUNSUPPORTED"] == N.LA_EUNSUPPORTED and c["LA_ERANGE"] == N.LA_ERANGE
    assert c["LA_EHIP"] == N.LA_EHIP
    assert c["LA_BF16"] == N.LA_BF16 and c["LA_FP32"] == N.LA_FP32
    assert c["LA_GATE_LOG"] == N.LA_GATE_LOG
    assert c["LA_GATE_BOUNDED_LOGIT"] == N.LA_GATE_BOUNDED_LOGIT


# Fake, never-dereferenced device addresses: validation looks at pointer values
# only, and every case below fails before any launch.
BASE = 1 << 40


def fake(i, size=1 << 30):
    return BASE + i * size


def chunk(**kw):
    a = dict(q=fake(0), k=fake(1), v=fake(2), gate=fake(3), gate_mode=0, G=5.0,
             beta=fake(4), h0=None, o=fake(5), hT=fake(6), B=1, T=64, H=2, Dk=128,
             Dv=128, dtype=0, ws=fake(8), ws_bytes=1 << 30, stream=None)
    a.update(kw)
    L = N.lib()
    rc = L.lin_attn_chunk_fwd(a["q"], a["k"], a["v"], a["gate"], a["gate_mode"], a["G"],
                              a["beta"], a["h0"], a["o"], a["hT"], a["B"], a["T"], a["H"],
                              a["Dk"], a["Dv"], a["dtype"], a["ws"], a["ws_bytes"],
                              a["stream"])
    return rc, L.lin_attn_last_error().decode()


@pytest.mark.parametrize("kw,code,needle", [
    (dict(q=None), N.LA_EINVAL, "q must not be NULL"),
    (dict(k=None), N.LA_EINVAL, "k must not be NULL"),
    (dict(beta=None), N.LA_EINVAL, "beta must not be NULL"),
    (dict(o=None), N.LA_EINVAL, "o must not be NULL"),
    (dict(B=-1), N.LA_EINVAL, "sizes"),
    (dict(T=-3), N.LA_EINVAL, "sizes"),
    (dict(dtype=7), N.LA_EINVAL, "dtype"),
    (dict(gate_mode=2), N.LA_EINVAL, "gate_mode"),
    (dict(G=-1.0), N.LA_ERANGE, "G must"),
    (dict(G=float("nan")), N.LA_ERANGE, "G must"),
    (dict(G=100.0), N.LA_ERANGE, "G must"),
    (dict(Dk=96), N.LA_EUNSUPPORTED, "Dk"),
    (dict(Dv=40), N.LA_EUNSUPPORTED, "Dv"),
    (dict(Dv=512), N.LA_EUNSUPPORTED, "Dv"),
    (dict(q=fake(0) + 8), N.LA_EINVAL, "aligned"),
    (dict(h0=fake(7) + 2), N.LA_EINVAL, "aligned"),
    (dict(v=fake(2) + 1), N.LA_EINVAL, "aligned"),
    (dict(o=fake(0) + 1024), N.LA_EINVAL, "o overlaps q"),
    (dict(o=fake(6)), N.LA_EINVAL, "o overlaps hT"),
    (dict(hT=fake(3)), N.LA_EINVAL, "hT overlaps gate"),
    (dict(h0=fake(7), hT=fake(7) + 4096), N.LA_EINVAL, "partially overlaps h0"),
    (dict(v=fake(2) + 8), N.LA_EINVAL, "v must be 16-byte aligned"),
    (dict(o=fake(5) + 4), N.LA_EINVAL, "o must be 8-byte aligned"),
    (dict(ws=None), N.LA_EINVAL, "workspace must not be NULL"),
    (dict(ws=fake(8) + 128), N.LA_EINVAL, "workspace must be 256-byte aligned"),
    (dict(ws_bytes=2 * 2 * 6656 - 1), N.LA_EINVAL, "workspace too small"),
    (dict(ws=fake(0) + 4096), N.LA_EINVAL, "workspace overlaps q"),
    (dict(ws=fake(5)), N.LA_EINVAL, "workspace overlaps o"),
])
def test_chunk_fwd_rejects(kw, code, needle):
    rc, msg = chunk(**kw)
    assert rc == code, (rc, msg)
    assert needle in msg


def test_workspace_size():
    L = N.lib()
    ws = L.lin_attn_chunk_fwd_workspace_size
    # bf16: one 6656-byte record per (sequence, head, 32 tokens)
    assert ws(1, 64, 2, 128, 128, N.LA_BF16) == 2 * 2 * 6656
    assert ws(4, 8192, 16, 128, 128, N.LA_BF16) == 4 * 16 * 256 * 6656
    assert ws(1, 33, 3, 64, 16, N.LA_BF16) == 3 * 2 * 6656
    # from 512 pairs of tiles on, one fp32 state per head follows the records
    assert ws(1, 32 * 511, 2, 128, 128, N.LA_BF16) == 2 * 511 * 6656
    assert ws(1, 32 * 511 + 1, 2, 128, 64, N.LA_BF16) == 2 * 512 * 6656 + 2 * 128 * 64 * 4
    assert ws(1, 32 * 1535, 2, 128, 64, N.LA_BF16) == 2 * 1535 * 6656 + 2 * 128 * 64 * 4
    # from 1536 pairs on, the segmented form's further states, state maps
    # and a 1 KB zero block follow
    seg = lambda B, H, dk, dv: B * H * (4 * dk * dv + 2 * dk * dk) * 4 + 1024
    assert ws(1, 32 * 1536, 2, 128, 64, N.LA_BF16) == \
        2 * 1536 * 6656 + 2 * 128 * 64 * 4 + seg(1, 2, 128, 64)
    assert ws(1, 65536, 16, 128, 128, N.LA_BF16) == \
        16 * 2048 * 6656 + 16 * 128 * 128 * 4 + seg(1, 16, 128, 128)
    assert ws(2, 0, 4, 128, 64, N.LA_BF16) == 0
    # fp32 runs one fused kernel without a workspace
    assert ws(1, 4096, 8, 128, 128, N.LA_FP32) == 0
    assert ws(1, 64, 2, 96, 128, N.LA_BF16) == -1
    assert "Dk" in L.lin_attn_last_error().decode()
    assert ws(-1, 64, 2, 128, 128, N.LA_BF16) == -1
    # the fp32 path accepts a NULL workspace
    rc, msg = chunk(dtype=N.LA_FP32, ws=None, ws_bytes=0, o=fake(5), q=fake(0) + 8)
    assert rc == N.LA_EINVAL and "q must be 16-byte aligned" in msg


def test_chunk_fwd_empty_is_noop():
    # B = 0 or H = 0: nothing to do, nothing launched, even with NULL arrays.
    for kw in (dict(B=0), dict(H=0)):
        rc, msg = chunk(q=None, k=None, v=None, gate=None, beta=None, o=None, hT=None, **kw)
        assert rc == N.LA_OK, msg
        assert msg == ""


def decode(**kw):
    a = dict(q=fake(0), k=fake(1), v=fake(2), gate=fake(3), gate_mode=1, G=5.0,
             beta=fake(4), S=fake(5), o=fake(6), B=4, H=2, Dk=128, Dv=128, dtype=0,
             stream=None)
    a.update(kw)
    L = N.lib()
    rc = L.lin_attn_decode_step(a["q"], a["k"], a["v"], a["gate"], a["gate_mode"], a["G"],
                                a["beta"], a["S"], a["o"], a["B"], a["H"], a["Dk"], a["Dv"],
                                a["dtype"], a["stream"])
    return rc, L.lin_attn_last_error().decode()


@pytest.mark.parametrize("kw,code,needle", [
    (dict(S=None), N.LA_EINVAL, "S must not be NULL"),
    (dict(H=-2), N.LA_EINVAL, "sizes"),
    (dict(Dv=256), N.LA_EUNSUPPORTED, "decode supports"),
    (dict(Dk=32), N.LA_EUNSUPPORTED, "decode supports"),
    (dict(o=fake(5)), N.LA_EINVAL, "o overlaps S"),
    (dict(S=fake(1)), N.LA_EINVAL, "S overlaps k"),
    (dict(v=fake(2) + 1), N.LA_EINVAL, "aligned"),
    (dict(S=fake(5) + 8), N.LA_EINVAL, "aligned"),
    (dict(G=20.0), N.LA_ERANGE, "G must"),
])
def test_decode_rejects(kw, code, needle):
    rc, msg = decode(**kw)
    assert rc == code, (rc, msg)
    assert needle in msg


def test_gate_rejects():
    L = N.lib()
    assert L.lin_attn_gate(fake(0), 5.0, fake(1), -1, None) == N.LA_EINVAL
    assert L.lin_attn_gate(None, 5.0, fake(1), 10, None) == N.LA_EINVAL
    assert L.lin_attn_gate(fake(0), 5.0, fake(0) + 16, 10, None) == N.LA_EINVAL
    assert "partially overlaps" in L.lin_attn_last_error().decode()
    assert L.lin_attn_gate(fake(0), -5.0, fake(1), 10, None) == N.LA_ERANGE
    assert L.lin_attn_gate(fake(0), 5.0, fake(1), 0, None) == N.LA_OK


def test_error_text_is_thread_local():
    import threading
    chunk(q=None)
    seen = {}

    def other():
        seen["msg"] = N.lib().lin_attn_last_error().decode()

    th = threading.Thread(target=other)
    th.start()
    th.join()
    assert seen["msg"] == ""
    assert "q must not be NULL" in N.lib().lin_attn_last_error().decode()


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(N, "_lib", None)
    monkeypatch.setattr(N, "LIB_PATH", str(tmp_path / "nope.so"))
    with pytest.raises(RuntimeError, match="no fallback"):
        N.lib()


def varlen(**kw):
    a = dict(q=fake(0), k=fake(1), v=fake(2), gate=fake(3), gate_mode=0, G=5.0,
             beta=fake(4), h0=None, o=fake(5), hT=fake(6), cu=fake(9), nseq=3, T=64, H=2,
             Dk=128, Dv=128, dtype=0, ws=fake(8), ws_bytes=1 << 30, stream=None)
    a.update(kw)
    L = N.lib()
    rc = L.lin_attn_chunk_fwd_varlen(a["q"], a["k"], a["v"], a["gate"], a["gate_mode"], a["G"],
                                     a["beta"], a["h0"], a["o"], a["hT"], a["cu"], a["nseq"],
                                     a["T"], a["H"], a["Dk"], a["Dv"], a["dtype"], a["ws"],
                                     a["ws_bytes"], a["stream"])
    return rc, L.lin_attn_last_error().decode()


@pytest.mark.parametrize("kw,code,needle", [
    (dict(cu=None), N.LA_EINVAL, "cu_seqlens must not be NULL"),
    (dict(cu=fake(9) + 2), N.LA_EINVAL, "cu_seqlens must be 4-byte aligned"),
    (dict(nseq=-1), N.LA_EINVAL, "nseq"),
    (dict(Dk=96), N.LA_EUNSUPPORTED, "Dk"),
    (dict(q=None), N.LA_EINVAL, "q must not be NULL"),
    (dict(gate_mode=5), N.LA_EINVAL, "gate_mode"),
    (dict(ws=None), N.LA_EINVAL, "workspace must not be NULL"),
    (dict(ws_bytes=2 * (64 // 32 + 3 + 1) * 6656 - 1), N.LA_EINVAL, "workspace too small"),
    (dict(o=fake(0) + 64), N.LA_EINVAL, "o overlaps q"),
    (dict(cu=fake(6)), N.LA_EINVAL, "hT overlaps cu_seqlens"),
    (dict(ws=fake(9)), N.LA_EINVAL, "workspace overlaps cu_seqlens"),
])
def test_varlen_rejects(kw, code, needle):
    rc, msg = varlen(**kw)
    assert rc == code, (rc, msg)
    assert needle in msg


def test_varlen_workspace_size_and_empty():
    L = N.lib()
    ws = L.lin_attn_chunk_fwd_varlen_workspace_size
    # one record slot per 32 tokens per head plus one per sequence and one spare
    assert ws(65536, 64, 16, 128, 128, N.LA_BF16) == 16 * (2048 + 64 + 1) * 6656
    assert ws(100, 3, 2, 64, 64, N.LA_BF16) == 2 * (3 + 3 + 1) * 6656
    assert ws(100, 3, 2, 64, 64, N.LA_FP32) == 0        # the fp32 path needs none
    # no sequences: nothing to do, nothing touched
    assert varlen(nseq=0, q=None, cu=None, ws=None)[0] == N.LA_OK


def test_raw_entry_checks():
    L = N.lib()
    base = [fake(0), fake(1), fake(2), fake(3), 0, 5.0, fake(4), None, fake(5), fake(6),
            1, 64, 2, 128, 128]
    bad = list(base)
    bad[13] = 96                                         # Dk
    assert L.lin_attn_chunk_fwd_raw(*bad, N.LA_FP32, None, 0, None) == N.LA_EUNSUPPORTED
    assert "Dk" in L.lin_attn_last_error().decode()
    bad = list(base)
    bad[0] = None
    assert L.lin_attn_chunk_fwd_raw(*bad, N.LA_BF16, fake(8), 1 << 30, None) == N.LA_EINVAL
    assert "q must not be NULL" in L.lin_attn_last_error().decode()
    assert L.lin_attn_chunk_fwd_raw(*base, N.LA_BF16, fake(8), 10, None) == N.LA_EINVAL
    assert "workspace too small" in L.lin_attn_last_error().decode()


def test_raw_affine_entry_checks():
    """The affine-gate entry points check their extra arrays on the host
    before anything touches the device."""
    L = N.lib()
    f = L.lin_attn_chunk_fwd_raw_affine
    args = lambda sc, bi, G=5.0: [fake(0), fake(1), fake(2), fake(3), G, sc, bi, fake(4), None,
                                  fake(5), fake(6), 1, 64, 2, 128, 128, N.LA_BF16, fake(8),
                                  1 << 30, None]
    misaligned = ctypes.c_void_p(fake(9) + 2)
    assert f(*args(misaligned, None)) == N.LA_EINVAL
    assert "gate_scale must be 4-byte aligned" in L.lin_attn_last_error().decode()
    assert f(*args(None, misaligned)) == N.LA_EINVAL
    assert "gate_bias must be 4-byte aligned" in L.lin_attn_last_error().decode()
    # an output that overlaps the scale array
    assert f(*args(ctypes.c_void_p(fake(5) + 64), None)) == N.LA_EINVAL
    assert "o overlaps gate_scale" in L.lin_attn_last_error().decode()
    assert f(*args(None, None, G=-1.0)) == N.LA_ERANGE
    fv = L.lin_attn_chunk_fwd_varlen_raw_affine
    cu = fake(10)
    assert fv(fake(0), fake(1), fake(2), fake(3), 5.0, misaligned, None, fake(4), None, fake(5),
              fake(6), cu, 2, 64, 2, 128, 128, N.LA_BF16, fake(8), 1 << 30, None) == N.LA_EINVAL
    assert "gate_scale must be 4-byte aligned" in L.lin_attn_last_error().decode()


def bwd(**kw):
    a = dict(q=fake(0), k=fake(1), v=fake(2), gate=fake(3), gate_mode=0, G=5.0,
             beta=fake(4), h0=None, dout=fake(5), dhT=None, dq=fake(6), dk=fake(7),
             dv=fake(8), dgate=fake(9), dbeta=fake(10), dh0=fake(11), B=1, T=64, H=2,
             Dk=128, Dv=128, dtype=0, ws=fake(12), ws_bytes=1 << 30, stream=None)
    a.update(kw)
    L = N.lib()
    rc = L.lin_attn_chunk_bwd(a["q"], a["k"], a["v"], a["gate"], a["gate_mode"], a["G"],
                              a["beta"], a["h0"], a["dout"], a["dhT"], a["dq"], a["dk"],
                              a["dv"], a["dgate"], a["dbeta"], a["dh0"], a["B"], a["T"],
                              a["H"], a["Dk"], a["Dv"], a["dtype"], a["ws"], a["ws_bytes"],
                              a["stream"])
    return rc, L.lin_attn_last_error().decode()


@pytest.mark.parametrize("kw,code,needle", [
    (dict(dout=None), N.LA_EINVAL, "dout must not be NULL"),
    (dict(dq=None), N.LA_EINVAL, "dq must not be NULL"),
    (dict(dgate=None), N.LA_EINVAL, "dgate must not be NULL"),
    (dict(dbeta=None), N.LA_EINVAL, "dbeta must not be NULL"),
    (dict(q=fake(0) + 8), N.LA_EINVAL, "q must be 16-byte aligned"),
    (dict(dv=fake(8) + 2), N.LA_EINVAL, "dv must be 16-byte aligned"),
    (dict(dq=fake(6) + 4), N.LA_EINVAL, "dq must be 16-byte aligned"),
    (dict(dh0=fake(11) + 2), N.LA_EINVAL, "dh0 must be 4-byte aligned"),
    (dict(gate_mode=3), N.LA_EINVAL, "gate_mode"),
    (dict(Dk=32), N.LA_EUNSUPPORTED, "Dk"),
    (dict(ws=None), N.LA_EINVAL, "workspace must not be NULL"),
    (dict(ws_bytes=100), N.LA_EINVAL, "workspace too small"),
    (dict(dq=fake(0) + 64), N.LA_EINVAL, "dq overlaps q"),
    (dict(dk=fake(6) + 4096), N.LA_EINVAL, "dk overlaps dq"),
    (dict(dh0=fake(1)), N.LA_EINVAL, "dh0 overlaps k"),
    (dict(ws=fake(9)), N.LA_EINVAL, "workspace overlaps dgate"),
    (dict(dhT=fake(11)), N.LA_EINVAL, "dh0 overlaps dhT"),
])
def test_chunk_bwd_rejects(kw, code, needle):
    rc, msg = bwd(**kw)
    assert rc == code, (rc, msg)
    assert needle in msg


def test_chunk_bwd_workspace_size_and_empty():
    L = N.lib()
    ws = L.lin_attn_chunk_bwd_workspace_size
    # float32 inputs (and d_v > 128): per 16-token tile and head a 3200-byte
    # record and two fp32 states
    assert ws(2, 17, 3, 64, 32, N.LA_FP32) == 2 * 3 * 2 * (3200 + 8 * 64 * 32)
    assert ws(1, 64, 2, 128, 144, N.LA_BF16) == 2 * 4 * (3200 + 8 * 128 * 144)
    # bf16 inputs: the records, plus per group of four tiles (a partial group
    # counts whole) two states and one state gradient as packed words
    assert ws(1, 64, 2, 128, 128, N.LA_BF16) == 2 * 4 * 3200 + 2 * 1 * 12 * 128 * 128
    assert ws(1, 65, 2, 128, 128, N.LA_BF16) == 2 * 5 * 3200 + 2 * 2 * 12 * 128 * 128
    assert ws(3, 300, 2, 64, 48, N.LA_BF16) == 6 * 19 * 3200 + 6 * 5 * 12 * 64 * 48
    assert ws(1, 0, 2, 128, 128, N.LA_BF16) == 0
    assert ws(1, 64, 2, 96, 128, N.LA_BF16) == -1
    for kw in (dict(B=0), dict(H=0)):
        rc, msg = bwd(q=None, k=None, v=None, dout=None, dq=None, **kw)
        assert rc == N.LA_OK, msg


def channel(**kw):
    a = dict(q=fake(0), k=fake(1), v=fake(2), gate=fake(3), gate_mode=1, G=5.0,
             beta=fake(4), h0=None, o=fake(5), hT=fake(6), B=1, T=64, H=2, Dk=128,
             Dv=128, dtype=0, ws=fake(8), ws_bytes=1 << 30, stream=None)
    a.update(kw)
    L = N.lib()
    rc = L.lin_attn_chunk_fwd_channel(a["q"], a["k"], a["v"], a["gate"], a["gate_mode"], a["G"],
                                      a["beta"], a["h0"], a["o"], a["hT"], a["B"], a["T"],
                                      a["H"], a["Dk"], a["Dv"], a["dtype"], a["ws"],
                                      a["ws_bytes"], a["stream"])
    return rc, L.lin_attn_last_error().decode()


@pytest.mark.parametrize("kw,code,needle", [
    (dict(gate=None), N.LA_EINVAL, "gate must not be NULL"),
    (dict(gate=fake(3) + 4), N.LA_EINVAL, "gate must be 16-byte aligned"),
    (dict(G=10.5), N.LA_ERANGE, "per-channel"),
    (dict(G=-0.5), N.LA_ERANGE, "G must"),
    (dict(Dk=96), N.LA_EUNSUPPORTED, "Dk"),
    (dict(Dv=24), N.LA_EUNSUPPORTED, "Dv"),
    (dict(dtype=5), N.LA_EINVAL, "dtype"),
    # the per-channel gate is T*H*Dk floats: an o placed inside it overlaps
    (dict(o=fake(3) + 64 * 2 * 4 * 64), N.LA_EINVAL, "o overlaps gate"),
    (dict(hT=fake(3) + 64 * 2 * 4 * 64), N.LA_EINVAL, "hT overlaps gate"),
    (dict(ws=None), N.LA_EINVAL, "workspace must not be NULL"),
    (dict(ws_bytes=1000), N.LA_EINVAL, "workspace too small"),
    (dict(ws=fake(8) + 16), N.LA_EINVAL, "workspace must be 256-byte aligned"),
    (dict(ws=fake(3)), N.LA_EINVAL, "workspace overlaps gate"),
])
def test_chunk_fwd_channel_rejects(kw, code, needle):
    rc, msg = channel(**kw)
    assert rc == code and needle in msg, (rc, msg)


def test_chunk_fwd_channel_empty_is_noop():
    # B = 0 or H = 0: nothing to do, nothing dereferenced
    assert channel(B=0)[0] == N.LA_OK
    assert channel(H=0, q=None, k=None)[0] == N.LA_OK


def test_chunk_fwd_channel_workspace_size():
    L = N.lib()
    assert L.lin_attn_chunk_fwd_channel_workspace_size(1, 64, 2, 128, 128, 0) == 2 * 4 * 18944
    assert L.lin_attn_chunk_fwd_channel_workspace_size(1, 64, 2, 128, 128, 1) == 2 * 4 * 27136
    # bf16: the larger of the 16-token records and the 32-token pair records
    # (31,232 / 18,688 bytes per pair at Dk = 128 / 64)
    assert L.lin_attn_chunk_fwd_channel_workspace_size(1, 16, 1, 64, 64, 0) == 18688
    assert L.lin_attn_chunk_fwd_channel_workspace_size(1, 32, 1, 128, 64, 0) == 37888
    assert L.lin_attn_chunk_fwd_channel_workspace_size(2, 17, 3, 64, 32, 1) == 2 * 3 * 2 * 14592
    assert L.lin_attn_chunk_fwd_channel_workspace_size(1, 0, 2, 128, 128, 0) == 0
    assert L.lin_attn_chunk_fwd_channel_workspace_size(1, 64, 2, 96, 128, 0) == -1


def decode_ch(**kw):
    a = dict(q=fake(0), k=fake(1), v=fake(2), gate=fake(3), gate_mode=1, G=5.0, beta=fake(4),
             S=fake(5), o=fake(6), B=2, H=4, Dk=128, Dv=128, dtype=0, stream=None)
    a.update(kw)
    L = N.lib()
    rc = L.lin_attn_decode_step_channel(a["q"], a["k"], a["v"], a["gate"], a["gate_mode"], a["G"],
                                        a["beta"], a["S"], a["o"], a["B"], a["H"], a["Dk"],
                                        a["Dv"], a["dtype"], a["stream"])
    return rc, L.lin_attn_last_error().decode()


@pytest.mark.parametrize("kw,code,needle", [
    (dict(gate=None), N.LA_EINVAL, "gate must not be NULL"),
    (dict(G=12.0), N.LA_ERANGE, "per-channel"),
    (dict(Dk=96), N.LA_EUNSUPPORTED, "decode supports"),
    # the per-channel gate is B*H*Dk floats: an o placed inside it overlaps
    (dict(o=fake(3) + 2 * 4 * 4 * 64), N.LA_EINVAL, "o overlaps gate"),
    (dict(S=fake(3) + 2 * 4 * 4 * 64), N.LA_EINVAL, "S overlaps gate"),
])
def test_decode_channel_rejects(kw, code, needle):
    rc, msg = decode_ch(**kw)
    assert rc == code and needle in msg, (rc, msg)


def test_decode_channel_empty_is_noop():
    assert decode_ch(B=0)[0] == N.LA_OK


def channel_varlen(**kw):
    a = dict(q=fake(0), k=fake(1), v=fake(2), gate=fake(3), gate_mode=1, G=5.0, beta=fake(4),
             h0=None, o=fake(5), hT=fake(6), cu=fake(7), nseq=3, T=64, H=2, Dk=128, Dv=128,
             dtype=0, ws=fake(8), ws_bytes=1 << 30, stream=None)
    a.update(kw)
    L = N.lib()
    rc = L.lin_attn_chunk_fwd_channel_varlen(a["q"], a["k"], a["v"], a["gate"], a["gate_mode"],
                                             a["G"], a["beta"], a["h0"], a["o"], a["hT"], a["cu"],
                                             a["nseq"], a["T"], a["H"], a["Dk"], a["Dv"],
                                             a["dtype"], a["ws"], a["ws_bytes"], a["stream"])
    return rc, L.lin_attn_last_error().decode()


@pytest.mark.parametrize("kw,code,needle", [
    (dict(cu=None), N.LA_EINVAL, "cu_seqlens must not be NULL"),
    (dict(nseq=-1), N.LA_EINVAL, "nseq"),
    (dict(G=11.0), N.LA_ERANGE, "per-channel"),
    (dict(gate=fake(3) + 8), N.LA_EINVAL, "gate must be 16-byte aligned"),
    (dict(ws_bytes=100), N.LA_EINVAL, "workspace too small"),
    (dict(o=fake(3) + 64 * 2 * 4 * 64), N.LA_EINVAL, "o overlaps gate"),
    (dict(hT=fake(7)), N.LA_EINVAL, "hT overlaps cu_seqlens"),
])
def test_channel_varlen_rejects(kw, code, needle):
    rc, msg = channel_varlen(**kw)
    assert rc == code and needle in msg, (rc, msg)


def test_channel_varlen_workspace_size_and_empty():
    L = N.lib()
    assert L.lin_attn_chunk_fwd_channel_varlen_workspace_size(100, 3, 2, 128, 128, 0) == \
        max(2 * (100 // 16 + 3 + 1) * 18944, 2 * (100 // 32 + 3 + 1) * 31232)
    assert L.lin_attn_chunk_fwd_channel_varlen_workspace_size(1000, 1, 2, 128, 128, 0) == \
        max(2 * (1000 // 16 + 1 + 1) * 18944, 2 * (1000 // 32 + 1 + 1) * 31232)
    assert L.lin_attn_chunk_fwd_channel_varlen_workspace_size(100, 3, 2, 64, 32, 1) == \
        2 * (100 // 16 + 3 + 1) * 14592
    assert channel_varlen(nseq=0)[0] == N.LA_OK


def bwd_varlen(**kw):
    a = dict(q=fake(0), k=fake(1), v=fake(2), gate=fake(3), gate_mode=0, G=5.0, beta=fake(4),
             h0=None, dout=fake(5), dhT=None, dq=fake(6), dk=fake(7), dv=fake(8),
             dgate=fake(9), dbeta=fake(10), dh0=None, cu=fake(11), nseq=3, T=64, H=2, Dk=128,
             Dv=128, dtype=N.LA_BF16, ws=fake(12), ws_bytes=1 << 40, stream=None)
    a.update(kw)
    L = N.lib()
    rc = L.lin_attn_chunk_bwd_varlen(*a.values())
    return rc, L.lin_attn_last_error().decode()


@pytest.mark.parametrize("kw,code,needle", [
    (dict(cu=None), N.LA_EINVAL, "cu_seqlens must not be NULL"),
    (dict(cu=fake(11) + 2), N.LA_EINVAL, "cu_seqlens must be 4-byte aligned"),
    (dict(nseq=-1), N.LA_EINVAL, "nseq"),
    (dict(Dk=96), N.LA_EUNSUPPORTED, "Dk"),
    (dict(dq=fake(6) + 4), N.LA_EINVAL, "dq must be 16-byte aligned"),
    (dict(ws=None), N.LA_EINVAL, "workspace must not be NULL"),
    (dict(ws_bytes=10), N.LA_EINVAL, "workspace too small"),
    (dict(dq=fake(0) + 64), N.LA_EINVAL, "dq overlaps q"),
    (dict(dh0=fake(11)), N.LA_EINVAL, "dh0 overlaps cu_seqlens"),
    (dict(gate_mode=7), N.LA_EINVAL, "gate_mode"),
])
def test_bwd_varlen_rejects(kw, code, needle):
    rc, msg = bwd_varlen(**kw)
    assert rc == code, (rc, msg)
    assert needle in msg


def test_bwd_segmented_workspace_size_and_validation():
    L = N.lib()
    ws = L.lin_attn_chunk_bwd_segmented_workspace_size
    one = L.lin_attn_chunk_bwd_workspace_size
    # one segment's workspace (rounded up to 256 bytes), then ceil(T / seg) + 1
    # float32 states per head, whatever B
    seg = one(1, 256, 2, 128, 128, N.LA_BF16)
    assert ws(3, 1000, 2, 128, 128, N.LA_BF16, 256) == (seg + 255) // 256 * 256 + 5 * 2 * 128 * 128 * 4
    short = one(1, 100, 2, 64, 32, N.LA_BF16)
    assert ws(1, 100, 2, 64, 32, N.LA_BF16, 256) == (short + 255) // 256 * 256 + 2 * 2 * 64 * 32 * 4
    assert ws(1, 0, 2, 128, 128, N.LA_BF16, 256) == 0
    for bad in (0, -64, 100, 32):
        assert ws(1, 1000, 2, 128, 128, N.LA_BF16, bad) == -1
    assert ws(1, 1000, 2, 128, 128, N.LA_FP32, 256) == -1
    assert ws(1, 1000, 2, 128, 144, N.LA_BF16, 256) == -1
    assert ws(1, 1000, 2, 96, 128, N.LA_BF16, 256) == -1


def test_bwd_varlen_workspace_size_and_empty():
    ws = N.lib().lin_attn_chunk_bwd_varlen_workspace_size
    per_tile = 3200 + 8 * 128 * 128
    assert ws(64, 3, 2, 128, 128, N.LA_FP32) == 2 * (64 // 16 + 3 + 1) * per_tile
    # bf16: records per tile slot; per group slot (H * (T / 64 + nseq + 1)
    # of them) two packed states and one packed state gradient
    assert ws(64, 3, 2, 128, 128, N.LA_BF16) == \
        2 * (64 // 16 + 3 + 1) * 3200 + 2 * (64 // 64 + 3 + 1) * 12 * 128 * 128
    assert ws(1000, 5, 3, 64, 32, N.LA_BF16) == \
        3 * (1000 // 16 + 5 + 1) * 3200 + 3 * (1000 // 64 + 5 + 1) * 12 * 64 * 32
    assert ws(64, -1, 2, 128, 128, N.LA_BF16) == -1
    # no sequences: nothing to do, nothing touched
    assert bwd_varlen(nseq=0, q=None, cu=None, ws=None)[0] == N.LA_OK


def test_check_inputs_host_validation():
    # host-side rejections happen before any device work (no GPU needed)
    L = N.lib()
    P = 0x10000
    args = dict(q=P, k=P, v=P, gate=P, gm=N.LA_GATE_LOG, G=5.0, beta=P, h0=None, ntok=4,
                nstate=1, H=2, Dk=128, Dv=128, ch=0, dt=N.LA_BF16, flags=P, st=None)

    def call(**kw):
        a = dict(args, **kw)
        return L.lin_attn_check_inputs(a["q"], a["k"], a["v"], a["gate"], a["gm"], a["G"],
                                       a["beta"], a["h0"], a["ntok"], a["nstate"], a["H"],
                                       a["Dk"], a["Dv"], a["ch"], a["dt"], a["flags"], a["st"])

    assert call(flags=None) == N.LA_EINVAL
    assert b"flags" in L.lin_attn_last_error()
    assert call(flags=P + 2) == N.LA_EINVAL
    assert call(G=20.0) == N.LA_ERANGE
    assert call(gm=7) == N.LA_EINVAL
    assert call(ntok=-1) == N.LA_EINVAL
    assert call(dt=5) == N.LA_EINVAL
    assert call(q=None) == N.LA_EINVAL
    assert b"q must not be NULL" in L.lin_attn_last_error()
