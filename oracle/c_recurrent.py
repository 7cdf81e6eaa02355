"""ctypes wrapper of recurrent.c (the same fp64 recurrences as
linattn_oracle.recurrent_fwd, recurrent_fwd_channel and the adjoint
recurrent_bwd, in plain C for speed on long sequences).

TEST INFRASTRUCTURE ONLY (see linattn_oracle.py's header).  Independent
(batch, head) streams run on a thread pool; each C call releases the GIL.
"""

from __future__ import annotations

import concurrent.futures as cf
import ctypes
import os
import subprocess
import threading

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "recurrent.c")
LIB = os.path.join(HERE, "liboracle_rec.so")
_lib = None
_lock = threading.Lock()


def build() -> str:
    """Compile recurrent.c with gcc (-O3, no target-specific flags)."""
    tmp = LIB + ".tmp"
    subprocess.run(["gcc", "-O3", "-fPIC", "-shared", SRC, "-o", tmp, "-lm"], check=True)
    os.replace(tmp, LIB)
    return LIB


def _load():
    global _lib
    with _lock:
        return _load_locked()


def _load_locked():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
            build()
        L = ctypes.CDLL(LIB)
        P = ctypes.c_void_p
        L.oracle_head_fwd.restype = ctypes.c_int
        LL, I = ctypes.c_longlong, ctypes.c_int
        L.oracle_head_fwd.argtypes = [P, P, P, P, P, LL, LL, LL, I, I, I, P, P]
        L.oracle_head_fwd_channel.restype = ctypes.c_int
        L.oracle_head_fwd_channel.argtypes = [P, P, P, P, P, LL, LL, LL, LL, I, I, I, P, P]
        L.oracle_head_bwd.restype = ctypes.c_int
        L.oracle_head_bwd.argtypes = [P, P, P, P, P, P, LL, LL, LL, I, I, I, P, P, P, P, P,
                                      P, P, I]
        _lib = L
    return _lib


def _c64(a):
    return np.ascontiguousarray(a, dtype=np.float64)


def head_fwd(q, k, v, g, beta, h=None, want_o=True):
    """One stream: q, k [T, Dk], v [T, Dv], g, beta [T]; h [Dk, Dv] initial state.
    Returns (o [T, Dv] or None, hT [Dk, Dv])."""
    L = _load()
    q, k, v, g, beta = map(_c64, (q, k, v, g, beta))
    T, Dk = q.shape
    Dv = v.shape[1]
    st = np.zeros((Dk, Dv)) if h is None else _c64(h).copy()
    o = np.empty((T, Dv)) if want_o else None
    rc = L.oracle_head_fwd(q.ctypes.data, k.ctypes.data, v.ctypes.data, g.ctypes.data,
                           beta.ctypes.data, Dk, Dv, 1, T, Dk, Dv, st.ctypes.data,
                           o.ctypes.data if want_o else None)
    if rc:
        raise MemoryError("oracle_head_fwd failed")
    return o, st


def recurrent_fwd_c(q, k, v, g, beta, h0=None, heads=None, t_range=None, workers=None):
    """recurrent_fwd on selected (b, h) streams over tokens [t0, t1) with h0 the
    state before t0.  Returns {(b, h): (o [t1-t0, Dv], hT [Dk, Dv])}."""
    B, T, H, _ = np.shape(q)
    if heads is None:
        heads = [(b, h) for b in range(B) for h in range(H)]
    t0, t1 = (0, T) if t_range is None else t_range
    if workers is None:
        workers = min(16, os.cpu_count() or 1)

    def one(bh):
        b, h = bh
        init = None if h0 is None else h0[b, h]
        return head_fwd(q[b, t0:t1, h], k[b, t0:t1, h], v[b, t0:t1, h], g[b, t0:t1, h],
                        beta[b, t0:t1, h], init)

    with cf.ThreadPoolExecutor(max(1, min(workers, len(heads)))) as ex:
        res = list(ex.map(one, heads))
    return dict(zip(heads, res))


def recurrent_fwd(q, k, v, g, beta, h0=None, workers=None):
    """Full-array form with the same signature and result as
    linattn_oracle.recurrent_fwd: (o [B,T,H,Dv], hT [B,H,Dk,Dv])."""
    B, T, H, Dk = np.shape(q)
    Dv = np.shape(v)[-1]
    res = recurrent_fwd_c(q, k, v, g, beta, h0, workers=workers)
    o = np.empty((B, T, H, Dv))
    hT = np.empty((B, H, Dk, Dv))
    for (b, h), (ob, hb) in res.items():
        o[b, :, h] = ob
        hT[b, h] = hb
    return o, hT


def recurrent_fwd_varlen(q, k, v, g, beta, cu_seqlens, h0=None, workers=None):
    """Packed sequences with the same signature and result as
    linattn_oracle.recurrent_fwd_varlen, one (sequence, head) stream per task."""
    cu = [int(x) for x in cu_seqlens]
    _, T, H, Dk = np.shape(q)
    Dv = np.shape(v)[-1]
    N = len(cu) - 1
    if workers is None:
        workers = min(16, os.cpu_count() or 1)
    tasks = [(s, h) for s in range(N) for h in range(H) if cu[s + 1] > cu[s]]

    def one(sh):
        s, h = sh
        a, b = cu[s], cu[s + 1]
        init = None if h0 is None else h0[s, h]
        return head_fwd(q[0, a:b, h], k[0, a:b, h], v[0, a:b, h], g[0, a:b, h], beta[0, a:b, h], init)

    o = np.empty((1, T, H, Dv))
    hT = np.zeros((N, H, Dk, Dv))
    if h0 is not None:
        hT[:] = np.asarray(h0, dtype=np.float64)
    with cf.ThreadPoolExecutor(max(1, min(workers, max(1, len(tasks))))) as ex:
        for (s, h), (os_, hs) in zip(tasks, ex.map(one, tasks)):
            o[0, cu[s]:cu[s + 1], h] = os_
            hT[s, h] = hs
    return o, hT


def head_fwd_channel(q, k, v, g, beta, h=None, want_o=True):
    """One stream with a per-channel gate: q, k, g [T, Dk], v [T, Dv], beta [T];
    h [Dk, Dv] initial state.  Returns (o [T, Dv] or None, hT [Dk, Dv])."""
    L = _load()
    q, k, v, g, beta = map(_c64, (q, k, v, g, beta))
    T, Dk = q.shape
    Dv = v.shape[1]
    st = np.zeros((Dk, Dv)) if h is None else _c64(h).copy()
    o = np.empty((T, Dv)) if want_o else None
    rc = L.oracle_head_fwd_channel(q.ctypes.data, k.ctypes.data, v.ctypes.data, g.ctypes.data,
                                   beta.ctypes.data, Dk, Dv, Dk, 1, T, Dk, Dv, st.ctypes.data,
                                   o.ctypes.data if want_o else None)
    if rc:
        raise MemoryError("oracle_head_fwd_channel failed")
    return o, st


def recurrent_fwd_channel_c(q, k, v, g, beta, h0=None, heads=None, t_range=None, workers=None):
    """recurrent_fwd_channel on selected (b, h) streams over tokens [t0, t1),
    h0 the state before t0 (g is [B, T, H, Dk]).  Returns
    {(b, h): (o [t1-t0, Dv], hT [Dk, Dv])}."""
    B, T, H, _ = np.shape(q)
    if heads is None:
        heads = [(b, h) for b in range(B) for h in range(H)]
    t0, t1 = (0, T) if t_range is None else t_range
    if workers is None:
        workers = min(16, os.cpu_count() or 1)

    def one(bh):
        b, h = bh
        init = None if h0 is None else h0[b, h]
        return head_fwd_channel(q[b, t0:t1, h], k[b, t0:t1, h], v[b, t0:t1, h], g[b, t0:t1, h],
                                beta[b, t0:t1, h], init)

    with cf.ThreadPoolExecutor(max(1, min(workers, len(heads)))) as ex:
        res = list(ex.map(one, heads))
    return dict(zip(heads, res))


def recurrent_fwd_channel(q, k, v, g, beta, h0=None, workers=None):
    """Full-array form with the signature and result of
    linattn_oracle.recurrent_fwd_channel: (o [B,T,H,Dv], hT [B,H,Dk,Dv])."""
    B, T, H, Dk = np.shape(q)
    Dv = np.shape(v)[-1]
    res = recurrent_fwd_channel_c(q, k, v, g, beta, h0, workers=workers)
    o = np.empty((B, T, H, Dv))
    hT = np.empty((B, H, Dk, Dv))
    for (b, h), (ob, hb) in res.items():
        o[b, :, h] = ob
        hT[b, h] = hb
    return o, hT


def head_bwd(q, k, v, g, beta, do, dhT=None, h0=None, seg=64):
    """Reverse mode of one stream: q, k [T, Dk], v, do [T, Dv], g, beta [T];
    dhT, h0 [Dk, Dv] or None.  Returns (dq, dk, dv, dg, dbeta, dh0) in float64."""
    L = _load()
    q, k, v, g, beta, do = map(_c64, (q, k, v, g, beta, do))
    T, Dk = q.shape
    Dv = v.shape[1]
    dh = np.zeros((Dk, Dv)) if dhT is None else _c64(dhT).copy()
    h0c = None if h0 is None else _c64(h0)
    dq, dk = np.zeros((T, Dk)), np.zeros((T, Dk))
    dv = np.zeros((T, Dv))
    dg, dbeta = np.zeros(T), np.zeros(T)
    rc = L.oracle_head_bwd(q.ctypes.data, k.ctypes.data, v.ctypes.data, g.ctypes.data,
                           beta.ctypes.data, do.ctypes.data, Dk, Dv, 1, T, Dk, Dv,
                           None if h0c is None else h0c.ctypes.data, dh.ctypes.data,
                           dq.ctypes.data, dk.ctypes.data, dv.ctypes.data, dg.ctypes.data,
                           dbeta.ctypes.data, int(seg))
    if rc:
        raise MemoryError("oracle_head_bwd failed")
    return dq, dk, dv, dg, dbeta, dh


def recurrent_bwd_c(q, k, v, g, beta, do, dhT=None, h0=None, heads=None, workers=None):
    """recurrent_bwd on selected (b, h) streams.  Returns
    {(b, h): (dq [T,Dk], dk [T,Dk], dv [T,Dv], dg [T], dbeta [T], dh0 [Dk,Dv])}."""
    B, T, H, _ = np.shape(q)
    if heads is None:
        heads = [(b, h) for b in range(B) for h in range(H)]
    if workers is None:
        workers = min(16, os.cpu_count() or 1)

    def one(bh):
        b, h = bh
        return head_bwd(q[b, :, h], k[b, :, h], v[b, :, h], g[b, :, h], beta[b, :, h],
                        do[b, :, h], None if dhT is None else dhT[b, h],
                        None if h0 is None else h0[b, h])

    with cf.ThreadPoolExecutor(max(1, min(workers, len(heads)))) as ex:
        res = list(ex.map(one, heads))
    return dict(zip(heads, res))


def recurrent_bwd(q, k, v, g, beta, do, dhT=None, h0=None, workers=None):
    """Full-array form with the signature and result of
    linattn_oracle.recurrent_bwd: (dq, dk, dv, dg, dbeta, dh0)."""
    B, T, H, Dk = np.shape(q)
    Dv = np.shape(v)[-1]
    res = recurrent_bwd_c(q, k, v, g, beta, do, dhT, h0, workers=workers)
    dq, dk = np.empty((B, T, H, Dk)), np.empty((B, T, H, Dk))
    dv = np.empty((B, T, H, Dv))
    dg, dbeta = np.empty((B, T, H)), np.empty((B, T, H))
    dh0 = np.empty((B, H, Dk, Dv))
    for (b, h), r in res.items():
        dq[b, :, h], dk[b, :, h], dv[b, :, h], dg[b, :, h], dbeta[b, :, h], dh0[b, h] = r
    return dq, dk, dv, dg, dbeta, dh0
