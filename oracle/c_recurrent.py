"""ctypes wrapper of recurrent.c (the same fp64 recurrence as
linattn_oracle.recurrent_fwd, in plain C for speed on long sequences).

TEST INFRASTRUCTURE ONLY (see linattn_oracle.py's header).  Independent
(batch, head) streams run on a thread pool; each C call releases the GIL.
"""

from __future__ import annotations

import concurrent.futures as cf
import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "recurrent.c")
LIB = os.path.join(HERE, "liboracle_rec.so")
_lib = None


def build() -> str:
    """Compile recurrent.c with gcc (-O3, no target-specific flags)."""
    tmp = LIB + ".tmp"
    subprocess.run(["gcc", "-O3", "-fPIC", "-shared", SRC, "-o", tmp, "-lm"], check=True)
    os.replace(tmp, LIB)
    return LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
            build()
        L = ctypes.CDLL(LIB)
        P = ctypes.c_void_p
        L.oracle_head_fwd.restype = ctypes.c_int
        L.oracle_head_fwd.argtypes = [P, P, P, P, P, ctypes.c_longlong, ctypes.c_longlong,
                                      ctypes.c_longlong, ctypes.c_int, ctypes.c_int,
                                      ctypes.c_int, P, P]
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
