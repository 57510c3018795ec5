"""ctypes loader for the C float64 oracle (``kda_oracle.c``).

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg, never by the GPU library.

``build()`` compiles ``kda_oracle.c`` with gcc + OpenMP into
``oracle/liboracle.so``; ``recurrent()`` and ``backward()`` call it on float64
NumPy arrays; ``recurrent_varlen()`` runs packed documents through ``recurrent()``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kda_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None

GATE_MODES = {"bounded": 0, "logsigmoid": 1}


def build(force: bool = True) -> str:
    """Compile the C oracle (gcc -O2 -fopenmp); returns the library path."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-fno-fast-math", "-fopenmp", "-fPIC", "-shared",
               "-std=c99", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=True)
        lib = ctypes.CDLL(_LIB)
        dp = ctypes.POINTER(ctypes.c_double)
        lib.kda_oracle_recurrent.argtypes = [dp, dp, dp, dp, dp] + [ctypes.c_long] * 5 + [
            ctypes.c_double, ctypes.c_int, ctypes.c_int, dp, dp, dp]
        lib.kda_oracle_recurrent.restype = ctypes.c_int
        lib.kda_oracle_threads.restype = ctypes.c_int
        lib.kda_oracle_set_threads.argtypes = [ctypes.c_int]
        lib.kda_oracle_set_threads.restype = ctypes.c_int
        lib.kda_oracle_backward.argtypes = [dp, dp, dp, dp, dp] + [ctypes.c_long] * 5 + [
            ctypes.c_double, ctypes.c_int, dp, dp, dp, dp, dp, dp, dp, dp, dp]
        lib.kda_oracle_backward.restype = ctypes.c_int
        _lib = lib
    return _lib


def threads() -> int:
    """OpenMP threads the oracle uses."""
    return int(_load().kda_oracle_threads())


def set_threads(n: int) -> int:
    """Threads of the calls that follow; returns the previous count."""
    return int(_load().kda_oracle_set_threads(int(n)))


def cpu_model() -> str:
    """The host CPU's model name (Linux), for reporting the oracle's timings."""
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _f64(x):
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(x):
    return None if x is None else x.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def recurrent(q, k, v, a, beta, g_min=-5.0, gate="bounded", erase=True, S0=None):
    """Token-by-token float64 recurrence (see kda_oracle.c for the definition).

    Shapes: q, k, a [B,H,T,dk]; v [B,H,T,dv]; beta [B,H,T]; S0 [B,H,dv,dk] or None.
    Returns (out [B,H,T,dv], final_state [B,H,dv,dk]) as float64 arrays.
    """
    q, k, v, a, beta = (_f64(x) for x in (q, k, v, a, beta))
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    assert k.shape == q.shape and a.shape == q.shape
    assert v.shape == (B, H, T, dv) and beta.shape == (B, H, T)
    S0 = None if S0 is None else _f64(S0)
    if S0 is not None:
        assert S0.shape == (B, H, dv, dk)
    out = np.empty((B, H, T, dv), dtype=np.float64)
    fin = np.empty((B, H, dv, dk), dtype=np.float64)
    rc = _load().kda_oracle_recurrent(_ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(beta),
                                      B, H, T, dk, dv, float(g_min), GATE_MODES[gate],
                                      1 if erase else 0, _ptr(S0), _ptr(out), _ptr(fin))
    if rc != 0:
        raise RuntimeError("kda_oracle_recurrent failed with %d" % rc)
    return out, fin


def backward(q, k, v, a, beta, dout, g_min=-5.0, gate="bounded", S0=None, dfinal=None):
    """Gradients of L = sum(dout * out) + sum(dfinal * final_state) of the token recurrence
    with respect to q, k, v, a, beta and the initial state (see kda_oracle.c for the
    adjoint, written out by hand).  Shapes as recurrent(); dout [B,H,T,dv], dfinal
    [B,H,dv,dk] or None.  Returns a dict of float64 arrays dq, dk, dv, da, dbeta, dS0."""
    q, k, v, a, beta, dout = (_f64(x) for x in (q, k, v, a, beta, dout))
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    assert dout.shape == v.shape
    S0 = None if S0 is None else _f64(S0)
    dfinal = None if dfinal is None else _f64(dfinal)
    res = {n: np.empty(s, dtype=np.float64) for n, s in (("dq", q.shape), ("dk", q.shape), ("dv", v.shape),
                                                          ("da", q.shape), ("dbeta", beta.shape),
                                                          ("dS0", (B, H, dv, dk)))}
    rc = _load().kda_oracle_backward(_ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(beta), B, H, T, dk, dv,
                                     float(g_min), GATE_MODES[gate], _ptr(S0), _ptr(dout), _ptr(dfinal),
                                     _ptr(res["dq"]), _ptr(res["dk"]), _ptr(res["dv"]), _ptr(res["da"]),
                                     _ptr(res["dbeta"]), _ptr(res["dS0"]))
    if rc != 0:
        raise RuntimeError("kda_oracle_backward failed with %d" % rc)
    return res


def recurrent_varlen(q, k, v, a, beta, cu_seqlens, g_min=-5.0, gate="bounded", S0=None):
    """Packed documents: N documents laid end to end in one token stream per head
    ("Breaking Through Trillion-Parameter Multimodal MoE ...", sec. 3: short
    documents packed into one long sequence in the 256K-1M phase).  Read as: every
    document is its own sequence of the recurrence -- it starts from its own state
    (S0[i], else zero) and nothing crosses a document boundary.

    Shapes: q, k, a [H,T,dk]; v [H,T,dv]; beta [H,T]; cu_seqlens [N+1] ints,
    nondecreasing, cu_seqlens[0] = 0, cu_seqlens[N] = T; S0 [N,H,dv,dk] or None.
    Returns (out [H,T,dv], final_state [N,H,dv,dk]) as float64 arrays.
    """
    q, k, v, a, beta = (_f64(x) for x in (q, k, v, a, beta))
    cu = [int(x) for x in np.asarray(cu_seqlens).ravel()]
    H, T, dk = q.shape
    dv = v.shape[-1]
    N = len(cu) - 1
    assert N >= 1 and cu[0] == 0 and cu[-1] == T and all(x <= y for x, y in zip(cu, cu[1:]))
    out = np.zeros((H, T, dv), dtype=np.float64)
    fin = np.empty((N, H, dv, dk), dtype=np.float64)
    for i in range(N):
        s, e = cu[i], cu[i + 1]
        o, f = recurrent(q[None, :, s:e], k[None, :, s:e], v[None, :, s:e], a[None, :, s:e], beta[None, :, s:e],
                         g_min, gate, S0=None if S0 is None else _f64(S0)[i:i + 1])
        out[:, s:e] = o[0]
        fin[i] = f[0]
    return out, fin
