"""fp64 CPU oracle for attention (test infrastructure only).

Only the test suite, the package's ``smoke()`` check and the benchmark's CPU
baseline may import this module. The HIP product path never does: it shares no
code with the oracle, and neither imports the other.

The oracle computes Eq. (1) of Rao et al., "Scheduling Data to Compute:
Hierarchical Data Pipelining for LLM Training on AMD GPUs", section 2.1, naively
in double precision, plus the exact gradient of that equation (the products
section 2.1's Table 3 lists for the backward pass). The C source,
``attn_oracle.c``, documents every reading of the page it takes.

Inputs are numpy ``uint16`` arrays of bf16 bit patterns in [B][H][S][D] layout
(V and dO may have their own last dimension Dv, the d_v of Eq. (1)); outputs are
float64 arrays.
"""
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "attn_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")


def build(force=True, src=_SRC, out=_LIB):
    """Compile the oracle with gcc (OpenMP, no fast-math) into a shared library."""
    if not force and os.path.exists(out) and os.path.getmtime(out) >= os.path.getmtime(src):
        return out
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c99", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra",
           "-o", tmp, src, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def _shapes(q, k, v, dout=None):
    for name, a in (("q", q), ("k", k), ("v", v), ("dout", dout)):
        if a is None:
            continue
        if a.dtype != np.uint16 or a.ndim != 4 or not a.flags.c_contiguous:
            raise ValueError("%s must be a C-contiguous uint16 [B][H][S][D] array of bf16 bits" % name)
    B, Hq, S, D = q.shape
    Hkv = k.shape[1]
    Dv = v.shape[3]
    if k.shape != (B, Hkv, S, D) or v.shape != (B, Hkv, S, Dv):
        raise ValueError("k must be [B][Hkv][S][D] and v [B][Hkv][S][Dv], matching q")
    if dout is not None and dout.shape != (B, Hq, S, Dv):
        raise ValueError("dout must be [B][Hq][S][Dv]")
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    return B, Hq, Hkv, S, D, Dv


class Oracle:
    """ctypes binding of one compiled oracle library."""

    def __init__(self, path):
        lib = ctypes.CDLL(path)
        P = ctypes.c_void_p
        I = ctypes.c_int
        I64 = ctypes.c_int64
        Dbl = ctypes.c_double
        lib.oracle_num_threads.restype = I
        lib.oracle_attn_fwd.argtypes = [P, P, P, P, P, I, I, I, I, I, I, I, I, Dbl]
        lib.oracle_attn_fwd_rows.argtypes = [P, P, P, P, I64, P, P, I, I, I, I, I, I, I, I, Dbl]
        lib.oracle_attn_bwd.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, I, I, I, Dbl]
        lib.oracle_attn_bwd_rows.argtypes = [P, P, P, P, P, I64, P, P, I64, P, P,
                                             I, I, I, I, I, I, I, I, Dbl]
        for f in (lib.oracle_attn_fwd, lib.oracle_attn_fwd_rows, lib.oracle_attn_bwd,
                  lib.oracle_attn_bwd_rows):
            f.restype = I
        self.lib = lib
        self.path = path

    def num_threads(self):
        """OpenMP threads the oracle uses (honours OMP_NUM_THREADS)."""
        return self.lib.oracle_num_threads()

    def fwd(self, q, k, v, causal, scale, window=0):
        """O [B,Hq,S,Dv] and lse [B,Hq,S] (natural log), float64. window > 0 (causal only):
        query i sees keys i-window+1 .. i."""
        B, Hq, Hkv, S, D, Dv = _shapes(q, k, v)
        o = np.empty((B, Hq, S, Dv), np.float64)
        lse = np.empty((B, Hq, S), np.float64)
        rc = self.lib.oracle_attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                                      B, Hq, Hkv, S, D, Dv, int(bool(causal)), int(window), float(scale))
        if rc:
            raise ValueError("oracle_attn_fwd failed: %d" % rc)
        return o, lse

    def fwd_rows(self, q, k, v, rows, causal, scale, window=0):
        """O and lse of selected flat query rows ((b*Hq + hq)*S + i)."""
        B, Hq, Hkv, S, D, Dv = _shapes(q, k, v)
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        o = np.empty((rows.size, Dv), np.float64)
        lse = np.empty((rows.size,), np.float64)
        rc = self.lib.oracle_attn_fwd_rows(_ptr(q), _ptr(k), _ptr(v), _ptr(rows), rows.size,
                                           _ptr(o), _ptr(lse), B, Hq, Hkv, S, D, Dv,
                                           int(bool(causal)), int(window), float(scale))
        if rc:
            raise ValueError("oracle_attn_fwd_rows failed: %d" % rc)
        return o, lse

    def bwd(self, q, k, v, dout, causal, scale, window=0):
        """dQ [B,Hq,S,D], dK [B,Hkv,S,D] and dV [B,Hkv,S,Dv] (summed over each group), float64."""
        B, Hq, Hkv, S, D, Dv = _shapes(q, k, v, dout)
        dq = np.empty((B, Hq, S, D), np.float64)
        dk = np.empty((B, Hkv, S, D), np.float64)
        dv = np.empty((B, Hkv, S, Dv), np.float64)
        rc = self.lib.oracle_attn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(dout), _ptr(dq),
                                      _ptr(dk), _ptr(dv), B, Hq, Hkv, S, D, Dv,
                                      int(bool(causal)), int(window), float(scale))
        if rc:
            raise ValueError("oracle_attn_bwd failed: %d" % rc)
        return dq, dk, dv

    def bwd_rows(self, q, k, v, dout, qrows, kvrows, causal, scale, window=0):
        """dQ of selected query rows; dK, dV of selected key rows ((b*Hkv + hkv)*S + j)."""
        B, Hq, Hkv, S, D, Dv = _shapes(q, k, v, dout)
        qrows = np.ascontiguousarray(qrows, dtype=np.int64)
        kvrows = np.ascontiguousarray(kvrows, dtype=np.int64)
        dq = np.empty((qrows.size, D), np.float64)
        dk = np.empty((kvrows.size, D), np.float64)
        dv = np.empty((kvrows.size, Dv), np.float64)
        rc = self.lib.oracle_attn_bwd_rows(_ptr(q), _ptr(k), _ptr(v), _ptr(dout), _ptr(qrows),
                                           qrows.size, _ptr(dq), _ptr(kvrows), kvrows.size,
                                           _ptr(dk), _ptr(dv), B, Hq, Hkv, S, D, Dv,
                                           int(bool(causal)), int(window), float(scale))
        if rc:
            raise ValueError("oracle_attn_bwd_rows failed: %d" % rc)
        return dq, dk, dv


_default = None


def default():
    """The oracle built from attn_oracle.c (built on first use if missing or stale)."""
    global _default
    if _default is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        _default = Oracle(_LIB)
    return _default


def num_threads():
    return default().num_threads()


def fwd(q, k, v, causal, scale, window=0):
    return default().fwd(q, k, v, causal, scale, window)


def fwd_rows(q, k, v, rows, causal, scale, window=0):
    return default().fwd_rows(q, k, v, rows, causal, scale, window)


def bwd(q, k, v, dout, causal, scale, window=0):
    return default().bwd(q, k, v, dout, causal, scale, window)


def bwd_rows(q, k, v, dout, qrows, kvrows, causal, scale, window=0):
    return default().bwd_rows(q, k, v, dout, qrows, kvrows, causal, scale, window)
