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
        lib.oracle_sparse_fwd_rows.argtypes = [P, P, P, P, P, I64, P, P, I, I, I, I, I, I, I, Dbl]
        lib.oracle_sparse_bwd_rows.argtypes = [P, P, P, P, P, P, I64, P, P, I64, P, P,
                                               I, I, I, I, I, I, I, Dbl]
        for f in (lib.oracle_attn_fwd, lib.oracle_attn_fwd_rows, lib.oracle_attn_bwd,
                  lib.oracle_attn_bwd_rows, lib.oracle_sparse_fwd_rows, lib.oracle_sparse_bwd_rows):
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


    # ------------------------------------------------------------ sparse attention

    def sparse_fwd(self, q, k, v, idx, scale, rows=None):
        """Attention over per-token index lists. q [B,Hq,S,D]; k, v [B,Hkv,N,D]; idx
        [B,S,topk] int32 (entries outside [0, N) are empty slots). O [B,Hq,S,D] and lse
        [B,Hq,S] (-inf for a token with no non-empty slot), or, with rows (flat query rows
        (b*Hq + hq)*S + i), O [n,D] and lse [n]."""
        B, Hq, Hkv, S, N, D, topk = _sparse_shapes(q, k, v, idx)
        if rows is None:
            o = np.empty((B, Hq, S, D), np.float64)
            lse = np.empty((B, Hq, S), np.float64)
            rp, n = None, 0
        else:
            rows = np.ascontiguousarray(rows, dtype=np.int64)
            o = np.empty((rows.size, D), np.float64)
            lse = np.empty((rows.size,), np.float64)
            rp, n = _ptr(rows), rows.size
        rc = self.lib.oracle_sparse_fwd_rows(_ptr(q), _ptr(k), _ptr(v), _ptr(idx), rp, n, _ptr(o), _ptr(lse),
                                             B, Hq, Hkv, S, N, D, topk, float(scale))
        if rc:
            raise ValueError("oracle_sparse_fwd_rows failed: %d" % rc)
        return o, lse

    def sparse_bwd(self, q, k, v, dout, idx, scale, qrows=None, kvrows=None):
        """Gradients of sparse_fwd: dQ [B,Hq,S,D], dK and dV [B,Hkv,N,D] (summed over every
        (token, slot) that names the row and over the group's heads); with qrows / kvrows
        (flat (b*Hkv + hkv)*N + j), only those rows, as [n,D] arrays."""
        B, Hq, Hkv, S, N, D, topk = _sparse_shapes(q, k, v, idx, dout)
        if qrows is None:
            dq = np.empty((B, Hq, S, D), np.float64)
            qp, nq = None, 0
        else:
            qrows = np.ascontiguousarray(qrows, dtype=np.int64)
            dq = np.empty((qrows.size, D), np.float64)
            qp, nq = _ptr(qrows), qrows.size
        if kvrows is None:
            dk = np.empty((B, Hkv, N, D), np.float64)
            dv = np.empty((B, Hkv, N, D), np.float64)
            kp, nkv = None, 0
        else:
            kvrows = np.ascontiguousarray(kvrows, dtype=np.int64)
            dk = np.empty((kvrows.size, D), np.float64)
            dv = np.empty((kvrows.size, D), np.float64)
            kp, nkv = _ptr(kvrows), kvrows.size
        rc = self.lib.oracle_sparse_bwd_rows(_ptr(q), _ptr(k), _ptr(v), _ptr(dout), _ptr(idx), qp, nq,
                                             _ptr(dq), kp, nkv, _ptr(dk), _ptr(dv), B, Hq, Hkv, S, N, D, topk,
                                             float(scale))
        if rc:
            raise ValueError("oracle_sparse_bwd_rows failed: %d" % rc)
        return dq, dk, dv


def _sparse_shapes(q, k, v, idx, dout=None):
    for name, a in (("q", q), ("k", k), ("v", v), ("dout", dout)):
        if a is None:
            continue
        if a.dtype != np.uint16 or a.ndim != 4 or not a.flags.c_contiguous:
            raise ValueError("%s must be a C-contiguous uint16 array of bf16 bits" % name)
    if idx.dtype != np.int32 or idx.ndim != 3 or not idx.flags.c_contiguous:
        raise ValueError("idx must be a C-contiguous int32 [B][S][topk] array")
    B, Hq, S, D = q.shape
    Hkv, N = k.shape[1], k.shape[2]
    if k.shape != (B, Hkv, N, D) or v.shape != k.shape:
        raise ValueError("k and v must be [B][Hkv][N][D]")
    if idx.shape[:2] != (B, S):
        raise ValueError("idx must be [B][S][topk]")
    if dout is not None and dout.shape != q.shape:
        raise ValueError("dout must match q")
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    return B, Hq, Hkv, S, N, D, idx.shape[2]


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


def sparse_fwd(q, k, v, idx, scale, rows=None):
    return default().sparse_fwd(q, k, v, idx, scale, rows)


def sparse_bwd(q, k, v, dout, idx, scale, qrows=None, kvrows=None):
    return default().sparse_bwd(q, k, v, dout, idx, scale, qrows, kvrows)
