"""Runner for the gfx950 LDS-to-register transpose microbenchmark (liblds_transpose.so,
declared in include/lds_transpose.h).

It repeats on MI355X the comparison of Rao et al., "Scheduling Data to Compute:
Hierarchical Data Pipelining for LLM Training on AMD GPUs", section 4.3.2, Table 10:
the bandwidth at which each way of bringing a transposed matrix operand from LDS into
registers runs, normalised to a plain 16-byte row load of an operand that needs no
transpose. Device memory comes from torch; the timing and the loads run in the
library's own kernels.
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liblds_transpose.so")
METHODS = ("ds_read_b128 (no transpose)", "ds_read_b64_tr_b16", "8 x 16-bit strided loads",
           "ds_read_b128 + XOR lane shuffle")
OPERAND_BYTES_PER_LANE = 16
LOADS_PER_ITER = 8
THREADS = 256
_lib = None


def load_library(path=None):
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError("liblds_transpose.so not found at %s: run flashattention_tiled_attention_amd/build.py" % p)
    lib = ctypes.CDLL(p)
    lib.lds_transpose_bench.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                        ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p,
                                        ctypes.c_void_p]
    lib.lds_transpose_bench.restype = ctypes.c_int
    if path is None:
        _lib = lib
    return lib


def expected_operand(method):
    """Words each of the 64 lanes of a wave should hold after its first load (position 0:
    tile rows 0..15, columns 0..31), as [64][4] uint32. The tile element (r, c) holds the
    16-bit pattern 64 r + c."""
    out = np.zeros((64, 4), np.uint32)
    for lane in range(64):
        h, c = lane >> 5, lane & 31
        if method == 0:
            row, col = c, 8 * h
            elems = [64 * row + col + e for e in range(8)]
        else:
            elems = [64 * (8 * (e >> 2) + 4 * h + (e & 3)) + c for e in range(8)]
        for k in range(4):
            out[lane, k] = elems[2 * k] | (elems[2 * k + 1] << 16)
    return out


def run(method, blocks=1024, iters=2000, reps=3):
    """Time one method; returns (milliseconds, operand [64][4] uint32, bytes loaded)."""
    import torch
    operand = torch.zeros(256, dtype=torch.int32, device="cuda")
    checksum = torch.zeros(blocks * THREADS, dtype=torch.int32, device="cuda")
    ms = ctypes.c_float(0.0)
    stream = torch.cuda.current_stream().cuda_stream
    rc = load_library().lds_transpose_bench(int(method), int(blocks), int(iters), int(reps), ctypes.byref(ms),
                                            ctypes.c_void_p(operand.data_ptr()),
                                            ctypes.c_void_p(checksum.data_ptr()), ctypes.c_void_p(stream))
    if rc:
        raise RuntimeError("lds_transpose_bench(method=%d) failed with %d" % (method, rc))
    words = operand.cpu().numpy().view(np.uint32).reshape(64, 4)
    nbytes = float(blocks) * THREADS * iters * LOADS_PER_ITER * OPERAND_BYTES_PER_LANE
    return ms.value, words, nbytes


def table(blocks=1024, iters=2000, reps=3):
    """All four methods: GB/s and bandwidth normalised to method 0, plus whether each
    delivered the operand it should."""
    rows = []
    for m in range(4):
        ms, words, nbytes = run(m, blocks, iters, reps)
        rows.append({"method": METHODS[m], "ms": round(ms, 4), "GB/s": round(nbytes / (ms * 1e-3) / 1e9, 1),
                     "operand_ok": bool(np.array_equal(words, expected_operand(m)))})
    base = rows[0]["GB/s"]
    for r in rows:
        r["normalized"] = round(r["GB/s"] / base, 3)
    return rows
