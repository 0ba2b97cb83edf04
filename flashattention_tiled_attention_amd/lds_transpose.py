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


def expected_operand(method, pos=0):
    """Words each of the 64 lanes of a wave should hold after its load at position `pos`
    (0..7), as [64][4] uint32. The tile element (r, c) holds the 16-bit pattern 64 r + c.
    Method 0 reads rows 32 (pos & 1) + lane % 32 at 8-column chunk 2 ((pos >> 1) & 3) +
    lane / 32; the transposing methods read the 16 x 32 block at rows 16 (pos & 3),
    columns 32 ((pos >> 2) & 1), element e of lane (c, h) from row 8 (e / 4) + 4 h + e % 4."""
    out = np.zeros((64, 4), np.uint32)
    for lane in range(64):
        h, c = lane >> 5, lane & 31
        if method == 0:
            row, col = 32 * (pos & 1) + c, 16 * ((pos >> 1) & 3) + 8 * h
            elems = [64 * row + col + e for e in range(8)]
        else:
            r0, c0 = 16 * (pos & 3), 32 * ((pos >> 2) & 1)
            elems = [64 * (r0 + 8 * (e >> 2) + 4 * h + (e & 3)) + c0 + c for e in range(8)]
        for k in range(4):
            out[lane, k] = elems[2 * k] | (elems[2 * k + 1] << 16)
    return out


def expected_checksum(method, iters):
    """Each thread's XOR of every word it loaded, [64] uint32 by lane: the eight operands
    of one iteration XOR-ed together, once for odd `iters` and cancelled for even."""
    x = np.zeros(64, np.uint32)
    if iters % 2:
        for p in range(LOADS_PER_ITER):
            w = expected_operand(method, p)
            x ^= w[:, 0] ^ w[:, 1] ^ w[:, 2] ^ w[:, 3]
    return x


def run(method, blocks=1024, iters=2000, reps=3):
    """Time one method; returns (milliseconds, operands [8][64][4] uint32 by position and
    lane, bytes loaded, per-thread checksums [blocks * 256] uint32)."""
    import torch
    operand = torch.zeros(LOADS_PER_ITER * 256, dtype=torch.int32, device="cuda")
    checksum = torch.zeros(blocks * THREADS, dtype=torch.int32, device="cuda")
    ms = ctypes.c_float(0.0)
    stream = torch.cuda.current_stream().cuda_stream
    rc = load_library().lds_transpose_bench(int(method), int(blocks), int(iters), int(reps), ctypes.byref(ms),
                                            ctypes.c_void_p(operand.data_ptr()),
                                            ctypes.c_void_p(checksum.data_ptr()), ctypes.c_void_p(stream))
    if rc:
        raise RuntimeError("lds_transpose_bench(method=%d) failed with %d" % (method, rc))
    words = operand.cpu().numpy().view(np.uint32).reshape(LOADS_PER_ITER, 64, 4)
    nbytes = float(blocks) * THREADS * iters * LOADS_PER_ITER * OPERAND_BYTES_PER_LANE
    return ms.value, words, nbytes, checksum.cpu().numpy().view(np.uint32)


def table(blocks=1024, iters=2000, reps=3):
    """All four methods: GB/s and bandwidth normalised to method 0, plus whether each
    delivered the operand it should."""
    rows = []
    for m in range(4):
        ms, words, nbytes, _ = run(m, blocks, iters, reps)
        ok = all(np.array_equal(words[p], expected_operand(m, p)) for p in range(LOADS_PER_ITER))
        rows.append({"method": METHODS[m], "ms": round(ms, 4), "GB/s": round(nbytes / (ms * 1e-3) / 1e9, 1),
                     "operand_ok": bool(ok)})
    base = rows[0]["GB/s"]
    for r in rows:
        r["normalized"] = round(r["GB/s"] / base, 3)
    return rows
