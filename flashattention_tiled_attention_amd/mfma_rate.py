"""Runner for the gfx950 matrix-core rate microbenchmark (libmfma_rate.so, declared in
include/mfma_rate.h): the chip's rate of v_mfma_f32_32x32x16_bf16 with operands in
registers, and the shader clock it runs at, for a given set of operand values.

Device memory comes from torch; the products and the timing run in the library's
own kernel.
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmfma_rate.so")
THREADS = 256
MFMA_PER_ITER = 8
FLOP_PER_MFMA = 2 * 32 * 32 * 16
CUS = 256
PEAK_BF16_TFLOPS = 2516.6   # 256 CU x 4096 dense bf16 flop/clk x 2.4 GHz
REALTIME_HZ = 100e6         # s_memrealtime ticks
_lib = None


def load_library(path=None):
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError("libmfma_rate.so not found at %s: run flashattention_tiled_attention_amd/build.py" % p)
    lib = ctypes.CDLL(p)
    lib.mfma_rate_bench.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.POINTER(ctypes.c_float),
                                    ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    lib.mfma_rate_bench.restype = ctypes.c_int
    if path is None:
        _lib = lib
    return lib


def operand_bits(kind, seed=0):
    """The 16 x 64 bf16x8 operands as uint16 bits [16][64][8]: 'random' (N(0,1) rounded
    to bf16, the attention inputs' distribution), 'zero', or 'ones'."""
    from flashattention_tiled_attention_amd.inputs import bf16_bits
    shape = (16, 64, 8)
    if kind == "random":
        x = np.random.default_rng(seed).standard_normal(shape, dtype=np.float32)
    elif kind == "zero":
        x = np.zeros(shape, np.float32)
    elif kind == "ones":
        x = np.ones(shape, np.float32)
    else:
        raise ValueError(kind)
    return bf16_bits(x)


def run(kind="random", waves_per_simd=2, iters=20000, seed=0):
    """One timed launch; returns a dict with TFLOP/s, its fraction of the 2.4 GHz spec
    peak, the mean shader clock of the workgroups' loops and the raw per-thread sums."""
    import torch
    bits = operand_bits(kind, seed)
    ops = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to("cuda")
    blocks = CUS * waves_per_simd
    sink = torch.zeros(blocks * THREADS, dtype=torch.float32, device="cuda")
    stamps = torch.zeros(4 * blocks, dtype=torch.int64, device="cuda")
    ms = ctypes.c_float(0.0)
    rc = load_library().mfma_rate_bench(ctypes.c_void_p(ops.data_ptr()), int(blocks), int(iters), ctypes.byref(ms),
                                        ctypes.c_void_p(sink.data_ptr()), ctypes.c_void_p(stamps.data_ptr()),
                                        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    if rc:
        raise RuntimeError("mfma_rate_bench failed with %d" % rc)
    st = stamps.cpu().numpy().view(np.uint64).reshape(blocks, 4).astype(np.float64)
    cycles, ticks = st[:, 1] - st[:, 0], st[:, 3] - st[:, 2]
    clock = float(np.mean(cycles / (ticks / REALTIME_HZ))) / 1e9
    flop = float(blocks) * 4 * iters * MFMA_PER_ITER * FLOP_PER_MFMA
    tflops = flop / (ms.value * 1e-3) / 1e12
    return {"operands": kind, "waves_per_simd": waves_per_simd, "iters": iters, "ms": round(ms.value, 3),
            "tflops": round(tflops, 1), "frac_of_peak": round(tflops / PEAK_BF16_TFLOPS, 4),
            "shader_clock_ghz": round(clock, 3),
            "tflops_at_measured_clock_peak": round(4096 * CUS * clock * 1e9 / 1e12, 1),
            "sink": sink.cpu().numpy()}


def table(iters=20000):
    """Random and zero operands at one and two waves per SIMD (JSON-ready rows)."""
    rows = []
    for kind in ("random", "zero"):
        for wps in (1, 2):
            r = run(kind, wps, iters)
            r.pop("sink")
            rows.append(r)
    return rows
