"""Runner for the gfx950 instruction-issue microbenchmark (libissue_rate.so, declared
in include/issue_rate.h): the vector-unit issue interval of v_fma_f32 and v_exp_f32
per wave, and the time a wave spends issuing global_load_lds_dwordx4 tile copies.

Device memory comes from torch; the timing runs in the library's own kernels.
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libissue_rate.so")
CUS = 256
MODES = {"fma_independent": 0, "exp_independent": 1, "fma_dependent": 2, "exp_dependent": 3}
_lib = None


def load_library(path=None):
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError("libissue_rate.so not found at %s: run flashattention_tiled_attention_amd/build.py" % p)
    lib = ctypes.CDLL(p)
    V, I, F = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    lib.valu_issue_bench.argtypes = [I, I, I, F, V, V, V]
    lib.valu_issue_bench.restype = I
    lib.copy_issue_bench.argtypes = [V, I, I, I, I, V, V, V]
    lib.copy_issue_bench.restype = I
    if path is None:
        _lib = lib
    return lib


def valu(mode, waves_per_simd=1, iters=20000, a=0.5):
    """Cycles per instruction per wave (mean over waves) and each thread's chain sum."""
    import torch
    blocks = CUS * waves_per_simd
    sink = torch.zeros(blocks * 256, dtype=torch.float32, device="cuda")
    cyc = torch.zeros(blocks * 4, dtype=torch.int64, device="cuda")
    rc = load_library().valu_issue_bench(MODES[mode], blocks, iters, a, ctypes.c_void_p(sink.data_ptr()),
                                         ctypes.c_void_p(cyc.data_ptr()),
                                         ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    if rc:
        raise RuntimeError("valu_issue_bench failed with %d" % rc)
    c = cyc.cpu().numpy().astype(np.float64)
    return {"mode": mode, "waves_per_simd": waves_per_simd, "iters": iters,
            "cycles_per_instr_per_wave": round(float(c.mean()) / (iters * 8), 2),
            "cycles_per_instr_per_simd": round(float(c.mean()) / (iters * 8) / waves_per_simd, 2),
            "sink": sink.cpu().numpy()}


def copies(copies_per_wave, active_waves, iters=2000, blocks=CUS, seed=0):
    """Mean cycles per active wave to issue its copies, and until they have landed;
    with the source and what the copies wrote back, for checking."""
    import torch
    rng = np.random.default_rng(seed)
    nbytes = blocks * 65536
    src = torch.from_numpy(rng.integers(0, 256, nbytes, dtype=np.uint8)).to("cuda")
    dst = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    cyc = torch.zeros(blocks * 16, dtype=torch.int64, device="cuda")
    rc = load_library().copy_issue_bench(ctypes.c_void_p(src.data_ptr()), blocks, copies_per_wave, active_waves,
                                         iters, ctypes.c_void_p(cyc.data_ptr()), ctypes.c_void_p(dst.data_ptr()),
                                         ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    if rc:
        raise RuntimeError("copy_issue_bench failed with %d" % rc)
    c = cyc.cpu().numpy().astype(np.float64).reshape(blocks, 8, 2)[:, :active_waves, :]
    issue = float(c[..., 0].mean()) / iters
    land = float(c[..., 1].mean()) / iters
    return {"copies_per_wave": copies_per_wave, "active_waves": active_waves, "iters": iters,
            "issue_cycles": round(issue, 1), "issue_cycles_per_copy": round(issue / copies_per_wave, 1),
            "issue_to_landed_cycles": round(land, 1),
            "src": src.cpu().numpy(), "dst": dst.cpu().numpy()}


def table():
    """JSON-ready rows: vector issue at 1, 2 and 4 waves per SIMD; copy issue for 4
    copies per wave at 1, 4 and 8 issuing waves, and 8 copies at 4 and 8."""
    rows = []
    for mode in MODES:
        for wps in (1, 2, 4):
            r = valu(mode, wps)
            r.pop("sink")
            rows.append(r)
    for n, act in ((4, 1), (4, 4), (4, 8), (8, 4), (8, 8), (1, 8)):
        r = copies(n, act)
        r.pop("src")
        r.pop("dst")
        rows.append(r)
    return rows
