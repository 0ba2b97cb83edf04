"""The C ABI library loads, exports what include/attn.h declares, and rejects bad
arguments before touching the GPU (CPU only: no kernel is ever launched here)."""
import ctypes
import math
import os
import re

import pytest

import flashattention_tiled_attention_amd as fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn.h")

P = ctypes.c_void_p(0x10000)      # aligned, non-null, never dereferenced: validation fails first
MIS = ctypes.c_void_p(0x10002)    # misaligned


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_abi():
    assert declared_functions() == sorted(fa.EXPORTED_SYMBOLS)


def test_library_exports_every_declared_symbol():
    lib = fa.load_library()
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_lds_transpose_library_exports_its_header():
    from flashattention_tiled_attention_amd import lds_transpose
    text = open(os.path.join(ROOT, "include", "lds_transpose.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = sorted(set(re.findall(r"\b(lds_[a-z_0-9]+)\s*\(", text)))
    assert names == ["lds_transpose_bench"]
    lib = lds_transpose.load_library()
    for n in names:
        assert hasattr(lib, n), n
    # argument checks happen before any HIP call
    import ctypes
    ms = ctypes.c_float(0)
    assert lib.lds_transpose_bench(7, 1, 1, 1, ctypes.byref(ms), P, P, None) == 1
    assert lib.lds_transpose_bench(0, 0, 1, 1, ctypes.byref(ms), P, P, None) == 2
    assert lib.lds_transpose_bench(0, 1, 1, 1, ctypes.byref(ms), MIS, P, None) == 2


def test_mfma_rate_library_exports_its_header():
    from flashattention_tiled_attention_amd import mfma_rate
    text = open(os.path.join(ROOT, "include", "mfma_rate.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = sorted(set(re.findall(r"\b(mfma_[a-z_0-9]+)\s*\(", text)))
    assert names == ["mfma_rate_bench"]
    lib = mfma_rate.load_library()
    ms = ctypes.c_float(0)
    # argument checks happen before any HIP call
    assert lib.mfma_rate_bench(None, 1, 1, ctypes.byref(ms), P, P, None) == 2
    assert lib.mfma_rate_bench(P, 0, 1, ctypes.byref(ms), P, P, None) == 2
    assert lib.mfma_rate_bench(MIS, 1, 1, ctypes.byref(ms), P, P, None) == 2


def test_issue_rate_library_exports_its_header():
    from flashattention_tiled_attention_amd import issue_rate
    text = open(os.path.join(ROOT, "include", "issue_rate.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = sorted(set(re.findall(r"\b([a-z]+_issue_bench)\s*\(", text)))
    assert names == ["copy_issue_bench", "valu_issue_bench"]
    lib = issue_rate.load_library()
    for n in names:
        assert hasattr(lib, n), n
    # argument checks happen before any HIP call
    assert lib.valu_issue_bench(4, 1, 1, 0.5, P, P, None) == 2        # no such mode
    assert lib.valu_issue_bench(0, 0, 1, 0.5, P, P, None) == 2        # no workgroups
    assert lib.valu_issue_bench(0, 1, 1, 0.5, None, P, None) == 2
    assert lib.copy_issue_bench(P, 1, 9, 1, 1, P, P, None) == 2       # more than 8 copies
    assert lib.copy_issue_bench(P, 1, 1, 0, 1, P, P, None) == 2       # no issuing wave
    assert lib.copy_issue_bench(MIS, 1, 1, 1, 1, P, P, None) == 2     # misaligned source


def test_status_strings():
    for code in range(0, 13):
        s = fa.attn_status_str(code)
        assert isinstance(s, str) and s
    assert fa.attn_status_str(0) == "ok"
    assert "unknown" in fa.attn_status_str(1234)


def fwd(*, q=P, k=P, v=P, o=P, lse=P, B=1, Hq=4, Hkv=2, S=128, D=128, causal=1, scale=0.088):
    return fa.load_library().attn_fwd(q, k, v, o, lse, B, Hq, Hkv, S, D, causal, scale, None)


def bwd(*, ptrs=None, B=1, Hq=4, Hkv=2, S=128, D=128, causal=1, scale=0.088, ws=P, wsb=None):
    lib = fa.load_library()
    if wsb is None:
        wsb = lib.attn_bwd_workspace_bytes(B, Hq, Hkv, S, D)
    p = dict(q=P, k=P, v=P, o=P, lse=P, dout=P, dq=P, dk=P, dv=P)
    p.update(ptrs or {})
    return lib.attn_bwd(p["q"], p["k"], p["v"], p["o"], p["lse"], p["dout"], p["dq"], p["dk"], p["dv"],
                        B, Hq, Hkv, S, D, causal, scale, ws, wsb, None)


@pytest.mark.parametrize("name", ["q", "k", "v", "o", "lse"])
def test_fwd_null(name):
    assert fwd(**{name: None}) == fa.ATTN_ERR_NULL


@pytest.mark.parametrize("kw,code", [
    (dict(B=0), fa.ATTN_ERR_SHAPE), (dict(Hq=0), fa.ATTN_ERR_SHAPE), (dict(Hkv=0), fa.ATTN_ERR_SHAPE),
    (dict(S=0), fa.ATTN_ERR_SHAPE), (dict(S=-5), fa.ATTN_ERR_SHAPE), (dict(D=0), fa.ATTN_ERR_SHAPE),
    (dict(B=1 << 20, Hq=1 << 10, Hkv=1 << 10, S=1 << 12, D=128), fa.ATTN_ERR_SHAPE),
    # one head's rows must be addressable with 32-bit offsets: S * D < 2^31
    (dict(B=1, Hq=1, Hkv=1, S=1 << 24, D=128), fa.ATTN_ERR_SHAPE),
    (dict(B=1, Hq=1, Hkv=1, S=(1 << 25) + 1, D=64), fa.ATTN_ERR_SHAPE),
    # launch grids: 2*S + 512 forward work-items per query head, 8*S + 512 dK/dV
    # work-items per kv head, each total below 2^32
    (dict(B=1, Hq=1 << 10, Hkv=1 << 10, S=1 << 21, D=64), fa.ATTN_ERR_SHAPE),
    (dict(B=64, Hq=64, Hkv=64, S=1 << 17, D=64), fa.ATTN_ERR_SHAPE),
    (dict(Hq=6, Hkv=4), fa.ATTN_ERR_GQA), (dict(D=96), fa.ATTN_ERR_UNSUPPORTED_D),
    (dict(D=256), fa.ATTN_ERR_UNSUPPORTED_D), (dict(scale=math.nan), fa.ATTN_ERR_SCALE),
    (dict(scale=math.inf), fa.ATTN_ERR_SCALE), (dict(q=MIS), fa.ATTN_ERR_ALIGN),
    (dict(lse=MIS), fa.ATTN_ERR_ALIGN), (dict(o=MIS), fa.ATTN_ERR_ALIGN),
])
def test_fwd_rejects(kw, code):
    assert fwd(**kw) == code


@pytest.mark.parametrize("name", ["q", "k", "v", "o", "lse", "dout", "dq", "dk", "dv"])
def test_bwd_null(name):
    assert bwd(ptrs={name: None}) == fa.ATTN_ERR_NULL


@pytest.mark.parametrize("name", ["q", "dout", "dq", "dk", "dv"])
def test_bwd_misaligned(name):
    assert bwd(ptrs={name: MIS}) == fa.ATTN_ERR_ALIGN


def test_bwd_workspace():
    lib = fa.load_library()
    need = lib.attn_bwd_workspace_bytes(1, 4, 2, 128, 128)
    assert need >= 4 * 4 * 128
    assert bwd(ws=None) == fa.ATTN_ERR_WORKSPACE
    assert bwd(wsb=need - 1) == fa.ATTN_ERR_WORKSPACE
    assert bwd(ws=MIS) == fa.ATTN_ERR_ALIGN
    assert bwd(Hq=6, Hkv=4) == fa.ATTN_ERR_GQA
    assert bwd(D=80) == fa.ATTN_ERR_UNSUPPORTED_D
    assert bwd(scale=-math.inf) == fa.ATTN_ERR_SCALE
    assert lib.attn_bwd_workspace_bytes(0, 4, 2, 128, 128) == 0
    assert lib.attn_bwd_workspace_bytes(1, 4, 2, 128, 96) == 0


def fwd_window(*, window=128, q=P, B=1, Hq=4, Hkv=2, S=128, D=128, scale=0.088):
    return fa.load_library().attn_fwd_window(q, P, P, P, P, B, Hq, Hkv, S, D, window, scale, None)


def bwd_window(*, window=128, dq=P, B=1, Hq=4, Hkv=2, S=128, D=128, scale=0.088, wsb=None):
    lib = fa.load_library()
    if wsb is None:
        wsb = lib.attn_bwd_workspace_bytes(B, Hq, Hkv, S, D)
    return lib.attn_bwd_window(P, P, P, P, P, P, dq, P, P, B, Hq, Hkv, S, D, window, scale, P, wsb, None)


@pytest.mark.parametrize("window", [0, -1, -(1 << 30)])
def test_window_rejects_empty_window(window):
    assert fwd_window(window=window) == fa.ATTN_ERR_WINDOW
    assert bwd_window(window=window) == fa.ATTN_ERR_WINDOW


def test_window_validates_like_the_plain_entry_points():
    assert fwd_window(q=None) == fa.ATTN_ERR_NULL
    assert fwd_window(Hq=6, Hkv=4) == fa.ATTN_ERR_GQA
    assert fwd_window(D=96) == fa.ATTN_ERR_UNSUPPORTED_D
    assert fwd_window(scale=math.nan) == fa.ATTN_ERR_SCALE
    assert fwd_window(q=MIS) == fa.ATTN_ERR_ALIGN
    assert bwd_window(dq=None) == fa.ATTN_ERR_NULL
    assert bwd_window(dq=MIS) == fa.ATTN_ERR_ALIGN
    assert bwd_window(wsb=16) == fa.ATTN_ERR_WORKSPACE
    assert bwd_window(S=0) == fa.ATTN_ERR_SHAPE


def fwd_vdim(*, window=0, causal=1, o=P, B=1, Hq=4, Hkv=2, S=128, D=128, Dv=64, scale=0.088):
    return fa.load_library().attn_fwd_vdim(P, P, P, o, P, B, Hq, Hkv, S, D, Dv, causal, window, scale, None)


def bwd_vdim(*, window=0, causal=1, dv=P, B=1, Hq=4, Hkv=2, S=128, D=128, Dv=64, scale=0.088, wsb=None):
    lib = fa.load_library()
    if wsb is None:
        wsb = lib.attn_bwd_workspace_bytes(B, Hq, Hkv, S, D)
    return lib.attn_bwd_vdim(P, P, P, P, P, P, P, P, dv, B, Hq, Hkv, S, D, Dv, causal, window, scale, P, wsb,
                             None)


@pytest.mark.parametrize("kw,code", [
    (dict(Dv=96), fa.ATTN_ERR_UNSUPPORTED_D), (dict(Dv=256), fa.ATTN_ERR_UNSUPPORTED_D),
    (dict(D=192), fa.ATTN_ERR_UNSUPPORTED_D), (dict(Dv=0), fa.ATTN_ERR_SHAPE),
    (dict(window=-1), fa.ATTN_ERR_WINDOW), (dict(window=8, causal=0), fa.ATTN_ERR_WINDOW),
    (dict(Hq=6, Hkv=4), fa.ATTN_ERR_GQA), (dict(scale=math.nan), fa.ATTN_ERR_SCALE),
    # the size limit counts the wider of the two head dimensions
    (dict(B=1 << 19, Hq=1 << 10, Hkv=1 << 10, S=1 << 12, D=64, Dv=128), fa.ATTN_ERR_SHAPE),
    (dict(B=1, Hq=1, Hkv=1, S=1 << 24, D=64, Dv=128), fa.ATTN_ERR_SHAPE),
])
def test_vdim_rejects(kw, code):
    assert fwd_vdim(**kw) == code
    assert bwd_vdim(**kw) == code


def test_vdim_validates_pointers_and_workspace():
    assert fwd_vdim(o=None) == fa.ATTN_ERR_NULL
    assert fwd_vdim(o=MIS) == fa.ATTN_ERR_ALIGN
    assert bwd_vdim(dv=None) == fa.ATTN_ERR_NULL
    assert bwd_vdim(dv=MIS) == fa.ATTN_ERR_ALIGN
    assert bwd_vdim(wsb=16) == fa.ATTN_ERR_WORKSPACE


def sp_fwd(*, idx=P, B=1, Hq=8, Hkv=1, S=256, N=320, D=128, topk=64, scale=0.088):
    return fa.load_library().attn_sparse_fwd(P, P, P, idx, P, P, B, Hq, Hkv, S, N, D, topk, scale, None)


def sp_bwd(*, dk=P, B=1, Hq=8, Hkv=1, S=256, N=320, D=128, topk=64, scale=0.088, wsb=None, ws=P):
    lib = fa.load_library()
    if wsb is None:
        wsb = lib.attn_sparse_bwd_workspace_bytes(B, Hq, Hkv, S, N, D, topk)
    return lib.attn_sparse_bwd(P, P, P, P, P, P, P, P, dk, P, B, Hq, Hkv, S, N, D, topk, scale, ws, wsb, None)


@pytest.mark.parametrize("kw,code", [
    (dict(N=0), fa.ATTN_ERR_SHAPE), (dict(topk=0), fa.ATTN_ERR_SHAPE), (dict(S=0), fa.ATTN_ERR_SHAPE),
    (dict(D=96), fa.ATTN_ERR_UNSUPPORTED_D), (dict(Hq=6, Hkv=4), fa.ATTN_ERR_GQA),
    (dict(topk=4097), fa.ATTN_ERR_SPARSE), (dict(Hq=256, Hkv=1), fa.ATTN_ERR_SPARSE),
    (dict(N=1 << 24), fa.ATTN_ERR_SPARSE), (dict(S=1 << 20, topk=4096), fa.ATTN_ERR_SPARSE),
    # the reduction's grid: 256 work-items per key/value row must stay under 2^32
    (dict(Hkv=8, Hq=8, N=(1 << 21)), fa.ATTN_ERR_SPARSE), (dict(B=2, Hkv=4, Hq=8, N=(1 << 21)), fa.ATTN_ERR_SPARSE),
    (dict(scale=math.inf), fa.ATTN_ERR_SCALE),
])
def test_sparse_rejects(kw, code):
    assert sp_fwd(**kw) == code
    assert sp_bwd(**kw) == code


def test_grid_limits_at_the_boundary():
    """The largest sizes whose every launch fits a 32-bit grid of work-items pass
    validation (and then fail at the device step here, with no GPU); one more kv
    head or key/value row is rejected before anything is launched."""
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present: valid sizes would launch")
    ok = (fa.ATTN_ERR_HIP, fa.ATTN_ERR_DEVICE)
    # dK/dV grid: B*Hkv*(8*S + 512) work-items; S = 2^16 gives 2^19 + 512 per kv head
    per = 8 * (1 << 16) + 512
    top = ((1 << 32) - 1) // per
    assert fwd(B=1, Hq=top, Hkv=top, S=1 << 16, D=64) in ok
    assert fwd(B=1, Hq=top + 1, Hkv=top + 1, S=1 << 16, D=64) == fa.ATTN_ERR_SHAPE
    # sparse reduction grid: 256 work-items per key/value row, B*Hkv*N < 2^24
    assert sp_fwd(Hq=4, Hkv=4, N=(1 << 22) - 1) in ok
    assert sp_fwd(Hq=4, Hkv=4, N=1 << 22) == fa.ATTN_ERR_SPARSE


def test_sparse_validates_pointers_and_workspace():
    lib = fa.load_library()
    assert sp_fwd(idx=None) == fa.ATTN_ERR_NULL
    assert sp_fwd(idx=MIS) == fa.ATTN_ERR_ALIGN
    assert sp_bwd(dk=None) == fa.ATTN_ERR_NULL
    assert sp_bwd(dk=MIS) == fa.ATTN_ERR_ALIGN
    need = lib.attn_sparse_bwd_workspace_bytes(1, 8, 1, 256, 320, 128, 64)
    # delta, two contribution arrays of S*topk*D fp32, the inverse map
    assert need >= 8 * 256 * 4 + 2 * 256 * 64 * 128 * 4 + 256 * 64 * 4
    assert sp_bwd(wsb=need - 1) == fa.ATTN_ERR_WORKSPACE
    assert sp_bwd(ws=None) == fa.ATTN_ERR_WORKSPACE
    assert lib.attn_sparse_bwd_workspace_bytes(1, 8, 1, 256, 320, 128, 0) == 0


def bwd_noalloc(*, ptrs=None, B=1, Hq=4, Hkv=2, S=128, D=128, causal=1, scale=0.088):
    p = dict(q=P, k=P, v=P, o=P, lse=P, dout=P, dq=P, dk=P, dv=P)
    p.update(ptrs or {})
    return fa.load_library().attn_bwd_noalloc(p["q"], p["k"], p["v"], p["o"], p["lse"], p["dout"], p["dq"],
                                              p["dk"], p["dv"], B, Hq, Hkv, S, D, causal, scale, None)


def test_noalloc_validates_before_any_call():
    """attn_bwd_noalloc checks its arguments like attn_bwd, and rejects sizes whose
    workspace exceeds its static scratch, before touching the GPU."""
    lib = fa.load_library()
    limit = lib.attn_bwd_noalloc_max_workspace_bytes()
    assert limit == 16 << 20
    assert bwd_noalloc(ptrs={"dq": None}) == fa.ATTN_ERR_NULL
    assert bwd_noalloc(ptrs={"dv": MIS}) == fa.ATTN_ERR_ALIGN
    assert bwd_noalloc(Hq=6, Hkv=4) == fa.ATTN_ERR_GQA
    assert bwd_noalloc(D=96) == fa.ATTN_ERR_UNSUPPORTED_D
    assert bwd_noalloc(scale=math.nan) == fa.ATTN_ERR_SCALE
    # two million query rows fit; 2^21 + 32 per head over four heads do not
    assert lib.attn_bwd_workspace_bytes(1, 32, 8, 62500, 128) <= limit
    assert lib.attn_bwd_workspace_bytes(1, 4, 1, (1 << 19) + 32, 128) > limit
    assert bwd_noalloc(B=1, Hq=4, Hkv=1, S=(1 << 19) + 32) == fa.ATTN_ERR_SCRATCH
    assert "scratch" in fa.attn_status_str(fa.ATTN_ERR_SCRATCH)


def test_no_gpu_reports_hip_error():
    """Valid arguments on a machine without a usable gfx950 device end in a HIP or device
    error from the set-up step, never in a launch."""
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    assert fwd() in (fa.ATTN_ERR_HIP, fa.ATTN_ERR_DEVICE)
    assert fwd_window() in (fa.ATTN_ERR_HIP, fa.ATTN_ERR_DEVICE)
    assert fwd_vdim() in (fa.ATTN_ERR_HIP, fa.ATTN_ERR_DEVICE)
    assert fwd_vdim(D=64, Dv=128, window=16) in (fa.ATTN_ERR_HIP, fa.ATTN_ERR_DEVICE)
    assert sp_fwd() in (fa.ATTN_ERR_HIP, fa.ATTN_ERR_DEVICE)
    assert bwd_noalloc(B=1, Hq=32, Hkv=8, S=62500) in (fa.ATTN_ERR_HIP, fa.ATTN_ERR_DEVICE)
