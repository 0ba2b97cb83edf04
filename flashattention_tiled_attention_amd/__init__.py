"""MI355X (gfx950) fused attention: thin Python binding over the C ABI in include/attn.h.

The binding only marshals arguments: torch tensors are used for device memory
and streams, their data pointers and the current HIP stream go to the C entry
points, and every step of the computation runs in the library's HIP kernels.
There is no fallback: if ``libattn.so`` is missing, every call raises.

Entry points with the C names (``attn_fwd``, ``attn_bwd``, ``attn_bwd_dq``,
``attn_bwd_dkdv``, ``attn_fwd_window``, ``attn_bwd_window``, ``attn_fwd_vdim``,
``attn_bwd_vdim``, ``attn_bwd_workspace_bytes``, ``attn_sparse_fwd``, ``attn_sparse_bwd``,
``attn_sparse_bwd_workspace_bytes``, ``attn_status_str``) take caller-allocated tensors;
``fwd``, ``bwd``, ``sparse_fwd`` and ``sparse_bwd`` allocate their outputs with torch.
"""
import ctypes
import math
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libattn.so")
_lib = None

# attn_status codes (include/attn.h)
ATTN_OK = 0
ATTN_ERR_NULL = 1
ATTN_ERR_SHAPE = 2
ATTN_ERR_GQA = 3
ATTN_ERR_UNSUPPORTED_D = 4
ATTN_ERR_ALIGN = 5
ATTN_ERR_WORKSPACE = 6
ATTN_ERR_SCALE = 7
ATTN_ERR_HIP = 8
ATTN_ERR_DEVICE = 9
ATTN_ERR_WINDOW = 10
ATTN_ERR_SPARSE = 11
ATTN_ERR_SCRATCH = 12

EXPORTED_SYMBOLS = ("attn_fwd", "attn_bwd", "attn_bwd_dq", "attn_bwd_dkdv", "attn_fwd_window",
                    "attn_bwd_window", "attn_fwd_vdim", "attn_bwd_vdim", "attn_bwd_workspace_bytes",
                    "attn_sparse_fwd", "attn_sparse_bwd", "attn_sparse_bwd_workspace_bytes", "attn_status_str",
                    "attn_bwd_noalloc", "attn_bwd_noalloc_max_workspace_bytes")


class AttnError(RuntimeError):
    def __init__(self, code, where):
        self.code = code
        super().__init__("%s: %s (status %d)" % (where, attn_status_str(code), code))


def load_library(path=None):
    """Load libattn.so (built by ``flashattention_tiled_attention_amd.build``)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError("libattn.so not found at %s: run flashattention_tiled_attention_amd/build.py "
                           "(or __graft_entry__.build()) first" % p)
    lib = ctypes.CDLL(p)
    V = ctypes.c_void_p
    I = ctypes.c_int
    F = ctypes.c_float
    Z = ctypes.c_size_t
    lib.attn_fwd.argtypes = [V, V, V, V, V, I, I, I, I, I, I, F, V]
    lib.attn_fwd.restype = I
    for f in (lib.attn_bwd, lib.attn_bwd_dq, lib.attn_bwd_dkdv):
        f.argtypes = [V, V, V, V, V, V, V, V, V, I, I, I, I, I, I, F, V, Z, V]
        f.restype = I
    lib.attn_fwd_window.argtypes = [V, V, V, V, V, I, I, I, I, I, I, F, V]
    lib.attn_fwd_window.restype = I
    lib.attn_bwd_window.argtypes = [V, V, V, V, V, V, V, V, V, I, I, I, I, I, I, F, V, Z, V]
    lib.attn_bwd_window.restype = I
    lib.attn_fwd_vdim.argtypes = [V, V, V, V, V, I, I, I, I, I, I, I, I, F, V]
    lib.attn_fwd_vdim.restype = I
    lib.attn_bwd_vdim.argtypes = [V, V, V, V, V, V, V, V, V, I, I, I, I, I, I, I, I, F, V, Z, V]
    lib.attn_bwd_vdim.restype = I
    lib.attn_sparse_fwd.argtypes = [V, V, V, V, V, V, I, I, I, I, I, I, I, F, V]
    lib.attn_sparse_fwd.restype = I
    lib.attn_sparse_bwd.argtypes = [V, V, V, V, V, V, V, V, V, V, I, I, I, I, I, I, I, F, V, Z, V]
    lib.attn_sparse_bwd.restype = I
    lib.attn_sparse_bwd_workspace_bytes.argtypes = [I, I, I, I, I, I, I]
    lib.attn_sparse_bwd_workspace_bytes.restype = Z
    lib.attn_bwd_workspace_bytes.argtypes = [I, I, I, I, I]
    lib.attn_bwd_workspace_bytes.restype = Z
    lib.attn_bwd_noalloc.argtypes = [V, V, V, V, V, V, V, V, V, I, I, I, I, I, I, F, V]
    lib.attn_bwd_noalloc.restype = I
    lib.attn_bwd_noalloc_max_workspace_bytes.argtypes = []
    lib.attn_bwd_noalloc_max_workspace_bytes.restype = Z
    lib.attn_status_str.argtypes = [I]
    lib.attn_status_str.restype = ctypes.c_char_p
    if path is None:
        _lib = lib
    return lib


def attn_status_str(code):
    return load_library().attn_status_str(int(code)).decode()


def _stream(stream):
    import torch
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, int):
        return ctypes.c_void_p(stream)
    return ctypes.c_void_p(stream.cuda_stream)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _check(t, name, dtype, shape):
    import torch
    if t is None:
        return
    if t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if t.device.type != "cuda":
        raise TypeError("%s must be a GPU tensor" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s must have shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))


def _dims(q, k, v=None):
    """(B, Hq, Hkv, S, D, Dv): D from q, Dv (the value head dimension) from v."""
    if q.dim() != 4 or k.dim() != 4 or (v is not None and v.dim() != 4):
        raise ValueError("q, k and v must be [B][H][S][D]")
    B, Hq, S, D = q.shape
    return B, Hq, k.shape[1], S, D, (D if v is None else v.shape[3])


def _fwd_call(name, q, k, v, o, lse, flags, scale, stream, vdim=False):
    """flags: the int arguments between the sizes and scale (causal or window; for
    the vdim entry point, causal and window after Dv)."""
    import torch
    B, Hq, Hkv, S, D, Dv = _dims(q, k, v if vdim else None)
    _check(q, "q", torch.bfloat16, (B, Hq, S, D))
    _check(k, "k", torch.bfloat16, (B, Hkv, S, D))
    _check(v, "v", torch.bfloat16, (B, Hkv, S, Dv))
    _check(o, "o", torch.bfloat16, (B, Hq, S, Dv))
    _check(lse, "lse", torch.float32, (B, Hq, S))
    dims = (B, Hq, Hkv, S, D, Dv) if vdim else (B, Hq, Hkv, S, D)
    rc = getattr(load_library(), name)(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), *dims,
                                       *[int(f) for f in flags], float(scale), _stream(stream))
    if rc:
        raise AttnError(rc, name)


def attn_fwd(q, k, v, o, lse, causal, scale, stream=None):
    """C attn_fwd on torch tensors: q [B,Hq,S,D], k/v [B,Hkv,S,D] bf16; writes o (bf16) and lse (fp32)."""
    _fwd_call("attn_fwd", q, k, v, o, lse, (bool(causal),), scale, stream)


def attn_fwd_window(q, k, v, o, lse, window, scale, stream=None):
    """C attn_fwd_window: causal attention where query i sees keys i-window+1 .. i."""
    _fwd_call("attn_fwd_window", q, k, v, o, lse, (window,), scale, stream)


def attn_fwd_vdim(q, k, v, o, lse, causal, window, scale, stream=None):
    """C attn_fwd_vdim: v [B,Hkv,S,Dv] and o [B,Hq,S,Dv] with their own head dimension
    Dv; window = 0 (none) or >= 1 with causal."""
    _fwd_call("attn_fwd_vdim", q, k, v, o, lse, (bool(causal), window), scale, stream, vdim=True)


def attn_bwd_workspace_bytes(B, Hq, Hkv, S, D):
    return int(load_library().attn_bwd_workspace_bytes(B, Hq, Hkv, S, D))


def _bwd_call(name, q, k, v, o, lse, dout, dq, dk, dv, flags, scale, workspace, stream, vdim=False):
    import torch
    B, Hq, Hkv, S, D, Dv = _dims(q, k, v if vdim else None)
    for t, n, dt, sh in ((q, "q", torch.bfloat16, (B, Hq, S, D)), (k, "k", torch.bfloat16, (B, Hkv, S, D)),
                         (v, "v", torch.bfloat16, (B, Hkv, S, Dv)), (o, "o", torch.bfloat16, (B, Hq, S, Dv)),
                         (lse, "lse", torch.float32, (B, Hq, S)), (dout, "dout", torch.bfloat16, (B, Hq, S, Dv)),
                         (dq, "dq", torch.float32, (B, Hq, S, D)), (dk, "dk", torch.float32, (B, Hkv, S, D)),
                         (dv, "dv", torch.float32, (B, Hkv, S, Dv))):
        _check(t, n, dt, sh)
    if workspace.device.type != "cuda":
        raise TypeError("workspace must be a GPU tensor")
    nbytes = workspace.numel() * workspace.element_size()
    dims = (B, Hq, Hkv, S, D, Dv) if vdim else (B, Hq, Hkv, S, D)
    rc = getattr(load_library(), name)(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout), _ptr(dq),
                                       _ptr(dk), _ptr(dv), *dims, *[int(f) for f in flags], float(scale),
                                       _ptr(workspace), nbytes, _stream(stream))
    if rc:
        raise AttnError(rc, name)


def attn_bwd(q, k, v, o, lse, dout, dq, dk, dv, causal, scale, workspace, stream=None):
    """C attn_bwd on torch tensors; dq/dk/dv are fp32; workspace is a uint8 GPU tensor."""
    _bwd_call("attn_bwd", q, k, v, o, lse, dout, dq, dk, dv, (bool(causal),), scale, workspace, stream)


def attn_bwd_noalloc(q, k, v, o, lse, dout, dq, dk, dv, causal, scale, stream=None):
    """C attn_bwd_noalloc: attn_bwd with the library's static per-GPU scratch as its
    workspace (nothing is allocated); calls that overlap on one GPU race."""
    import torch
    B, Hq, Hkv, S, D, Dv = _dims(q, k)
    for t, n, dt, sh in ((q, "q", torch.bfloat16, (B, Hq, S, D)), (k, "k", torch.bfloat16, (B, Hkv, S, D)),
                         (v, "v", torch.bfloat16, (B, Hkv, S, D)), (o, "o", torch.bfloat16, (B, Hq, S, D)),
                         (lse, "lse", torch.float32, (B, Hq, S)), (dout, "dout", torch.bfloat16, (B, Hq, S, D)),
                         (dq, "dq", torch.float32, (B, Hq, S, D)), (dk, "dk", torch.float32, (B, Hkv, S, D)),
                         (dv, "dv", torch.float32, (B, Hkv, S, D))):
        _check(t, n, dt, sh)
    rc = load_library().attn_bwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout), _ptr(dq),
                                         _ptr(dk), _ptr(dv), B, Hq, Hkv, S, D, int(bool(causal)), float(scale),
                                         _stream(stream))
    if rc:
        raise AttnError(rc, "attn_bwd_noalloc")


def attn_bwd_noalloc_max_workspace_bytes():
    return int(load_library().attn_bwd_noalloc_max_workspace_bytes())


def attn_bwd_dq(q, k, v, o, lse, dout, dq, dk, dv, causal, scale, workspace, stream=None):
    """First backward stage: delta into the workspace and dq."""
    _bwd_call("attn_bwd_dq", q, k, v, o, lse, dout, dq, dk, dv, (bool(causal),), scale, workspace, stream)


def attn_bwd_dkdv(q, k, v, o, lse, dout, dq, dk, dv, causal, scale, workspace, stream=None):
    """Second backward stage: dk and dv from the workspace's delta."""
    _bwd_call("attn_bwd_dkdv", q, k, v, o, lse, dout, dq, dk, dv, (bool(causal),), scale, workspace, stream)


def attn_bwd_window(q, k, v, o, lse, dout, dq, dk, dv, window, scale, workspace, stream=None):
    """C attn_bwd_window: gradient of attn_fwd_window with the same window."""
    _bwd_call("attn_bwd_window", q, k, v, o, lse, dout, dq, dk, dv, (window,), scale, workspace, stream)


def attn_bwd_vdim(q, k, v, o, lse, dout, dq, dk, dv, causal, window, scale, workspace, stream=None):
    """C attn_bwd_vdim: gradient of attn_fwd_vdim with the same arguments; v, o, dout
    and dv have the value head dimension Dv."""
    _bwd_call("attn_bwd_vdim", q, k, v, o, lse, dout, dq, dk, dv, (bool(causal), window), scale, workspace,
              stream, vdim=True)


def fwd(q, k, v, causal=False, scale=None, window=0):
    """Allocate o and lse and run attn_fwd (attn_fwd_window when window > 0, which
    implies causal; attn_fwd_vdim when v's head dimension differs from q's).
    scale defaults to 1/sqrt(D)."""
    import torch
    B, Hq, Hkv, S, D, Dv = _dims(q, k, v)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    o = torch.empty((B, Hq, S, Dv), dtype=torch.bfloat16, device=q.device)
    lse = torch.empty((B, Hq, S), dtype=torch.float32, device=q.device)
    if Dv != D:
        attn_fwd_vdim(q, k, v, o, lse, causal or bool(window), window, scale)
    elif window:
        attn_fwd_window(q, k, v, o, lse, window, scale)
    else:
        attn_fwd(q, k, v, o, lse, causal, scale)
    return o, lse


def bwd(q, k, v, o, lse, dout, causal=False, scale=None, window=0):
    """Allocate dq/dk/dv (fp32) and the workspace and run attn_bwd (attn_bwd_window
    when window > 0; attn_bwd_vdim when v's head dimension differs from q's)."""
    import torch
    B, Hq, Hkv, S, D, Dv = _dims(q, k, v)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    dq = torch.empty((B, Hq, S, D), dtype=torch.float32, device=q.device)
    dk = torch.empty((B, Hkv, S, D), dtype=torch.float32, device=q.device)
    dv = torch.empty((B, Hkv, S, Dv), dtype=torch.float32, device=q.device)
    ws = torch.empty((attn_bwd_workspace_bytes(B, Hq, Hkv, S, D),),
                     dtype=torch.uint8, device=q.device)
    if Dv != D:
        attn_bwd_vdim(q, k, v, o, lse, dout, dq, dk, dv, causal or bool(window), window, scale, ws)
    elif window:
        attn_bwd_window(q, k, v, o, lse, dout, dq, dk, dv, window, scale, ws)
    else:
        attn_bwd(q, k, v, o, lse, dout, dq, dk, dv, causal, scale, ws)
    return dq, dk, dv


# ------------------------------------------------------------------ sparse attention

def _sparse_dims(q, k, idx):
    if q.dim() != 4 or k.dim() != 4 or idx.dim() != 3:
        raise ValueError("q, k must be [B][H][rows][D] and idx [B][S][topk]")
    B, Hq, S, D = q.shape
    return B, Hq, k.shape[1], S, k.shape[2], D, idx.shape[2]


def _sparse_check(q, k, v, idx, tensors):
    import torch
    B, Hq, Hkv, S, N, D, topk = _sparse_dims(q, k, idx)
    _check(q, "q", torch.bfloat16, (B, Hq, S, D))
    _check(k, "k", torch.bfloat16, (B, Hkv, N, D))
    _check(v, "v", torch.bfloat16, (B, Hkv, N, D))
    _check(idx, "idx", torch.int32, (B, S, topk))
    shapes = {"o": ((B, Hq, S, D), torch.bfloat16), "lse": ((B, Hq, S), torch.float32),
              "dout": ((B, Hq, S, D), torch.bfloat16), "dq": ((B, Hq, S, D), torch.float32),
              "dk": ((B, Hkv, N, D), torch.float32), "dv": ((B, Hkv, N, D), torch.float32)}
    for name, t in tensors.items():
        _check(t, name, shapes[name][1], shapes[name][0])
    return B, Hq, Hkv, S, N, D, topk


def attn_sparse_fwd(q, k, v, idx, o, lse, scale, stream=None):
    """C attn_sparse_fwd: q [B,Hq,S,D], k/v [B,Hkv,N,D] bf16, idx [B,S,topk] int32 (entries
    outside [0, N) are empty slots); writes o (bf16) and lse (fp32)."""
    dims = _sparse_check(q, k, v, idx, {"o": o, "lse": lse})
    rc = load_library().attn_sparse_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(idx), _ptr(o), _ptr(lse), *dims,
                                        float(scale), _stream(stream))
    if rc:
        raise AttnError(rc, "attn_sparse_fwd")


def attn_sparse_bwd_workspace_bytes(B, Hq, Hkv, S, N, D, topk):
    return int(load_library().attn_sparse_bwd_workspace_bytes(B, Hq, Hkv, S, N, D, topk))


def attn_sparse_bwd(q, k, v, idx, o, lse, dout, dq, dk, dv, scale, workspace, stream=None):
    """C attn_sparse_bwd: gradients of attn_sparse_fwd (dq, dk, dv fp32); workspace is a
    uint8 GPU tensor of attn_sparse_bwd_workspace_bytes() bytes."""
    dims = _sparse_check(q, k, v, idx, {"o": o, "lse": lse, "dout": dout, "dq": dq, "dk": dk, "dv": dv})
    if workspace.device.type != "cuda":
        raise TypeError("workspace must be a GPU tensor")
    nbytes = workspace.numel() * workspace.element_size()
    rc = load_library().attn_sparse_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(idx), _ptr(o), _ptr(lse), _ptr(dout),
                                        _ptr(dq), _ptr(dk), _ptr(dv), *dims, float(scale), _ptr(workspace),
                                        nbytes, _stream(stream))
    if rc:
        raise AttnError(rc, "attn_sparse_bwd")


def sparse_fwd(q, k, v, idx, scale=None):
    """Allocate o and lse and run attn_sparse_fwd. scale defaults to 1/sqrt(D)."""
    import torch
    B, Hq, Hkv, S, N, D, topk = _sparse_dims(q, k, idx)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    o = torch.empty((B, Hq, S, D), dtype=torch.bfloat16, device=q.device)
    lse = torch.empty((B, Hq, S), dtype=torch.float32, device=q.device)
    attn_sparse_fwd(q, k, v, idx, o, lse, scale)
    return o, lse


def sparse_bwd(q, k, v, idx, o, lse, dout, scale=None):
    """Allocate dq/dk/dv (fp32) and the workspace and run attn_sparse_bwd."""
    import torch
    B, Hq, Hkv, S, N, D, topk = _sparse_dims(q, k, idx)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    dq = torch.empty((B, Hq, S, D), dtype=torch.float32, device=q.device)
    dk = torch.empty((B, Hkv, N, D), dtype=torch.float32, device=q.device)
    dv = torch.empty((B, Hkv, N, D), dtype=torch.float32, device=q.device)
    ws = torch.empty((attn_sparse_bwd_workspace_bytes(B, Hq, Hkv, S, N, D, topk),), dtype=torch.uint8,
                     device=q.device)
    attn_sparse_bwd(q, k, v, idx, o, lse, dout, dq, dk, dv, scale, ws)
    return dq, dk, dv
