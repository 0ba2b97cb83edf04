"""Helpers for the GPU parity tests: moving bf16 bit arrays to the device and
comparing against the oracle at the tolerances the method is held to."""
import numpy as np

from flashattention_tiled_attention_amd.inputs import bf16_to_f32

# Parity bar: O, dQ, dK, dV max-abs <= 1e-2 and mean-abs <= 1e-3; lse max-abs <= 1e-3.
TOL_MAX = 1e-2
TOL_MEAN = 1e-3
TOL_LSE = 1e-3


def to_dev(bits):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to("cuda")


def bf16_dev_to_f64(t):
    import torch
    bits = t.detach().to("cpu").contiguous().view(torch.int16).numpy().view(np.uint16)
    return bf16_to_f32(bits).astype(np.float64)


def f32_dev_to_f64(t):
    return t.detach().to("cpu").numpy().astype(np.float64)


def errors(got, ref):
    d = np.abs(np.asarray(got, np.float64) - np.asarray(ref, np.float64))
    if d.size == 0:
        return 0.0, 0.0
    return float(d.max()), float(d.mean())


def assert_close(got, ref, what, tol_max=TOL_MAX, tol_mean=TOL_MEAN):
    assert np.all(np.isfinite(got)), "%s: non-finite values" % what
    mx, mean = errors(got, ref)
    assert mx <= tol_max and mean <= tol_mean, \
        "%s: max-abs %.3e (bar %.0e), mean-abs %.3e (bar %.0e)" % (what, mx, tol_max, mean, tol_mean)
    return mx, mean


def sample_rows(B, H, S, n, seed=0, tile=128):
    """Flat row indices (b*H + h)*S + i: every head's first and last rows, rows
    around tile boundaries, plus n uniformly random rows."""
    rng = np.random.default_rng(seed)
    rows = set()
    for bh in range(B * H):
        for i in (0, 1, 2, S - 1):
            rows.add(bh * S + min(max(i, 0), S - 1))
    for i in range(tile - 1, S, tile):
        bh = int(rng.integers(B * H))
        rows.add(bh * S + i)
        if i + 1 < S:
            rows.add(bh * S + i + 1)
    rows.update(int(x) for x in rng.integers(0, B * H * S, size=n))
    return np.array(sorted(rows), dtype=np.int64)
