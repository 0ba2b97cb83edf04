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


def peaked(q, k, v, mode, spike_rows, key_axis_len=None):
    """Inputs whose softmax rows concentrate on few keys at the usual scale 1/sqrt(D),
    as bf16 bits (q, k, v in, q, k, v out; dO is left as drawn):
      ramp   key norms grow fourfold along the key axis, so a row's maximum keeps moving;
      spike  every query gets +1 in each component and the keys in `spike_rows` are
             2.5 in every component, so rows that see one of them put nearly all their
             weight on it;
      wide   Q and K scaled by 2.5: score variance 39 instead of 1.
    V is halved so that |O| stays below 4, where the bf16 store of O alone could miss
    the 1e-2 bar (the bf16 spacing there is 2^-5)."""
    from flashattention_tiled_attention_amd.inputs import bf16_bits
    qf, kf = bf16_to_f32(q), bf16_to_f32(k)
    n = kf.shape[2] if key_axis_len is None else key_axis_len
    if mode == "ramp":
        kf = kf.copy()
        kf[:, :, :n] *= (1.0 + 3.0 * np.arange(n, dtype=np.float32) / n)[None, None, :, None]
    elif mode == "spike":
        qf = qf + 1.0
        kf = kf.copy()
        for t in spike_rows:
            kf[:, :, t, :] = 2.5
    elif mode == "wide":
        qf, kf = qf * 2.5, kf * 2.5
    else:
        raise ValueError(mode)
    return bf16_bits(qf), bf16_bits(kf), bf16_bits(bf16_to_f32(v) * 0.5)


def head_offset_rows(B, H, S, stride):
    """Flat row indices (b*H + h)*S + i with i = (b*H + h) % stride (mod stride): every
    stride-th query row of each head, the residue moving from head to head so every
    lane position of a row tile is covered, plus each head's last row."""
    rows = []
    for bh in range(B * H):
        i = np.arange(bh % stride, S, stride, dtype=np.int64)
        rows.append(bh * S + i)
        rows.append(np.array([bh * S + S - 1], np.int64))
    return np.unique(np.concatenate(rows))
