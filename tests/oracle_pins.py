"""Checks that pin the fp64 oracle to facts other than its own code.

Each check takes an oracle object (``oracle.Oracle``) and raises AssertionError
when the oracle disagrees with the fact. The facts come from section 2.1 of
Rao et al., "Scheduling Data to Compute: Hierarchical Data Pipelining for LLM
Training on AMD GPUs" (Eq. (1): O = softmax(Q K^T / sqrt(d)) V), the sliding
window of its Table 7 (query i sees the keys i-W+1 .. i), the separate value
width d_v that Eq. (1) allows, the per-token index lists of its compressed sparse
attention (section 2.1, Table 7), and from
mathematics: an independent brute force on tiny inputs, closed forms,
invariants, torch's float64 CPU attention and autograd as a library routine,
and central finite differences for the gradient.

The same checks run against deliberately broken copies of the oracle
(tests/test_oracle.py) to show that each plausible mistake trips at least one.
"""
import math

import numpy as np
import torch

from flashattention_tiled_attention_amd.inputs import bf16_bits, bf16_to_f32, qkv, sparse_qkv


def _f64(bits):
    return bf16_to_f32(bits).astype(np.float64)


def _visible(causal, S, i, window=0):
    if window:
        return range(max(0, i - window + 1), i + 1)
    return range(i + 1) if causal else range(S)


def brute_force_fwd(q, k, v, causal, scale, window=0):
    """Eq. (1) on tiny inputs in pure Python: exp(s)/sum(exp(s)) with math.fsum,
    no max subtraction, no numpy linear algebra."""
    qf, kf, vf = _f64(q), _f64(k), _f64(v)
    B, Hq, S, D = q.shape
    Dv = v.shape[3]
    G = Hq // k.shape[1]
    o = np.zeros((B, Hq, S, Dv))
    lse = np.zeros((B, Hq, S))
    for b in range(B):
        for h in range(Hq):
            g = h // G
            for i in range(S):
                js = list(_visible(causal, S, i, window))
                e = [math.exp(scale * math.fsum(qf[b, h, i, d] * kf[b, g, j, d] for d in range(D)))
                     for j in js]
                z = math.fsum(e)
                lse[b, h, i] = math.log(z)
                for d in range(Dv):
                    o[b, h, i, d] = math.fsum(e[t] / z * vf[b, g, j, d] for t, j in enumerate(js))
    return o, lse


def _loss_py(qf, kf, vf, dof, causal, scale, G, window=0):
    """L = sum(O * dO) of Eq. (1), float64 arrays in, pure Python out."""
    B, Hq, S, D = qf.shape
    total = []
    for b in range(B):
        for h in range(Hq):
            g = h // G
            for i in range(S):
                js = list(_visible(causal, S, i, window))
                s = [scale * float(np.dot(qf[b, h, i], kf[b, g, j])) for j in js]
                m = max(s)
                e = [math.exp(x - m) for x in s]
                z = math.fsum(e)
                for t, j in enumerate(js):
                    total.append(e[t] / z * float(np.dot(vf[b, g, j], dof[b, h, i])))
    return math.fsum(total)


def _band_mask(S, window):
    """Boolean [S, S] mask, True where query i may attend key j: i - window < j <= i."""
    i = np.arange(S)[:, None]
    j = np.arange(S)[None, :]
    return torch.from_numpy((j <= i) & (j > i - window))


def _torch_ref(q, k, v, causal, scale, dout=None, window=0):
    """torch float64 CPU scaled_dot_product_attention (+ autograd) as a library routine;
    a window is passed to it as an explicit boolean attention mask."""
    G = q.shape[1] // k.shape[1]
    tq = torch.from_numpy(_f64(q)).requires_grad_(dout is not None)
    tk = torch.from_numpy(_f64(k)).requires_grad_(dout is not None)
    tv = torch.from_numpy(_f64(v)).requires_grad_(dout is not None)
    if window:
        o = torch.nn.functional.scaled_dot_product_attention(
            tq, tk, tv, attn_mask=_band_mask(q.shape[2], window), scale=float(scale), enable_gqa=G > 1)
    else:
        o = torch.nn.functional.scaled_dot_product_attention(
            tq, tk, tv, is_causal=bool(causal), scale=float(scale), enable_gqa=G > 1)
    if dout is None:
        return o.detach().numpy(), None
    o.backward(torch.from_numpy(_f64(dout)))
    return o.detach().numpy(), (tq.grad.numpy(), tk.grad.numpy(), tv.grad.numpy())


def _close(a, b, tol, what):
    err = float(np.max(np.abs(np.asarray(a) - np.asarray(b)))) if np.size(a) else 0.0
    assert err <= tol, "%s: max abs diff %.3e > %.1e" % (what, err, tol)


# ---------------------------------------------------------------- forward pins

def pin_brute_force(orc):
    """Oracle forward equals the pure-Python brute force on tiny shapes."""
    for (B, Hq, Hkv, S, D, causal, seed) in [(1, 1, 1, 5, 4, False, 1), (1, 2, 1, 7, 8, True, 2),
                                             (2, 4, 2, 6, 3, False, 3), (1, 2, 2, 8, 5, True, 4)]:
        q, k, v = qkv(B, Hq, Hkv, S, D, seed)
        scale = 1.0 / math.sqrt(D)
        o, lse = orc.fwd(q, k, v, causal, scale)
        ob, lb = brute_force_fwd(q, k, v, causal, scale)
        _close(o, ob, 1e-12, "O vs brute force %s" % ((B, Hq, Hkv, S, D, causal),))
        _close(lse, lb, 1e-12, "lse vs brute force")


def pin_torch_sdpa(orc):
    """Oracle forward equals torch's float64 scaled_dot_product_attention."""
    for (B, Hq, Hkv, S, D, causal, seed) in [(2, 4, 2, 33, 16, True, 5), (1, 3, 3, 40, 8, False, 6),
                                             (1, 8, 2, 17, 64, True, 7)]:
        q, k, v = qkv(B, Hq, Hkv, S, D, seed)
        scale = 1.0 / math.sqrt(D)
        o, _ = orc.fwd(q, k, v, causal, scale)
        ot, _ = _torch_ref(q, k, v, causal, scale)
        _close(o, ot, 1e-12, "O vs torch sdpa")


def pin_single_key(orc):
    """S=1: the single key gets weight 1, so O = V_0 and lse = scale * q.k_0."""
    q, k, v = qkv(2, 4, 2, 1, 16, 11)
    scale = 0.3
    for causal in (False, True):
        o, lse = orc.fwd(q, k, v, causal, scale)
        vf = _f64(v)
        _close(o, np.repeat(vf, 2, axis=1), 0.0, "S=1 O")
        expect = scale * np.einsum("bhsd,bhsd->bhs", _f64(q), np.repeat(_f64(k), 2, axis=1))
        _close(lse, expect, 1e-14, "S=1 lse")


def pin_zero_query(orc):
    """Q=0: all scores are 0, so O is the (prefix) mean of V and lse = ln(#visible keys)."""
    B, Hq, Hkv, S, D = 1, 2, 1, 9, 4
    _, k, v = qkv(B, Hq, Hkv, S, D, 12)
    q = np.zeros((B, Hq, S, D), np.uint16)
    vf = _f64(v)
    o, lse = orc.fwd(q, k, v, False, 0.125)
    _close(o, np.broadcast_to(vf.mean(axis=2, keepdims=True), o.shape), 1e-14, "Q=0 O")
    _close(lse, np.full(lse.shape, math.log(S)), 1e-14, "Q=0 lse")
    o, lse = orc.fwd(q, k, v, True, 0.125)
    prefix = np.cumsum(vf, axis=2) / np.arange(1, S + 1)[None, None, :, None]
    _close(o, np.broadcast_to(prefix, o.shape), 1e-14, "Q=0 causal O")
    _close(lse, np.broadcast_to(np.log(np.arange(1, S + 1.0)), lse.shape), 1e-14, "Q=0 causal lse")


def pin_causal_first_row(orc):
    """Causal row 0 sees only key 0: O_0 = V_0 exactly, lse_0 = scale q_0.k_0."""
    q, k, v = qkv(1, 4, 4, 12, 8, 13)
    o, lse = orc.fwd(q, k, v, True, 0.5)
    _close(o[:, :, 0], _f64(v)[:, :, 0], 0.0, "causal row 0")
    _close(lse[:, :, 0], 0.5 * np.einsum("bhd,bhd->bh", _f64(q)[:, :, 0], _f64(k)[:, :, 0]), 1e-14,
           "causal row 0 lse")


def pin_permutation(orc):
    """Non-causal: permuting the key/value rows together leaves O and lse unchanged."""
    q, k, v = qkv(1, 2, 2, 16, 8, 14)
    perm = np.random.default_rng(0).permutation(16)
    o1, l1 = orc.fwd(q, k, v, False, 0.35)
    o2, l2 = orc.fwd(q, np.ascontiguousarray(k[:, :, perm]), np.ascontiguousarray(v[:, :, perm]),
                     False, 0.35)
    _close(o1, o2, 1e-13, "permuted O")
    _close(l1, l2, 1e-13, "permuted lse")


def pin_gqa_is_repeated_mha(orc):
    """GQA with G query heads per key/value head equals MHA with each K/V head repeated
    G times consecutively (query head h reads K/V head h // G)."""
    q, k, v = qkv(2, 6, 2, 10, 8, 15)
    for causal in (False, True):
        o1, l1 = orc.fwd(q, k, v, causal, 0.4)
        o2, l2 = orc.fwd(q, np.ascontiguousarray(np.repeat(k, 3, axis=1)),
                         np.ascontiguousarray(np.repeat(v, 3, axis=1)), causal, 0.4)
        _close(o1, o2, 0.0, "GQA vs repeated MHA")
        _close(l1, l2, 0.0, "GQA lse")


def pin_sharp_softmax(orc):
    """A large scale with a unique maximum score concentrates all weight on its key."""
    B, H, S, D = 1, 1, 6, 4
    q = bf16_bits(np.array([[[[1, 0, 0, 0]] * S]], np.float32))
    kf = np.zeros((B, H, S, D), np.float32)
    kf[0, 0, :, 0] = [0.5, -1, 2, 0.25, 1, -2]   # key 2 has the unique largest score
    _, _, v = qkv(B, H, H, S, D, 16)
    o, lse = orc.fwd(q, bf16_bits(kf), v, False, 200.0)
    _close(o[0, 0], np.broadcast_to(_f64(v)[0, 0, 2], (S, D)), 1e-30, "sharp softmax")
    _close(lse, np.full(lse.shape, 400.0), 1e-12, "sharp lse")


def pin_rows_match_full(orc):
    """The sampled-row entry points agree exactly with the full ones."""
    q, k, v, do = qkv(2, 4, 2, 24, 8, 17, with_dout=True)
    for causal in (False, True):
        o, lse = orc.fwd(q, k, v, causal, 0.3)
        rows = np.array([0, 5, 23, 24, 77, 150, 191])
        o_r, l_r = orc.fwd_rows(q, k, v, rows, causal, 0.3)
        _close(o_r, o.reshape(-1, 8)[rows], 0.0, "fwd rows")
        _close(l_r, lse.reshape(-1)[rows], 0.0, "fwd rows lse")
        dq, dk, dv = orc.bwd(q, k, v, do, causal, 0.3)
        kvr = np.array([0, 3, 23, 30, 47, 60, 95, 94])
        dq_r, dk_r, dv_r = orc.bwd_rows(q, k, v, do, rows, kvr, causal, 0.3)
        _close(dq_r, dq.reshape(-1, 8)[rows], 1e-15, "dq rows")
        _close(dk_r, dk.reshape(-1, 8)[kvr], 1e-15, "dk rows")
        _close(dv_r, dv.reshape(-1, 8)[kvr], 1e-15, "dv rows")


# ---------------------------------------------------------------- backward pins

def pin_finite_differences(orc):
    """Analytic gradients equal central differences of L = sum(O * dO), where O comes
    from an independent pure-Python forward evaluated at perturbed float64 inputs."""
    h = 1e-6
    for (B, Hq, Hkv, S, D, causal, seed) in [(1, 2, 1, 5, 3, True, 21), (1, 2, 2, 4, 3, False, 22)]:
        q, k, v, do = qkv(B, Hq, Hkv, S, D, seed, with_dout=True)
        scale = 0.7
        dq, dk, dv = orc.bwd(q, k, v, do, causal, scale)
        G = Hq // Hkv
        base = [_f64(q), _f64(k), _f64(v)]
        dof = _f64(do)
        for which, grad in enumerate((dq, dk, dv)):
            for idx in np.ndindex(*base[which].shape):
                plus = [a.copy() for a in base]
                minus = [a.copy() for a in base]
                plus[which][idx] += h
                minus[which][idx] -= h
                fd = (_loss_py(*plus, dof, causal, scale, G) - _loss_py(*minus, dof, causal, scale, G)) / (2 * h)
                assert abs(fd - grad[idx]) <= 1e-7 * max(1.0, abs(fd)), \
                    "finite difference %s%s: fd %.9f analytic %.9f" % ("qkv"[which], idx, fd, grad[idx])


def pin_torch_autograd(orc):
    """Oracle gradients equal torch float64 autograd of scaled_dot_product_attention
    (dK, dV summed over the query heads of each group)."""
    for (B, Hq, Hkv, S, D, causal, seed) in [(2, 4, 2, 29, 16, True, 23), (1, 3, 3, 20, 8, False, 24),
                                             (1, 8, 2, 13, 64, True, 25)]:
        q, k, v, do = qkv(B, Hq, Hkv, S, D, seed, with_dout=True)
        scale = 1.0 / math.sqrt(D)
        dq, dk, dv = orc.bwd(q, k, v, do, causal, scale)
        _, (tq, tk, tv) = _torch_ref(q, k, v, causal, scale, do)
        _close(dq, tq, 1e-12, "dQ vs torch autograd")
        _close(dk, tk, 1e-12, "dK vs torch autograd")
        _close(dv, tv, 1e-12, "dV vs torch autograd")


def pin_backward_invariants(orc):
    """Rows of P sum to 1, so sum_j dV_j = sum of dO over the group's heads and rows;
    rows of dS sum to 0, so sum_j dK_j = 0; causal row 0 has dQ = 0."""
    B, Hq, Hkv, S, D = 2, 4, 2, 19, 8
    q, k, v, do = qkv(B, Hq, Hkv, S, D, 26, with_dout=True)
    for causal in (False, True):
        dq, dk, dv = orc.bwd(q, k, v, do, causal, 0.35)
        dof = _f64(do).reshape(B, Hkv, Hq // Hkv, S, D)
        _close(dv.sum(axis=2), dof.sum(axis=(2, 3)), 1e-12, "sum dV")
        _close(dk.sum(axis=2), np.zeros((B, Hkv, D)), 1e-12, "sum dK")
        if causal:
            _close(dq[:, :, 0], np.zeros((B, Hq, D)), 1e-15, "causal dQ row 0")


def pin_equal_keys(orc):
    """With every key equal, scores do not depend on Q, so dQ = 0."""
    B, Hq, Hkv, S, D = 1, 2, 1, 7, 4
    q, k, v, do = qkv(B, Hq, Hkv, S, D, 27, with_dout=True)
    k = np.ascontiguousarray(np.broadcast_to(k[:, :, :1], k.shape))
    for causal in (False, True):
        dq, _, _ = orc.bwd(q, k, v, do, causal, 0.5)
        _close(dq, np.zeros_like(dq), 1e-14, "equal keys dQ")


# ---------------------------------------------------------------- sliding-window pins

def pin_window_brute_force(orc):
    """Windowed forward equals the pure-Python brute force over the band i-W < j <= i."""
    for (B, Hq, Hkv, S, D, W, seed) in [(1, 2, 1, 9, 4, 1, 31), (1, 2, 2, 8, 3, 2, 32),
                                        (2, 4, 2, 7, 5, 3, 33), (1, 1, 1, 9, 4, 5, 34)]:
        q, k, v = qkv(B, Hq, Hkv, S, D, seed)
        o, lse = orc.fwd(q, k, v, True, 0.6, W)
        ob, lb = brute_force_fwd(q, k, v, True, 0.6, W)
        _close(o, ob, 1e-12, "windowed O vs brute force W=%d" % W)
        _close(lse, lb, 1e-12, "windowed lse vs brute force W=%d" % W)


def pin_window_torch(orc):
    """Windowed forward and gradients equal torch float64 SDPA (and its autograd) given
    the band as an explicit boolean mask."""
    for (B, Hq, Hkv, S, D, W, seed) in [(1, 4, 2, 37, 16, 8, 35), (2, 2, 2, 30, 8, 1, 36),
                                        (1, 8, 2, 21, 32, 13, 37)]:
        q, k, v, do = qkv(B, Hq, Hkv, S, D, seed, with_dout=True)
        scale = 1.0 / math.sqrt(D)
        o, _ = orc.fwd(q, k, v, True, scale, W)
        dq, dk, dv = orc.bwd(q, k, v, do, True, scale, W)
        ot, (tq, tk, tv) = _torch_ref(q, k, v, True, scale, do, window=W)
        _close(o, ot, 1e-12, "windowed O vs torch sdpa W=%d" % W)
        _close(dq, tq, 1e-12, "windowed dQ vs torch autograd")
        _close(dk, tk, 1e-12, "windowed dK vs torch autograd")
        _close(dv, tv, 1e-12, "windowed dV vs torch autograd")


def pin_window_closed_forms(orc):
    """W = 1: each query sees only its own key, so O_i = V_i, lse_i = scale q_i.k_i and
    dQ = dK = 0. W >= S: the band is the whole causal triangle, so the result is the
    causal one exactly. Q = 0: O_i is the mean of V over the min(i+1, W) keys in the band."""
    B, Hq, Hkv, S, D = 1, 4, 2, 11, 8
    q, k, v, do = qkv(B, Hq, Hkv, S, D, 38, with_dout=True)
    o, lse = orc.fwd(q, k, v, True, 0.45, 1)
    _close(o, np.repeat(_f64(v), 2, axis=1), 0.0, "W=1 O")
    _close(lse, 0.45 * np.einsum("bhsd,bhsd->bhs", _f64(q), np.repeat(_f64(k), 2, axis=1)), 1e-14,
           "W=1 lse")
    dq, dk, dv = orc.bwd(q, k, v, do, True, 0.45, 1)
    _close(dq, np.zeros_like(dq), 0.0, "W=1 dQ")
    _close(dk, np.zeros_like(dk), 0.0, "W=1 dK")
    _close(dv, _f64(do).reshape(B, Hkv, 2, S, D).sum(axis=2), 1e-15, "W=1 dV")
    for W in (S, S + 5):
        o1, l1 = orc.fwd(q, k, v, True, 0.45, W)
        o2, l2 = orc.fwd(q, k, v, True, 0.45)
        _close(o1, o2, 0.0, "W>=S O")
        _close(l1, l2, 0.0, "W>=S lse")
        g1 = orc.bwd(q, k, v, do, True, 0.45, W)
        g2 = orc.bwd(q, k, v, do, True, 0.45)
        for a, b in zip(g1, g2):
            _close(a, b, 0.0, "W>=S gradients")
    q0 = np.zeros_like(q)
    W = 4
    o, lse = orc.fwd(q0, k, v, True, 0.45, W)
    vf = _f64(v)
    for i in range(S):
        j0 = max(0, i - W + 1)
        _close(o[:, :, i], np.repeat(vf[:, :, j0:i + 1].mean(axis=2), 2, axis=1), 1e-14, "Q=0 band mean")
        _close(lse[:, :, i], np.full((B, Hq), math.log(i + 1 - j0)), 1e-14, "Q=0 band lse")


def pin_window_gradients(orc):
    """Windowed gradients equal central differences of L = sum(O * dO) from the
    pure-Python forward; rows of P still sum to 1 and rows of dS to 0 inside the band;
    the sampled-row entry points agree with the full ones."""
    h = 1e-6
    B, Hq, Hkv, S, D, W = 1, 2, 1, 6, 3, 2
    q, k, v, do = qkv(B, Hq, Hkv, S, D, 39, with_dout=True)
    dq, dk, dv = orc.bwd(q, k, v, do, True, 0.8, W)
    base = [_f64(q), _f64(k), _f64(v)]
    dof = _f64(do)
    for which, grad in enumerate((dq, dk, dv)):
        for idx in np.ndindex(*base[which].shape):
            plus = [a.copy() for a in base]
            minus = [a.copy() for a in base]
            plus[which][idx] += h
            minus[which][idx] -= h
            fd = (_loss_py(*plus, dof, True, 0.8, Hq // Hkv, W)
                  - _loss_py(*minus, dof, True, 0.8, Hq // Hkv, W)) / (2 * h)
            assert abs(fd - grad[idx]) <= 1e-7 * max(1.0, abs(fd)), \
                "windowed finite difference %s%s: fd %.9f analytic %.9f" % ("qkv"[which], idx, fd, grad[idx])
    B, Hq, Hkv, S, D, W = 2, 4, 2, 23, 8, 5
    q, k, v, do = qkv(B, Hq, Hkv, S, D, 40, with_dout=True)
    dq, dk, dv = orc.bwd(q, k, v, do, True, 0.35, W)
    dofull = _f64(do).reshape(B, Hkv, Hq // Hkv, S, D)
    _close(dv.sum(axis=2), dofull.sum(axis=(2, 3)), 1e-12, "windowed sum dV")
    _close(dk.sum(axis=2), np.zeros((B, Hkv, D)), 1e-12, "windowed sum dK")
    o, lse = orc.fwd(q, k, v, True, 0.35, W)
    rows = np.array([0, 4, 5, 22, 23, 99, 183])
    o_r, l_r = orc.fwd_rows(q, k, v, rows, True, 0.35, W)
    _close(o_r, o.reshape(-1, D)[rows], 0.0, "windowed fwd rows")
    _close(l_r, lse.reshape(-1)[rows], 0.0, "windowed fwd rows lse")
    kvr = np.array([0, 3, 22, 23, 40, 91])
    dq_r, dk_r, dv_r = orc.bwd_rows(q, k, v, do, rows, kvr, True, 0.35, W)
    _close(dq_r, dq.reshape(-1, D)[rows], 1e-15, "windowed dq rows")
    _close(dk_r, dk.reshape(-1, D)[kvr], 1e-15, "windowed dk rows")
    _close(dv_r, dv.reshape(-1, D)[kvr], 1e-15, "windowed dv rows")


# ------------------------------------------------------ value head dim d_v != d

def _fd_check(orc, B, Hq, Hkv, S, D, Dv, causal, scale, seed, window=0):
    """Central differences of L = sum(O * dO) (pure-Python forward) against the
    oracle's analytic gradients."""
    h = 1e-6
    q, k, v, do = qkv(B, Hq, Hkv, S, D, seed, with_dout=True, Dv=Dv)
    dq, dk, dv = orc.bwd(q, k, v, do, causal, scale, window)
    base = [_f64(q), _f64(k), _f64(v)]
    dof = _f64(do)
    for which, grad in enumerate((dq, dk, dv)):
        assert grad.shape == base[which].shape, "gradient shape %s" % (grad.shape,)
        for idx in np.ndindex(*base[which].shape):
            plus = [a.copy() for a in base]
            minus = [a.copy() for a in base]
            plus[which][idx] += h
            minus[which][idx] -= h
            fd = (_loss_py(*plus, dof, causal, scale, Hq // Hkv, window)
                  - _loss_py(*minus, dof, causal, scale, Hq // Hkv, window)) / (2 * h)
            assert abs(fd - grad[idx]) <= 1e-7 * max(1.0, abs(fd)), \
                "d_v != d finite difference %s%s: fd %.9f analytic %.9f" % ("qkv"[which], idx, fd, grad[idx])


def pin_value_dim(orc):
    """Eq. (1) lets the value width d_v differ from the query/key width d. With
    Dv != D: the forward equals the pure-Python brute force and torch's float64
    attention (which takes V of its own width), the gradients equal central
    differences and torch autograd, Q = 0 gives prefix means of V, and the
    sampled-row entry points agree with the full ones. Every Dv > D case runs
    before any Dv < D case."""
    # Dv > D
    for (B, Hq, Hkv, S, D, Dv, causal, seed) in [(1, 2, 1, 6, 3, 5, True, 41), (2, 4, 2, 5, 4, 7, False, 42)]:
        q, k, v = qkv(B, Hq, Hkv, S, D, seed, Dv=Dv)
        scale = 1.0 / math.sqrt(D)
        o, lse = orc.fwd(q, k, v, causal, scale)
        ob, lb = brute_force_fwd(q, k, v, causal, scale)
        _close(o, ob, 1e-12, "d_v > d: O vs brute force %s" % ((B, Hq, Hkv, S, D, Dv, causal),))
        _close(lse, lb, 1e-12, "d_v > d: lse vs brute force")
    q, k, v, do = qkv(1, 4, 2, 21, 8, 0, with_dout=True, Dv=16)
    dq, dk, dv = orc.bwd(q, k, v, do, True, 0.3)
    o, _ = orc.fwd(q, k, v, True, 0.3)
    ot, (tq, tk, tv) = _torch_ref(q, k, v, True, 0.3, do)
    _close(o, ot, 1e-12, "d_v > d: O vs torch sdpa")
    _close(dq, tq, 1e-12, "d_v > d: dQ vs torch autograd")
    _close(dk, tk, 1e-12, "d_v > d: dK vs torch autograd")
    _close(dv, tv, 1e-12, "d_v > d: dV vs torch autograd")
    _fd_check(orc, 1, 2, 1, 4, 2, 3, True, 0.7, 43)
    q, k, v = qkv(1, 2, 1, 9, 4, 44, Dv=6)
    q = np.zeros_like(q)
    o, _ = orc.fwd(q, k, v, True, 0.5)
    vf = _f64(v)
    prefix = np.cumsum(vf, axis=2) / np.arange(1, 10.0)[None, None, :, None]
    _close(o, np.broadcast_to(prefix, o.shape), 1e-14, "d_v > d: Q=0 causal O")
    B, Hq, Hkv, S, D, Dv = 2, 4, 2, 23, 8, 12
    q, k, v, do = qkv(B, Hq, Hkv, S, D, 45, with_dout=True, Dv=Dv)
    rows = np.array([0, 4, 5, 22, 23, 99, 183])
    kvr = np.array([0, 3, 22, 23, 40, 91])
    for causal, window in ((False, 0), (True, 0), (True, 4)):
        o, lse = orc.fwd(q, k, v, causal, 0.35, window)
        o_r, l_r = orc.fwd_rows(q, k, v, rows, causal, 0.35, window)
        _close(o_r, o.reshape(-1, Dv)[rows], 0.0, "d_v > d: fwd rows")
        _close(l_r, lse.reshape(-1)[rows], 0.0, "d_v > d: fwd rows lse")
        dq, dk, dv = orc.bwd(q, k, v, do, causal, 0.35, window)
        dq_r, dk_r, dv_r = orc.bwd_rows(q, k, v, do, rows, kvr, causal, 0.35, window)
        _close(dq_r, dq.reshape(-1, D)[rows], 1e-15, "d_v > d: dq rows")
        _close(dk_r, dk.reshape(-1, D)[kvr], 1e-15, "d_v > d: dk rows")
        _close(dv_r, dv.reshape(-1, Dv)[kvr], 1e-15, "d_v > d: dv rows")
        # rows of P sum to 1 and rows of dS to 0
        _close(dv.sum(axis=2), _f64(do).reshape(B, Hkv, 2, S, Dv).sum(axis=(2, 3)), 1e-12, "d_v > d: sum dV")
        _close(dk.sum(axis=2), np.zeros((B, Hkv, D)), 1e-12, "d_v > d: sum dK")
    # Dv < D
    for (B, Hq, Hkv, S, D, Dv, causal, seed) in [(1, 2, 2, 5, 6, 3, True, 46), (1, 3, 1, 4, 5, 2, False, 47)]:
        q, k, v = qkv(B, Hq, Hkv, S, D, seed, Dv=Dv)
        o, lse = orc.fwd(q, k, v, causal, 0.45)
        ob, lb = brute_force_fwd(q, k, v, causal, 0.45)
        _close(o, ob, 1e-12, "d_v < d: O vs brute force")
        _close(lse, lb, 1e-12, "d_v < d: lse vs brute force")
    for causal, window in ((False, 0), (True, 0), (True, 6)):
        q, k, v, do = qkv(2, 4, 2, 19, 16, 48, with_dout=True, Dv=8)
        o, _ = orc.fwd(q, k, v, causal, 0.25, window)
        dq, dk, dv = orc.bwd(q, k, v, do, causal, 0.25, window)
        ot, (tq, tk, tv) = _torch_ref(q, k, v, causal, 0.25, do, window)
        _close(o, ot, 1e-12, "d_v < d: O vs torch sdpa")
        _close(dq, tq, 1e-12, "d_v < d: dQ vs torch autograd")
        _close(dk, tk, 1e-12, "d_v < d: dK vs torch autograd")
        _close(dv, tv, 1e-12, "d_v < d: dV vs torch autograd")
    _fd_check(orc, 1, 2, 1, 5, 3, 2, True, 0.6, 49, window=2)


# ------------------------------------------------ sparse (index-list) attention

def _lists(S, causal=True, window=0, holes=0, seed=None):
    """idx [1,S,topk] naming each visible key of a dense pattern in ascending order,
    with `holes` empty slots (-1) scattered among them when seed is given."""
    rows = [list(_visible(causal, S, i, window)) for i in range(S)]
    if seed is not None:
        rng = np.random.default_rng(seed)
        for r in rows:
            for _ in range(holes):
                r.insert(int(rng.integers(0, len(r) + 1)), -1)
    topk = max(len(r) for r in rows)
    idx = np.full((1, S, topk), -1, dtype=np.int32)
    for i, r in enumerate(rows):
        idx[0, i, :len(r)] = r
    return idx


def _sparse_brute(q, k, v, idx, scale):
    """Slot-by-slot pure-Python evaluation: softmax over a token's non-empty slots."""
    qf, kf, vf = _f64(q), _f64(k), _f64(v)
    B, Hq, S, D = q.shape
    Hkv, N = k.shape[1], k.shape[2]
    G = Hq // Hkv
    o = np.zeros((B, Hq, S, D))
    lse = np.full((B, Hq, S), -np.inf)
    for b in range(B):
        for h in range(Hq):
            for i in range(S):
                js = [int(j) for j in idx[b, i] if 0 <= j < N]
                if not js:
                    continue
                e = [math.exp(scale * math.fsum(qf[b, h, i, d] * kf[b, h // G, j, d] for d in range(D)))
                     for j in js]
                z = math.fsum(e)
                lse[b, h, i] = math.log(z)
                for d in range(D):
                    o[b, h, i, d] = math.fsum(e[t] / z * vf[b, h // G, j, d] for t, j in enumerate(js))
    return o, lse


def _sparse_loss_py(qf, kf, vf, dof, idx, scale, G):
    """L = sum(O * dO) of slot-wise sparse attention, pure Python out."""
    B, Hq, S, D = qf.shape
    N = kf.shape[2]
    total = []
    for b in range(B):
        for h in range(Hq):
            for i in range(S):
                js = [int(j) for j in idx[b, i] if 0 <= j < N]
                if not js:
                    continue
                sc = [scale * float(np.dot(qf[b, h, i], kf[b, h // G, j])) for j in js]
                m = max(sc)
                e = [math.exp(x - m) for x in sc]
                z = math.fsum(e)
                for t, j in enumerate(js):
                    total.append(e[t] / z * float(np.dot(vf[b, h // G, j], dof[b, h, i])))
    return math.fsum(total)


def pin_sparse_matches_dense(orc):
    """Lists naming exactly the keys a dense pattern shows (causal, sliding window or all,
    with empty slots scattered in) give the dense oracle's O, lse, dQ, dK and dV."""
    B, Hq, Hkv, S, D = 1, 4, 2, 13, 8
    q, k, v, do = qkv(B, Hq, Hkv, S, D, 50, with_dout=True)
    for causal, window, holes in ((True, 0, 0), (False, 0, 2), (True, 4, 3), (True, 1, 1)):
        idx = _lists(S, causal, window, holes, seed=51 if holes else None)
        o, lse = orc.sparse_fwd(q, k, v, idx, 0.4)
        od, ld = orc.fwd(q, k, v, causal, 0.4, window)
        _close(o, od, 1e-13, "sparse vs dense O %s" % ((causal, window, holes),))
        _close(lse, ld, 1e-13, "sparse vs dense lse")
        dq, dk, dv = orc.sparse_bwd(q, k, v, do, idx, 0.4)
        rq, rk, rv = orc.bwd(q, k, v, do, causal, 0.4, window)
        _close(dq, rq, 1e-13, "sparse vs dense dQ")
        _close(dk, rk, 1e-13, "sparse vs dense dK")
        _close(dv, rv, 1e-13, "sparse vs dense dV")


def pin_sparse_torch(orc):
    """Random duplicate-free lists over N != S rows equal torch float64 attention (and
    autograd) with the lists passed as a boolean [S, N] mask."""
    B, Hq, Hkv, S, N, D = 2, 4, 2, 11, 17, 8
    rng = np.random.default_rng(52)
    q, k, v, do = sparse_qkv(B, Hq, Hkv, S, N, D, 53, with_dout=True)
    topk = 7
    idx = np.full((B, S, topk), -1, dtype=np.int32)
    mask = np.zeros((B, 1, S, N), dtype=bool)
    for b in range(B):
        for i in range(S):
            m = int(rng.integers(1, topk + 1))
            js = rng.choice(N, size=m, replace=False)
            slots = rng.choice(topk, size=m, replace=False)
            idx[b, i, slots] = js
            mask[b, 0, i, js] = True
    tq = torch.from_numpy(_f64(q)).requires_grad_(True)
    tk = torch.from_numpy(_f64(k)).requires_grad_(True)
    tv = torch.from_numpy(_f64(v)).requires_grad_(True)
    ot = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=torch.from_numpy(mask),
                                                          scale=0.3, enable_gqa=True)
    ot.backward(torch.from_numpy(_f64(do)))
    o, _ = orc.sparse_fwd(q, k, v, idx, 0.3)
    dq, dk, dv = orc.sparse_bwd(q, k, v, do, idx, 0.3)
    _close(o, ot.detach().numpy(), 1e-12, "sparse O vs torch masked sdpa")
    _close(dq, tq.grad.numpy(), 1e-12, "sparse dQ vs torch autograd")
    _close(dk, tk.grad.numpy(), 1e-12, "sparse dK vs torch autograd")
    _close(dv, tv.grad.numpy(), 1e-12, "sparse dV vs torch autograd")


def pin_sparse_brute_force(orc):
    """Pure-Python slot-wise evaluation on tiny shapes, with rows listed twice, empty
    slots, out-of-range entries and a token whose list is empty."""
    B, Hq, Hkv, S, N, D = 1, 4, 2, 6, 9, 5
    q, k, v = sparse_qkv(B, Hq, Hkv, S, N, D, 54)
    idx = np.array([[[3, -1, 3, 8], [-1, -1, -1, -1], [0, 1, 2, 9], [8, 7, 6, 5],
                     [4, -7, 4, 4], [2, 2, 100, 0]]], dtype=np.int32)
    o, lse = orc.sparse_fwd(q, k, v, idx, 0.6)
    ob, lb = _sparse_brute(q, k, v, idx, 0.6)
    _close(o, ob, 1e-12, "sparse O vs brute force")
    assert np.array_equal(np.isinf(lse), np.isinf(lb)), "sparse lse -inf pattern"
    fin = np.isfinite(lb)
    _close(lse[fin], lb[fin], 1e-12, "sparse lse vs brute force")


def pin_sparse_closed_forms(orc):
    """Empty list: O = 0, lse = -inf, dQ = 0. One non-empty slot: O = V_j,
    lse = scale q.k_j, dQ = 0. A row listed twice where it stands alone: same O, lse
    larger by ln 2. Permuting a token's slots changes nothing. Rows no list names get
    dK = dV = 0."""
    B, Hq, Hkv, S, N, D = 1, 2, 1, 4, 6, 8
    q, k, v, do = sparse_qkv(B, Hq, Hkv, S, N, D, 55, with_dout=True)
    idx = np.array([[[-1, -1, -1], [4, -1, -1], [-1, 2, 2], [1, 3, 0]]], dtype=np.int32)
    o, lse = orc.sparse_fwd(q, k, v, idx, 0.5)
    dq, dk, dv = orc.sparse_bwd(q, k, v, do, idx, 0.5)
    qf, kf, vf = _f64(q), _f64(k), _f64(v)
    _close(o[0, :, 0], np.zeros((Hq, D)), 0.0, "empty list O")
    assert np.all(np.isneginf(lse[0, :, 0])), "empty list lse"
    _close(dq[0, :, 0], np.zeros((Hq, D)), 0.0, "empty list dQ")
    _close(o[0, :, 1], np.broadcast_to(vf[0, 0, 4], (Hq, D)), 1e-15, "single slot O")
    _close(lse[0, :, 1], 0.5 * qf[0, :, 1] @ kf[0, 0, 4], 1e-13, "single slot lse")
    _close(dq[0, :, 1], np.zeros((Hq, D)), 1e-14, "single slot dQ")
    _close(o[0, :, 2], np.broadcast_to(vf[0, 0, 2], (Hq, D)), 1e-15, "doubled slot O")
    _close(lse[0, :, 2], 0.5 * qf[0, :, 2] @ kf[0, 0, 2] + math.log(2.0), 1e-13, "doubled slot lse")
    _close(dk[0, 0, 5], np.zeros(D), 0.0, "unnamed row dK")
    _close(dv[0, 0, 5], np.zeros(D), 0.0, "unnamed row dV")
    perm = idx.copy()
    perm[0, 3] = [0, 1, 3]
    o2, l2 = orc.sparse_fwd(q, k, v, perm, 0.5)
    g2 = orc.sparse_bwd(q, k, v, do, perm, 0.5)
    _close(o2, o, 1e-14, "slot permutation O")
    assert np.array_equal(np.isneginf(l2), np.isneginf(lse)), "slot permutation lse -inf pattern"
    _close(l2[np.isfinite(lse)], lse[np.isfinite(lse)], 1e-14, "slot permutation lse")
    for a, b_, n in zip(g2, (dq, dk, dv), ("dQ", "dK", "dV")):
        _close(a, b_, 1e-14, "slot permutation " + n)


def pin_sparse_gradients(orc):
    """Central differences of L = sum(O * dO) (pure-Python slot-wise forward) match the
    gradients, with duplicates and an empty list; rows of P sum to 1 and rows of dS to
    0, so sum_j dV_j = sum of dO over tokens with a non-empty list and sum_j dK_j = 0;
    the sampled-row forms agree with the full ones."""
    h = 1e-6
    B, Hq, Hkv, S, N, D = 1, 2, 1, 4, 5, 3
    q, k, v, do = sparse_qkv(B, Hq, Hkv, S, N, D, 56, with_dout=True)
    idx = np.array([[[2, 2, 0], [-1, -1, -1], [4, 1, -1], [0, 3, 4]]], dtype=np.int32)
    dq, dk, dv = orc.sparse_bwd(q, k, v, do, idx, 0.8)
    base = [_f64(q), _f64(k), _f64(v)]
    dof = _f64(do)
    for which, grad in enumerate((dq, dk, dv)):
        for ix in np.ndindex(*base[which].shape):
            plus = [a.copy() for a in base]
            minus = [a.copy() for a in base]
            plus[which][ix] += h
            minus[which][ix] -= h
            fd = (_sparse_loss_py(*plus, dof, idx, 0.8, Hq // Hkv)
                  - _sparse_loss_py(*minus, dof, idx, 0.8, Hq // Hkv)) / (2 * h)
            assert abs(fd - grad[ix]) <= 1e-7 * max(1.0, abs(fd)), \
                "sparse finite difference %s%s: fd %.9f analytic %.9f" % ("qkv"[which], ix, fd, grad[ix])
    B, Hq, Hkv, S, N, D = 2, 4, 2, 9, 14, 8
    q, k, v, do = sparse_qkv(B, Hq, Hkv, S, N, D, 57, with_dout=True)
    rng = np.random.default_rng(58)
    idx = rng.integers(-3, N, size=(B, S, 6)).astype(np.int32)
    idx[0, 4] = -1
    dq, dk, dv = orc.sparse_bwd(q, k, v, do, idx, 0.45)
    live = (idx >= 0).any(axis=2)                                   # [B][S]
    dof = _f64(do) * live[:, None, :, None]
    _close(dv.sum(axis=2), dof.reshape(B, Hkv, Hq // Hkv, S, D).sum(axis=(2, 3)), 1e-12, "sparse sum dV")
    _close(dk.sum(axis=2), np.zeros((B, Hkv, D)), 1e-12, "sparse sum dK")
    rows = np.array([0, 4, 13, 40, 71])
    kvr = np.array([0, 5, 13, 27, 30, 55])
    o, lse = orc.sparse_fwd(q, k, v, idx, 0.45)
    o_r, l_r = orc.sparse_fwd(q, k, v, idx, 0.45, rows=rows)
    _close(o_r, o.reshape(-1, D)[rows], 0.0, "sparse fwd rows")
    assert np.array_equal(l_r, lse.reshape(-1)[rows]), "sparse fwd rows lse"
    dq_r, dk_r, dv_r = orc.sparse_bwd(q, k, v, do, idx, 0.45, qrows=rows, kvrows=kvr)
    _close(dq_r, dq.reshape(-1, D)[rows], 0.0, "sparse dq rows")
    _close(dk_r, dk.reshape(-1, D)[kvr], 0.0, "sparse dk rows")
    _close(dv_r, dv.reshape(-1, D)[kvr], 0.0, "sparse dv rows")


FORWARD_PINS = [pin_brute_force, pin_torch_sdpa, pin_single_key, pin_zero_query,
                pin_causal_first_row, pin_permutation, pin_gqa_is_repeated_mha, pin_sharp_softmax,
                pin_rows_match_full]
BACKWARD_PINS = [pin_finite_differences, pin_torch_autograd, pin_backward_invariants, pin_equal_keys]
WINDOW_PINS = [pin_window_brute_force, pin_window_torch, pin_window_closed_forms, pin_window_gradients]
VALUE_DIM_PINS = [pin_value_dim]
SPARSE_PINS = [pin_sparse_matches_dense, pin_sparse_torch, pin_sparse_brute_force, pin_sparse_closed_forms,
               pin_sparse_gradients]
ALL_PINS = FORWARD_PINS + BACKWARD_PINS + WINDOW_PINS + VALUE_DIM_PINS + SPARSE_PINS
