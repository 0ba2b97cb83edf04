"""Sliding-window causal attention on the GPU (attn_fwd_window / attn_bwd_window through
the C ABI) against the fp64 oracle with the same window: query i sees keys i-W+1 .. i."""
import math

import numpy as np
import pytest

import oracle
import flashattention_tiled_attention_amd as fa
from flashattention_tiled_attention_amd.inputs import CONFIGS, bf16_to_f32, qkv
from tests.gpu_util import TOL_LSE, assert_close, bf16_dev_to_f64, f32_dev_to_f64, to_dev

pytestmark = pytest.mark.gpu


def run(q, k, v, do, window, scale):
    import torch
    tq, tk, tv = to_dev(q), to_dev(k), to_dev(v)
    o, lse = fa.fwd(tq, tk, tv, scale=scale, window=window)
    grads = None
    if do is not None:
        grads = fa.bwd(tq, tk, tv, o, lse, to_dev(do), scale=scale, window=window)
    torch.cuda.synchronize()
    out = [bf16_dev_to_f64(o), f32_dev_to_f64(lse)]
    if grads is not None:
        out += [f32_dev_to_f64(g) for g in grads]
    return out


def check(B, Hq, Hkv, S, D, W, seed, scale=None, backward=True):
    print("case B=%d Hq=%d Hkv=%d S=%d D=%d window=%d seed=%d scale=%s backward=%d"
          % (B, Hq, Hkv, S, D, W, seed, scale, backward), flush=True)
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    q, k, v, do = qkv(B, Hq, Hkv, S, D, seed, with_dout=True)
    got = run(q, k, v, do if backward else None, W, scale)
    o_ref, lse_ref = oracle.fwd(q, k, v, True, scale, W)
    assert_close(got[0], o_ref, "O")
    assert_close(got[1], lse_ref, "lse", tol_max=TOL_LSE, tol_mean=TOL_LSE)
    if backward:
        rq, rk, rv = oracle.bwd(q, k, v, do, True, scale, W)
        assert_close(got[2], rq, "dQ")
        assert_close(got[3], rk, "dK")
        assert_close(got[4], rv, "dV")


@pytest.mark.parametrize("W", [1, 2, 31, 64, 65, 127, 128, 129, 200, 300])
@pytest.mark.parametrize("D", [64, 128])
def test_windows(W, D):
    check(1, 4, 2, 390, D, W, seed=W + D)


@pytest.mark.parametrize("S", [1, 5, 63, 64, 65, 129, 257])
def test_ragged_lengths(S):
    check(2, 2, 1, S, 128, 128, seed=S)


@pytest.mark.parametrize("Hq,Hkv", [(1, 1), (8, 2), (8, 1), (16, 16)])
def test_gqa_groups(Hq, Hkv):
    check(2, Hq, Hkv, 300, 128, 100, seed=Hq * 10 + Hkv)


@pytest.mark.parametrize("scale", [0.0, -0.0884, 0.5])
def test_scales(scale):
    check(1, 4, 2, 333, 128, 128, seed=7, scale=scale)


def test_multi_tile():
    check(2, 8, 2, 1500, 128, 500, seed=11)
    check(1, 16, 8, 1100, 64, 128, seed=12)


def test_window_covering_sequence_is_causal():
    """A window of S or more keys is the causal triangle: the results equal attn_fwd /
    attn_bwd with causal set, bit for bit."""
    import torch
    B, Hq, Hkv, S, D = 1, 8, 2, 700, 128
    q, k, v, do = qkv(B, Hq, Hkv, S, D, 13, with_dout=True)
    tq, tk, tv, tdo = to_dev(q), to_dev(k), to_dev(v), to_dev(do)
    o1, l1 = fa.fwd(tq, tk, tv, causal=True)
    o2, l2 = fa.fwd(tq, tk, tv, window=S)
    g1 = fa.bwd(tq, tk, tv, o1, l1, tdo, causal=True)
    g2 = fa.bwd(tq, tk, tv, o2, l2, tdo, window=S + 50)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)


def test_full_size_window128():
    """The Llama-3.1-8B attention shape (B=1, Hq=32, Hkv=8, S=4096, D=128) with the
    128-key window: every element of O, lse, dQ, dK and dV against the oracle's full
    forward and backward with the same window, plus sum_j dV_j = sum of dO over each
    group."""
    c = CONFIGS["llama8b_window128_s4096"]
    B, Hq, Hkv, S, D, W = c["B"], c["Hq"], c["Hkv"], c["S"], c["D"], c["window"]
    scale = 1.0 / math.sqrt(D)
    print("case full-size window B=%d Hq=%d Hkv=%d S=%d D=%d W=%d" % (B, Hq, Hkv, S, D, W), flush=True)
    q, k, v, do = qkv(B, Hq, Hkv, S, D, 0, with_dout=True)
    o, lse, dq, dk, dv = run(q, k, v, do, W, scale)
    ro, rl = oracle.fwd(q, k, v, True, scale, W)
    assert_close(o, ro, "O")
    assert_close(lse, rl, "lse", tol_max=TOL_LSE, tol_mean=TOL_LSE)
    rq, rk, rv = oracle.bwd(q, k, v, do, True, scale, W)
    assert_close(dq, rq, "dQ (full tensor)")
    assert_close(dk, rk, "dK (full tensor)")
    assert_close(dv, rv, "dV (full tensor)")
    dof = bf16_to_f32(do).astype(np.float64).reshape(B, Hkv, Hq // Hkv, S, D)
    # Rows past the first 128 enter the dV product with P rounded to bf16, so each
    # row's sum_j P_ij misses 1 by an unbiased rounding error, and sum_j dV_j misses
    # sum_i dO_i by a Gaussian error per column of standard deviation
    #   sigma = r * sqrt(E[sum_j P_ij^2]) * sqrt(sum_i dO_ic^2),
    # r = 1.66e-3 the rms relative error of rounding to bf16 (8 significant bits, a
    # log-uniform mantissa) and E[sum_j P_ij^2] = exp(s2) / W for scores of variance
    # s2 = scale^2 * D (unit-variance inputs) spread over W keys. Bars: mean-abs at
    # twice the Gaussian's 0.8 sigma, max-abs at 6 sigma.
    r = 2.0 ** -7 * math.sqrt(0.375 / math.log(2.0) / 12.0)
    sigma = r * math.sqrt(math.exp(scale * scale * D) / W) * np.sqrt((dof ** 2).sum(axis=(2, 3)))
    assert_close(dv.sum(axis=2), dof.sum(axis=(2, 3)), "sum_j dV_j",
                 tol_max=6.0 * sigma.max(), tol_mean=1.6 * sigma.mean())
