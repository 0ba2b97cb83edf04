"""Separate value head dimension on the GPU (attn_fwd_vdim / attn_bwd_vdim through the
C ABI): Q and K are D wide, V, O, dO and dV are Dv wide (the d and d_v of Eq. (1)),
against the fp64 oracle with the same shapes."""
import math

import numpy as np
import pytest

import oracle
import flashattention_tiled_attention_amd as fa
from flashattention_tiled_attention_amd.inputs import CONFIGS, bf16_to_f32, qkv
from tests.gpu_util import TOL_LSE, assert_close, bf16_dev_to_f64, f32_dev_to_f64, to_dev

pytestmark = pytest.mark.gpu

PAIRS = [(128, 64), (64, 128)]


def run(q, k, v, do, causal, window, scale):
    import torch
    tq, tk, tv = to_dev(q), to_dev(k), to_dev(v)
    o, lse = fa.fwd(tq, tk, tv, causal=causal, scale=scale, window=window)
    grads = None
    if do is not None:
        grads = fa.bwd(tq, tk, tv, o, lse, to_dev(do), causal=causal, scale=scale, window=window)
    torch.cuda.synchronize()
    out = [bf16_dev_to_f64(o), f32_dev_to_f64(lse)]
    if grads is not None:
        out += [f32_dev_to_f64(g) for g in grads]
    return out


def check(B, Hq, Hkv, S, D, Dv, causal, seed, window=0, scale=None, backward=True):
    print("case B=%d Hq=%d Hkv=%d S=%d D=%d Dv=%d causal=%d window=%d seed=%d scale=%s"
          % (B, Hq, Hkv, S, D, Dv, causal, window, seed, scale), flush=True)
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    q, k, v, do = qkv(B, Hq, Hkv, S, D, seed, with_dout=True, Dv=Dv)
    got = run(q, k, v, do if backward else None, causal, window, scale)
    o_ref, lse_ref = oracle.fwd(q, k, v, causal, scale, window)
    assert got[0].shape == (B, Hq, S, Dv)
    assert_close(got[0], o_ref, "O")
    assert_close(got[1], lse_ref, "lse", tol_max=TOL_LSE, tol_mean=TOL_LSE)
    if backward:
        rq, rk, rv = oracle.bwd(q, k, v, do, causal, scale, window)
        assert got[4].shape == (B, Hkv, S, Dv)
        assert_close(got[2], rq, "dQ")
        assert_close(got[3], rk, "dK")
        assert_close(got[4], rv, "dV")


@pytest.mark.parametrize("S", [1, 5, 63, 64, 65, 128, 129, 200, 383])
@pytest.mark.parametrize("D,Dv", PAIRS)
@pytest.mark.parametrize("causal", [False, True])
def test_ragged_lengths(S, D, Dv, causal):
    check(1, 2, 1, S, D, Dv, causal, seed=S + D)


@pytest.mark.parametrize("D,Dv", PAIRS)
@pytest.mark.parametrize("Hq,Hkv", [(1, 1), (8, 2), (8, 1)])
def test_gqa_groups(D, Dv, Hq, Hkv):
    check(2, Hq, Hkv, 300, D, Dv, True, seed=Hq * 10 + Hkv + Dv)


@pytest.mark.parametrize("D,Dv", PAIRS)
def test_multi_tile(D, Dv):
    check(2, 8, 2, 1000, D, Dv, True, seed=D + 1)
    check(1, 4, 4, 700, D, Dv, False, seed=D + 2)


@pytest.mark.parametrize("D,Dv", PAIRS)
@pytest.mark.parametrize("W", [1, 100, 128, 300])
def test_window(D, Dv, W):
    check(1, 4, 2, 450, D, Dv, True, seed=W + Dv, window=W)


@pytest.mark.parametrize("scale", [0.0, -0.0884, 0.5])
def test_scales(scale):
    check(1, 4, 2, 257, 128, 64, True, seed=3, scale=scale)
    check(1, 2, 2, 130, 64, 128, False, seed=4, scale=scale)


def test_equal_dims_match_plain_entry_points():
    """attn_fwd_vdim / attn_bwd_vdim with Dv == D run the same kernels as attn_fwd /
    attn_bwd (window = 0) and attn_fwd_window / attn_bwd_window: identical bits."""
    import torch
    B, Hq, Hkv, S, D = 1, 4, 2, 333, 128
    q, k, v, do = qkv(B, Hq, Hkv, S, D, 14, with_dout=True)
    tq, tk, tv, tdo = to_dev(q), to_dev(k), to_dev(v), to_dev(do)
    scale = 1.0 / math.sqrt(D)
    for causal, window in ((True, 0), (False, 0), (True, 100)):
        o1, l1 = fa.fwd(tq, tk, tv, causal=causal, window=window)
        g1 = fa.bwd(tq, tk, tv, o1, l1, tdo, causal=causal, window=window)
        o2 = torch.empty_like(o1)
        l2 = torch.empty_like(l1)
        fa.attn_fwd_vdim(tq, tk, tv, o2, l2, causal, window, scale)
        g2 = [torch.empty_like(g) for g in g1]
        ws = torch.empty((fa.attn_bwd_workspace_bytes(B, Hq, Hkv, S, D),), dtype=torch.uint8,
                         device="cuda")
        fa.attn_bwd_vdim(tq, tk, tv, o2, l2, tdo, g2[0], g2[1], g2[2], causal, window, scale, ws)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2) and torch.equal(l1, l2)
        for a, b in zip(g1, g2):
            assert torch.equal(a, b)


def test_deterministic():
    import torch
    q, k, v, do = qkv(1, 8, 2, 1024, 128, 15, with_dout=True, Dv=64)
    tq, tk, tv, tdo = to_dev(q), to_dev(k), to_dev(v), to_dev(do)
    o, lse = fa.fwd(tq, tk, tv, causal=True)
    a = fa.bwd(tq, tk, tv, o, lse, tdo, causal=True)
    b = fa.bwd(tq, tk, tv, o, lse, tdo, causal=True)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_full_size_dqk128_dv64():
    """B=1, Hq=32, Hkv=8, S=4096, causal, D=128 and Dv=64: every element of O, lse, dQ,
    dK and dV against the oracle's full forward and backward, plus causal dQ row 0 = 0
    and sum_j dV_j = sum of dO over each group."""
    c = CONFIGS["gqa_dqk128_dv64_s4096"]
    B, Hq, Hkv, S, D, Dv = c["B"], c["Hq"], c["Hkv"], c["S"], c["D"], c["Dv"]
    scale = 1.0 / math.sqrt(D)
    print("case full-size vdim B=%d Hq=%d Hkv=%d S=%d D=%d Dv=%d" % (B, Hq, Hkv, S, D, Dv), flush=True)
    q, k, v, do = qkv(B, Hq, Hkv, S, D, 0, with_dout=True, Dv=Dv)
    o, lse, dq, dk, dv = run(q, k, v, do, True, 0, scale)
    ro, rl = oracle.fwd(q, k, v, True, scale)
    assert_close(o, ro, "O")
    assert_close(lse, rl, "lse", tol_max=TOL_LSE, tol_mean=TOL_LSE)
    del ro, rl
    rq, rk, rv = oracle.bwd(q, k, v, do, True, scale)
    assert_close(dq, rq, "dQ (full tensor)")
    assert_close(dk, rk, "dK (full tensor)")
    assert_close(dv, rv, "dV (full tensor)")
    del rq, rk, rv
    assert np.max(np.abs(dq[:, :, 0])) < 1e-5
    dof = bf16_to_f32(do).astype(np.float64).reshape(B, Hkv, Hq // Hkv, S, Dv)
    assert_close(dv.sum(axis=2), dof.sum(axis=(2, 3)), "sum_j dV_j", tol_max=0.05, tol_mean=0.01)
