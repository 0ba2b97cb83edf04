"""Backward parity on the GPU: dQ, dK, dV from the HIP kernels (through the C ABI)
against the fp64 oracle's exact gradient. O and lse come from the GPU forward."""
import math

import numpy as np
import pytest

import oracle
import flashattention_tiled_attention_amd as fa
from flashattention_tiled_attention_amd.inputs import CONFIGS, bf16_to_f32, qkv
from tests.gpu_util import TOL_LSE, assert_close, bf16_dev_to_f64, f32_dev_to_f64, to_dev

pytestmark = pytest.mark.gpu


def run_bwd(q, k, v, do, causal, scale):
    import torch
    tq, tk, tv, tdo = to_dev(q), to_dev(k), to_dev(v), to_dev(do)
    o, lse = fa.fwd(tq, tk, tv, causal=causal, scale=scale)
    dq, dk, dv = fa.bwd(tq, tk, tv, o, lse, tdo, causal=causal, scale=scale)
    torch.cuda.synchronize()
    return f32_dev_to_f64(dq), f32_dev_to_f64(dk), f32_dev_to_f64(dv)


def check_full(B, Hq, Hkv, S, D, causal, seed=0, scale=None):
    print("case B=%d Hq=%d Hkv=%d S=%d D=%d causal=%d seed=%d scale=%s" % (B, Hq, Hkv, S, D, causal, seed, scale),
          flush=True)
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    q, k, v, do = qkv(B, Hq, Hkv, S, D, seed, with_dout=True)
    dq, dk, dv = run_bwd(q, k, v, do, causal, scale)
    rq, rk, rv = oracle.bwd(q, k, v, do, causal, scale)
    assert_close(dq, rq, "dQ")
    assert_close(dk, rk, "dK")
    assert_close(dv, rv, "dV")


def test_single_head_s128_d64():
    check_full(1, 1, 1, 128, 64, False, seed=0)


@pytest.mark.parametrize("S", [1, 2, 5, 63, 64, 65, 127, 128, 129, 200, 383])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_ragged_lengths(S, D, causal):
    check_full(1, 2, 1, S, D, causal, seed=S)


@pytest.mark.parametrize("Hq,Hkv", [(1, 1), (4, 2), (8, 2), (8, 1), (16, 16)])
def test_gqa_groups(Hq, Hkv):
    check_full(2, Hq, Hkv, 300, 128, True, seed=Hq * 10 + Hkv)


@pytest.mark.parametrize("B,Hq,Hkv,S,D,causal", [
    (2, 8, 2, 1024, 128, True),
    (1, 16, 8, 777, 128, True),
    (3, 4, 4, 640, 64, False),
    (2, 8, 8, 1000, 64, True),
    (1, 4, 1, 700, 128, False),
])
def test_multi_tile(B, Hq, Hkv, S, D, causal):
    check_full(B, Hq, Hkv, S, D, causal, seed=B + S)


@pytest.mark.parametrize("scale", [0.0, -0.0884, 0.5, -1.3])
def test_scales(scale):
    check_full(1, 4, 2, 257, 128, True, seed=3, scale=scale)
    check_full(1, 2, 2, 130, 64, False, seed=4, scale=scale)


@pytest.mark.parametrize("seed", [1, 2])
def test_seeds_small(seed):
    check_full(1, 8, 2, 512, 128, True, seed=seed)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_full_size_llama8b(seed):
    """B=1, Hq=32, Hkv=8, S=4096, D=128 causal, the workload the benchmark times: every
    element of O, lse, dQ, dK and dV against the oracle's full forward and backward, plus
    invariants over the whole output that hold whatever the oracle says: causal row 0 has
    dQ = 0; rows of P sum to 1, so sum_j dV_j equals the sum of dO over the group's heads
    and rows; rows of dS sum to 0, so sum_j dK_j = 0."""
    import torch
    c = CONFIGS["llama8b_causal_gqa_s4096_bwd"]
    B, Hq, Hkv, S, D, causal = c["B"], c["Hq"], c["Hkv"], c["S"], c["D"], c["causal"]
    print("case llama8b fwd+bwd full tensors seed=%d" % seed, flush=True)
    scale = 1.0 / math.sqrt(D)
    q, k, v, do = qkv(B, Hq, Hkv, S, D, seed, with_dout=True)
    tq, tk, tv, tdo = to_dev(q), to_dev(k), to_dev(v), to_dev(do)
    o, lse = fa.fwd(tq, tk, tv, causal=causal, scale=scale)
    dq, dk, dv = fa.bwd(tq, tk, tv, o, lse, tdo, causal=causal, scale=scale)
    torch.cuda.synchronize()
    o, lse = bf16_dev_to_f64(o), f32_dev_to_f64(lse)
    dq, dk, dv = f32_dev_to_f64(dq), f32_dev_to_f64(dk), f32_dev_to_f64(dv)
    ro, rl = oracle.fwd(q, k, v, causal, scale)
    assert_close(o, ro, "O")
    assert_close(lse, rl, "lse", tol_max=TOL_LSE, tol_mean=TOL_LSE)
    del ro, rl
    rq, rk, rv = oracle.bwd(q, k, v, do, causal, scale)
    for got, ref, what in ((dq, rq, "dQ"), (dk, rk, "dK"), (dv, rv, "dV")):
        mx, mean = assert_close(got, ref, what + " (full tensor)")
        print("%s max-abs %.3e mean-abs %.3e" % (what, mx, mean), flush=True)
    del rq, rk, rv
    assert np.max(np.abs(dq[:, :, 0])) < 1e-5
    dof = bf16_to_f32(do).astype(np.float64).reshape(B, Hkv, Hq // Hkv, S, D)
    # Both sums carry the unbiased bf16 rounding of P and dS summed over the group's
    # 16384 rows (about 0.016 rms per column for dV by the rounding model, less for dK)
    assert_close(dv.sum(axis=2), dof.sum(axis=(2, 3)), "sum_j dV_j", tol_max=0.05, tol_mean=0.01)
    assert_close(dk.sum(axis=2), np.zeros((B, Hkv, D)), "sum_j dK_j", tol_max=0.05, tol_mean=0.01)


@pytest.mark.parametrize("mode", ["ramp", "spike", "wide"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal,window", [(False, 0), (True, 0), (True, 100), (True, 300)])
def test_peaked_rows_backward(mode, D, causal, window):
    """The backward on rows that put most of their weight on one or a few keys at the
    usual scale 1/sqrt(D): key norms growing along the sequence (ramp), two keys that
    every later query points at (spike), and inputs of standard deviation 2.5 (wide).
    The exact gradient of Eq. (1) holds for any data, not only unit-variance inputs."""
    import torch
    from tests.gpu_util import peaked
    B, Hq, Hkv, S = 1, 4, 2, 700
    print("case peaked backward mode=%s D=%d causal=%d window=%d S=%d" % (mode, D, causal, window, S),
          flush=True)
    q, k, v, do = qkv(B, Hq, Hkv, S, D, 31 + D, with_dout=True)
    q, k, v = peaked(q, k, v, mode, spike_rows=(300, 650))
    scale = 1.0 / math.sqrt(D)
    tq, tk, tv, tdo = to_dev(q), to_dev(k), to_dev(v), to_dev(do)
    o, lse = fa.fwd(tq, tk, tv, causal=causal, scale=scale, window=window)
    g = fa.bwd(tq, tk, tv, o, lse, tdo, causal=causal, scale=scale, window=window)
    torch.cuda.synchronize()
    ro, rl = oracle.fwd(q, k, v, causal, scale, window)
    assert_close(bf16_dev_to_f64(o), ro, "O")
    assert_close(f32_dev_to_f64(lse), rl, "lse", tol_max=TOL_LSE, tol_mean=TOL_LSE)
    rq, rk, rv = oracle.bwd(q, k, v, do, causal, scale, window)
    assert_close(f32_dev_to_f64(g[0]), rq, "dQ")
    assert_close(f32_dev_to_f64(g[1]), rk, "dK")
    assert_close(f32_dev_to_f64(g[2]), rv, "dV")


def test_deterministic():
    import torch
    q, k, v, do = qkv(1, 8, 2, 1024, 128, 5, with_dout=True)
    tq, tk, tv, tdo = to_dev(q), to_dev(k), to_dev(v), to_dev(do)
    o, lse = fa.fwd(tq, tk, tv, causal=True)
    a = fa.bwd(tq, tk, tv, o, lse, tdo, causal=True)
    b = fa.bwd(tq, tk, tv, o, lse, tdo, causal=True)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_stage_entry_points_match_attn_bwd():
    """attn_bwd_dq followed by attn_bwd_dkdv gives exactly what attn_bwd gives."""
    import torch
    B, Hq, Hkv, S, D = 1, 8, 2, 700, 128
    q, k, v, do = qkv(B, Hq, Hkv, S, D, 6, with_dout=True)
    tq, tk, tv, tdo = to_dev(q), to_dev(k), to_dev(v), to_dev(do)
    o, lse = fa.fwd(tq, tk, tv, causal=True)
    ref = fa.bwd(tq, tk, tv, o, lse, tdo, causal=True)
    dq = torch.full((B, Hq, S, D), float("nan"), dtype=torch.float32, device="cuda")
    dk = torch.full((B, Hkv, S, D), float("nan"), dtype=torch.float32, device="cuda")
    dv = torch.full((B, Hkv, S, D), float("nan"), dtype=torch.float32, device="cuda")
    ws = torch.empty((fa.attn_bwd_workspace_bytes(B, Hq, Hkv, S, D),), dtype=torch.uint8, device="cuda")
    scale = 1.0 / math.sqrt(D)
    fa.attn_bwd_dq(tq, tk, tv, o, lse, tdo, dq, dk, dv, True, scale, ws)
    torch.cuda.synchronize()
    assert torch.isnan(dk).all() and torch.isnan(dv).all()   # stage 1 leaves dk, dv alone
    fa.attn_bwd_dkdv(tq, tk, tv, o, lse, tdo, dq, dk, dv, True, scale, ws)
    torch.cuda.synchronize()
    for x, y in zip((dq, dk, dv), ref):
        assert torch.equal(x, y)
