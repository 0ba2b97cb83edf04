"""Backward parity on the GPU: dQ, dK, dV from the HIP kernels (through the C ABI)
against the fp64 oracle's exact gradient. O and lse come from the GPU forward."""
import math

import numpy as np
import pytest

import oracle
import flashattention_tiled_attention_amd as fa
from flashattention_tiled_attention_amd.inputs import CONFIGS, bf16_to_f32, qkv
from tests.gpu_util import assert_close, f32_dev_to_f64, sample_rows, to_dev

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


def test_full_size_llama8b_bwd_sampled():
    """B=1, Hq=32, Hkv=8, S=4096, D=128 causal: the workload the benchmark times. dQ is
    checked on sampled rows, dK/dV on sampled keys of two KV heads (the oracle recomputes
    every row statistic of those heads), plus invariants over the whole output."""
    c = CONFIGS["llama8b_causal_gqa_s4096_bwd"]
    B, Hq, Hkv, S, D, causal = c["B"], c["Hq"], c["Hkv"], c["S"], c["D"], c["causal"]
    scale = 1.0 / math.sqrt(D)
    q, k, v, do = qkv(B, Hq, Hkv, S, D, 0, with_dout=True)
    dq, dk, dv = run_bwd(q, k, v, do, causal, scale)
    assert np.all(np.isfinite(dq)) and np.all(np.isfinite(dk)) and np.all(np.isfinite(dv))
    qrows = sample_rows(B, Hq, S, 300, seed=2)
    rng = np.random.default_rng(3)
    keys = []
    for grp in (0, Hkv - 1):
        ks = set([0, 1, 2, 63, 64, 127, 128, S - 1]) | set(int(x) for x in rng.integers(0, S, 40))
        keys += [grp * S + j for j in sorted(ks)]
    kvrows = np.array(keys, dtype=np.int64)
    rq, rk, rv = oracle.bwd_rows(q, k, v, do, qrows, kvrows, causal, scale)
    assert_close(dq.reshape(-1, D)[qrows], rq, "dQ (%d sampled rows)" % qrows.size)
    assert_close(dk.reshape(-1, D)[kvrows], rk, "dK (%d sampled keys)" % kvrows.size)
    assert_close(dv.reshape(-1, D)[kvrows], rv, "dV (%d sampled keys)" % kvrows.size)
    # invariants over everything: causal row 0 has dQ = 0; rows of P sum to one, so
    # sum_j dV_j equals the sum of dO over the group's heads and rows
    assert np.max(np.abs(dq[:, :, 0])) < 1e-5
    dof = bf16_to_f32(do).astype(np.float64).reshape(B, Hkv, Hq // Hkv, S, D)
    assert_close(dv.sum(axis=2), dof.sum(axis=(2, 3)), "sum_j dV_j", tol_max=0.05, tol_mean=0.01)


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
    ws = torch.empty((fa.attn_bwd_workspace_bytes(B, Hq, Hkv, S, D, True),), dtype=torch.uint8, device="cuda")
    scale = 1.0 / math.sqrt(D)
    fa.attn_bwd_dq(tq, tk, tv, o, lse, tdo, dq, dk, dv, True, scale, ws)
    torch.cuda.synchronize()
    assert torch.isnan(dk).all() and torch.isnan(dv).all()   # stage 1 leaves dk, dv alone
    fa.attn_bwd_dkdv(tq, tk, tv, o, lse, tdo, dq, dk, dv, True, scale, ws)
    torch.cuda.synchronize()
    for x, y in zip((dq, dk, dv), ref):
        assert torch.equal(x, y)
