"""Forward parity on the GPU: the HIP kernel through the C ABI against the fp64 oracle."""
import math
import sys

import numpy as np
import pytest

import oracle
import flashattention_tiled_attention_amd as fa
from flashattention_tiled_attention_amd.inputs import CONFIGS, qkv
from tests.gpu_util import TOL_LSE, assert_close, bf16_dev_to_f64, f32_dev_to_f64, to_dev

pytestmark = pytest.mark.gpu


def run_fwd(q, k, v, causal, scale):
    import torch
    o, lse = fa.fwd(to_dev(q), to_dev(k), to_dev(v), causal=causal, scale=scale)
    torch.cuda.synchronize()
    return bf16_dev_to_f64(o), f32_dev_to_f64(lse)


def check_full(B, Hq, Hkv, S, D, causal, seed=0, scale=None):
    print("case B=%d Hq=%d Hkv=%d S=%d D=%d causal=%d seed=%d scale=%s" % (B, Hq, Hkv, S, D, causal, seed, scale),
          flush=True)
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    q, k, v = qkv(B, Hq, Hkv, S, D, seed)
    o, lse = run_fwd(q, k, v, causal, scale)
    o_ref, lse_ref = oracle.fwd(q, k, v, causal, scale)
    assert_close(o, o_ref, "O")
    assert_close(lse, lse_ref, "lse", tol_max=TOL_LSE, tol_mean=TOL_LSE)


def test_single_head_s128_d64():
    c = CONFIGS["single_head_s128_d64"]
    check_full(c["B"], c["Hq"], c["Hkv"], c["S"], c["D"], c["causal"], seed=0)


@pytest.mark.parametrize("S", [1, 2, 5, 63, 64, 65, 127, 128, 129, 200, 383])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_ragged_lengths(S, D, causal):
    check_full(1, 2, 1, S, D, causal, seed=S)


@pytest.mark.parametrize("Hq,Hkv", [(1, 1), (4, 2), (8, 2), (8, 1), (16, 16)])
def test_gqa_groups(Hq, Hkv):
    check_full(2, Hq, Hkv, 300, 128, True, seed=Hq * 10 + Hkv)


@pytest.mark.parametrize("B,Hq,Hkv,S,D,causal", [
    (2, 8, 2, 1024, 128, True),     # several tiles, GQA, (B*Hkv) % 8 != 0
    (1, 16, 8, 777, 128, True),     # groups spread over all 8 XCDs, ragged tail
    (3, 4, 4, 640, 64, False),
    (2, 8, 8, 1000, 64, True),
])
def test_multi_tile(B, Hq, Hkv, S, D, causal):
    check_full(B, Hq, Hkv, S, D, causal, seed=B + S)


@pytest.mark.parametrize("scale", [0.0, -0.0884, 0.5, -1.3])
def test_scales(scale):
    check_full(1, 4, 2, 257, 128, True, seed=3, scale=scale)
    check_full(1, 2, 2, 130, 64, False, seed=4, scale=scale)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("scale", [0.0, -0.0884, 0.0884])
def test_scales_one_wave_forward(scale, causal):
    """Scales the 64-rows-per-wave forward takes (128-wide heads, S a multiple of 256,
    |scale| sqrt(D) <= 2): zero (every probability equal) and negative (Q's sign flipped
    on load)."""
    check_full(1, 4, 2, 512, 128, causal, seed=5, scale=scale)


@pytest.mark.parametrize("B,Hq,Hkv,S,causal", [
    (1, 2, 1, 256, False),    # one query tile, four key tiles
    (1, 2, 1, 256, True),     # only the first causal tile: the exact body alone
    (2, 8, 2, 768, False),    # (B*Hkv) % 8 != 0: one group after another on each XCD
    (1, 16, 8, 512, False),   # groups dealt round-robin over the 8 XCDs
    (3, 4, 1, 1280, True),    # five query tiles, G = 4
])
def test_one_wave_forward_shapes(B, Hq, Hkv, S, causal):
    check_full(B, Hq, Hkv, S, 128, causal, seed=B * 7 + S)


@pytest.mark.parametrize("seed", [1, 2])
def test_seeds_small(seed):
    check_full(1, 8, 2, 512, 128, True, seed=seed)


@pytest.mark.parametrize("name", ["llama8b_causal_gqa_s4096", "mha_noncausal_s2048_d64"])
def test_full_size(name):
    """Full-size workloads in the launch configuration the benchmark times, every element
    of O and lse against the oracle's full forward."""
    c = CONFIGS[name]
    B, Hq, Hkv, S, D, causal = c["B"], c["Hq"], c["Hkv"], c["S"], c["D"], c["causal"]
    print("case %s (full tensors)" % name, flush=True)
    scale = 1.0 / math.sqrt(D)
    q, k, v = qkv(B, Hq, Hkv, S, D, 0)
    o, lse = run_fwd(q, k, v, causal, scale)
    o_ref, lse_ref = oracle.fwd(q, k, v, causal, scale)
    mx, mean = assert_close(o, o_ref, "O (all %d rows)" % (B * Hq * S))
    assert_close(lse, lse_ref, "lse", tol_max=TOL_LSE, tol_mean=TOL_LSE)
    print("O max-abs %.3e mean-abs %.3e" % (mx, mean), flush=True)


def test_full_size_long_sequence():
    """B=2, Hq=32, Hkv=8, S=8192, D=128 causal (1.1 TFLOP of fp64 oracle work in full):
    the GPU's whole output, checked on every 8th query row of each head (the residue
    moving from head to head, so every row position of a tile is covered) and on each
    head's last row; the forward is row-independent, so those rows are exact checks."""
    from tests.gpu_util import head_offset_rows
    c = CONFIGS["long_causal_gqa_s8192"]
    B, Hq, Hkv, S, D, causal = c["B"], c["Hq"], c["Hkv"], c["S"], c["D"], c["causal"]
    print("case long_causal_gqa_s8192 (every 8th row)", flush=True)
    scale = 1.0 / math.sqrt(D)
    q, k, v = qkv(B, Hq, Hkv, S, D, 0)
    o, lse = run_fwd(q, k, v, causal, scale)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    rows = head_offset_rows(B, Hq, S, 8)
    o_ref, lse_ref = oracle.fwd_rows(q, k, v, rows, causal, scale)
    mx, mean = assert_close(o.reshape(-1, D)[rows], o_ref, "O (%d rows)" % rows.size)
    assert_close(lse.reshape(-1)[rows], lse_ref, "lse", tol_max=TOL_LSE, tol_mean=TOL_LSE)
    print("O max-abs %.3e mean-abs %.3e" % (mx, mean), flush=True)


def test_deterministic():
    import torch
    q, k, v = qkv(1, 8, 2, 1024, 128, 5)
    dq, dk, dv = to_dev(q), to_dev(k), to_dev(v)
    o1, l1 = fa.fwd(dq, dk, dv, causal=True)
    o2, l2 = fa.fwd(dq, dk, dv, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1, l2)


def test_zero_query_gives_prefix_mean():
    """Closed form checked directly on GPU output: Q=0 gives the prefix mean of V."""
    B, H, S, D = 1, 2, 700, 128
    _, k, v = qkv(B, H, H, S, D, 9)
    q = np.zeros((B, H, S, D), np.uint16)
    o, lse = run_fwd(q, k, v, True, 0.0884)
    from flashattention_tiled_attention_amd.inputs import bf16_to_f32
    vf = bf16_to_f32(v).astype(np.float64)
    prefix = np.cumsum(vf, axis=2) / np.arange(1, S + 1)[None, None, :, None]
    assert_close(o, prefix, "Q=0 prefix mean")
    assert_close(lse, np.broadcast_to(np.log(np.arange(1, S + 1.0)), lse.shape), "Q=0 lse",
                 tol_max=TOL_LSE, tol_mean=TOL_LSE)


@pytest.mark.parametrize("D,S", [(128, 512), (64, 300)])
@pytest.mark.parametrize("causal", [False, True])
def test_nan_key_reaches_exactly_the_rows_that_see_it(D, S, causal):
    """A NaN in one key makes every score against it NaN, so softmax gives NaN O and lse
    on exactly the rows that see that key (all rows; with a causal mask those at or
    past it) and leaves the other rows as they were. For 128-wide heads the NaN fails
    the one-wave forward's bound test, and the workgroup's rows are made again on the
    exact path."""
    from flashattention_tiled_attention_amd.inputs import bf16_bits, bf16_to_f32
    B, Hq, Hkv, t = 1, 4, 2, 100
    print("case nan key D=%d S=%d causal=%d" % (D, S, causal), flush=True)
    q, k, v = qkv(B, Hq, Hkv, S, D, 17)
    kf = bf16_to_f32(k)
    kf[0, 1, t, 5] = np.nan          # key t of kv head 1: query heads 2 and 3 see it
    k = bf16_bits(kf)
    scale = 1.0 / math.sqrt(D)
    o, lse = run_fwd(q, k, v, causal, scale)
    o_ref, lse_ref = oracle.fwd(q, k, v, causal, scale)
    rows = np.arange(S)
    sees = np.zeros((B, Hq, S), bool)
    sees[0, 2:] = (rows >= t) if causal else True
    assert np.array_equal(np.isnan(lse_ref), sees), "the oracle's NaN rows"
    assert np.array_equal(np.isnan(lse), sees), "NaN lse on exactly the rows that see the key"
    assert np.array_equal(np.isnan(o).all(axis=-1), sees) and not np.isnan(o[~sees]).any(), "NaN O rows"
    assert_close(o[~sees], o_ref[~sees], "O")
    assert_close(lse[~sees], lse_ref[~sees], "lse", tol_max=TOL_LSE, tol_mean=TOL_LSE)


@pytest.mark.parametrize("mode", ["mild", "spike", "ramp"])
@pytest.mark.parametrize("causal", [False, True])
def test_reference_maximum_of_the_first_tile(mode, causal):
    """128-wide heads with S a multiple of 256 take the kernel whose loop keeps each
    row's maximum from its first key tile and never rescales O. Later keys far above
    it (spike: about 40 log2 units; ramp: key norms growing fourfold) push a lane's
    probability sum past its bound, and the workgroup recomputes its rows on the exact
    path; a mild spike (5 to 8 units) stays on the loop with probabilities up to
    about 2^8. Both must match the definition."""
    from flashattention_tiled_attention_amd.inputs import bf16_bits, bf16_to_f32
    B, Hq, Hkv, S, D = 1, 4, 2, 768, 128
    print("case mode=%s causal=%d S=%d" % (mode, causal, S), flush=True)
    q, k, v = qkv(B, Hq, Hkv, S, D, 13)
    qf, kf = bf16_to_f32(q), bf16_to_f32(k)
    if mode == "ramp":
        kf = kf * (1.0 + 3.0 * np.arange(S, dtype=np.float32) / S)[None, None, :, None]
    else:
        qf = qf + 1.0
        for t in (300, 650):
            kf[:, :, t, :] = 2.5 if mode == "spike" else 0.6
    q, k, v = bf16_bits(qf), bf16_bits(kf), bf16_bits(bf16_to_f32(v) * 0.5)
    scale = 1.0 / math.sqrt(D)
    o, lse = run_fwd(q, k, v, causal, scale)
    o_ref, lse_ref = oracle.fwd(q, k, v, causal, scale)
    assert_close(o, o_ref, "O")
    assert_close(lse, lse_ref, "lse", tol_max=TOL_LSE, tol_mean=TOL_LSE)


@pytest.mark.parametrize("mode", ["ramp", "spike"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal,window", [(False, 0), (True, 0), (True, 100), (True, 300)])
def test_row_maximum_moving_after_the_first_tile(mode, D, causal, window):
    """Rows whose maximum keeps growing, or jumps, after their first key tile: past a
    wave's first tile the forward takes the row maximum only when the tile's
    probabilities against the running maximum sum past a bound, so these inputs
    drive both the skipped and the full step, and the O rescale."""
    from flashattention_tiled_attention_amd.inputs import bf16_bits, bf16_to_f32
    B, Hq, Hkv, S = 1, 4, 2, 700
    print("case mode=%s D=%d causal=%d window=%d S=%d" % (mode, D, causal, window, S), flush=True)
    q, k, v = qkv(B, Hq, Hkv, S, D, 11)
    qf, kf = bf16_to_f32(q), bf16_to_f32(k)
    if mode == "ramp":   # key norms grow fourfold along the sequence
        kf = kf * (1.0 + 3.0 * np.arange(S, dtype=np.float32) / S)[None, None, :, None]
    else:                # queries share a direction that two late keys point along
        qf = qf + 1.0
        for t in (300, 650):
            kf[:, :, t, :] = 2.5
    # halved values keep |O| below 4 where a row is dominated by one or two keys: the
    # bf16 store of O alone costs up to 2^-6 at |O| >= 4, more than the bar
    q, k, v = bf16_bits(qf), bf16_bits(kf), bf16_bits(bf16_to_f32(v) * 0.5)
    scale = 1.0 / math.sqrt(D)
    if window:   # the sliding-window kernel (several query heads per workgroup)
        import torch
        o, lse = fa.fwd(to_dev(q), to_dev(k), to_dev(v), causal=True, scale=scale, window=window)
        torch.cuda.synchronize()
        o, lse = bf16_dev_to_f64(o), f32_dev_to_f64(lse)
    else:
        o, lse = run_fwd(q, k, v, causal, scale)
    o_ref, lse_ref = oracle.fwd(q, k, v, causal, scale, window)
    assert_close(o, o_ref, "O")
    assert_close(lse, lse_ref, "lse", tol_max=TOL_LSE, tol_mean=TOL_LSE)
