"""Sparse attention over per-token index lists on the GPU (attn_sparse_fwd /
attn_sparse_bwd through the C ABI) against the fp64 oracle with the same lists."""
import math

import numpy as np
import pytest

import oracle
import flashattention_tiled_attention_amd as fa
from flashattention_tiled_attention_amd.inputs import CONFIGS, bf16_to_f32, csa_index_lists, sparse_qkv
from tests.gpu_util import TOL_LSE, assert_close, bf16_dev_to_f64, f32_dev_to_f64, sample_rows, to_dev

pytestmark = pytest.mark.gpu


def to_dev_idx(idx):
    import torch
    return torch.from_numpy(np.ascontiguousarray(idx, dtype=np.int32)).to("cuda")


def run(q, k, v, idx, do, scale):
    import torch
    tq, tk, tv, ti = to_dev(q), to_dev(k), to_dev(v), to_dev_idx(idx)
    o, lse = fa.sparse_fwd(tq, tk, tv, ti, scale)
    grads = None
    if do is not None:
        grads = fa.sparse_bwd(tq, tk, tv, ti, o, lse, to_dev(do), scale)
    torch.cuda.synchronize()
    out = [bf16_dev_to_f64(o), f32_dev_to_f64(lse)]
    if grads is not None:
        out += [f32_dev_to_f64(g) for g in grads]
    return out


def random_lists(B, S, N, topk, seed, empty_frac=0.2, dup=True, empty_tokens=()):
    """Random lists with empty slots (-1 and out-of-range entries), optional repeats."""
    rng = np.random.default_rng(seed)
    idx = rng.integers(0, N, size=(B, S, topk)).astype(np.int32)
    if not dup:
        for b in range(B):
            for i in range(S):
                idx[b, i] = rng.choice(N, size=topk, replace=False) if topk <= N else idx[b, i]
    holes = rng.random((B, S, topk)) < empty_frac
    idx[holes] = np.where(rng.random(int(holes.sum())) < 0.5, -1, N + 3)
    for t in empty_tokens:
        idx[:, t] = -1
    return idx


def check(q, k, v, idx, do, scale, what):
    print("case %s q=%s k=%s topk=%d scale=%s" % (what, q.shape, k.shape, idx.shape[2], scale), flush=True)
    got = run(q, k, v, idx, do, scale)
    o_ref, lse_ref = oracle.sparse_fwd(q, k, v, idx, scale)
    assert_close(got[0], o_ref, "O")
    fin = np.isfinite(lse_ref)
    assert np.array_equal(np.isneginf(got[1]), ~fin), "lse = -inf exactly for tokens with empty lists"
    assert_close(got[1][fin], lse_ref[fin], "lse", tol_max=TOL_LSE, tol_mean=TOL_LSE)
    if do is not None:
        rq, rk, rv = oracle.sparse_bwd(q, k, v, do, idx, scale)
        assert_close(got[2], rq, "dQ")
        assert_close(got[3], rk, "dK")
        assert_close(got[4], rv, "dV")


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("Hq,Hkv", [(1, 1), (4, 2), (64, 1), (100, 1), (128, 1)])
def test_random_lists(D, Hq, Hkv):
    B, S, N, topk = 2, 40, 150, 70
    q, k, v, do = sparse_qkv(B, Hq, Hkv, S, N, D, seed=Hq + D, with_dout=True)
    idx = random_lists(B, S, N, topk, seed=Hq * 3 + D, empty_tokens=(0, 17))
    check(q, k, v, idx, do, 1.0 / math.sqrt(D), "random G=%d D=%d" % (Hq // Hkv, D))


# 1..300, then one length in each range of the inverse map's per-thread entry counts
# (up to 512, 1024, 2048 and the 4096 maximum; rows repeat within a list once topk > N)
@pytest.mark.parametrize("topk", [1, 2, 31, 32, 33, 64, 129, 300, 600, 1100, 2100, 4096])
def test_list_lengths(topk):
    B, Hq, Hkv, S, N, D = 1, 8, 2, 30, 400, 128
    q, k, v, do = sparse_qkv(B, Hq, Hkv, S, N, D, seed=topk, with_dout=True)
    idx = random_lists(B, S, N, topk, seed=topk + 1, empty_frac=0.1, empty_tokens=(3,))
    check(q, k, v, idx, do, 1.0 / math.sqrt(D), "topk=%d" % topk)


# The inverse map keeps a chunk's per-row counters in LDS up to N = 16384 rows and
# in global memory beyond: both sides of that boundary.
@pytest.mark.parametrize("N", [16384, 16385, 20000])
def test_many_rows(N):
    B, Hq, Hkv, S, D, topk = 1, 4, 1, 40, 128, 200
    q, k, v, do = sparse_qkv(B, Hq, Hkv, S, N, D, seed=N % 1000, with_dout=True)
    idx = random_lists(B, S, N, topk, seed=N % 997, empty_frac=0.1)
    idx[0, :8, :64] = np.arange(64, dtype=np.int32)  # shared rows: several tokens per row
    check(q, k, v, idx, do, 1.0 / math.sqrt(D), "N=%d" % N)


def test_chunked_work_order_batches_and_kv_heads():
    """2 batches x 2 kv heads x 512 tokens: the item count divides into whole rounds of
    64-token chunks over the 8 XCDs, so the forward, dQ and partial kernels take the
    chunked order with more than one item per token."""
    B, Hq, Hkv, S, N, D, topk = 2, 8, 2, 512, 640, 128, 96
    q, k, v, do = sparse_qkv(B, Hq, Hkv, S, N, D, seed=21, with_dout=True)
    idx = random_lists(B, S, N, topk, seed=22, empty_frac=0.15, empty_tokens=(5, 300))
    check(q, k, v, idx, do, 1.0 / math.sqrt(D), "chunked order B=2 Hkv=2 S=512")


def test_all_empty_and_single_slot():
    B, Hq, Hkv, S, N, D = 1, 64, 1, 12, 50, 128
    q, k, v, do = sparse_qkv(B, Hq, Hkv, S, N, D, seed=7, with_dout=True)
    idx = np.full((B, S, 9), -1, dtype=np.int32)
    idx[0, 1, 4] = 7          # one key
    idx[0, 2, :] = 7          # the same key nine times
    idx[0, 3, [0, 8]] = [3, 49]
    check(q, k, v, idx, do, 1.0 / math.sqrt(D), "mostly empty")


@pytest.mark.parametrize("scale", [0.0, -0.0884, 0.5, -1.3])
def test_scales(scale):
    B, Hq, Hkv, S, N, D = 1, 16, 2, 25, 90, 128
    q, k, v, do = sparse_qkv(B, Hq, Hkv, S, N, D, seed=11, with_dout=True)
    idx = random_lists(B, S, N, 80, seed=12)
    check(q, k, v, idx, do, scale, "scale")


@pytest.mark.parametrize("D", [64, 128])
def test_csa_lists_small(D):
    """Lists of the compressed-sparse-attention shape (window + top-k of a pool of S/4
    rows), at a size the full oracle handles."""
    B, Hq, Hkv, S = 1, 64, 1, 300
    idx, N = csa_index_lists(B, S, window=64, ratio=4, pool_topk=48, seed=13)
    q, k, v, do = sparse_qkv(B, Hq, Hkv, S, N, D, seed=14, with_dout=True)
    check(q, k, v, idx, do, 1.0 / math.sqrt(D), "csa small D=%d" % D)


def test_multi_head_groups_and_batches():
    B, Hq, Hkv, S = 2, 32, 4, 200
    idx, N = csa_index_lists(B, S, window=32, ratio=4, pool_topk=40, seed=15)
    q, k, v, do = sparse_qkv(B, Hq, Hkv, S, N, 128, seed=16, with_dout=True)
    check(q, k, v, idx, do, 1.0 / math.sqrt(128), "batches x groups")


def test_deterministic():
    import torch
    B, Hq, Hkv, S = 1, 64, 1, 512
    idx, N = csa_index_lists(B, S, window=128, ratio=4, pool_topk=64, seed=17)
    q, k, v, do = sparse_qkv(B, Hq, Hkv, S, N, 128, seed=18, with_dout=True)
    tq, tk, tv, ti, tdo = to_dev(q), to_dev(k), to_dev(v), to_dev_idx(idx), to_dev(do)
    o, lse = fa.sparse_fwd(tq, tk, tv, ti)
    a = fa.sparse_bwd(tq, tk, tv, ti, o, lse, tdo)
    b = fa.sparse_bwd(tq, tk, tv, ti, o, lse, tdo)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


@pytest.mark.parametrize("name", ["csa_cr4_flash_s4096", "csa_cr128_flash_s4096", "csa_cr4_pro_s4096"])
def test_full_size_csa_sampled(name):
    """The compressed-sparse-attention shapes at S=4096 (cr4 "Flash": 64 query heads on one
    K/V head, a 128-token window plus top-512 of 1024 pool rows; cr128: the window plus
    every visible row of a 32-row pool; cr4 "Pro": 128 heads, top-1024): O/lse and dQ on
    sampled rows, dK/dV on sampled window and pool rows, plus sum_j dV_j = sum of dO and
    sum_j dK_j = 0."""
    c = CONFIGS[name]
    B, Hq, Hkv, S, D = c["B"], c["Hq"], c["Hkv"], c["S"], c["D"]
    idx, N = csa_index_lists(B, S, c["window"], c["ratio"], c["pool_topk"], seed=0)
    print("case full-size %s B=%d Hq=%d Hkv=%d S=%d N=%d D=%d topk=%d"
          % (name, B, Hq, Hkv, S, N, D, idx.shape[2]), flush=True)
    q, k, v, do = sparse_qkv(B, Hq, Hkv, S, N, D, seed=0, with_dout=True)
    scale = 1.0 / math.sqrt(D)
    o, lse, dq, dk, dv = run(q, k, v, idx, do, scale)
    rows = sample_rows(B, Hq, S, 200, seed=8)
    ro, rl = oracle.sparse_fwd(q, k, v, idx, scale, rows=rows)
    assert_close(o.reshape(-1, D)[rows], ro, "O (%d sampled rows)" % rows.size)
    assert_close(lse.reshape(-1)[rows], rl, "lse", tol_max=TOL_LSE, tol_mean=TOL_LSE)
    rng = np.random.default_rng(9)
    keys = sorted(set([0, 1, 127, 128, S - 1, S, S + 1, N - 1]) | set(int(x) for x in rng.integers(0, N, 24)))
    kvrows = np.array(keys, dtype=np.int64)
    print("oracle backward on %d sampled rows, %d sampled keys" % (rows.size, kvrows.size), flush=True)
    rq, rk, rv = oracle.sparse_bwd(q, k, v, do, idx, scale, qrows=rows, kvrows=kvrows)
    assert_close(dq.reshape(-1, D)[rows], rq, "dQ (%d sampled rows)" % rows.size)
    assert_close(dk.reshape(-1, D)[kvrows], rk, "dK (%d sampled keys)" % kvrows.size)
    assert_close(dv.reshape(-1, D)[kvrows], rv, "dV (%d sampled keys)" % kvrows.size)
    # Invariants over the whole output, a check for gross errors of the inverse map (a
    # misplaced chunk moves these sums by O(1) or more). Their rounding noise: each of
    # the 262144 (524288) query rows carries P rounded to bf16, so sum_s P differs from 1 by
    # about 2^-9/sqrt(3) * sqrt(sum_s P^2), roughly 1e-4 for 100-200 keys; summed over
    # the rows against unit-variance dO that is about 0.05 per element (0.1 with 128 heads).
    dof = bf16_to_f32(do).astype(np.float64)
    assert_close(dv.sum(axis=2), dof.reshape(B, Hkv, Hq // Hkv, S, D).sum(axis=(2, 3)), "sum_j dV_j",
                 tol_max=0.5, tol_mean=0.15)
    assert_close(dk.sum(axis=2), np.zeros((B, Hkv, D)), "sum_j dK_j", tol_max=0.5, tol_mean=0.15)


@pytest.mark.parametrize("mode", ["ramp", "spike"])
@pytest.mark.parametrize("D", [64, 128])
def test_row_maximum_moving_after_the_first_tile(mode, D):
    """Lists whose later slots score far above their first 32: past a row block's first
    tile the sparse forward takes the row maximum only when the probabilities against
    the running maximum sum past a bound, so these lists drive both the skipped and
    the full step, and the O rescale. Values are halved to keep |O| where the bf16
    store of O stays within the bar."""
    from flashattention_tiled_attention_amd.inputs import bf16_bits
    B, Hq, Hkv, S, N, topk = 1, 4, 1, 48, 400, 300
    q, k, v = sparse_qkv(B, Hq, Hkv, S, N, D, seed=21 + D)[:3]
    qf, kf = bf16_to_f32(q), bf16_to_f32(k)
    idx = np.tile(np.arange(topk, dtype=np.int32)[None, None, :], (B, S, 1))  # slot j lists row j
    if mode == "ramp":   # row norms grow fourfold along the slots
        kf[:, :, :topk] *= (1.0 + 3.0 * np.arange(topk, dtype=np.float32) / topk)[None, None, :, None]
    else:                # queries share a direction that two late rows point along
        qf = qf + 1.0
        for r in (150, 290):
            kf[:, :, r, :] = 2.5
    q, k, v = bf16_bits(qf), bf16_bits(kf), bf16_bits(bf16_to_f32(v) * 0.5)
    check(q, k, v, idx, None, 1.0 / math.sqrt(D), "max moving %s D=%d" % (mode, D))


@pytest.mark.parametrize("mode", ["ramp", "spike", "wide"])
@pytest.mark.parametrize("D", [64, 128])
def test_peaked_rows_backward(mode, D):
    """The sparse backward on lists whose rows put most of their weight on one or a few
    slots at the usual scale 1/sqrt(D) (the inputs of the dense test of the same name):
    growing row norms along the pool, two pool rows every query points at, and inputs of
    standard deviation 2.5. Lists are the compressed-attention shape (a 128-token window
    plus up to 256 pool rows): tokens past 515 list more than 256 rows, beyond which the
    sparse kernels leave the exact path to the data."""
    from tests.gpu_util import peaked
    B, Hq, Hkv, S = 1, 16, 1, 1200
    idx, N = csa_index_lists(B, S, window=128, ratio=4, pool_topk=256, seed=23)
    assert (idx >= 0).sum(axis=2).max() > 256
    q, k, v, do = sparse_qkv(B, Hq, Hkv, S, N, D, seed=24 + D, with_dout=True)
    q, k, v = peaked(q, k, v, mode, spike_rows=(S + 10, S + 140))
    check(q, k, v, idx, do, 1.0 / math.sqrt(D), "peaked backward %s D=%d" % (mode, D))
