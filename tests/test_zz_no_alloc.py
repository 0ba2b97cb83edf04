"""attn_bwd_noalloc (the backward with the library's static per-GPU scratch as its
workspace) against attn_bwd with a caller-allocated workspace, through the C ABI: two
calls in a row, the second on a smaller problem, each bit-equal to attn_bwd."""
import math

import pytest

import flashattention_tiled_attention_amd as fa
from flashattention_tiled_attention_amd.inputs import qkv
from tests.gpu_util import to_dev

pytestmark = pytest.mark.gpu


def check(B, Hq, Hkv, S, D, causal, seed):
    import torch
    print("case attn_bwd_noalloc B=%d Hq=%d Hkv=%d S=%d D=%d causal=%d" % (B, Hq, Hkv, S, D, causal), flush=True)
    scale = 1.0 / math.sqrt(D)
    q, k, v, do = qkv(B, Hq, Hkv, S, D, seed, with_dout=True)
    tq, tk, tv, tdo = to_dev(q), to_dev(k), to_dev(v), to_dev(do)
    o, lse = fa.fwd(tq, tk, tv, causal=causal, scale=scale)
    ref = fa.bwd(tq, tk, tv, o, lse, tdo, causal=causal, scale=scale)
    got = [torch.full_like(r, float("nan")) for r in ref]
    fa.attn_bwd_noalloc(tq, tk, tv, o, lse, tdo, got[0], got[1], got[2], causal, scale)
    torch.cuda.synchronize()
    for g, r, what in zip(got, ref, ("dQ", "dK", "dV")):
        assert torch.equal(g, r), what


def test_noalloc_matches_attn_bwd_twice():
    # the first call fills more of the scratch than the second needs: the second
    # must not depend on what the first left behind
    check(2, 16, 4, 1500, 128, True, seed=41)
    check(1, 4, 2, 333, 64, False, seed=42)


def test_noalloc_at_the_workload_shape():
    check(1, 32, 8, 4096, 128, True, seed=0)
