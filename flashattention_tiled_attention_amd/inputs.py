"""Seeded synthetic inputs shared by the tests, the benchmark and the oracle checks.

This module holds no attention arithmetic: only the random draw and the
float32 -> bf16 encoding. Recipe: ``numpy.random.default_rng(seed)`` (PCG64),
``standard_normal(shape, dtype=float32)`` drawn in the order Q, K, V, dO, each
over its whole contiguous [B][H][S][D] tensor, then rounded to bf16 with
round-to-nearest-even on the bit pattern.
"""
import numpy as np


def bf16_bits(x):
    """float32 array -> uint16 bf16 bit patterns, round to nearest even (NaN stays NaN)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    nan = np.isnan(x)
    out = rounded.astype(np.uint16)
    if nan.any():
        out[nan] = ((u[nan] >> 16) | 0x40).astype(np.uint16)
    return out


def bf16_to_f32(bits):
    """uint16 bf16 bit patterns -> float32 (exact)."""
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32)


def qkv(B, Hq, Hkv, S, D, seed=0, with_dout=False, Dv=None):
    """Q [B,Hq,S,D], K [B,Hkv,S,D], V [B,Hkv,S,Dv] (and dO [B,Hq,S,Dv]) as bf16 bits,
    iid N(0,1). Dv (the value head dimension) defaults to D."""
    Dv = D if Dv is None else Dv
    rng = np.random.default_rng(seed)
    q = bf16_bits(rng.standard_normal((B, Hq, S, D), dtype=np.float32))
    k = bf16_bits(rng.standard_normal((B, Hkv, S, D), dtype=np.float32))
    v = bf16_bits(rng.standard_normal((B, Hkv, S, Dv), dtype=np.float32))
    if not with_dout:
        return q, k, v
    dout = bf16_bits(rng.standard_normal((B, Hq, S, Dv), dtype=np.float32))
    return q, k, v, dout


def sparse_qkv(B, Hq, Hkv, S, N, D, seed=0, with_dout=False):
    """Q [B,Hq,S,D], K and V [B,Hkv,N,D] over N key/value rows (and dO like Q), as bf16
    bits, iid N(0,1), drawn in the order Q, K, V, dO."""
    rng = np.random.default_rng(seed)
    q = bf16_bits(rng.standard_normal((B, Hq, S, D), dtype=np.float32))
    k = bf16_bits(rng.standard_normal((B, Hkv, N, D), dtype=np.float32))
    v = bf16_bits(rng.standard_normal((B, Hkv, N, D), dtype=np.float32))
    if not with_dout:
        return q, k, v
    dout = bf16_bits(rng.standard_normal((B, Hq, S, D), dtype=np.float32))
    return q, k, v, dout


def csa_index_lists(B, S, window, ratio, pool_topk, seed=0):
    """Per-token key/value row lists shaped like the compressed sparse attention of
    Table 7 (window + top-k of a compressed pool), with random picks standing in for a
    trained indexer. Rows 0..S-1 are the raw tokens, rows S .. S + S//ratio - 1 the
    pool. Token i lists its window rows max(0, i-window+1) .. i in ascending order, then
    min(pool_topk, P_i) pool rows drawn uniformly without replacement (in draw order)
    from the P_i = (i+1)//ratio pool rows whose block of `ratio` tokens ends at or
    before i; unused slots are -1. Returns (idx int32 [B][S][window+pool_topk], N)."""
    rng = np.random.default_rng(seed)
    npool = S // ratio if ratio else 0
    topk = window + (pool_topk if ratio else 0)
    idx = np.full((B, S, topk), -1, dtype=np.int32)
    for b in range(B):
        for i in range(S):
            w0 = max(0, i - window + 1)
            idx[b, i, :i - w0 + 1] = np.arange(w0, i + 1, dtype=np.int32)
            if ratio:
                vis = min((i + 1) // ratio, npool)
                m = min(pool_topk, vis)
                if m:
                    idx[b, i, window:window + m] = S + rng.choice(vis, size=m, replace=False)
    return idx, S + npool


# The workloads the benchmark and the parity tests run: (name, B, Hq, Hkv, S, D, causal, pass;
# optional window and value head dimension Dv, which defaults to D).
CONFIGS = {
    "single_head_s128_d64": dict(B=1, Hq=1, Hkv=1, S=128, D=64, causal=False, bwd=False),
    "llama8b_causal_gqa_s4096": dict(B=1, Hq=32, Hkv=8, S=4096, D=128, causal=True, bwd=False),
    "long_causal_gqa_s8192": dict(B=2, Hq=32, Hkv=8, S=8192, D=128, causal=True, bwd=False),
    "mha_noncausal_s2048_d64": dict(B=8, Hq=16, Hkv=16, S=2048, D=64, causal=False, bwd=False),
    "llama8b_causal_gqa_s4096_bwd": dict(B=1, Hq=32, Hkv=8, S=4096, D=128, causal=True, bwd=True),
    # causal sliding window of 128 keys (the window of the compressed sparse attention, Table 7)
    "llama8b_window128_s4096": dict(B=1, Hq=32, Hkv=8, S=4096, D=128, causal=True, window=128, bwd=True),
    # value head dimension d_v != d (Eq. 1): 128-wide queries/keys, 64-wide values
    "gqa_dqk128_dv64_s4096": dict(B=1, Hq=32, Hkv=8, S=4096, D=128, Dv=64, causal=True, bwd=True),
    # index-gather sparse attention in the cr4 shape of the compressed sparse attention
    # (Table 7, "Flash" family: 64 heads, top-k 640 = 128-token window + top-512 of S/4
    # pool rows), one K/V head shared by all query heads, synthetic lists
    "csa_cr4_flash_s4096": dict(B=1, Hq=64, Hkv=1, S=4096, D=128, causal=False, sparse=True, window=128,
                                ratio=4, pool_topk=512, bwd=True),
    # the cr128 shape (window + every visible row of an S/128 pool) and the cr4 "Pro"
    # shape (128 heads, window + top-1024 of S/4 pool rows), same recipe
    "csa_cr128_flash_s4096": dict(B=1, Hq=64, Hkv=1, S=4096, D=128, causal=False, sparse=True, window=128,
                                  ratio=128, pool_topk=32, bwd=True),
    "csa_cr4_pro_s4096": dict(B=1, Hq=128, Hkv=1, S=4096, D=128, causal=False, sparse=True, window=128,
                              ratio=4, pool_topk=1024, bwd=True),
}
