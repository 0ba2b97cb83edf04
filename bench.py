"""Benchmark of the MI355X attention hot path; prints one JSON line.

A step is one pass of the whole hot path over one batch of synthetic input:
the forward kernel (O, lse) and the backward kernels (delta, dK/dV, dQ) on the
Llama-3.1-8B-shaped causal GQA workload B=1, Hq=32, Hkv=8, S=4096, D=128,
inputs resident in HBM. FLOP convention: forward 4*B*Hq*S^2*D (halved when
causal), backward 2.5x the forward; softmax and exp work is not counted.

    python bench.py [--gpus 1] [--steps K] [--warmup W]
"""
import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # 256 CU x 4096 dense bf16 flop/clk x 2.4 GHz
WORKLOAD = "llama8b_causal_gqa_s4096"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def fwd_flops(B, Hq, S, D, causal):
    f = 4.0 * B * Hq * S * S * D
    return f / 2 if causal else f


def cpu_baseline(q, k, v, dout, cfg, target_s, with_bwd):
    """Time the fp64 oracle (as it stands) on a bounded sample of the workload's query
    rows (forward) and key rows (backward); scale to TFLOP/s of the same convention."""
    import numpy as np
    import oracle
    B, Hq, Hkv, S, D, causal = cfg["B"], cfg["Hq"], cfg["Hkv"], cfg["S"], cfg["D"], cfg["causal"]
    scale = 1.0 / math.sqrt(D)
    rng = np.random.default_rng(123)

    def row_flops(rows):
        i = rows % S
        n = (i + 1) if causal else np.full_like(i, S)
        return float(np.sum(4.0 * n * D))

    # calibrate on a small sample, then size the timed sample to ~target_s
    cal = rng.integers(0, B * Hq * S, size=64)
    t = time.perf_counter()
    oracle.fwd_rows(q, k, v, cal, causal, scale)
    per_flop = (time.perf_counter() - t) / row_flops(cal)
    budget = target_s * (0.5 if with_bwd else 1.0)
    n = int(min(B * Hq * S, max(64, budget / per_flop / (row_flops(cal) / cal.size))))
    rows = rng.choice(B * Hq * S, size=n, replace=False)
    t = time.perf_counter()
    oracle.fwd_rows(q, k, v, rows, causal, scale)
    t_f = time.perf_counter() - t
    flops, secs = row_flops(rows), t_f
    sample = "forward: %d of %d query rows (uniform without replacement)" % (n, B * Hq * S)
    if with_bwd:
        # one group's key rows: the group's per-row statistics plus dK/dV of sampled keys
        nk = 64
        keys = np.sort(rng.choice(S, size=nk, replace=False)).astype(np.int64)
        t = time.perf_counter()
        oracle.bwd_rows(q, k, v, dout, np.zeros(0, np.int64), keys, causal, scale)
        t_b = time.perf_counter() - t
        G = Hq // Hkv
        stat_flops = G * row_flops(np.arange(S, dtype=np.int64))           # S, P and dP rows of the group
        key_flops = float(np.sum(G * 8.0 * D * ((S - keys) if causal else S)))
        # the group's statistics are counted as work at the forward rate; their time is in t_b
        flops += stat_flops + key_flops
        secs += t_b
        sample += "; backward: row statistics of 1 of %d kv groups + dK/dV of %d of its %d keys" % (
            B * Hkv, nk, S)
    return {"value": flops / secs / 1e12, "unit": "TFLOP/s", "cores": oracle.num_threads(),
            "kind": "oracle", "sample": sample, "seconds": round(secs, 2)}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--fwd-only", action="store_true", help="time the forward kernel alone")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py runs on exactly one GPU: this build has no multi-GPU path "
              "(sharding is described in DESIGN.md); use --gpus 1", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import flashattention_tiled_attention_amd as fa
    from flashattention_tiled_attention_amd.inputs import CONFIGS, qkv
    from tests.gpu_util import to_dev

    cfg = CONFIGS[WORKLOAD]
    B, Hq, Hkv, S, D, causal = cfg["B"], cfg["Hq"], cfg["Hkv"], cfg["S"], cfg["D"], cfg["causal"]
    scale = 1.0 / math.sqrt(D)
    q, k, v, dout = qkv(B, Hq, Hkv, S, D, seed=0, with_dout=True)
    dq_, dk_, dv_, ddo = to_dev(q), to_dev(k), to_dev(v), to_dev(dout)
    o = torch.empty((B, Hq, S, D), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, Hq, S), dtype=torch.float32, device="cuda")
    gq = torch.empty((B, Hq, S, D), dtype=torch.float32, device="cuda")
    gk = torch.empty((B, Hkv, S, D), dtype=torch.float32, device="cuda")
    gv = torch.empty((B, Hkv, S, D), dtype=torch.float32, device="cuda")
    ws = torch.empty((fa.attn_bwd_workspace_bytes(B, Hq, Hkv, S, D, causal),), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()

    fa.attn_fwd(dq_, dk_, dv_, o, lse, causal, scale)
    with_bwd = not args.fwd_only
    if with_bwd:
        try:
            fa.attn_bwd(dq_, dk_, dv_, o, lse, ddo, gq, gk, gv, causal, scale, ws)
        except fa.AttnError as e:
            log("backward unavailable (%s): timing the forward only" % e)
            with_bwd = False
    torch.cuda.synchronize()

    def step():
        fa.attn_fwd(dq_, dk_, dv_, o, lse, causal, scale, stream)
        if with_bwd:
            fa.attn_bwd(dq_, dk_, dv_, o, lse, ddo, gq, gk, gv, causal, scale, ws, stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps

    # Per-kernel launch durations, with HIP events on the stream the kernels run on.
    def time_calls(fn, n):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(n):
            fn()
        e1.record(stream)
        e1.synchronize()
        return e0.elapsed_time(e1) / n

    n_rep = max(args.steps, 10)
    fwd_ms = time_calls(lambda: fa.attn_fwd(dq_, dk_, dv_, o, lse, causal, scale, stream), n_rep)
    bwd_ms = None
    if with_bwd:
        bwd_ms = time_calls(lambda: fa.attn_bwd(dq_, dk_, dv_, o, lse, ddo, gq, gk, gv, causal, scale, ws,
                                                stream), n_rep)

    f_fwd = fwd_flops(B, Hq, S, D, causal)
    f_bwd = 2.5 * f_fwd
    step_flops = f_fwd + (f_bwd if with_bwd else 0.0)
    value = step_flops / (ms_per_step * 1e-3) / 1e12
    fwd_tflops = f_fwd / (fwd_ms * 1e-3) / 1e12

    roofline = {"bound": "mfma", "kernel": "fwd_kernel<128,causal>", "achieved": round(fwd_tflops, 2),
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(fwd_tflops / PEAK_BF16_TFLOPS, 4),
                "traffic": None, "flop_per_launch": f_fwd, "launch_ms": round(fwd_ms, 4)}

    result = {
        "metric": "attention fwd/bwd TFLOP/s and % of bf16 MFMA peak on 1 MI355X",
        "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": WORKLOAD + ("" if with_bwd else "_fwd_only"), "B": B, "Hq": Hq, "Hkv": Hkv,
                   "S": S, "D": D, "causal": bool(causal), "pass": "fwd+bwd" if with_bwd else "fwd",
                   "seed": 0},
        "frac_of_peak": round(value / PEAK_BF16_TFLOPS, 4),
        "fwd": {"tflops": round(fwd_tflops, 2), "ms": round(fwd_ms, 4),
                "frac_of_peak": round(fwd_tflops / PEAK_BF16_TFLOPS, 4)},
        "roofline": roofline,
    }
    if with_bwd:
        bwd_tflops = f_bwd / (bwd_ms * 1e-3) / 1e12
        result["bwd"] = {"tflops": round(bwd_tflops, 2), "ms": round(bwd_ms, 4),
                         "frac_of_peak": round(bwd_tflops / PEAK_BF16_TFLOPS, 4)}
    if not args.no_cpu_baseline:
        log("timing the oracle on a bounded sample (~%.0f s)" % args.cpu_seconds)
        result["cpu_baseline"] = cpu_baseline(q, k, v, dout, cfg, args.cpu_seconds, with_bwd)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
