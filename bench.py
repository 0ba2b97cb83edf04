"""Benchmark of the MI355X attention hot path; prints one JSON line.

A step is one pass of the whole hot path over one batch of synthetic input:
the forward kernel (O, lse) and the backward kernels (delta, dK/dV, dQ) on the
Llama-3.1-8B-shaped causal GQA workload B=1, Hq=32, Hkv=8, S=4096, D=128,
inputs resident in HBM. FLOP convention, per visible (query, key) pair of a
head (S^2, S^2/2 when causal, S*W - W(W-1)/2 for a causal window of W keys):
forward 2*D (Q K^T) + 2*Dv (P V), backward 2*D (recomputed scores) + 2*Dv
(dO V^T) + 2*Dv (P^T dO) + 2*D (dS K) + 2*D (dS^T Q), which is 2.5x the forward
when Dv = D; softmax and exp work is not counted.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--fwd-only]

--workload picks another entry of inputs.CONFIGS (the default is the headline
workload above); a config with a "window" runs attn_fwd_window/attn_bwd_window,
one with a value head dimension "Dv" other than D runs attn_fwd_vdim/attn_bwd_vdim,
and a "sparse" one runs attn_sparse_fwd/attn_sparse_bwd on synthetic index lists
(FLOPs counted per non-empty list slot of every query head).
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


def visible_pairs(S, causal, window=0):
    """(query, key) pairs per head the FLOP convention counts."""
    if window and window < S:
        return float(S) * window - window * (window - 1) / 2.0
    return S * S / 2.0 if causal else float(S) * S


def pair_flops(D, Dv):
    """FLOP per visible (query, key) pair: each launch's products and the pass totals."""
    return {"fwd_kernel": 2.0 * (D + Dv),          # S = Q K^T, O = P V
            "dq_kernel": 4.0 * D + 2.0 * Dv,       # S, dP = dO V^T, dQ = dS K
            "dkv_kernel": 4.0 * (D + Dv),          # S, dP, dV = P^T dO, dK = dS^T Q
            "bwd_kernels": 8.0 * D + 6.0 * Dv,     # both backward launches
            "fwd": 2.0 * (D + Dv),
            "bwd": 6.0 * D + 4.0 * Dv}


def algorithmic_pair_flops(D, Dv):
    """The share of the algorithmic work (forward 2D + 2Dv, backward 6D + 4Dv per pair)
    each launch computes: the dQ kernel recomputes S and dP, which the dK/dV kernel also
    computes, so only its dQ = dS K product counts as its own."""
    return {"fwd_kernel": 2.0 * (D + Dv), "dq_kernel": 2.0 * D, "dkv_kernel": 4.0 * (D + Dv),
            "bwd_kernels": 6.0 * D + 4.0 * Dv}


def host_cpu():
    """CPU model and the cores this process may use."""
    model = None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"model": model, "cores": len(os.sched_getaffinity(0))}


def time_calls(fn, n, stream):
    """Durations of fn (one or more launches on `stream`) with HIP events recorded on
    that stream: the mean over n back-to-back calls, then the median and minimum of n
    calls with an event between consecutive calls."""
    import torch
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(n):
        fn()
    e1.record(stream)
    e1.synchronize()
    mean = e0.elapsed_time(e1) / n
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
    evs[0].record(stream)
    for i in range(n):
        fn()
        evs[i + 1].record(stream)
    evs[-1].synchronize()
    per = sorted(evs[i].elapsed_time(evs[i + 1]) for i in range(n))
    return mean, per[n // 2], per[0]


# The other dense workloads, reported beside the headline step: forward for all three,
# the backward too for the non-causal D = 64 one.
SIDE_CONFIGS = (("single_head_s128_d64", False), ("long_causal_gqa_s8192", False),
                ("mha_noncausal_s2048_d64", True))


def side_configs(n_rep):
    """Per-entry-point figures of SIDE_CONFIGS, timed like the headline's."""
    import torch
    import flashattention_tiled_attention_amd as fa
    from flashattention_tiled_attention_amd.inputs import CONFIGS, qkv
    from tests.gpu_util import to_dev
    stream = torch.cuda.current_stream()
    out = {}
    for name, with_bwd in SIDE_CONFIGS:
        c = CONFIGS[name]
        B, Hq, Hkv, S, D, causal = c["B"], c["Hq"], c["Hkv"], c["S"], c["D"], c["causal"]
        log("side workload %s" % name)
        scale = 1.0 / math.sqrt(D)
        q, k, v, dout = qkv(B, Hq, Hkv, S, D, seed=0, with_dout=True)
        tq, tk, tv, tdo = to_dev(q), to_dev(k), to_dev(v), to_dev(dout)
        o = torch.empty((B, Hq, S, D), dtype=torch.bfloat16, device="cuda")
        lse = torch.empty((B, Hq, S), dtype=torch.float32, device="cuda")
        fns = {"fwd_kernel": lambda: fa.attn_fwd(tq, tk, tv, o, lse, causal, scale, stream)}
        if with_bwd:
            gq = torch.empty((B, Hq, S, D), dtype=torch.float32, device="cuda")
            gk = torch.empty((B, Hkv, S, D), dtype=torch.float32, device="cuda")
            gv = torch.empty((B, Hkv, S, D), dtype=torch.float32, device="cuda")
            ws = torch.empty((fa.attn_bwd_workspace_bytes(B, Hq, Hkv, S, D),), dtype=torch.uint8, device="cuda")
            bargs = (tq, tk, tv, o, lse, tdo, gq, gk, gv, causal, scale, ws, stream)
            fns["dq_kernel"] = lambda: fa.attn_bwd_dq(*bargs)
            fns["dkv_kernel"] = lambda: fa.attn_bwd_dkdv(*bargs)
        pairs = B * Hq * visible_pairs(S, causal)
        pf = pair_flops(D, D)
        entry = {"B": B, "Hq": Hq, "Hkv": Hkv, "S": S, "D": D, "causal": bool(causal)}
        ms = {}
        for kname, fn in fns.items():   # the forward runs first: the backward reads its o, lse
            for _ in range(5):          # warm-up: the clocks ramp up from the host-side set-up
                fn()
            torch.cuda.synchronize()
            mean, med, mn = time_calls(fn, n_rep, stream)
            ms[kname] = mean
            tf = pf[kname] * pairs / (mean * 1e-3) / 1e12
            entry[kname] = {"kernel": launched_kernel(kname, D, D, S, causal, 0, scale),
                            "ms": round(mean, 4), "ms_median": round(med, 4), "ms_min": round(mn, 4),
                            "tflops": round(tf, 2), "frac_of_peak": round(tf / PEAK_BF16_TFLOPS, 4)}
        entry["fwd"] = {k: entry["fwd_kernel"][k] for k in ("ms", "tflops", "frac_of_peak")}
        if with_bwd:
            bms = ms["dq_kernel"] + ms["dkv_kernel"]
            tf = pf["bwd"] * pairs / (bms * 1e-3) / 1e12
            entry["bwd"] = {"ms": round(bms, 4), "tflops": round(tf, 2), "frac_of_peak": round(tf / PEAK_BF16_TFLOPS, 4)}
        out[name] = entry
        del tq, tk, tv, tdo, o, lse
        if with_bwd:
            del gq, gk, gv, ws
        torch.cuda.empty_cache()
    return out


def clock_probe():
    """The chip's matrix-core rate and shader clock on a register-only MFMA loop with
    random bf16 operands (libmfma_rate), measured in the same run as the kernels."""
    from flashattention_tiled_attention_amd import mfma_rate
    r = mfma_rate.run("random", waves_per_simd=2, iters=50000)
    return {"source": "register-only v_mfma_f32_32x32x16_bf16 loop, random bf16 operands, 2 waves/SIMD",
            "shader_clock_ghz": r["shader_clock_ghz"], "mfma_tflops": r["tflops"],
            "frac_of_peak": r["frac_of_peak"]}


def cpu_baseline(q, k, v, dout, cfg, target_s, with_bwd):
    """Time the fp64 oracle (as it stands) on a bounded sample of the workload's query
    rows (forward) and key rows (backward); scale to TFLOP/s of the same convention."""
    import numpy as np
    import oracle
    B, Hq, Hkv, S, D, causal = cfg["B"], cfg["Hq"], cfg["Hkv"], cfg["S"], cfg["D"], cfg["causal"]
    W = cfg.get("window", 0)
    Dv = cfg.get("Dv", D)
    pf = pair_flops(D, Dv)
    scale = 1.0 / math.sqrt(D)
    rng = np.random.default_rng(123)

    def row_flops(rows):
        i = rows % S
        n = (i + 1) if causal else np.full_like(i, S)
        if W:
            n = np.minimum(n, W)
        return float(np.sum(pf["fwd"] * n))

    # calibrate on a small sample, then size the timed sample to ~target_s
    cal = rng.integers(0, B * Hq * S, size=64)
    t = time.perf_counter()
    oracle.fwd_rows(q, k, v, cal, causal, scale, W)
    per_flop = (time.perf_counter() - t) / row_flops(cal)
    budget = target_s * (0.5 if with_bwd else 1.0)
    n = int(min(B * Hq * S, max(64, budget / per_flop / (row_flops(cal) / cal.size))))
    rows = rng.choice(B * Hq * S, size=n, replace=False)
    t = time.perf_counter()
    oracle.fwd_rows(q, k, v, rows, causal, scale, W)
    t_f = time.perf_counter() - t
    flops, secs = row_flops(rows), t_f
    sample = "forward: %d of %d query rows (uniform without replacement)" % (n, B * Hq * S)
    if with_bwd:
        # whole K/V groups, one oracle call each, until the budget is spent: a group's
        # per-row statistics (S, P and dP rows of its query heads) and dK/dV of all its keys
        G = Hq // Hkv
        stat_flops = G * row_flops(np.arange(S, dtype=np.int64))
        seen_by = (S - np.arange(S)) if causal else np.full(S, S)          # query rows that see each key
        if W:
            seen_by = np.minimum(seen_by, W)
        key_flops = float(np.sum(G * pf["dkv_kernel"] * seen_by))
        rest = max(target_s - t_f, 0.0)
        t_b, groups = 0.0, 0
        for g in range(B * Hkv):
            keys = g * S + np.arange(S, dtype=np.int64)
            t = time.perf_counter()
            oracle.bwd_rows(q, k, v, dout, np.zeros(0, np.int64), keys, causal, scale, W)
            t_b += time.perf_counter() - t
            groups += 1
            if t_b >= rest:
                break
        # the groups' statistics are counted as work at the forward rate; their time is in t_b
        flops += groups * (stat_flops + key_flops)
        secs += t_b
        sample += "; backward: row statistics and dK/dV of all keys of %d of %d kv groups" % (
            groups, B * Hkv)
    return {"value": flops / secs / 1e12, "unit": "TFLOP/s", "cores": oracle.num_threads(),
            "kind": "oracle", "sample": sample, "seconds": round(secs, 2), "flop": flops}


def cpu_baseline_sparse(q, k, v, dout, idx, cfg, target_s, with_bwd):
    """The fp64 oracle on a bounded sample of the sparse workload: forward query rows
    (~half the budget), then the backward of a sample of key/value rows (which first
    needs every query row's lse and delta); TFLOP/s in the bench's convention."""
    import numpy as np
    import oracle
    B, Hq, Hkv, S, D = cfg["B"], cfg["Hq"], cfg["Hkv"], cfg["S"], cfg["D"]
    N = k.shape[2]
    scale = 1.0 / math.sqrt(D)
    rng = np.random.default_rng(123)
    nval = (idx >= 0).sum(axis=2)                                  # [B][S]

    def row_flops(rows):
        bh, i = rows // S, rows % S
        return float(np.sum(4.0 * D * nval[bh // Hq, i]))

    cal = rng.integers(0, B * Hq * S, size=256)
    t = time.perf_counter()
    oracle.sparse_fwd(q, k, v, idx, scale, rows=cal)
    per_flop = (time.perf_counter() - t) / row_flops(cal)
    budget = target_s * (0.5 if with_bwd else 1.0)
    n = int(min(B * Hq * S, max(256, budget / per_flop / (row_flops(cal) / cal.size))))
    rows = rng.choice(B * Hq * S, size=n, replace=False)
    t = time.perf_counter()
    oracle.sparse_fwd(q, k, v, idx, scale, rows=rows)
    secs = time.perf_counter() - t
    flops = row_flops(rows)
    sample = "forward: %d of %d query rows (uniform without replacement)" % (n, B * Hq * S)
    if with_bwd:
        keys = np.sort(rng.choice(B * Hkv * N, size=16, replace=False)).astype(np.int64)
        t = time.perf_counter()
        oracle.sparse_bwd(q, k, v, dout, idx, scale, qrows=np.zeros(0, np.int64), kvrows=keys)
        secs += time.perf_counter() - t
        # every query row's scores and dP (the row statistics), then 8*D per (entry, head)
        # for each sampled key
        entries = sum(int(np.sum(idx[(r // N) // Hkv] == r % N)) for r in keys)
        flops += 4.0 * D * Hq * float(nval.sum()) + 8.0 * D * (Hq // Hkv) * entries
        sample += "; backward: all row statistics + dK/dV of 16 of %d key/value rows" % (B * Hkv * N)
    return {"value": flops / secs / 1e12, "unit": "TFLOP/s", "cores": oracle.num_threads(),
            "kind": "oracle", "sample": sample, "seconds": round(secs, 2)}


_CSRC = "flashattention_tiled_attention_amd/csrc/"
KERNEL_SOURCES = {   # every source a kernel's machine code depends on
    "fwd_kernel": [_CSRC + "attn_fwd.hip", _CSRC + "device.h", _CSRC + "kernels.h"],
    "fwd1_kernel": [_CSRC + "attn_fwd.hip", _CSRC + "device.h", _CSRC + "kernels.h"],
    "dq_kernel": [_CSRC + "attn_bwd.hip", _CSRC + "device.h", _CSRC + "kernels.h"],
    "dkv_kernel": [_CSRC + "attn_bwd.hip", _CSRC + "device.h", _CSRC + "kernels.h"],
}


def launched_kernel(role, D, Dv, S, causal, window, scale, sparse=False):
    """Name of the kernel an entry point launches for a dense workload, by the launchers'
    rules: the forward takes fwd1_kernel for 128-wide heads with the running-maximum
    slack on (|scale| sqrt(D) <= 2) and S a multiple of 256; a window takes the window
    kernels; dK/dV takes dkv1_kernel when all heads are 64 wide. role is the timing
    label (fwd_kernel, dq_kernel or dkv_kernel; bwd_kernels for a backward entry point
    timed as a whole, which launches several)."""
    if sparse:
        return "sparse_fwd_kernel" if role == "fwd_kernel" else role
    if role == "fwd_kernel":
        if window:
            return "fwd_win_kernel"
        if D == 128 and Dv == 128 and abs(scale) * math.sqrt(D) <= 2.0 and S % 256 == 0 and S > 128:
            return "fwd1_kernel"
        return "fwd_kernel"
    if role == "dq_kernel":
        return "dq_win_kernel" if window else "dq_kernel"
    if role == "dkv_kernel":
        return "dkv1_kernel" if D == 64 and Dv == 64 else "dkv_kernel"
    return role


def source_sha(kernel):
    """First 16 hex digits of sha256 over the kernel's sources, concatenated in order."""
    import hashlib
    h = hashlib.sha256()
    for path in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, path), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def hbm_traffic(kernel):
    """HBM bytes per launch from profiles/hbm_traffic_<kernel>.txt (rocprofv3 FETCH_SIZE and
    WRITE_SIZE, each scaled by the factor a plain copy of known size gives), or None when
    the record is missing or was taken on a different kernel source."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic_%s_llama8b_s4096.txt" % kernel)
    if kernel not in KERNEL_SOURCES or not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if "=" in line and not line.lstrip().startswith("#"):
            key, val = line.split("=", 1)
            kv[key.strip()] = val.strip()
    if kv.get("source_sha256_16") != source_sha(kernel):
        return None
    fetch = float(kv["fetch_kib_per_launch"]) * 1024 * float(kv["copy_factor_fetch"])
    write = float(kv["write_kib_per_launch"]) * 1024 * float(kv["copy_factor_write"])
    return fetch + write


def copy_probe():
    """A plain device-to-device copy of a known size, for calibrating FETCH_SIZE/WRITE_SIZE."""
    import torch
    n = 256 * 1024 * 1024
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": n, "launches": 3}))


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-side-configs", action="store_true",
                    help="skip the clock probe and the other dense workloads' figures (profiling runs)")
    ap.add_argument("--fwd-only", action="store_true", help="time the forward kernel alone")
    ap.add_argument("--workload", default=WORKLOAD, help="an entry of inputs.CONFIGS (default %(default)s)")
    ap.add_argument("--copy-probe", action="store_true", help="run only the HBM counter calibration copy")
    ap.add_argument("--lds-transpose", action="store_true",
                    help="run only the LDS-to-register transpose microbenchmark (one JSON line)")
    ap.add_argument("--mfma-rate", action="store_true",
                    help="run only the matrix-core rate microbenchmark (one JSON line)")
    ap.add_argument("--issue-rates", action="store_true",
                    help="run only the vector-issue and copy-issue microbenchmark (one JSON line)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py runs on exactly one GPU: there is no multi-GPU path; use --gpus 1",
              file=sys.stderr)
        sys.exit(2)
    if args.copy_probe:
        copy_probe()
        return
    if args.lds_transpose:
        from flashattention_tiled_attention_amd import lds_transpose
        rows = lds_transpose.table()
        print(json.dumps({"metric": "LDS-to-register operand bandwidth, normalized to ds_read_b128",
                          "unit": "GB/s", "device": "MI355X (gfx950)", "methods": rows}), flush=True)
        return

    if args.mfma_rate:
        from flashattention_tiled_attention_amd import mfma_rate
        print(json.dumps({"metric": "v_mfma_f32_32x32x16_bf16 rate with operands in registers, whole chip",
                          "unit": "TFLOP/s", "device": "MI355X (gfx950)", "peak": PEAK_BF16_TFLOPS,
                          "runs": mfma_rate.table()}), flush=True)
        return

    if args.issue_rates:
        from flashattention_tiled_attention_amd import issue_rate
        print(json.dumps({"metric": "cycles a wave spends issuing vector instructions and tile copies",
                          "unit": "shader cycles", "device": "MI355X (gfx950)", "runs": issue_rate.table()}),
              flush=True)
        return

    import torch
    import flashattention_tiled_attention_amd as fa
    from flashattention_tiled_attention_amd.inputs import CONFIGS, qkv
    from tests.gpu_util import to_dev

    if args.workload not in CONFIGS:
        print("unknown workload %r; choose from %s" % (args.workload, ", ".join(CONFIGS)), file=sys.stderr)
        sys.exit(2)
    name = args.workload
    headline = name == WORKLOAD
    cfg = CONFIGS[name]
    B, Hq, Hkv, S, D, causal = cfg["B"], cfg["Hq"], cfg["Hkv"], cfg["S"], cfg["D"], cfg["causal"]
    W = cfg.get("window", 0)
    Dv = cfg.get("Dv", D)
    scale = 1.0 / math.sqrt(D)
    stream = torch.cuda.current_stream()
    with_bwd = not args.fwd_only
    sparse = cfg.get("sparse", False)
    if sparse:
        from flashattention_tiled_attention_amd.inputs import csa_index_lists, sparse_qkv
        idx, N = csa_index_lists(B, S, W, cfg["ratio"], cfg["pool_topk"], seed=0)
        q, k, v, dout = sparse_qkv(B, Hq, Hkv, S, N, D, seed=0, with_dout=True)
        topk = idx.shape[2]
        tq, tk, tv, tdo = to_dev(q), to_dev(k), to_dev(v), to_dev(dout)
        ti = torch.from_numpy(idx).to("cuda")
        o = torch.empty((B, Hq, S, D), dtype=torch.bfloat16, device="cuda")
        lse = torch.empty((B, Hq, S), dtype=torch.float32, device="cuda")
        gq = torch.empty((B, Hq, S, D), dtype=torch.float32, device="cuda")
        gk = torch.empty((B, Hkv, N, D), dtype=torch.float32, device="cuda")
        gv = torch.empty((B, Hkv, N, D), dtype=torch.float32, device="cuda")
        ws = torch.empty((fa.attn_sparse_bwd_workspace_bytes(B, Hq, Hkv, S, N, D, topk),), dtype=torch.uint8,
                         device="cuda")

        def run_fwd():
            fa.attn_sparse_fwd(tq, tk, tv, ti, o, lse, scale, stream)

        def run_bwd():
            fa.attn_sparse_bwd(tq, tk, tv, ti, o, lse, tdo, gq, gk, gv, scale, ws, stream)
        calls = {"fwd_kernel": run_fwd}
        if with_bwd:
            calls["bwd_kernels"] = run_bwd
        # every query head of a token sees the token's non-empty slots
        pairs = float(Hq) * float((idx >= 0).sum())
    else:
        pairs = B * Hq * visible_pairs(S, causal, W)
        q, k, v, dout = qkv(B, Hq, Hkv, S, D, seed=0, with_dout=True, Dv=Dv)
        dq_, dk_, dv_, ddo = to_dev(q), to_dev(k), to_dev(v), to_dev(dout)
        o = torch.empty((B, Hq, S, Dv), dtype=torch.bfloat16, device="cuda")
        lse = torch.empty((B, Hq, S), dtype=torch.float32, device="cuda")
        gq = torch.empty((B, Hq, S, D), dtype=torch.float32, device="cuda")
        gk = torch.empty((B, Hkv, S, D), dtype=torch.float32, device="cuda")
        gv = torch.empty((B, Hkv, S, Dv), dtype=torch.float32, device="cuda")
        ws = torch.empty((fa.attn_bwd_workspace_bytes(B, Hq, Hkv, S, D),), dtype=torch.uint8, device="cuda")

        bargs = (dq_, dk_, dv_, o, lse, ddo, gq, gk, gv, causal, scale, ws, stream)
        wargs = (dq_, dk_, dv_, o, lse, ddo, gq, gk, gv, W, scale, ws, stream)
        if Dv != D:
            def run_fwd():
                fa.attn_fwd_vdim(dq_, dk_, dv_, o, lse, causal, W, scale, stream)

            def run_bwd():
                fa.attn_bwd_vdim(dq_, dk_, dv_, o, lse, ddo, gq, gk, gv, causal, W, scale, ws, stream)
            calls = {"fwd_kernel": run_fwd}
            if with_bwd:
                calls["bwd_kernels"] = run_bwd
        elif W:
            def run_fwd():
                fa.attn_fwd_window(dq_, dk_, dv_, o, lse, W, scale, stream)

            def run_bwd():
                fa.attn_bwd_window(*wargs)
            calls = {"fwd_kernel": run_fwd}
            if with_bwd:
                calls["bwd_kernels"] = run_bwd
        else:
            def run_fwd():
                fa.attn_fwd(dq_, dk_, dv_, o, lse, causal, scale, stream)

            def run_bwd():
                fa.attn_bwd(*bargs)
            calls = {"fwd_kernel": run_fwd}
            if with_bwd:
                calls["dq_kernel"] = lambda: fa.attn_bwd_dq(*bargs)
                calls["dkv_kernel"] = lambda: fa.attn_bwd_dkdv(*bargs)

    def step():
        run_fwd()
        if with_bwd:
            run_bwd()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps

    # Per-entry-point durations with HIP events recorded on the stream the kernels run
    # on: attn_fwd, attn_bwd_dq and attn_bwd_dkdv are one launch each (the exact-path
    # tiles run inside the same launch); a windowed, d_v or sparse workload times its
    # forward and its whole backward entry point.
    n_rep = max(args.steps, 10)
    kernel_stats = {name: time_calls(fn, n_rep, stream) for name, fn in calls.items()}
    kernel_ms = {name: st[0] for name, st in kernel_stats.items()}

    # FLOP convention (pair_flops): each launch's products over the visible pairs; the
    # step's algorithmic work is the forward plus the backward's five products.
    pf = pair_flops(D, Dv)
    f_fwd = pf["fwd"] * pairs
    f_bwd = pf["bwd"] * pairs
    step_flops = f_fwd + (f_bwd if with_bwd else 0.0)
    value = step_flops / (ms_per_step * 1e-3) / 1e12

    dominant = max(kernel_ms, key=kernel_ms.get)
    launched = {k: launched_kernel(k, D, Dv, S, causal, W, scale, sparse) for k in kernel_ms}
    dom_flops = pf[dominant] * pairs
    achieved = dom_flops / (kernel_ms[dominant] * 1e-3) / 1e12
    roofline = {"bound": "mfma", "kernel": launched[dominant], "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                "traffic": hbm_traffic(launched[dominant]) if headline else None,
                "flop_per_launch": dom_flops, "launch_ms": round(kernel_ms[dominant], 4)}

    kernels = {}
    apf = algorithmic_pair_flops(D, Dv)
    for kname, ms in kernel_ms.items():
        fl = pf[kname] * pairs
        kernels[kname] = {"kernel": launched[kname], "ms": round(ms, 4), "tflops": round(fl / (ms * 1e-3) / 1e12, 2),
                          "frac_of_peak": round(fl / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                          "ms_median": round(kernel_stats[kname][1], 4), "ms_min": round(kernel_stats[kname][2], 4),
                          "calls": n_rep, "hbm_bytes": hbm_traffic(launched[kname]) if headline else None}
        if not sparse and kname in apf:
            # the kernel's share of the algorithmic work: below its executed work only
            # where it recomputes products another launch also computes (dQ's S and dP)
            atf = apf[kname] * pairs / (ms * 1e-3) / 1e12
            kernels[kname]["algorithmic_tflops"] = round(atf, 2)
            kernels[kname]["algorithmic_frac_of_peak"] = round(atf / PEAK_BF16_TFLOPS, 4)

    result = {
        "metric": "attention fwd/bwd TFLOP/s and % of bf16 MFMA peak on 1 MI355X",
        "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": name + ("" if with_bwd else "_fwd_only"), "B": B, "Hq": Hq, "Hkv": Hkv,
                   "S": S, "D": D, "Dv": Dv, "causal": bool(causal), "window": W or None,
                   "sparse_lists": ({"topk": int(topk), "N": int(N), "pool_ratio": cfg["ratio"],
                                     "pool_topk": cfg["pool_topk"], "nonempty_slots": int((idx >= 0).sum())}
                                    if sparse else None),
                   "pass": "fwd+bwd" if with_bwd else "fwd", "seed": 0},
        "frac_of_peak": round(value / PEAK_BF16_TFLOPS, 4),
        "fwd": {"tflops": kernels["fwd_kernel"]["tflops"], "ms": kernels["fwd_kernel"]["ms"],
                "frac_of_peak": kernels["fwd_kernel"]["frac_of_peak"]},
        "kernels": kernels,
        "roofline": roofline,
    }
    if with_bwd:
        bwd_ms = kernel_ms["bwd_kernels"] if "bwd_kernels" in kernel_ms else kernel_ms["dq_kernel"] + kernel_ms["dkv_kernel"]
        result["bwd"] = {"tflops": round(f_bwd / (bwd_ms * 1e-3) / 1e12, 2), "ms": round(bwd_ms, 4),
                         "frac_of_peak": round(f_bwd / (bwd_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}
    result["host_cpu"] = host_cpu()
    if headline and not args.no_side_configs:
        result["clock"] = clock_probe()
        result["side_configs"] = side_configs(n_rep)
    if not args.no_cpu_baseline:
        log("timing the oracle on a bounded sample (~%.0f s)" % args.cpu_seconds)
        if sparse:
            result["cpu_baseline"] = cpu_baseline_sparse(q, k, v, dout, idx, cfg, args.cpu_seconds, with_bwd)
        else:
            result["cpu_baseline"] = cpu_baseline(q, k, v, dout, cfg, args.cpu_seconds, with_bwd)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
