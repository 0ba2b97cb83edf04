"""Host logic of bench.py, without a GPU: the one-GPU refusal, the FLOP convention and
the HBM traffic records it attaches to the roofline."""
import math
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "exactly one GPU" in r.stderr
    assert r.stdout == ""


# windows narrower than the sequence (a wider one is the causal triangle, below)
@pytest.mark.parametrize("S,W", [(2, 1), (5, 1), (5, 3), (9, 4), (65, 64), (129, 128), (300, 128), (4096, 128)])
def test_window_pairs_match_brute_force(S, W):
    brute = sum(min(i + 1, W) for i in range(S))
    assert bench.visible_pairs(S, True, W) == brute


def test_causal_and_full_pair_conventions():
    # the causal convention counts S^2 / 2 pairs (the masked half of the square);
    # a window of S or more keys is the causal triangle
    assert bench.visible_pairs(4096, True) == 4096 * 4096 / 2
    assert bench.visible_pairs(2048, False) == 2048.0 * 2048
    assert bench.visible_pairs(300, True, 300) == 300 * 300 / 2


@pytest.mark.parametrize("D,Dv", [(64, 64), (128, 128), (128, 64), (64, 128)])
def test_pair_flops_identities(D, Dv):
    pf = bench.pair_flops(D, Dv)
    assert pf["fwd_kernel"] == pf["fwd"] == 2 * D + 2 * Dv       # S = Q K^T, O = P V
    assert pf["bwd"] == 6 * D + 4 * Dv                           # S, dP, dQ, dK, dV
    assert pf["bwd_kernels"] == pf["dq_kernel"] + pf["dkv_kernel"]
    if D == Dv:
        assert pf["fwd"] == 4 * D and pf["bwd"] == 2.5 * pf["fwd"]


def test_headline_step_flops():
    # Llama-3.1-8B shape: 137.4 GFLOP forward, 343.6 GFLOP backward per step
    pairs = 1 * 32 * bench.visible_pairs(4096, True)
    pf = bench.pair_flops(128, 128)
    assert abs(pf["fwd"] * pairs / 1e9 - 137.44) < 0.01
    assert abs(pf["bwd"] * pairs / 1e9 - 343.60) < 0.01


def _copy_tree(tmp_path, kernel):
    """A copy of the kernel's sources and traffic record under tmp_path."""
    for rel in bench.KERNEL_SOURCES[kernel] + ["profiles/hbm_traffic_%s_llama8b_s4096.txt" % kernel]:
        dst = tmp_path / rel
        dst.parent.mkdir(parents=True, exist_ok=True)
        shutil.copy(os.path.join(ROOT, rel), dst)
    return tmp_path / ("profiles/hbm_traffic_%s_llama8b_s4096.txt" % kernel)


@pytest.mark.parametrize("kernel", ["fwd1_kernel", "dq_kernel", "dkv_kernel"])
def test_traffic_record_follows_the_source_hash(tmp_path, monkeypatch, kernel):
    rec = _copy_tree(tmp_path, kernel)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    text = rec.read_text()
    kv = dict(l.split("=", 1) for l in text.splitlines() if "=" in l and not l.startswith("#"))
    kv = {k.strip(): v.strip() for k, v in kv.items()}
    # a record taken on other sources is not reported
    rec.write_text(text.replace(kv["source_sha256_16"], "0" * 16))
    assert bench.hbm_traffic(kernel) is None
    # a record whose hash matches the sources gives fetch and write, each scaled
    rec.write_text(text.replace(kv["source_sha256_16"], bench.source_sha(kernel)))
    want = (float(kv["fetch_kib_per_launch"]) * 1024 * float(kv["copy_factor_fetch"])
            + float(kv["write_kib_per_launch"]) * 1024 * float(kv["copy_factor_write"]))
    assert bench.hbm_traffic(kernel) == pytest.approx(want)
    # an edited source invalidates it
    src = tmp_path / bench.KERNEL_SOURCES[kernel][0]
    src.write_text(src.read_text() + "\n")
    assert bench.hbm_traffic(kernel) is None
    # no record, no figure
    rec.unlink()
    assert bench.hbm_traffic(kernel) is None


@pytest.mark.parametrize("causal,window", [(True, 0), (False, 0), (True, 16)])
def test_cpu_baseline_counts_whole_groups(causal, window):
    """The oracle baseline on a small workload: with a generous budget it takes every
    query row and every K/V group, and counts the oracle's own work: per visible pair,
    the forward's products for every query row, and per K/V group its rows' statistics
    (at the forward rate) plus the dK/dV kernel's products."""
    from flashattention_tiled_attention_amd import inputs
    B, Hq, Hkv, S, D = 1, 4, 2, 64, 64
    cfg = dict(B=B, Hq=Hq, Hkv=Hkv, S=S, D=D, causal=causal, window=window)
    q, k, v, do = inputs.qkv(B, Hq, Hkv, S, D, 0, with_dout=True)
    r = bench.cpu_baseline(q, k, v, do, cfg, 30.0, True)
    assert "%d of %d query rows" % (B * Hq * S, B * Hq * S) in r["sample"]
    assert "%d of %d kv groups" % (B * Hkv, B * Hkv) in r["sample"]
    # the oracle's own work: every visible pair (row i of a causal head sees i + 1 keys)
    pairs = sum(min(i + 1, window) if window else (i + 1 if causal else S) for i in range(S))
    pf = bench.pair_flops(D, D)
    # forward rows + per group: the statistics (at the forward rate) and the dK/dV products
    expect = B * Hq * pairs * pf["fwd"] + B * Hkv * (Hq // Hkv) * pairs * (pf["fwd"] + pf["dkv_kernel"])
    assert r["flop"] == pytest.approx(expect, rel=1e-12)
    assert r["kind"] == "oracle" and r["cores"] >= 1


def test_launched_kernel_follows_the_launchers():
    """The kernel names bench.py reports per entry point follow the launchers' rules
    (attn_fwd.hip launch_fwd_t, attn_bwd.hip): 128-wide heads with the slack on and
    whole 256-row tiles take fwd1_kernel; peaked scales, ragged S and 64-wide heads
    take fwd_kernel; windows take the window kernels."""
    import bench
    s128 = 1 / math.sqrt(128)
    assert bench.launched_kernel("fwd_kernel", 128, 128, 4096, True, 0, s128) == "fwd1_kernel"
    assert bench.launched_kernel("fwd_kernel", 128, 128, 4096, False, 0, s128) == "fwd1_kernel"
    assert bench.launched_kernel("fwd_kernel", 128, 128, 4000, True, 0, s128) == "fwd_kernel"
    assert bench.launched_kernel("fwd_kernel", 128, 128, 128, False, 0, s128) == "fwd_kernel"
    assert bench.launched_kernel("fwd_kernel", 128, 128, 4096, True, 0, 0.5) == "fwd_kernel"
    assert bench.launched_kernel("fwd_kernel", 128, 64, 4096, True, 0, s128) == "fwd_kernel"
    assert bench.launched_kernel("fwd_kernel", 64, 64, 2048, False, 0, 0.125) == "fwd_kernel"
    assert bench.launched_kernel("fwd_kernel", 128, 128, 4096, True, 512, s128) == "fwd_win_kernel"
    assert bench.launched_kernel("dq_kernel", 128, 128, 4096, True, 512, s128) == "dq_win_kernel"
    assert bench.launched_kernel("dkv_kernel", 64, 64, 2048, False, 0, 0.125) == "dkv1_kernel"
    assert bench.launched_kernel("dkv_kernel", 128, 128, 4096, True, 0, s128) == "dkv_kernel"
    assert bench.launched_kernel("fwd_kernel", 128, 128, 4096, True, 4, s128, sparse=True) == "sparse_fwd_kernel"
