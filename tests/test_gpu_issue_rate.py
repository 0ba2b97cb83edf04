"""The instruction-issue microbenchmark (libissue_rate.so) on the GPU: its chains
compute what they claim, its copies move the bytes they claim, and its cycle counts
are sane."""
import numpy as np
import pytest

from flashattention_tiled_attention_amd import issue_rate

pytestmark = pytest.mark.gpu


def chain_start():
    lane = np.arange(256, dtype=np.float64) % 64
    return lane[:, None] / 1024.0 + 0.125 * np.arange(8)[None, :]


@pytest.mark.parametrize("mode", ["fma_independent", "fma_dependent", "exp_independent", "exp_dependent"])
def test_chains(mode):
    print("case issue_rate valu mode=%s" % mode, flush=True)
    # dependent chains run 8 steps per iteration: one iteration keeps the fma chain
    # exact in fp32 (18 fraction bits)
    iters = 1 if "independent" not in mode else 2
    r = issue_rate.valu(mode, waves_per_simd=1, iters=iters, a=0.5)
    x = chain_start()
    for _ in range(iters * 8 if "independent" not in mode else iters):
        if mode == "fma_independent":
            x = x * 0.5 + 1.0                 # exact in fp32 for these values
        elif mode == "fma_dependent":
            x[:, 0] = x[:, 0] * 0.5 + 1.0
        elif mode == "exp_independent":
            x = np.exp2(-x)
        else:
            x[:, 0] = np.exp2(-x[:, 0])
    want = x.sum(axis=1)
    sink = r["sink"].reshape(-1, 256)          # every workgroup computes the same values
    tol = 0.0 if "fma" in mode else 2e-5       # v_exp_f32 is within about 1 ulp
    assert np.allclose(sink, want[None, :], rtol=tol, atol=0.0)
    assert 1.0 <= r["cycles_per_instr_per_wave"] < 200.0


@pytest.mark.parametrize("copies,active", [(1, 1), (4, 8), (8, 3)])
def test_copies_move_their_bytes(copies, active):
    print("case issue_rate copies=%d active=%d" % (copies, active), flush=True)
    r = issue_rate.copies(copies, active, iters=3, blocks=16, seed=copies)
    n = copies * 1024
    src = r["src"].reshape(16, 65536)
    dst = r["dst"].reshape(16, 65536)
    for w in range(8):
        part = slice(w * n, (w + 1) * n)
        if w < active:
            assert np.array_equal(dst[:, part], src[:, part]), w
        elif (w + 1) * n <= 65536:
            assert not dst[:, part].any(), w      # an idle wave copies nothing
    assert 0 < r["issue_cycles"] <= r["issue_to_landed_cycles"]
