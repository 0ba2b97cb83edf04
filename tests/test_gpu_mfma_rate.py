"""The matrix-core rate microbenchmark (libmfma_rate.so) on the GPU: its products are
the ones it claims (exact sums on known operands, and the random operands' products
against a numpy evaluation of one loop iteration), and its clock stamps are sane."""
import numpy as np
import pytest

from flashattention_tiled_attention_amd import mfma_rate
from flashattention_tiled_attention_amd.inputs import bf16_to_f32

pytestmark = pytest.mark.gpu


def expected_sums(bits):
    """Each lane's sum of its 64 accumulator values after one loop iteration: chain c
    holds A_c B_(c+3)%8 + A_(c+4) B_(c+7)%8, with lane l giving row l % 32 of A_k
    (columns 8 (l/32) .. +7) and column l % 32 of B_k (rows 8 (l/32) .. +7), and
    holding rows 8 (r/4) + 4 (l/32) + r % 4 (r = 0..15) of column l % 32 of C."""
    x = bf16_to_f32(bits).astype(np.float64)            # [16][64][8]
    A = np.zeros((8, 32, 16))
    B = np.zeros((8, 16, 32))
    for k in range(8):
        for lane in range(64):
            h, j = lane >> 5, lane & 31
            A[k, j, 8 * h:8 * h + 8] = x[k, lane]
            B[k, 8 * h:8 * h + 8, j] = x[8 + k, lane]
    C = sum(A[c] @ B[(c + 3) % 8] + A[c + 4] @ B[(c + 7) % 8] for c in range(4))
    out = np.zeros(64)
    for lane in range(64):
        h, j = lane >> 5, lane & 31
        rows = [8 * (r >> 2) + 4 * h + (r & 3) for r in range(16)]
        out[lane] = C[rows, j].sum()
    return out


@pytest.mark.parametrize("kind", ["random", "ones", "zero"])
def test_products_and_clock(kind):
    print("case mfma_rate operands=%s" % kind, flush=True)
    r = mfma_rate.run(kind, waves_per_simd=1, iters=1 if kind == "random" else 100)
    sink = r["sink"].reshape(-1, 64)   # every wave computes the same per-lane sums
    if kind == "ones":
        assert np.all(sink == 2048.0 * 100)
    elif kind == "zero":
        assert np.all(sink == 0.0)
    else:
        want = expected_sums(mfma_rate.operand_bits("random"))
        assert np.allclose(sink, want[None, :], rtol=1e-5, atol=1e-3)
    assert 0.5 < r["shader_clock_ghz"] < 3.0
    assert r["tflops"] > 0
