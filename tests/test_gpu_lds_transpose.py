"""The LDS transpose microbenchmark (liblds_transpose.so) on the GPU: every method that
transposes delivers exactly the operand the transpose load delivers, at each of the eight
positions a loop iteration loads, and the baseline delivers its untransposed ones; the
per-thread checksums of every loaded word match the host's."""
import pytest

from flashattention_tiled_attention_amd import lds_transpose

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("iters", [4, 5])
@pytest.mark.parametrize("method", [0, 1, 2, 3])
def test_operand_matches(method, iters):
    import numpy as np
    print("case lds_transpose method=%d iters=%d" % (method, iters), flush=True)
    blocks = 8
    ms, words, nbytes, checksum = lds_transpose.run(method, blocks=blocks, iters=iters, reps=1)
    assert ms > 0
    for p in range(lds_transpose.LOADS_PER_ITER):
        assert np.array_equal(words[p], lds_transpose.expected_operand(method, p)), "position %d" % p
    want = np.tile(lds_transpose.expected_checksum(method, iters), blocks * lds_transpose.THREADS // 64)
    assert np.array_equal(checksum, want)
