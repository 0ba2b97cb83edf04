"""The LDS transpose microbenchmark (liblds_transpose.so) on the GPU: every method that
transposes delivers exactly the operand the transpose load delivers, and the baseline
delivers its untransposed one."""
import pytest

from flashattention_tiled_attention_amd import lds_transpose

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("method", [0, 1, 2, 3])
def test_operand_matches(method):
    import numpy as np
    print("case lds_transpose method=%d" % method, flush=True)
    ms, words, nbytes = lds_transpose.run(method, blocks=8, iters=4, reps=1)
    assert ms > 0
    assert np.array_equal(words, lds_transpose.expected_operand(method))
