"""The CPU oracle against its pins (closed forms, exact brute force, independent
library routines, hand-worked fixtures).  CPU only."""
import pytest

import oracle
from oracle_pins import ALL_PINS


@pytest.mark.parametrize("pin", ALL_PINS, ids=[p.__name__ for p in ALL_PINS])
def test_oracle_pin(pin):
    ok, msg = pin(oracle.default())
    assert ok, msg


def test_oracle_thread_count_invariance():
    """Threads split output rows only: 1 thread and many threads give identical bits."""
    import numpy as np
    from oracle_pins import rand_bits
    rng = np.random.default_rng(5)
    A = rand_bits(rng, (61, 77), oracle.BF16)
    B = rand_bits(rng, (77, 45), oracle.BF16)
    C1, S1 = oracle.gemm(61, 45, 77, A, 77, 0, B, 45, 0, oracle.BF16, threads=1)
    C8, S8 = oracle.gemm(61, 45, 77, A, 77, 0, B, 45, 0, oracle.BF16, threads=8)
    assert oracle.last_threads() == 8
    assert np.array_equal(C1, C8) and np.array_equal(S1, S8)


def test_oracle_rejects_bad_arguments():
    import numpy as np
    A = np.zeros((4, 4), np.uint16)
    with pytest.raises(ValueError):
        oracle.gemm(4, 4, 4, A, 3, 0, A, 4, 0, oracle.BF16)   # lda < K
    with pytest.raises(ValueError):
        oracle.gemm_sample(4, 4, 4, A, 4, 0, A, 4, 0, oracle.BF16, [4], [0])  # row out of range
