"""The CPU oracle against its pins (closed forms, invariants, printed offsets, brute force)."""
import numpy as np
import pytest

import oracle
from oracle_pins import ALL_PINS


@pytest.fixture(scope="module")
def orc():
    return oracle.Oracle()


@pytest.mark.parametrize("name,pin", ALL_PINS, ids=[n for n, _ in ALL_PINS])
def test_pin(orc, name, pin):
    pin(orc)


def test_oracle_results_do_not_depend_on_thread_count():
    """Every output element is computed by one thread in a fixed order: 1 and 8 threads agree bit for bit."""
    orc = oracle.default()
    rng = np.random.default_rng(77)
    B, S, H, d = 2, 70, 3, 32
    q, k, v = (rng.standard_normal((B, S, H * d), dtype=np.float32) for _ in range(3))
    threads = orc.num_threads()
    try:
        orc.set_num_threads(1)
        one = orc.prefill(q, k, v, B, S, H, d, 0.2, True)
        orc.set_num_threads(8)
        many = orc.prefill(q, k, v, B, S, H, d, 0.2, True)
    finally:
        orc.set_num_threads(threads)
    assert np.array_equal(one.view(np.uint64), many.view(np.uint64))
