"""The CPU oracle against its pins (CPU only)."""
import numpy as np
import pytest

import oracle
import oracle_pins as pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(oracle)


def test_quantize():
    pins.pin_quantize(oracle)


def test_im2col_bruteforce_exhaustive():
    """Every small case: N<=2, H,W<=7, Cin,Cout<=5, k in {1,3}, s in {1,2}, p in {0,1}."""
    pins.pin_im2col_bruteforce(oracle, exhaustive=True)


def test_thread_count_invariance():
    """One output is one thread's fixed-order sum, so 1 thread and all threads agree bit for
    bit."""
    r = np.random.default_rng(5)
    x = r.standard_normal((2, 17, 13, 8))
    w = r.standard_normal((7, 3, 3, 8))
    b = r.uniform(-1, 1, 7)
    y1 = oracle.conv2d(x, w, b, stride=2, pad=1, act="silu", threads=1)
    yn = oracle.conv2d(x, w, b, stride=2, pad=1, act="silu", threads=0)
    assert np.array_equal(y1, yn)
    p1 = oracle.maxpool3x3s2(x, threads=1)
    assert np.array_equal(p1, oracle.maxpool3x3s2(x, threads=0))


def test_rejects_bad_arguments():
    x = np.zeros((1, 4, 4, 2))
    with pytest.raises(ValueError):
        oracle.conv2d(x, np.zeros((3, 3, 3, 5)))  # Cin mismatch
    with pytest.raises(ValueError):
        oracle.conv2d(x, np.zeros((3, 7, 7, 2)))  # kernel larger than the padded input
    with pytest.raises(ValueError):
        oracle.conv2d(x, np.zeros((3, 1, 1, 2)), act="prelu")  # PReLU without slopes
