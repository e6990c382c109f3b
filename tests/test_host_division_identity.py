"""The kernels form fp32 quotients x / s as fp32(x * fp64(1 / s)) (the activation
quantiser, the weight quantiser, requantisation, fake quantisation), relying on that
product rounding to the IEEE fp32 quotient.  This checks the identity itself with
NumPy on the CPU, over random pairs across the whole exponent range, subnormal
quotients, exact and tie quotients, and divisors with all-ones significands."""
import numpy as np


def _via_reciprocal(x, s):
    return (x.astype(np.float64) * (1.0 / s.astype(np.float64))).astype(np.float32)


def _ieee(x, s):
    with np.errstate(over="ignore", under="ignore"):
        return (x / s).astype(np.float32)


def _check(x, s):
    with np.errstate(over="ignore", under="ignore"):
        got, want = _via_reciprocal(x, s), _ieee(x, s)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), \
        (x[got != want][:5], s[got != want][:5])


def test_random_pairs_over_the_exponent_range():
    rng = np.random.default_rng(20261203)
    for _ in range(8):
        bits = rng.integers(0, 0x7F800000, size=(2, 1 << 20), dtype=np.uint32)
        x, s = bits[0].view(np.float32), bits[1].view(np.float32)
        s = s[s > 0]
        x = x[: s.size] * np.where(rng.random(s.size) < 0.5, -1, 1).astype(np.float32)
        _check(x, s)


def test_quotients_near_one_and_tie_candidates():
    rng = np.random.default_rng(7)
    s = rng.uniform(1.0, 2.0, 1 << 20).astype(np.float32)
    # x = s * q for q near the quotient grid, nudged by a few ulps: quotients that land on
    # or next to fp32 values and midpoints
    q = rng.uniform(1.0, 2.0, 1 << 20).astype(np.float32)
    x = (s.astype(np.float64) * q.astype(np.float64)).astype(np.float32)
    for d in (-2, -1, 0, 1, 2):
        _check(np.nextafter(x, np.float32(np.inf)) if d > 0 else (np.nextafter(x, np.float32(-np.inf)) if d < 0 else x), s)


def test_subnormal_quotients_and_all_ones_divisors():
    rng = np.random.default_rng(11)
    x = (rng.integers(1, 1 << 24, 1 << 18).astype(np.float32) * np.float32(2.0 ** -149 * 2 ** 10))
    s = rng.uniform(1.0, 4096.0, 1 << 18).astype(np.float32)
    _check(x, s)                                              # many subnormal results
    ones = np.float32(2.0 - 2.0 ** -23) * np.float32(2.0) ** rng.integers(-20, 20, 1 << 18).astype(np.float32)
    _check(rng.standard_normal(1 << 18).astype(np.float32), ones)
    tiny = np.array([2.0 ** -149, 3 * 2.0 ** -149, 2.0 ** -126], dtype=np.float32)
    _check(np.repeat(tiny, 3), np.tile(np.array([2.0, 3.0, 0.75], np.float32), 3))
