"""Pins for the oracle's ConvRot rotation: closed form of the regular Hadamard
matrix, orthogonality, involution, an independent fast transform, and the
basis-change identity the layer relies on."""

import numpy as np
import pytest

import oracle as O


def _digits4(i, n=4):
    return [(i >> (2 * d)) & 3 for d in range(n)]


def test_hadamard_closed_form_digit_rule():
    # H4 is all ones except -1 where row + column = 3 (the anti-diagonal), so every
    # entry of its 4th Kronecker power is (-1)^(number of base-4 digit positions
    # where the row and column digits add up to 3), scaled by 1/16.
    h = O.hadamard(256) * 16
    for i in range(256):
        di = _digits4(i)
        for j in range(0, 256, 7):
            dj = _digits4(j)
            sign = (-1) ** sum(1 for a, b in zip(di, dj) if a + b == 3)
            assert h[i, j] == sign


def test_hadamard_orthogonal_symmetric_involution():
    h = O.hadamard(256)
    hu = np.rint(h * 16)
    assert np.array_equal(hu @ hu.T, 256 * np.eye(256))
    assert np.array_equal(h, h.T)
    assert np.array_equal(h @ h, np.eye(256))
    assert np.all(hu.sum(axis=0) == 16) and np.all(hu.sum(axis=1) == 16)


def test_hadamard_small_sizes_and_errors():
    assert np.array_equal(np.rint(O.hadamard(4) * 2), [[1, 1, 1, -1], [1, 1, -1, 1], [1, -1, 1, 1], [-1, 1, 1, 1]])
    assert O.hadamard(16).shape == (16, 16)
    for bad in (2, 8, 32, 128, 300):
        with pytest.raises(ValueError):
            O.hadamard(bad)


def test_not_the_walsh_sylvester_matrix():
    h2 = np.array([[1, 1], [1, -1]])
    w = h2
    for _ in range(7):
        w = np.kron(w, h2)
    assert not np.array_equal(np.rint(O.hadamard(256) * 16), w)


def _fast_rotate(x):
    """Independent radix-4 form: for each base-4 digit of the index, every group of
    4 values (a0..a3) becomes out_i = (a0 + a1 + a2 + a3) - 2 * a_(3-i); /16 at the end."""
    y = np.array(x, dtype=np.float64).reshape(-1, 256)
    for d in range(4):
        stride = 4 ** d
        v = y.reshape(y.shape[0], -1, 4, stride)        # [rows, groups, digit, inner]
        s = v.sum(axis=2, keepdims=True)
        y = (s - 2 * v[:, :, ::-1, :]).reshape(y.shape[0], 256)
    return (y / 16).reshape(np.shape(x))


def test_rotate_equals_independent_fast_transform():
    rng = np.random.default_rng(11)
    x = rng.standard_normal((5, 1024))
    assert np.allclose(O.rotate(x), _fast_rotate(x), rtol=0, atol=1e-12)


def test_rotate_ones_and_one_hot():
    assert np.array_equal(O.rotate(np.ones((2, 512))), np.ones((2, 512)))
    e0 = np.zeros((1, 256))
    e0[0, 0] = 1.0
    r = O.rotate(e0)[0] * 16
    # first row of H: (-1)^(number of digits of j equal to 3)
    expect = [(-1) ** sum(1 for d in _digits4(j) if d == 3) for j in range(256)]
    assert np.array_equal(r, expect)


def test_rotate_acts_blockwise():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((3, 768))
    y = O.rotate(x)
    for b in range(3):
        assert np.allclose(y[:, 256 * b:256 * (b + 1)], O.rotate(x[:, 256 * b:256 * (b + 1)]), atol=1e-14)


def test_rotation_preserves_products():
    # rotating both activations and weights leaves x @ W^T unchanged (orthogonal basis change)
    rng = np.random.default_rng(2)
    x = rng.standard_normal((6, 1024))
    w = rng.standard_normal((9, 1024))
    ref = x @ w.T
    got = O.rotate(x) @ O.rotate(w).T
    assert np.max(np.abs(got - ref)) <= 1e-12 * np.max(np.abs(ref))


def test_rotate_bf16_inputs_is_exact_before_fp32_rounding():
    # bf16 inputs have 8 significant bits; with a moderate exponent spread every
    # +-x/16 partial sum is exact in fp64, so dense and fast forms agree exactly
    from bit_codebook_quantized_amd.synth import activations
    x = activations(4, 1024, seed=99).astype(np.float64)
    assert np.array_equal(O.rotate(x), _fast_rotate(x))
