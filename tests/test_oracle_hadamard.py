"""Pins of the oracle's Hadamard rotation (CPU only): the transform's matrix against the closed
form and the Kronecker-power construction, exactness of the fp64 transform against rational
sums, the scale constant against a 60-digit square root, the double rounding of the result,
and agreement with the dense-matrix path."""
from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np

from oracle import oscar_oracle as O
from int2_rotated_kv_rotate_amd import workload as W


def _signs(seed):
    return np.random.default_rng(seed).choice([-1, 1], 128).astype(np.int8)


def test_transform_matrix_is_the_sylvester_hadamard_matrix():
    h = O.fwht(np.eye(128))
    kron = np.array([[1.0]])
    for _ in range(7):
        kron = np.kron(kron, np.array([[1.0, 1.0], [1.0, -1.0]]))
    assert np.array_equal(h, kron)
    i, j = np.meshgrid(np.arange(128), np.arange(128), indexing="ij")
    pop = np.vectorize(lambda v: bin(v).count("1"))(i & j)
    assert np.array_equal(h, np.where(pop % 2 == 0, 1.0, -1.0))
    assert np.array_equal(h @ h.T, 128.0 * np.eye(128))


def test_transform_is_exact_and_an_involution_up_to_128():
    rng = np.random.default_rng(40)
    x = W.bf16_bits_to_f32(W.to_bf16_bits((rng.standard_normal((6, 128)) * 3).astype(np.float32)))
    t = O.fwht(x.astype(np.float64))
    assert np.array_equal(O.fwht(t), 128.0 * x.astype(np.float64))
    h = O.fwht(np.eye(128))
    for r in range(6):
        for jj in (0, 1, 77, 127):
            exact = sum(Fraction(float(x[r, i])) * int(h[i, jj]) for i in range(128))
            assert Fraction(float(t[r, jj])) == exact


def test_scale_is_the_nearest_double_to_two_to_minus_three_and_a_half():
    getcontext().prec = 60
    true = Decimal(2).sqrt() / Decimal(16)
    err = abs(Decimal(O.HADAMARD_SCALE) - true)
    assert err <= Decimal(2) ** -57          # half an ulp of doubles in [2^-4, 2^-3)


def test_rotated_values_are_the_defined_double_rounding():
    """y = fp32(fp64(T * r)) with T exact: rebuilt from rational arithmetic (float(Fraction) is
    correctly rounded)."""
    rng = np.random.default_rng(41)
    s = _signs(42)
    xb = W.to_bf16_bits((rng.standard_normal((4, 128)) * 5).astype(np.float32))
    y = O.rotate_rows_hadamard(xb, s)
    x = W.bf16_bits_to_f32(xb)
    h = O.fwht(np.eye(128))
    r = Fraction(O.HADAMARD_SCALE)
    for row in range(4):
        for jj in range(0, 128, 11):
            t = sum(Fraction(float(x[row, i])) * int(s[i]) * int(h[i, jj]) for i in range(128))
            assert y[row, jj] == np.float32(float(t * r))


def test_signs_flip_input_channels():
    rng = np.random.default_rng(43)
    xb = W.to_bf16_bits((rng.standard_normal((3, 128))).astype(np.float32))
    s = _signs(44)
    flipped = np.where(s[None, :] < 0, xb ^ np.uint16(0x8000), xb)   # negate in bf16 bits
    assert np.array_equal(O.rotate_rows_hadamard(xb, s).view(np.uint32),
                          O.rotate_rows_hadamard(flipped, None).view(np.uint32))


def test_dense_matrix_agrees_with_the_transform():
    rng = np.random.default_rng(45)
    s = _signs(46)
    R = O.hadamard_rotation32(s)
    assert np.abs(R.astype(np.float64) @ R.T.astype(np.float64) - np.eye(128)).max() <= 1e-6
    xb = W.to_bf16_bits((rng.standard_normal((16, 128)) * 4).astype(np.float32))
    x = W.bf16_bits_to_f32(xb).astype(np.float64)
    a = O.rotate_rows(xb, R).astype(np.float64)
    b = O.rotate_rows_hadamard(xb, s).astype(np.float64)
    bound = 2.0 ** -22 * np.abs(x).sum(axis=1, keepdims=True) * O.HADAMARD_SCALE + 2.0 ** -23 * np.abs(b)
    assert np.all(np.abs(a - b) <= bound)


def test_hadamard_spreads_outlier_channels():
    """The workload's x15 outlier key channels spread over all 128 rotated channels: the largest
    rotated channel variance is far below the largest input channel variance."""
    w = W.scaled(W.WORKLOADS["qwen3_4b"], batch=1, ctx=1024, name="had")
    kb, _ = W.sequence_kv(w, 0, 1024)
    x = W.bf16_bits_to_f32(kb[:, 0]).astype(np.float64)
    y = O.rotate_rows_hadamard(kb[:, 0], _signs(47)).astype(np.float64)
    assert y.var(axis=0).max() < 0.25 * x.var(axis=0).max()
    assert abs(np.sum(y ** 2) / np.sum(x ** 2) - 1.0) < 1e-5     # norm preserving
