"""Pins of the offline calibration tool (CPU only): the spectral rotation is orthogonal and
diagonalises the covariance it was built from (a planted eigenbasis is recovered up to signs),
and the key mean and covariance match their definitions computed exactly on small samples."""
from fractions import Fraction

import numpy as np

from int2_rotated_kv_rotate_amd import offline as OF
from int2_rotated_kv_rotate_amd import workload as W
from oracle import oscar_oracle as O


def test_planted_eigenbasis_is_recovered():
    rng = np.random.default_rng(30)
    q, _ = np.linalg.qr(rng.standard_normal((128, 128)))
    lam = np.sort(rng.uniform(0.1, 50.0, 128))[::-1]
    cov = (q * lam) @ q.T
    R = OF.spectral_rotation(cov)
    assert np.abs(R.T @ R - np.eye(128)).max() <= 1e-12
    d = R.T @ cov @ R
    assert np.abs(d - np.diag(lam)).max() <= 1e-10 * lam.max()
    # columns are the planted eigenvectors up to sign, with the largest entry positive
    assert np.abs(np.abs(np.sum(R * q, axis=0)) - 1.0).max() <= 1e-9
    assert np.all(R[np.abs(R).argmax(axis=0), np.arange(128)] > 0)


def test_sample_covariance_is_diagonalised_in_decreasing_order():
    w = W.scaled(W.WORKLOADS["qwen3_4b"], batch=1, ctx=2048, name="calib")
    kb, vb = W.sequence_kv(w, 0, 2048)
    cov = OF.covariance(kb)
    R = OF.spectral_rotation(cov)
    for h in range(w.num_kv_heads):
        assert np.abs(R[h].T @ R[h] - np.eye(128)).max() <= 1e-12
        d = R[h].T @ cov[h] @ R[h]
        off = d - np.diag(np.diag(d))
        assert np.abs(off).max() <= 1e-10 * np.trace(cov[h])
        assert np.all(np.diff(np.diag(d)) <= 1e-9 * np.trace(cov[h]))


def test_equal_eigenvalues_still_give_an_orthogonal_rotation():
    R = OF.spectral_rotation(np.eye(128) * 3.0)
    assert np.abs(R.T @ R - np.eye(128)).max() <= 1e-12


def test_mean_and_covariance_match_exact_sums():
    rng = np.random.default_rng(31)
    x = W.to_bf16_bits((rng.standard_normal((7, 2, 128)) * 3 + 1).astype(np.float32))
    xf = W.bf16_bits_to_f32(x)
    mu = OF.channel_mean(x)
    cov = OF.covariance(x)
    for h in range(2):
        for c in (0, 17, 127):
            exact = sum(Fraction(float(xf[n, h, c])) for n in range(7)) / 7
            assert mu[h, c] == np.float32(float(exact))
        for i, j in ((0, 0), (3, 90), (127, 5)):
            mi = sum(Fraction(float(xf[n, h, i])) for n in range(7)) / 7
            mj = sum(Fraction(float(xf[n, h, j])) for n in range(7)) / 7
            exact = sum((Fraction(float(xf[n, h, i])) - mi) * (Fraction(float(xf[n, h, j])) - mj)
                        for n in range(7)) / 7
            assert abs(cov[h, i, j] - float(exact)) <= 1e-12 * max(1.0, abs(float(exact)))


def test_calibrated_parameters_shapes_and_quantisation_error():
    """calibrate() returns fp32 arrays of the library's shapes; the INT2 error of the keys under
    the spectral rotation (with the mean removed) is reported next to the seeded random one."""
    w = W.scaled(W.WORKLOADS["qwen3_4b"], batch=1, ctx=1024, name="calib_q")
    kb, vb = W.sequence_kv(w, 0, 1024)
    rk, rv, mu = OF.calibrate(kb[:512], vb[:512])
    assert rk.shape == (8, 128, 128) and rk.dtype == np.float32
    assert rv.shape == (8, 128, 128) and mu.shape == (8, 128) and mu.dtype == np.float32
    rr = W.rotations(w, "k").astype(np.float32)
    errs = {}
    for name, R, m in (("random", rr, None), ("random_centered", rr, mu), ("spectral", rk, mu)):
        e = []
        for h in range(2):
            y, c, s16, z16 = O.quantize_rows(kb[512:, h], R[h], w.clip, None if m is None else m[h])
            e.append(np.mean((O.dequant(c, s16, z16) - y) ** 2))
        errs[name] = float(np.mean(e))
    print("key INT2 mse on held-out rows:", errs)
    assert all(np.isfinite(v) for v in errs.values())


def test_dense_hadamard_matrix_matches_the_oracle():
    """The library-side dense Hadamard matrix (popcount formula) is bit-identical to the
    oracle's (built from its fast transform of the identity)."""
    s = OF.hadamard_signs(50, 3)
    assert s.dtype == np.int8 and set(np.unique(s)) == {-1, 1}
    dense = OF.hadamard_rotation(s)
    for h in range(3):
        assert np.array_equal(dense[h].view(np.uint32), O.hadamard_rotation32(s[h]).view(np.uint32))
    assert np.array_equal(OF.hadamard_rotation(None).view(np.uint32),
                          O.hadamard_rotation32(None).view(np.uint32))
