"""Pins of the oracle's key-mean reparameterisation (CPU only).

The keys are stored as (k - mu) . R_K for a fixed per-(KV head, channel) mean mu.  These tests
tie rotate_rows_centered to exact arithmetic (identity and signed-permutation rotations, where
the definition reduces to one correctly rounded fp32 subtraction, and exact rational sums), to
the attention invariance that motivates it (fp64, unquantised), and to the reduction of the
quantisation error it is for (seeded keys with large channel offsets).
"""
from fractions import Fraction

import numpy as np

from oracle import oscar_oracle as O
from int2_rotated_kv_rotate_amd import workload as W


def _mean(rng, scale=20.0):
    return (rng.standard_normal(128) * scale).astype(np.float32)


def test_zero_or_no_mean_is_the_plain_rotation():
    rng = np.random.default_rng(10)
    x = W.to_bf16_bits((rng.standard_normal((16, 128)) * 5).astype(np.float32))
    R = W.rotations(W.WORKLOADS["tiny"], "k")[0].astype(np.float32)
    y0 = O.rotate_rows(x, R)
    assert np.array_equal(O.rotate_rows_centered(x, R, None).view(np.uint32), y0.view(np.uint32))
    assert np.array_equal(O.rotate_rows_centered(x, R, np.zeros(128, np.float32)).view(np.uint32),
                          y0.view(np.uint32))


def test_identity_rotation_is_one_rounded_subtraction():
    """R = I: y = fp32(x - mu), which numpy's float32 subtraction computes correctly rounded
    (x - mu is exact in fp64 here: |x|, |mu| within [2^-10, 2^10])."""
    rng = np.random.default_rng(11)
    xf = rng.uniform(2.0 ** -10, 2.0 ** 10, (32, 128)) * rng.choice([-1, 1], (32, 128))
    x = W.to_bf16_bits(xf.astype(np.float32))
    mu = (rng.uniform(2.0 ** -10, 2.0 ** 10, 128) * rng.choice([-1, 1], 128)).astype(np.float32)
    y = O.rotate_rows_centered(x, np.eye(128, dtype=np.float32), mu)
    ref = W.bf16_bits_to_f32(x) - mu[None, :]
    assert ref.dtype == np.float32
    assert np.array_equal(y.view(np.uint32), ref.view(np.uint32))


def test_signed_permutation_moves_the_mean_with_its_channel():
    """y_j = s_j x_{p(j)} - s_j mu_{p(j)}: a transposed R or a mean applied after the rotation
    to the wrong channel fails this."""
    rng = np.random.default_rng(12)
    perm = rng.permutation(128)
    sign = rng.choice([-1.0, 1.0], 128).astype(np.float32)
    R = np.zeros((128, 128), np.float32)
    R[perm, np.arange(128)] = sign
    x = W.to_bf16_bits((rng.standard_normal((24, 128)) * 9).astype(np.float32))
    mu = _mean(rng)
    y = O.rotate_rows_centered(x, R, mu)
    xf = W.bf16_bits_to_f32(x)
    ref = (xf[:, perm] * sign) - (mu[perm] * sign)
    assert np.array_equal(y.view(np.uint32), ref.astype(np.float32).view(np.uint32))


def test_centered_rotation_matches_exact_rationals():
    """y_j is fp32 of (S_j - C_j) with S_j, C_j the fp64 ascending sums: within one fp32 ulp
    (plus the two fp64 sums' tiny error) of the exact rational (x - mu) . R."""
    rng = np.random.default_rng(13)
    R = W.rotations(W.WORKLOADS["tiny"], "k")[0].astype(np.float32)
    x = W.to_bf16_bits((rng.standard_normal((3, 128)) * 4).astype(np.float32))
    mu = _mean(rng, 3.0)
    y = O.rotate_rows_centered(x, R, mu)
    xf = W.bf16_bits_to_f32(x)
    for r in range(3):
        for j in range(0, 128, 9):
            exact = sum((Fraction(float(xf[r, i])) - Fraction(float(mu[i]))) * Fraction(float(R[i, j]))
                        for i in range(128))
            got = Fraction(float(y[r, j]))
            ulp = Fraction(float(np.spacing(np.float32(abs(float(exact)) + 1e-30))))
            assert abs(got - exact) <= ulp


def test_attention_is_unchanged_by_a_key_mean_fp64():
    """softmax(sm q (k - mu)^T) == softmax(sm q k^T), in the rotated frame too; the log-sum-exp
    moves by exactly sm (q . mu)."""
    rng = np.random.default_rng(14)
    R = W.rotations(W.WORKLOADS["qwen3_4b"], "k")[0]
    Rv = W.rotations(W.WORKLOADS["qwen3_4b"], "v")[0]
    q = rng.standard_normal(128)
    k = rng.standard_normal((300, 128)) + rng.standard_normal(128) * 6
    v = rng.standard_normal((300, 128))
    mu = rng.standard_normal(128) * 6
    sm = 1.0 / np.sqrt(128.0)
    o0, lse0, a0 = O.softmax_attention(q, k, v, sm)
    o1, lse1, a1 = O.softmax_attention(q @ R, (k - mu) @ R, v @ Rv, sm)
    assert np.abs(a1 - a0).max() <= 1e-12 * a0.max()
    assert np.abs(o1 @ Rv.T - o0).max() <= 1e-12 * np.abs(o0).max()
    smf = float(np.float32(sm))          # the scale the attention applies
    assert abs((lse0 - lse1) - smf * (q @ mu)) <= 1e-10 * max(1.0, abs(lse0))


def test_mean_removal_lowers_the_quantisation_error():
    """Keys with the workload's channel offsets (N(0, 2), x15 on 4 outlier channels): removing
    the channel means before the rotation shrinks the groups' ranges, so the INT2 error of the
    rotated keys drops (measured against each version's own unquantised rotated keys)."""
    w = W.scaled(W.WORKLOADS["qwen3_4b"], batch=1, ctx=512, name="reparam")
    kb, _ = W.sequence_kv(w, 0, 512)
    mu_all = W.key_channel_means(w)
    R_all = W.rotations(w, "k").astype(np.float32)
    ratios = []
    for h in range(2):
        x = kb[:, h]
        errs = []
        for mu in (None, mu_all[h]):
            y, codes, s16, z16 = O.quantize_rows(x, R_all[h], w.clip, mu)
            errs.append(np.mean((O.dequant(codes, s16, z16) - y.astype(np.float64)) ** 2))
        ratios.append(errs[1] / errs[0])
    assert max(ratios) < 0.7, ratios


def test_key_channel_means_match_the_generated_keys():
    """The generator's stated means agree with the sample mean of its keys (4 sigma)."""
    w = W.scaled(W.WORKLOADS["qwen3_4b"], batch=1, ctx=4096, name="means")
    kb, _ = W.sequence_kv(w, 0, 4096)
    k = W.bf16_bits_to_f32(kb).astype(np.float64)
    mu = W.key_channel_means(w).astype(np.float64)
    out = W.outlier_channels(w)
    sd = np.ones_like(mu)
    for h in range(w.num_kv_heads):
        sd[h, out[h]] = 15.0
    assert np.all(np.abs(k.mean(axis=0) - mu) <= 4 * sd / np.sqrt(4096) + 0.01 * np.abs(mu))
