"""Offline calibration on the host: the fixed parameters the append kernels take.

The OSCAR paper's "Abstract" (page "OSCAR: Offline Spectral Covariance-Aware Rotation for 2-bit
KV Cache Quantization") derives its fixed rotations offline from covariance structures of the
keys and values; the project card ("FutureMLS-Lab/OSCAR", "How it works") says the same of the
per-layer rotations.  The pages do not give the attention-aware weighting of that covariance,
so this module takes the plain reading: the rotation of a head is the eigenvector basis of the
covariance of a calibration sample of its (post-RoPE) rows, columns ordered by decreasing
eigenvalue, so that y = x . R has uncorrelated channels.  The OptR abstract on the same page
adds a per-channel key offset removed before the rotation (an attention-equivalent
reparameterisation); its plain estimate is the sample mean.

Everything here is fp64 numpy on calibration data and runs once, before serving; the results
are handed to oscar_rotate_quantize_append_ex as fp32 arrays.
"""
from __future__ import annotations

import numpy as np

HEAD_DIM = 128


def _rows_f64(rows) -> np.ndarray:
    """bf16 bit patterns (uint16/int16) or float arrays [N][..][128] -> fp64."""
    a = np.asarray(rows)
    if a.dtype in (np.uint16, np.int16):
        a = (a.view(np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)
    return a.astype(np.float64)


def channel_mean(rows) -> np.ndarray:
    """Per-(head, channel) mean over the calibration tokens: rows [N][Hkv][128] (bf16 bits or
    floats) -> fp32 [Hkv][128] (the fp64 mean, rounded once)."""
    x = _rows_f64(rows)
    return x.mean(axis=0).astype(np.float32)


def covariance(rows, center: bool = True) -> np.ndarray:
    """Per-head covariance over the calibration tokens: rows [N][Hkv][128] -> fp64
    [Hkv][128][128], (x - m)^T (x - m) / N with m the sample mean (or 0 when center is False,
    which gives the second-moment matrix)."""
    x = _rows_f64(rows)
    if center:
        x = x - x.mean(axis=0, keepdims=True)
    n = x.shape[0]
    return np.einsum("nhi,nhj->hij", x, x) / max(n, 1)


def spectral_rotation(cov: np.ndarray) -> np.ndarray:
    """Orthogonal R per head from a symmetric covariance [Hkv][128][128] (or [128][128]):
    R[:, j] is the unit eigenvector of the j-th largest eigenvalue, its sign fixed so that its
    largest-magnitude entry is positive.  Then R^T C R is diagonal with decreasing entries.
    Returns fp64 with the input's leading shape."""
    c = np.asarray(cov, dtype=np.float64)
    single = c.ndim == 2
    c = c[None] if single else c
    out = np.empty_like(c)
    for h in range(c.shape[0]):
        sym = 0.5 * (c[h] + c[h].T)
        lam, vec = np.linalg.eigh(sym)          # ascending
        vec = vec[:, ::-1]
        idx = np.abs(vec).argmax(axis=0)
        sgn = np.sign(vec[idx, np.arange(vec.shape[1])])
        out[h] = vec * np.where(sgn == 0, 1.0, sgn)[None, :]
    return out[0] if single else out


def calibrate(k_rows, v_rows, center_keys: bool = True):
    """Rotations and key mean from calibration rows k_rows, v_rows [N][Hkv][128]:
    (rot_k fp32 [Hkv][128][128], rot_v fp32 [Hkv][128][128], k_mean fp32 [Hkv][128] or None).
    With center_keys the key rotation is taken from the covariance of the centered keys and the
    mean is returned for removal before the rotation; otherwise from the keys' second moments."""
    k_mean = channel_mean(k_rows) if center_keys else None
    rot_k = spectral_rotation(covariance(k_rows, center=center_keys)).astype(np.float32)
    rot_v = spectral_rotation(covariance(v_rows, center=False)).astype(np.float32)
    return rot_k, rot_v, k_mean


HADAMARD_SCALE = float(np.sqrt(2.0) / 16.0)   # the double nearest to 1/sqrt(128)


def hadamard_signs(seed: int, num_kv_heads: int) -> np.ndarray:
    """Seeded random signs int8 [Hkv][128] for oscar_rotate_quantize_append_hadamard."""
    rng = np.random.default_rng(seed)
    return rng.choice(np.array([-1, 1], dtype=np.int8), size=(num_kv_heads, HEAD_DIM))


def hadamard_rotation(signs) -> np.ndarray:
    """Dense fp32 form of diag(s) . H / sqrt(128), H_ij = (-1)^popcount(i & j), for the parts of
    the path that take a matrix (rot_k of oscar_decode_attention, rot_v of oscar_combine).
    signs: None, [128] or [Hkv][128] (negative entries flip).  Returns fp32 [128][128] or
    [Hkv][128][128]: fp32(s_i H_ij r) with r the double nearest to 1/sqrt(128)."""
    i = np.arange(HEAD_DIM)
    par = np.bitwise_and(i[:, None], i[None, :])
    bits = np.zeros_like(par)
    for k in range(7):
        bits += (par >> k) & 1
    h = np.where(bits % 2 == 0, 1.0, -1.0)
    if signs is None:
        return (h * HADAMARD_SCALE).astype(np.float32)
    s = np.where(np.asarray(signs) < 0, -1.0, 1.0)
    return (s[..., :, None] * h * HADAMARD_SCALE).astype(np.float32)

