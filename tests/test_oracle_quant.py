"""Pins of the oracle's rotation, quantiser and record layout (CPU only).

Each test ties the oracle to something other than itself: exact rational arithmetic, a
brute-force search over the four levels, a hand-derived worked example, or a structural
property of the layout (every bit of a record belongs to exactly one field).
"""
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import oscar_oracle as O
from int2_rotated_kv_rotate_amd import workload as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _bf16_rows(rng, n, scale=1.0):
    return W.to_bf16_bits((rng.standard_normal((n, 128)) * scale).astype(np.float32))


# ---------------------------------------------------------------------------- rotation

def test_generated_rotations_are_orthogonal():
    for name in ("tiny", "qwen3_4b"):
        for which in ("k", "v"):
            R = W.rotations(W.WORKLOADS[name], which)
            for h in range(R.shape[0]):
                assert np.abs(R[h] @ R[h].T - np.eye(128)).max() <= 1e-12
                assert np.abs(R[h].T @ R[h] - np.eye(128)).max() <= 1e-12


def test_k_and_v_rotations_differ():
    w = W.WORKLOADS["tiny"]
    assert np.abs(W.rotations(w, "k") - W.rotations(w, "v")).max() > 0.1


def test_rotate_identity_is_exact():
    rng = np.random.default_rng(1)
    x = _bf16_rows(rng, 64, 7.0)
    y = O.rotate_rows(x, np.eye(128, dtype=np.float32))
    assert np.array_equal(y, W.bf16_bits_to_f32(x))


def test_rotate_signed_permutation_is_exact():
    rng = np.random.default_rng(2)
    perm = rng.permutation(128)
    sign = rng.choice([-1.0, 1.0], 128)
    R = np.zeros((128, 128), np.float32)
    R[perm, np.arange(128)] = sign          # y_j = sign_j * x_{perm_j}
    x = _bf16_rows(rng, 32, 3.0)
    y = O.rotate_rows(x, R)
    xf = W.bf16_bits_to_f32(x)
    assert np.array_equal(y, (xf[:, perm] * sign).astype(np.float32))


def test_rotate_matches_exact_rational_dot_product():
    """y_j must be the fp32 rounding of the exact sum_i x_i R_ij (computed with Fractions)."""
    rng = np.random.default_rng(3)
    R = W.rotations(W.WORKLOADS["tiny"], "k")[0].astype(np.float32)
    x = _bf16_rows(rng, 6, 5.0)
    y = O.rotate_rows(x, R)
    xf = W.bf16_bits_to_f32(x)
    Rf = [[Fraction(float(R[i, j])) for j in range(128)] for i in range(128)]
    for n in range(x.shape[0]):
        xs = [Fraction(float(v)) for v in xf[n]]
        for j in range(128):
            exact = sum(xs[i] * Rf[i][j] for i in range(128))
            assert y[n, j] == np.float32(float(exact)), (n, j)


def test_rotate_query_uses_group_heads():
    rng = np.random.default_rng(4)
    Rk = np.stack([W.rotations(W.WORKLOADS["qwen3_4b"], "k")[h] for h in range(2)]).astype(np.float32)
    q = _bf16_rows(rng, 8)  # 8 query heads over 2 KV heads -> group 4
    qr = O.rotate_query(q, Rk, 4)
    qf = W.bf16_bits_to_f32(q).astype(np.float64)
    for j in range(8):
        assert np.allclose(qr[j], qf[j] @ Rk[j // 4].astype(np.float64), rtol=0, atol=1e-12)
    assert not np.allclose(qr[0], qf[0] @ Rk[1].astype(np.float64))


# ---------------------------------------------------------------------------- quantiser

def _load_quant_example():
    clip = scale = zero = None
    rows = []
    with open(os.path.join(GOLDEN, "quant_worked_example.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if not line:
                continue
            parts = line.split()
            if parts[0] == "clip":
                clip = float(parts[1])
            elif parts[0] == "scale":
                scale = float(parts[1])
            elif parts[0] == "zero":
                zero = float(parts[1])
            else:
                rows.append((int(parts[0]), float(parts[1]), int(parts[2])))
    return clip, scale, zero, rows


def test_worked_example_from_golden_file():
    clip, scale, zero, rows = _load_quant_example()
    y = np.zeros((1, 128), np.float32)
    y[0, 32:] = 1.0  # other groups: irrelevant here
    for c, v, _ in rows:
        y[0, c] = v
    s16, z16 = O.group_params(y, clip)
    assert float(s16[0, 0]) == scale and float(z16[0, 0]) == zero
    codes = O.group_codes(y, s16, z16)
    for c, _, code in rows:
        assert codes[0, c] == code, c
    untouched = [c for c in range(32) if c not in {r[0] for r in rows}]
    assert all(codes[0, c] == 2 for c in untouched)
    levels = O.dequant(codes, s16, z16)[0, :32]
    assert set(np.unique(levels)) <= {-3.0, -1.0, 1.0, 3.0}


def _exact_argmin_codes(y, s16, z16):
    """Nearest of the four levels z + k s in exact arithmetic; flags near-ties."""
    n = y.shape[0]
    best = np.zeros((n, 128), np.uint8)
    tie = np.zeros((n, 128), bool)
    for i in range(n):
        for g in range(4):
            s = Fraction(float(s16[i, g]))
            z = Fraction(float(z16[i, g]))
            for c in range(32 * g, 32 * g + 32):
                v = Fraction(float(y[i, c]))
                d = [abs(v - (z + k * s)) for k in range(4)]
                m = min(d)
                best[i, c] = d.index(m)
                srt = sorted(d)
                # near-tie: the two closest levels within 4 fp32 ulps of t of each other
                if s != 0 and (srt[1] - srt[0]) / s < Fraction(4, 2 ** 22):
                    tie[i, c] = True
    return best, tie


@pytest.mark.parametrize("clip", [0.95, 1.0, 0.6])
def test_codes_are_nearest_level_brute_force(clip):
    rng = np.random.default_rng(5)
    x = _bf16_rows(rng, 24, 2.0)
    R = W.rotations(W.WORKLOADS["tiny"], "k")[0].astype(np.float32)
    y, codes, s16, z16 = O.quantize_rows(x, R, clip)
    best, tie = _exact_argmin_codes(y, s16, z16)
    ok = (codes == best) | tie
    assert ok.all()
    assert tie.sum() <= 2


def test_scale_and_zero_follow_clipped_range():
    rng = np.random.default_rng(6)
    y = (rng.standard_normal((200, 128)) * rng.uniform(0.01, 50, (200, 1))).astype(np.float32)
    for clip in (0.95, 0.8):
        s16, z16 = O.group_params(y, clip)
        g = y.reshape(200, 4, 32).astype(np.float64)
        mx, mn = g.max(2), g.min(2)
        lo = clip * mn
        hi = clip * mx
        # bottom level is the clipped min, top level the clipped max, within fp16 rounding
        assert np.all(np.abs(z16.astype(np.float64) - lo) <= np.abs(lo) * 2 ** -11 + 1e-7)
        top = z16.astype(np.float64) + 3 * s16.astype(np.float64)
        assert np.all(np.abs(top - hi) <= (np.abs(hi) + np.abs(lo)) * 2 ** -9 + 1e-6)
        assert np.all(s16 >= 0)


def test_levels_and_error_bound():
    rng = np.random.default_rng(7)
    x = _bf16_rows(rng, 64, 3.0)
    R = W.rotations(W.WORKLOADS["tiny"], "v")[0].astype(np.float32)
    y, codes, s16, z16 = O.quantize_rows(x, R, 0.95)
    yh = O.dequant(codes, s16, z16)
    s = np.repeat(s16.astype(np.float64), 32, axis=1)
    z = np.repeat(z16.astype(np.float64), 32, axis=1)
    k = (yh - z) / s
    assert np.allclose(k, np.rint(k), atol=0) and k.min() >= 0 and k.max() <= 3
    inside = (y >= z) & (y <= z + 3 * s)
    err = np.abs(y.astype(np.float64) - yh)
    assert np.all(err[inside] <= s[inside] * (0.5 + 2 ** -20))


def test_constant_group_has_zero_scale():
    y = np.full((1, 128), 1.5, np.float32)
    s16, z16 = O.group_params(y, 0.95)
    assert np.all(s16 == 0)
    codes = O.group_codes(y, s16, z16)
    assert np.all(codes == 0)
    assert np.all(O.dequant(codes, s16, z16) == float(np.float16(np.float32(0.95) * np.float32(1.5))))


def test_signed_zero_extreme_gives_positive_zero():
    y = np.zeros((2, 128), np.float32)
    y[0, :32] = np.abs(np.linspace(0, 3, 32, dtype=np.float32))
    y[0, 5] = -0.0                     # min is a signed zero
    y[1, :32] = -np.abs(np.linspace(0, 3, 32, dtype=np.float32))
    y[1, 7] = -0.0                     # max is a signed zero
    s16, z16 = O.group_params(y, 0.95)
    assert z16[0, 0].view(np.uint16) == 0x0000
    assert s16[1, 0] > 0 and np.float16(z16[1, 0]) < 0


def test_exhaustive_bf16_sweep_between_anchors():
    """R = I; anchor a group's max and min, sweep every bf16 value between them."""
    lo, hi = -3.0, 5.0
    allbits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    vals = W.bf16_bits_to_f32(allbits)
    vals = vals[np.isfinite(vals) & (vals > lo) & (vals < hi)]
    n = len(vals)
    pad = (-n) % 30
    vals = np.concatenate([vals, np.zeros(pad, np.float32)])
    rows = vals.reshape(-1, 30)
    y = np.zeros((rows.shape[0], 128), np.float32)
    y[:, 0] = hi
    y[:, 1] = lo
    y[:, 2:32] = rows
    y[:, 32:] = np.linspace(-1, 1, 96, dtype=np.float32)
    s16, z16 = O.group_params(y, 0.95)
    codes = O.group_codes(y, s16, z16)
    s = float(s16[0, 0])
    z = float(z16[0, 0])
    assert np.all(s16[:, 0] == s16[0, 0]) and np.all(z16[:, 0] == z16[0, 0])
    # nearest level, computed in fp64 (exact here: every quantity is a short binary fraction)
    t = (y[:, :32].astype(np.float64) - z) / s
    nearest = np.clip(np.floor(t + 0.5), 0, 3)
    halfway = np.abs(t - np.floor(t) - 0.5) < 1e-6
    ok = (codes[:, :32] == nearest) | halfway
    assert ok.all()
    assert n > 30000


# ---------------------------------------------------------------------------- layout

def test_record_layout_is_a_bijection():
    """Every bit of the 1536-byte record belongs to exactly one (slot, field, channel/group)."""
    owner = np.zeros(1536 * 8, np.int32)
    for r in range(16):
        for c in range(128):
            for loc in (O.k_code_location, O.v_code_location):
                byte, bit = loc(r, c)
                owner[8 * byte + bit] += 1
                owner[8 * byte + bit + 1] += 1
        for g in range(4):
            for kind in ("k", "v"):
                o = O.meta_location(kind, r, g)
                owner[8 * o:8 * (o + 4)] += 1
    assert owner.min() == 1 and owner.max() == 1


def test_record_bytes_golden():
    rec = np.zeros(1536, np.uint8)
    expect = {}
    with open(os.path.join(GOLDEN, "record_bytes_example.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if not line:
                continue
            p = line.split()
            if p[0] == "write":
                kind, r, c, code = p[1], int(p[2]), int(p[3]), int(p[4])
                byte, bit = (O.k_code_location if kind == "k" else O.v_code_location)(r, c)
                rec[byte] = (int(rec[byte]) & ~(3 << bit) & 0xFF) | (code << bit)
            elif p[0] == "meta":
                kind, r, g, s, z = p[1], int(p[2]), int(p[3]), float(p[4]), float(p[5])
                o = O.meta_location(kind, r, g)
                rec[o:o + 2] = np.frombuffer(np.float16(s).tobytes(), np.uint8)
                rec[o + 2:o + 4] = np.frombuffer(np.float16(z).tobytes(), np.uint8)
            elif p[0] == "expect":
                expect[int(p[1])] = int(p[2], 16)
    nz = {i: int(v) for i, v in enumerate(rec) if v}
    assert nz == expect


def test_write_slot_touches_only_its_slot():
    rng = np.random.default_rng(8)
    rec = np.full(1536, 0xA5, np.uint8)
    before = rec.copy()
    kc, vc = rng.integers(0, 4, 128), rng.integers(0, 4, 128)
    s = np.float16(rng.uniform(0, 2, 4))
    z = np.float16(rng.uniform(-2, 0, 4))
    O.write_slot(rec, 9, kc, s, z, vc, s, z)
    mask = np.zeros(1536 * 8, bool)
    for c in range(128):
        for loc in (O.k_code_location, O.v_code_location):
            byte, bit = loc(9, c)
            mask[8 * byte + bit:8 * byte + bit + 2] = True
    for g in range(4):
        for kind in ("k", "v"):
            o = O.meta_location(kind, 9, g)
            mask[8 * o:8 * o + 32] = True
    bits_before = np.unpackbits(before, bitorder="little")
    bits_after = np.unpackbits(rec, bitorder="little")
    assert np.array_equal(bits_before[~mask], bits_after[~mask])
    out = O.read_slot(rec, 9)
    assert np.array_equal(out[0], kc) and np.array_equal(out[3], vc)
    assert np.array_equal(out[1], s) and np.array_equal(out[2], z)


def test_vector_write_read_round_trip():
    rng = np.random.default_rng(9)
    pool = np.zeros(3 * 1536, np.uint8)
    n = 40
    base = rng.integers(0, 3, n) * 1536
    r = rng.permutation(48)[:n] % 16
    # avoid writing the same (record, slot) twice
    key = base // 1536 * 16 + r
    _, first = np.unique(key, return_index=True)
    base, r = base[first], r[first]
    n = len(base)
    kc, vc = rng.integers(0, 4, (n, 128)), rng.integers(0, 4, (n, 128))
    ks, kz, vs, vz = (np.float16(rng.uniform(-3, 3, (n, 4))) for _ in range(4))
    O.write_slots(pool, base, r, kc, ks, kz, vc, vs, vz)
    out = O.read_slots(pool, base, r)
    for a, b in zip(out, (kc, ks, kz, vc, vs, vz)):
        assert np.array_equal(a, b)
