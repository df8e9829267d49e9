"""Pins of the oracle's INT4 codec (CPU only): 16-level codes against an exact brute-force
search, the levels and the error bound, the clipped range, the 2560-byte record layout (every
bit owned once, a hand-derived byte, slot isolation, round trip), and the error reduction over
INT2 that is the point of the wider code."""
from fractions import Fraction

import numpy as np

from oracle import oscar_oracle as O
from int2_rotated_kv_rotate_amd import workload as W


def _rows(seed, n, scale):
    rng = np.random.default_rng(seed)
    return W.to_bf16_bits((rng.standard_normal((n, 128)) * scale).astype(np.float32))


def test_codes_are_the_nearest_of_sixteen_levels():
    R = W.rotations(W.WORKLOADS["tiny"], "k")[0].astype(np.float32)
    y, codes, s16, z16 = O.quantize_rows(_rows(80, 12, 2.0), R, 0.95, levels=16)
    ties = 0
    for i in range(12):
        for g in range(4):
            s, z = Fraction(float(s16[i, g])), Fraction(float(z16[i, g]))
            for c in range(32 * g, 32 * g + 32):
                v = Fraction(float(y[i, c]))
                d = [abs(v - (z + k * s)) for k in range(16)]
                best = d.index(min(d))
                srt = sorted(d)
                near_tie = s != 0 and (srt[1] - srt[0]) / s < Fraction(4, 2 ** 22)
                ties += near_tie
                assert codes[i, c] == best or near_tie
    assert ties <= 2


def test_levels_error_bound_and_clipped_range():
    R = W.rotations(W.WORKLOADS["tiny"], "v")[0].astype(np.float32)
    y, codes, s16, z16 = O.quantize_rows(_rows(81, 64, 3.0), R, 0.95, levels=16)
    yh = O.dequant(codes, s16, z16)
    s = np.repeat(s16.astype(np.float64), 32, axis=1)
    z = np.repeat(z16.astype(np.float64), 32, axis=1)
    k = (yh - z) / s
    assert np.array_equal(k, np.rint(k)) and k.min() >= 0 and k.max() <= 15
    inside = (y >= z) & (y <= z + 15 * s)
    assert np.all(np.abs(y - yh)[inside] <= s[inside] * (0.5 + 2 ** -20))
    g = y.reshape(64, 4, 32).astype(np.float64)
    lo, hi = 0.95 * g.min(2), 0.95 * g.max(2)
    assert np.all(np.abs(z16.astype(np.float64) - lo) <= np.abs(lo) * 2 ** -11 + 1e-7)
    top = z16.astype(np.float64) + 15 * s16.astype(np.float64)
    assert np.all(np.abs(top - hi) <= (np.abs(hi) + np.abs(lo)) * 2 ** -8 + 1e-6)


def test_int4_record_layout_is_a_bijection():
    owner = np.zeros(O.RECORD4 * 8, np.int32)
    for r in range(16):
        for c in range(128):
            for loc in (O.k4_code_location, O.v4_code_location):
                byte, bit = loc(r, c)
                owner[8 * byte + bit:8 * byte + bit + 4] += 1
        for g in range(4):
            for kind in ("k", "v"):
                o = O.meta4_location(kind, r, g)
                owner[8 * o:8 * (o + 4)] += 1
    assert owner.min() == 1 and owner.max() == 1


def test_int4_hand_derived_bytes():
    """K codes 3 and 12 for channels 0 and 1 of slot 0 make K byte 0 = 0xC3; V codes 7 and 9
    for channels 0 and 1 of slot 5 make byte 1024 + 64 * 5 = 0x97; K scale 1.0 / zero -2.0 of
    group 1 of slot 2 are the fp16 bytes 00 3C 00 C0 at 2048 + 32 + 4."""
    rec = np.zeros(O.RECORD4, np.uint8)
    kc = np.zeros((3, 128), np.uint8)
    vc = np.zeros((6, 128), np.uint8)
    kc[0, 0], kc[0, 1] = 3, 12
    vc[5, 0], vc[5, 1] = 7, 9
    ones = np.ones((6, 4), np.float16)
    zeros = np.zeros((6, 4), np.float16)
    ks, kz = ones.copy(), zeros.copy()
    kz[2, 1] = -2.0
    O.write_slots(rec, np.zeros(6, np.int64), np.arange(6), np.vstack([kc, np.zeros((3, 128), np.uint8)]),
                  ks, kz, vc, ones, zeros, bits=4)
    assert rec[0] == 0xC3
    assert rec[1024 + 64 * 5] == 0x97
    assert list(rec[2048 + 32 + 4:2048 + 32 + 8]) == [0x00, 0x3C, 0x00, 0xC0]


def test_int4_slots_are_isolated_and_round_trip():
    rng = np.random.default_rng(82)
    rec = np.full(O.RECORD4, 0xA5, np.uint8)
    kc = rng.integers(0, 16, (1, 128)).astype(np.uint8)
    vc = rng.integers(0, 16, (1, 128)).astype(np.uint8)
    meta = rng.standard_normal((1, 4)).astype(np.float16)
    before = rec.copy()
    O.write_slots(rec, [0], [7], kc, meta, meta, vc, meta, meta, bits=4)
    owned = np.zeros(O.RECORD4, bool)
    for c in range(128):
        owned[O.k4_code_location(7, c)[0]] = True
        owned[O.v4_code_location(7, c)[0]] = True
    for g in range(4):
        for kind in ("k", "v"):
            o = O.meta4_location(kind, 7, g)
            owned[o:o + 4] = True
    assert np.array_equal(rec[~owned], before[~owned])
    got = O.read_slots(rec, [0], [7], bits=4)
    assert np.array_equal(got[0], kc) and np.array_equal(got[3], vc)
    assert np.array_equal(got[1].view(np.uint16), meta.view(np.uint16))


def test_int4_error_is_far_below_int2():
    R = W.rotations(W.WORKLOADS["tiny"], "k")[0].astype(np.float32)
    x = _rows(83, 256, 1.0)
    errs = []
    for levels in (4, 16):
        y, c, s16, z16 = O.quantize_rows(x, R, 0.95, levels=levels)
        errs.append(np.mean((O.dequant(c, s16, z16) - y) ** 2))
    assert errs[1] < errs[0] / 10
