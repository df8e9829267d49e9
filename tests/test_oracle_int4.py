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
    """Bytes worked out by hand from the layout's description.

    K, slot 3 (chunk 16*q + 3): channel 0 (q 0, i 0) -> byte 48, low nibble; channel 2 (i 2:
    second dword) -> byte 52, low; channel 5 (j 5: byte 1 of the dword, i 1) -> byte 49, high;
    channel 19 (q 1, j 3, i 3) -> byte 16*19 + 4 = 308, high; channel 70 (h 1: +8, j 6: byte 1
    of the second dword) -> byte 48 + 8 + 4 + 1 = 61, low.
    V, slots 5 and 6 (token quad 1, u 1 and 2: byte 2 and byte 1 of a dword): channel 0 and
    channel 16 (column blocks 0 and 1 share the dword's byte, low and high nibble) of slot 5 ->
    byte 1024 + 16*16 + 2 = 1282; channel 0 of slot 6 -> byte 1281, low; channel 33 of slot 5
    (residue 1: chunk 17, block 2: dword 1) -> byte 1024 + 16*17 + 4 + 2 = 1302, low.
    K scale 1.0 / zero -2.0 of group 1 of slot 2 are the fp16 bytes 00 3C 00 C0 at 2048 + 36."""
    rec = np.zeros(O.RECORD4, np.uint8)
    kc = np.zeros((7, 128), np.uint8)
    vc = np.zeros((7, 128), np.uint8)
    kc[3, 0], kc[3, 2], kc[3, 5], kc[3, 19], kc[3, 70] = 1, 2, 5, 9, 14
    vc[5, 0], vc[5, 16], vc[6, 0], vc[5, 33] = 7, 9, 11, 4
    ones = np.ones((7, 4), np.float16)
    zeros = np.zeros((7, 4), np.float16)
    ks, kz = ones.copy(), zeros.copy()
    kz[2, 1] = -2.0
    O.write_slots(rec, np.zeros(7, np.int64), np.arange(7), kc, ks, kz, vc, ones, zeros, bits=4)
    assert (rec[48], rec[49], rec[52], rec[61], rec[308]) == (0x01, 0x50, 0x02, 0x0E, 0x90)
    assert (rec[1281], rec[1282], rec[1302]) == (0x0B, 0x97, 0x04)
    assert list(rec[2048 + 32 + 4:2048 + 32 + 8]) == [0x00, 0x3C, 0x00, 0xC0]
    # every other code byte is zero (no stray writes)
    touched = {48, 49, 52, 61, 308, 1281, 1282, 1302}
    others = [i for i in range(2048) if i not in touched]
    assert not rec[others].any()


def test_int4_k_chunk_masks_give_the_int2_operand_order():
    """Masking a K chunk's dwords (x, y for channels below 64, z, w above) with 0x0F0F0F0F at
    shifts 0 and 4 yields the same int8 vectors, channel for channel, as the INT2 record's 2-bit
    masks at shifts 0, 2, 4, 6 of its lane dwords: byte b of vector i holds channel 16q + 4b + i
    (and 64 + 16q + 4b + i).  The decode kernels share one encoding of q' on that property."""
    rng = np.random.default_rng(84)
    codes4 = rng.integers(0, 16, (16, 128)).astype(np.uint8)
    codes2 = rng.integers(0, 4, (16, 128)).astype(np.uint8)
    rec4 = np.zeros(O.RECORD4, np.uint8)
    rec2 = np.zeros(O.RECORD, np.uint8)
    meta = np.zeros((16, 4), np.float16)
    O.write_slots(rec4, np.zeros(16, np.int64), np.arange(16), codes4, meta, meta, codes4, meta,
                  meta, bits=4)
    O.write_slots(rec2, np.zeros(16, np.int64), np.arange(16), codes2, meta, meta, codes2, meta,
                  meta)
    for q in range(4):
        for r in range(16):
            chunk = rec4[16 * (16 * q + r):16 * (16 * q + r) + 16].view(np.uint32)
            for half in range(2):
                x, y = int(chunk[2 * half]), int(chunk[2 * half + 1])
                vec4 = [x & 0x0F0F0F0F, (x >> 4) & 0x0F0F0F0F, y & 0x0F0F0F0F, (y >> 4) & 0x0F0F0F0F]
                d = q + 4 * half                      # INT2 lane dword of these channels
                off = 8 * (16 * (d % 4) + r) + 4 * (d // 4)
                w2 = int(rec2[off:off + 4].view(np.uint32)[0])
                vec2 = [(w2 >> (2 * i)) & 0x03030303 for i in range(4)]
                for i in range(4):
                    for b in range(4):
                        c = 64 * half + 16 * q + 4 * b + i
                        assert (vec4[i] >> (8 * b)) & 0xFF == codes4[r, c]
                        assert (vec2[i] >> (8 * b)) & 0xFF == codes2[r, c]


def test_int4_v_chunk_shifts_give_bf16_token_pairs():
    """For V chunk 16*tq + cr and dword k, each masked with 0x00780078: (w << 3) and (w >> 5)
    put column block 2k's codes of tokens (0, 1) and (2, 3) of the quad at the mantissa bits
    3..6 and 19..22 of two bf16 halves, (w >> 1) and (w >> 9) those of block 2k + 1; OR-ing
    0x3F80 makes the halves bf16 1 + code/16 exactly."""
    rng = np.random.default_rng(85)
    codes = rng.integers(0, 16, (16, 128)).astype(np.uint8)
    rec = np.zeros(O.RECORD4, np.uint8)
    meta = np.zeros((16, 4), np.float16)
    O.write_slots(rec, np.zeros(16, np.int64), np.arange(16), codes, meta, meta, codes, meta,
                  meta, bits=4)
    for tq in range(4):
        for cr in range(16):
            base = O.V4_CODES + 16 * (16 * tq + cr)
            words = rec[base:base + 16].view(np.uint32)
            for k in range(4):
                w = int(words[k])
                parts = [(w << 3) & 0x00780078, (w >> 1) & 0x00780078,
                         (w >> 5) & 0x00780078, (w >> 9) & 0x00780078]
                for e in range(2):
                    c = 16 * (2 * k + e) + cr
                    for pair in range(2):
                        v = parts[e + 2 * pair] | 0x3F803F80
                        for half in range(2):
                            u = 2 * pair + half
                            bits = (v >> (16 * half)) & 0xFFFF
                            val = np.array([bits << 16], np.uint32).view(np.float32)[0]
                            assert val == 1 + codes[4 * tq + u, c] / 16


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
