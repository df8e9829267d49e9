"""Pins of the oracle's fp32 -> bf16 rounding (CPU only).

The BF16 sink/window store holds bf16 copies of rotated K/V rows (project card
"FutureMLS-Lab/OSCAR", "How it works": sinks and the recent window stay in BF16), and the
workload generator rounds its inputs to bf16.  The oracle's ``f32_to_bf16_bits`` must round to
nearest, ties to even.  Two independent pins:

* hand-derived bit patterns: halfway cases on both sides of an even / odd bf16 neighbour,
  values just above and below a tie, a carry that moves into the next binade, the largest
  finite tie (rounds to infinity), subnormals and signed zeros;
* torch's CPU conversion (``Tensor.to(torch.bfloat16)``, round to nearest even) over random
  finite bit patterns and over every halfway pattern of a range of exponents.

A round-half-up rule passes the non-tie cases but fails the ties, and the test shows that.
"""
import numpy as np
import pytest
import torch

from oracle import oscar_oracle as O

# (fp32 bits, expected bf16 bits), each derived by hand from the bit pattern: the upper 16
# bits are the truncated bf16, the lower 16 bits decide (below 0x8000 down, above up, exactly
# 0x8000 to the even upper half).
HAND = [
    (0x3F800000, 0x3F80),   # 1.0, exact
    (0x3F808000, 0x3F80),   # tie, 0x3F80 is even: stays
    (0x3F818000, 0x3F82),   # tie, 0x3F81 is odd: up to 0x3F82
    (0xBF808000, 0xBF80),   # negative tie, even: stays (magnitude rounding)
    (0xBF818000, 0xBF82),   # negative tie, odd: magnitude up
    (0x3F80C000, 0x3F81),   # above the tie: up
    (0x3F807FFF, 0x3F80),   # just below the tie: down
    (0x3F808001, 0x3F81),   # just above the tie: up
    (0x3FFF8000, 0x4000),   # tie on odd 0x3FFF: carry into the next binade (2.0)
    (0x3FFFFFFF, 0x4000),   # above the tie on the last mantissa value: 2.0
    (0x7F7F8000, 0x7F80),   # largest finite tie, odd: rounds to +infinity
    (0x7F7F7FFF, 0x7F7F),   # just below it: largest finite bf16
    (0x00008000, 0x0000),   # subnormal tie onto 0 (even)
    (0x00018000, 0x0002),   # subnormal tie, odd 0x0001: up
    (0x0000C000, 0x0001),   # subnormal above the tie
    (0x00010001, 0x0001),   # subnormal below the tie
    (0x007F8000, 0x0080),   # largest subnormal bf16 tie, odd: up into the normal range
    (0x80000000, 0x8000),   # -0 keeps its sign
    (0x80008000, 0x8000),   # negative tiny tie onto -0
    (0x7F800000, 0x7F80),   # +infinity
    (0xFF800000, 0xFF80),   # -infinity
]


def _bits_to_f32(bits):
    return np.asarray(bits, dtype=np.uint32).view(np.float32)


def _torch_bf16_bits(x32: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("src,want", HAND, ids=[f"{s:08x}" for s, _ in HAND])
def test_hand_derived_rounding(src, want):
    got = int(O.f32_to_bf16_bits(_bits_to_f32([src]))[0])
    assert got == want, f"{src:#010x} -> {got:#06x}, expected {want:#06x}"


def test_matches_torch_on_random_finite_patterns():
    rng = np.random.default_rng(20241203)
    u = rng.integers(0, 1 << 32, size=1 << 20, dtype=np.uint64).astype(np.uint32)
    x = u.view(np.float32)
    x = x[np.isfinite(x)]
    assert np.array_equal(O.f32_to_bf16_bits(x), _torch_bf16_bits(x))


def test_matches_torch_on_every_tie_of_a_range():
    # every exact halfway pattern (lower 16 bits 0x8000) for all mantissas of the
    # exponents 0 (subnormal) .. 3 and 125 .. 130 and 253 .. 254, both signs
    hi = []
    for e in list(range(0, 4)) + list(range(125, 131)) + [253, 254]:
        m = np.arange(128, dtype=np.uint32)
        hi.append((np.uint32(e) << 7) | m)
    hi = np.concatenate(hi)
    hi = np.concatenate([hi, hi | 0x8000])
    u = (hi.astype(np.uint32) << 16) | 0x8000
    x = u.view(np.float32)
    assert np.array_equal(O.f32_to_bf16_bits(x), _torch_bf16_bits(x))


def test_round_half_up_would_fail_the_pins():
    """The pins discriminate: rounding ties away from zero differs on the even-side ties."""
    def half_up(x):
        u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
        return ((u + 0x8000) >> 16).astype(np.uint16)
    srcs = np.array([s for s, _ in HAND], dtype=np.uint32)
    wants = np.array([w for _, w in HAND], dtype=np.uint16)
    x = srcs.view(np.float32)
    assert not np.array_equal(half_up(x), wants)
    assert np.array_equal(O.f32_to_bf16_bits(x), wants)
