"""CPU check of the input mapping that lets the gfx950 stochastic-rounding
converter reproduce the oracle's rule (host logic, no GPU).

The oracle's rule (page "MXFP4 和 NVFP4 的区别", section "随机舍入": a value
rounds up with probability equal to its position between the two
neighbouring grid points): with p = (|v| - lo) / (hi - lo) and a 16-bit draw
h, the magnitude rounds up iff h < p * 2^16.

The converter, as characterised on the GPU (the in-tree proof is
tests/test_gpu_converters.py), divides its operand by the power-of-two scale,
keeps the 22 fraction bits below the E2M1 step, F = floor(p' * 2^22), and
rounds up iff F plus the top 22 bits of its random word carry out of 22
bits. The library feeds it the operand ceil(2^23 |v|) (signed) with scale
2^23, and the random word (~h << 16) | 0xFFFF. This test models that rule in
exact integer arithmetic and checks, for every one of the 65,536 draws, that
the mapped converter and the oracle give the same code: magnitudes in every
binade from 2^-30 to 8, at and next to every grid point and midpoint, and
the saturation range. A mistake in the mapping (no ceil, a truncated
operand, a random word without the ones below the draw, the draw not
complemented) fails it; the last test plants each of those.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle

H = np.arange(1 << 16, dtype=np.int64)


def grid_interval(m: Fraction):
    """E2M1 interval [lo, lo + step) holding the magnitude m < 6."""
    if m < 2:
        step = Fraction(1, 2)
    elif m < 4:
        step = Fraction(1)
    else:
        step = Fraction(2)
    lo = (m // step) * step
    return lo, step


def code_of(mag: Fraction) -> int:
    grid = [Fraction(x) for x in (0, 0.5, 1, 1.5, 2, 3, 4, 6)]
    return grid.index(mag)


def converter_codes(operand: int, word_of_h) -> np.ndarray:
    """Model of the converter for a non-negative integer operand (the value
    times 2^23) and scale 2^23, for all draws: the magnitude codes."""
    m = Fraction(operand, 1 << 23)
    if m >= 6:
        return np.full(H.shape, 7, np.int64)
    lo, step = grid_interval(m)
    F = ((m - lo) / step * (1 << 22)).__floor__()
    top22 = word_of_h(H) >> 10
    up = (F + top22) >= (1 << 22)
    base = code_of(lo)
    nxt = code_of(min(lo + step, Fraction(6)))
    return np.where(up, nxt, base)


def library_word(h):
    return ((~h & 0xFFFF) << 16) | 0xFFFF


def library_operand(v: float) -> int:
    """ceil(2^23 |v|) of the binary32 value v (exact: |v| 2^23 is a dyadic
    rational, its ceiling an integer)."""
    return (Fraction(float(np.float32(abs(v)))) * (1 << 23)).__ceil__()


def oracle_codes(v: float) -> np.ndarray:
    vals = np.full(H.shape, np.float32(abs(v)), np.float32)
    return oracle.e2m1_sr_array(vals, H.astype(np.uint16)).astype(np.int64) & 7


def magnitudes():
    rng = np.random.default_rng(21)
    out = []
    for e in range(-30, 3):  # random mantissas in each binade 2^-30 .. 8
        out += list((np.float32(2.0 ** e) * (1 + rng.random(3, dtype=np.float32))).astype(np.float32))
    for p in (0.25, 0.5, 0.75, 1, 1.25, 1.5, 1.75, 2, 2.5, 3, 3.5, 4, 5, 6):
        u = int(np.float32(p).view(np.uint32))
        out += list(np.array([u - 2, u - 1, u, u + 1, u + 2], np.uint32).view(np.float32))
    out += [np.float32(x) for x in (0.0, 1e-45, 1.17e-38, 5.999, 6.5, 100.0)]
    return [float(v) for v in out]


@pytest.mark.parametrize("v", magnitudes())
def test_mapped_converter_equals_oracle_rule(v):
    got = converter_codes(library_operand(v), library_word)
    assert np.array_equal(got, oracle_codes(v)), v


def test_model_reproduces_plain_rounding_steps():
    """Sanity of the model itself: a value on a grid point never moves; a
    value just above 1 rounds up only for the lowest draws."""
    assert np.all(converter_codes(1 << 23, library_word) == 2)  # 1.0
    codes = converter_codes((1 << 23) + 1, library_word)         # 1 + 2^-23
    assert codes[0] == 3 and np.all(codes[1:] == 2)


@pytest.mark.parametrize("mutant", ["no_ceil", "zeros_below_draw", "draw_not_complemented"])
def test_planted_mapping_mistakes_fail(mutant):
    """Each plausible mistake in the mapping gives a different code for some
    value and draw."""
    def operand(v):
        if mutant == "no_ceil":
            return (Fraction(float(np.float32(abs(v)))) * (1 << 23)).__floor__()
        return library_operand(v)

    def word(h):
        if mutant == "zeros_below_draw":
            return (~h & 0xFFFF) << 16
        if mutant == "draw_not_complemented":
            return ((h & 0xFFFF) << 16) | 0xFFFF
        return library_word(h)

    assert any(not np.array_equal(converter_codes(operand(v), word), oracle_codes(v)) for v in magnitudes())
