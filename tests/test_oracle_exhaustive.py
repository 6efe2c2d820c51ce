"""Exhaustive pins of the oracle's FP8 E4M3 and FP4 E2M1 encoders: every fp32 bit pattern
(NaN excluded: outside the contract) against a second encoder written here a different way.
The oracle finds the two codes whose values bracket the input and compares the input with
their midpoint in fp64; the encoders below round the input's binary significand directly
with integer arithmetic -- round to nearest, ties to even, on the bits below the format's
last mantissa bit -- and saturate at the format's largest finite value (448 for E4M3, 6 for
E2M1), the conversions fixed by the FastVideo branch compare's minimax_h3_swiglu_quant.cuh
(scale_fp8, fp4_pair) and the OCP microscaling formats they name.

E4M3: 4 exponent bits (bias 7), 3 mantissa bits, subnormals m * 2^-9, 0x7F the NaN code.
E2M1: 2 exponent bits (bias 1), 1 mantissa bit, subnormal 0.5, sign in bit 3.
"""
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest

import oracle

CHUNK = 1 << 24
WORKERS = max(1, min(8, os.cpu_count() or 1))


def rne_shift(v, s):
    """v >> s rounded to nearest, ties to even (v < 2^24 uint32, s >= 1 per element; s is
    clamped at 25, where every v rounds to 0 as it would for any larger s)."""
    s = np.minimum(s, 25).astype(np.uint32)
    q = v >> s
    rem = v & ((np.uint32(1) << s) - np.uint32(1))
    half = np.uint32(1) << (s - np.uint32(1))
    up = (rem > half) | ((rem == half) & ((q & np.uint32(1)) == 1))
    return q + up.astype(np.uint32)


def significand(u):
    """(24-bit significand with the implicit bit, biased exponent) of fp32 bit patterns."""
    e = ((u >> 23) & 0xFF).astype(np.int32)
    m = u & np.uint32(0x7FFFFF)
    full = np.where(e > 0, m | np.uint32(1 << 23), m)
    return full, np.maximum(e, 1)          # fp32 subnormals scale like exponent 1


def e4m3_bits(u):
    """E4M3 code of the non-negative fp32 patterns u (inf included)."""
    full, e = significand(u)
    # value = full * 2^(e - 150); code units: normal 2^(E - 7) * (1 + m/8), subnormal m * 2^-9
    E = e - 120                              # E4M3 biased exponent of the input's binade
    normal = E >= 1
    q = rne_shift(full, np.where(normal, 20, 141 - e))
    # normal: q in [8, 16] (16: carry into the next binade); subnormal: q in [0, 8]
    carry = normal & (q == 16)
    Eo = np.where(carry, E + 1, E)
    qo = np.where(carry, 8, q).astype(np.int32)
    code = np.where(normal, (Eo << 3) | (qo - 8), qo)
    return np.where((code > 0x7E) | (u >= 0x7F800000), 0x7E, code).astype(np.uint8)


def e2m1_bits(u):
    """E2M1 code (sign in bit 3) of the fp32 patterns u (inf included)."""
    sign = ((u >> 31) & 1).astype(np.uint8) << 3
    a = u & 0x7FFFFFFF
    full, e = significand(a)
    E = e - 126                              # E2M1 biased exponent: 2^(E - 1) * (1 + m/2)
    normal = E >= 1
    q = rne_shift(full, np.where(normal, 22, 149 - e))
    carry = normal & (q == 4)
    Eo = np.where(carry, E + 1, E)
    qo = np.where(carry, 2, q).astype(np.int32)
    code = np.where(normal, (Eo << 1) | (qo - 2), qo)
    code = np.where((code > 7) | (a >= 0x7F800000), 7, code).astype(np.uint8)
    return sign | code


def test_bit_encoders_on_hand_values():
    f = lambda *v: np.array(v, np.float32).view(np.uint32)
    # E4M3: 0, min subnormal 2^-9 and half of it (tie -> 0), the 1.0 binade, ties, 448, overflow
    assert list(e4m3_bits(f(0.0, 2 ** -9, 2 ** -10, 1.5 * 2 ** -10, 1.0, 1.0625, 1.1875, 448.0, 464.0, 1e30,
                            np.inf))) == [0, 1, 0, 1, 0x38, 0x38, 0x3A, 0x7E, 0x7E, 0x7E, 0x7E]
    # E2M1: the eight magnitudes, the ties between them (to even), signs, saturation
    assert list(e2m1_bits(f(0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0))) == [0, 1, 2, 3, 4, 5, 6, 7]
    assert list(e2m1_bits(f(0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 7.0))) == [0, 2, 2, 4, 4, 6, 6, 7]
    assert list(e2m1_bits(f(-0.0, -0.2, -5.0, -np.inf, 1e-45))) == [8, 8, 14, 15, 0]


def sweep(first, last, check):
    """Run check(bits) over the fp32 patterns [first, last) in chunks on a thread pool."""
    starts = range(first, last, CHUNK)

    def one(s):
        n = min(CHUNK, last - s)
        u = np.arange(n, dtype=np.uint32) + np.uint32(s)
        keep = ~(((u & 0x7F800000) == 0x7F800000) & ((u & 0x7FFFFF) != 0))
        return check(u[keep])

    with ThreadPoolExecutor(WORKERS) as pool:
        bad = [b for b in pool.map(one, starts) if b]
    assert not bad, bad[:5]


def test_e4m3_encode_every_non_negative_fp32():
    def check(u):
        want, got = e4m3_bits(u), oracle.e4m3_encode(u.view(np.float32))
        i = np.nonzero(want != got)[0]
        return None if i.size == 0 else "x=0x%08x oracle 0x%02x bits 0x%02x" % (u[i[0]], got[i[0]], want[i[0]])
    sweep(0, 0x7F800001, check)


def test_e4m3_encode_signed_every_negative_fp32():
    def check(u):
        want = np.uint8(0x80) | e4m3_bits(u & 0x7FFFFFFF)
        got = oracle.e4m3_encode_signed(u.view(np.float32))
        i = np.nonzero(want != got)[0]
        return None if i.size == 0 else "x=0x%08x oracle 0x%02x bits 0x%02x" % (u[i[0]], got[i[0]], want[i[0]])
    sweep(0x80000000, 0x100000000, check)


def test_e2m1_encode_every_fp32():
    def check(u):
        want, got = e2m1_bits(u), oracle.e2m1_encode(u.view(np.float32))
        i = np.nonzero(want != got)[0]
        return None if i.size == 0 else "x=0x%08x oracle 0x%x bits 0x%x" % (u[i[0]], got[i[0]], want[i[0]])
    sweep(0, 1 << 32, check)
