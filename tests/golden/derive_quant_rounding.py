"""Exact derivation of the rounding blocks in quant_rounding_blocks.json.

The affine block quantiser (P1 "a small dictionary before we start" and
"step 4: three shelves, all on the GPU": fewer bits per weight, three
widths) is read as

    lo, hi = min, max of the block (fp32 inputs)
    m = RN_f16(lo)
    d = RN_f16(RN_f32(RN_f32(hi - lo) / L))
    q = clamp(rint_half_even(RN_f32(RN_f32(x - m) / d)), 0, L),  d == 0 -> q = 0

Everything here is exact rational arithmetic (``fractions.Fraction``) with
IEEE round-to-nearest-even written out from the format definitions: binary16
has 11 significant bits and minimum normal exponent -14, binary32 has 24 and
-126; below the minimum normal the quantum stays 2^(emin - p + 1)
(subnormals).  Nothing is imported from the oracle or from NumPy's float
types, so the stored values pin the oracle rather than restate it.

Each block is built so that one rounding step matters:

* ``m_tie_up``: lo = -(1 + 3*2^-11) lies half-way between the binary16
  values -(1 + 2^-10) (odd significand) and -(1 + 2^-9) (even); ties to even
  give the larger magnitude, truncation the smaller.
* ``span_inexact``: hi - lo = 3 + 3*2^-11 + 2^-26 needs 27 bits, so RN_f32
  drops 2^-26 and (hi - lo)/3 becomes exactly the binary16 tie 1 + 2^-11,
  which rounds to even (1); without the fp32 rounding of hi - lo the
  quotient sits just above the tie and rounds up to 1 + 2^-10.  lo = -2^-26
  also rounds to a negative zero min.
* ``sub_to_half_code``: m = -2^-24 and x = 2.5: x - m = 2.5 + 2^-24 rounds to
  2.5 in fp32, so with d = 1 the code is the half-way value 2.5, which rounds
  to even (2); the unrounded difference gives 3.  (The division step itself
  cannot create such a tie: an fp32 dividend over a binary16 divisor is never
  within half an fp32 ulp of a half-integer it does not equal, so the
  half-way code has to come from the subtraction.)
* ``subnormal_scale_tie``: (hi - lo)/7 = 5.5 * 2^-24 is half-way between the
  binary16 subnormals 5 * 2^-24 and 6 * 2^-24; ties to even give 6 * 2^-24,
  truncation 5 * 2^-24.

    python tests/golden/derive_quant_rounding.py   # rewrites the JSON
"""

from __future__ import annotations

import json
import os
import struct
from fractions import Fraction as F

BLOCK = 32
P2 = F(2)


def ilog2(a: F) -> int:
    """floor(log2(a)) of a positive rational."""
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if P2 ** e > a:
        e -= 1
    if P2 ** (e + 1) <= a:
        e += 1
    return e


def rint_half_even(v: F) -> int:
    fl = v.numerator // v.denominator
    r = v - fl
    if r > F(1, 2) or (r == F(1, 2) and fl % 2 == 1):
        fl += 1
    return fl


def round_to(x: F, p: int, emin: int, neg: bool = False):
    """IEEE round-to-nearest-even of x to p significant bits, minimum normal
    exponent emin.  Returns (negative, value): the sign is kept so that a
    negative number that rounds to zero gives -0."""
    if x == 0:
        return (neg, F(0))
    s = x < 0
    a = -x if s else x
    e = max(ilog2(a), emin)
    quantum = P2 ** (e - p + 1)
    return (s, rint_half_even(a / quantum) * quantum)


def trunc_to(x: F, p: int, emin: int):
    """Rounding toward zero (a wrong quantiser variant the pins must catch)."""
    if x == 0:
        return (False, F(0))
    s = x < 0
    a = -x if s else x
    e = max(ilog2(a), emin)
    quantum = P2 ** (e - p + 1)
    n = a / quantum
    return (s, (n.numerator // n.denominator) * quantum)


def val(sv):
    s, v = sv
    return -v if s else v


def rn16(x):
    return round_to(x, 11, -14)


def rn32(x):
    return val(round_to(x, 24, -126))


def f16_bits(sv) -> int:
    """binary16 bit pattern of an exactly representable (sign, magnitude)."""
    s, a = sv
    sign = 0x8000 if s else 0
    if a == 0:
        return sign
    e = ilog2(a)
    if e < -14:                                   # subnormal: a = n * 2^-24
        n = a / P2 ** -24
        assert n.denominator == 1 and n.numerator < 1024
        return sign | int(n)
    frac = a / P2 ** e - 1
    mant = frac * 1024
    assert mant.denominator == 1 and 0 <= mant < 1024 and e <= 15
    return sign | ((e + 15) << 10) | int(mant)


def f32_hex(x: F) -> str:
    """float.hex of an fp32-representable rational (also a float64)."""
    v = float(x)
    assert F(v) == x and struct.unpack("<f", struct.pack("<f", v))[0] == v, x
    return v.hex()


def quantise(xs, bits, f16=rn16, f32=rn32):
    """The reading above, step by step; f16 / f32 swap in other roundings."""
    L = (1 << bits) - 1
    lo, hi = min(xs), max(xs)
    m = f16(lo)
    d = f16(f32(f32(hi - lo) / L))
    q = []
    for x in xs:
        if val(d) == 0:
            q.append(0)
            continue
        t = f32(f32(x - val(m)) / val(d))
        q.append(min(max(rint_half_even(t), 0), L))
    return d, m, q


def quantise_trunc16(xs, bits):
    return quantise(xs, bits, f16=lambda x: trunc_to(x, 11, -14))


def quantise_f64_steps(xs, bits):
    # no fp32 rounding of the intermediate steps (a wrong variant)
    return quantise(xs, bits, f32=lambda x: x)


def blocks():
    out = []
    lo = -(1 + 3 * P2 ** -11)
    xs = [lo, F(13, 2)] + [lo + F(k, 2) for k in range(15)] + \
         [F(k, 2) - 1 + P2 ** -9 + F(1, 4) for k in range(15)]
    out.append(("m_tie_up", 4, xs, "trunc16"))
    xs = [-P2 ** -26, 3 + 3 * P2 ** -11] + [F(k, 16) for k in range(30)]
    out.append(("span_inexact", 2, xs, "f64_steps"))
    xs = [-P2 ** -24, F(3), F(5, 2), F(3, 2), F(1, 2), F(5, 2)] + [F(k % 4) for k in range(26)]
    out.append(("sub_to_half_code", 2, xs, "f64_steps"))
    xs = [F(0), 77 * P2 ** -25] + [F(k) * P2 ** -27 for k in range(30)]
    out.append(("subnormal_scale_tie", 3, xs, "trunc16"))
    return out


def derive():
    cases = []
    for name, bits, xs, catches in blocks():
        assert len(xs) == BLOCK
        d, m, q = quantise(xs, bits)
        wrong = quantise_trunc16(xs, bits) if catches == "trunc16" else quantise_f64_steps(xs, bits)
        assert (f16_bits(wrong[0]), f16_bits(wrong[1]), wrong[2]) != (f16_bits(d), f16_bits(m), q)
        cases.append({"name": name, "bits": bits, "x_hex": [f32_hex(x) for x in xs],
                      "d_bits": f16_bits(d), "m_bits": f16_bits(m), "q": q,
                      "catches": catches})
    return cases


def main():
    doc = {
        "about": "Blocks whose quantisation depends on the rounding of each step of the affine "
                 "block quantiser (binary16 d and m, fp32 intermediates, codes rounded half to "
                 "even). Derived in exact rational arithmetic by derive_quant_rounding.py, which "
                 "documents each block; P1 'a small dictionary before we start' and 'step 4: three "
                 "shelves, all on the GPU' (fewer bits per weight at three widths). x_hex: the 32 "
                 "fp32 inputs; d_bits, m_bits: binary16 bit patterns; catches: the wrong variant "
                 "(truncating binary16 rounding, or unrounded fp32 steps) that gives another result.",
        "cases": derive(),
    }
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "quant_rounding_blocks.json")
    with open(path, "w") as fh:
        json.dump(doc, fh, indent=1)
        fh.write("\n")
    print(f"wrote {path}")


if __name__ == "__main__":
    main()
