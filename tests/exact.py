"""Exact rational arithmetic used to pin the oracle (brute force on tiny inputs).

Nothing here imports the oracle: decoding uses torch's own dtype conversions
(float8_e4m3fn, bfloat16, float8_e8m0fnu) or the page's printed e2m1 table,
and rounding is done on Fractions by comparing against the two neighbouring
lattice points.
"""
from fractions import Fraction

import numpy as np
import torch


def e4m3_values(codes):
    """uint8 codes -> list of Fractions via torch's float8_e4m3fn decode."""
    t = torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8)).view(torch.float8_e4m3fn).float()
    return [Fraction(float(v)) for v in t.reshape(-1).tolist()]


def bf16_values(bits):
    t = torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16)).view(torch.bfloat16).float()
    return [Fraction(float(v)) for v in t.reshape(-1).tolist()]


def e8m0_value(e):
    return Fraction(2) ** (int(e) - 127)


def _round_half_even(q):
    """Nearest integer to a non-negative Fraction, ties to even."""
    fl = q.numerator // q.denominator
    rem = q - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        return fl + 1
    return fl


def bf16_round(v):
    """Exact Fraction -> Fraction on the bf16 lattice (RNE, subnormal quantum 2**-133)."""
    if v == 0:
        return Fraction(0)
    a = abs(v)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    e = max(e, -126)
    quantum = Fraction(2) ** (e - 7)
    r = _round_half_even(a / quantum) * quantum
    return r if v > 0 else -r


def fraction_to_bf16_bits(v):
    """A Fraction already on the bf16 lattice -> its bit pattern (via torch)."""
    t = torch.tensor([float(v)], dtype=torch.float32).to(torch.bfloat16)
    return int(t.view(torch.int16).item()) & 0xFFFF


def e4m3_round(v):
    """Exact Fraction with |v| <= 448 -> nearest e4m3 value (ties to even code)."""
    # the finite non-negative e4m3 lattice, from torch's decode
    lattice = sorted(set(e4m3_values(np.arange(0, 0x7F, dtype=np.uint8))))
    a = abs(v)
    best = None
    for i, p in enumerate(lattice):
        if p >= a:
            lo = lattice[i - 1] if i > 0 else p
            hi = p
            if a - lo < hi - a:
                best = (lo, i - 1)
            elif a - lo > hi - a:
                best = (hi, i)
            else:   # tie: the even code; code index == lattice index for 0..0x7E
                best = (lo, i - 1) if (i - 1) % 2 == 0 else (hi, i)
            break
    assert best is not None, "value beyond 448"
    return best[0] if v >= 0 else -best[0]
