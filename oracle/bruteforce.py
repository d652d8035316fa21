"""Exact-rational brute force of the multi-LoRA shrink/expand (tiny inputs).

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).  Every bf16 input is a
dyadic rational, so with ``fractions.Fraction`` the whole computation is exact;
it pins the fp64 oracle to within its rounding error.  Shares nothing with the
C++ oracle: its own bit decoding, its own grouping, its own loops.
"""

from __future__ import annotations

import struct
from fractions import Fraction
from typing import Dict, List

import numpy as np


def bf16_to_fraction(bits: int) -> Fraction:
    """Exact value of a finite bfloat16 bit pattern, decoded field by field."""
    bits = int(bits) & 0xFFFF
    sign = -1 if bits & 0x8000 else 1
    exp = (bits >> 7) & 0xFF
    man = bits & 0x7F
    if exp == 0xFF:
        raise ValueError("non-finite bf16")
    if exp == 0:
        return sign * Fraction(man, 1 << 7) * Fraction(1, 1 << 126)
    val = Fraction(128 + man, 128)
    e = exp - 127
    return sign * (val * (1 << e) if e >= 0 else val / (1 << -e))


def fraction_to_bf16(v: Fraction) -> int:
    """Nearest bfloat16 to an exact rational, ties to an even significand."""
    if v == 0:
        return 0
    sign = 0x8000 if v < 0 else 0
    a = abs(v)
    # exponent e with 2^e <= a < 2^(e+1)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    q = max(e - 7, -133)                      # unit in the last place
    scaled = a / (Fraction(2) ** q)
    r = scaled.numerator // scaled.denominator
    frac = scaled - r
    if frac > Fraction(1, 2) or (frac == Fraction(1, 2) and r % 2 == 1):
        r += 1
    val = Fraction(r) * (Fraction(2) ** q)
    if val >= Fraction(2) ** 128:
        return sign | 0x7F80
    # encode: find bits by packing through float32 (val is exact in float32)
    f = float(val)
    (u,) = struct.unpack("<I", struct.pack("<f", f))
    assert u & 0xFFFF == 0
    return sign | (u >> 16)


def metadata(mapping, max_loras: int) -> Dict[str, list]:
    """Grouping by repeated selection: for each id in ascending order (-1 first),
    list the tokens carrying it in index order."""
    ids = [m if -1 <= m < max_loras else -1 for m in (int(v) for v in mapping)]
    order, active, counts, starts = [], [], [], []
    for lid in range(-1, max_loras):
        members = [t for t, v in enumerate(ids) if v == lid]
        if lid >= 0 and members:
            active.append(lid)
            counts.append(len(members))
            starts.append(len(order))
        order.extend(members)
    na = len(active)
    pad = max_loras - na
    return dict(sorted_token_ids=order, active_lora_ids=active + [-1] * pad,
                num_tokens_per_lora=counts + [0] * pad,
                lora_token_start=starts + [len(ids)] * pad, num_active=[na])


def lora_exact(mapping, x, lora_a: List[np.ndarray], lora_b: List[np.ndarray], y0,
               max_loras: int, rank: int, scale: float):
    """Exact buf [S][T][r] and y [T][ldy] as Fractions (None for rows left alone)."""
    T = len(mapping)
    S = len(lora_a)
    sc = Fraction(float(scale))
    ldy = y0.shape[1]
    buf = [[None] * T for _ in range(S)]
    y = []
    for t in range(T):
        m = int(mapping[t])
        lid = m if -1 <= m < max_loras else -1
        row = [bf16_to_fraction(v) for v in y0[t]]
        if lid >= 0:
            xr = [bf16_to_fraction(v) for v in x[t]]
            off = 0
            for s in range(S):
                a = lora_a[s][lid]
                bvec = []
                for k in range(rank):
                    acc = Fraction(0)
                    for h, xv in enumerate(xr):
                        if xv:
                            acc += xv * bf16_to_fraction(a[k][h])
                    bvec.append(sc * acc)
                buf[s][t] = bvec
                bmat = lora_b[s][lid]
                for n in range(bmat.shape[0]):
                    d = Fraction(0)
                    for k in range(rank):
                        d += bvec[k] * bf16_to_fraction(bmat[n][k])
                    row[off + n] = row[off + n] + d
                off += bmat.shape[0]
        y.append(row)
    assert all(len(r) == ldy for r in y)
    return buf, y
