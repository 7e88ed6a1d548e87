"""Scalar pure-Python oracle of one Kamera reuse block.  TEST INFRASTRUCTURE ONLY.

A second, independent reading of the same definition as ``kamera_oracle``
(Kamera summary on gist.science, paper 2606.23581, section 2, reuse
equation), written with Python floats, ``math.cos``/``math.sin`` and exact
rational rounding.  It exists only to cross-check the vectorised oracle on
small blocks; it is far too slow for anything else.  Only ``tests/`` imports it.
"""

from __future__ import annotations

import math
import struct
from fractions import Fraction


def bf16_to_float(bits: int) -> float:
    return struct.unpack(">f", struct.pack(">I", (bits & 0xFFFF) << 16))[0]


def round_to_bf16(x: float) -> int:
    """Exact round-half-even of a real x to bfloat16 (8 significant bits)."""
    if math.isnan(x):
        return 0x7FC0
    sign = 0x8000 if math.copysign(1.0, x) < 0 else 0
    if x == 0:
        return sign
    a = Fraction(abs(x))
    e = math.frexp(abs(x))[1] - 1          # 2^e <= a < 2^(e+1)
    q = max(e - 7, -133)                   # spacing of bfloat16 values near a
    step = Fraction(2) ** q
    n = round(a / step)                    # Fraction rounds half to even
    val = n * step
    if val >= Fraction(2) ** 128:
        return sign | 0x7F80
    return sign | (struct.unpack(">I", struct.pack(">f", float(val)))[0] >> 16)


def reuse_block(x_bits, delta, u_bits, v_bits, num_heads, head_dim, rope_offset,
                rope_dim, rope_base, rotate, interleaved=False):
    """Rows x_bits[t][f] (ints) -> output bits, one element at a time.

    out = round(R(delta) x + sum_k U[t][k] V[f][k]); elements touched by
    neither term keep their bits.
    """
    T, F = len(x_bits), len(x_bits[0])
    m = 0 if u_bits is None else len(u_bits[0])
    half = rope_dim // 2
    out = []
    for t in range(T):
        x = [bf16_to_float(b) for b in x_bits[t]]
        y = list(x)
        touched = [m > 0] * F
        if rotate:
            for h in range(num_heads):
                for j in range(half):
                    if interleaved:
                        ia = h * head_dim + rope_offset + 2 * j
                        ib = ia + 1
                    else:
                        ia = h * head_dim + rope_offset + j
                        ib = ia + half
                    ang = delta * (rope_base ** (-(2.0 * j) / rope_dim))
                    c, s = math.cos(ang), math.sin(ang)
                    y[ia] = x[ia] * c - x[ib] * s
                    y[ib] = x[ib] * c + x[ia] * s
                    touched[ia] = touched[ib] = True
        row = []
        for f in range(F):
            acc = y[f]
            for k in range(m):
                acc += bf16_to_float(u_bits[t][k]) * bf16_to_float(v_bits[f][k])
            row.append(round_to_bf16(acc) if touched[f] else x_bits[t][f])
        out.append(row)
    return out
