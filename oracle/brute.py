"""Pure-Python brute force for tiny inputs: exact rationals for the latent, the
scales and the codes, ``math.fsum`` for attention.  TEST INFRASTRUCTURE ONLY.

It follows the same steps as ``starkv_oracle`` (STAR-KV summary page, Methodology
sections 2 and 3) but with no NumPy, no BLAS and no vectorisation, so that a
mistake of either one (an index, a transposition, a rounding) shows up as a
disagreement.  Rounding to a binary format is done here from its definition
(round to nearest, ties to even, on exact rationals).
"""

from __future__ import annotations

import math
from fractions import Fraction
from typing import List, Sequence


def round_binary(x: Fraction, mant_bits: int, min_exp: int) -> Fraction:
    """Round an exact rational to a binary float with ``mant_bits`` significant bits
    (including the leading one) and smallest normal exponent ``min_exp``; ties to even."""
    if x == 0:
        return Fraction(0)
    sign = -1 if x < 0 else 1
    a = abs(x)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, min_exp)
    ulp = Fraction(2) ** (e - (mant_bits - 1))
    q = a / ulp
    n = q.numerator // q.denominator
    rem = q - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return sign * n * ulp


def fp32(x: Fraction) -> Fraction:
    return round_binary(Fraction(x), 24, -126)


def fp16(x: Fraction) -> Fraction:
    return round_binary(Fraction(x), 11, -14)


def rne_int(x: Fraction) -> int:
    n = math.floor(x)
    rem = x - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return int(n)


def matmul(X: List[List[Fraction]], A: List[List[Fraction]]) -> List[List[Fraction]]:
    n, k, m = len(X), len(A), len(A[0]) if A else 0
    return [[sum((X[i][t] * A[t][j] for t in range(k)), Fraction(0)) for j in range(m)] for i in range(n)]


def scales(X_cal, A, qmax: Sequence[int]) -> List[Fraction]:
    L = matmul(X_cal, A)
    out = []
    for c in range(len(qmax)):
        amax = fp32(max(abs(L[i][c]) for i in range(len(L))))
        out.append(fp16(fp32(amax / qmax[c])))
    return out


def codes(X, A, sc: Sequence[Fraction], qmax: Sequence[int]) -> List[List[int]]:
    L = matmul(X, A)
    out = []
    for row in L:
        cr = []
        for c, x in enumerate(row):
            if sc[c] == 0:
                cr.append(0)
                continue
            y = fp32(fp32(x) / sc[c])
            cr.append(max(-qmax[c], min(qmax[c], rne_int(y))))
        out.append(cr)
    return out


def attention(q, key_lat, val_lat, B_k, key_off, B_v, H_q: int, H_kv: int, d_h: int, n_q: int):
    """Reconstruct-then-attend with floats and math.fsum.

    q[j][h][e]; key_lat[t][c] / val_lat[t][c] dequantised latents (floats);
    B_k[c][e]; B_v[c][g*d_h + e]; key_off = per-head channel offsets (len H_kv + 1).
    """
    T = len(key_lat)
    G = H_q // H_kv
    r_v = len(B_v)
    K = [[[math.fsum(key_lat[t][c] * B_k[c][e] for c in range(key_off[g], key_off[g + 1]))
           for e in range(d_h)] for g in range(H_kv)] for t in range(T)]
    V = [[[math.fsum(val_lat[t][c] * B_v[c][g * d_h + e] for c in range(r_v))
           for e in range(d_h)] for g in range(H_kv)] for t in range(T)]
    out = []
    for j in range(n_q):
        pos = T - n_q + j
        oj = []
        for h in range(H_q):
            g = h // G
            s = [math.fsum(q[j][h][e] * K[t][g][e] for e in range(d_h)) / math.sqrt(d_h) for t in range(pos + 1)]
            m = max(s)
            p = [math.exp(x - m) for x in s]
            l = math.fsum(p)
            oj.append([math.fsum(p[t] * V[t][g][e] for t in range(pos + 1)) / l for e in range(d_h)])
        out.append(oj)
    return out
