"""Scalar pure-Python MoE layer for micro shapes (CPU oracle pin; test infrastructure only).

A second, independent transcription of the same layer definition as ``moe_ref`` (X-Stage
paper, Introduction, MoE-layer paragraph, with the same readings), written with plain loops:
selection by repeated linear scans, a counting sort by hand, dot products summed exactly as
rationals, and bfloat16 rounding done on exact fractions. It shares no helper with
``moe_ref``; the tests compare the two on micro shapes.
"""
from __future__ import annotations

import math
import struct
from fractions import Fraction


def bf16_decode(bits: int) -> float:
    """bfloat16 bit pattern -> Python float (exact)."""
    return struct.unpack("<f", struct.pack("<I", (int(bits) & 0xFFFF) << 16))[0]


def bf16_nearest(v) -> Fraction | float:
    """Nearest bfloat16 value to the exact rational v (ties to even); returns a Fraction,
    or +-inf beyond the largest finite bfloat16."""
    v = Fraction(v)
    if v == 0:
        return Fraction(0)
    sign = -1 if v < 0 else 1
    a = -v if v < 0 else v
    # find e with 2^e <= a < 2^(e+1)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    elif Fraction(2) ** (e + 1) <= a:
        e += 1
    q = max(e - 7, -133)  # weight of the last of 8 significant bits; subnormal floor 2^-133
    scaled = a / Fraction(2) ** q
    n = round(scaled)  # Fraction rounding: half to even
    r = n * Fraction(2) ** q
    if r > Fraction(255, 128) * Fraction(2) ** 127:
        return sign * math.inf
    return sign * r


def bf16_encode(v) -> int:
    """Bit pattern of a bfloat16-representable value."""
    f = float(v)
    return struct.unpack("<I", struct.pack("<f", f))[0] >> 16


def route(logits, k):
    """Top-k by repeated scans (largest logit, lowest id on ties); weights = full softmax,
    kept entries renormalised (math.exp in float64; result rounded to float32)."""
    ids, ws = [], []
    for row in logits:
        row = [float(v) for v in row]
        E = len(row)
        taken = [False] * E
        sel = []
        for _ in range(k):
            best = -1
            for e in range(E):
                if taken[e]:
                    continue
                if best < 0 or row[e] > row[best]:
                    best = e
            taken[best] = True
            sel.append(best)
        m = max(row)
        z = sum(math.exp(v - m) for v in row)
        p = [math.exp(row[e] - m) / z for e in sel]
        s = sum(p)
        ids.append(sel)
        ws.append([struct.unpack("<f", struct.pack("<f", q / s))[0] for q in p])
    return ids, ws


def plan(ids, E):
    """Counting sort of slots by expert, stable in slot order."""
    flat = [e for row in ids for e in row]
    counts = [0] * E
    for e in flat:
        counts[e] += 1
    offsets = [0] * (E + 1)
    for e in range(E):
        offsets[e + 1] = offsets[e] + counts[e]
    cursor = list(offsets[:E])
    perm = [0] * len(flat)
    pos = [0] * len(flat)
    for f, e in enumerate(flat):
        perm[cursor[e]] = f
        pos[f] = cursor[e]
        cursor[e] += 1
    return counts, offsets, perm, pos


def layer(x_bits, logits, w1_bits, w2_bits, k):
    """Whole layer with scalar loops. x_bits [T][H], w1_bits [E][2I][H], w2_bits [E][H][I]
    are nested lists (or arrays) of bfloat16 bit patterns. Returns a dict of nested lists:
    ids, w, counts, offsets, perm, pos, a (bf16 bits [T*k][I]), yd (bits [T*k][H]),
    out (bits [T][H])."""
    T = len(x_bits)
    E = len(w1_bits)
    I = len(w1_bits[0]) // 2
    H = len(w1_bits[0][0])
    ids, w = route(logits, k)
    counts, offsets, perm, pos = plan(ids, E)
    a_bits = [None] * (T * k)
    y_bits = [None] * (T * k)
    for r in range(T * k):
        f = perm[r]
        t, j = divmod(f, k)
        e = ids[t][j]
        x = [Fraction(bf16_decode(v)) for v in x_bits[t]]
        arow = []
        for n in range(I):
            g = sum(x[h] * Fraction(bf16_decode(w1_bits[e][n][h])) for h in range(H))
            u = sum(x[h] * Fraction(bf16_decode(w1_bits[e][I + n][h])) for h in range(H))
            gf = float(g)
            s = Fraction(gf / (1.0 + math.exp(-gf))) if gf > -700 else Fraction(0)
            arow.append(bf16_nearest(s * u))
        a_bits[r] = [bf16_encode(v) for v in arow]
        yrow = []
        for n in range(H):
            acc = sum(arow[i] * Fraction(bf16_decode(w2_bits[e][n][i])) for i in range(I))
            yrow.append(bf16_nearest(acc))
        y_bits[r] = [bf16_encode(v) for v in yrow]
    out = []
    for t in range(T):
        row = []
        for n in range(H):
            acc = Fraction(0)
            for j in range(k):
                acc += Fraction(w[t][j]) * Fraction(bf16_decode(y_bits[pos[t * k + j]][n]))
            row.append(bf16_encode(bf16_nearest(acc)))
        out.append(row)
    return dict(ids=ids, w=w, counts=counts, offsets=offsets, perm=perm, pos=pos,
                a=a_bits, yd=y_bits, out=out)
