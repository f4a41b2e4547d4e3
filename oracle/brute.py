"""Brute-force twin of the oracle, in pure Python loops, for tiny inputs only.

TEST INFRASTRUCTURE ONLY (same import rule as ``oracle/kivi.py``).

It computes the same quantizer as ``oracle.kivi`` through a different arithmetic route:
Python floats (IEEE binary64) with an explicit rounding to binary32 or binary16 after every
operation, done with ``struct``. Rounding a binary64 result of one +, -, * or / on binary32
operands back to binary32 gives the correctly rounded binary32 result (binary64 carries more
than 2*24+2 significant bits), so this route reproduces IEEE single precision without numpy.
Attention is written as explicit sums with ``math.exp``.

Sources are the same passages as ``oracle.kivi``: "Changelog" v0.8.0 (KIVI: per-channel
keys, per-token values, residual window), v0.42.0 (codes plus per-group (scale, zero),
softmax attention over the reconstruction), v0.30.0 (lo/scale, fp16 metadata; SKVQ-adapted:
channel reordering by range, per-group clip search), v0.9.0 (KIVI-Sink: high key-norm tokens
kept in fp16, outside the group statistics).
"""
from __future__ import annotations

import math
import struct


def r32(x: float) -> float:
    """Round a Python float to the nearest binary32 value (ties to even)."""
    return struct.unpack("<f", struct.pack("<f", x))[0]


def r16(x: float) -> float:
    """Round a Python float to the nearest binary16 value (ties to even, subnormals kept)."""
    return struct.unpack("<e", struct.pack("<e", x))[0]


def round_half_even(x: float) -> float:
    """Nearest integer, ties to the even neighbour (Python's round on floats does this)."""
    return float(round(x))


def quantize_group(xs: list[float], bits: int, skip=()):
    """One group of fp16 values -> (codes, scale16, zero16) with one rounding per op.

    Elements whose index is in ``skip`` are left out of the min and max (they still get codes).
    """
    L = float(2 ** bits - 1)
    kept = [x for i, x in enumerate(xs) if i not in skip]
    lo = r32(min(kept) + 0.0)
    hi = r32(max(kept) + 0.0)
    s32 = r32(r32(hi - lo) / L)
    scale16 = r16(s32)
    zero16 = r16(lo)
    codes = []
    if scale16 == 0.0:
        return [0] * len(xs), scale16, zero16
    inv = r32(1.0 / scale16)
    for x in xs:
        t = r32(r32(x - lo) * inv)
        c = round_half_even(t)
        c = min(max(c, 0.0), L)
        codes.append(int(c))
    return codes, scale16, zero16


def encode_keys(K: list[list[float]], bits: int, g: int, sinks=()):
    """K[t][d] -> codes[t][d], scale[j][d], zero[j][d]; group = g tokens of one channel.
    Tokens in ``sinks`` stay out of their groups' min and max."""
    T, D = len(K), len(K[0])
    codes = [[0] * D for _ in range(T)]
    scale = [[0.0] * D for _ in range(T // g)]
    zero = [[0.0] * D for _ in range(T // g)]
    for j in range(T // g):
        for d in range(D):
            col = [K[j * g + i][d] for i in range(g)]
            skip = {i for i in range(g) if j * g + i in sinks}
            c, s, z = quantize_group(col, bits, skip)
            scale[j][d], zero[j][d] = s, z
            for i in range(g):
                codes[j * g + i][d] = c[i]
    return codes, scale, zero


def encode_values(V: list[list[float]], bits: int, g: int):
    """V[t][d] -> codes[t][d], scale[t][k], zero[t][k]; group = g channels of one token."""
    T, D = len(V), len(V[0])
    codes = [[0] * D for _ in range(T)]
    scale = [[0.0] * (D // g) for _ in range(T)]
    zero = [[0.0] * (D // g) for _ in range(T)]
    for t in range(T):
        for k in range(D // g):
            c, s, z = quantize_group(V[t][k * g:(k + 1) * g], bits)
            scale[t][k], zero[t][k] = s, z
            codes[t][k * g:(k + 1) * g] = c
    return codes, scale, zero


def select_sinks(K: list[list[float]], n: int) -> list[int]:
    """Positions of the n rows of largest squared norm (binary32 squares added channel by
    channel), earlier row first on equal norms; returned in ascending order."""
    norms = []
    for t, row in enumerate(K):
        acc = 0.0
        for x in row:
            acc = r32(acc + r32(x * x))
        norms.append((-acc, t))
    return sorted(t for _, t in sorted(norms)[:n])


def clipped_group_quant(xs: list[float], bits: int, fracs: list[float]):
    """One group with the clip search: for each clip fraction c (window [lo + d, hi - d],
    d = (hi - lo) * c), quantize with the stored fp16 step and low end and take the fp32 sum
    of squared errors in element order; the smallest error wins, the first on ties.
    Returns (codes, scale16, zero16, index of the chosen fraction)."""
    L = float(2 ** bits - 1)
    lo = r32(min(xs) + 0.0)
    hi = r32(max(xs) + 0.0)
    best = None
    for k, c in enumerate(fracs):
        d = r32(r32(hi - lo) * c)
        lo_c, hi_c = r32(lo + d), r32(hi - d)
        scale16 = r16(r32(r32(hi_c - lo_c) / L))
        zero16 = r16(lo_c)
        if scale16 == 0.0:
            codes = [0] * len(xs)
        else:
            inv = r32(1.0 / scale16)
            codes = [int(min(max(round_half_even(r32(r32(x - zero16) * inv)), 0.0), L)) for x in xs]
        err = 0.0
        for x, cd in zip(xs, codes):
            xh = r32(r32(cd * scale16) + zero16)
            diff = r32(x - xh)
            err = r32(err + r32(diff * diff))
        if best is None or err < best[4]:
            best = (codes, scale16, zero16, k, err)
    return best[:4]


def channel_permutation(rows: list[list[float]]) -> list[int]:
    """Channels in ascending order of binary32 (max - min) over the rows, stable on ties."""
    D = len(rows[0])
    rng = [r32(max(r[d] for r in rows) - min(r[d] for r in rows)) for d in range(D)]
    return sorted(range(D), key=lambda d: (rng[d], d))


def attend(q: list[float], keys: list[list[float]], values: list[list[float]], sm_scale: float = 1.0):
    """softmax(sm_scale * q . k_t) weighted sum of v_t, with explicit loops."""
    scores = [sm_scale * sum(qd * kd for qd, kd in zip(q, k)) for k in keys]
    m = max(scores)
    w = [math.exp(s - m) for s in scores]
    tot = sum(w)
    D = len(values[0])
    return [sum(w[t] * values[t][d] for t in range(len(values))) / tot for d in range(D)]


def kitty_encode_keys(K: list[list[float]], n_hi: int, hi_bits: int, lo_bits: int, g: int):
    """Kitty keys ("Changelog" v0.11.0) by brute force: for key group j, each channel's
    population variance over tokens 0 .. (j+1)g - 1, recomputed from scratch in exact
    rational arithmetic (mean first, then the mean squared deviation); the n_hi channels of
    largest variance (lower index first on ties) are quantized at hi_bits, the rest at lo_bits.
    Returns codes[t][d], scale[j][d], zero[j][d], hi[j][d]."""
    from fractions import Fraction

    T, D = len(K), len(K[0])
    codes = [[0] * D for _ in range(T)]
    scale, zero, hi = [], [], []
    for j in range(T // g):
        n = (j + 1) * g
        var = []
        for d in range(D):
            xs = [Fraction(K[t][d]) for t in range(n)]
            mean = sum(xs) / n
            var.append(sum((x - mean) ** 2 for x in xs) / n)
        order = sorted(range(D), key=lambda d: (-var[d], d))
        top = set(order[:n_hi])
        srow, zrow, hrow = [0.0] * D, [0.0] * D, [False] * D
        for d in range(D):
            col = [K[j * g + i][d] for i in range(g)]
            c, s, z = quantize_group(col, hi_bits if d in top else lo_bits)
            srow[d], zrow[d], hrow[d] = s, z, d in top
            for i in range(g):
                codes[j * g + i][d] = c[i]
        scale.append(srow)
        zero.append(zrow)
        hi.append(hrow)
    return codes, scale, zero, hi
