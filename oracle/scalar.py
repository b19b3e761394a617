"""Pure-Python loop form of the oracle, for tiny inputs (test infrastructure only).

Same definitions as :mod:`oracle.batquant`, written element by element with
Python floats (fp64) and exactly-rounded sums (``math.fsum``), so the vectorised
form can be checked against an independent spelling of each step:

* P_i[a*r + c][a*r' + c'] = B_i[r][r'] * A[c][c'] built entry by entry
  [nubint.ai review, 提案手法: P_i = B_i (x) A];
* y_j = sum_k x_k P_i[k][j] (row-vector convention);
* clip to [sigmoid(beta_i) * min, sigmoid(alpha_i) * max] with fp32 bounds
  [en.papernotes.org, Key Designs §3];
* scale exponent floor(log2 amax) - 2 by repeated halving/doubling;
* nearest E2M1 value by exhaustive search over the eight magnitudes, ties to the
  even code [en.papernotes.org, Background & Motivation].
"""
from __future__ import annotations

import math
import struct
from typing import List, Optional, Sequence, Tuple

GRID = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)


def to_f32(x: float) -> float:
    """Round a Python float to the nearest fp32 value (ties to even)."""
    return struct.unpack("<f", struct.pack("<f", x))[0]


def f32_mul(a: float, b: float) -> float:
    """fp32 product of two fp32 values (the exact product rounded once)."""
    return to_f32(a * b)  # a*b of two 24-bit significands is exact in fp64


def bf16_to_float(bits: int) -> float:
    return struct.unpack("<f", struct.pack("<I", (int(bits) & 0xFFFF) << 16))[0]


def sigmoid_f32(logit: float) -> float:
    return to_f32(1.0 / (1.0 + math.exp(-float(logit))))


def floor_log2(x: float) -> int:
    """floor(log2 x) for x > 0 by repeated doubling/halving (exact)."""
    e = 0
    while x >= 2.0:
        x /= 2.0
        e += 1
    while x < 1.0:
        x *= 2.0
        e -= 1
    return e


def scale_exponent(amax: float) -> int:
    if amax == 0.0:
        return -127
    return max(-127, min(127, floor_log2(amax) - 2))


def round_e2m1(v: float) -> int:
    """Nearest of the 15 E2M1 values by exhaustive search; a tie goes to the even
    code; the sign bit follows the sign of v (so -0.1 -> code 8)."""
    mag = abs(v)
    best, best_d = 0, None
    for code, g in enumerate(GRID):
        d = abs(mag - g)
        if best_d is None or d < best_d or (d == best_d and code % 2 == 0):
            best, best_d = code, d
    return best | (8 if math.copysign(1.0, v) < 0 else 0)


def block_matrix(A: Sequence[Sequence[float]], Bi: Sequence[Sequence[float]]) -> List[List[float]]:
    a = len(A)
    b = len(Bi)
    n = a * b
    P = [[0.0] * n for _ in range(n)]
    for r in range(b):
        for rp in range(b):
            for c in range(a):
                for cp in range(a):
                    P[a * r + c][a * rp + cp] = float(Bi[r][rp]) * float(A[c][cp])
    return P


def invert(Mx: List[List[float]]) -> List[List[float]]:
    """Gauss-Jordan inverse with partial pivoting (fp64)."""
    n = len(Mx)
    aug = [list(map(float, row)) + [1.0 if i == j else 0.0 for j in range(n)] for i, row in enumerate(Mx)]
    for col in range(n):
        piv = max(range(col, n), key=lambda r: abs(aug[r][col]))
        aug[col], aug[piv] = aug[piv], aug[col]
        p = aug[col][col]
        if p == 0.0:
            raise ZeroDivisionError("singular")
        aug[col] = [v / p for v in aug[col]]
        for r in range(n):
            if r != col and aug[r][col] != 0.0:
                f = aug[r][col]
                aug[r] = [vr - f * vc for vr, vc in zip(aug[r], aug[col])]
    return [row[n:] for row in aug]


def quantize_block(y: Sequence[float], r_hi: float, r_lo: float) -> Tuple[List[int], int]:
    """Clip and quantise one block of 32 transformed values (fp64 in, decisions in
    fp32).  Returns (codes, scale byte)."""
    y32 = [to_f32(v) for v in y]
    hi, lo = max(y32), min(y32)
    u, l = f32_mul(r_hi, hi), f32_mul(r_lo, lo)
    z = [min(max(v, l), u) for v in y32]
    amax = max(abs(v) for v in z)
    e = scale_exponent(amax)
    codes = [round_e2m1(math.ldexp(v, -e)) for v in z]
    return codes, e + 127


def act_transform_quant(X_bits, A, B, alpha, beta):
    """Loop form of the online activation path.  Returns (codes[rows][K], scales[rows][nb])."""
    rows = len(X_bits)
    K = len(X_bits[0]) if rows else 0
    nb = K // 32
    Ps = [block_matrix(A, B[i]) for i in range(nb)]
    codes, scales = [], []
    for m in range(rows):
        x = [bf16_to_float(v) for v in X_bits[m]]
        crow, srow = [], []
        for i in range(nb):
            xb = x[32 * i: 32 * i + 32]
            P = Ps[i]
            y = [math.fsum(xb[k] * P[k][j] for k in range(32)) for j in range(32)]
            c, s = quantize_block(y, sigmoid_f32(alpha[i]), sigmoid_f32(beta[i]))
            crow += c
            srow.append(s)
        codes.append(crow)
        scales.append(srow)
    return codes, scales


def weight_prep(W_bits, A, B, walpha: Optional[Sequence] = None, wbeta: Optional[Sequence] = None):
    """Loop form of the offline weight side: W'_b = W_b P_i^-T, clip, quantise."""
    rows = len(W_bits)
    K = len(W_bits[0])
    nb = K // 32
    Pinv = [invert(block_matrix(A, B[i])) for i in range(nb)]
    codes, scales = [], []
    for n in range(rows):
        w = [bf16_to_float(v) for v in W_bits[n]]
        crow, srow = [], []
        for i in range(nb):
            wb = w[32 * i: 32 * i + 32]
            Q = Pinv[i]
            # (w P^-T)_j = sum_k w_k P^-1[j][k]
            y = [math.fsum(wb[k] * Q[j][k] for k in range(32)) for j in range(32)]
            rh = 1.0 if walpha is None else sigmoid_f32(walpha[n][i])
            rl = 1.0 if wbeta is None else sigmoid_f32(wbeta[n][i])
            c, s = quantize_block(y, rh, rl)
            crow += c
            srow.append(s)
        codes.append(crow)
        scales.append(srow)
    return codes, scales


def gemm_exact(xc, xs, wc, ws):
    """Exact W4A4 product with integers: every element is (2g) * 2^(byte-128)
    with 2g an integer, so each product is an integer times a power of two.
    Returns a list of lists of Python ``fractions.Fraction``."""
    from fractions import Fraction

    def val(code: int, sbyte: int) -> Fraction:
        twice = int(2 * GRID[code & 7])
        sgn = -1 if code & 8 else 1
        return Fraction(sgn * twice) * (Fraction(2) ** (sbyte - 128))

    M, K = len(xc), len(xc[0])
    N = len(wc)
    Xv = [[val(xc[m][k], xs[m][k // 32]) for k in range(K)] for m in range(M)]
    Wv = [[val(wc[n][k], ws[n][k // 32]) for k in range(K)] for n in range(N)]
    return [[sum((Xv[m][k] * Wv[n][k] for k in range(K)), Fraction(0)) for n in range(N)] for m in range(M)]
