"""Exact rational brute force of the MLP shard, for tiny shapes.

Independent of the oracle: it decodes bfloat16/e4m3 with its own code, forms
every dot product as an exact `fractions.Fraction`, evaluates GeLU with
Python's `math.erfc`, and rounds with its own integer round-half-even.
"""
from __future__ import annotations

import math
import struct
from fractions import Fraction

HALF = Fraction(1, 2)


def bf16_value(bits: int) -> Fraction:
    """Exact value of a bfloat16 bit pattern."""
    f = struct.unpack("<f", struct.pack("<I", (int(bits) & 0xFFFF) << 16))[0]
    return Fraction(f)


def e4m3_value(code: int) -> Fraction:
    """Exact value of an OCP e4m3 code (NaN codes are rejected)."""
    code = int(code) & 0xFF
    sign = -1 if code & 0x80 else 1
    E = (code >> 3) & 0xF
    m = code & 7
    if E == 15 and m == 7:
        raise ValueError("NaN code")
    if E == 0:
        return sign * Fraction(m, 2 ** 9)
    return sign * (1 + Fraction(m, 8)) * Fraction(2) ** (E - 7)


def round_half_even(v: Fraction, frac_bits: int, emin: int) -> Fraction:
    """Round v to the binary grid with `frac_bits` fraction bits, subnormal
    spacing 2^(emin - frac_bits), ties to even (no overflow handling)."""
    if v == 0:
        return Fraction(0)
    sign = -1 if v < 0 else 1
    a = abs(v)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, emin)
    q = Fraction(2) ** (e - frac_bits)
    n = a / q
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > HALF or (rem == HALF and fl % 2 == 1):
        fl += 1
    return sign * fl * q


def bf16_round(v: Fraction) -> Fraction:
    return round_half_even(v, 7, -126)


def gelu_float(x: float) -> float:
    """x·Φ(x) with Φ(x) = erfc(−x/√2)/2, in Python floats."""
    return x * 0.5 * math.erfc(-x / math.sqrt(2.0))


def matmul_exact(P, Q):
    """Exact product of two nested lists of Fractions."""
    n_in = len(Q)
    cols = len(Q[0])
    return [[sum((row[k] * Q[k][j] for k in range(n_in)), Fraction(0)) for j in range(cols)]
            for row in P]


def shard_exact(X_bits, A_bits, B_bits, N, rank):
    """(Z_i, Y_i) of rank `rank`: Z as exact Fractions on the bf16 grid, Y exact."""
    X = [[bf16_value(b) for b in row] for row in X_bits.tolist()]
    A = [[bf16_value(b) for b in row] for row in A_bits.tolist()]
    B = [[bf16_value(b) for b in row] for row in B_bits.tolist()]
    H = len(A[0])
    F = H // N
    lo, hi = rank * F, (rank + 1) * F
    A_i = [row[lo:hi] for row in A]
    B_i = B[lo:hi]
    S = matmul_exact(X, A_i)
    Z = [[bf16_round(Fraction(gelu_float(float(s)))) for s in row] for row in S]
    Y = matmul_exact(Z, B_i)
    return Z, Y


def shard_bias_exact(X_bits, A_bits, b1_bits, B_bits, N, rank):
    """(Z_i, Y_i) with the first layer's bias: Z_i = bf16(GeLU(S + b1_i)) with
    S + b1_i exact, Y_i = Z_i·B_i exact."""
    X = [[bf16_value(b) for b in row] for row in X_bits.tolist()]
    A = [[bf16_value(b) for b in row] for row in A_bits.tolist()]
    B = [[bf16_value(b) for b in row] for row in B_bits.tolist()]
    b1 = [bf16_value(b) for b in b1_bits.tolist()]
    H = len(A[0])
    F = H // N
    lo, hi = rank * F, (rank + 1) * F
    S = matmul_exact(X, [row[lo:hi] for row in A])
    Z = [[bf16_round(Fraction(gelu_float(float(s + b1[lo + j])))) for j, s in enumerate(row)]
         for row in S]
    return Z, matmul_exact(Z, B[lo:hi])


def fp8_shard_exact(Xq, sX, Aq, sA, Bq, sB, sZ_given=None):
    """Exact fp8 path on codes: returns (Z on the bf16 grid, Z codes, sZ, Y).
    sZ is Z's own amax scale unless sZ_given (a predicted scale) is passed."""
    X = [[e4m3_value(c) for c in row] for row in Xq.tolist()]
    A = [[e4m3_value(c) for c in row] for row in Aq.tolist()]
    B = [[e4m3_value(c) for c in row] for row in Bq.tolist()]
    S = matmul_exact(X, A)
    den = Fraction(float(sX)) * Fraction(float(sA))
    Z = [[bf16_round(Fraction(gelu_float(float(s / den)))) for s in row] for row in S]
    zmax = max(abs(z) for row in Z for z in row)
    import numpy as np
    sZ = np.float32(1.0) if zmax == 0 else np.float32(np.float32(448.0) / np.float32(float(zmax)))
    if sZ_given is not None:
        sZ = np.float32(sZ_given)
    codes = []
    Zq = []
    for row in Z:
        qrow = []
        for z in row:
            # product in fp32 (RNE), clamp, then one e4m3 rounding
            p = Fraction(float(np.float32(np.float32(float(z)) * sZ)))
            p = max(min(p, Fraction(448)), Fraction(-448))
            qrow.append(round_half_even(p, 3, -6))
        Zq.append(qrow)
    Y = matmul_exact(Zq, B)
    den2 = Fraction(float(sZ)) * Fraction(float(sB))
    Y = [[y / den2 for y in row] for row in Y]
    return Z, Zq, sZ, Y


def gelu_grad_float(x: float) -> float:
    """GeLU'(x) = Φ(x) + x·φ(x) with Python's math.erfc and math.exp."""
    return 0.5 * math.erfc(-x / math.sqrt(2.0)) + x * math.exp(-0.5 * x * x) / math.sqrt(2.0 * math.pi)


def shard_backward_exact(X_bits, A_bits, B_bits, dY_bits, N, rank):
    """Exact backward of one rank's shard: (Z, dS on the bf16 grid, dX, dA, dB)
    with every GEMM an exact rational sum."""
    H = A_bits.shape[1]
    F = H // N
    lo = rank * F
    X = [[bf16_value(v) for v in row] for row in X_bits.tolist()]
    A = [[bf16_value(v) for v in row[lo:lo + F]] for row in A_bits.tolist()]
    B = [[bf16_value(v) for v in row] for row in B_bits.tolist()[lo:lo + F]]
    dY = [[bf16_value(v) for v in row] for row in dY_bits.tolist()]
    S = matmul_exact(X, A)
    Bt = [list(col) for col in zip(*B)]
    dZ = matmul_exact(dY, Bt)
    Z = [[bf16_round(Fraction(gelu_float(float(s)))) for s in row] for row in S]
    dS = [[bf16_round(Fraction(float(dz) * gelu_grad_float(float(s)))) for dz, s in zip(rz, rs)]
          for rz, rs in zip(dZ, S)]
    At = [list(col) for col in zip(*A)]
    Xt = [list(col) for col in zip(*X)]
    Zt = [list(col) for col in zip(*Z)]
    return Z, dS, matmul_exact(dS, At), matmul_exact(Xt, dS), matmul_exact(Zt, dY)


def attention_exact(qkv_bits, B, S, heads, dh, causal=True):
    """Per-head scaled dot-product attention with pure-Python loops: exact
    rational scores q·k, each weight exp(score/√dh − max) by math.exp, the
    weighted sums with math.fsum.  qkv_bits: list of rows of bfloat16 bits in
    the head-major layout ([Q_h | K_h | V_h] per head).  Returns a list of
    float rows [B·S][heads·dh] (unrounded)."""
    val = [[float(bf16_value(b)) for b in row] for row in qkv_bits]
    inv = 1.0 / math.sqrt(dh)
    out = [[0.0] * (heads * dh) for _ in range(B * S)]
    for b in range(B):
        for h in range(heads):
            c = 3 * h * dh
            for t in range(S):
                q = [Fraction(x) for x in val[b * S + t][c:c + dh]]
                keys = range(t + 1) if causal else range(S)
                sc = []
                for j in keys:
                    k = val[b * S + j][c + dh:c + 2 * dh]
                    sc.append(float(sum(qi * Fraction(kj) for qi, kj in zip(q, k))) * inv)
                mx = max(sc)
                w = [math.exp(x - mx) for x in sc]
                den = math.fsum(w)
                for e in range(dh):
                    vs = [val[b * S + j][c + 2 * dh + e] for j in keys]
                    out[b * S + t][h * dh + e] = math.fsum(wi * vi for wi, vi in zip(w, vs)) / den
    return out


def e5m2_value(code: int) -> Fraction:
    """Exact value of a finite OCP e5m2 code (infinities and NaNs are rejected)."""
    code = int(code) & 0xFF
    sign = -1 if code & 0x80 else 1
    E = (code >> 2) & 0x1F
    m = code & 3
    if E == 31:
        raise ValueError("non-finite code")
    if E == 0:
        return sign * Fraction(m, 2 ** 16)
    return sign * (1 + Fraction(m, 4)) * Fraction(2) ** (E - 15)


def _quant_exact(vals, fmt):
    """Codes (as exact values) and scale of a list of rows under the tensor's own amax:
    s = MAX/amax as an fp32 division, the product in fp32, clamp, one RNE rounding."""
    import numpy as np
    top, frac_bits, emin = (448.0, 3, -6) if fmt == "e4m3" else (57344.0, 2, -14)
    amax = max(abs(v) for row in vals for v in row)
    s = np.float32(1.0) if amax == 0 else np.float32(np.float32(top) / np.float32(float(amax)))
    out = []
    for row in vals:
        q = []
        for v in row:
            p = Fraction(float(np.float32(np.float32(float(v)) * s)))
            p = max(min(p, Fraction(top)), Fraction(-top))
            q.append(round_half_even(p, frac_bits, emin))
        out.append(q)
    return out, s


def shard_backward_fp8_exact(X_bits, A_bits, B_bits, dY_bits, N, rank):
    """Exact fp8 backward in the hybrid formats: every tensor quantised with its
    own amax scale (e4m3 for X, A, B, Z; e5m2 for dY, dS), every GEMM an exact
    rational sum divided by its scales. Returns a dict of exact values."""
    H = A_bits.shape[1]
    F = H // N
    lo = rank * F
    X = [[bf16_value(v) for v in row] for row in X_bits.tolist()]
    A = [[bf16_value(v) for v in row] for row in A_bits.tolist()]
    B = [[bf16_value(v) for v in row] for row in B_bits.tolist()]
    dY = [[bf16_value(v) for v in row] for row in dY_bits.tolist()]
    Xq, sX = _quant_exact(X, "e4m3")
    Aq, sA = _quant_exact(A, "e4m3")
    Bq, sB = _quant_exact(B, "e4m3")
    dYq, sdY = _quant_exact(dY, "e5m2")
    Aq_i = [row[lo:lo + F] for row in Aq]
    Bq_i = Bq[lo:lo + F]
    S = [[v / (Fraction(float(sX)) * Fraction(float(sA))) for v in row] for row in matmul_exact(Xq, Aq_i)]
    Bt = [list(col) for col in zip(*Bq_i)]
    dZ = [[v / (Fraction(float(sdY)) * Fraction(float(sB))) for v in row] for row in matmul_exact(dYq, Bt)]
    Z = [[bf16_round(Fraction(gelu_float(float(s)))) for s in row] for row in S]
    dS = [[bf16_round(Fraction(float(dz) * gelu_grad_float(float(s)))) for dz, s in zip(rz, rs)]
          for rz, rs in zip(dZ, S)]
    dSq, sdS = _quant_exact(dS, "e5m2")
    Zq, sZ = _quant_exact(Z, "e4m3")
    At = [list(col) for col in zip(*Aq_i)]
    Xt = [list(col) for col in zip(*Xq)]
    Zt = [list(col) for col in zip(*Zq)]
    def scaled(M, a, b):
        den = Fraction(float(a)) * Fraction(float(b))
        return [[v / den for v in row] for row in M]
    return {"sX": sX, "sA": sA, "sB": sB, "sdY": sdY, "sdS": sdS, "sZ": sZ,
            "Xq": Xq, "Aq_i": Aq_i, "Bq_i": Bq_i, "dYq": dYq, "S": S, "dZ": dZ, "Z": Z, "dS": dS,
            "dSq": dSq, "Zq": Zq,
            "dX": scaled(matmul_exact(dSq, At), sdS, sA),
            "dA": scaled(matmul_exact(Xt, dSq), sX, sdS),
            "dB": scaled(matmul_exact(Zt, dYq), sZ, sdY)}
