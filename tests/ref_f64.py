"""Independent float64 brute force of the MoE layer, used to pin the oracle.

Written from the same pages as the oracle but with none of its code: it works
on the generator's unpacked codes (not on packed bytes), evaluates every dot
product as an exact integer sum followed by float64 arithmetic, and takes
quantisation decisions in float64.  Stage functions accept the oracle's
intermediate values so that each stage can be checked against its own error
bound.
"""
from __future__ import annotations

import math
from fractions import Fraction

import numpy as np

U32 = 2.0 ** -24  # unit roundoff of binary32


def ulp32(v):
    """Spacing of binary32 numbers at |v| (vectorised)."""
    a = np.abs(np.asarray(v, dtype=np.float64))
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -149)))
    return np.where(a >= 2.0 ** -126, 2.0 ** (e - 23), 2.0 ** -149)


def round_half_away(r):
    r = np.asarray(r, dtype=np.float64)
    return np.sign(r) * np.floor(np.abs(r) + 0.5)


def q8_0_f64(v, near=1e-4):
    """Q8_0 with float64 decisions; returns (q, d, near_tie_mask)."""
    v = np.asarray(v, dtype=np.float64)
    n = v.shape[-1]
    vb = v.reshape(v.shape[:-1] + (n // 32, 32))
    d = np.max(np.abs(vb), axis=-1) / 127.0
    with np.errstate(divide="ignore", invalid="ignore"):
        r = np.where(d[..., None] > 0, vb / d[..., None], 0.0)
    q = np.clip(round_half_away(r), -127, 127)
    frac = np.abs(r) - np.floor(np.abs(r))
    nt = np.abs(frac - 0.5) < near
    return q.reshape(v.shape), d, nt.reshape(v.shape)


def block_isums(codes, q):
    """isum[..., b] = sum_j codes*q over each 32-block, exact (int64)."""
    codes = np.asarray(codes, dtype=np.int64)
    q = np.asarray(q, dtype=np.int64)
    n = codes.shape[-1]
    prod = codes * q
    return prod.reshape(prod.shape[:-1] + (n // 32, 32)).sum(-1)


def matvec_q(codes, scales, q, d):
    """y_r = s_r * sum_b d_b * isum_{r,b} in float64, with the bound of a
    binary32 fma chain over the blocks followed by the row-scale product:
    |y32 - y64| <= ((nb + 1) * u) * sum_b |d_b isum_b| * |s_r| (+ tiny)."""
    isum = block_isums(codes, q[None, :]).astype(np.float64)     # [R, nb]
    terms = isum * np.asarray(d, np.float64)[None, :]
    nb = terms.shape[1]
    s = np.asarray(scales, np.float64)
    y = np.array([math.fsum(t) for t in terms]) * s
    bound = (nb + 2) * U32 * np.abs(terms).sum(1) * np.abs(s) + 2.0 ** -149
    return y, bound


def matvec_qg(codes, gscales, q, d):
    """Group-scaled rows: gscales [R, n / group], code j of row r weighted by
    gscales[r, j / group]: y_r = sum_b d_b * s_{r, g(b)} * isum_{r,b} in
    float64, with the bound of a binary32 fma chain over the blocks whose
    multipliers d_b * s are themselves rounded:
    |y32 - y64| <= ((nb + 2) * u) * sum_b |d_b s isum_b| (+ tiny)."""
    isum = block_isums(codes, q[None, :]).astype(np.float64)     # [R, nb]
    gs = np.asarray(gscales, np.float64)
    nb = isum.shape[1]
    per_block = np.repeat(gs, nb // gs.shape[1], axis=1)          # [R, nb]
    terms = isum * np.asarray(d, np.float64)[None, :] * per_block
    y = np.array([math.fsum(t) for t in terms])
    bound = (nb + 3) * U32 * np.abs(terms).sum(1) + 2.0 ** -149
    return y, bound


def _matvec_any(codes, scales, q, d):
    s = np.asarray(scales)
    return matvec_qg(codes, s, q, d) if s.ndim == 2 else matvec_q(codes, s, q, d)


def swiglu64(g, u):
    g = np.asarray(g, np.float64)
    u = np.asarray(u, np.float64)
    return g / (1.0 + np.exp(-g)) * u


def sigmoid64(v):
    return 1.0 / (1.0 + np.exp(-np.asarray(v, np.float64)))


def full_sort_topk(score, K):
    """First K experts of a full stable sort by (score desc, id asc)."""
    score = np.asarray(score, np.float64)
    ids = np.arange(score.shape[-1])
    order = np.lexsort((ids, -score))
    return order[:K]


def expert64(parts, qx, dx, qh_override=None, near=1e-4):
    """One expert on one token in float64 from unpacked codes.

    parts: dict with gate/up [I,H] codes, down [H,I] codes, s_gate/s_up/s_down
    (per-row vectors, or [rows, cols / group] arrays of group scales).
    Returns dict g, u, h, qh, dh, y, and nflips: the number of h codes taken
    from qh_override because the float64 value sits within `near` of a
    rounding boundary (only when qh_override is given)."""
    g, _ = _matvec_any(parts["gate"], parts["s_gate"], qx, dx)
    u, _ = _matvec_any(parts["up"], parts["s_up"], qx, dx)
    h = swiglu64(g, u)
    qh, dh, nt = q8_0_f64(h, near)
    nflips = 0
    if qh_override is not None:
        take = nt & (qh != qh_override)
        nflips = int(take.sum())
        qh = np.where(nt, qh_override, qh)
    y, _ = _matvec_any(parts["down"], parts["s_down"], qh, dh)
    return {"g": g, "u": u, "h": h, "qh": qh, "dh": dh, "y": y, "nflips": nflips}


def rn32(x: Fraction) -> Fraction:
    """Round an exact rational to the nearest binary32 (ties to even)."""
    if x == 0:
        return Fraction(0)
    sign = -1 if x < 0 else 1
    a = abs(x)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    quantum = Fraction(2) ** (max(e, -126) - 23)
    m = a / quantum
    fl = m.numerator // m.denominator
    rem = m - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return sign * fl * quantum
