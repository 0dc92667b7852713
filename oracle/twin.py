"""A pure-Python twin of the C oracle's layout, dispatch (BF16 and FP8),
un-permute and combine, for tiny inputs.  TEST INFRASTRUCTURE ONLY, like the
rest of oracle/: it exists so that the C oracle can be cross-checked against
an independently written second implementation of the same definitions (a
consistency check, not a pin: the pins are the independent facts in the
oracle tests).  It uses Python integers, lists, struct and fractions only --
no numpy arithmetic and nothing from ep_oracle.c.

Pages: [Perplexity blog] "Lower latency and higher throughput with multi-node
DeepSeek deployment", "MoE-beirari" (routing summed per expert), "Magntölun"
(per-128-element activation scales, amax/448) and "Sérfræðinga-samsíðun"
(weighted sum of the routed results); [DeepEP overview] "DeepSeek merilis
library open source DeepEP ...", "Pola penggunaan ..." (dispatch, handle,
combine).

Arithmetic.  binary32 values are Python floats holding binary32 numbers.  A
binary32 quotient is computed as a binary64 quotient rounded to binary32:
for +, -, *, / of binary32 operands the binary64 result rounded again to
binary32 equals the correctly rounded binary32 result (binary64 carries at
least 2*24 + 2 significand bits).  The fused multiply-add of the combine is
not covered by that argument, so it is evaluated exactly with Fractions and
rounded once.
"""
from __future__ import annotations

import math
import struct
from fractions import Fraction


# ------------------------------------------------------------ binary32 / bf16
def f32(v: float) -> float:
    """Round a binary64 value to binary32 (nearest, ties to even)."""
    return struct.unpack("<f", struct.pack("<f", v))[0]


def f32_bits(v: float) -> int:
    return struct.unpack("<I", struct.pack("<f", v))[0]


def bits_f32(b: int) -> float:
    return struct.unpack("<f", struct.pack("<I", b & 0xFFFFFFFF))[0]


def bf16_to_f32(b: int) -> float:
    return bits_f32(b << 16)


def f32_to_bf16(v: float) -> int:
    """binary32 -> bf16 bits, nearest with ties to even (NaN stays NaN)."""
    u = f32_bits(v)
    if (u & 0x7FFFFFFF) > 0x7F800000:
        return (u >> 16) | 0x40
    keep, rest = u >> 16, u & 0xFFFF
    if rest > 0x8000 or (rest == 0x8000 and keep & 1):
        keep += 1
    return keep & 0xFFFF


def round_f32_exact(q: Fraction) -> float:
    """The binary32 number nearest to the rational q (ties to even), or +-inf
    past the largest finite value."""
    if q == 0:
        return 0.0
    sign = -1.0 if q < 0 else 1.0
    a = abs(q)
    # exponent e with 2^e <= a < 2^(e+1)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    e = max(e, -126)                       # subnormals share the spacing 2^-149
    ulp = Fraction(2) ** (e - 23)
    n, r = divmod(a, ulp)
    n = int(n)
    if r > ulp / 2 or (r == ulp / 2 and n % 2 == 1):
        n += 1
    mag = n * ulp
    if mag > Fraction((2 - Fraction(1, 2 ** 23))) * Fraction(2) ** 127:
        return sign * float("inf")
    return sign * float(mag)


# ------------------------------------------------------------------ E4M3
def e4m3_value(code: int) -> float:
    """Value of an OCP E4M3 code (bias 7, subnormals m * 2^-9, no infinity)."""
    s = -1.0 if code & 0x80 else 1.0
    e, m = (code >> 3) & 0xF, code & 7
    if e == 0xF and m == 7:
        return float("nan")
    if e == 0:
        return s * m * 2.0 ** -9
    return s * (1 + m / 8) * 2.0 ** (e - 7)


_POS_CODES = [c for c in range(0x7F)]          # 0x00 .. 0x7E: every finite magnitude


def e4m3_encode(v: float) -> int:
    """Nearest finite E4M3 code by brute force over the 127 magnitudes, ties
    to the code with an even mantissa; beyond 448 the code of 448; the sign
    of zero is kept; a NaN gives the NaN code S.1111.111."""
    sign = 0x80 if (f32_bits(v) >> 31) else 0
    if v != v:
        return sign | 0x7F
    a = abs(v)
    best = 0
    for c in _POS_CODES:
        d, db = abs(e4m3_value(c) - a), abs(e4m3_value(best) - a)
        if d < db or (d == db and (c & 1) == 0 and (best & 1) == 1):
            best = c
    return sign | best


# ------------------------------------------------------------------ layout
def layout(topk_idx, E: int, R: int):
    """Counts, offsets, rank ranges and the stable slot of every pair, by a
    sequential pass (topk_idx: list of T lists of k ints)."""
    pairs = [e for row in topk_idx for e in row]
    cnt = [0] * E
    for e in pairs:
        cnt[e] += 1
    off = [0] * (E + 1)
    for e in range(E):
        off[e + 1] = off[e] + cnt[e]
    El = E // R
    roff = [off[r * El] for r in range(R)] + [off[E]]
    rcnt = [roff[r + 1] - roff[r] for r in range(R)]
    fill = [0] * E
    slot = [0] * len(pairs)
    src = [0] * len(pairs)
    for p, e in enumerate(pairs):
        slot[p] = off[e] + fill[e]
        fill[e] += 1
        src[slot[p]] = p
    return dict(expert_counts=cnt, expert_offsets=off, rank_counts=rcnt, rank_offsets=roff,
                slot_of=slot, src_of=src)


def _row(L, p, E, R):
    """(rank, row) of pair p."""
    s = L["slot_of"][p]
    r = max(i for i in range(R) if L["rank_offsets"][i] <= s)
    return r, s - L["rank_offsets"][r]


# ---------------------------------------------------------------- dispatch
def dispatch_bf16(x, topk_idx, E, R, L):
    """recv[r] = list of rows (lists of bf16 bits) in row order."""
    k = len(topk_idx[0])
    recv = [[None] * L["rank_counts"][r] for r in range(R)]
    for t, row in enumerate(x):
        for j in range(k):
            r, i = _row(L, t * k + j, E, R)
            recv[r][i] = list(row)
    return recv


def _ieee_div(x: float, y: float) -> float:
    """x / y with IEEE results for the operands Python leaves to exceptions
    or does not reach here (y is never 0: an all-zero block is handled
    before)."""
    if x != x or y != y or (math.isinf(x) and math.isinf(y)):
        return math.nan
    return x / y


def quantize_row(row):
    """One token row of bf16 bits -> (codes, scales): per 128 channels
    a = max|x| (NaN if the block holds a NaN), s = a/448 in binary32, code =
    E4M3(binary32 x/s) with IEEE division (x/inf = 0, inf/inf = NaN); a = 0
    gives s = 0 and codes 0."""
    codes, scales = [], []
    for b0 in range(0, len(row), 128):
        vals = [bf16_to_f32(v) for v in row[b0:b0 + 128]]
        a = math.nan if any(v != v for v in vals) else max(abs(v) for v in vals)
        if a == 0:
            scales.append(0.0)
            codes.extend([0] * len(vals))
            continue
        s = f32(a / 448.0)
        scales.append(s)
        codes.extend(e4m3_encode(f32(_ieee_div(v, s))) for v in vals)
    return codes, scales


def dispatch_fp8(x, topk_idx, E, R, L):
    k = len(topk_idx[0])
    rq = [[None] * L["rank_counts"][r] for r in range(R)]
    rs = [[None] * L["rank_counts"][r] for r in range(R)]
    for t, row in enumerate(x):
        q, s = quantize_row(row)
        for j in range(k):
            r, i = _row(L, t * k + j, E, R)
            rq[r][i], rs[r][i] = q, s
    return rq, rs


# -------------------------------------------------------- unpermute/combine
def unpermute(recv_y, topk_idx, E, R, L):
    k = len(topk_idx[0])
    out = []
    for p in range(len(topk_idx) * k):
        r, i = _row(L, p, E, R)
        out.append(list(recv_y[r][i]))
    return out


def combine(recv_y, topk_idx, E, R, L, weights=None):
    """out[t][h] = bf16(fold over j of fma(w, y, acc) from +0), each fma the
    exact w*y + acc rounded once to binary32."""
    k = len(topk_idx[0])
    H = len(recv_y[next(r for r in range(R) if recv_y[r])][0])
    out = []
    for t in range(len(topk_idx)):
        rows = []
        for j in range(k):
            r, i = _row(L, t * k + j, E, R)
            rows.append(recv_y[r][i])
        orow = []
        for h in range(H):
            acc = 0.0
            for j in range(k):
                w = 1.0 if weights is None else weights[t][j]
                y = bf16_to_f32(rows[j][h])
                acc = round_f32_exact(Fraction(w) * Fraction(y) + Fraction(acc))
            orow.append(f32_to_bf16(acc))
        out.append(orow)
    return out
