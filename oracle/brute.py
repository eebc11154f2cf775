"""Loop-per-element attention for tiny shapes, written apart from attn_ref.

TEST INFRASTRUCTURE ONLY.  Pure Python (math.exp, fractions), one output row
at a time, so a reader can follow each step against the pages:

  * decode: walk positions down from the row's own position, find each one's
    slot (p mod R in a ring, p itself in a linear cache), stop at the window
    or at the first unwritten position; two-pass softmax with unrounded p
    (TensorFold PR #1183, window_rows notes: 256-key chunk partials, fp32
    accumulation -- the chunking does not change the exact value);
  * prefill: the online softmax as a kernel runs it (PR #975, prompt
    attention commits: maxima and probabilities cross once per key block),
    block by block in ascending absolute position, rescaling the running sum
    and accumulator by exp(m_old - m_new) whenever the maximum moves, and
    rounding each p against the running maximum of its block.

attn_ref instead uses per-slot position formulas and the telescoped weights
exp(m_b - m_last); agreement of the two pins both.
"""
from __future__ import annotations

import math
from fractions import Fraction

P_FP32, P_BF16, P_BF16X2 = 0, 1, 2


def bf16_value(x: float) -> float:
    """bf16 round-to-nearest-even of a Python float, by exact fractions."""
    if x != x or x == 0.0 or math.isinf(x):
        return x
    a = Fraction(abs(x))
    e = 0
    while a >= 2 ** (e + 1):
        e += 1
    while a < Fraction(2) ** e:
        e -= 1
    e = max(e, -126)
    quantum = Fraction(2) ** (e - 7)
    n = round(a / quantum)           # Fraction.__round__: ties to even
    val = n * quantum
    if val >= 2 ** 128:
        return math.copysign(math.inf, x)
    return math.copysign(float(val), x)


def bf16_bits_value(b: int) -> float:
    """Value of a bf16 bit pattern (sign, 8 exponent bits, 7 mantissa bits)."""
    sign = -1.0 if b & 0x8000 else 1.0
    e = (b >> 7) & 0xFF
    m = b & 0x7F
    if e == 0xFF:
        return math.nan if m else sign * math.inf
    if e == 0:
        return sign * m * 2.0 ** -133
    return sign * (1 + m / 128.0) * 2.0 ** (e - 127)


def _round_p(p: float, p_mode: int) -> float:
    if p_mode == P_FP32:
        return p
    hi = bf16_value(p)
    if p_mode == P_BF16:
        return hi
    return hi + bf16_value(p - hi)


def _dot(a, b) -> float:
    s = 0.0
    for x, y in zip(a, b):
        s += x * y
    return s


def decode_row(q, kcache, vcache, t: int, ring: int, window: int, scale: float):
    """q [D]; kcache, vcache [cap][D] (floats) of one KV head; returns [D]."""
    cap = len(kcache)
    D = len(q)
    slots = []
    p = t
    while p >= 0:
        if window and t - p >= window:
            break
        if ring:
            if t - p >= cap:
                break
            slots.append(p % cap)
        else:
            if p < cap:
                slots.append(p)
        p -= 1
    if not slots:
        return [0.0] * D
    scores = [scale * _dot(q, kcache[s]) for s in slots]
    m = max(scores)
    e = [math.exp(s - m) for s in scores]
    l = sum(e)
    out = []
    for d in range(D):
        out.append(sum(e[i] * vcache[s][d] for i, s in enumerate(slots)) / l)
    return out


def prefill_row(q, keys, values, t: int, window: int, scale: float,
                p_mode: int, kb: int, hi: int | None = None):
    """q [D]; keys, values [n_pos][D] by absolute position; returns [D].
    hi: the row's last key (default its own position t)."""
    D = len(q)
    lo = max(0, t - window + 1) if window else 0
    hi = t if hi is None else hi
    m = -math.inf
    l = 0.0
    acc = [0.0] * D
    b = lo // kb
    while b * kb <= hi:
        first = max(lo, b * kb)
        last = min(hi, b * kb + kb - 1)
        s = [scale * _dot(q, keys[j]) for j in range(first, last + 1)]
        m_new = max(m, max(s))
        alpha = math.exp(m - m_new) if m != -math.inf else 0.0
        l *= alpha
        acc = [a * alpha for a in acc]
        for i, j in enumerate(range(first, last + 1)):
            p = math.exp(s[i] - m_new)
            l += p
            pr = _round_p(p, p_mode)
            for d in range(D):
                acc[d] += pr * values[j][d]
        m = m_new
        b += 1
    return [a / l for a in acc]
