"""Decode prologue of one stacked projection row: the RMS norms of q and k,
their rotary embedding, and the unit RMS norm of v.

TEST INFRASTRUCTURE ONLY: called by tests/ and by nothing on the product
path.  Float64 at the rounding points (the bf16 points of MLX's gemma
norms), with the range fp32 allows around each of them.

What it computes (TensorFold PR #1183 squashed commit bodies, the qk_rows
note: q and k are bf16(w * bf16(x * inv)) before the rotary embedding, as the
Metal prologue computes them, and v may be normed by a unit RMS norm; the
prologue's own check compares every output with float64's value at the
rounding points as a range over the fp32 inverse's spread and cosf's ulps;
PR #975 decode commits: the partial kernel norms and ropes its query heads
from the stacked row and writes the row's key and value to the cache).  For
a row at position t and one head's D bf16 values x:

  inv = 1 / sqrt(mean(x^2) + eps)
  y   = bf16(w * bf16(x * inv))        (q and k; w: bf16 [D], the head's scale)
  v'  = bf16(x * inv)                  (v, when the unit norm is asked for;
                                        else v unchanged)
  rotary embedding of y at t, pairs (i, i + D/2) for i < D/2:
      a = fp32(fp32(t) * inv_freq[i])  (inv_freq: fp32 [D/2], the caller's
                                        table; 0 leaves a pair unrotated)
      out_i       = bf16(y_i cos a - y_{i+D/2} sin a)
      out_{i+D/2} = bf16(y_{i+D/2} cos a + y_i sin a)

Readings where the pages are silent: eps and the frequency table are the
caller's; the pairs are the two halves of the head (the non-interleaved
form); the angle is the fp32 product the pages' MLX code forms.

The range: inv within EPS_INV relative of float64's (an fp32 sum of D
squares, square root and division); x * inv rounded once in fp32; cos and
sin within COS_ABS of float64's cos/sin of the same fp32 angle; the rotary
products and sum within ROPE_REL of |y_i cos| + |y_{i+D/2} sin|.  Each output
gets the lowest and highest bf16 an fp32 kernel can produce (ordered keys),
and the bf16 of the float64 value (exact inv, exact cos/sin) as its center.
"""
from __future__ import annotations

import numpy as np

from oracle import bf16

EPS_INV = 2.0 ** -16
FP32_REL = 2.0 ** -24
COS_ABS = 2.0 ** -22
ROPE_REL = 2.0 ** -22


def rms_inv(x: np.ndarray, eps: float) -> np.ndarray:
    """1 / sqrt(mean(x^2) + eps) over the last axis, float64 (eps as fp32)."""
    x = np.asarray(x, dtype=np.float64)
    return 1.0 / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + float(np.float32(eps)))


def angles(t: int, inv_freq) -> np.ndarray:
    """fp32(fp32(t) * inv_freq[i]) as float64."""
    f = np.asarray(inv_freq, dtype=np.float32)
    return (np.float32(t) * f).astype(np.float32).astype(np.float64)


def _keys_of(lo, hi):
    """Ordered keys of bf16_RNE at both ends of a value interval."""
    return bf16.ordered(bf16.bits_from_f64(lo)), bf16.ordered(bf16.bits_from_f64(hi))


def _values_between(klo, khi):
    """Up to three bf16 values whose ordered keys run from klo to khi (the
    candidates of an intermediate rounding point): value arrays lo, mid, hi."""
    def val(k):
        k = np.asarray(k, dtype=np.int32)
        b = np.where(k >= 0x8000, k - 0x8000, (0x7FFF - k) | 0x8000).astype(np.uint16)
        return bf16.f64_from_bits(b)
    if np.any(khi - klo > 2):
        raise ValueError("intermediate rounding spread over more than three bf16 values")
    return val(klo), val(np.minimum(klo + 1, khi)), val(khi)


def normed(x_bits, w_bits, eps: float):
    """bf16(w * bf16(x * inv)) (w None: bf16(x * inv)) per row of the last
    axis: center value, and the lowest / highest value an fp32 kernel can
    produce."""
    x = bf16.f64_from_bits(x_bits)
    inv = rms_inv(x, eps)
    p = x * inv
    hw = np.abs(p) * (EPS_INV + FP32_REL)
    t_c = bf16.round_f64(p)
    klo, khi = _keys_of(p - hw, p + hw)
    cands = _values_between(klo, khi)
    if w_bits is None:
        return t_c, cands[0], cands[2]
    w = bf16.f64_from_bits(w_bits)
    ys = [bf16.round_f64(w * c) for c in cands]
    return bf16.round_f64(w * t_c), np.minimum.reduce(ys), np.maximum.reduce(ys)


def _mul_range(alo, ahi, blo, bhi):
    c = [alo * blo, alo * bhi, ahi * blo, ahi * bhi]
    return np.minimum.reduce(c), np.maximum.reduce(c)


def rope(y_c, y_lo, y_hi, t: int, inv_freq):
    """Rotary embedding of normed values (center and range per element) at
    position t: returns (center bits, lowest key, highest key)."""
    D = y_c.shape[-1]
    h = D // 2
    a = angles(t, inv_freq)
    c0, s0 = np.cos(a), np.sin(a)
    ya_c, yb_c = y_c[..., :h], y_c[..., h:]
    out_c = np.concatenate([ya_c * c0 - yb_c * s0, yb_c * c0 + ya_c * s0], axis=-1)
    clo, chi = c0 - COS_ABS, c0 + COS_ABS
    slo, shi = s0 - COS_ABS, s0 + COS_ABS
    ya_lo, ya_hi = y_lo[..., :h], y_hi[..., :h]
    yb_lo, yb_hi = y_lo[..., h:], y_hi[..., h:]
    # out_i = ya c - yb s ; out_{i+h} = yb c + ya s
    p1 = _mul_range(ya_lo, ya_hi, clo, chi)
    p2 = _mul_range(yb_lo, yb_hi, slo, shi)
    p3 = _mul_range(yb_lo, yb_hi, clo, chi)
    p4 = _mul_range(ya_lo, ya_hi, slo, shi)
    mag_a = np.maximum(np.abs(ya_lo), np.abs(ya_hi))
    mag_b = np.maximum(np.abs(yb_lo), np.abs(yb_hi))
    err = ROPE_REL * (mag_a * (np.abs(c0) + COS_ABS) + mag_b * (np.abs(s0) + COS_ABS))
    err2 = ROPE_REL * (mag_b * (np.abs(c0) + COS_ABS) + mag_a * (np.abs(s0) + COS_ABS))
    lo = np.concatenate([p1[0] - p2[1] - err, p3[0] + p4[0] - err2], axis=-1)
    hi = np.concatenate([p1[1] - p2[0] + err, p3[1] + p4[1] + err2], axis=-1)
    klo, khi = _keys_of(lo, hi)
    return bf16.bits_from_f64(out_c), klo, khi


def qkv_prep(qkv_bits, q_w_bits, k_w_bits, inv_freq, eps: float, v_norm: int, pos,
             n_q_heads: int, n_kv_heads: int, head_dim: int):
    """Prologue of S stacked rows qkv [S][(Hq + 2 Hkv) D] (bf16 bits) at
    positions pos[s].  Returns dict with, for q [S][Hq][D], k and v
    [S][Hkv][D]: '<x>_bits' (center), '<x>_lo', '<x>_hi' (ordered keys)."""
    S = qkv_bits.shape[0]
    Hq, Hkv, D = n_q_heads, n_kv_heads, head_dim
    rows = np.asarray(qkv_bits, dtype=np.uint16).reshape(S, Hq + 2 * Hkv, D)
    out = {}
    for name, sl, w in (("q", slice(0, Hq), q_w_bits), ("k", slice(Hq, Hq + Hkv), k_w_bits)):
        xb = rows[:, sl]
        c, lo, hi = normed(xb, w, eps)
        bits, klo, khi = [], [], []
        for s in range(S):
            b, l_, h_ = rope(c[s], lo[s], hi[s], int(pos[s]), inv_freq)
            bits.append(b)
            klo.append(l_)
            khi.append(h_)
        out[name + "_bits"] = np.stack(bits)
        out[name + "_lo"] = np.stack(klo)
        out[name + "_hi"] = np.stack(khi)
    vb = rows[:, Hq + Hkv:]
    if v_norm:
        c, lo, hi = normed(vb, None, eps)
        out["v_bits"] = bf16.bits_from_f64(c)
        out["v_lo"], out["v_hi"] = _keys_of(lo, hi)
    else:
        out["v_bits"] = vb.copy()
        out["v_lo"] = out["v_hi"] = bf16.ordered(vb)
    return out


def check_range(gpu_bits, center_bits, klo, khi) -> dict:
    """Every GPU output within its [lo, hi] bf16 range; the share equal to
    the center's bf16 is reported (a systematic error drops it far)."""
    g = bf16.ordered(np.asarray(gpu_bits, dtype=np.uint16))
    inside = (g >= klo) & (g <= khi)
    return {"n": int(g.size), "fails": int(np.sum(~inside)), "ok": bool(np.all(inside)),
            "bit_equal": float(np.mean(np.asarray(gpu_bits) == np.asarray(center_bits))),
            "max_width": int(np.max(khi - klo)) if g.size else 0}
