"""A float32 NumPy model of a kernel's schedule (test helper, not the oracle).

It computes what an fp32 GPU kernel computes, in the kernel's order, so the
tests can show that the oracle's error radius admits an honest fp32 kernel
(0 fails) while each planted mistake (a dropped or moved rounding point, a
wrong key block) is refused.  It is written from the method's description,
not from the oracle's code.
"""
from __future__ import annotations

import numpy as np

P_FP32, P_BF16, P_BF16X2 = 0, 1, 2


def _bf16_f32(x: np.ndarray) -> np.ndarray:
    """float32 -> nearest-even bf16 value, as float32."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return r.astype(np.uint32).view(np.float32)


def _bf16_bits(x: np.ndarray) -> np.ndarray:
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    r[np.isnan(x)] = 0x7FC0
    return r


def _f32(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32)


def _round_p(p, mode):
    if mode == P_FP32:
        return p
    hi = _bf16_f32(p)
    if mode == P_BF16:
        return hi
    return hi + _bf16_f32(p - hi)


def decode(q_bits, k_bits, v_bits, pos, n_kv_heads, ring, window, scale,
           chunk=256, p_mode=P_FP32):
    """fp32 chunk partials, merged in chunk order; returns bf16 bits."""
    q, kc, vc = _f32(q_bits), _f32(k_bits), _f32(v_bits)
    S, Hq, D = q.shape
    cap = kc.shape[2]
    G = Hq // n_kv_heads
    sc = np.float32(scale)
    out = np.zeros((S, Hq, D), np.float32)
    for s in range(S):
        t = int(pos[s])
        i = np.arange(cap)
        p_of = (t - np.mod(t - i, cap)) if ring else i
        valid = (p_of >= 0) & (p_of <= t)
        if window:
            valid &= (t - p_of) < window
        for g in range(n_kv_heads):
            Qg = q[s, g * G:(g + 1) * G]
            ms, ls, accs = [], [], []
            for c0 in range(0, cap, chunk):
                idx = c0 + np.flatnonzero(valid[c0:c0 + chunk])
                if idx.size == 0:
                    continue
                sg = (Qg @ kc[s, g, idx].T) * sc
                m = sg.max(axis=1, keepdims=True)
                p = np.exp(sg - m).astype(np.float32)
                ms.append(m)
                ls.append(p.sum(axis=1, keepdims=True, dtype=np.float32))
                accs.append(_round_p(p, p_mode) @ vc[s, g, idx])
            if not ms:
                continue
            M = np.max(np.concatenate(ms, axis=1), axis=1, keepdims=True)
            L = np.zeros((G, 1), np.float32)
            A = np.zeros((G, D), np.float32)
            for m, l, a in zip(ms, ls, accs):
                e = np.exp(m - M).astype(np.float32)
                L = L + e * l
                A = A + e * a
            out[s, g * G:(g + 1) * G] = A / L
    return _bf16_bits(out)


def prefill(q_bits, k_bits, v_bits, pos0, n_kv_heads, window, scale, p_mode,
            kb, final_max=False):
    """fp32 online softmax over KB-key blocks by absolute position."""
    q, k, v = _f32(q_bits), _f32(k_bits), _f32(v_bits)
    n, Hq, D = q.shape
    G = Hq // n_kv_heads
    sc = np.float32(scale)
    out = np.zeros((n, Hq, D), np.float32)
    t = pos0 + np.arange(n)
    lo = np.maximum(0, t - window + 1) if window else np.zeros(n, np.int64)
    for h in range(Hq):
        g = h // G
        Sfull = (q[:, h] @ k[: t.max() + 1, g].T) * sc      # [n][keys]
        j = np.arange(t.max() + 1)
        mask = (j[None] >= lo[:, None]) & (j[None] <= t[:, None])
        Sm = np.where(mask, Sfull, -np.inf).astype(np.float32)
        if final_max:
            mfin = Sm.max(axis=1, keepdims=True)
        m = np.full((n, 1), -np.inf, np.float32)
        l = np.zeros((n, 1), np.float32)
        acc = np.zeros((n, D), np.float32)
        for b0 in range(0, t.max() + 1, kb):
            blk = Sm[:, b0:b0 + kb]
            if not np.isfinite(blk).any():
                continue
            m_new = np.maximum(m, blk.max(axis=1, keepdims=True))
            with np.errstate(invalid="ignore"):
                alpha = np.where(np.isfinite(m), np.exp(m - m_new), 0).astype(np.float32)
                ref = m_new
                if final_max:
                    alpha = np.ones_like(alpha)
                    ref = mfin
                p = np.where(np.isfinite(blk), np.exp(blk - ref), 0).astype(np.float32)
            l = l * alpha + p.sum(axis=1, keepdims=True, dtype=np.float32)
            acc = acc * alpha + _round_p(p, p_mode) @ v[b0:b0 + kb, g]
            m = m_new
        out[:, h] = acc / l
    return _bf16_bits(out)
