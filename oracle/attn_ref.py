"""Float64 oracle of grouped-query attention over a KV cache (decode, prefill).

TEST INFRASTRUCTURE ONLY: used by tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py, never by the product path.

Sources (TensorFold pull-request pages):
  * PR #1183 "cuda gemma4: images on the 12B ...", squashed commit bodies,
    window_rows notes: decode splits a head's keys into 256-key chunks with a
    partial (max, sum, accumulator) each, merged in chunk order; prompt tiles
    over 128-dim slices; P kept to 16 bits as two bf16 halves; the checker
    holds float64 at the rounding points plus the spread fp32 allows.  At head dim
    512: no window over a linear cache to 262144 keys, GQA 8 and 16.
  * PR #1183, same commit bodies, the Gemma 4 CUDA engine note: sliding
    layers use a ring (window plus a chunk) and keep each sliding layer's last
    1023 keys besides the row itself; global layers use a linear cache.
  * PR #975 "Gemma 4 12B on the native Metal engine", commit bodies: prompt
    attention under causal and sliding-window masks with an online softmax
    whose row maxima and fp32 probabilities cross once a key block; value
    reads stop at the tile's last written key (an unwritten V row times a zero
    probability gave NaN); the key/value cache is written before attention.

Definitions used here (readings where the pages are silent are marked R#):
  q, k, v are bf16 values; all arithmetic is float64.
  Score  s_j = scale * sum_d q_d k_jd, with scale the float32 value the
         kernel receives (R3: scale multiplies the dot product).
  Window a row at position t sees key positions p with p <= t and, when the
         window W > 0, t - p < W: the row itself plus the W-1 before it (R1).
  Slots  linear cache: slot j holds position j.  ring of R slots: slot i
         holds position t - ((t - i) mod R); negative positions were never
         written.
  Decode p_j = exp(s_j - m), m the row maximum, no rounding of p (R7);
         o = sum_j p_j v_j / sum_j p_j; out = bf16(o).  Empty key set gives 0.
  Prefill keys are taken in blocks B_b = {j : j // KB = b} by absolute
         position, ascending; m_b = max(m_{b-1}, max_{j in B_b} s_j);
         p_j = exp(s_j - m_b(j)); P_j = round(p_j) per P mode (R4, R6);
         l = sum_j p_j w_j and acc = sum_j P_j w_j v_j with
         w_j = exp(m_b(j) - m_last) (the product of the online rescales,
         exact in real arithmetic); the row sum takes unrounded p (R5);
         out = bf16(acc / l).
"""
from __future__ import annotations

import numpy as np

from . import bf16
from .contract import (DECODE_CHUNK, EPS_ACC, EPS_P, MEAN_REL_ERR_MAX,
                       P_BF16, P_BF16X2, P_FP32, ULP_SLACK)


# --------------------------------------------------------------------------
# inputs


def as_f64(bits) -> np.ndarray:
    """bf16 bit patterns -> exact float64 values."""
    return bf16.f64_from_bits(bits)


def fp32_scale(scale: float) -> float:
    """The scale as the float32 the kernel receives, widened exactly."""
    return float(np.float32(scale))


# --------------------------------------------------------------------------
# key sets (which slots a row reads, at which positions)


def slot_positions(t: int, cap: int, ring: int) -> np.ndarray:
    """Position held by each cache slot for a row at position t.

    Linear cache: slot j holds position j.  Ring of cap slots: slot i holds
    the latest position p <= t with p = i (mod cap), i.e. t - ((t - i) mod
    cap); a negative value means the slot was never written.
    """
    i = np.arange(cap, dtype=np.int64)
    if not ring:
        return i
    return t - np.mod(t - i, cap)


def key_valid(positions: np.ndarray, t: int, window: int) -> np.ndarray:
    """Causal + sliding window: 0 <= p <= t and (W == 0 or t - p < W)."""
    ok = (positions >= 0) & (positions <= t)
    if window > 0:
        ok &= (t - positions) < window
    return ok


def prefill_key_range(t: int, window: int, hi: int | None = None) -> tuple[int, int]:
    """First and last key position a prompt row at position t attends.

    hi is the row's last key (PR #975 commit body: the prompt attention takes
    each row's last key, its own position for text rows, so an image's rows
    see each other on sliding layers); None means the row's own position.
    The window's first key stays t - W + 1.
    """
    lo = max(0, t - window + 1) if window > 0 else 0
    return lo, (t if hi is None else hi)


def clamp_last_key(last_key, pos0: int, n_rows: int) -> np.ndarray:
    """Last keys of the rows of one call, clamped to [own position, last row]:
    a row never attends fewer keys than causal, nor a key past the call's
    last row (the cache holds nothing later)."""
    t = pos0 + np.arange(n_rows)
    lk = np.asarray(last_key, dtype=np.int64)
    return np.minimum(np.maximum(lk, t), pos0 + n_rows - 1)


# --------------------------------------------------------------------------
# rounding of P


def round_p(p: np.ndarray, p_mode: int) -> np.ndarray:
    if p_mode == P_FP32:
        return p
    hi = bf16.round_f64(p)
    if p_mode == P_BF16:
        return hi
    if p_mode == P_BF16X2:
        return hi + bf16.round_f64(p - hi)
    raise ValueError(f"unknown p_mode {p_mode}")


# --------------------------------------------------------------------------
# softmax-weighted sum with block-wise running maxima


def attend(S: np.ndarray, mask: np.ndarray, V: np.ndarray, blk: np.ndarray,
           p_mode: int):
    """Rows of scores S [R][K] (float64) over keys with values V [K][D].

    mask [R][K] marks the keys each row attends; blk [K] is each key's block
    index, non-decreasing along K.  Returns (o, r): o [R][D] = acc / l and
    the radius r [R][D] of the range an fp32 kernel may reach.
    """
    R, K = S.shape
    D = V.shape[1]
    o = np.zeros((R, D))
    r = np.zeros((R, D))
    if K == 0 or R == 0:
        return o, r
    # a NaN in an attended score poisons its row; a NaN in an attended value
    # poisons that output column (0 * NaN is NaN).  Masked keys never count.
    nan_score_rows = np.any(mask & np.isnan(S), axis=1)
    vnan = np.isnan(V)
    if vnan.any():
        nan_cols = (mask.astype(np.float64) @ vnan.astype(np.float64)) > 0
        V = np.where(vnan, 0.0, V)
    else:
        nan_cols = np.zeros((R, D), dtype=bool)
    S = np.where(np.isnan(S), 0.0, S)
    Sm = np.where(mask, S, -np.inf)
    starts = np.flatnonzero(np.r_[True, blk[1:] != blk[:-1]])
    bidx = np.cumsum(np.r_[0, (blk[1:] != blk[:-1]).astype(np.int64)])
    block_max = np.maximum.reduceat(Sm, starts, axis=1)        # [R][nb]
    run_max = np.maximum.accumulate(block_max, axis=1)          # m_b
    m_key = run_max[:, bidx]                                    # m_b(j)
    m_last = run_max[:, -1:]
    with np.errstate(invalid="ignore", over="ignore"):
        live = mask & np.isfinite(m_key)
        p = np.where(live, np.exp(np.where(live, Sm - m_key, 0.0)), 0.0)
        w = np.where(live, np.exp(np.where(live, m_key - m_last, 0.0)), 0.0)
    P = round_p(p, p_mode)
    l = np.sum(p * w, axis=1, keepdims=True)
    acc = (P * w) @ V
    # uncertainty of the kernel's rounded P from its fp32 p (relative EPS_P)
    if p_mode == P_FP32:
        dP = EPS_P * p
    else:
        up = round_p(p * (1 + EPS_P), p_mode)
        dn = round_p(p * (1 - EPS_P), p_mode)
        dP = np.maximum(np.abs(up - P), np.abs(P - dn))
    spread = ((dP + EPS_ACC * P) * w) @ np.abs(V)
    has = l[:, 0] > 0
    with np.errstate(invalid="ignore", divide="ignore"):
        o[has] = acc[has] / l[has]
        r[has] = spread[has] / l[has] + (EPS_P + EPS_ACC) * np.abs(o[has])
    o[nan_cols] = np.nan
    o[nan_score_rows] = np.nan
    return o, r


# --------------------------------------------------------------------------
# decode


def decode(q_bits, k_bits, v_bits, pos, n_kv_heads: int, ring: int,
           window: int, scale: float):
    """One decode row per stream against its cache.

    q [S][Hq][D], caches [S][Hkv][cap][D] as bf16 bits, pos [S] the row's
    position.  Returns dict(o, r, bits) with o, r [S][Hq][D].
    """
    q = as_f64(q_bits)
    kc = as_f64(k_bits)
    vc = as_f64(v_bits)
    S, Hq, D = q.shape
    cap = kc.shape[2]
    G = Hq // n_kv_heads
    sc = fp32_scale(scale)
    o = np.zeros((S, Hq, D))
    r = np.zeros((S, Hq, D))
    for s in range(S):
        t = int(pos[s])
        slot_pos = slot_positions(t, cap, ring)
        idx = np.flatnonzero(key_valid(slot_pos, t, window))
        if idx.size == 0:
            continue
        idx = idx[np.argsort(slot_pos[idx], kind="stable")]   # by position
        for g in range(n_kv_heads):
            K = kc[s, g, idx]
            V = vc[s, g, idx]
            Qg = q[s, g * G:(g + 1) * G]
            Sg = sc * (Qg @ K.T)
            blk = np.zeros(idx.size, dtype=np.int64)
            og, rg = attend(Sg, np.ones_like(Sg, dtype=bool), V, blk, P_FP32)
            o[s, g * G:(g + 1) * G] = og
            r[s, g * G:(g + 1) * G] = rg
    return dict(o=o, r=r, bits=bf16.bits_from_f64(o))


def decode_rows(q_bits, k_bits, v_bits, pos, n_kv_heads: int, ring: int,
                window: int, scale: float):
    """A decode window of R rows per stream: row r of stream s sits at
    position pos[s] + r and is an ordinary decode row of that position
    (PR #975 decode commits: a key head's query heads and several decode rows
    share one 16-row tile; every row keeps its bits at any window width, so
    a row's value does not depend on the rows beside it).

    q [S][R][Hq][D]; caches [S][Hkv][cap][D] hold every row's key and value
    (written before attention).  A ring must still hold the window of the
    first row after the later rows' writes: window >= 1 and cap >= window +
    R - 1.  Returns dict(o, r, bits) with o, r [S][R][Hq][D].
    """
    S, R = q_bits.shape[:2]
    cap = k_bits.shape[2]
    if ring and (window < 1 or cap < window + R - 1):
        raise ValueError("a ring needs window >= 1 and cap >= window + rows - 1")
    pos = np.asarray(pos, dtype=np.int64)
    o = np.zeros(q_bits.shape)
    r = np.zeros(q_bits.shape)
    for i in range(R):
        res = decode(q_bits[:, i], k_bits, v_bits, pos + i, n_kv_heads, ring, window, scale)
        o[:, i] = res["o"]
        r[:, i] = res["r"]
    return dict(o=o, r=r, bits=bf16.bits_from_f64(o))


def decode_chunked(q_bits, k_bits, v_bits, pos, n_kv_heads: int, ring: int,
                   window: int, scale: float, chunk: int = DECODE_CHUNK):
    """Decode by chunk partials merged in chunk order (float64 values).

    Chunk c holds slots [c*chunk, (c+1)*chunk).  Each non-empty chunk yields
    (m_c, l_c, acc_c) with m_c its own maximum; the merge takes the maximum
    M of the m_c and sums e^(m_c - M) acc_c and e^(m_c - M) l_c over c in
    ascending order.  Equal to decode() up to float64 rounding.
    """
    q = as_f64(q_bits)
    kc = as_f64(k_bits)
    vc = as_f64(v_bits)
    S, Hq, D = q.shape
    cap = kc.shape[2]
    G = Hq // n_kv_heads
    sc = fp32_scale(scale)
    o = np.zeros((S, Hq, D))
    for s in range(S):
        t = int(pos[s])
        valid = key_valid(slot_positions(t, cap, ring), t, window)
        for g in range(n_kv_heads):
            Qg = q[s, g * G:(g + 1) * G]
            parts = []
            for c0 in range(0, cap, chunk):
                idx = c0 + np.flatnonzero(valid[c0:c0 + chunk])
                if idx.size == 0:
                    continue
                Sg = sc * (Qg @ kc[s, g, idx].T)
                m = Sg.max(axis=1, keepdims=True)
                p = np.exp(Sg - m)
                parts.append((m, p.sum(axis=1, keepdims=True), p @ vc[s, g, idx]))
            if not parts:
                continue
            M = np.max(np.concatenate([m for m, _, _ in parts], axis=1), axis=1,
                       keepdims=True)
            L = np.zeros((G, 1))
            A = np.zeros((G, D))
            for m, l, a in parts:
                e = np.exp(m - M)
                L = L + e * l
                A = A + e * a
            o[s, g * G:(g + 1) * G] = A / L
    return o


# --------------------------------------------------------------------------
# prefill


def prefill(q_bits, k_bits, v_bits, pos0: int, n_kv_heads: int, window: int,
            scale: float, p_mode: int, kb: int, rows=None, heads=None,
            row_batch: int = 256, last_key=None):
    """Prompt rows at positions pos0 + i against keys by absolute position.

    q [n][Hq][D]; k, v [n_pos][Hkv][D] with row p the key/value at position
    p (n_pos > pos0 + n - 1).  rows / heads select the outputs to compute
    (default all).  last_key [n] (optional): each row's last key position,
    used as given (callers clamp with clamp_last_key).  Returns dict(o, r,
    bits) of shape [len(rows)][len(heads)][D].
    """
    q = q_bits if q_bits.dtype == np.float64 else as_f64(q_bits)
    k = k_bits if k_bits.dtype == np.float64 else as_f64(k_bits)
    v = v_bits if v_bits.dtype == np.float64 else as_f64(v_bits)
    n, Hq, D = q.shape
    G = Hq // n_kv_heads
    sc = fp32_scale(scale)
    rows = np.arange(n) if rows is None else np.asarray(rows, dtype=np.int64)
    heads = np.arange(Hq) if heads is None else np.asarray(heads, dtype=np.int64)
    order = np.argsort(rows, kind="stable")
    o = np.zeros((rows.size, heads.size, D))
    r = np.zeros((rows.size, heads.size, D))
    for b0 in range(0, rows.size, row_batch):
        sel = order[b0:b0 + row_batch]
        rr = rows[sel]
        t = pos0 + rr
        lo = np.array([prefill_key_range(int(x), window)[0] for x in t])
        hi = t if last_key is None else np.asarray(last_key, dtype=np.int64)[rr]
        j0, j1 = int(lo.min()), int(hi.max())
        j = np.arange(j0, j1 + 1)
        mask = (j[None, :] >= lo[:, None]) & (j[None, :] <= hi[:, None])
        blk = j // kb
        for hi, h in enumerate(heads):
            g = int(h) // G
            Sg = sc * (q[rr, h] @ k[j0:j1 + 1, g].T)
            oh, rh = attend(Sg, mask, v[j0:j1 + 1, g], blk, p_mode)
            o[sel, hi] = oh
            r[sel, hi] = rh
    return dict(o=o, r=r, bits=bf16.bits_from_f64(o))


# --------------------------------------------------------------------------
# pass criterion


def check(gpu_bits, o, r, slack: int = ULP_SLACK) -> dict:
    """Compare kernel bf16 outputs with the oracle's value and radius.

    An element passes iff its ordered key lies within `slack` steps of
    [bf16(o - r), bf16(o + r)]; NaN matches only NaN.  Also returns the mean
    relative error against bf16(o) and the fraction of bit-equal outputs.
    """
    g = np.asarray(gpu_bits, dtype=np.uint16)
    o = np.asarray(o, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    want = bf16.bits_from_f64(o)
    lo = bf16.ordered(bf16.bits_from_f64(o - r))
    hi = bf16.ordered(bf16.bits_from_f64(o + r))
    kg = bf16.ordered(g)
    gnan = bf16.is_nan_bits(g)
    onan = np.isnan(o)
    ok = (kg >= lo - slack) & (kg <= hi + slack) & ~gnan & ~onan
    ok |= gnan & onan
    fin = ~onan & ~gnan
    gv = bf16.f64_from_bits(g[fin])
    wv = bf16.f64_from_bits(want[fin])
    den = np.sum(np.abs(wv))
    mre = float(np.sum(np.abs(gv - wv)) / den) if den > 0 else 0.0
    bad = np.flatnonzero(~ok.ravel())
    steps = np.where(kg < lo, lo - kg, np.where(kg > hi, kg - hi, 0))
    return dict(n=int(g.size), fails=int(bad.size), first_bad=bad[:8].tolist(),
                max_steps_out=int(steps.max()) if steps.size else 0,
                mean_rel_err=mre,
                bit_equal=float(np.mean(g == want)) if g.size else 1.0,
                ok=bool(bad.size == 0 and mre <= MEAN_REL_ERR_MAX))
