"""Pins of the attention oracle (CPU only).

The oracle (oracle/attn_ref.py) is checked against things other than itself:
  * brute force: oracle/brute.py, loops written apart (positions walked down
    to slots, the online-softmax recurrence), on tiny shapes, every mask,
    cache kind and P mode;
  * library routines: scipy's softmax for decode and torch's float64
    scaled_dot_product_attention with an explicit mask for unrounded prefill;
  * closed forms: a single key returns V exactly; identical keys return the
    bf16 of V's mean; a key whose score dominates returns its V exactly, at
    the window edge and never from one step outside it;
  * identities: the 256-slot chunk merge equals the one-pass softmax; a
    window over a ring equals the same window over a linear cache;
  * the two-halves P is within 2^-16 of unrounded P, term by term;
  * unwritten or masked slots poisoned with NaN change nothing.
"""
import math

import numpy as np
import pytest
import scipy.special
import torch

from oracle import attn_ref, bf16, brute
from oracle.contract import P_BF16, P_BF16X2, P_FP32, key_block
from synthetic.gen import f32_to_bf16_bits


def _bits(rng, shape, sd=1.0):
    return f32_to_bf16_bits((rng.standard_normal(shape) * sd).astype(np.float32))


def _f(b):
    return bf16.f64_from_bits(b)


# ---------------------------------------------------------------- brute force

@pytest.mark.parametrize("ring,window,cap,t", [
    (0, 0, 40, 39), (0, 0, 40, 17), (0, 8, 40, 30), (0, 40, 40, 39),
    (1, 16, 16, 50), (1, 12, 16, 50), (1, 0, 16, 9), (1, 16, 16, 7),
    (1, 5, 24, 100),
])
def test_decode_matches_brute(ring, window, cap, t):
    rng = np.random.default_rng(100 + cap + t)
    S, Hkv, G, D = 1, 2, 3, 8
    q = _bits(rng, (S, Hkv * G, D))
    k = _bits(rng, (S, Hkv, cap, D))
    v = _bits(rng, (S, Hkv, cap, D))
    scale = 0.35
    ref = attn_ref.decode(q, k, v, [t], Hkv, ring, window, scale)
    sc = attn_ref.fp32_scale(scale)
    for h in range(Hkv * G):
        g = h // G
        want = brute.decode_row(_f(q[0, h]).tolist(), _f(k[0, g]).tolist(),
                                _f(v[0, g]).tolist(), t, ring, window, sc)
        np.testing.assert_allclose(ref["o"][0, h], want, rtol=0, atol=1e-13)


@pytest.mark.parametrize("p_mode", [P_FP32, P_BF16, P_BF16X2])
@pytest.mark.parametrize("window,kb,pos0,n", [
    (0, 8, 0, 37), (0, 4, 13, 20), (6, 8, 0, 30), (11, 4, 5, 28), (1, 8, 0, 9),
    (0, 64, 0, 40),
])
def test_prefill_matches_brute(p_mode, window, kb, pos0, n):
    rng = np.random.default_rng(7 * kb + n + window)
    Hkv, G, D = 2, 2, 8
    n_pos = pos0 + n
    q = _bits(rng, (n, Hkv * G, D))
    k = _bits(rng, (n_pos, Hkv, D), sd=1.5)
    v = _bits(rng, (n_pos, Hkv, D))
    scale = 0.5
    ref = attn_ref.prefill(q, k, v, pos0, Hkv, window, scale, p_mode, kb)
    sc = attn_ref.fp32_scale(scale)
    for i in range(n):
        for h in range(Hkv * G):
            g = h // G
            want = brute.prefill_row(_f(q[i, h]).tolist(), _f(k[:, g]).tolist(),
                                     _f(v[:, g]).tolist(), pos0 + i, window, sc,
                                     p_mode, kb)
            np.testing.assert_allclose(ref["o"][i, h], want, rtol=0, atol=1e-12)


# ---------------------------------------------------------- library routines

def test_decode_matches_scipy_softmax():
    rng = np.random.default_rng(5)
    S, Hkv, G, D, cap = 2, 2, 4, 32, 300
    q = _bits(rng, (S, Hkv * G, D))
    k = _bits(rng, (S, Hkv, cap, D))
    v = _bits(rng, (S, Hkv, cap, D))
    pos = [299, 120]
    ref = attn_ref.decode(q, k, v, pos, Hkv, 0, 0, 0.125)
    for s in range(S):
        t = pos[s]
        for h in range(Hkv * G):
            g = h // G
            sc = 0.125 * (_f(k[s, g, :t + 1]) @ _f(q[s, h]))
            want = scipy.special.softmax(sc) @ _f(v[s, g, :t + 1])
            np.testing.assert_allclose(ref["o"][s, h], want, rtol=0, atol=1e-13)


@pytest.mark.parametrize("window", [0, 9])
def test_unrounded_prefill_matches_torch_sdpa(window):
    rng = np.random.default_rng(9 + window)
    n, Hkv, G, D, pos0 = 33, 2, 2, 16, 4
    q = _bits(rng, (n, Hkv * G, D))
    k = _bits(rng, (pos0 + n, Hkv, D))
    v = _bits(rng, (pos0 + n, Hkv, D))
    scale = 0.25
    ref = attn_ref.prefill(q, k, v, pos0, Hkv, window, scale, P_FP32, kb=8)
    t = pos0 + np.arange(n)
    j = np.arange(pos0 + n)
    mask = (j[None] <= t[:, None])
    if window:
        mask &= (t[:, None] - j[None]) < window
    for h in range(Hkv * G):
        g = h // G
        out = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(_f(q[:, h]))[None], torch.from_numpy(_f(k[:, g]))[None],
            torch.from_numpy(_f(v[:, g]))[None], attn_mask=torch.from_numpy(mask)[None],
            scale=scale)[0].numpy()
        np.testing.assert_allclose(ref["o"][:, h], out, rtol=0, atol=1e-13)


# -------------------------------------------------------------- closed forms

@pytest.mark.parametrize("p_mode", [P_BF16, P_BF16X2])
def test_single_key_returns_v(p_mode):
    rng = np.random.default_rng(1)
    D = 256
    q = _bits(rng, (1, 8, D))
    k = _bits(rng, (1, 1, 64, D))
    v = _bits(rng, (1, 1, 64, D))
    dec = attn_ref.decode(q, k, v, [0], 1, 0, 0, 1 / 16)
    assert np.array_equal(dec["bits"][0], np.broadcast_to(v[0, 0, 0], (8, D)))
    pre = attn_ref.prefill(q, k[0].transpose(1, 0, 2), v[0].transpose(1, 0, 2),
                           0, 1, 1024, 1 / 16, p_mode, key_block(256, p_mode))
    assert np.array_equal(pre["bits"][0], np.broadcast_to(v[0, 0, 0], (8, D)))


@pytest.mark.parametrize("p_mode", [P_FP32, P_BF16, P_BF16X2])
def test_identical_keys_return_mean_v(p_mode):
    rng = np.random.default_rng(2)
    D, n = 64, 128                       # n a power of two: the mean is exact
    q = _bits(rng, (n, 4, D))
    k = np.broadcast_to(_bits(rng, (1, 1, D)), (n, 1, D)).copy()
    v = _bits(rng, (n, 1, D))
    pre = attn_ref.prefill(q, k, v, 0, 1, 0, 0.1, p_mode, kb=16, rows=[n - 1])
    want = bf16.bits_from_f64(_f(v[:, 0]).mean(axis=0))
    assert np.array_equal(pre["bits"][0], np.broadcast_to(want, (4, D)))
    dec = attn_ref.decode(q[:1], k.transpose(1, 0, 2)[None], v.transpose(1, 0, 2)[None],
                          [n - 1], 1, 0, 0, 0.1)
    assert np.array_equal(dec["bits"][0], np.broadcast_to(want, (4, D)))


def _dominating(D, rng, where, t, cap, ring, window):
    """Decode inputs where slot `where` has k = 8 q (a dominating score)."""
    q = _bits(rng, (1, 1, D), sd=0.5)
    k = _bits(rng, (1, 1, cap, D), sd=0.05)
    v = _bits(rng, (1, 1, cap, D))
    k[0, 0, where] = f32_to_bf16_bits(8 * _f(q[0, 0]).astype(np.float32))
    return q, k, v


@pytest.mark.parametrize("ring", [0, 1])
def test_dominating_key_at_window_edge_and_outside(ring):
    rng = np.random.default_rng(3)
    D, W = 64, 16
    cap = 64 if not ring else 32
    t = 50 if not ring else 77                  # ring wraps
    slot = (lambda p: p % cap) if ring else (lambda p: p)
    edge = t - W + 1
    q, k, v = _dominating(D, rng, slot(edge), t, cap, ring, W)
    out = attn_ref.decode(q, k, v, [t], 1, ring, W, 1.0)
    assert np.array_equal(out["bits"][0, 0], v[0, 0, slot(edge)])
    outside = t - W
    q, k, v = _dominating(D, rng, slot(outside), t, cap, ring, W)
    out = attn_ref.decode(q, k, v, [t], 1, ring, W, 1.0)
    assert not np.array_equal(out["bits"][0, 0], v[0, 0, slot(outside)])
    assert np.all(np.abs(out["o"][0, 0]) < 1.0)


def test_dominating_key_prefill_window_edge():
    rng = np.random.default_rng(4)
    D, W, n = 32, 10, 40
    q = _bits(rng, (n, 1, D), sd=0.5)
    k = _bits(rng, (n, 1, D), sd=0.05)
    v = _bits(rng, (n, 1, D))
    i = 30
    k[i - W + 1, 0] = f32_to_bf16_bits(8 * _f(q[i, 0]).astype(np.float32))
    out = attn_ref.prefill(q, k, v, 0, 1, W, 1.0, P_BF16, 8, rows=[i])
    assert np.array_equal(out["bits"][0, 0], v[i - W + 1, 0])
    k2 = _bits(rng, (n, 1, D), sd=0.05)
    k2[i - W, 0] = f32_to_bf16_bits(8 * _f(q[i, 0]).astype(np.float32))
    out = attn_ref.prefill(q, k2, v, 0, 1, W, 1.0, P_BF16, 8, rows=[i])
    assert not np.array_equal(out["bits"][0, 0], v[i - W, 0])


def test_two_key_closed_form():
    # q = (1, 0, ...), keys e1 * a and e1 * b: scores a*s, b*s; the output is
    # (e^{a s} v1 + e^{b s} v2) / (e^{a s} + e^{b s}) with P unrounded.
    D = 8
    q = np.zeros((1, 1, D), np.float32); q[0, 0, 0] = 1
    k = np.zeros((1, 1, 4, D), np.float32); k[0, 0, 0, 0] = 2; k[0, 0, 1, 0] = -1
    v = np.zeros((1, 1, 4, D), np.float32); v[0, 0, 0, :] = 1; v[0, 0, 1, :] = -3
    out = attn_ref.decode(f32_to_bf16_bits(q), f32_to_bf16_bits(k),
                          f32_to_bf16_bits(v), [1], 1, 0, 0, 0.5)
    w1, w2 = math.exp(1.0), math.exp(-0.5)
    want = (w1 * 1 + w2 * -3) / (w1 + w2)
    np.testing.assert_allclose(out["o"][0, 0], want, rtol=1e-15)


# ---------------------------------------------------------------- identities

@pytest.mark.parametrize("ring,window,cap,pos", [
    (0, 0, 1000, [999, 600, 255, 256]), (1, 700, 1024, [5000, 700, 100, 1023]),
    (0, 300, 900, [899, 10, 300, 512])])
def test_chunked_merge_equals_one_pass(ring, window, cap, pos):
    rng = np.random.default_rng(11)
    S, Hkv, G, D = 4, 1, 4, 32
    q = _bits(rng, (S, Hkv * G, D))
    k = _bits(rng, (S, Hkv, cap, D), sd=2.0)
    v = _bits(rng, (S, Hkv, cap, D))
    one = attn_ref.decode(q, k, v, pos, Hkv, ring, window, 0.3)["o"]
    chunked = attn_ref.decode_chunked(q, k, v, pos, Hkv, ring, window, 0.3)
    np.testing.assert_allclose(chunked, one, rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("W,R,t", [(16, 16, 70), (10, 16, 70), (16, 16, 15), (7, 12, 5)])
def test_window_over_ring_equals_masked_linear(W, R, t):
    rng = np.random.default_rng(12)
    D = 16
    n_pos = t + 1
    q = _bits(rng, (1, 4, D))
    kpos = _bits(rng, (n_pos, D))
    vpos = _bits(rng, (n_pos, D))
    lin_k = kpos[None, None]
    lin_v = vpos[None, None]
    ring_k = np.full((1, 1, R, D), 0x7FC0, np.uint16)   # unwritten: NaN
    ring_v = np.full((1, 1, R, D), 0x7FC0, np.uint16)
    for p in range(n_pos):
        ring_k[0, 0, p % R] = kpos[p]
        ring_v[0, 0, p % R] = vpos[p]
    a = attn_ref.decode(q, lin_k, lin_v, [t], 1, 0, W, 0.4)
    b = attn_ref.decode(q, ring_k, ring_v, [t], 1, 1, W, 0.4)
    assert np.array_equal(a["bits"], b["bits"])
    assert np.array_equal(a["o"], b["o"])


def test_two_halves_p_within_2_pow_16():
    rng = np.random.default_rng(13)
    p = np.exp(-np.abs(rng.standard_normal(100000)) * 20)
    p = p[p >= 2.0 ** -100]          # hi and lo both normal numbers
    two = attn_ref.round_p(p, P_BF16X2)
    assert np.all(np.abs(two - p) <= 2.0 ** -16 * p)
    one = attn_ref.round_p(p, P_BF16)
    assert np.all(np.abs(one - p) <= 2.0 ** -8 * p)
    assert np.mean(np.abs(one - p) > 2.0 ** -16 * p) > 0.9


def test_nan_in_unattended_slots_changes_nothing():
    rng = np.random.default_rng(14)
    D, cap, t, W = 32, 64, 40, 20
    q = _bits(rng, (1, 2, D))
    k = _bits(rng, (1, 1, cap, D))
    v = _bits(rng, (1, 1, cap, D))
    a = attn_ref.decode(q, k, v, [t], 1, 0, W, 0.3)
    k2, v2 = k.copy(), v.copy()
    dead = [p for p in range(cap) if p > t or t - p >= W]
    k2[0, 0, dead] = 0x7FC0
    v2[0, 0, dead] = 0x7FC0
    b = attn_ref.decode(q, k2, v2, [t], 1, 0, W, 0.3)
    assert np.array_equal(a["bits"], b["bits"])
    # a NaN in an attended value does propagate
    v2[0, 0, t, 3] = 0x7FC0
    c = attn_ref.decode(q, k2, v2, [t], 1, 0, W, 0.3)
    assert np.isnan(c["o"][0, :, 3]).all() and np.isfinite(c["o"][0, :, 4]).all()


def test_empty_key_set_gives_zero():
    rng = np.random.default_rng(15)
    q = _bits(rng, (2, 4, 16))
    k = _bits(rng, (2, 1, 32, 16))
    v = _bits(rng, (2, 1, 32, 16))
    out = attn_ref.decode(q, k, v, [-1, 5], 1, 1, 8, 0.3)
    assert np.all(out["bits"][0] == 0)
    assert np.all(out["o"][1] != 0)
