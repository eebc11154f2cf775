"""Pins of the oracle's per-row last key (prompt rows of an image see each
other on sliding layers: PR #975 commit body, each row's last key, its own
position for text rows; PR #1183 body, window_attention's last-key rows).

The oracle's masked prefill with last keys is checked against
  * brute force (oracle/brute.py's online recurrence, walked up to the row's
    last key) on tiny shapes, every P mode, with and without a window;
  * torch's float64 scaled_dot_product_attention with the explicit
    bidirectional-span mask (unrounded P);
  * the causal prefill, bit for bit, when every last key is the row's own
    position;
  * a closed form: a dominating key later in the row's image span is
    returned exactly by an earlier row of the span, and never by a text row
    before the image;
  * the clamp of out-of-range last keys to [own position, last row].
"""
import numpy as np
import pytest
import torch

from oracle import attn_ref, bf16, brute
from oracle.contract import P_BF16, P_BF16X2, P_FP32
from synthetic.gen import f32_to_bf16_bits


def _bits(rng, shape, sd=1.0):
    return f32_to_bf16_bits((rng.standard_normal(shape) * sd).astype(np.float32))


def _f(b):
    return bf16.f64_from_bits(b)


def _spans_last_key(pos0, n, spans):
    """last key per row: own position, or the span's last position for rows
    inside an image span [a, b] (absolute positions)."""
    t = pos0 + np.arange(n)
    lk = t.copy()
    for a, b in spans:
        inside = (t >= a) & (t <= b)
        lk[inside] = b
    return lk


@pytest.mark.parametrize("p_mode", [P_FP32, P_BF16, P_BF16X2])
@pytest.mark.parametrize("window,kb,pos0,n,spans", [
    (0, 8, 0, 30, [(5, 12), (20, 23)]),
    (6, 4, 3, 25, [(8, 14)]),
    (9, 8, 0, 33, [(0, 7), (16, 31)]),
    (1, 4, 0, 12, [(2, 9)]),
])
def test_last_key_prefill_matches_brute(p_mode, window, kb, pos0, n, spans):
    rng = np.random.default_rng(31 + n + window + kb)
    Hkv, G, D = 2, 2, 8
    q = _bits(rng, (n, Hkv * G, D))
    k = _bits(rng, (pos0 + n, Hkv, D), sd=1.5)
    v = _bits(rng, (pos0 + n, Hkv, D))
    lk = _spans_last_key(pos0, n, spans)
    scale = 0.5
    ref = attn_ref.prefill(q, k, v, pos0, Hkv, window, scale, p_mode, kb, last_key=lk)
    sc = attn_ref.fp32_scale(scale)
    for i in range(n):
        for h in range(Hkv * G):
            g = h // G
            want = brute.prefill_row(_f(q[i, h]).tolist(), _f(k[:, g]).tolist(),
                                     _f(v[:, g]).tolist(), pos0 + i, window, sc,
                                     p_mode, kb, hi=int(lk[i]))
            np.testing.assert_allclose(ref["o"][i, h], want, rtol=0, atol=1e-12)


@pytest.mark.parametrize("window", [0, 10])
def test_last_key_unrounded_matches_torch_sdpa(window):
    rng = np.random.default_rng(77 + window)
    n, Hkv, G, D, pos0 = 40, 2, 2, 16, 4
    q = _bits(rng, (n, Hkv * G, D))
    k = _bits(rng, (pos0 + n, Hkv, D))
    v = _bits(rng, (pos0 + n, Hkv, D))
    lk = _spans_last_key(pos0, n, [(9, 20), (30, 43)])
    ref = attn_ref.prefill(q, k, v, pos0, Hkv, window, 0.25, P_FP32, kb=8, last_key=lk)
    t = pos0 + np.arange(n)
    j = np.arange(pos0 + n)
    mask = j[None] <= lk[:, None]
    if window:
        mask &= (t[:, None] - j[None]) < window
    for h in range(Hkv * G):
        g = h // G
        out = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(_f(q[:, h]))[None], torch.from_numpy(_f(k[:, g]))[None],
            torch.from_numpy(_f(v[:, g]))[None], attn_mask=torch.from_numpy(mask)[None],
            scale=0.25)[0].numpy()
        np.testing.assert_allclose(ref["o"][:, h], out, rtol=0, atol=1e-13)


@pytest.mark.parametrize("p_mode", [P_BF16, P_BF16X2])
def test_own_position_last_key_is_causal_bit_for_bit(p_mode):
    rng = np.random.default_rng(5)
    n, Hkv, G, D, pos0 = 29, 1, 3, 16, 7
    q = _bits(rng, (n, Hkv * G, D))
    k = _bits(rng, (pos0 + n, Hkv, D))
    v = _bits(rng, (pos0 + n, Hkv, D))
    a = attn_ref.prefill(q, k, v, pos0, Hkv, 12, 0.3, p_mode, 8)
    b = attn_ref.prefill(q, k, v, pos0, Hkv, 12, 0.3, p_mode, 8,
                         last_key=pos0 + np.arange(n))
    assert np.array_equal(a["bits"], b["bits"])
    assert np.array_equal(a["o"], b["o"]) and np.array_equal(a["r"], b["r"])


@pytest.mark.parametrize("p_mode", [P_BF16, P_BF16X2])
def test_image_row_sees_a_later_image_key(p_mode):
    """k = 8 q at the span's last position: an earlier row of the span
    returns that key's V exactly; a text row before the image does not."""
    rng = np.random.default_rng(8)
    n, D, span = 24, 16, (10, 17)
    q = _bits(rng, (n, 1, D))
    q[:] = q[:1]                                     # one query for every row
    k = f32_to_bf16_bits((rng.standard_normal((n, 1, D)) * 0.02).astype(np.float32))
    v = _bits(rng, (n, 1, D))
    qf = _f(q[0, 0])
    k[span[1], 0] = f32_to_bf16_bits((8 * qf).astype(np.float32))
    lk = _spans_last_key(0, n, [span])
    ref = attn_ref.prefill(q, k, v, 0, 1, 0, 1.0, p_mode, 4, last_key=lk)
    for i in range(span[0], span[1] + 1):
        assert np.array_equal(ref["bits"][i, 0], v[span[1], 0]), i
    for i in range(0, span[0]):
        assert not np.array_equal(ref["bits"][i, 0], v[span[1], 0]), i


def test_clamp_last_key():
    pos0, n = 100, 8
    lk = np.array([90, 101, 103, 500, 104, 104, -5, 107])
    c = attn_ref.clamp_last_key(lk, pos0, n)
    assert c.tolist() == [100, 101, 103, 107, 104, 105, 106, 107]


def test_prefill_key_range_with_last_key():
    assert attn_ref.prefill_key_range(50, 10) == (41, 50)
    assert attn_ref.prefill_key_range(50, 10, hi=60) == (41, 60)
    assert attn_ref.prefill_key_range(5, 0, hi=9) == (0, 9)
