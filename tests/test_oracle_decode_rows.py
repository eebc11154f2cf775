"""Pins of the oracle's multi-row decode windows (PR #975 decode commits: a
key head's query heads and two decode rows share one 16-row tile; windows of
up to 16 rows a stream, PR #1183 engine note).

Caches are filled the way an engine fills them: every position's key and
value written in position order (slot p, or p mod cap in a ring), the
window's own rows included, before attention.  The expected rows come from
brute force over the keys by absolute position (never through the cache), so
a ring that lost a key the first row still needs, or a wrong slot formula,
shows up as a mismatch.
"""
import numpy as np
import pytest

from oracle import attn_ref, bf16, brute
from synthetic.gen import f32_to_bf16_bits


def _bits(rng, shape, sd=1.0):
    return f32_to_bf16_bits((rng.standard_normal(shape) * sd).astype(np.float32))


def _filled_caches(kp, vp, last, cap, ring):
    """[S][Hkv][cap][D] caches after writing positions 0..last[s] in order."""
    S, n_pos, Hkv, D = kp.shape
    kc = np.full((S, Hkv, cap, D), 0x7FC0, dtype=np.uint16)    # unwritten = NaN
    vc = np.full((S, Hkv, cap, D), 0x7FC0, dtype=np.uint16)
    for s in range(S):
        for p in range(int(last[s]) + 1):
            slot = p % cap if ring else p
            kc[s, :, slot] = kp[s, p]
            vc[s, :, slot] = vp[s, p]
    return kc, vc


@pytest.mark.parametrize("ring,cap,window,R,G,pos", [
    (1, 20, 12, 9, 2, [30, 11, 0]),          # ring exactly window + R - 1
    (1, 24, 7, 16, 1, [50, 3]),
    (0, 40, 0, 5, 4, [0, 17, 35]),           # causal linear, last row at cap - 1
    (0, 40, 9, 8, 8, [25, 2]),               # windowed linear
    (1, 17, 1, 16, 2, [40]),                 # window of one
])
def test_decode_rows_match_brute_by_position(ring, cap, window, R, G, pos):
    rng = np.random.default_rng(cap + R + G)
    S, Hkv, D = len(pos), 2, 8
    Hq = Hkv * G
    pos = np.array(pos)
    n_pos = int(pos.max()) + R
    kp = _bits(rng, (S, n_pos, Hkv, D), sd=1.3)
    vp = _bits(rng, (S, n_pos, Hkv, D))
    q = _bits(rng, (S, R, Hq, D))
    kc, vc = _filled_caches(kp, vp, pos + R - 1, cap, ring)
    scale = 0.4
    ref = attn_ref.decode_rows(q, kc, vc, pos, Hkv, ring, window, scale)
    sc = attn_ref.fp32_scale(scale)
    kf, vf, qf = bf16.f64_from_bits(kp), bf16.f64_from_bits(vp), bf16.f64_from_bits(q)
    for s in range(S):
        for r in range(R):
            t = int(pos[s]) + r
            for h in range(Hq):
                g = h // G
                want = brute.decode_row(qf[s, r, h].tolist(), kf[s, :, g].tolist(),
                                        vf[s, :, g].tolist(), t, 0, window, sc)
                np.testing.assert_allclose(ref["o"][s, r, h], want, rtol=0, atol=1e-12)


def test_one_row_window_is_decode():
    rng = np.random.default_rng(3)
    S, Hkv, G, D, cap = 3, 2, 4, 16, 64
    q = _bits(rng, (S, 1, Hkv * G, D))
    kc = _bits(rng, (S, Hkv, cap, D))
    vc = _bits(rng, (S, Hkv, cap, D))
    pos = [63, 100, 7]
    a = attn_ref.decode_rows(q, kc, vc, pos, Hkv, 1, 40, 0.2)
    b = attn_ref.decode(q[:, 0], kc, vc, pos, Hkv, 1, 40, 0.2)
    assert np.array_equal(a["o"][:, 0], b["o"]) and np.array_equal(a["bits"][:, 0], b["bits"])


def test_short_ring_is_refused_and_would_be_wrong():
    """cap = window + R - 2: the first row's oldest key was overwritten by
    the window's last row, so the oracle refuses the geometry; reading the
    cache anyway (row by row as decode) gives a value brute force rejects."""
    rng = np.random.default_rng(4)
    S, Hkv, D, R, W = 1, 1, 8, 4, 6
    cap = W + R - 2
    pos = np.array([20])
    kp = _bits(rng, (S, 30, Hkv, D), sd=2.0)
    vp = _bits(rng, (S, 30, Hkv, D))
    q = _bits(rng, (S, R, Hkv, D))
    kc, vc = _filled_caches(kp, vp, pos + R - 1, cap, 1)
    with pytest.raises(ValueError):
        attn_ref.decode_rows(q, kc, vc, pos, Hkv, 1, W, 0.5)
    # the row at pos[0] needs position 15, whose slot now holds position 23
    got = attn_ref.decode(q[:, 0], kc, vc, pos, Hkv, 1, W, 0.5)["o"][0, 0]
    want = brute.decode_row(bf16.f64_from_bits(q[0, 0, 0]).tolist(),
                            bf16.f64_from_bits(kp[0, :, 0]).tolist(),
                            bf16.f64_from_bits(vp[0, :, 0]).tolist(), 20, 0, W, 0.5)
    assert not np.allclose(got, want, rtol=0, atol=1e-9)
