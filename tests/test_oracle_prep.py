"""Pins of the decode prologue oracle (oracle/prep_ref.py): RMS norms with
MLX's rounding points, the rotary embedding, the unit RMS norm of v (PR
#1183 squashed commit bodies, the qk_rows note), against values fixed by
the mathematics rather than by the oracle's own formulas:

  * exact cases: a constant row whose mean square is a power of four, at
    position 0, gives exact values and ranges one bf16 wide;
  * the norm against torch's float64 rms_norm;
  * the rotation against complex multiplication, its norm preservation and
    its inverse;
  * the ranges hold the center, are at most a few bf16 steps wide, and
    refuse planted mistakes (interleaved pairs, a flipped sine, a dropped
    intermediate rounding, a wrong position).
"""
import numpy as np
import pytest
import torch

from oracle import bf16, prep_ref
from synthetic.gen import f32_to_bf16_bits


def _bits(rng, shape, sd=1.0):
    return f32_to_bf16_bits((rng.standard_normal(shape) * sd).astype(np.float32))


def _freqs(D, theta=10000.0):
    return (1.0 / theta ** (np.arange(0, D, 2) / D)).astype(np.float32)


def test_constant_row_is_exact():
    D, Hq, Hkv = 16, 2, 1
    x = np.full((1, (Hq + 2 * Hkv) * D), f32_to_bf16_bits(np.float32(2.0)), dtype=np.uint16)
    w = np.full(D, f32_to_bf16_bits(np.float32(1.5)), dtype=np.uint16)
    r = prep_ref.qkv_prep(x, w, w, _freqs(D), 0.0, 1, [0], Hq, Hkv, D)
    one5 = f32_to_bf16_bits(np.float32(1.5))
    one = f32_to_bf16_bits(np.float32(1.0))
    assert np.all(r["q_bits"] == one5) and np.all(r["k_bits"] == one5)
    assert np.all(r["v_bits"] == one)
    for n in ("q", "k", "v"):
        assert np.array_equal(r[n + "_lo"], r[n + "_hi"])
        assert np.array_equal(r[n + "_lo"], bf16.ordered(r[n + "_bits"]))


def test_norm_matches_torch_rms_norm():
    rng = np.random.default_rng(1)
    xb = _bits(rng, (6, 512), sd=3.0)
    x = bf16.f64_from_bits(xb)
    eps = 1e-6
    got = x * prep_ref.rms_inv(x, eps)
    want = torch.nn.functional.rms_norm(torch.from_numpy(x), (512,),
                                        eps=float(np.float32(eps))).numpy()
    np.testing.assert_allclose(got, want, rtol=1e-14, atol=0)


@pytest.mark.parametrize("t", [0, 1, 37, 4095, 262143])
def test_rope_is_complex_rotation(t):
    rng = np.random.default_rng(t + 2)
    D = 256
    y = bf16.f64_from_bits(_bits(rng, (3, D)))
    f = _freqs(D, 1e6)
    bits, klo, khi = prep_ref.rope(y, y, y, t, f)
    a = prep_ref.angles(t, f)
    z = (y[:, :D // 2] + 1j * y[:, D // 2:]) * np.exp(1j * a)
    want = np.concatenate([z.real, z.imag], axis=-1)
    assert np.array_equal(bits, bf16.bits_from_f64(want))
    # before rounding: the pair norms are kept, and rotating back restores y
    out = np.concatenate([y[:, :D // 2] * np.cos(a) - y[:, D // 2:] * np.sin(a),
                          y[:, D // 2:] * np.cos(a) + y[:, :D // 2] * np.sin(a)], axis=-1)
    np.testing.assert_allclose(np.hypot(out[:, :D // 2], out[:, D // 2:]),
                               np.hypot(y[:, :D // 2], y[:, D // 2:]), rtol=1e-14)
    back = (out[:, :D // 2] + 1j * out[:, D // 2:]) * np.exp(-1j * a)
    np.testing.assert_allclose(np.concatenate([back.real, back.imag], axis=-1), y,
                               rtol=0, atol=1e-12)


def test_angle_is_the_fp32_product():
    f = np.array([0.3, 1e-4, 0.0], dtype=np.float32)
    t = 16777217                        # not an fp32 integer: rounds to 2^24
    a = prep_ref.angles(t, f)
    assert a[0] == float(np.float32(np.float32(2.0 ** 24) * np.float32(0.3)))
    assert a[2] == 0.0


def _case(seed, D=256, Hq=4, Hkv=2, S=3):
    rng = np.random.default_rng(seed)
    qkv = _bits(rng, (S, (Hq + 2 * Hkv) * D), sd=2.0)
    qw = _bits(rng, D, sd=0.5)
    kw = _bits(rng, D, sd=0.5)
    pos = rng.integers(0, 70000, S)
    return qkv, qw, kw, pos, Hq, Hkv, D


@pytest.mark.parametrize("seed", [3, 4])
def test_ranges_hold_center_and_are_tight(seed):
    """Ranges hold the center; almost all are one bf16 wide, and a range
    wider than three steps only where the rotation cancels (the output far
    below the products it is the difference of) or where a normed input of
    the pair sits at a bf16 tie (two candidates, one normed step apart)."""
    qkv, qw, kw, pos, Hq, Hkv, D = _case(seed)
    r = prep_ref.qkv_prep(qkv, qw, kw, _freqs(D), 1e-6, 1, pos, Hq, Hkv, D)
    S, h = qkv.shape[0], D // 2
    rows = qkv.reshape(S, Hq + 2 * Hkv, D)
    for n, sl, w in (("q", slice(0, Hq), qw), ("k", slice(Hq, Hq + Hkv), kw), ("v", None, None)):
        c = bf16.ordered(r[n + "_bits"])
        assert np.all(r[n + "_lo"] <= c) and np.all(c <= r[n + "_hi"])
        width = r[n + "_hi"] - r[n + "_lo"]
        assert np.mean(width == 0) > 0.9, n
        if n == "v":
            assert width.max() <= 1
            continue
        y, ylo, yhi = prep_ref.normed(rows[:, sl], w, 1e-6)
        terms = np.concatenate([np.abs(y[..., :h]) + np.abs(y[..., h:])] * 2, axis=-1)
        tie = (ylo != yhi)
        tie_pair = np.concatenate([tie[..., :h] | tie[..., h:]] * 2, axis=-1)
        out = np.abs(bf16.f64_from_bits(r[n + "_bits"]))
        wide = width > 3
        assert np.all((out[wide] < terms[wide] * 2.0 ** -6) | tie_pair[wide]), n


def _prep_variant(qkv, qw, kw, pos, Hq, Hkv, D, f, eps, mode):
    """The prologue with one planted mistake, center values only."""
    S = qkv.shape[0]
    rows = qkv.reshape(S, Hq + 2 * Hkv, D)
    x = bf16.f64_from_bits(rows[:, :Hq])
    inv = prep_ref.rms_inv(x, eps)
    w = bf16.f64_from_bits(qw)
    y = bf16.round_f64(w * (x * inv if mode == "one_round" else bf16.round_f64(x * inv)))
    out = np.empty_like(y)
    h = D // 2
    for s in range(S):
        t = int(pos[s]) + (1 if mode == "pos_plus_one" else 0)
        a = prep_ref.angles(t, f)
        c, sn = np.cos(a), np.sin(a)
        if mode == "flip_sin":
            sn = -sn
        ys = y[s]
        if mode == "interleaved":
            e, o = ys[..., 0::2], ys[..., 1::2]
            r = np.empty_like(ys)
            r[..., 0::2] = e * c - o * sn
            r[..., 1::2] = o * c + e * sn
        else:
            r = np.concatenate([ys[..., :h] * c - ys[..., h:] * sn,
                                ys[..., h:] * c + ys[..., :h] * sn], axis=-1)
        out[s] = r
    return bf16.bits_from_f64(out)


@pytest.mark.parametrize("mode", ["interleaved", "flip_sin", "one_round", "pos_plus_one"])
def test_ranges_refuse_planted_mistakes(mode):
    qkv, qw, kw, pos, Hq, Hkv, D = _case(5)
    f = _freqs(D)
    r = prep_ref.qkv_prep(qkv, qw, kw, f, 1e-6, 1, pos, Hq, Hkv, D)
    bad = _prep_variant(qkv, qw, kw, pos, Hq, Hkv, D, f, 1e-6, mode)
    res = prep_ref.check_range(bad, r["q_bits"], r["q_lo"], r["q_hi"])
    assert not res["ok"], (mode, res)
    good = prep_ref.check_range(r["q_bits"], r["q_bits"], r["q_lo"], r["q_hi"])
    assert good["ok"] and good["bit_equal"] == 1.0


def test_v_without_norm_is_copied():
    qkv, qw, kw, pos, Hq, Hkv, D = _case(6)
    r = prep_ref.qkv_prep(qkv, qw, kw, _freqs(D), 1e-6, 0, pos, Hq, Hkv, D)
    v = qkv.reshape(qkv.shape[0], Hq + 2 * Hkv, D)[:, Hq + Hkv:]
    assert np.array_equal(r["v_bits"], v)
