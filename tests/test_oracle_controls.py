"""The pass criterion has teeth, and admits an honest fp32 kernel (CPU only).

  * An fp32 NumPy model of the kernel schedule (tests/fp32_emulation.py:
    chunk partials for decode, KB-block online softmax for prefill) passes
    attn_ref.check with 0 fails.
  * Controls (planted mistakes, after the pages' practice of controls that
    each remove one rounding point and must fail, TensorFold PR #1183,
    receipt): P left unrounded, the wrong key block, P rounded against
    the final maximum, bf16 P in decode, a window one key too wide -- each one
    is refused by the check.
  * Planted mistakes inside the oracle itself (a dropped scale, a wrong ring
    formula, K of the wrong KV head, a window off by one) are caught by the
    brute-force and identity pins.
"""
import numpy as np
import pytest

import fp32_emulation as emu
from oracle import attn_ref, brute
from oracle.contract import P_BF16, P_BF16X2, P_FP32, key_block
from synthetic.gen import f32_to_bf16_bits


def _bits(rng, shape, sd=1.0):
    return f32_to_bf16_bits((rng.standard_normal(shape) * sd).astype(np.float32))


@pytest.fixture(scope="module")
def prefill_case():
    rng = np.random.default_rng(21)
    n, Hkv, G, D = 384, 1, 8, 256
    q = _bits(rng, (n, Hkv * G, D))
    k = _bits(rng, (n, Hkv, D))
    v = _bits(rng, (n, Hkv, D))
    return q, k, v, Hkv, D


@pytest.fixture(scope="module")
def prefill_ref(prefill_case):
    q, k, v, Hkv, D = prefill_case
    return attn_ref.prefill(q, k, v, 0, Hkv, 160, 1 / 16, P_BF16,
                            key_block(D, P_BF16))


def test_fp32_prefill_schedule_passes(prefill_case, prefill_ref):
    q, k, v, Hkv, D = prefill_case
    got = emu.prefill(q, k, v, 0, Hkv, 160, 1 / 16, P_BF16, key_block(D, P_BF16))
    res = attn_ref.check(got, prefill_ref["o"], prefill_ref["r"])
    assert res["fails"] == 0 and res["ok"], res


def test_fp32_prefill_two_halves_passes():
    rng = np.random.default_rng(22)
    n, Hkv, G, D = 256, 1, 4, 512
    q = _bits(rng, (n, Hkv * G, D))
    k = _bits(rng, (n, Hkv, D))
    v = _bits(rng, (n, Hkv, D))
    kb = key_block(D, P_BF16X2)
    ref = attn_ref.prefill(q, k, v, 0, Hkv, 0, 1 / np.sqrt(512), P_BF16X2, kb)
    got = emu.prefill(q, k, v, 0, Hkv, 0, 1 / np.sqrt(512), P_BF16X2, kb)
    res = attn_ref.check(got, ref["o"], ref["r"])
    assert res["fails"] == 0 and res["ok"], res


def test_fp32_decode_schedule_passes():
    rng = np.random.default_rng(23)
    S, Hkv, G, D, cap = 2, 1, 16, 512, 4096
    q = _bits(rng, (S, Hkv * G, D))
    k = _bits(rng, (S, Hkv, cap, D))
    v = _bits(rng, (S, Hkv, cap, D))
    pos = [4095, 3000]
    ref = attn_ref.decode(q, k, v, pos, Hkv, 0, 0, 1 / np.sqrt(512))
    got = emu.decode(q, k, v, pos, Hkv, 0, 0, 1 / np.sqrt(512))
    res = attn_ref.check(got, ref["o"], ref["r"])
    assert res["fails"] == 0 and res["ok"], res


@pytest.mark.parametrize("control", ["p_unrounded", "kb_double", "kb_half",
                                     "final_max", "window_wide"])
def test_prefill_controls_are_red(prefill_case, prefill_ref, control):
    q, k, v, Hkv, D = prefill_case
    kb = key_block(D, P_BF16)
    args = dict(p_mode=P_BF16, kb=kb, window=160, final_max=False)
    if control == "p_unrounded":
        args["p_mode"] = P_FP32
    elif control == "kb_double":
        args["kb"] = 2 * kb
    elif control == "kb_half":
        args["kb"] = kb // 2
    elif control == "final_max":
        args["final_max"] = True
    elif control == "window_wide":
        args["window"] = 161
    got = emu.prefill(q, k, v, 0, Hkv, args["window"], 1 / 16, args["p_mode"],
                      args["kb"], final_max=args["final_max"])
    res = attn_ref.check(got, prefill_ref["o"], prefill_ref["r"])
    assert res["fails"] > 0, (control, res)


def test_decode_control_bf16_p_is_red():
    rng = np.random.default_rng(24)
    S, Hkv, G, D, cap = 1, 1, 16, 256, 2048
    q = _bits(rng, (S, Hkv * G, D))
    k = _bits(rng, (S, Hkv, cap, D))
    v = _bits(rng, (S, Hkv, cap, D))
    ref = attn_ref.decode(q, k, v, [2047], Hkv, 0, 0, 1 / 16)
    got = emu.decode(q, k, v, [2047], Hkv, 0, 0, 1 / 16, p_mode=P_BF16)
    assert attn_ref.check(got, ref["o"], ref["r"])["fails"] > 0


# ------------------------------------------------- mistakes planted in oracle

def _tiny_decode(ring):
    rng = np.random.default_rng(31 + ring)
    S, Hkv, G, D, cap = 1, 2, 2, 8, 16
    q = _bits(rng, (S, Hkv * G, D))
    k = _bits(rng, (S, Hkv, cap, D))
    v = _bits(rng, (S, Hkv, cap, D))
    return q, k, v, Hkv, cap


def _brute_all(q, k, v, t, Hkv, ring, window, scale):
    G = q.shape[1] // Hkv
    f = attn_ref.as_f64
    sc = attn_ref.fp32_scale(scale)
    return np.array([brute.decode_row(f(q[0, h]).tolist(), f(k[0, h // G]).tolist(),
                                      f(v[0, h // G]).tolist(), t, ring, window, sc)
                     for h in range(q.shape[1])])


def test_planted_dropped_scale_is_caught(monkeypatch):
    q, k, v, Hkv, cap = _tiny_decode(0)
    monkeypatch.setattr(attn_ref, "fp32_scale", lambda s: 1.0)
    bad = attn_ref.decode(q, k, v, [15], Hkv, 0, 0, 0.3)["o"][0]
    monkeypatch.undo()
    assert not np.allclose(bad, _brute_all(q, k, v, 15, Hkv, 0, 0, 0.3), atol=1e-9)


def test_planted_wrong_ring_formula_is_caught(monkeypatch):
    q, k, v, Hkv, cap = _tiny_decode(1)
    good = attn_ref.slot_positions
    monkeypatch.setattr(attn_ref, "slot_positions",
                        lambda t, c, ring: good(t + 1, c, ring) - 1)
    bad = attn_ref.decode(q, k, v, [37], Hkv, 1, 12, 0.3)["o"][0]
    monkeypatch.undo()
    assert not np.allclose(bad, _brute_all(q, k, v, 37, Hkv, 1, 12, 0.3), atol=1e-9)


def test_planted_window_off_by_one_is_caught(monkeypatch):
    q, k, v, Hkv, cap = _tiny_decode(0)
    good = attn_ref.key_valid
    monkeypatch.setattr(attn_ref, "key_valid", lambda p, t, w: good(p, t, w + 1))
    bad = attn_ref.decode(q, k, v, [15], Hkv, 0, 6, 0.3)["o"][0]
    monkeypatch.undo()
    assert not np.allclose(bad, _brute_all(q, k, v, 15, Hkv, 0, 6, 0.3), atol=1e-9)


def test_planted_wrong_kv_head_is_caught():
    q, k, v, Hkv, cap = _tiny_decode(0)
    good = attn_ref.decode(q, k, v, [15], Hkv, 0, 0, 0.3)["o"][0]
    swapped = attn_ref.decode(q, k[:, ::-1].copy(), v, [15], Hkv, 0, 0, 0.3)["o"][0]
    want = _brute_all(q, k, v, 15, Hkv, 0, 0, 0.3)
    assert np.allclose(good, want, atol=1e-12)
    assert not np.allclose(swapped, want, atol=1e-9)


def test_planted_p_rounding_dropped_is_caught(monkeypatch):
    rng = np.random.default_rng(33)
    n, D = 24, 8
    q = _bits(rng, (n, 1, D))
    k = _bits(rng, (n, 1, D), sd=2.0)
    v = _bits(rng, (n, 1, D))
    monkeypatch.setattr(attn_ref, "round_p", lambda p, mode: p)
    bad = attn_ref.prefill(q, k, v, 0, 1, 0, 0.5, P_BF16, 4)["o"]
    monkeypatch.undo()
    f = attn_ref.as_f64
    want = np.array([brute.prefill_row(f(q[i, 0]).tolist(), f(k[:, 0]).tolist(),
                                       f(v[:, 0]).tolist(), i, 0, 0.5, P_BF16, 4)
                     for i in range(n)])
    assert not np.allclose(bad[:, 0], want, atol=1e-9)
