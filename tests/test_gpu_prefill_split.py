"""GPU parity of the split prompt attention (attn_prefill_ws) against the CPU
oracle, and against the unsplit attn_prefill.

At head dim 256 a short chunk's tiles split their key blocks over up to four
workgroups; each range after the first walks the blocks before it for their
maxima so that every rounded P equals the unsplit walk's, and the ranges'
partials are merged.  The 8k sliding prompt (64-workgroup chunks, four
ranges a tile) is checked on every output; small shapes cover ragged tiles,
windows, rings, both P modes, per-row last keys and NaN-poisoned unwritten
slots.  The split differs from attn_prefill by fp32 addition order only, so
the two agree bit for bit almost everywhere and elsewhere within two bf16
steps (near zero, within a small fraction of the row's largest output); with
a NULL workspace, or at head dim 512, attn_prefill_ws is attn_prefill bit for
bit.
"""
import numpy as np
import pytest
import torch

from gpu_util import DEV, down, run_prefill, say, up
from oracle import attn_ref
from oracle.contract import P_BF16, P_BF16X2, key_block
from synthetic.gen import WORKLOADS, prefill_inputs, randn_bf16_bits

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ga():
    import global_gqa_attention_window_amd as ga
    return ga


def _check(tag, got, ref):
    res = attn_ref.check(got, ref["o"], ref["r"])
    say(tag, {k: res[k] for k in ("n", "fails", "max_steps_out", "mean_rel_err", "bit_equal")})
    assert res["ok"], (tag, res)
    assert res["bit_equal"] >= 0.9, (tag, res)


def _far(a, b):
    """Outputs of two bf16 bit arrays [rows][heads][D] that differ by more than
    two bf16 steps of the larger magnitude, where that is also more than 2^-12
    of the (row, head)'s largest output (values near zero, summed from terms
    of either sign, may change sign with the addition order)."""
    from oracle import bf16
    x, y = bf16.f64_from_bits(a), bf16.f64_from_bits(b)
    big = np.maximum(np.abs(x), np.abs(y))
    step = np.exp2(np.floor(np.log2(np.maximum(big, 1e-300))) - 7)
    scale = np.max(np.abs(y), axis=-1, keepdims=True)
    d = np.abs(x - y)
    return int(np.count_nonzero((d > 2 * step) & (d > scale * 2.0 ** -12)))


@pytest.fixture(scope="module")
def sliding_8k_split(ga):
    """The 8192-token sliding prompt through the split path, and unsplit."""
    w = WORKLOADS["prefill_sliding_8k"]
    say("prefill workload (split)", w.name)
    q, k, v = prefill_inputs(w)
    got, _ = run_prefill(ga, q, k, v, w.Hkv, w.cap, w.ring, w.window, w.scale,
                         w.p_mode, w.chunk, split=True)
    plain, _ = run_prefill(ga, q, k, v, w.Hkv, w.cap, w.ring, w.window, w.scale,
                           w.p_mode, w.chunk)
    return w, q, k, v, got, plain


@pytest.mark.parametrize("part", range(4))
def test_split_sliding_8k_every_row(sliding_8k_split, part):
    w, q, k, v, got, _ = sliding_8k_split
    rows = np.arange(part * 2048, (part + 1) * 2048)
    say("rows", rows[0], "..", rows[-1])
    ref = attn_ref.prefill(q, k, v, 0, w.Hkv, w.window, w.scale, w.p_mode,
                           key_block(w.D, w.p_mode), rows=rows, row_batch=64)
    _check(f"{w.name} (split) rows {rows[0]}..{rows[-1]}", got[rows], ref)


def test_split_sliding_8k_close_to_unsplit(sliding_8k_split):
    """Same P bits, other fp32 addition order: almost every output equal to
    the unsplit one, and none farther than two bf16 steps (or, near zero, a
    small fraction of its row's largest output)."""
    _, _, _, _, got, plain = sliding_8k_split
    same = float(np.mean(got == plain))
    far = _far(got, plain)
    say("split vs unsplit", {"bit_equal": same, "far": far})
    assert far == 0 and same >= 0.99


@pytest.mark.parametrize("Hq,Hkv,ring,cap,window,chunk,n,pos0,p_mode", [
    (32, 4, 1, 1152, 1024, 128, 1500, 0, P_BF16),        # the sliding shape, wraps
    (32, 4, 1, 1152, 1024, 128, 300, 0, P_BF16X2),       # both P modes
    (8, 1, 1, 200, 150, 37, 300, 0, P_BF16),             # ragged chunks, short ranges
    (16, 2, 0, 900, 0, 100, 333, 400, P_BF16X2),         # pos0 > 0, ragged tile, causal
    (6, 2, 0, 200, 5, 16, 100, 0, P_BF16),               # G = 3, tiny window (empty ranges)
    (2, 2, 1, 64, 1, 16, 130, 0, P_BF16X2),              # window of 1
    (8, 1, 0, 2100, 0, 64, 2048, 0, P_BF16),             # long causal walks, one KV head
])
def test_split_shapes(ga, Hq, Hkv, ring, cap, window, chunk, n, pos0, p_mode):
    D = 256
    say("split prefill shape", Hq, Hkv, ring, cap, window, chunk, n, pos0, p_mode)
    rng = np.random.default_rng(Hq + cap + n + 11)
    q = randn_bf16_bits(rng, (n, Hq, D))
    k = randn_bf16_bits(rng, (pos0 + n, Hkv, D))
    v = randn_bf16_bits(rng, (pos0 + n, Hkv, D))
    scale = 1 / np.sqrt(D)
    caches = None
    if pos0:
        kc = torch.zeros((Hkv, cap, D), dtype=torch.int16, device=DEV)
        vc = torch.zeros_like(kc)
        ga.attn_cache_write(kc, vc, up(k[:pos0]), up(v[:pos0]), 0, pos0, Hkv, D, cap, ring)
        caches = (kc, vc)
    got, _ = run_prefill(ga, q, k, v, Hkv, cap, ring, window, scale, p_mode, chunk,
                         pos0=pos0, caches=caches, split=True)
    ref = attn_ref.prefill(q, k, v, pos0, Hkv, window, scale, p_mode, key_block(D, p_mode))
    _check(f"split shape G={Hq // Hkv} ring={ring} W={window} chunk={chunk}", got, ref)


def test_split_last_key(ga):
    """Per-row last keys (an image span seeing itself) through the split path."""
    D, Hq, Hkv, cap, W, chunk, n = 256, 16, 2, 600, 512, 64, 400
    rng = np.random.default_rng(5)
    q = randn_bf16_bits(rng, (n, Hq, D))
    k = randn_bf16_bits(rng, (n, Hkv, D))
    v = randn_bf16_bits(rng, (n, Hkv, D))
    last = np.arange(n, dtype=np.int64)
    last[200:260] = 259                         # rows 200..259 see the whole span
    clamped = np.concatenate([attn_ref.clamp_last_key(last[r0:r0 + chunk], r0, min(chunk, n - r0))
                              for r0 in range(0, n, chunk)])
    got, _ = run_prefill(ga, q, k, v, Hkv, cap, 1, W, 1 / 16, P_BF16, chunk,
                         last_key=last, split=True)
    ref = attn_ref.prefill(q, k, v, 0, Hkv, W, 1 / 16, P_BF16, key_block(D, P_BF16),
                           last_key=clamped)
    _check("split last_key", got, ref)


def test_split_nan_in_unwritten_slots(ga):
    """Unwritten ring slots hold NaN: no output may become NaN."""
    D, Hq, Hkv, cap, W, chunk, n = 256, 32, 4, 1152, 1024, 128, 512
    rng = np.random.default_rng(9)
    q = randn_bf16_bits(rng, (n, Hq, D))
    k = randn_bf16_bits(rng, (n, Hkv, D))
    v = randn_bf16_bits(rng, (n, Hkv, D))
    kc = torch.full((Hkv, cap, D), 0x7FC0, dtype=torch.int16, device=DEV)
    vc = torch.full((Hkv, cap, D), 0x7FC0, dtype=torch.int16, device=DEV)
    got, _ = run_prefill(ga, q, k, v, Hkv, cap, 1, W, 1 / 16, P_BF16, chunk,
                         caches=(kc, vc), split=True)
    ref = attn_ref.prefill(q, k, v, 0, Hkv, W, 1 / 16, P_BF16, key_block(D, P_BF16))
    _check("split with NaN-poisoned unwritten slots", got, ref)


@pytest.mark.parametrize("D,ws", [(256, False), (512, True)])
def test_ws_without_split_is_attn_prefill(ga, D, ws):
    """A NULL workspace, or head dim 512, gives attn_prefill's bits."""
    Hq, Hkv, cap, n = 16, 2, 256, 200
    rng = np.random.default_rng(D + 3)
    q = randn_bf16_bits(rng, (n, Hq, D))
    k = randn_bf16_bits(rng, (n, Hkv, D))
    v = randn_bf16_bits(rng, (n, Hkv, D))
    kc = torch.zeros((Hkv, cap, D), dtype=torch.int16, device=DEV)
    vc = torch.zeros_like(kc)
    ga.attn_cache_write(kc, vc, up(k), up(v), 0, n, Hkv, D, cap, 0)
    a = torch.empty((n, Hq, D), dtype=torch.int16, device=DEV)
    b = torch.empty_like(a)
    ga.attn_prefill(a, up(q), kc, vc, 0, n, Hq, Hkv, D, cap, 0, 0, D ** -0.5, P_BF16X2)
    w = torch.empty(ga.attn_prefill_workspace_bytes(n, Hq, D), dtype=torch.uint8,
                    device=DEV) if ws else None
    ga.attn_prefill_ws(b, up(q), kc, vc, 0, n, Hq, Hkv, D, cap, 0, 0, D ** -0.5, P_BF16X2, w)
    assert np.array_equal(down(a), down(b))
