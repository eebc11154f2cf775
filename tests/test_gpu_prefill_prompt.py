"""GPU checks of attn_prefill_prompt, the whole-prompt entry point: its
outputs and final caches equal attn_cache_write + attn_prefill chunk by chunk
bit for bit (one attention launch over the whole prompt: key blocks sit on
absolute positions; a ring's attended span goes to a linear copy first; large
launches take eight heads a workgroup, with the same per-head arithmetic), on
the 8k sliding prompt and on small shapes with ragged chunks, rings that wrap,
positions past the cache start, per-row last keys clamped per chunk, NaN in
unwritten slots and both head dims; two shapes are also checked against the
oracle.
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


def _prompt(ga, q, k, v, Hkv, cap, ring, window, scale, p_mode, chunk, pos0=0, caches=None,
            last_key=None):
    n, Hq, D = q.shape
    if caches is None:
        kc = torch.zeros((Hkv, cap, D), dtype=torch.int16, device=DEV)
        vc = torch.zeros_like(kc)
    else:
        kc, vc = (c.clone() for c in caches)
    out = torch.empty((n, Hq, D), dtype=torch.int16, device=DEV)
    ws = None
    nb = ga.attn_prefill_prompt_workspace_bytes(pos0, n, Hkv, D, ring, window)
    if ring:
        assert nb > 0
        ws = torch.full((nb,), 0xFF, dtype=torch.uint8, device=DEV)   # contents ignored
    lk = None if last_key is None else up(np.asarray(last_key, dtype=np.int32))
    ga.attn_prefill_prompt(out, up(q), up(k[pos0:pos0 + n]), up(v[pos0:pos0 + n]), kc, vc, pos0,
                           n, chunk, Hq, Hkv, D, cap, ring, window, scale, p_mode, workspace=ws,
                           last_key=lk)
    return down(out), down(kc), down(vc)


def test_prompt_sliding_8k_equals_chunk_calls(ga):
    """The 8192-token sliding prompt (128-row chunks, four ranges a tile)."""
    w = WORKLOADS["prefill_sliding_8k"]
    say("prompt entry point,", w.name)
    q, k, v = prefill_inputs(w)
    got, gk, gv = _prompt(ga, q, k, v, w.Hkv, w.cap, w.ring, w.window, w.scale, w.p_mode,
                          w.chunk)
    want, (kc, vc) = run_prefill(ga, q, k, v, w.Hkv, w.cap, w.ring, w.window, w.scale,
                                 w.p_mode, w.chunk)
    assert np.array_equal(got, want)
    assert np.array_equal(gk, down(kc)) and np.array_equal(gv, down(vc))


@pytest.mark.parametrize("D,Hq,Hkv,ring,cap,window,chunk,n,pos0,p_mode", [
    (256, 32, 4, 1, 1152, 1024, 128, 1500, 0, P_BF16),      # wraps, ragged last chunk
    (256, 32, 4, 1, 1152, 1024, 128, 700, 2900, P_BF16),    # ring already wrapped before pos0
    (256, 16, 2, 0, 900, 0, 100, 333, 400, P_BF16X2),       # pos0 > 0, causal
    (256, 8, 1, 1, 200, 150, 37, 300, 0, P_BF16),           # ragged chunks in a small ring
    (512, 32, 2, 0, 1500, 0, 512, 1100, 0, P_BF16X2),       # head dim 512
    (512, 16, 1, 1, 96, 33, 64, 200, 0, P_BF16),            # ring < block span
    (512, 8, 2, 1, 300, 200, 50, 260, 77, P_BF16X2),        # head dim 512 ring, pos0 > 0
    (512, 8, 2, 1, 300, 200, 50, 260, 500, P_BF16X2),       # ... staged span not from slot 0
    (256, 6, 2, 0, 200, 5, 16, 100, 0, P_BF16),             # G = 3, tiny window
    (256, 8, 1, 0, 64, 0, 1000, 60, 0, P_BF16),             # one chunk shorter than chunk
    (256, 12, 2, 1, 1100, 1000, 100, 2048, 0, P_BF16X2),    # G = 6 on eight-wave workgroups
    (256, 2, 2, 1, 64, 1, 16, 130, 5, P_BF16X2),            # window of 1, pos0 > 0
])
def test_prompt_shapes_equal_chunk_calls(ga, D, Hq, Hkv, ring, cap, window, chunk, n, pos0,
                                         p_mode):
    say("prompt shape", D, Hq, Hkv, ring, cap, window, chunk, n, pos0, p_mode)
    rng = np.random.default_rng(D + Hq + cap + n + 5)
    q = randn_bf16_bits(rng, (n, Hq, D))
    k = randn_bf16_bits(rng, (pos0 + n, Hkv, D))
    v = randn_bf16_bits(rng, (pos0 + n, Hkv, D))
    scale = 1 / np.sqrt(D)
    caches = None
    if pos0:
        # earlier positions already in the cache (a ring keeps the last cap)
        kc = torch.zeros((Hkv, cap, D), dtype=torch.int16, device=DEV)
        vc = torch.zeros_like(kc)
        p1 = max(0, pos0 - cap) if ring else 0
        ga.attn_cache_write(kc, vc, up(k[p1:pos0]), up(v[p1:pos0]), p1, pos0 - p1, Hkv, D, cap,
                            ring)
        caches = (kc, vc)
    got, gk, gv = _prompt(ga, q, k, v, Hkv, cap, ring, window, scale, p_mode, chunk, pos0=pos0,
                          caches=caches)
    want, (wk, wv) = run_prefill(ga, q, k, v, Hkv, cap, ring, window, scale, p_mode, chunk,
                                 pos0=pos0, caches=None if caches is None else
                                 tuple(c.clone() for c in caches))
    assert np.array_equal(got, want)
    assert np.array_equal(gk, down(wk)) and np.array_equal(gv, down(wv))
    if ring == 1 and n >= 500:
        ref = attn_ref.prefill(q, k, v, pos0, Hkv, window, scale, p_mode, key_block(D, p_mode))
        res = attn_ref.check(got, ref["o"], ref["r"])
        say("vs oracle", {x: res[x] for x in ("n", "fails", "mean_rel_err", "bit_equal")})
        assert res["ok"] and res["bit_equal"] >= 0.9, res


def test_prompt_last_key(ga):
    """Per-row last keys, taken chunk by chunk."""
    D, Hq, Hkv, cap, W, chunk, n = 256, 16, 2, 600, 512, 64, 400
    rng = np.random.default_rng(6)
    q = randn_bf16_bits(rng, (n, Hq, D))
    k = randn_bf16_bits(rng, (n, Hkv, D))
    v = randn_bf16_bits(rng, (n, Hkv, D))
    last = np.arange(n, dtype=np.int64)
    last[200:260] = 259
    got, _, _ = _prompt(ga, q, k, v, Hkv, cap, 1, W, 1 / 16, P_BF16, chunk, last_key=last)
    want, _ = run_prefill(ga, q, k, v, Hkv, cap, 1, W, 1 / 16, P_BF16, chunk, last_key=last)
    assert np.array_equal(got, want)
    # the clamp is per chunk: rows 200..255 reach key 255, rows 256..259 key 259
    clamped = np.concatenate([attn_ref.clamp_last_key(last[r0:r0 + chunk], r0, min(chunk, n - r0))
                              for r0 in range(0, n, chunk)])
    ref = attn_ref.prefill(q, k, v, 0, Hkv, W, 1 / 16, P_BF16, key_block(D, P_BF16),
                           last_key=clamped)
    res = attn_ref.check(got, ref["o"], ref["r"])
    assert res["ok"] and res["bit_equal"] >= 0.9, res


def test_prompt_nan_in_unwritten_slots(ga):
    """A ring whose unwritten slots hold NaN, and a NaN-filled workspace: no
    output becomes NaN, and the bits equal the chunked path's."""
    D, Hq, Hkv, cap, W, chunk, n = 256, 32, 4, 1152, 1024, 128, 512
    rng = np.random.default_rng(10)
    q = randn_bf16_bits(rng, (n, Hq, D))
    k = randn_bf16_bits(rng, (n, Hkv, D))
    v = randn_bf16_bits(rng, (n, Hkv, D))
    kc = torch.full((Hkv, cap, D), 0x7FC0, dtype=torch.int16, device=DEV)
    vc = torch.full((Hkv, cap, D), 0x7FC0, dtype=torch.int16, device=DEV)
    got, _, _ = _prompt(ga, q, k, v, Hkv, cap, 1, W, 1 / 16, P_BF16, chunk, caches=(kc, vc))
    assert not np.any(((got & 0x7F80) == 0x7F80) & ((got & 0x7F) != 0))
    want, _ = run_prefill(ga, q, k, v, Hkv, cap, 1, W, 1 / 16, P_BF16, chunk,
                          caches=(kc.clone(), vc.clone()))
    assert np.array_equal(got, want)


def test_prompt_last_key_eight_wave_launch(ga):
    """Per-row last keys (image spans, some crossing chunk ends) in a launch
    large enough for eight-wave workgroups: the chunked path's bits."""
    D, Hq, Hkv, cap, W, chunk, n = 256, 32, 4, 1152, 1024, 128, 2048
    rng = np.random.default_rng(12)
    q = randn_bf16_bits(rng, (n, Hq, D))
    k = randn_bf16_bits(rng, (n, Hkv, D))
    v = randn_bf16_bits(rng, (n, Hkv, D))
    last = np.arange(n, dtype=np.int64)
    for a, b in ((100, 180), (250, 270), (700, 900), (1500, 1536), (2000, 2047)):
        last[a:b] = b - 1
    got, _, _ = _prompt(ga, q, k, v, Hkv, cap, 1, W, 1 / 16, P_BF16, chunk, last_key=last)
    want, _ = run_prefill(ga, q, k, v, Hkv, cap, 1, W, 1 / 16, P_BF16, chunk, last_key=last)
    assert np.array_equal(got, want)
