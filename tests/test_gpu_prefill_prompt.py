"""GPU checks of attn_prefill_prompt, the whole-prompt entry point: its
outputs and caches equal attn_cache_write + attn_prefill(_ws) chunk by chunk
bit for bit (the same kernels in the same order; a split chunk's merge shares
a launch with the next chunk's cache write), on the 8k sliding prompt and on
small shapes with ragged chunks, rings, positions past the cache start, per-row
last keys and both head dims; one shape is also checked against the oracle.
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
            last_key=None, split=True):
    n, Hq, D = q.shape
    if caches is None:
        kc = torch.zeros((Hkv, cap, D), dtype=torch.int16, device=DEV)
        vc = torch.zeros_like(kc)
    else:
        kc, vc = (c.clone() for c in caches)
    out = torch.empty((n, Hq, D), dtype=torch.int16, device=DEV)
    ws = None
    if split:
        ws = torch.empty(ga.attn_prefill_workspace_bytes(min(chunk, n), Hq, D), dtype=torch.uint8,
                         device=DEV)
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
                                 w.p_mode, w.chunk, split=True)
    assert np.array_equal(got, want)
    assert np.array_equal(gk, down(kc)) and np.array_equal(gv, down(vc))


@pytest.mark.parametrize("D,Hq,Hkv,ring,cap,window,chunk,n,pos0,p_mode,split", [
    (256, 32, 4, 1, 1152, 1024, 128, 1500, 0, P_BF16, True),      # wraps, ragged last chunk
    (256, 16, 2, 0, 900, 0, 100, 333, 400, P_BF16X2, True),       # pos0 > 0, causal
    (256, 8, 1, 1, 200, 150, 37, 300, 0, P_BF16, False),          # no workspace
    (512, 32, 2, 0, 1500, 0, 512, 1100, 0, P_BF16X2, True),       # head dim 512 (no split)
    (512, 16, 1, 1, 96, 33, 64, 200, 0, P_BF16, False),           # ring < block span
    (256, 6, 2, 0, 200, 5, 16, 100, 0, P_BF16, True),             # G = 3, tiny window
    (256, 8, 1, 0, 64, 0, 1000, 60, 0, P_BF16, True),             # one chunk shorter than chunk
])
def test_prompt_shapes_equal_chunk_calls(ga, D, Hq, Hkv, ring, cap, window, chunk, n, pos0,
                                         p_mode, split):
    say("prompt shape", D, Hq, Hkv, ring, cap, window, chunk, n, pos0, p_mode, split)
    rng = np.random.default_rng(D + Hq + cap + n + 5)
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
    got, gk, gv = _prompt(ga, q, k, v, Hkv, cap, ring, window, scale, p_mode, chunk, pos0=pos0,
                          caches=caches, split=split)
    want, (wk, wv) = run_prefill(ga, q, k, v, Hkv, cap, ring, window, scale, p_mode, chunk,
                                 pos0=pos0, caches=None if caches is None else
                                 tuple(c.clone() for c in caches), split=split)
    assert np.array_equal(got, want)
    assert np.array_equal(gk, down(wk)) and np.array_equal(gv, down(wv))
    if D == 256 and ring == 1 and split:
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
    want, _ = run_prefill(ga, q, k, v, Hkv, cap, 1, W, 1 / 16, P_BF16, chunk, last_key=last,
                          split=True)
    assert np.array_equal(got, want)
