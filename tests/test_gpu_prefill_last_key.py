"""GPU parity of attn_prefill with per-row last keys (the rows of an image
see each other on sliding layers: PR #975 commit body, each row's last key,
its own position for text rows; PR #1183 body, the last-key rows of the
sliding-window attention).

The prompt is fed chunk by chunk; the library clamps each row's last key to
[own position, the chunk's last row], so the expected last keys are the
oracle's clamp applied per chunk.  Spans cross 16-row tiles, key blocks and
chunk boundaries; the full-size sliding workload is checked on sampled rows.
"""
import numpy as np
import pytest

from gpu_util import run_prefill, say
from oracle import attn_ref
from oracle.contract import P_BF16, P_BF16X2, key_block
from synthetic.gen import (WORKLOADS, chunk_starts, f32_to_bf16_bits,
                           image_span_last_keys, image_spans, prefill_inputs,
                           randn_bf16_bits)

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


def _per_chunk(lk, pos0, n, chunk):
    """The last keys the library uses: clamped within each chunk."""
    return np.concatenate([attn_ref.clamp_last_key(lk[r0:r0 + chunk], pos0 + r0,
                                                   min(chunk, n - r0))
                           for r0 in range(0, n, chunk)])


@pytest.mark.parametrize("D,Hq,Hkv,ring,cap,window,chunk,n,pos0,p_mode,spans", [
    # sliding layer, ring wraps, spans across tiles, key blocks and a chunk end
    (256, 32, 4, 1, 1152, 1024, 128, 640, 0, P_BF16,
     [(10, 75), (130, 250), (300, 301), (400, 527)]),
    # small window: a span longer than the window, ragged chunks
    (256, 8, 1, 1, 200, 150, 37, 300, 0, P_BF16X2, [(20, 60), (100, 290)]),
    # pos0 > 0, ragged last tile
    (256, 16, 2, 0, 700, 0, 100, 333, 200, P_BF16, [(205, 299), (310, 332)]),
    # global layer
    (512, 32, 2, 0, 1500, 0, 512, 1100, 0, P_BF16X2, [(0, 40), (600, 1000)]),
    # G = 2 (idle waves), windowed ring at D = 512
    (512, 4, 2, 1, 300, 100, 50, 400, 0, P_BF16, [(45, 90), (210, 260)]),
    # G = 1, window of 1: a row sees only keys at and after its own position
    (256, 2, 2, 1, 64, 1, 16, 130, 0, P_BF16X2, [(3, 12), (40, 71)]),
])
def test_prefill_last_key_spans(ga, D, Hq, Hkv, ring, cap, window, chunk, n, pos0,
                                p_mode, spans):
    say("prefill last key", D, Hq, Hkv, ring, cap, window, chunk, n, pos0, p_mode, spans)
    rng = np.random.default_rng(D + Hq + cap + n + 7)
    q = randn_bf16_bits(rng, (n, Hq, D))
    k = randn_bf16_bits(rng, (pos0 + n, Hkv, D))
    v = randn_bf16_bits(rng, (pos0 + n, Hkv, D))
    scale = 1 / np.sqrt(D)
    lk = image_span_last_keys(pos0, n, spans)
    caches = None
    if pos0:
        import torch
        from gpu_util import up, DEV
        kc = torch.zeros((Hkv, cap, D), dtype=torch.int16, device=DEV)
        vc = torch.zeros_like(kc)
        ga.attn_cache_write(kc, vc, up(k[:pos0]), up(v[:pos0]), 0, pos0, Hkv, D, cap, ring)
        caches = (kc, vc)
    got, _ = run_prefill(ga, q, k, v, Hkv, cap, ring, window, scale, p_mode, chunk,
                         pos0=pos0, caches=caches, last_key=lk)
    ref = attn_ref.prefill(q, k, v, pos0, Hkv, window, scale, p_mode, key_block(D, p_mode),
                           last_key=_per_chunk(lk, pos0, n, chunk))
    _check(f"last key D={D} ring={ring} W={window} chunk={chunk}", got, ref)


@pytest.mark.parametrize("D,p_mode", [(256, P_BF16), (512, P_BF16X2)])
def test_prefill_last_key_clamps_out_of_range(ga, D, p_mode):
    """Values before the own position or past the chunk are clamped."""
    say("prefill last key clamp", D)
    rng = np.random.default_rng(21 + D)
    Hq, Hkv, n, cap, chunk = 8, 1, 200, 256, 64
    q = randn_bf16_bits(rng, (n, Hq, D))
    k = randn_bf16_bits(rng, (n, Hkv, D))
    v = randn_bf16_bits(rng, (n, Hkv, D))
    lk = rng.integers(-1000, 1000, n).astype(np.int64)
    lk[::7] = np.iinfo(np.int32).max
    lk[3::7] = np.iinfo(np.int32).min
    got, _ = run_prefill(ga, q, k, v, Hkv, cap, 0, 0, 0.06, p_mode, chunk, last_key=lk)
    ref = attn_ref.prefill(q, k, v, 0, Hkv, 0, 0.06, p_mode, key_block(D, p_mode),
                           last_key=_per_chunk(lk, 0, n, chunk))
    _check(f"last key clamp D={D}", got, ref)


@pytest.mark.parametrize("D,p_mode", [(256, P_BF16X2), (512, P_BF16)])
def test_prefill_own_position_last_key_equals_causal(ga, D, p_mode):
    say("prefill last key = own position", D)
    rng = np.random.default_rng(33 + D)
    Hq, Hkv, n, cap, chunk, W = 16, 2, 300, 400, 96, 70
    q = randn_bf16_bits(rng, (n, Hq, D))
    k = randn_bf16_bits(rng, (n, Hkv, D))
    v = randn_bf16_bits(rng, (n, Hkv, D))
    a, _ = run_prefill(ga, q, k, v, Hkv, cap, 1, W, 0.05, p_mode, chunk)
    b, _ = run_prefill(ga, q, k, v, Hkv, cap, 1, W, 0.05, p_mode, chunk,
                       last_key=np.arange(n))
    assert np.array_equal(a, b)


@pytest.mark.parametrize("D", [256, 512])
def test_prefill_image_row_sees_later_image_key(ga, D):
    """A dominating key at an image's last position is returned exactly by
    every row of the image, and by no text row before it."""
    say("prefill later image key", D)
    rng = np.random.default_rng(40 + D)
    Hq, Hkv, n, cap, span = 4, 1, 160, 160, (37, 120)
    q = randn_bf16_bits(rng, (n, Hq, D))
    q[:] = q[:1, :1]
    k = f32_to_bf16_bits((rng.standard_normal((n, Hkv, D)) * 0.02).astype(np.float32))
    v = randn_bf16_bits(rng, (n, Hkv, D))
    qf = (q[0, 0].astype(np.uint32) << 16).view(np.float32)
    k[span[1], 0] = f32_to_bf16_bits(8 * qf)
    lk = image_span_last_keys(0, n, [span])
    got, _ = run_prefill(ga, q, k, v, Hkv, cap, 0, 128, 1.0, P_BF16, n, last_key=lk)
    for i in range(span[0], span[1] + 1):
        assert np.all(got[i] == v[span[1], 0][None, :]), i
    for i in range(span[0]):
        assert not np.all(got[i] == v[span[1], 0][None, :]), i


def test_prefill_sliding_8k_image_spans_full(ga):
    """The full-size sliding prompt with six images (64 to 280 rows each),
    fed in chunks of up to 512 rows that never cut an image, over a
    1536-slot ring; sampled rows, one image whole."""
    w = WORKLOADS["prefill_sliding_8k"]
    say("prefill workload with image spans", w.name)
    q, k, v = prefill_inputs(w)
    spans = image_spans(np.random.default_rng(w.seed + 1), w.n_rows)
    lk = image_span_last_keys(0, w.n_rows, spans)
    starts = chunk_starts(w.n_rows, 512, spans)
    got, _ = run_prefill(ga, q, k, v, w.Hkv, 1536, 1, w.window, w.scale, w.p_mode,
                         None, last_key=lk, starts=starts)
    rng = np.random.default_rng(3)
    a, b = spans[2]
    rows = set(range(max(0, a - 8), min(w.n_rows, b + 9)))     # one image whole
    rows |= set(range(w.n_rows - 16, w.n_rows))
    rows |= set(int(x) for x in rng.integers(0, w.n_rows, 96))
    rows = np.array(sorted(rows))
    ref = attn_ref.prefill(q, k, v, 0, w.Hkv, w.window, w.scale, w.p_mode,
                           key_block(w.D, w.p_mode), rows=rows, last_key=lk)
    _check(w.name + " + image spans", got[rows], ref)
