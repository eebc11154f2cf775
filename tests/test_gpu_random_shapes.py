"""Seeded random shapes through the C ABI against the CPU oracle.

Each case draws its geometry from its own seed: head dim 256 or 512, 1-4 KV
heads, a GQA group of 1-16 query heads (including sizes no fixed test uses,
such as 5, 6 and 12), a linear or ring cache, a window or none, positions
before, inside and past the cache, decode windows of 1-16 rows, prompt
chunks of 1-519 rows and either P mode.  Every output element is checked
with the oracle's range test, as in the fixed-shape tests; each prompt also
goes through attn_prefill_prompt (one launch), which must give the chunked
path's outputs and final caches bit for bit.
"""
import numpy as np
import pytest

from gpu_util import DEV, down, run_decode, run_decode_rows, run_prefill, say, up
from oracle import attn_ref
from oracle.contract import key_block
from synthetic.gen import randn_bf16_bits

pytestmark = pytest.mark.gpu

N_CASES = 48


@pytest.fixture(scope="module")
def ga():
    import global_gqa_attention_window_amd as ga
    return ga


def _decode_case(rng, kind):
    D = int(rng.choice([256, 512]))
    Hkv = int(rng.integers(1, 5))
    G = int(rng.choice([1, 2, 3, 4, 5, 6, 8, 12, 16]))
    ring = int(rng.integers(0, 2))
    R = 1 if kind == "decode" else int(rng.integers(1, 17))
    big = rng.random() < 0.1
    S = 1 if big else int(rng.integers(1, 4))
    cap = max(R, int(rng.integers(1, 40000 if big else 3000)))
    if ring:
        W = int(rng.integers(1, cap - R + 2))
        pos = rng.integers(-R, 4 * cap, S)
    else:
        W = 0 if rng.random() < 0.5 else int(rng.integers(1, cap + 1))
        pos = rng.integers(-R, max(1, cap - R + 1), S)
    return dict(D=D, Hkv=Hkv, Hq=G * Hkv, ring=ring, R=R, S=S, cap=cap, W=W,
                pos=[int(p) for p in pos], scale=float(rng.uniform(0.02, 0.1)))


def _prefill_case(rng):
    D = int(rng.choice([256, 512]))
    Hkv = int(rng.integers(1, 5))
    G = int(rng.choice([1, 2, 3, 4, 5, 6, 8, 12, 16]))
    ring = int(rng.integers(0, 2))
    n = int(rng.integers(1, 700))
    chunk = int(rng.integers(1, 520))
    pos0 = int(rng.integers(0, 300)) if rng.random() < 0.3 else 0
    if ring:
        W = int(rng.integers(1, 1200))
        cap = W + min(chunk, n) - 1 + int(rng.integers(0, 200))
    else:
        W = 0 if rng.random() < 0.6 else int(rng.integers(1, 1200))
        cap = pos0 + n + int(rng.integers(0, 100))
    return dict(D=D, Hkv=Hkv, Hq=G * Hkv, ring=ring, n=n, chunk=chunk, pos0=pos0, cap=cap,
                W=W, p_mode=int(rng.choice([1, 2])), scale=float(rng.uniform(0.02, 0.1)))


@pytest.mark.parametrize("case", range(N_CASES))
def test_random_shape(ga, case):
    import torch
    rng = np.random.default_rng(90000 + case)
    kind = str(rng.choice(["decode", "rows", "prefill"], p=[0.3, 0.35, 0.35]))
    if kind == "prefill":
        c = _prefill_case(rng)
        say("random prefill", case, c)
        D, Hkv, Hq, n, pos0, cap, ring, W = (c[x] for x in
                                              ("D", "Hkv", "Hq", "n", "pos0", "cap", "ring", "W"))
        q = randn_bf16_bits(rng, (n, Hq, D))
        k = randn_bf16_bits(rng, (pos0 + n, Hkv, D))
        v = randn_bf16_bits(rng, (pos0 + n, Hkv, D))
        caches = None
        if pos0:
            # the rows before pos0 go into the cache first, in pieces the ring holds
            kc = torch.zeros((Hkv, cap, D), dtype=torch.int16, device=DEV)
            vc = torch.zeros_like(kc)
            step = max(1, cap - W + 1) if ring else pos0
            for a in range(0, pos0, step):
                b = min(pos0, a + step)
                ga.attn_cache_write(kc, vc, up(k[a:b]), up(v[a:b]), a, b - a, Hkv, D, cap, ring)
            caches = (kc, vc)
        before = None if caches is None else tuple(t.clone() for t in caches)
        got, (kc1, vc1) = run_prefill(ga, q, k, v, Hkv, cap, ring, W, c["scale"], c["p_mode"],
                                      c["chunk"], pos0=pos0, caches=caches)
        # the whole prompt in one launch: the same bits and the same caches
        if before is None:
            kc2 = torch.zeros((Hkv, cap, D), dtype=torch.int16, device=DEV)
            vc2 = torch.zeros_like(kc2)
        else:
            kc2, vc2 = before
        out2 = torch.empty((n, Hq, D), dtype=torch.int16, device=DEV)
        nb = ga.attn_prefill_prompt_workspace_bytes(pos0, n, Hkv, D, ring, W)
        ws = torch.empty(nb, dtype=torch.uint8, device=DEV) if ring else None
        ga.attn_prefill_prompt(out2, up(q), up(k[pos0:]), up(v[pos0:]), kc2, vc2, pos0, n,
                               c["chunk"], Hq, Hkv, D, cap, ring, W, c["scale"], c["p_mode"],
                               workspace=ws)
        assert np.array_equal(down(out2), got), (case, c)
        assert np.array_equal(down(kc2), down(kc1)) and np.array_equal(down(vc2), down(vc1))
        ref = attn_ref.prefill(q, k, v, pos0, Hkv, W, c["scale"], c["p_mode"],
                               key_block(D, c["p_mode"]))
    else:
        c = _decode_case(rng, kind)
        say("random", kind, case, c)
        D, Hkv, Hq, S, R, cap = (c[x] for x in ("D", "Hkv", "Hq", "S", "R", "cap"))
        q = randn_bf16_bits(rng, (S, R, Hq, D))
        k = randn_bf16_bits(rng, (S, Hkv, cap, D))
        v = randn_bf16_bits(rng, (S, Hkv, cap, D))
        if kind == "decode":
            got = run_decode(ga, q[:, 0], k, v, c["pos"], Hkv, c["ring"], c["W"], c["scale"])
            got = got[:, None]
        else:
            got = run_decode_rows(ga, q, k, v, c["pos"], Hkv, c["ring"], c["W"], c["scale"])
        ref = attn_ref.decode_rows(q, k, v, c["pos"], Hkv, c["ring"], c["W"], c["scale"])
    res = attn_ref.check(got.reshape(ref["o"].shape), ref["o"], ref["r"])
    say("  ", {x: res[x] for x in ("n", "fails", "max_steps_out", "mean_rel_err", "bit_equal")})
    assert res["ok"], (case, c, res)
    assert res["bit_equal"] >= 0.9, (case, c, res)
