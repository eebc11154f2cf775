"""GPU checks of the decode prologue: attn_qkv_prep against the oracle's
per-element ranges (PR #1183 qk_rows note: float64 at the rounding points,
a range over the fp32 inverse's spread and cosf's ulps), and
attn_decode_prep_fused, which runs the prologue inside the decode kernel
(PR #975 decode commits), against attn_qkv_prep + attn_decode_rows_fused bit
for bit (outputs and caches), against the oracle's attention on the
prologue's own outputs, and from a replayed HIP graph."""
import numpy as np
import pytest

from gpu_util import DEV, down, say, up
from oracle import attn_ref, bf16, prep_ref
from synthetic.gen import randn_bf16_bits

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ga():
    import global_gqa_attention_window_amd as ga
    return ga


def _freqs(D, theta):
    return (1.0 / theta ** (np.arange(0, D, 2) / D)).astype(np.float32)


def _inputs(seed, S, Hq, Hkv, D, cap):
    rng = np.random.default_rng(seed)
    qkv = randn_bf16_bits(rng, (S, (Hq + 2 * Hkv) * D))
    qkv = bf16.bits_from_f64(bf16.f64_from_bits(qkv) * 3.0)       # rows of RMS 3
    qw = bf16.bits_from_f64(1.0 + 0.25 * rng.standard_normal(D))
    kw = bf16.bits_from_f64(1.0 + 0.25 * rng.standard_normal(D))
    k = randn_bf16_bits(rng, (S, Hkv, cap, D))
    v = randn_bf16_bits(rng, (S, Hkv, cap, D))
    return qkv, qw, kw, k, v


def _prep(ga, qkv, qw, kw, f, eps, v_norm, pos, Hq, Hkv, D, kd, vd, ring):
    import torch
    S = qkv.shape[0]
    q_out = torch.empty((S, Hq, D), dtype=torch.int16, device=DEV)
    ga.attn_qkv_prep(q_out, kd, vd, up(qkv), up(qw), up(kw), torch.from_numpy(f).to(DEV), eps,
                     v_norm, up(np.asarray(pos, np.int32)), S, Hq, Hkv, D, kd.shape[2], ring)
    return q_out


def _slot(t, cap, ring):
    return t % cap if ring else t


@pytest.mark.parametrize("D,Hq,Hkv,cap,ring,v_norm,theta,pos", [
    (256, 32, 4, 1536, 1, 1, 1e4, [4095, 1535, 70001, 0]),
    (512, 32, 2, 32768, 0, 0, 1e6, [32767, 5, 20000]),
    (512, 16, 1, 300, 1, 1, 1e6, [262143, 299]),
    (256, 24, 3, 512, 0, 1, 1e4, [511, 100]),
])
def test_prep_within_oracle_ranges(ga, D, Hq, Hkv, cap, ring, v_norm, theta, pos):
    say("prep", D, Hq, Hkv, cap, ring, v_norm, pos)
    S = len(pos)
    qkv, qw, kw, k, v = _inputs(D + cap, S, Hq, Hkv, D, cap)
    f = _freqs(D, theta)
    kd, vd = up(k), up(v)
    q_out = down(_prep(ga, qkv, qw, kw, f, 1e-6, v_norm, pos, Hq, Hkv, D, kd, vd, ring))
    kc, vc = down(kd), down(vd)
    ref = prep_ref.qkv_prep(qkv, qw, kw, f, 1e-6, v_norm, pos, Hq, Hkv, D)
    slots = [_slot(t, cap, ring) for t in pos]
    gk = np.stack([kc[s, :, slots[s]] for s in range(S)])
    gv = np.stack([vc[s, :, slots[s]] for s in range(S)])
    for name, got in (("q", q_out), ("k", gk), ("v", gv)):
        res = prep_ref.check_range(got, ref[name + "_bits"], ref[name + "_lo"], ref[name + "_hi"])
        say(name, res)
        assert res["ok"], (name, res)
        assert res["bit_equal"] >= 0.97, (name, res)
    # every other slot untouched
    mask = np.ones(kc.shape[:3], bool)
    for s in range(S):
        mask[s, :, slots[s]] = False
    assert np.array_equal(kc[mask], k[mask]) and np.array_equal(vc[mask], v[mask])


@pytest.mark.parametrize("D,Hq,Hkv,cap,ring,window,v_norm,pos", [
    (256, 32, 4, 1024, 1, 1024, 1, [4095 + 1000 * s for s in range(8)]),   # sliding ring
    (256, 8, 1, 512, 0, 512, 0, [511]),                                    # two runs
    (512, 32, 2, 256, 0, 0, 1, [255, 100, 7]),                             # one run, in place
    (512, 32, 2, 32768, 0, 0, 1, [32767, 12345]),                          # 16 runs: last-workgroup merge
    (512, 32, 2, 65536, 0, 0, 1, [65535, 40000]),                          # 32 runs: two launches
])
def test_prep_fused_equals_prep_then_decode(ga, D, Hq, Hkv, cap, ring, window, v_norm, pos):
    import torch
    say("prep fused", D, Hq, Hkv, cap, ring, window, v_norm, pos)
    S = len(pos)
    qkv, qw, kw, k, v = _inputs(7 * D + cap, S, Hq, Hkv, D, cap)
    f = _freqs(D, 1e4 if D == 256 else 1e6)
    n = ga.ATTN_DECODE_COUNTER_BYTES + ga.attn_decode_rows_workspace_bytes(S, 1, Hq, D, cap)
    ws = torch.zeros(n, dtype=torch.uint8, device=DEV)
    ga.attn_decode_workspace_init(ws)
    pd = up(np.asarray(pos, np.int32))
    fd = torch.from_numpy(f).to(DEV)
    # two calls: prologue, then the one-row decode
    k1, v1 = up(k), up(v)
    q_out = _prep(ga, qkv, qw, kw, f, 1e-6, v_norm, pos, Hq, Hkv, D, k1, v1, ring)
    o1 = torch.empty((S, 1, Hq, D), dtype=torch.int16, device=DEV)
    ga.attn_decode_rows_fused(o1, q_out.view(S, 1, Hq, D), k1, v1, pd, S, 1, Hq, Hkv, D, cap,
                              ring, window, 0.05, ws)
    # one call
    k2, v2 = up(k), up(v)
    o2 = torch.empty((S, Hq, D), dtype=torch.int16, device=DEV)
    ga.attn_decode_prep_fused(o2, up(qkv), up(qw), up(kw), fd, 1e-6, v_norm, k2, v2, pd, S, Hq,
                              Hkv, D, cap, ring, window, 0.05, ws)
    a, b = down(o1)[:, 0], down(o2)
    assert np.array_equal(a, b)
    assert np.array_equal(down(k1), down(k2)) and np.array_equal(down(v1), down(v2))
    # the attention itself against the oracle, on the prologue's outputs
    ref = attn_ref.decode(down(q_out), down(k2), down(v2), pos, Hkv, ring, window, 0.05)
    res = attn_ref.check(b, ref["o"], ref["r"])
    say("vs oracle", {x: res[x] for x in ("n", "fails", "mean_rel_err", "bit_equal")})
    assert res["ok"] and res["bit_equal"] >= 0.9, res
    assert int(ws[:ga.ATTN_DECODE_COUNTER_BYTES].count_nonzero()) == 0


@pytest.mark.parametrize("D,Hq,Hkv,cap,ring,window,pos", [
    (256, 8, 1, 512, 0, 0, [300]),                  # linear, unwritten slots after t
    (256, 8, 1, 512, 0, 0, [256]),                  # t alone in its run
    (256, 8, 1, 512, 0, 1, [200]),                  # window of one: t alone
    (256, 32, 4, 1024, 1, 1024, [500, 7, 1023]),    # ring not yet filled
    (512, 32, 2, 32768, 0, 0, [12345, 4096]),       # 16 runs, last-workgroup merge
    (512, 16, 1, 1024, 1, 512, [700]),              # ring, window inside the filled part
])
def test_prep_fused_never_reads_the_slot_it_writes(ga, D, Hq, Hkv, cap, ring, window, pos):
    """The row's own slot and every slot no position has reached hold NaN
    before the call (e.g. fresh torch.empty memory).  The fused call writes
    the row's slot and must give the finite outputs of prologue + decode,
    whose decode reads the slot after the prologue wrote it."""
    import torch
    say("prep fused, poisoned own slot", D, Hq, Hkv, cap, ring, window, pos)
    S = len(pos)
    qkv, qw, kw, k, v = _inputs(11 * D + cap + pos[0], S, Hq, Hkv, D, cap)
    for s, t in enumerate(pos):
        written = np.arange(cap) < t if not ring else np.arange(cap) < min(t, cap)
        if ring and t >= cap:
            written[:] = True
        k[s, :, ~written] = 0x7FC0
        v[s, :, ~written] = 0x7FC0
        k[s, :, _slot(t, cap, ring)] = 0x7FC0
        v[s, :, _slot(t, cap, ring)] = 0x7FC0
    f = _freqs(D, 1e4 if D == 256 else 1e6)
    n = ga.ATTN_DECODE_COUNTER_BYTES + ga.attn_decode_rows_workspace_bytes(S, 1, Hq, D, cap)
    ws = torch.zeros(n, dtype=torch.uint8, device=DEV)
    ga.attn_decode_workspace_init(ws)
    pd = up(np.asarray(pos, np.int32))
    k1, v1 = up(k), up(v)
    q_out = _prep(ga, qkv, qw, kw, f, 1e-6, 1, pos, Hq, Hkv, D, k1, v1, ring)
    o1 = torch.empty((S, 1, Hq, D), dtype=torch.int16, device=DEV)
    ga.attn_decode_rows_fused(o1, q_out.view(S, 1, Hq, D), k1, v1, pd, S, 1, Hq, Hkv, D, cap,
                              ring, window, 0.05, ws)
    k2, v2 = up(k), up(v)
    o2 = torch.empty((S, Hq, D), dtype=torch.int16, device=DEV)
    ga.attn_decode_prep_fused(o2, up(qkv), up(qw), up(kw), torch.from_numpy(f).to(DEV), 1e-6,
                              1, k2, v2, pd, S, Hq, Hkv, D, cap, ring, window, 0.05, ws)
    a, b = down(o1)[:, 0], down(o2)
    assert not np.any((a & 0x7FFF) > 0x7F80), "prologue + decode gave NaN"
    assert np.array_equal(a, b)
    assert np.array_equal(down(k1), down(k2)) and np.array_equal(down(v1), down(v2))


def test_prep_fused_graph_replay(ga):
    """A captured prologue + decode, replayed for new rows and positions: each
    replay writes the row's key/value and equals the eager call."""
    import torch
    say("prep fused graph replay")
    S, Hq, Hkv, D, cap, W = 4, 32, 4, 256, 1024, 1024
    rng = np.random.default_rng(50)
    _, qw, kw, k, v = _inputs(50, S, Hq, Hkv, D, cap)
    f = torch.from_numpy(_freqs(D, 1e4)).to(DEV)
    qwd, kwd = up(qw), up(kw)
    n = ga.ATTN_DECODE_COUNTER_BYTES + ga.attn_decode_rows_workspace_bytes(S, 1, Hq, D, cap)
    ws = torch.zeros(n, dtype=torch.uint8, device=DEV)
    ga.attn_decode_workspace_init(ws)
    kg, vg = up(k), up(v)
    qkv_d = torch.zeros((S, (Hq + 2 * Hkv) * D), dtype=torch.int16, device=DEV)
    pd = torch.zeros(S, dtype=torch.int32, device=DEV)
    out = torch.empty((S, Hq, D), dtype=torch.int16, device=DEV)

    def call(kc, vc, o, stream=None):
        ga.attn_decode_prep_fused(o, qkv_d, qwd, kwd, f, 1e-6, 1, kc, vc, pd, S, Hq, Hkv, D,
                                  cap, 1, W, 0.0625, ws, stream=stream)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call(kg, vg, out)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(kg, vg, out)
    torch.cuda.synchronize()
    ke, ve = kg.clone(), vg.clone()                 # eager twin of the caches
    oe = torch.empty_like(out)
    for step in range(4):
        qkv = randn_bf16_bits(rng, (S, (Hq + 2 * Hkv) * D))
        pos = rng.integers(2000, 90000, S).astype(np.int32)
        qkv_d.copy_(up(qkv))
        pd.copy_(up(pos))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        call(ke, ve, oe)                            # eager, between replays
        torch.cuda.synchronize()
        assert np.array_equal(down(out), down(oe)), step
        assert torch.equal(kg, ke) and torch.equal(vg, ve), step
