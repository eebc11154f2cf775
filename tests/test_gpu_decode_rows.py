"""GPU parity of attn_decode_rows (decode windows of up to 16 rows a
stream) against the CPU oracle's decode_rows, element by element with the
radius check; masks and indexing bit for bit with dominating keys and NaN
poison; and the pages' property that a row keeps its bits at any window
width (PR #975 decode attention commits)."""
import numpy as np
import pytest

from gpu_util import run_decode_rows, say
from oracle import attn_ref
from synthetic.gen import WORKLOADS, decode_rows_inputs, f32_to_bf16_bits, randn_bf16_bits

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


def test_decode_rows_sliding_1536_full(ga):
    w = WORKLOADS["decode_rows_sliding_1536"]
    say("decode rows workload", w.name)
    q, k, v, pos = decode_rows_inputs(w)
    got = run_decode_rows(ga, q, k, v, pos, w.Hkv, w.ring, w.window, w.scale)
    ref = attn_ref.decode_rows(q, k, v, pos, w.Hkv, w.ring, w.window, w.scale)
    _check(w.name, got, ref)


def test_decode_rows_global_32k_sampled_streams(ga):
    """Full size (8 streams x 16 rows over 32768 keys, the launch the bench
    times); the oracle takes every row and head of streams 0 and 5."""
    w = WORKLOADS["decode_rows_global_32k"]
    say("decode rows workload", w.name)
    q, k, v, pos = decode_rows_inputs(w)
    got = run_decode_rows(ga, q, k, v, pos, w.Hkv, w.ring, w.window, w.scale)
    sel = [0, 5]
    ref = attn_ref.decode_rows(q[sel], k[sel], v[sel], pos[sel], w.Hkv, w.ring, w.window,
                               w.scale)
    _check(w.name + " streams 0, 5", got[sel], ref)


@pytest.mark.parametrize("D,Hq,Hkv,cap,ring,window,R,pos", [
    (256, 32, 4, 1000, 0, 0, 5, [995, 0, 250, 300, -3]),       # ragged; rows before 0
    (256, 16, 2, 1100, 1, 1024, 7, [5000, 1023, 70000, 3]),     # ring wraps
    (512, 32, 2, 3000, 0, 700, 16, [2984, 690, 10, 2048]),      # G = 16: four workgroups
    (512, 16, 1, 600, 1, 333, 3, [1000, 33, 5]),
    (256, 12, 3, 300, 0, 0, 9, [291, 128, 0]),                  # G = 4: three tiles
    (512, 2, 2, 256, 0, 0, 16, [240, 100]),                     # G = 1: one tile of 16 rows
    (256, 6, 2, 200, 1, 50, 13, [400, 62]),                     # G = 3, ring of W + R - 1
    (256, 8, 1, 512, 0, 512, 1, [511]),                         # one row
    (512, 32, 2, 24576, 0, 5000, 6, [24570, 1530, 9000]),      # runs of six chunks, window
])
def test_decode_rows_shapes(ga, D, Hq, Hkv, cap, ring, window, R, pos):
    say("decode rows shape", D, Hq, Hkv, cap, ring, window, R, pos)
    rng = np.random.default_rng(cap + D + Hq + R)
    S = len(pos)
    q = randn_bf16_bits(rng, (S, R, Hq, D))
    k = randn_bf16_bits(rng, (S, Hkv, cap, D))
    v = randn_bf16_bits(rng, (S, Hkv, cap, D))
    got = run_decode_rows(ga, q, k, v, pos, Hkv, ring, window, 0.07)
    ref = attn_ref.decode_rows(q, k, v, pos, Hkv, ring, window, 0.07)
    _check(f"rows D={D} G={Hq // Hkv} R={R} ring={ring} W={window}", got, ref)


@pytest.mark.parametrize("D,Hq,Hkv,cap,ring,window,S", [
    (512, 32, 2, 4096, 0, 0, 2), (256, 32, 4, 1536, 1, 1024, 2),
    # sixteen streams: enough (stream, KV head, run) items that the full
    # head-dim-256 window takes the eight-wave two-role form while its single
    # rows take the four-wave one
    (256, 32, 4, 1536, 1, 1024, 16)])
def test_decode_rows_bits_independent_of_width(ga, D, Hq, Hkv, cap, ring, window, S):
    say("decode rows width invariance", D, S)
    rng = np.random.default_rng(17 + D if S == 2 else 17 + D + S)
    R = 16
    if S == 2:
        p = np.array([3000, 1500], dtype=np.int32) if ring else np.array([4080, 900], np.int32)
    else:
        p = np.array([5000 + 37 * s for s in range(S)], dtype=np.int32)
    q = randn_bf16_bits(rng, (S, R, Hq, D))
    k = randn_bf16_bits(rng, (S, Hkv, cap, D))
    v = randn_bf16_bits(rng, (S, Hkv, cap, D))
    full = run_decode_rows(ga, q, k, v, p, Hkv, ring, window, 0.05)
    for r in (0, 7, 15):
        one = run_decode_rows(ga, q[:, r:r + 1], k, v, p + r, Hkv, ring, window, 0.05)
        assert np.array_equal(one[:, 0], full[:, r]), r
    five = run_decode_rows(ga, q[:, 3:8], k, v, p + 3, Hkv, ring, window, 0.05)
    assert np.array_equal(five, full[:, 3:8])


def test_decode_rows_nan_in_unwritten_slots(ga):
    say("decode rows NaN poison")
    rng = np.random.default_rng(23)
    S, R, Hq, Hkv, D, cap = 2, 16, 32, 2, 512, 700
    pos = np.array([600, 250], dtype=np.int32)
    q = randn_bf16_bits(rng, (S, R, Hq, D))
    k = randn_bf16_bits(rng, (S, Hkv, cap, D))
    v = randn_bf16_bits(rng, (S, Hkv, cap, D))
    for s in range(S):                       # slots past the window's last row
        k[s, :, pos[s] + R:] = 0x7FC0
        v[s, :, pos[s] + R:] = 0x7FC0
    got = run_decode_rows(ga, q, k, v, pos, Hkv, 0, 0, 0.05)
    assert not np.any(((got & 0x7F80) == 0x7F80) & ((got & 0x7F) != 0))
    ref = attn_ref.decode_rows(q, k, v, pos, Hkv, 0, 0, 0.05)
    _check("rows nan poison", got, ref)


def test_decode_rows_dominating_key_window_edge(ga):
    """The first row's oldest key dominates: that row returns its V exactly;
    the later rows, whose windows have moved past it, never see it."""
    say("decode rows dominating key")
    rng = np.random.default_rng(29)
    S, R, Hq, Hkv, D, cap, W = 1, 8, 8, 1, 256, 300, 200
    t0 = 1000
    q = randn_bf16_bits(rng, (S, R, Hq, D))
    q[:] = q[:, :1, :1]                      # one query everywhere
    k = f32_to_bf16_bits((rng.standard_normal((S, Hkv, cap, D)) * 0.02).astype(np.float32))
    v = randn_bf16_bits(rng, (S, Hkv, cap, D))
    qf = (q[0, 0, 0].astype(np.uint32) << 16).view(np.float32)
    edge = (t0 - W + 1) % cap
    k[0, 0, edge] = f32_to_bf16_bits(8 * qf)
    got = run_decode_rows(ga, q, k, v, [t0], Hkv, 1, W, 1.0)
    assert np.all(got[0, 0] == v[0, 0, edge][None, :])
    for r in range(1, R):
        assert not np.all(got[0, r] == v[0, 0, edge][None, :]), r
    ref = attn_ref.decode_rows(q, k, v, [t0], Hkv, 1, W, 1.0)
    _check("rows dominating", got, ref)


def test_decode_rows_bits_independent_of_stream_count(ga):
    """A stream's rows have the same bits alone and inside a batch (PR #975:
    4- and 8-stream replies equal the plain ones), and attn_decode is the
    one-row window."""
    from gpu_util import run_decode
    say("decode rows stream-count invariance")
    rng = np.random.default_rng(31)
    S, R, Hq, Hkv, D, cap = 4, 4, 32, 2, 512, 32768
    pos = np.array([32764, 20000, 9000, 31000], dtype=np.int32)
    q = randn_bf16_bits(rng, (S, R, Hq, D))
    k = randn_bf16_bits(rng, (S, Hkv, cap, D))
    v = randn_bf16_bits(rng, (S, Hkv, cap, D))
    full = run_decode_rows(ga, q, k, v, pos, Hkv, 0, 0, 0.044)
    alone = run_decode_rows(ga, q[2:3], k[2:3], v[2:3], pos[2:3], Hkv, 0, 0, 0.044)
    assert np.array_equal(alone, full[2:3])
    one = run_decode(ga, q[:, 1], k, v, pos + 1, Hkv, 0, 0, 0.044)
    assert np.array_equal(one, full[:, 1])
