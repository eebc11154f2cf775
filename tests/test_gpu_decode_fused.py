"""GPU checks of attn_decode_rows_fused (one launch: a single run writes the
output itself, up to 16 runs merge in the last workgroup; PR #975 decode
commits) and of its replay from a captured HIP graph with positions read on
the device (PR #1183 engine note).  Its outputs must equal attn_decode_rows
bit for bit, which the oracle parity tests already tie to the oracle; the
counter area must be left at zero."""
import numpy as np
import pytest

from gpu_util import DEV, down, run_decode_rows, say, up
from oracle import attn_ref
from synthetic.gen import randn_bf16_bits

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ga():
    import global_gqa_attention_window_amd as ga
    return ga


def _fused(ga, q, kd, vd, pos, Hkv, ring, window, scale, ws, stream=None):
    import torch
    S, R, Hq, D = q.shape
    cap = kd.shape[2]
    out = torch.empty((S, R, Hq, D), dtype=torch.int16, device=DEV)
    ga.attn_decode_rows_fused(out, q, kd, vd, pos, S, R, Hq, Hkv, D, cap, ring, window, scale,
                              ws, stream=stream)
    return out


def _workspace(ga, S, R, Hq, D, cap):
    import torch
    n = ga.ATTN_DECODE_COUNTER_BYTES + ga.attn_decode_rows_workspace_bytes(S, R, Hq, D, cap)
    ws = torch.empty(n, dtype=torch.uint8, device=DEV)
    ws.fill_(0xA5)                               # not zero: init must clear the counters
    ga.attn_decode_workspace_init(ws)
    return ws


@pytest.mark.parametrize("D,Hq,Hkv,cap,ring,window,R,pos", [
    (256, 8, 1, 512, 0, 512, 1, [511]),                       # two runs (512 keys)
    (256, 32, 4, 1024, 1, 1024, 1, [4095 + 1000 * s for s in range(8)]),  # four runs
    (256, 32, 4, 1536, 1, 1024, 16, [4080, 5080, 6080]),      # six runs, 16-row windows
    (512, 32, 2, 256, 0, 0, 1, [255, 100, 0, -1]),            # one run: written in place
    (512, 16, 1, 4096, 0, 700, 5, [4091, 2000]),              # sixteen runs
    (512, 32, 2, 32768, 0, 0, 16, [32752, 20000]),            # sixteen runs of eight chunks
    (512, 32, 2, 65536, 0, 0, 3, [65535, 30000]),             # 32 runs: partials + merge
    (256, 12, 3, 300, 0, 0, 9, [291, 128, 0]),                # G = 4, ragged chunk
])
def test_fused_equals_two_launch_path(ga, D, Hq, Hkv, cap, ring, window, R, pos):
    import torch
    say("fused decode", D, Hq, Hkv, cap, ring, window, R, pos)
    rng = np.random.default_rng(cap + R + D)
    S = len(pos)
    q = randn_bf16_bits(rng, (S, R, Hq, D))
    k = randn_bf16_bits(rng, (S, Hkv, cap, D))
    v = randn_bf16_bits(rng, (S, Hkv, cap, D))
    kd, vd = up(k), up(v)
    want = run_decode_rows(ga, q, kd, vd, pos, Hkv, ring, window, 0.06)
    ws = _workspace(ga, S, R, Hq, D, cap)
    pd = up(np.asarray(pos, np.int32))
    for _ in range(3):                           # the counters reset themselves
        got = down(_fused(ga, up(q), kd, vd, pd, Hkv, ring, window, 0.06, ws))
        assert np.array_equal(got, want)
    torch.cuda.synchronize()
    assert int(ws[:ga.ATTN_DECODE_COUNTER_BYTES].count_nonzero()) == 0


def test_fused_graph_replay_with_device_positions(ga):
    """One capture per row count, replayed for new positions and queries:
    every replay equals the eager two-launch result for its inputs."""
    import torch
    say("fused decode graph replay")
    rng = np.random.default_rng(41)
    S, R, Hq, Hkv, D, cap, W = 4, 2, 32, 4, 256, 1536, 1024
    k = randn_bf16_bits(rng, (S, Hkv, cap, D))
    v = randn_bf16_bits(rng, (S, Hkv, cap, D))
    kd, vd = up(k), up(v)
    qd = torch.zeros((S, R, Hq, D), dtype=torch.int16, device=DEV)
    pd = torch.zeros(S, dtype=torch.int32, device=DEV)
    ws = _workspace(ga, S, R, Hq, D, cap)
    out = torch.empty((S, R, Hq, D), dtype=torch.int16, device=DEV)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):                # warm-up call outside the capture
        ga.attn_decode_rows_fused(out, qd, kd, vd, pd, S, R, Hq, Hkv, D, cap, 1, W, 0.0625, ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        ga.attn_decode_rows_fused(out, qd, kd, vd, pd, S, R, Hq, Hkv, D, cap, 1, W, 0.0625, ws)
    torch.cuda.synchronize()
    for step in range(4):
        q = randn_bf16_bits(rng, (S, R, Hq, D))
        pos = rng.integers(2000, 90000, S).astype(np.int32)
        qd.copy_(up(q))
        pd.copy_(up(pos))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = down(out)
        want = run_decode_rows(ga, q, kd, vd, pos, Hkv, 1, W, 0.0625)   # eager, between replays
        assert np.array_equal(got, want), step
        if step == 0:
            ref = attn_ref.decode_rows(q, k, v, pos, Hkv, 1, W, 0.0625)
            res = attn_ref.check(got, ref["o"], ref["r"])
            say("replay 0 vs oracle", {x: res[x] for x in ("n", "fails", "mean_rel_err")})
            assert res["ok"], res
    assert int(ws[:ga.ATTN_DECODE_COUNTER_BYTES].count_nonzero()) == 0
