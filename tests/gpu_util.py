"""Helpers for the GPU tests: move bf16 bit arrays to and from the device and
call the library through its Python binding (which calls the C ABI)."""
from __future__ import annotations

import sys

import numpy as np
import torch

DEV = torch.device("cuda:0")


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def up(a: np.ndarray) -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to(DEV)


def down(t: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    return t.cpu().numpy().view(np.uint16)


def run_decode(ga, q, k, v, pos, Hkv, ring, window, scale, ws_pad=0):
    S, Hq, D = q.shape
    cap = k.shape[2]
    out = torch.empty((S, Hq, D), dtype=torch.int16, device=DEV)
    nbytes = ga.attn_decode_workspace_bytes(S, Hq, D, cap)
    ws = torch.empty(nbytes + ws_pad, dtype=torch.uint8, device=DEV)
    ga.attn_decode(out, up(q), up(k), up(v), up(np.asarray(pos, np.int32)), S, Hq, Hkv,
                   D, cap, ring, window, scale, ws)
    return down(out)


def run_decode_rows(ga, q, k, v, pos, Hkv, ring, window, scale):
    """q [S][R][Hq][D] bf16 bits; returns out [S][R][Hq][D] bits."""
    S, R, Hq, D = q.shape
    cap = k.shape[2]
    out = torch.empty((S, R, Hq, D), dtype=torch.int16, device=DEV)
    nbytes = ga.attn_decode_rows_workspace_bytes(S, R, Hq, D, cap)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
    kd = k if isinstance(k, torch.Tensor) else up(k)
    vd = v if isinstance(v, torch.Tensor) else up(v)
    ga.attn_decode_rows(out, up(q), kd, vd, up(np.asarray(pos, np.int32)), S, R, Hq, Hkv, D,
                        cap, ring, window, scale, ws)
    return down(out)


def run_prefill(ga, q, k, v, Hkv, cap, ring, window, scale, p_mode, chunk,
                pos0=0, caches=None, last_key=None, starts=None, split=False):
    """Prompt rows pos0.. in chunks: cache write, then attention, per chunk.
    Chunks of `chunk` rows, or starting at `starts` (row indices) when given.
    last_key [n] (absolute positions, optional) is passed per chunk as given.
    split: attention through attn_prefill_ws with a workspace."""
    n, Hq, D = q.shape
    if caches is None:
        kc = torch.zeros((Hkv, cap, D), dtype=torch.int16, device=DEV)
        vc = torch.zeros_like(kc)
    else:
        kc, vc = caches
    qd, kd, vd = up(q), up(k[pos0:pos0 + n]), up(v[pos0:pos0 + n])
    out = torch.empty((n, Hq, D), dtype=torch.int16, device=DEV)
    lkd = None if last_key is None else up(np.asarray(last_key, dtype=np.int32))
    starts = list(range(0, n, chunk)) if starts is None else list(starts)
    ws = None
    if split:
        longest = max(b - a for a, b in zip(starts, starts[1:] + [n]))
        ws = torch.empty(ga.attn_prefill_workspace_bytes(longest, Hq, D), dtype=torch.uint8,
                         device=DEV)
    for r0, r1 in zip(starts, starts[1:] + [n]):
        m = r1 - r0
        ga.attn_cache_write(kc, vc, kd[r0:r0 + m], vd[r0:r0 + m], pos0 + r0, m, Hkv, D,
                            cap, ring)
        lk = None if lkd is None else lkd[r0:r0 + m]
        if split:
            ga.attn_prefill_ws(out[r0:r0 + m], qd[r0:r0 + m], kc, vc, pos0 + r0, m, Hq, Hkv,
                               D, cap, ring, window, scale, p_mode, ws, last_key=lk)
        else:
            ga.attn_prefill(out[r0:r0 + m], qd[r0:r0 + m], kc, vc, pos0 + r0, m, Hq, Hkv, D,
                            cap, ring, window, scale, p_mode, last_key=lk)
    return down(out), (kc, vc)
