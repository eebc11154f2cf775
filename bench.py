"""Benchmark of the attention hot path on one MI355X.

One step = the whole path over one synthetic prompt of the global-layer
workload: a 32768-token causal prompt (32 query heads over 2 KV heads, head
dim 512, P kept as two bf16 halves) fed in 64 chunks of 512 rows, each chunk
a cache write then prompt attention; then one decode row over a 262144-key
linear cache with the same heads.  Inputs are resident in HBM before timing.

Prints one JSON line: whole-step tokens/s (prompt tokens + the decode token),
the prefill kernel against the bf16 matrix-core roofline (duration from HIP
events recorded on the launch stream around every prefill launch), the decode
kernels against HBM bandwidth (the call inside the step, right after the
prompt's matrix-heavy launches, and the same call 20 times back to back), and
the CPU oracle timed on a bounded sample.
Apart from the step: the 8192-token sliding-layer prompt (128-row chunks
through a 1152-slot ring, window 1024, head dim 256, P rounded to bf16) in
prompt tokens/s against the bf16 matrix-core peak, through attn_prefill_ws
(each tile's key blocks split over four workgroups, then merged) and, for
reference, attn_prefill; the one-row decode
workloads of 512 keys, of 8 streams over a 1024-slot sliding ring and of 8
streams over 32768 global-layer keys against HBM bandwidth (the two small
ones also cold, rotating over K/V sets larger than the last-level cache);
decode windows (16 rows a stream, 8 streams, 32768 keys) against the bf16
matrix-core peak; the attainable rates on the part beside the published
peaks (library kernels: a device copy and a bf16 matrix product; kernels of
our own: a read-only HBM stream and a loop of bf16 matrix products); the
shader clock measured right after the timed steps (cycle counter against the
100 MHz real-time counter); and the oracle on the other workloads (decodes in
GB/s of attended K/V, the 8k prompt in tokens/s) with the host's CPU count
and model.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "decode attn HBM GB/s & prefill tokens/s (8k/32k) vs MI355X roofline"
PEAK_BF16_TFLOPS = 2516.6      # MI355X dense bf16 matrix peak
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=128,
                    help="prompt rows of the oracle's timed sample")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run 4 plain device copies of MIB MiB each (the known-size "
                         "kernel that scales the FETCH_SIZE / WRITE_SIZE counters) and exit")
    return ap.parse_args()


def copy_calibration(mib: int):
    import torch
    n = mib * 1024 * 1024 // 2
    src = torch.ones(n, dtype=torch.int16, device="cuda:0")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(4):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read": n * 2, "bytes_written": n * 2,
                      "launches": 4}), flush=True)


def causal_pairs(n_rows: int, window: int) -> int:
    """Attended (row, key) pairs of a prompt of n_rows at positions 0.."""
    if window <= 0:
        return n_rows * (n_rows + 1) // 2
    w = min(window, n_rows)
    return w * (w + 1) // 2 + (n_rows - w) * window


def traffic_from_profile(kernel_src: str):
    """HBM bytes per launch from a committed --pmc summary, if it was taken
    on the current kernel source (else None)."""
    path = os.path.join(ROOT, "profiles", "prefill_global_32k_pmc.md")
    if not os.path.exists(path):
        return None
    txt = open(path).read()
    m_sha = re.search(r"source_sha256:\s*([0-9a-f]{64})", txt)
    m_b = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", txt)
    if not (m_sha and m_b):
        return None
    sha = hashlib.sha256(open(kernel_src, "rb").read()).hexdigest()
    return float(m_b.group(1)) if sha == m_sha.group(1) else None


def decode_windows(ga, torch, dev, iters: int = 10):
    """Decode windows of 16 rows a stream, 8 streams (128 rows), over a
    32768-key global-layer cache, timed apart from the step (HIP events on
    the launch stream): algorithmic flops 4 D per (row, head, attended key),
    K/V bytes once per (stream, KV head)."""
    from synthetic.gen import WORKLOADS
    w = WORKLOADS["decode_rows_global_32k"]
    S, R = w.S, w.rows
    g = torch.Generator(device=dev).manual_seed(w.seed)
    q = torch.randn((S, R, w.Hq, w.D), generator=g, device=dev, dtype=torch.bfloat16)
    kc = torch.randn((S, w.Hkv, w.cap, w.D), generator=g, device=dev, dtype=torch.bfloat16)
    vc = torch.randn((S, w.Hkv, w.cap, w.D), generator=g, device=dev, dtype=torch.bfloat16)
    pos = torch.tensor(w.pos, dtype=torch.int32, device=dev)
    out = torch.empty_like(q)
    ws = torch.empty(ga.attn_decode_rows_workspace_bytes(S, R, w.Hq, w.D, w.cap),
                     dtype=torch.uint8, device=dev)

    def call():
        ga.attn_decode_rows(out, q, kc, vc, pos, S, R, w.Hq, w.Hkv, w.D, w.cap, w.ring,
                            w.window, w.scale, ws)
    for _ in range(3):
        call()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(iters):
        call()
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / iters
    pairs = sum(int(p) + r + 1 for p in w.pos for r in range(R))     # (row, key) attended
    flops = 4 * w.D * w.Hq * pairs
    kv_bytes = 2 * S * w.Hkv * w.cap * w.D * 2
    tf = flops / (us * 1e-6) / 1e12
    return {"workload": w.name, "streams": S, "rows_per_stream": R, "cache_keys": w.cap,
            "us": round(us, 1), "rows_per_s": round(S * R / (us * 1e-6), 1),
            "TFLOP/s": round(tf, 1), "frac_bf16_peak": round(tf / PEAK_BF16_TFLOPS, 4),
            "kv_GB/s": round(kv_bytes / (us * 1e-6) / 1e9, 1)}


def prefill_sliding(ga, torch, dev, reps: int = 3, split: bool = True):
    """The 8192-token sliding-layer prompt: 64 chunks of 128 rows, each a
    cache write into the 1152-slot ring then prompt attention over it
    (split: attn_prefill_ws, whose 64-workgroup chunks split each tile's key
    blocks over four workgroups and merge; else attn_prefill).  Prompt
    tokens/s over the summed attention durations (HIP events on the launch
    stream around each attention call, its merge launch included) and over
    the whole chunk sequence with its cache writes (a separate pass with no
    events between launches); with split, also the whole prompt through one
    attn_prefill_prompt call (the bits of the unsplit chunked path, cache
    writes included: the prompt's attended keys copied to a linear span, one
    attention launch over all rows, the last rows into the ring).  Algorithmic
    flops 4 D per attended (row, key, query head)."""
    from synthetic.gen import WORKLOADS
    w = WORKLOADS["prefill_sliding_8k"]
    n, ch, Hq, Hkv, D = w.n_rows, w.chunk, w.Hq, w.Hkv, w.D
    g = torch.Generator(device=dev).manual_seed(w.seed)
    q = torch.randn((n, Hq, D), generator=g, device=dev, dtype=torch.bfloat16)
    k = torch.randn((n, Hkv, D), generator=g, device=dev, dtype=torch.bfloat16)
    v = torch.randn((n, Hkv, D), generator=g, device=dev, dtype=torch.bfloat16)
    kc = torch.zeros((Hkv, w.cap, D), dtype=torch.bfloat16, device=dev)
    vc = torch.zeros_like(kc)
    out = torch.empty_like(q)
    ws = (torch.empty(ga.attn_prefill_workspace_bytes(ch, Hq, D), dtype=torch.uint8, device=dev)
          if split else None)
    starts = list(range(0, n, ch))
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in starts]
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def prompt(record: bool):
        for i, r0 in enumerate(starts):
            m = min(ch, n - r0)
            ga.attn_cache_write(kc, vc, k[r0:r0 + m], v[r0:r0 + m], r0, m, Hkv, D, w.cap, w.ring)
            if record:
                ev[i][0].record()
            ga.attn_prefill_ws(out[r0:r0 + m], q[r0:r0 + m], kc, vc, r0, m, Hq, Hkv, D, w.cap,
                               w.ring, w.window, w.scale, w.p_mode, ws)
            if record:
                ev[i][1].record()
    prompt(False)
    torch.cuda.synchronize()
    kern_ms, wall_ms = [], []
    for _ in range(reps):
        # launch durations (events around each prefill launch), then the whole
        # sequence in a pass of its own with no events between the launches
        prompt(True)
        torch.cuda.synchronize()
        kern_ms.append(sum(a.elapsed_time(b) for a, b in ev))
        e0.record()
        prompt(False)
        e1.record()
        torch.cuda.synchronize()
        wall_ms.append(e0.elapsed_time(e1))
    kms = sorted(kern_ms)[reps // 2]
    wms = sorted(wall_ms)[reps // 2]
    flops = causal_pairs(n, w.window) * Hq * 4 * D
    tf = flops / (kms * 1e-3) / 1e12
    whole = None
    if split:
        pws = torch.empty(ga.attn_prefill_prompt_workspace_bytes(0, n, Hkv, D, w.ring, w.window),
                          dtype=torch.uint8, device=dev)

        def prompt_call():
            ga.attn_prefill_prompt(out, q, k, v, kc, vc, 0, n, ch, Hq, Hkv, D, w.cap, w.ring,
                                   w.window, w.scale, w.p_mode, workspace=pws)
        pms = call_ms(torch, prompt_call, reps)
        ptf = flops / (pms * 1e-3) / 1e12
        whole = {"ms": round(pms, 3), "tokens_per_s": round(n / (pms * 1e-3), 1),
                 "TFLOP/s": round(ptf, 1), "frac_bf16_peak": round(ptf / PEAK_BF16_TFLOPS, 4)}
    res = {"workload": w.name, "entry_point": "attn_prefill_ws" if split else "attn_prefill",
            "prompt_tokens": n, "chunk_rows": ch, "ring_slots": w.cap,
            "window": w.window, "head_dim": D, "q_heads": Hq, "kv_heads": Hkv, "p_mode": "bf16",
            "kernel_ms": round(kms, 3), "tokens_per_s_kernels": round(n / (kms * 1e-3), 1),
            "wall_ms_with_cache_writes": round(wms, 3),
            "tokens_per_s_wall": round(n / (wms * 1e-3), 1),
            "TFLOP/s": round(tf, 1), "frac_bf16_peak": round(tf / PEAK_BF16_TFLOPS, 4),
            "launch_us": round(kms * 1e3 / len(starts), 2)}
    if whole is not None:
        res["attn_prefill_prompt_with_cache_writes"] = whole
    return res


def call_ms(torch, fn, reps: int) -> float:
    """Median ms of fn() (one warm-up call first), HIP events around each."""
    fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t = []
    for _ in range(reps):
        e0.record()
        fn()
        e1.record()
        torch.cuda.synchronize()
        t.append(e0.elapsed_time(e1))
    return sorted(t)[reps // 2]


def graph_us(torch, calls, n_calls: int, reps: int = 5):
    """Device time per call of `calls` (a function that enqueues n_calls
    library calls on the current stream), replayed from a captured HIP graph:
    the calls' launches run back to back with no host work between them (a
    decode step replayed as a graph, as a serving loop runs it).  Median of
    reps replays, events around each."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):                # warm-up outside the capture
        calls()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        calls()
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t = []
    for _ in range(reps):
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        t.append(e0.elapsed_time(e1) * 1e3 / n_calls)
    del g
    return sorted(t)[reps // 2]


def decode_configs(ga, torch, dev, iters: int = 20):
    """One-row decode workloads (512 keys; 8 streams over a 1024-slot sliding
    ring; 8 streams over 32768 global-layer keys): us per call from HIP
    events over back-to-back calls replayed from a captured graph (the
    eager calls' time, which the Python binding's per-call checks bound for
    the small ones, beside it), K/V bytes attended once per (stream, KV
    head) plus q and out.  The two smaller caches stay in the 256 MB
    last-level cache between calls (warm); the 32768-key one (1 GiB) does not."""
    from synthetic.gen import WORKLOADS
    res = {}
    for name in ("decode_g8_d256_512", "decode_sliding_ring1024", "decode_global_32k"):
        w = WORKLOADS[name]
        g = torch.Generator(device=dev).manual_seed(w.seed)
        q = torch.randn((w.S, w.Hq, w.D), generator=g, device=dev, dtype=torch.bfloat16)
        kc = torch.randn((w.S, w.Hkv, w.cap, w.D), generator=g, device=dev, dtype=torch.bfloat16)
        vc = torch.randn((w.S, w.Hkv, w.cap, w.D), generator=g, device=dev, dtype=torch.bfloat16)
        pos = torch.tensor(w.pos, dtype=torch.int32, device=dev)
        out = torch.empty_like(q)
        ws = torch.empty(ga.attn_decode_workspace_bytes(w.S, w.Hq, w.D, w.cap),
                         dtype=torch.uint8, device=dev)

        def call():
            ga.attn_decode(out, q, kc, vc, pos, w.S, w.Hq, w.Hkv, w.D, w.cap, w.ring, w.window,
                           w.scale, ws)
        for _ in range(3):
            call()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(iters):
            call()
        e1.record()
        torch.cuda.synchronize()
        us_eager = e0.elapsed_time(e1) * 1e3 / iters

        def calls():
            for _ in range(iters):
                call()
        us = graph_us(torch, calls, iters)
        keys = sum(min(w.cap, p + 1) if w.window <= 0 else min(w.cap, p + 1, w.window)
                   for p in w.pos)
        nbytes = 2 * w.Hkv * keys * w.D * 2 + 2 * w.S * w.Hq * w.D * 2
        gbs = nbytes / (us * 1e-6) / 1e9
        res[name] = {"us": round(us, 2), "GB/s": round(gbs, 1),
                     "frac_hbm": round(gbs / PEAK_HBM_GBS, 4), "bytes": nbytes,
                     "cache": "warm" if nbytes < (256 << 20) else "cold",
                     "timing": "graph replay", "us_eager": round(us_eager, 2)}
        del q, kc, vc, out, ws
    torch.cuda.empty_cache()
    return res


def decode_cold(ga, torch, dev, min_bytes: int = 600 << 20):
    """The two small one-row decode workloads with their K/V out of the
    last-level cache: calls rotate over distinct K/V sets totalling more than
    600 MB (over twice the 256 MB cache), so every call's K/V comes from
    HBM; us per call (HIP events over one pass of the rotation replayed from
    a captured graph; the eager pass beside it)."""
    from synthetic.gen import WORKLOADS
    res = {}
    for name in ("decode_g8_d256_512", "decode_sliding_ring1024"):
        w = WORKLOADS[name]
        per_set = 2 * w.S * w.Hkv * w.cap * w.D * 2
        n_sets = max(16, -(-min_bytes // per_set))
        g = torch.Generator(device=dev).manual_seed(w.seed)
        q = torch.randn((w.S, w.Hq, w.D), generator=g, device=dev, dtype=torch.bfloat16)
        kv = torch.randn((n_sets, 2, w.S, w.Hkv, w.cap, w.D), generator=g, device=dev,
                         dtype=torch.bfloat16)
        pos = torch.tensor(w.pos, dtype=torch.int32, device=dev)
        out = torch.empty_like(q)
        ws = torch.empty(ga.attn_decode_workspace_bytes(w.S, w.Hq, w.D, w.cap),
                         dtype=torch.uint8, device=dev)

        def call(i):
            ga.attn_decode(out, q, kv[i, 0], kv[i, 1], pos, w.S, w.Hq, w.Hkv, w.D, w.cap,
                           w.ring, w.window, w.scale, ws)
        for i in range(n_sets):
            call(i)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(n_sets):
            call(i)
        e1.record()
        torch.cuda.synchronize()
        us_eager = e0.elapsed_time(e1) * 1e3 / n_sets

        def calls():
            for i in range(n_sets):
                call(i)
        us = graph_us(torch, calls, n_sets, reps=3)
        keys = sum(min(w.cap, p + 1, w.window) for p in w.pos)
        nbytes = 2 * w.Hkv * keys * w.D * 2 + 2 * w.S * w.Hq * w.D * 2
        gbs = nbytes / (us * 1e-6) / 1e9
        res[name] = {"us": round(us, 2), "GB/s": round(gbs, 1),
                     "frac_hbm": round(gbs / PEAK_HBM_GBS, 4), "kv_sets": n_sets,
                     "rotated_MB": round(n_sets * per_set / 1e6, 1),
                     "timing": "graph replay", "us_eager": round(us_eager, 2)}
        del q, kv, out, ws
    torch.cuda.empty_cache()
    return res


def calib_lib():
    """The calibration kernels (libgqa_calib.so, built with the package), or
    None when they were not built."""
    import ctypes
    path = os.path.join(ROOT, "global_gqa_attention_window_amd", "libgqa_calib.so")
    if not os.path.exists(path):
        return None
    lib = ctypes.CDLL(path)
    lib.calib_read_stream.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                      ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    lib.calib_read_chunks.argtypes = lib.calib_read_stream.argtypes
    lib.calib_mfma_loop.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    lib.calib_clock.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    return lib


def gpu_clock_mhz(torch, dev):
    """The shader clock right now: each of 256 workgroups (one per CU) times
    a matrix-core loop of about a millisecond with the cycle counter and the
    100 MHz real-time counter; the median ratio in MHz.  Run right after a
    timed region, it tells the clock that region ran at (None without the
    calibration library)."""
    lib = calib_lib()
    if lib is None:
        return None
    out = torch.zeros(3 * 256, dtype=torch.int64, device=dev)
    stream = torch.cuda.current_stream().cuda_stream
    assert lib.calib_clock(20000, out.data_ptr(), 256, stream) == 0
    torch.cuda.synchronize()
    o = out.view(256, 3).cpu().tolist()
    r = sorted(c / t * 100.0 for c, t, _ in o if t > 0)
    return round(r[len(r) // 2], 1) if r else None


def attainable_kernels(torch, dev):
    """Measured ceilings of this part from kernels of our own: a read-only
    stream over 1 GiB (every byte read once with 16-byte loads over the whole
    chip, as a grid-stride walk or as contiguous per-workgroup shares with
    nontemporal loads; the best of a few grid sizes and loads in flight) and a loop of bf16
    16x16x32 matrix products from registers, two waves on every SIMD (16384
    flops each); the shader clock measured right after each."""
    lib = calib_lib()
    if lib is None:
        return {"error": "libgqa_calib.so not built"}
    stream = torch.cuda.current_stream().cuda_stream
    res = {}
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device=dev)
    src.fill_(1)
    sink = torch.empty(8192 * 256, dtype=torch.int32, device=dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    best, rates = None, {}
    for fn, grid, unroll in (("stride", 512, 8), ("stride", 2048, 8), ("stride", 4096, 4),
                             ("chunks_nt", 256, 16), ("chunks_nt", 512, 8),
                             ("chunks_nt", 1024, 8)):
        f = lib.calib_read_stream if fn == "stride" else lib.calib_read_chunks
        for _ in range(2):
            assert f(src.data_ptr(), n, sink.data_ptr(), grid, unroll, stream) == 0
        torch.cuda.synchronize()
        reps = 10
        e0.record()
        for _ in range(reps):
            f(src.data_ptr(), n, sink.data_ptr(), grid, unroll, stream)
        e1.record()
        torch.cuda.synchronize()
        gbs = n * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9
        rates[f"{fn} grid {grid} x{unroll}"] = round(gbs, 1)
        if best is None or gbs > best[0]:
            best = (gbs, fn, grid, unroll)
    gbs, fn, grid, unroll = best
    res["read_stream"] = {"GB/s": round(gbs, 1), "frac_hbm_peak": round(gbs / PEAK_HBM_GBS, 4),
                          "bytes": n, "pattern": fn, "grid": grid, "loads_in_flight": unroll,
                          "all_GB/s": rates, "clock_MHz_after": gpu_clock_mhz(torch, dev)}
    del src, sink
    grid, iters = 512, 40000
    sink = torch.empty(grid * 256, dtype=torch.float32, device=dev)
    assert lib.calib_mfma_loop(100, sink.data_ptr(), grid, stream) == 0
    torch.cuda.synchronize()
    e0.record()
    for _ in range(3):
        lib.calib_mfma_loop(iters, sink.data_ptr(), grid, stream)
    e1.record()
    torch.cuda.synchronize()
    flops = 3 * grid * 4 * iters * 8 * 16384
    tf = flops / (e0.elapsed_time(e1) * 1e-3) / 1e12
    res["mfma_loop_bf16"] = {"TFLOP/s": round(tf, 1), "frac_bf16_peak": round(tf / PEAK_BF16_TFLOPS, 4),
                             "clock_MHz_after": gpu_clock_mhz(torch, dev)}
    del sink
    torch.cuda.empty_cache()
    return res


def attainable(torch, dev):
    """Attainable rates on this part with library kernels, beside the
    published peaks: a 1 GiB device-to-device copy (bytes read + written per
    second) and an 8192 x 8192 x 8192 bf16 matrix product (torch.matmul,
    contiguous operands)."""
    n = 1 << 29
    a = torch.ones(n, dtype=torch.bfloat16, device=dev)
    b = torch.empty_like(a)
    for _ in range(2):
        b.copy_(a)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(10):
        b.copy_(a)
    e1.record()
    torch.cuda.synchronize()
    copy_gbs = 2 * n * 2 * 10 / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del a, b
    m = 8192
    x = torch.randn((m, m), device=dev, dtype=torch.bfloat16)
    y = torch.randn((m, m), device=dev, dtype=torch.bfloat16)
    for _ in range(2):
        z = torch.matmul(x, y)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(10):
        z = torch.matmul(x, y)
    e1.record()
    torch.cuda.synchronize()
    mm_tf = 2 * m ** 3 * 10 / (e0.elapsed_time(e1) * 1e-3) / 1e12
    del x, y, z
    torch.cuda.empty_cache()
    return {"copy_GB/s": round(copy_gbs, 1), "copy_frac_hbm_peak": round(copy_gbs / PEAK_HBM_GBS, 4),
            "bf16_gemm_TFLOP/s": round(mm_tf, 1),
            "bf16_gemm_frac_peak": round(mm_tf / PEAK_BF16_TFLOPS, 4)}


def host_cpu():
    """The host's logical CPUs (this process's affinity and os.cpu_count())
    and its CPU model (/proc/cpuinfo)."""
    model = None
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.startswith("model name"):
                model = ln.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"logical_cpus_affinity": len(os.sched_getaffinity(0)),
            "os_cpu_count": os.cpu_count(), "cpu_model": model}


def blas_threads():
    from threadpoolctl import threadpool_info
    return int(max([p.get("num_threads", 1) for p in threadpool_info()] + [1]))


def cpu_baseline(q, k, v, w, n_rows_sample: int):
    """The oracle as it stands, on prompt rows spread evenly over the prompt
    (per-row cost grows with position, so an even spread has the prompt's
    mean cost), every head; tokens/s = rows / seconds.  `cores` is the BLAS
    thread count the oracle's float64 products ran on (it has no other
    parallelism); the host's CPU count and model are beside it."""
    import numpy as np

    from oracle import attn_ref
    from oracle.contract import key_block

    n = w.n_rows
    rows = np.linspace(n // (2 * n_rows_sample), n - 1, n_rows_sample).astype(np.int64)
    t0 = time.perf_counter()
    attn_ref.prefill(q, k, v, 0, w.Hkv, w.window, w.scale, w.p_mode,
                     key_block(w.D, w.p_mode), rows=rows, row_batch=8)
    dt = time.perf_counter() - t0
    return {"value": round(n_rows_sample / dt, 3), "unit": "tokens/s", "cores": blas_threads(),
            "kind": "oracle", "host": host_cpu(),
            "sample": f"{n_rows_sample} prompt rows evenly spread over positions 0..{n - 1} "
                      f"of the 32768-token prompt, all 32 heads, float64 NumPy; "
                      f"{dt:.1f} s"}


def cpu_oracle_workloads(n_prompt_rows: int = 256):
    """The oracle as it stands on the other workloads, in the GPU's units:
    the one-row decodes in GB/s of attended K/V (+ q, out) — the two small
    ones whole, the 8-stream 32768-key decode on one stream of the eight, the
    262144-key decode on one KV head of the two (its 16 query heads) — and the
    8192-token sliding prompt on rows spread evenly over it, in tokens/s."""
    import numpy as np

    from oracle import attn_ref
    from oracle.contract import key_block
    from synthetic.gen import WORKLOADS, decode_inputs, prefill_inputs, randn_bf16_bits

    res = {"cores": blas_threads()}

    def dec(name, q, k, v, pos, Hkv, ring, window, scale, note):
        S, Hq, D = q.shape
        cap = k.shape[2]
        keys = sum(min(cap, int(p) + 1) if window <= 0 else min(cap, int(p) + 1, window)
                   for p in pos)
        nbytes = 2 * Hkv * keys * D * 2 + 2 * S * Hq * D * 2
        t0 = time.perf_counter()
        attn_ref.decode(q, k, v, pos, Hkv, ring, window, scale)
        dt = time.perf_counter() - t0
        res[name] = {"GB/s": round(nbytes / dt / 1e9, 4), "s": round(dt, 3), "bytes": nbytes,
                     "sample": note}

    for name in ("decode_g8_d256_512", "decode_sliding_ring1024"):
        w = WORKLOADS[name]
        q, k, v, pos = decode_inputs(w)
        dec(name, q, k, v, pos, w.Hkv, w.ring, w.window, w.scale, "whole workload")
    w = WORKLOADS["decode_global_32k"]
    q, k, v, pos = decode_inputs(w, S=1, pos=w.pos[:1])
    dec(w.name, q, k, v, pos, w.Hkv, w.ring, w.window, w.scale, "one stream of the eight")
    del q, k, v
    wp = WORKLOADS["prefill_global_32k"]
    cap = wp.extra["decode_cap"]
    rng = np.random.default_rng(wp.extra["decode_seed"])
    q = randn_bf16_bits(rng, (1, wp.Hq // wp.Hkv, wp.D))
    k = randn_bf16_bits(rng, (1, 1, cap, wp.D))
    v = randn_bf16_bits(rng, (1, 1, cap, wp.D))
    dec("decode_262144", q, k, v, [wp.extra["decode_pos"]], 1, 0, 0, wp.scale,
        "one KV head of the two (its 16 query heads)")
    del q, k, v
    w = WORKLOADS["prefill_sliding_8k"]
    q, k, v = prefill_inputs(w)
    n = w.n_rows
    rows = np.linspace(n // (2 * n_prompt_rows), n - 1, n_prompt_rows).astype(np.int64)
    t0 = time.perf_counter()
    attn_ref.prefill(q, k, v, 0, w.Hkv, w.window, w.scale, w.p_mode, key_block(w.D, w.p_mode),
                     rows=rows, row_batch=16)
    dt = time.perf_counter() - t0
    res[w.name] = {"tokens_per_s": round(n_prompt_rows / dt, 3), "s": round(dt, 3),
                   "sample": f"{n_prompt_rows} prompt rows evenly spread over the 8192, "
                             "all 32 heads"}
    return res


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the library has no multi-GPU path).", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return

    import numpy as np
    import torch

    import global_gqa_attention_window_amd as ga
    from synthetic.gen import WORKLOADS, prefill_inputs, randn_bf16_bits

    w = WORKLOADS["prefill_global_32k"]
    dev = torch.device("cuda:0")
    n, ch, Hq, Hkv, D = w.n_rows, w.chunk, w.Hq, w.Hkv, w.D
    dcap, dpos = w.extra["decode_cap"], w.extra["decode_pos"]

    def up(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev)

    q_np, k_np, v_np = prefill_inputs(w)
    q, k, v = up(q_np), up(k_np), up(v_np)
    rng = np.random.default_rng(w.extra["decode_seed"])
    dq = up(randn_bf16_bits(rng, (1, Hq, D)))
    dk = up(randn_bf16_bits(rng, (1, Hkv, dcap, D)))
    dv = up(randn_bf16_bits(rng, (1, Hkv, dcap, D)))
    dpos_t = torch.tensor([dpos], dtype=torch.int32, device=dev)
    dout = torch.empty((1, Hq, D), dtype=torch.int16, device=dev)
    ws = torch.empty(ga.attn_decode_workspace_bytes(1, Hq, D, dcap), dtype=torch.uint8,
                     device=dev)
    kc = torch.zeros((Hkv, w.cap, D), dtype=torch.int16, device=dev)
    vc = torch.zeros_like(kc)
    out = torch.empty((n, Hq, D), dtype=torch.int16, device=dev)
    torch.cuda.synchronize()

    n_chunks = (n + ch - 1) // ch
    ev_pf = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
             for _ in range(n_chunks)]
    ev_dec = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))

    def step(record: bool):
        for i, r0 in enumerate(range(0, n, ch)):
            m = min(ch, n - r0)
            ga.attn_cache_write(kc, vc, k[r0:r0 + m], v[r0:r0 + m], r0, m, Hkv, D,
                                w.cap, w.ring)
            if record:
                ev_pf[i][0].record()
            ga.attn_prefill(out[r0:r0 + m], q[r0:r0 + m], kc, vc, r0, m, Hq, Hkv, D,
                            w.cap, w.ring, w.window, w.scale, w.p_mode)
            if record:
                ev_pf[i][1].record()
        if record:
            ev_dec[0].record()
        ga.attn_decode(dout, dq, dk, dv, dpos_t, 1, Hq, Hkv, D, dcap, 0, 0, w.scale, ws)
        if record:
            ev_dec[1].record()

    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()

    pf_ms, dec_ms = 0.0, 0.0
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(True)
        torch.cuda.synchronize()
        pf_ms += sum(a.elapsed_time(b) for a, b in ev_pf)
        dec_ms += ev_dec[0].elapsed_time(ev_dec[1])
    wall = time.perf_counter() - t0
    torch.cuda.synchronize()
    step_clock = gpu_clock_mhz(torch, dev)

    ms_step = wall * 1e3 / args.steps
    tokens = n + 1
    pf_launch_ms = pf_ms / (args.steps * n_chunks)
    dec_us = dec_ms * 1e3 / args.steps

    flops_prompt = causal_pairs(n, w.window) * Hq * 4 * D        # algorithmic
    flops_launch = flops_prompt / n_chunks
    pf_tflops = flops_launch / (pf_launch_ms * 1e-3) / 1e12
    src = os.path.join(ROOT, "global_gqa_attention_window_amd", "csrc", "prefill512.hip")
    traffic = traffic_from_profile(src)
    dec_bytes = 2 * Hkv * dcap * D * 2 + 2 * Hq * D * 2           # K+V read, q, out
    dec_gbs = dec_bytes / (dec_us * 1e-6) / 1e9

    rec = {
        "metric": METRIC,
        "value": round(tokens / (ms_step * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "global_layer_prompt_32k_then_decode_262144",
                   "prompt_tokens": n, "chunk_rows": ch, "q_heads": Hq, "kv_heads": Hkv,
                   "head_dim": D, "p_mode": "bf16x2", "window": 0,
                   "decode_cache_keys": dcap, "seed": w.seed},
        "roofline": {"kernel": "prefill_roles_kernel<bf16x2>", "bound": "mfma",
                     "achieved": round(pf_tflops, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(pf_tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic,
                     "launch_ms": round(pf_launch_ms, 4),
                     "flops_per_launch": flops_launch},
        "prefill": {"tokens_per_s_kernels": round(n / (pf_ms / args.steps * 1e-3), 1),
                    "kernel_ms_per_prompt": round(pf_ms / args.steps, 3)},
        "decode": {"us": round(dec_us, 2), "GB/s": round(dec_gbs, 1),
                   "frac_hbm": round(dec_gbs / PEAK_HBM_GBS, 4), "bytes": dec_bytes},
        "gpu_clock_MHz_after_steps": step_clock,
    }
    # the same decode call 20 times back to back (its 1 GiB K/V still comes
    # from HBM each time: it is four times the last-level cache)
    for _ in range(3):
        ga.attn_decode(dout, dq, dk, dv, dpos_t, 1, Hq, Hkv, D, dcap, 0, 0, w.scale, ws)
    torch.cuda.synchronize()
    ev_dec[0].record()
    for _ in range(20):
        ga.attn_decode(dout, dq, dk, dv, dpos_t, 1, Hq, Hkv, D, dcap, 0, 0, w.scale, ws)
    ev_dec[1].record()
    torch.cuda.synchronize()
    rep_us = ev_dec[0].elapsed_time(ev_dec[1]) * 1e3 / 20
    rep_gbs = dec_bytes / (rep_us * 1e-6) / 1e9
    rec["decode"].update({"us_back_to_back": round(rep_us, 2),
                          "GB/s_back_to_back": round(rep_gbs, 1),
                          "frac_hbm_back_to_back": round(rep_gbs / PEAK_HBM_GBS, 4)})
    # the same prompt through one attn_prefill_prompt call (its bits; a linear
    # cache takes every row first, then one attention launch)
    rec["prefill"]["attn_prefill_prompt_ms"] = round(call_ms(
        torch, lambda: ga.attn_prefill_prompt(out, q, k, v, kc, vc, 0, n, ch, Hq, Hkv, D, w.cap,
                                              w.ring, w.window, w.scale, w.p_mode), 2), 3)
    del q, k, v, kc, vc, out, dk, dv
    torch.cuda.empty_cache()
    split = prefill_sliding(ga, torch, dev)
    plain = prefill_sliding(ga, torch, dev, split=False)
    keep = ("kernel_ms", "tokens_per_s_kernels", "wall_ms_with_cache_writes", "TFLOP/s",
            "frac_bf16_peak", "launch_us")
    whole = split.pop("attn_prefill_prompt_with_cache_writes")
    rec["prefill_sliding_8k"] = {
        **{k: split[k] for k in ("workload", "prompt_tokens", "chunk_rows", "ring_slots",
                                 "window", "head_dim", "q_heads", "kv_heads", "p_mode")},
        "entry_point": "attn_prefill_prompt", "timing": "one call, cache writes included",
        **whole,
        "per_chunk_attn_prefill_ws": {k: split[k] for k in keep},
        "per_chunk_attn_prefill": {k: plain[k] for k in keep},
    }
    rec["decode_configs"] = decode_configs(ga, torch, dev)
    rec["decode_configs_cold"] = decode_cold(ga, torch, dev)
    rec["decode_windows"] = decode_windows(ga, torch, dev)
    rec["attainable"] = attainable(torch, dev)
    rec["attainable"].update(attainable_kernels(torch, dev))
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(q_np, k_np, v_np, w, args.cpu_rows)
        rec["cpu_oracle_workloads"] = cpu_oracle_workloads()
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
