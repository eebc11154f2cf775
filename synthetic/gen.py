"""Seeded N(0,1) bf16 inputs shaped like the pages' attention workloads.

Recipe (the same for every workload):
  * numpy PCG64 seeded with the workload's seed;
  * draws in the order q, then k, then v, each ``standard_normal`` in float32;
  * each float32 draw is stored as bf16 by round-to-nearest-even on its bit
    pattern (the textbook integer form, done here only to make storage; it is
    not a rounding point of the method);
  * arrays are returned as uint16 bf16 bit patterns, C-contiguous.

Layouts:
  decode  q [S][Hq][D], k_cache / v_cache [S][Hkv][cap][D], every slot drawn
          (a fully populated cache; which slots a row may read is the method's
          business, not this module's), pos [S] int32.
  prefill q [n_rows][Hq][D] for prompt positions 0..n_rows-1, and k / v
          [n_rows][Hkv][D] indexed by absolute position.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

P_FP32, P_BF16, P_BF16X2 = 0, 1, 2


@dataclass(frozen=True)
class Workload:
    name: str
    kind: str                 # "decode" or "prefill"
    Hq: int
    Hkv: int
    D: int
    scale: float
    seed: int
    # decode
    S: int = 1
    cap: int = 0
    ring: int = 0
    window: int = 0
    pos: tuple = ()
    rows: int = 1             # decode window: rows per stream at pos .. pos + rows - 1
    # prefill
    n_rows: int = 0
    chunk: int = 0
    p_mode: int = P_BF16
    extra: dict = field(default_factory=dict)


def _f32(x: float) -> float:
    return float(np.float32(x))


# The five workloads of the pages' attention path: shapes, windows, scales and
# seeds.  Sliding layers: head dim 256, window 1024.  Global layers: head dim
# 512, no window, linear cache up to 262144 keys.
WORKLOADS: dict[str, Workload] = {
    # decode, one row, 8 query heads over one KV head, 512 cached keys
    "decode_g8_d256_512": Workload(
        name="decode_g8_d256_512", kind="decode", Hq=8, Hkv=1, D=256,
        scale=_f32(1 / 16), seed=1001, S=1, cap=512, ring=0, window=512,
        pos=(511,)),
    # sliding-layer decode: 8 streams, ring of window 1024 fully populated
    "decode_sliding_ring1024": Workload(
        name="decode_sliding_ring1024", kind="decode", Hq=32, Hkv=4, D=256,
        scale=_f32(1 / 16), seed=1002, S=8, cap=1024, ring=1, window=1024,
        pos=tuple(4095 + 1000 * s for s in range(8))),
    # global-layer decode: 8 streams over a 32768-key linear cache, GQA 16
    "decode_global_32k": Workload(
        name="decode_global_32k", kind="decode", Hq=32, Hkv=2, D=512,
        scale=_f32(1 / math.sqrt(512)), seed=1003, S=8, cap=32768, ring=0,
        window=0, pos=tuple(32767 for _ in range(8))),
    # decode windows of 16 rows a stream (128 rows a forward) on a global
    # layer: 8 streams over a 32768-key linear cache, last rows at its end
    "decode_rows_global_32k": Workload(
        name="decode_rows_global_32k", kind="decode", Hq=32, Hkv=2, D=512,
        scale=_f32(1 / math.sqrt(512)), seed=1006, S=8, cap=32768, ring=0,
        window=0, pos=tuple(32752 for _ in range(8)), rows=16),
    # ... on a sliding layer: ring of 1536 slots (window 1024 plus room for
    # the window's later rows), streams at different ring phases
    "decode_rows_sliding_1536": Workload(
        name="decode_rows_sliding_1536", kind="decode", Hq=32, Hkv=4, D=256,
        scale=_f32(1 / 16), seed=1007, S=8, cap=1536, ring=1, window=1024,
        pos=tuple(4080 + 1000 * s for s in range(8)), rows=16),
    # sliding-layer prefill: 8192-token prompt in 128-row chunks, ring of
    # window + chunk = 1152 slots, P rounded to bf16
    "prefill_sliding_8k": Workload(
        name="prefill_sliding_8k", kind="prefill", Hq=32, Hkv=4, D=256,
        scale=_f32(1 / 16), seed=1004, cap=1152, ring=1, window=1024,
        n_rows=8192, chunk=128, p_mode=P_BF16),
    # global-layer prefill: 32768-token causal prompt in 512-row chunks over
    # a linear cache, P kept as two bf16 halves; then one-row decode over a
    # 262144-key linear cache with the same heads
    "prefill_global_32k": Workload(
        name="prefill_global_32k", kind="prefill", Hq=32, Hkv=2, D=512,
        scale=_f32(1 / math.sqrt(512)), seed=1005, cap=32768, ring=0,
        window=0, n_rows=32768, chunk=512, p_mode=P_BF16X2,
        extra={"decode_cap": 262144, "decode_pos": 262143,
               "decode_seed": 2005}),
}


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 array -> uint16 bf16 bits, round to nearest even (storage)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    nan = (u & 0x7FFFFFFF) > 0x7F800000
    r = (u + np.uint32(0x7FFF) + ((u >> 16) & np.uint32(1))) >> 16
    r = r.astype(np.uint16)
    r[nan] = 0x7FC0
    return r


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """uint16 bf16 bits -> float32 (exact widening)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def randn_bf16_bits(rng: np.random.Generator, shape, block: int = 1 << 24) -> np.ndarray:
    """N(0,1) float32 draws stored as bf16 bits, drawn in C order in blocks."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16)
    for i in range(0, n, block):
        m = min(block, n - i)
        out[i:i + m] = f32_to_bf16_bits(rng.standard_normal(m, dtype=np.float32))
    return out.reshape(shape)


def decode_inputs(w: Workload, S: int | None = None, cap: int | None = None,
                  pos=None, seed: int | None = None):
    """q [S][Hq][D], k_cache, v_cache [S][Hkv][cap][D] (bf16 bits), pos [S] int32."""
    S = w.S if S is None else S
    cap = w.cap if cap is None else cap
    pos = w.pos if pos is None else pos
    rng = np.random.default_rng(w.seed if seed is None else seed)
    q = randn_bf16_bits(rng, (S, w.Hq, w.D))
    k = randn_bf16_bits(rng, (S, w.Hkv, cap, w.D))
    v = randn_bf16_bits(rng, (S, w.Hkv, cap, w.D))
    return q, k, v, np.asarray(pos, dtype=np.int32).reshape(S)


def decode_rows_inputs(w: Workload, S: int | None = None, seed: int | None = None):
    """q [S][rows][Hq][D], k_cache, v_cache [S][Hkv][cap][D] (bf16 bits), pos
    [S] int32 (first row of each window); every slot holds a written key."""
    S = w.S if S is None else S
    rng = np.random.default_rng(w.seed if seed is None else seed)
    q = randn_bf16_bits(rng, (S, w.rows, w.Hq, w.D))
    k = randn_bf16_bits(rng, (S, w.Hkv, w.cap, w.D))
    v = randn_bf16_bits(rng, (S, w.Hkv, w.cap, w.D))
    return q, k, v, np.asarray(w.pos[:S], dtype=np.int32)


def prefill_inputs(w: Workload, n_rows: int | None = None, seed: int | None = None):
    """q [n][Hq][D], k, v [n][Hkv][D] (bf16 bits), positions 0..n-1."""
    n = w.n_rows if n_rows is None else n_rows
    rng = np.random.default_rng(w.seed if seed is None else seed)
    q = randn_bf16_bits(rng, (n, w.Hq, w.D))
    k = randn_bf16_bits(rng, (n, w.Hkv, w.D))
    v = randn_bf16_bits(rng, (n, w.Hkv, w.D))
    return q, k, v


def image_spans(rng: np.random.Generator, n: int, n_images: int = 6, min_len: int = 64,
                max_len: int = 280) -> list[tuple[int, int]]:
    """Row spans [a, b] (inclusive, ascending, disjoint) of n_images images in
    an n-row prompt: lengths uniform in [min_len, max_len] (an image takes up
    to 280 rows), text between them split at uniform random cuts."""
    lens = rng.integers(min_len, max_len + 1, n_images)
    text = n - int(lens.sum())
    if text < 0:
        raise ValueError("images longer than the prompt")
    gaps = np.diff(np.concatenate([[0], np.sort(rng.integers(0, text + 1, n_images)),
                                   [text]]))
    spans, p = [], 0
    for i in range(n_images):
        p += int(gaps[i])
        spans.append((p, p + int(lens[i]) - 1))
        p += int(lens[i])
    return spans


def image_span_last_keys(pos0: int, n: int, spans) -> np.ndarray:
    """Each row's last key: its own position, or its image's last position
    for rows inside a span (spans in absolute positions)."""
    t = pos0 + np.arange(n, dtype=np.int64)
    lk = t.copy()
    for a, b in spans:
        inside = (t >= a) & (t <= b)
        lk[inside] = b
    return lk


def chunk_starts(n: int, max_rows: int, spans) -> list[int]:
    """Starts of prompt chunks of up to max_rows rows that never cut an
    image: a cut inside a span moves to the span's start, or past its end
    when the chunk itself starts there (that chunk is then longer)."""
    starts, s = [], 0
    while s < n:
        starts.append(s)
        e = min(n, s + max_rows)
        for a, b in spans:
            if a < e <= b:
                e = a if a > s else b + 1
        s = e
    return starts
