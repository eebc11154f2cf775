"""Host-side checks of the C ABI (no GPU, no compute calls).

The library must load, export every function include/gqa_attn.h declares,
refuse bad arguments with the named status before touching the device, and
report the key block the oracle's contract names.
"""
import ctypes
import os
import re

import pytest

from oracle.contract import DECODE_CHUNK, P_BF16, P_BF16X2, P_FP32, key_block

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gqa_attn.h")
LIB = os.path.join(ROOT, "global_gqa_attention_window_amd", "libgqa_attn.so")

pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="library not built")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_\w+)\s*\(", src)))


def _status(name):
    src = open(HEADER).read()
    return int(re.search(rf"\b{name}\s*=\s*(-?\d+)", src).group(1))


@pytest.fixture(scope="module")
def lib():
    return ctypes.CDLL(LIB)


@pytest.fixture(scope="module")
def ga():
    import global_gqa_attention_window_amd as ga
    return ga


def test_exports_every_declared_function(lib):
    names = _declared()
    assert set(names) >= {"attn_decode", "attn_prefill", "attn_cache_write",
                          "attn_decode_workspace_bytes", "attn_prefill_key_block",
                          "attn_status_string"}
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings(ga):
    for name in ["ATTN_OK", "ATTN_E_NULL", "ATTN_E_HEAD_DIM", "ATTN_E_GQA",
                 "ATTN_E_WINDOW", "ATTN_E_CACHE", "ATTN_E_ALIGN", "ATTN_E_WORKSPACE",
                 "ATTN_E_P_MODE", "ATTN_E_RANGE", "ATTN_E_LAUNCH", "ATTN_E_UNSUPPORTED"]:
        assert ga.attn_status_string(_status(name)) == name
    assert ga.attn_status_string(12345) == "ATTN_E_UNKNOWN"


def test_key_block_matches_contract(ga):
    for D in (256, 512):
        for pm in (P_BF16, P_BF16X2):
            assert ga.attn_prefill_key_block(D, pm) == key_block(D, pm)
    assert ga._lib.attn_prefill_key_block(128, P_BF16) == _status("ATTN_E_HEAD_DIM")
    assert ga._lib.attn_prefill_key_block(256, P_FP32) == _status("ATTN_E_P_MODE")
    assert ga.ATTN_DECODE_CHUNK == DECODE_CHUNK


def test_workspace_bytes(ga):
    # one fp32 (max, sum, acc[D]) per (stream, query head, 256-slot chunk);
    # caches of at most 1024 (512) slots run half (quarter) chunks, one
    # partial each
    assert ga.attn_decode_workspace_bytes(8, 32, 512, 32768) == 8 * 32 * 128 * 514 * 4
    assert ga.attn_decode_workspace_bytes(1, 8, 256, 512) == 1 * 8 * 8 * 258 * 4
    assert ga.attn_decode_workspace_bytes(1, 8, 256, 300) == 1 * 8 * 5 * 258 * 4
    assert ga.attn_decode_workspace_bytes(1, 8, 256, 1024) == 1 * 8 * 8 * 258 * 4
    assert ga.attn_decode_workspace_bytes(1, 8, 256, 1025) == 1 * 8 * 5 * 258 * 4
    assert ga.attn_decode_workspace_bytes(1, 8, 128, 512) == 0
    assert ga.attn_decode_workspace_bytes(1, 8, 256, 0) == 0
    assert ga.attn_decode_workspace_bytes(-1, 8, 256, 10) == 0


# fake device pointers: refusals happen before any use, so these are never read.
# The refusal tests pass them to real entry points, so they run only where no
# GPU is visible: if a check ever let a call through, its launch would fail on
# the host instead of touching unmapped device memory.
P = 1 << 20


def _gpu_visible():
    try:
        import torch
        return torch.cuda.device_count() > 0
    except Exception:          # no torch: no GPU either
        return False


no_gpu = pytest.mark.skipif(_gpu_visible(), reason="fake device pointers; CPU-only checks")


def _decode(ga, **kw):
    a = dict(out=P, q=P, k=P, v=P, pos=P, S=1, Hq=8, Hkv=1, D=256, cap=512, ring=0,
             window=0, scale=0.0625, ws=P, ws_bytes=1 << 30)
    a.update(kw)
    return ga._lib.attn_decode(a["out"], a["q"], a["k"], a["v"], a["pos"], a["S"], a["Hq"],
                               a["Hkv"], a["D"], a["cap"], a["ring"], a["window"], a["scale"],
                               a["ws"], a["ws_bytes"], None)


def _prefill(ga, **kw):
    a = dict(out=P, q=P, k=P, v=P, pos0=0, n=128, Hq=32, Hkv=4, D=256, cap=1152, ring=1,
             window=1024, scale=0.0625, p_mode=P_BF16, last=None)
    a.update(kw)
    return ga._lib.attn_prefill(a["out"], a["q"], a["k"], a["v"], a["pos0"], a["n"], a["Hq"],
                                a["Hkv"], a["D"], a["cap"], a["ring"], a["window"],
                                a["scale"], a["p_mode"], a["last"], None)


def _cw(ga, **kw):
    a = dict(kc=P, vc=P, k=P, v=P, pos0=0, n=128, Hkv=4, D=256, cap=1152, ring=1)
    a.update(kw)
    return ga._lib.attn_cache_write(a["kc"], a["vc"], a["k"], a["v"], a["pos0"], a["n"],
                                    a["Hkv"], a["D"], a["cap"], a["ring"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(out=None), "ATTN_E_NULL"), (dict(q=None), "ATTN_E_NULL"),
    (dict(k=None), "ATTN_E_NULL"), (dict(v=None), "ATTN_E_NULL"),
    (dict(pos=None), "ATTN_E_NULL"), (dict(ws=None), "ATTN_E_WORKSPACE"),
    (dict(D=128), "ATTN_E_HEAD_DIM"), (dict(D=384), "ATTN_E_HEAD_DIM"),
    (dict(Hq=12, Hkv=8), "ATTN_E_GQA"), (dict(Hq=34, Hkv=2), "ATTN_E_GQA"),
    (dict(Hkv=0), "ATTN_E_GQA"), (dict(Hq=0), "ATTN_E_GQA"),
    (dict(window=-1), "ATTN_E_WINDOW"), (dict(ring=1, window=513), "ATTN_E_WINDOW"),
    (dict(cap=0), "ATTN_E_CACHE"), (dict(S=-1), "ATTN_E_RANGE"),
    (dict(ring=2), "ATTN_E_RANGE"), (dict(scale=float("inf")), "ATTN_E_RANGE"),
    (dict(scale=float("nan")), "ATTN_E_RANGE"),
    (dict(out=P + 2), "ATTN_E_ALIGN"), (dict(k=P + 8), "ATTN_E_ALIGN"),
    (dict(ws=P + 4), "ATTN_E_ALIGN"), (dict(pos=P + 2), "ATTN_E_ALIGN"),
    (dict(ws_bytes=100), "ATTN_E_WORKSPACE"),
    (dict(S=1 << 20, cap=1 << 30, Hkv=1 << 10, Hq=1 << 10), "ATTN_E_RANGE"),
])
@no_gpu
def test_decode_refusals(ga, kw, status):
    assert _decode(ga, **kw) == _status(status)


@no_gpu
def test_decode_zero_streams_is_a_no_op(ga):
    assert _decode(ga, S=0, out=None, q=None, ws=None) == 0


@pytest.mark.parametrize("kw,status", [
    (dict(out=None), "ATTN_E_NULL"), (dict(k=None), "ATTN_E_NULL"),
    (dict(D=64), "ATTN_E_HEAD_DIM"), (dict(Hq=30), "ATTN_E_GQA"),
    (dict(p_mode=P_FP32), "ATTN_E_P_MODE"), (dict(p_mode=7), "ATTN_E_P_MODE"),
    (dict(last=P + 2), "ATTN_E_ALIGN"),
    (dict(ring=1, window=0), "ATTN_E_WINDOW"), (dict(window=1153), "ATTN_E_WINDOW"),
    (dict(window=-3), "ATTN_E_WINDOW"),
    (dict(cap=1150), "ATTN_E_CACHE"),              # ring < window + rows - 1
    (dict(ring=0, window=0, cap=1000, pos0=900), "ATTN_E_CACHE"),
    (dict(cap=0), "ATTN_E_CACHE"), (dict(n=-1), "ATTN_E_RANGE"),
    (dict(pos0=-5), "ATTN_E_RANGE"), (dict(scale=float("-inf")), "ATTN_E_RANGE"),
    (dict(q=P + 6), "ATTN_E_ALIGN"),
])
@no_gpu
def test_prefill_refusals(ga, kw, status):
    assert _prefill(ga, **kw) == _status(status)


@no_gpu
def test_prefill_refuses_slices_past_32_bit_offsets(ga):
    # one head's cache slice is addressed with 32-bit byte offsets
    assert _prefill(ga, ring=0, window=0, D=512, cap=1 << 22, n=0) == _status("ATTN_E_RANGE")
    assert _prefill(ga, ring=0, window=0, D=512, cap=(1 << 22) - 1, n=0) == 0


@no_gpu
def test_prefill_refuses_positions_past_int32(ga):
    # a ring's positions grow past its capacity; the kernels add up to one
    # key block (64) to the last row's position in 32-bit ints
    imax = 0x7FFFFFFF
    assert _prefill(ga, pos0=imax - 128 - 64 + 1, n=128) == _status("ATTN_E_RANGE")
    assert _prefill(ga, pos0=imax, n=1) == _status("ATTN_E_RANGE")
    assert _prefill(ga, pos0=imax - 64, n=0) == 0


@no_gpu
def test_prefill_edges_accepted_by_checks(ga):
    # exact fits pass the checks; n = 0 returns before any launch
    assert _prefill(ga, n=0, out=None) == 0
    assert _prefill(ga, ring=0, window=0, cap=1000, pos0=872, n=0) == 0


def _prefill_ws(ga, ws=P, ws_bytes=1 << 30, **kw):
    a = dict(out=P, q=P, k=P, v=P, pos0=0, n=128, Hq=32, Hkv=4, D=256, cap=1152, ring=1,
             window=1024, scale=0.0625, p_mode=P_BF16, last=None)
    a.update(kw)
    return ga._lib.attn_prefill_ws(a["out"], a["q"], a["k"], a["v"], a["pos0"], a["n"],
                                   a["Hq"], a["Hkv"], a["D"], a["cap"], a["ring"], a["window"],
                                   a["scale"], a["p_mode"], a["last"], ws, ws_bytes, None)


def test_prefill_workspace_bytes(ga):
    # fp32 (max, sum, accumulator[D]) for up to four key ranges per row and head
    assert ga.attn_prefill_workspace_bytes(128, 32, 256) == 128 * 32 * 4 * 258 * 4
    assert ga.attn_prefill_workspace_bytes(0, 32, 256) == 0
    assert ga.attn_prefill_workspace_bytes(128, 32, 384) == 0
    assert ga.attn_prefill_workspace_bytes(-1, 32, 256) == 0


@pytest.mark.parametrize("kw,status", [
    (dict(ws_bytes=100), "ATTN_E_WORKSPACE"), (dict(ws=P + 8), "ATTN_E_ALIGN"),
    (dict(out=None), "ATTN_E_NULL"), (dict(D=64), "ATTN_E_HEAD_DIM"),
    (dict(p_mode=P_FP32), "ATTN_E_P_MODE"), (dict(cap=1150), "ATTN_E_CACHE"),
    (dict(pos0=-5), "ATTN_E_RANGE"), (dict(last=P + 2), "ATTN_E_ALIGN"),
    # a NULL workspace takes attn_prefill's path and checks
    (dict(ws=None, q=None), "ATTN_E_NULL"), (dict(ws=None, window=-1), "ATTN_E_WINDOW"),
])
@no_gpu
def test_prefill_ws_refusals(ga, kw, status):
    assert _prefill_ws(ga, **kw) == _status(status)


@no_gpu
def test_prefill_ws_zero_rows_is_a_no_op(ga):
    assert _prefill_ws(ga, n=0, out=None, ws_bytes=0) == 0


def _prompt(ga, ws=P, ws_bytes=1 << 30, **kw):
    a = dict(out=P, q=P, k=P, v=P, kc=P, vc=P, pos0=0, n=8192, chunk=128, Hq=32, Hkv=4, D=256,
             cap=1152, ring=1, window=1024, scale=0.0625, p_mode=P_BF16, last=None)
    a.update(kw)
    return ga._lib.attn_prefill_prompt(a["out"], a["q"], a["k"], a["v"], a["kc"], a["vc"],
                                       a["pos0"], a["n"], a["chunk"], a["Hq"], a["Hkv"], a["D"],
                                       a["cap"], a["ring"], a["window"], a["scale"], a["p_mode"],
                                       a["last"], ws, ws_bytes, None)


def test_prefill_prompt_workspace_bytes(ga):
    # a ring's attended span (the window before pos0 and the prompt) as K and
    # V copies [Hkv][span][D]; a linear cache needs none
    f = ga.attn_prefill_prompt_workspace_bytes
    assert f(0, 8192, 4, 256, 1, 1024) == 2 * 4 * 8192 * 256 * 2
    assert f(5000, 8192, 4, 256, 1, 1024) == 2 * 4 * (1023 + 8192) * 256 * 2
    assert f(100, 50, 2, 512, 1, 1024) == 2 * 2 * 150 * 512 * 2
    assert f(0, 32768, 2, 512, 0, 0) == 0
    assert f(0, 10, 2, 384, 1, 8) == 0 and f(0, 10, 2, 256, 1, 0) == 0


@pytest.mark.parametrize("kw,status", [
    (dict(chunk=0), "ATTN_E_RANGE"), (dict(n=-1), "ATTN_E_RANGE"),
    (dict(ws=None, ws_bytes=0), "ATTN_E_WORKSPACE"),   # a ring needs the span's copy
    (dict(chunk=130), "ATTN_E_CACHE"),                 # ring: cap < W + chunk - 1
    (dict(ring=0, window=0, cap=8000), "ATTN_E_CACHE"),  # linear: the prompt passes cap
    (dict(ws_bytes=100), "ATTN_E_WORKSPACE"), (dict(ws=P + 8), "ATTN_E_ALIGN"),
    (dict(k=None), "ATTN_E_NULL"), (dict(vc=None), "ATTN_E_NULL"),
    (dict(v=P + 2), "ATTN_E_ALIGN"), (dict(last=P + 2), "ATTN_E_ALIGN"),
    (dict(D=64), "ATTN_E_HEAD_DIM"), (dict(p_mode=P_FP32), "ATTN_E_P_MODE"),
    (dict(pos0=0x7FFFFFFF - 8192), "ATTN_E_RANGE"),
])
@no_gpu
def test_prefill_prompt_refusals(ga, kw, status):
    assert _prompt(ga, **kw) == _status(status)


@no_gpu
def test_prefill_prompt_zero_rows_is_a_no_op(ga):
    assert _prompt(ga, n=0, out=None, k=None, ws=None, ws_bytes=0) == 0


@no_gpu
def test_prefill_prompt_linear_needs_no_workspace(ga):
    # a linear cache passes every check without a workspace (the first
    # refusal left is the NULL output)
    assert _prompt(ga, ring=0, window=0, cap=8192, ws=None, ws_bytes=0,
                   out=None) == _status("ATTN_E_NULL")


@pytest.mark.parametrize("kw,status", [
    (dict(kc=None), "ATTN_E_NULL"), (dict(v=None), "ATTN_E_NULL"),
    (dict(D=100), "ATTN_E_HEAD_DIM"), (dict(Hkv=0), "ATTN_E_GQA"),
    (dict(ring=0, cap=1000, pos0=900), "ATTN_E_CACHE"),
    (dict(n=1153), "ATTN_E_CACHE"), (dict(pos0=-1), "ATTN_E_RANGE"),
    (dict(k=P + 2), "ATTN_E_ALIGN"),
])
@no_gpu
def test_cache_write_refusals(ga, kw, status):
    assert _cw(ga, **kw) == _status(status)


def _rows(ga, **kw):
    a = dict(out=P, q=P, k=P, v=P, pos=P, S=2, R=16, Hq=32, Hkv=2, D=512, cap=32768, ring=0,
             window=0, scale=0.044, ws=P, ws_bytes=1 << 34)
    a.update(kw)
    return ga._lib.attn_decode_rows(a["out"], a["q"], a["k"], a["v"], a["pos"], a["S"], a["R"],
                                    a["Hq"], a["Hkv"], a["D"], a["cap"], a["ring"], a["window"],
                                    a["scale"], a["ws"], a["ws_bytes"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(R=0), "ATTN_E_RANGE"), (dict(R=17), "ATTN_E_RANGE"), (dict(R=-1), "ATTN_E_RANGE"),
    (dict(ring=1, window=0, cap=1024), "ATTN_E_WINDOW"),
    (dict(ring=1, window=1024, cap=1038), "ATTN_E_WINDOW"),     # W + R - 1 = 1039 slots
    (dict(window=-1), "ATTN_E_WINDOW"),
    (dict(out=None), "ATTN_E_NULL"), (dict(pos=None), "ATTN_E_NULL"),
    (dict(ws=None), "ATTN_E_WORKSPACE"), (dict(ws_bytes=1000), "ATTN_E_WORKSPACE"),
    (dict(D=128), "ATTN_E_HEAD_DIM"), (dict(Hq=34), "ATTN_E_GQA"), (dict(Hq=64), "ATTN_E_GQA"),
    (dict(pos=P + 2), "ATTN_E_ALIGN"), (dict(q=P + 8), "ATTN_E_ALIGN"),
    (dict(scale=float("nan")), "ATTN_E_RANGE"), (dict(cap=0), "ATTN_E_CACHE"),
])
@no_gpu
def test_decode_rows_refusals(ga, kw, status):
    assert _rows(ga, **kw) == _status(status)


@no_gpu
def test_decode_rows_edges_and_workspace(ga):
    assert _rows(ga, S=0, out=None, q=None, ws=None) == 0
    # a ring of exactly W + R - 1 slots passes the geometry check (then n_seq = 0)
    assert _rows(ga, S=0, ring=1, window=1024, cap=1039) == 0
    # partials of every (stream, row, head, 256-slot chunk), as S * R one-row streams
    assert ga.attn_decode_rows_workspace_bytes(8, 16, 32, 512, 32768) == \
        ga.attn_decode_workspace_bytes(128, 32, 512, 32768)
    assert ga.attn_decode_rows_workspace_bytes(1, 0, 8, 256, 512) == 0
    assert ga.attn_decode_rows_workspace_bytes(1, 17, 8, 256, 512) == 0
    assert ga.ATTN_DECODE_MAX_ROWS == 16


@no_gpu
def test_fused_decode_refusals(ga):
    lib = ga._lib
    n = 1 << 34
    # counter area beyond its limit (n_seq * Hkv > 4096)
    assert lib.attn_decode_rows_fused(P, P, P, P, P, 4097, 1, 8, 1, 256, 512, 0, 0, 0.1, P, n,
                                      None) == _status("ATTN_E_RANGE")
    # workspace without room for the counters
    need = ga.attn_decode_rows_workspace_bytes(1, 1, 8, 256, 512)
    assert lib.attn_decode_rows_fused(P, P, P, P, P, 1, 1, 8, 1, 256, 512, 0, 0, 0.1, P, need,
                                      None) == _status("ATTN_E_WORKSPACE")
    assert lib.attn_decode_rows_fused(P, P, P, P, P, 0, 1, 8, 1, 256, 512, 0, 0, 0.1, None, 0,
                                      None) == 0
    assert lib.attn_decode_workspace_init(None, 1 << 20, None) == _status("ATTN_E_WORKSPACE")
    assert lib.attn_decode_workspace_init(P, 1000, None) == _status("ATTN_E_WORKSPACE")
    assert lib.attn_decode_workspace_init(P + 4, 1 << 20, None) == _status("ATTN_E_ALIGN")


@no_gpu
def test_noalloc_decode_refusals(ga):
    lib = ga._lib

    def call(**kw):
        a = dict(out=P, q=P, k=P, v=P, pos=P, S=8, Hq=32, Hkv=2, D=512, cap=32768, ring=0,
                 window=0, scale=0.044)
        a.update(kw)
        return lib.attn_decode_noalloc(a["out"], a["q"], a["k"], a["v"], a["pos"], a["S"],
                                       a["Hq"], a["Hkv"], a["D"], a["cap"], a["ring"],
                                       a["window"], a["scale"], None)
    # partials past the library's array: 8 x 32 heads x 32 runs x 514 x 4 B > 16 MiB
    assert 8 * 32 * 32 * 514 * 4 > ga.ATTN_DECODE_SCRATCH_BYTES
    assert call(cap=65536) == _status("ATTN_E_WORKSPACE")
    assert call(S=17) == _status("ATTN_E_WORKSPACE")
    # the other checks are attn_decode's
    assert call(S=0, out=None) == 0
    assert call(out=None) == _status("ATTN_E_NULL")
    assert call(D=128) == _status("ATTN_E_HEAD_DIM")
    assert call(Hq=31) == _status("ATTN_E_GQA")
    assert call(q=P + 2) == _status("ATTN_E_ALIGN")
    assert call(ring=1, window=40000) == _status("ATTN_E_WINDOW")
    assert call(scale=float("nan")) == _status("ATTN_E_RANGE")
