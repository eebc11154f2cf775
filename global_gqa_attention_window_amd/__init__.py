"""Python binding of libgqa_attn.so (MI355X GQA window attention).

Argument marshalling only: each function passes tensor data pointers, sizes
and the current HIP stream to the C entry point of the same name declared in
include/gqa_attn.h, and raises AttnError on a non-zero status.  Every step of
the attention runs in the library's gfx950 kernels; there is no fallback.  If
the library has not been built, importing this package raises ImportError.

PyTorch is used for device memory and streams only.  bf16 tensors may be
torch.bfloat16 or 16-bit integer tensors holding bf16 bit patterns.
"""
from __future__ import annotations

import ctypes
import os

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libgqa_attn.so")
if not os.path.exists(_LIB_PATH):
    raise ImportError(
        f"{_LIB_PATH} is missing: build it with "
        "`python -c 'import __graft_entry__ as g; g.build()'` (hipcc, gfx950)")
_lib = ctypes.CDLL(_LIB_PATH)

ATTN_OK = 0
ATTN_P_FP32, ATTN_P_BF16, ATTN_P_BF16X2 = 0, 1, 2
ATTN_DECODE_CHUNK = 256
ATTN_DECODE_MAX_ROWS = 16
ATTN_DECODE_COUNTER_BYTES = 65536

_c_int, _c_void_p, _c_float, _c_size_t = ctypes.c_int, ctypes.c_void_p, ctypes.c_float, ctypes.c_size_t

_lib.attn_decode_workspace_bytes.restype = _c_size_t
_lib.attn_decode_workspace_bytes.argtypes = [_c_int] * 4
_lib.attn_decode.restype = _c_int
_lib.attn_decode.argtypes = ([_c_void_p] * 5 + [_c_int] * 7 + [_c_float, _c_void_p, _c_size_t, _c_void_p])
_lib.attn_decode_rows_workspace_bytes.restype = _c_size_t
_lib.attn_decode_rows_workspace_bytes.argtypes = [_c_int] * 5
_lib.attn_decode_rows.restype = _c_int
_lib.attn_decode_rows.argtypes = ([_c_void_p] * 5 + [_c_int] * 8 +
                                  [_c_float, _c_void_p, _c_size_t, _c_void_p])
_lib.attn_decode_rows_fused.restype = _c_int
_lib.attn_decode_rows_fused.argtypes = _lib.attn_decode_rows.argtypes
_lib.attn_decode_workspace_init.restype = _c_int
_lib.attn_decode_workspace_init.argtypes = [_c_void_p, _c_size_t, _c_void_p]
_lib.attn_qkv_prep.restype = _c_int
_lib.attn_qkv_prep.argtypes = ([_c_void_p] * 7 + [_c_float, _c_int, _c_void_p] + [_c_int] * 6 +
                               [_c_void_p])
_lib.attn_decode_prep_fused.restype = _c_int
_lib.attn_decode_prep_fused.argtypes = ([_c_void_p] * 5 + [_c_float, _c_int] + [_c_void_p] * 3 +
                                        [_c_int] * 7 + [_c_float, _c_void_p, _c_size_t,
                                                        _c_void_p])
_lib.attn_prefill.restype = _c_int
_lib.attn_prefill.argtypes = ([_c_void_p] * 4 + [_c_int] * 8 + [_c_float, _c_int, _c_void_p, _c_void_p])
_lib.attn_cache_write.restype = _c_int
_lib.attn_cache_write.argtypes = [_c_void_p] * 4 + [_c_int] * 6 + [_c_void_p]
_lib.attn_prefill_key_block.restype = _c_int
_lib.attn_prefill_key_block.argtypes = [_c_int, _c_int]
_lib.attn_status_string.restype = ctypes.c_char_p
_lib.attn_status_string.argtypes = [_c_int]


class AttnError(RuntimeError):
    def __init__(self, status: int, call: str):
        self.status = status
        super().__init__(f"{call}: {attn_status_string(status)} ({status})")


def library_path() -> str:
    return _LIB_PATH


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(stream)


def _ok(status: int, call: str) -> None:
    if status != ATTN_OK:
        raise AttnError(status, call)


def attn_status_string(status: int) -> str:
    return _lib.attn_status_string(int(status)).decode()


def attn_decode_workspace_bytes(n_seq: int, n_q_heads: int, head_dim: int, cache_cap: int) -> int:
    return int(_lib.attn_decode_workspace_bytes(n_seq, n_q_heads, head_dim, cache_cap))


def attn_decode_rows_workspace_bytes(n_seq: int, rows: int, n_q_heads: int, head_dim: int,
                                     cache_cap: int) -> int:
    return int(_lib.attn_decode_rows_workspace_bytes(n_seq, rows, n_q_heads, head_dim,
                                                     cache_cap))


def attn_prefill_key_block(head_dim: int, p_mode: int) -> int:
    kb = int(_lib.attn_prefill_key_block(head_dim, p_mode))
    _ok(min(kb, 0), "attn_prefill_key_block")
    return kb


def attn_decode(out, q, k_cache, v_cache, pos, n_seq, n_q_heads, n_kv_heads,
                head_dim, cache_cap, ring, window, scale, workspace,
                workspace_bytes=None, stream=None) -> None:
    """out/q [S][Hq][D], caches [S][Hkv][cap][D] (bf16), pos int32 [S]."""
    if workspace_bytes is None:
        workspace_bytes = workspace.numel() * workspace.element_size()
    st = _lib.attn_decode(_ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(pos),
                          n_seq, n_q_heads, n_kv_heads, head_dim, cache_cap, ring,
                          window, float(scale), _ptr(workspace), int(workspace_bytes),
                          _stream(stream))
    _ok(st, "attn_decode")


def attn_decode_rows(out, q, k_cache, v_cache, pos, n_seq, rows, n_q_heads, n_kv_heads,
                     head_dim, cache_cap, ring, window, scale, workspace,
                     workspace_bytes=None, stream=None) -> None:
    """out/q [S][rows][Hq][D], caches [S][Hkv][cap][D] (bf16), pos int32 [S]
    (the first row's position)."""
    if workspace_bytes is None:
        workspace_bytes = workspace.numel() * workspace.element_size()
    st = _lib.attn_decode_rows(_ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(pos),
                               n_seq, rows, n_q_heads, n_kv_heads, head_dim, cache_cap, ring,
                               window, float(scale), _ptr(workspace), int(workspace_bytes),
                               _stream(stream))
    _ok(st, "attn_decode_rows")


def attn_decode_rows_fused(out, q, k_cache, v_cache, pos, n_seq, rows, n_q_heads, n_kv_heads,
                           head_dim, cache_cap, ring, window, scale, workspace,
                           workspace_bytes=None, stream=None) -> None:
    """attn_decode_rows in one launch where it can; the workspace starts with
    ATTN_DECODE_COUNTER_BYTES of counters set up by attn_decode_workspace_init."""
    if workspace_bytes is None:
        workspace_bytes = workspace.numel() * workspace.element_size()
    st = _lib.attn_decode_rows_fused(_ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                     _ptr(pos), n_seq, rows, n_q_heads, n_kv_heads, head_dim,
                                     cache_cap, ring, window, float(scale), _ptr(workspace),
                                     int(workspace_bytes), _stream(stream))
    _ok(st, "attn_decode_rows_fused")


def attn_qkv_prep(q_out, k_cache, v_cache, qkv, q_norm_w, k_norm_w, inv_freq, eps, v_norm,
                  pos, n_seq, n_q_heads, n_kv_heads, head_dim, cache_cap, ring,
                  stream=None) -> None:
    """qkv [S][(Hq + 2 Hkv) D] bf16 -> q_out [S][Hq][D], key/value at each
    row's cache slot; inv_freq fp32 [D/2]."""
    st = _lib.attn_qkv_prep(_ptr(q_out), _ptr(k_cache), _ptr(v_cache), _ptr(qkv),
                            _ptr(q_norm_w), _ptr(k_norm_w), _ptr(inv_freq), float(eps),
                            int(v_norm), _ptr(pos), n_seq, n_q_heads, n_kv_heads, head_dim,
                            cache_cap, ring, _stream(stream))
    _ok(st, "attn_qkv_prep")


def attn_decode_prep_fused(out, qkv, q_norm_w, k_norm_w, inv_freq, eps, v_norm, k_cache,
                           v_cache, pos, n_seq, n_q_heads, n_kv_heads, head_dim, cache_cap,
                           ring, window, scale, workspace, workspace_bytes=None,
                           stream=None) -> None:
    """attn_qkv_prep + one-row attn_decode_rows_fused in the decode kernel."""
    if workspace_bytes is None:
        workspace_bytes = workspace.numel() * workspace.element_size()
    st = _lib.attn_decode_prep_fused(_ptr(out), _ptr(qkv), _ptr(q_norm_w), _ptr(k_norm_w),
                                     _ptr(inv_freq), float(eps), int(v_norm), _ptr(k_cache),
                                     _ptr(v_cache), _ptr(pos), n_seq, n_q_heads, n_kv_heads,
                                     head_dim, cache_cap, ring, window, float(scale),
                                     _ptr(workspace), int(workspace_bytes), _stream(stream))
    _ok(st, "attn_decode_prep_fused")


def attn_decode_workspace_init(workspace, workspace_bytes=None, stream=None) -> None:
    if workspace_bytes is None:
        workspace_bytes = workspace.numel() * workspace.element_size()
    _ok(_lib.attn_decode_workspace_init(_ptr(workspace), int(workspace_bytes), _stream(stream)),
        "attn_decode_workspace_init")


def attn_prefill(out, q, k_cache, v_cache, pos0, n_rows, n_q_heads, n_kv_heads,
                 head_dim, cache_cap, ring, window, scale, p_mode,
                 last_key=None, stream=None) -> None:
    """out/q [n_rows][Hq][D], caches [Hkv][cap][D] (bf16); last_key: None
    (causal) or a device int32 [n_rows] of each row's last key position."""
    st = _lib.attn_prefill(_ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), pos0,
                           n_rows, n_q_heads, n_kv_heads, head_dim, cache_cap, ring,
                           window, float(scale), p_mode, _ptr(last_key), _stream(stream))
    _ok(st, "attn_prefill")


def attn_cache_write(k_cache, v_cache, k, v, pos0, n_rows, n_kv_heads, head_dim,
                     cache_cap, ring, stream=None) -> None:
    """k/v [n_rows][Hkv][D] into caches [Hkv][cap][D] (bf16)."""
    st = _lib.attn_cache_write(_ptr(k_cache), _ptr(v_cache), _ptr(k), _ptr(v), pos0,
                               n_rows, n_kv_heads, head_dim, cache_cap, ring,
                               _stream(stream))
    _ok(st, "attn_cache_write")
