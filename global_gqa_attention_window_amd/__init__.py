"""Python binding of libgqa_attn.so (MI355X GQA window attention).

Argument marshalling only: each function passes tensor data pointers, sizes
and the current HIP stream to the C entry point of the same name declared in
include/gqa_attn.h, and raises AttnError on a non-zero status.  Every step of
the attention runs in the library's gfx950 kernels; there is no fallback.  If
the library has not been built, importing this package raises ImportError.

PyTorch is used for device memory and streams only.  bf16 tensors may be
torch.bfloat16 or 16-bit integer tensors holding bf16 bit patterns.  Before
each call the binding checks that every tensor it passes is contiguous, on
the current GPU, of the element size the call takes and at least as large as
the sizes given (the C ABI receives bare pointers and cannot check sizes).
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
ATTN_DECODE_COUNTER_BYTES = 262144
ATTN_DECODE_SCRATCH_BYTES = 16 << 20

_c_int, _c_void_p, _c_float, _c_size_t = ctypes.c_int, ctypes.c_void_p, ctypes.c_float, ctypes.c_size_t

_lib.attn_decode_workspace_bytes.restype = _c_size_t
_lib.attn_decode_workspace_bytes.argtypes = [_c_int] * 4
_lib.attn_decode.restype = _c_int
_lib.attn_decode.argtypes = ([_c_void_p] * 5 + [_c_int] * 7 + [_c_float, _c_void_p, _c_size_t, _c_void_p])
_lib.attn_decode_noalloc.restype = _c_int
_lib.attn_decode_noalloc.argtypes = [_c_void_p] * 5 + [_c_int] * 7 + [_c_float, _c_void_p]
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
_lib.attn_prefill_workspace_bytes.restype = _c_size_t
_lib.attn_prefill_workspace_bytes.argtypes = [_c_int] * 3
_lib.attn_prefill_ws.restype = _c_int
_lib.attn_prefill_ws.argtypes = ([_c_void_p] * 4 + [_c_int] * 8 +
                                 [_c_float, _c_int, _c_void_p, _c_void_p, _c_size_t, _c_void_p])
_lib.attn_prefill_prompt_workspace_bytes.restype = _c_size_t
_lib.attn_prefill_prompt_workspace_bytes.argtypes = [_c_int] * 6
_lib.attn_prefill_prompt.restype = _c_int
_lib.attn_prefill_prompt.argtypes = ([_c_void_p] * 6 + [_c_int] * 9 +
                                     [_c_float, _c_int, _c_void_p, _c_void_p, _c_size_t, _c_void_p])
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


def _arg(t, name: str, numel: int, esize: int = 2):
    """Data pointer of a tensor on the current GPU that holds at least
    `numel` contiguous elements of `esize` bytes, checked here because the C
    ABI receives bare pointers and cannot.  None passes through as NULL (the
    library refuses it where the call needs the buffer)."""
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch.Tensor, got {type(t).__name__}")
    if t.device.type != "cuda" or t.get_device() != torch.cuda.current_device():
        raise ValueError(f"{name}: on {t.device}, not the current GPU")
    if t.element_size() != esize:
        raise ValueError(f"{name}: {t.dtype} has {t.element_size()}-byte elements, "
                         f"expected {esize}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: not contiguous")
    if t.numel() < numel:
        raise ValueError(f"{name}: {t.numel()} elements, the sizes given need {numel}")
    return t.data_ptr()


def _ws(workspace, workspace_bytes):
    """Pointer and byte count of a workspace tensor; an explicit byte count
    may not exceed the tensor."""
    if workspace is None:
        return None, int(workspace_bytes or 0)
    if not isinstance(workspace, torch.Tensor):
        raise TypeError(f"workspace: expected a torch.Tensor, got {type(workspace).__name__}")
    have = workspace.numel() * workspace.element_size()
    if workspace_bytes is None:
        workspace_bytes = have
    if workspace_bytes > have:
        raise ValueError(f"workspace: {have} bytes, workspace_bytes says {workspace_bytes}")
    return _arg(workspace, "workspace", 0, workspace.element_size()), int(workspace_bytes)


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
    nq, nc = n_seq * n_q_heads * head_dim, n_seq * n_kv_heads * cache_cap * head_dim
    wp, wb = _ws(workspace, workspace_bytes)
    st = _lib.attn_decode(_arg(out, "out", nq), _arg(q, "q", nq), _arg(k_cache, "k_cache", nc),
                          _arg(v_cache, "v_cache", nc), _arg(pos, "pos", n_seq, 4),
                          n_seq, n_q_heads, n_kv_heads, head_dim, cache_cap, ring,
                          window, float(scale), wp, wb, _stream(stream))
    _ok(st, "attn_decode")


def attn_decode_noalloc(out, q, k_cache, v_cache, pos, n_seq, n_q_heads, n_kv_heads,
                        head_dim, cache_cap, ring, window, scale, stream=None) -> None:
    """attn_decode with its partials in the library's own device array (no
    workspace, nothing allocated); calls that overlap on one GPU race."""
    nq, nc = n_seq * n_q_heads * head_dim, n_seq * n_kv_heads * cache_cap * head_dim
    st = _lib.attn_decode_noalloc(_arg(out, "out", nq), _arg(q, "q", nq),
                                  _arg(k_cache, "k_cache", nc), _arg(v_cache, "v_cache", nc),
                                  _arg(pos, "pos", n_seq, 4), n_seq, n_q_heads, n_kv_heads,
                                  head_dim, cache_cap, ring, window, float(scale),
                                  _stream(stream))
    _ok(st, "attn_decode_noalloc")


def attn_decode_rows(out, q, k_cache, v_cache, pos, n_seq, rows, n_q_heads, n_kv_heads,
                     head_dim, cache_cap, ring, window, scale, workspace,
                     workspace_bytes=None, stream=None) -> None:
    """out/q [S][rows][Hq][D], caches [S][Hkv][cap][D] (bf16), pos int32 [S]
    (the first row's position)."""
    nq, nc = n_seq * rows * n_q_heads * head_dim, n_seq * n_kv_heads * cache_cap * head_dim
    wp, wb = _ws(workspace, workspace_bytes)
    st = _lib.attn_decode_rows(_arg(out, "out", nq), _arg(q, "q", nq),
                               _arg(k_cache, "k_cache", nc), _arg(v_cache, "v_cache", nc),
                               _arg(pos, "pos", n_seq, 4), n_seq, rows, n_q_heads, n_kv_heads,
                               head_dim, cache_cap, ring, window, float(scale), wp, wb,
                               _stream(stream))
    _ok(st, "attn_decode_rows")


def attn_decode_rows_fused(out, q, k_cache, v_cache, pos, n_seq, rows, n_q_heads, n_kv_heads,
                           head_dim, cache_cap, ring, window, scale, workspace,
                           workspace_bytes=None, stream=None) -> None:
    """attn_decode_rows in one launch where it can; the workspace starts with
    ATTN_DECODE_COUNTER_BYTES of counters set up by attn_decode_workspace_init."""
    nq, nc = n_seq * rows * n_q_heads * head_dim, n_seq * n_kv_heads * cache_cap * head_dim
    wp, wb = _ws(workspace, workspace_bytes)
    st = _lib.attn_decode_rows_fused(_arg(out, "out", nq), _arg(q, "q", nq),
                                     _arg(k_cache, "k_cache", nc), _arg(v_cache, "v_cache", nc),
                                     _arg(pos, "pos", n_seq, 4), n_seq, rows, n_q_heads,
                                     n_kv_heads, head_dim, cache_cap, ring, window,
                                     float(scale), wp, wb, _stream(stream))
    _ok(st, "attn_decode_rows_fused")


def attn_qkv_prep(q_out, k_cache, v_cache, qkv, q_norm_w, k_norm_w, inv_freq, eps, v_norm,
                  pos, n_seq, n_q_heads, n_kv_heads, head_dim, cache_cap, ring,
                  stream=None) -> None:
    """qkv [S][(Hq + 2 Hkv) D] bf16 -> q_out [S][Hq][D], key/value at each
    row's cache slot; inv_freq fp32 [D/2]."""
    nq, nc = n_seq * n_q_heads * head_dim, n_seq * n_kv_heads * cache_cap * head_dim
    nx = n_seq * (n_q_heads + 2 * n_kv_heads) * head_dim
    st = _lib.attn_qkv_prep(_arg(q_out, "q_out", nq), _arg(k_cache, "k_cache", nc),
                            _arg(v_cache, "v_cache", nc), _arg(qkv, "qkv", nx),
                            _arg(q_norm_w, "q_norm_w", head_dim),
                            _arg(k_norm_w, "k_norm_w", head_dim),
                            _arg(inv_freq, "inv_freq", head_dim // 2, 4), float(eps),
                            int(v_norm), _arg(pos, "pos", n_seq, 4), n_seq, n_q_heads,
                            n_kv_heads, head_dim, cache_cap, ring, _stream(stream))
    _ok(st, "attn_qkv_prep")


def attn_decode_prep_fused(out, qkv, q_norm_w, k_norm_w, inv_freq, eps, v_norm, k_cache,
                           v_cache, pos, n_seq, n_q_heads, n_kv_heads, head_dim, cache_cap,
                           ring, window, scale, workspace, workspace_bytes=None,
                           stream=None) -> None:
    """attn_qkv_prep + one-row attn_decode_rows_fused in the decode kernel."""
    nq, nc = n_seq * n_q_heads * head_dim, n_seq * n_kv_heads * cache_cap * head_dim
    nx = n_seq * (n_q_heads + 2 * n_kv_heads) * head_dim
    wp, wb = _ws(workspace, workspace_bytes)
    st = _lib.attn_decode_prep_fused(_arg(out, "out", nq), _arg(qkv, "qkv", nx),
                                     _arg(q_norm_w, "q_norm_w", head_dim),
                                     _arg(k_norm_w, "k_norm_w", head_dim),
                                     _arg(inv_freq, "inv_freq", head_dim // 2, 4), float(eps),
                                     int(v_norm), _arg(k_cache, "k_cache", nc),
                                     _arg(v_cache, "v_cache", nc), _arg(pos, "pos", n_seq, 4),
                                     n_seq, n_q_heads, n_kv_heads, head_dim, cache_cap, ring,
                                     window, float(scale), wp, wb, _stream(stream))
    _ok(st, "attn_decode_prep_fused")


def attn_decode_workspace_init(workspace, workspace_bytes=None, stream=None) -> None:
    wp, wb = _ws(workspace, workspace_bytes)
    _ok(_lib.attn_decode_workspace_init(wp, wb, _stream(stream)), "attn_decode_workspace_init")


def attn_prefill(out, q, k_cache, v_cache, pos0, n_rows, n_q_heads, n_kv_heads,
                 head_dim, cache_cap, ring, window, scale, p_mode,
                 last_key=None, stream=None) -> None:
    """out/q [n_rows][Hq][D], caches [Hkv][cap][D] (bf16); last_key: None
    (causal) or a device int32 [n_rows] of each row's last key position."""
    nq, nc = n_rows * n_q_heads * head_dim, n_kv_heads * cache_cap * head_dim
    st = _lib.attn_prefill(_arg(out, "out", nq), _arg(q, "q", nq), _arg(k_cache, "k_cache", nc),
                           _arg(v_cache, "v_cache", nc), pos0, n_rows, n_q_heads, n_kv_heads,
                           head_dim, cache_cap, ring, window, float(scale), p_mode,
                           _arg(last_key, "last_key", n_rows, 4), _stream(stream))
    _ok(st, "attn_prefill")


def attn_prefill_workspace_bytes(n_rows, n_q_heads, head_dim) -> int:
    return _lib.attn_prefill_workspace_bytes(n_rows, n_q_heads, head_dim)


def attn_prefill_ws(out, q, k_cache, v_cache, pos0, n_rows, n_q_heads, n_kv_heads,
                    head_dim, cache_cap, ring, window, scale, p_mode, workspace,
                    last_key=None, stream=None) -> None:
    """attn_prefill with a device workspace (uint8, attn_prefill_workspace_bytes
    bytes; None gives attn_prefill): a short chunk's key blocks may split over
    several workgroups, joined by a merge launch."""
    nq, nc = n_rows * n_q_heads * head_dim, n_kv_heads * cache_cap * head_dim
    ws, wsb = _ws(workspace, None)
    st = _lib.attn_prefill_ws(_arg(out, "out", nq), _arg(q, "q", nq),
                              _arg(k_cache, "k_cache", nc), _arg(v_cache, "v_cache", nc),
                              pos0, n_rows, n_q_heads, n_kv_heads, head_dim, cache_cap, ring,
                              window, float(scale), p_mode, _arg(last_key, "last_key", n_rows, 4),
                              ws, wsb, _stream(stream))
    _ok(st, "attn_prefill_ws")


def attn_prefill_prompt_workspace_bytes(pos0, n_rows, n_kv_heads, head_dim, ring, window) -> int:
    return _lib.attn_prefill_prompt_workspace_bytes(pos0, n_rows, n_kv_heads, head_dim, ring,
                                                    window)


def attn_prefill_prompt(out, q, k, v, k_cache, v_cache, pos0, n_rows, chunk, n_q_heads,
                        n_kv_heads, head_dim, cache_cap, ring, window, scale, p_mode,
                        workspace=None, last_key=None, stream=None) -> None:
    """A whole prompt with the bits of cache write + attention chunk by chunk
    (`chunk` rows each), in one attention launch: out/q [n_rows][Hq][D], k/v
    [n_rows][Hkv][D], caches [Hkv][cap][D] (bf16); workspace (uint8,
    attn_prefill_prompt_workspace_bytes) for a ring, None for a linear cache."""
    nq, nk = n_rows * n_q_heads * head_dim, n_rows * n_kv_heads * head_dim
    nc = n_kv_heads * cache_cap * head_dim
    ws, wsb = _ws(workspace, None)
    st = _lib.attn_prefill_prompt(_arg(out, "out", nq), _arg(q, "q", nq), _arg(k, "k", nk),
                                  _arg(v, "v", nk), _arg(k_cache, "k_cache", nc),
                                  _arg(v_cache, "v_cache", nc), pos0, n_rows, chunk, n_q_heads,
                                  n_kv_heads, head_dim, cache_cap, ring, window, float(scale),
                                  p_mode, _arg(last_key, "last_key", n_rows, 4), ws, wsb,
                                  _stream(stream))
    _ok(st, "attn_prefill_prompt")


def attn_cache_write(k_cache, v_cache, k, v, pos0, n_rows, n_kv_heads, head_dim,
                     cache_cap, ring, stream=None) -> None:
    """k/v [n_rows][Hkv][D] into caches [Hkv][cap][D] (bf16)."""
    nc, nk = n_kv_heads * cache_cap * head_dim, n_rows * n_kv_heads * head_dim
    st = _lib.attn_cache_write(_arg(k_cache, "k_cache", nc), _arg(v_cache, "v_cache", nc),
                               _arg(k, "k", nk), _arg(v, "v", nk), pos0, n_rows, n_kv_heads,
                               head_dim, cache_cap, ring, _stream(stream))
    _ok(st, "attn_cache_write")
