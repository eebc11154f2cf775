"""attn_decode_noalloc (partials in the library's own device array, no
workspace) against attn_decode (caller's workspace), bit for bit, on two calls
in a row whose second is smaller, then the first shape again."""
import numpy as np
import pytest
import torch

from gpu_util import DEV, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ga():
    import global_gqa_attention_window_amd as ga
    return ga


def _case(seed, S, Hq, Hkv, D, cap, ring, window, pos):
    g = torch.Generator(device=DEV).manual_seed(seed)
    q = torch.randn((S, Hq, D), generator=g, device=DEV, dtype=torch.bfloat16)
    k = torch.randn((S, Hkv, cap, D), generator=g, device=DEV, dtype=torch.bfloat16)
    v = torch.randn((S, Hkv, cap, D), generator=g, device=DEV, dtype=torch.bfloat16)
    p = torch.tensor(pos, dtype=torch.int32, device=DEV)
    return q, k, v, p


def _both(ga, args, S, Hq, Hkv, D, cap, ring, window, scale):
    q, k, v, p = args
    ref = torch.empty_like(q)
    ws = torch.empty(ga.attn_decode_workspace_bytes(S, Hq, D, cap), dtype=torch.uint8,
                     device=DEV)
    ga.attn_decode(ref, q, k, v, p, S, Hq, Hkv, D, cap, ring, window, scale, ws)
    out = torch.full_like(q, float("nan"))
    ga.attn_decode_noalloc(out, q, k, v, p, S, Hq, Hkv, D, cap, ring, window, scale)
    torch.cuda.synchronize()
    return ref.view(torch.int16).cpu().numpy(), out.view(torch.int16).cpu().numpy()


def test_noalloc_decode_equals_attn_decode(ga):
    big = dict(S=4, Hq=32, Hkv=2, D=512, cap=32768, ring=0, window=0)
    small = dict(S=2, Hq=8, Hkv=1, D=256, cap=1024, ring=1, window=1024)
    cases = [("32768-key global decode, 4 streams", 301, big, [32767, 20000, 5, 32000], 0.0442),
             ("1024-slot sliding ring, 2 streams", 302, small, [4095, 1500], 0.0625),
             ("32768-key global decode again", 303, big, [100, 32767, 12345, 2047], 0.0442)]
    for name, seed, shp, pos, scale in cases:
        say("noalloc decode:", name)
        args = _case(seed, pos=pos, **shp)
        ref, got = _both(ga, args, scale=scale, **shp)
        assert np.array_equal(ref, got), name
        del args
    torch.cuda.empty_cache()


def test_noalloc_decode_refuses_partials_past_its_array(ga):
    # refused before any device work: 8 streams x 32 heads x 32 runs at D = 512
    # (the binding would refuse the small tensors first, so the C ABI is called)
    q = torch.empty((8, 32, 512), dtype=torch.bfloat16, device=DEV)
    k = torch.empty((8, 2, 1, 512), dtype=torch.bfloat16, device=DEV)
    p = torch.zeros(8, dtype=torch.int32, device=DEV)
    st = ga._lib.attn_decode_noalloc(q.data_ptr(), q.data_ptr(), k.data_ptr(), k.data_ptr(),
                                     p.data_ptr(), 8, 32, 2, 512, 65536, 0, 0, 0.044, None)
    assert ga.attn_status_string(st) == "ATTN_E_WORKSPACE"
