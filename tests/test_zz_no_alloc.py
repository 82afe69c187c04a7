"""The workspace-free GDN forward (sa_gdn_forward_noalloc) against the workspace forward.

Both run the same kernels; only the scratch differs (a fixed device array inside the library
instead of the caller's workspace), so the outputs and final states must be identical, bit for
bit, on every call. Two calls in a row, the second with a smaller input (the scratch keeps the
first call's contents), then sizes beyond SA_GDN_SCRATCH_BYTES are refused before any device
work. The calls go through the C ABI (the binding only marshals pointers).
"""
import numpy as np
import pytest
import torch

import causal_windowed_attention_amd as cwa
import synth
from causal_windowed_attention_amd import _lib as L
from gpu_util import say

pytestmark = pytest.mark.gpu


def _dev(x, bf16):
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return (t.to(torch.bfloat16) if bf16 else t).cuda()


def _both(B, N, H, D, seed):
    q, k, v, a, b_, s0 = synth.gdn_inputs(B, N, H, D, seed=seed)
    q, k, v = (_dev(x, True) for x in (q, k, v))
    a, b_, s0 = (_dev(x, False) for x in (a, b_, s0))
    need = cwa.sa_gdn_workspace_bytes(B, N, H, D)
    assert 0 < need <= L.SA_GDN_SCRATCH_BYTES
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    out_ws, st_ws = torch.empty_like(v), torch.empty_like(s0)
    out_na, st_na = torch.full_like(v, float("nan")), torch.full_like(s0, float("nan"))
    cwa.sa_gdn_forward(B, N, H, D, q, k, v, a, b_, s0, st_ws, out_ws, ws, need)
    cwa.sa_gdn_forward_noalloc(B, N, H, D, q, k, v, a, b_, s0, st_na, out_na)
    torch.cuda.synchronize()
    return out_ws, st_ws, out_na, st_na


@pytest.mark.parametrize("first,second", [((1, 1000, 4, 128), (1, 300, 2, 128)),
                                          ((2, 500, 3, 64), (1, 70, 1, 64))])
def test_noalloc_equals_workspace_forward(first, second):
    for i, (B, N, H, D) in enumerate((first, second)):
        say(f"gdn noalloc call {i}: B {B} N {N} H {H} D {D}")
        out_ws, st_ws, out_na, st_na = _both(B, N, H, D, seed=17 + i)
        assert torch.equal(out_ws, out_na), "outputs differ"
        assert torch.equal(st_ws, st_na), "final states differ"
        assert torch.isfinite(out_na.float()).all()


def test_noalloc_refuses_sizes_beyond_the_scratch():
    B, H, D = 1, 16, 128
    per_token = cwa.sa_gdn_workspace_bytes(B, 6400, H, D) / 6400.0
    N = int(L.SA_GDN_SCRATCH_BYTES / per_token) + 200
    assert cwa.sa_gdn_workspace_bytes(B, N, H, D) > L.SA_GDN_SCRATCH_BYTES
    t = torch.zeros(16, dtype=torch.float32, device="cuda")   # never read: refused before any launch
    with pytest.raises(cwa.SaError) as e:
        cwa.sa_gdn_forward_noalloc(B, N, H, D, t, t, t, t, t, None, t, t)
    assert e.value.status == L.SA_ERR_WORKSPACE_TOO_SMALL
