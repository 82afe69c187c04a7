"""Helpers shared by the GPU parity tests (not a test module).

Inputs come from ``synth`` (seeded, host-side); expected values come from the
fp64 oracle only. The HIP path is reached through the C ABI
(causal_windowed_attention_amd), never through the oracle.
"""
import sys

import numpy as np
import torch

import causal_windowed_attention_amd as cwa
import synth
from oracle import StreamSpec


def say(*a):
    """Progress line that names the case before a GPU step (flushed)."""
    print("[gpu]", *a, flush=True)
    sys.stdout.flush()


def config_for(w: synth.Workload, **kw):
    return cwa.make_config(w.batch, w.heads, w.head_dim, w.frame_h, w.frame_w,
                           w.frames_per_chunk, w.sink_chunks, w.window_chunks, dtype=w.dtype, **kw)


def spec_for(w: synth.Workload, heads=None) -> StreamSpec:
    s = StreamSpec.from_workload(w)
    if heads is not None:
        from dataclasses import replace
        s = replace(s, heads=len(heads))
    return s


def dev(x: np.ndarray, dtype: str) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    if dtype in ("bf16", "fp8"):
        t = t.to(torch.bfloat16)            # exact: the inputs are bf16-representable
    return t.cuda()


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def err(got: np.ndarray, want: np.ndarray):
    """(max abs error, relative L2 error) over the entries that are not NaN in want."""
    m = ~np.isnan(want)
    d = got[m] - want[m]
    return float(np.max(np.abs(d))), float(np.linalg.norm(d) / max(np.linalg.norm(want[m]), 1e-30))


def bf16_ulp_distance(a: torch.Tensor, b: np.ndarray) -> int:
    """Max distance in bf16 representable steps between a bf16 tensor and bf16-exact fp64 values."""
    bb = torch.from_numpy(np.ascontiguousarray(b, dtype=np.float32)).to(torch.bfloat16)
    assert torch.equal(bb.float().double(), torch.from_numpy(np.ascontiguousarray(b)).double()), \
        "expected values must be bf16-exact"

    def ordered(t):
        i = t.contiguous().view(torch.int16).to(torch.int32)
        return torch.where(i < 0, -(i & 0x7FFF), i)
    return int((ordered(a.cpu()) - ordered(bb)).abs().max().item())


# bf16 tolerances (fp32 accumulation): max abs and relative L2 must both hold
BF16_ABS, BF16_REL = 2e-2, 1e-2
F32_ABS = 1e-4
