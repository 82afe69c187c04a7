"""The fp8 variant's error budget against the fp64 definition, checked on the CPU.

fp8_pure_tolerance (gpu_util) bounds, element by element, how far an attend over E4M3-rounded
Q, K and V (plus E4M3 weights) may land from the fp64 definition. Here it is held against the
oracle alone: the storage-emulating ring oracle (exact softmax over the E4M3-rounded operands
the device stores) must stay inside the budget on every attend of a stream with a refresh, and
the budget must not be vacuous (the emulated error reaches a fair share of it).
"""
import numpy as np
import pytest

import synth
from gpu_util import fp8_pure_tolerance, spec_for
from oracle import HistoryOracle, RingOracle, fp8_q_scale

CASES = {
    "d128_s1w3": dict(heads=2, frame_h=6, frame_w=10, frames_per_chunk=3, window_chunks=3),
    "d128_s2w2": dict(heads=1, frame_h=5, frame_w=7, frames_per_chunk=2, sink_chunks=2, window_chunks=2),
}


@pytest.mark.parametrize("case", list(CASES))
def test_budget_covers_storage_emulation(case):
    w = synth.small_variant(synth.WORKLOADS["wan1.3b"], dtype="fp8", **CASES[case])
    spec = spec_for(w)
    emu, pure, hist = RingOracle(spec, storage="fp8"), RingOracle(spec), HistoryOracle(spec)
    ratios = []
    for c in range(w.sink_chunks + w.window_chunks + 3):
        if c == w.sink_chunks + w.window_chunks + 1:
            assert emu.refresh(None, 0) == pure.refresh(None, 0) == hist.refresh(None, 0)
        q, k, v = synth.chunk_qkv(w, c)
        eo, el = emu.attend(q, k, v)
        po, pl = hist.attend(q, k, v)
        tol, ltol = fp8_pure_tolerance(*pure.operands(q, k, v), spec.softmax_scale, fp8_q_scale(spec))
        r, lr = float((np.abs(eo - po) / tol).max()), float((np.abs(el - pl) / ltol).max())
        assert r <= 1.0 and lr <= 1.0, (c, r, lr)
        ratios.append(r)
        for o in (emu, pure, hist):
            o.append(k, v)
    assert max(ratios) >= 0.15, ratios          # the bound is a few sigma, not orders of magnitude
