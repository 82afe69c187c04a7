"""The C ABI from plain C: tests/c_abi/sa_c_demo (a C program linked against libsa.so
and the HIP runtime only, no Python in its process) runs a bf16 stream over chunk files
written here; its outputs and log-sum-exps are held against the fp64 oracle with the
same bf16 bar as the Python-path parity tests (max abs 2e-2 and relative L2 1e-2 against
the pure oracle; the storage-emulating oracle's error is printed)."""
import os
import subprocess

import numpy as np
import pytest

import synth
from causal_windowed_attention_amd import build as _build
from gpu_util import BF16_ABS, BF16_REL, err, say, spec_for
from oracle import HistoryOracle, RingOracle

pytestmark = pytest.mark.gpu

# two streams, three heads, a ragged last query tile (Nc = 105), one sink chunk and a window
# of two that wraps before the end
W = synth.Workload(name="c_abi_bf16", cfg_id=131, batch=2, heads=3, head_dim=128, frame_h=5, frame_w=7,
                   frames_per_chunk=3, sink_chunks=1, window_chunks=2, n_chunks=6)


def _bf16_bits(x):
    a = np.ascontiguousarray(x, dtype=np.float32)
    bits = a.view(np.uint32)
    assert not np.any(bits & 0xFFFF), "inputs must be bf16-exact"
    return (bits >> 16).astype(np.uint16)


def test_c_program_stream_matches_oracle(tmp_path):
    assert os.path.exists(_build.C_DEMO), "tests/c_abi/sa_c_demo is missing: run __graft_entry__.build()"
    nc = W.tokens_per_chunk
    chunks = [synth.chunk_qkv(W, c) for c in range(W.n_chunks)]
    for c, (q, k, v) in enumerate(chunks):
        for name, x in (("q", q), ("k", k), ("v", v)):
            _bf16_bits(x).tofile(tmp_path / f"{name}{c}.bin")
    args = [_build.C_DEMO, str(tmp_path)] + [str(a) for a in (W.batch, W.heads, W.head_dim, W.frame_h, W.frame_w,
                                                              W.frames_per_chunk, W.sink_chunks, W.window_chunks,
                                                              W.n_chunks)]
    say("c_abi program:", " ".join(args[1:]))
    r = subprocess.run(args, capture_output=True, text=True, timeout=120)
    say("  exit", r.returncode, r.stdout.strip(), r.stderr.strip())
    assert r.returncode == 0, r.stderr
    hist, ring = HistoryOracle(spec_for(W)), RingOracle(spec_for(W), storage="bf16")
    for c, (q, k, v) in enumerate(chunks):
        want, want_lse = hist.attend(q, k, v)
        emu, _ = ring.attend(q, k, v)
        out = np.fromfile(tmp_path / f"out{c}.bin", dtype=np.uint16).astype(np.uint32) << 16
        got = out.view(np.float32).astype(np.float64).reshape(W.batch, nc, W.heads, W.head_dim)
        lse = np.fromfile(tmp_path / f"lse{c}.bin", dtype=np.float32).astype(np.float64)
        lse = lse.reshape(W.batch, W.heads, nc)
        a, rel = err(got, want)
        ae, re_ = err(got, emu)
        la, _ = err(lse, want_lse)
        say(f"  chunk {c}: vs fp64 max {a:.2e} rel {rel:.2e}; vs storage max {ae:.2e} rel {re_:.2e}; lse {la:.2e}")
        assert a <= BF16_ABS and rel <= BF16_REL, (c, a, rel)
        assert la <= BF16_ABS, (c, la)
        hist.append(k, v)
        ring.append(k, v)
    expect_keys = (W.sink_chunks + W.window_chunks + 1) * nc
    assert f"visible_keys {expect_keys}" in r.stdout, r.stdout
