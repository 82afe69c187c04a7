"""GPU parity of the ragged batch (sa_batch_attend): several streams, each at its own chunk
index, positions and window fill, attended in one launch. By definition the batch equals one
sa_chunk_attend per stream, so every entry is checked against its own fp64 HistoryOracle;
zero-copy commits of the staged chunks between rounds check that each entry staged its own
chunk in its own cache.
"""
import numpy as np
import pytest
import torch

import causal_windowed_attention_amd as cwa
import synth
from gpu_util import (BF16_ABS, BF16_REL, F32_ABS, check_fp8_attend, config_for, dev, err, fp8_tolerance, host,
                      say, spec_for)
from oracle import HistoryOracle, RingOracle

CASES = {
    "f32_tiny": ("tiny_f32", {}),
    "bf16_d128": ("wan1.3b", dict(heads=2, frame_h=6, frame_w=10, frames_per_chunk=3, window_chunks=3)),
    "bf16_d64_b2": ("wan1.3b", dict(batch=2, heads=2, head_dim=64, frame_h=5, frame_w=7, frames_per_chunk=2,
                                    sink_chunks=2, window_chunks=2)),
    # fp8 cache: each entry against its own fp8 storage-emulating oracle (derived tolerance)
    "fp8_d128_b2": ("wan1.3b", dict(batch=2, heads=2, frame_h=5, frame_w=7, frames_per_chunk=2,
                                    sink_chunks=1, window_chunks=2, dtype="fp8")),
}


@pytest.mark.gpu
@pytest.mark.parametrize("case", list(CASES))
def test_batch_attend_matches_per_stream_oracles(case):
    base, kw = CASES[case]
    w = synth.small_variant(synth.WORKLOADS[base], **kw)
    n = 4
    say("batch", case, w.dtype, "B", w.batch, "H", w.heads, "D", w.head_dim, "Nc", w.tokens_per_chunk,
        "S", w.sink_chunks, "W", w.window_chunks, "streams", n)
    cfg = config_for(w)
    streams = [cwa.Stream(cfg) for _ in range(n)]
    fp8 = w.dtype == "fp8"
    hists = [RingOracle(spec_for(w), storage="fp8") if fp8 else HistoryOracle(spec_for(w)) for _ in range(n)]
    seq = [0] * n

    def chunk(i):
        seq[i] += 1
        return synth.chunk_qkv(w, 1000 * i + seq[i])

    for i in range(n):                           # different states: 0, 1, 3 and 6 commits
        for _ in range((0, 1, 3, 6)[i]):
            _, k, v = chunk(i)
            streams[i].kv_append(dev(k, w.dtype), dev(v, w.dtype))
            hists[i].append(k, v)
    assert streams[2].rope_refresh(-1, 0) == hists[2].refresh(None, 0)
    for rnd in range(3):
        data = [chunk(i) for i in range(n)]
        qs, ks, vs = ([dev(d[j], w.dtype) for d in data] for j in range(3))
        outs = [torch.empty_like(x) for x in qs]
        lses = [torch.empty((w.batch, w.heads, w.tokens_per_chunk), dtype=torch.float32, device="cuda")
                for _ in range(n)]
        cwa.sa_batch_attend(streams, qs, ks, vs, outs, lses)
        torch.cuda.synchronize()
        for i in range(n):
            want, want_lse = hists[i].attend(*data[i])
            if fp8:
                tol, ltol, emu_out = fp8_tolerance(*hists[i].operands(*data[i]), spec_for(w).softmax_scale)
                check_fp8_attend(f"  round {rnd} stream {i}", outs[i], lses[i], emu_out, want_lse, tol, ltol)
                continue
            a, r = err(host(outs[i]), want)
            la, _ = err(host(lses[i]), want_lse)
            say(f"  round {rnd} stream {i} ({streams[i].query()['visible_keys']} keys): "
                f"max {a:.2e} rel {r:.2e}; lse {la:.2e}")
            if w.dtype == "bf16":
                assert a <= BF16_ABS and r <= BF16_REL and la <= BF16_ABS, (rnd, i, a, r, la)
            else:
                assert a <= F32_ABS and la <= F32_ABS, (rnd, i, a, la)
        for i in range(n):                       # commit the chunk each entry staged
            streams[i].kv_append(None, None)
            hists[i].append(data[i][1], data[i][2])
    for s in streams:
        s.close()


@pytest.mark.gpu
def test_batch_attend_full_size_sampled():
    """The launch bench.py times: eight long512p streams (H = 24, Nc = 2048, S = 1, W = 3) at 0 to 7
    commits (empty, partly filled and wrapped windows; one refreshed) in one ragged launch.
    Sampled query rows of two heads of every stream against that stream's fp64 oracle."""
    w = synth.WORKLOADS["long512p"]
    n, heads = 8, [0, w.heads - 1]
    nc = w.tokens_per_chunk
    say("batch full size long512p: streams", n, "H", w.heads, "Nc", nc, "heads checked", heads)
    cfg = config_for(w)
    streams = [cwa.Stream(cfg) for _ in range(n)]
    hists = [HistoryOracle(spec_for(w, heads)) for _ in range(n)]
    for i in range(n):
        for c in range(i):
            _, k, v = synth.chunk_qkv(w, 100 * i + c)
            streams[i].kv_append(dev(k, w.dtype), dev(v, w.dtype))
            hists[i].append(k[:, :, heads], v[:, :, heads])
    assert streams[6].rope_refresh(-1, 0) == hists[6].refresh(None, 0)
    data = [synth.chunk_qkv(w, 100 * i + 99) for i in range(n)]
    qs, ks, vs = ([dev(d[j], w.dtype) for d in data] for j in range(3))
    outs = [torch.empty_like(x) for x in qs]
    lses = [torch.empty((w.batch, w.heads, nc), dtype=torch.float32, device="cuda") for _ in range(n)]
    cwa.sa_batch_attend(streams, qs, ks, vs, outs, lses)
    torch.cuda.synchronize()
    g = np.random.default_rng(5)
    rows = np.unique(np.concatenate([np.arange(2), np.arange(nc - 2, nc), g.choice(nc, 28, replace=False)]))
    for i in range(n):
        q, k, v = (x[:, :, heads] for x in data[i])
        want, want_lse = hists[i].attend(q, k, v, rows=list(rows))
        got = host(outs[i])[:, rows][:, :, heads]
        got_lse = host(lses[i])[:, heads][:, :, rows]
        a, r = err(got, want[:, rows])
        la, _ = err(got_lse, want_lse[:, :, rows])
        say(f"  stream {i} ({streams[i].query()['visible_keys']} keys): max {a:.2e} rel {r:.2e}; lse {la:.2e}")
        assert a <= BF16_ABS and r <= BF16_REL and la <= BF16_ABS, (i, a, r, la)
    for s in streams:
        s.close()
