"""GPU parity of the buffer attend (sa_buffer_attend) against the fp64 oracle, in both modes.

The oracle's HistoryOracle.buffer_attend is the definition (moving buffer: each buffer chunk
sees what an attend would show it after the earlier buffer chunks were committed; steps: each
sees the committed context and itself); it is pinned in tests/test_oracle_stream.py against
explicitly enumerated windows. Streams are driven
through commits, refreshes and buffers of several sizes, so the key segments cover the
sink, wrapped and unwrapped ring ranges and buffer ranges whose chunk boundaries cut
64-key tiles (Nc not a multiple of 64).
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
    # name: (base workload, overrides, max_buffer_chunks)
    "f32_tiny": ("tiny_f32", {}, 4),
    "bf16_d128": ("wan1.3b", dict(heads=2, frame_h=6, frame_w=10, frames_per_chunk=3, window_chunks=3), 5),
    "bf16_d64": ("wan1.3b", dict(heads=2, head_dim=64, frame_h=5, frame_w=7, frames_per_chunk=2,
                                 sink_chunks=2, window_chunks=2), 4),
    "bf16_w0": ("wan1.3b", dict(heads=1, frame_h=4, frame_w=9, frames_per_chunk=2, window_chunks=0), 3),
    "bf16_s0": ("wan1.3b", dict(heads=1, frame_h=4, frame_w=9, frames_per_chunk=2, sink_chunks=0,
                                window_chunks=2), 3),
    # fp8 cache: judged against the fp8 storage-emulating oracle with the derived tolerance
    "fp8_d128": ("wan1.3b", dict(heads=2, frame_h=6, frame_w=10, frames_per_chunk=3, window_chunks=3,
                                 dtype="fp8"), 5),
}


def _buffer(w, first, n):
    parts = [synth.chunk_qkv(w, first + j) for j in range(n)]
    return [np.concatenate([p[i] for p in parts], axis=1) for i in range(3)]


def _check(w, got, want, got_lse, want_lse, what):
    a, r = err(host(got), want)
    la, _ = err(host(got_lse), want_lse)
    say(f"  {what}: max {a:.2e} rel {r:.2e}; lse {la:.2e}")
    if w.dtype == "bf16":
        assert a <= BF16_ABS and r <= BF16_REL and la <= BF16_ABS, (what, a, r, la)
    else:
        assert a <= F32_ABS and la <= F32_ABS, (what, a, la)


@pytest.mark.gpu
@pytest.mark.parametrize("steps", [False, True])
@pytest.mark.parametrize("case", list(CASES))
def test_buffer_attend_matches_oracle(case, steps):
    base, kw, nb = CASES[case]
    w = synth.small_variant(synth.WORKLOADS[base], **kw)
    say("buffer", case, "steps" if steps else "banded", w.dtype, "H", w.heads, "D", w.head_dim, "Nc", w.tokens_per_chunk,
        "S", w.sink_chunks, "W", w.window_chunks, "NB", nb)
    s = cwa.Stream(config_for(w, max_buffer_chunks=nb))
    spec = spec_for(w)
    hist = HistoryOracle(spec)
    emu = RingOracle(spec, storage="fp8") if w.dtype == "fp8" else None
    state = {"c": 0}

    def commit(k_times):
        for _ in range(k_times):
            _, k, v = synth.chunk_qkv(w, state["c"])
            s.kv_append(dev(k, w.dtype), dev(v, w.dtype))
            hist.append(k, v)
            if emu is not None:
                emu.append(k, v)
            state["c"] += 1

    def check(out, lse, q, k, v, what, steps_mode, n):
        if emu is None:
            want, want_lse = hist.buffer_attend(q, k, v, steps=steps_mode)
            _check(w, out, want, lse, want_lse, what)
            return
        nc = w.tokens_per_chunk
        want_lse = emu.buffer_attend(q, k, v, steps=steps_mode)[1]
        for j, (qrot, keys, vals) in enumerate(emu.buffer_operands(q, k, v, steps=steps_mode)):
            tol, ltol, emu_out = fp8_tolerance(qrot, keys, vals, spec.softmax_scale)
            sl = slice(j * nc, (j + 1) * nc)
            check_fp8_attend(f"{what}, chunk {j}", out[:, sl], lse[:, :, sl], emu_out, want_lse[:, :, sl],
                             tol, ltol)

    # a moving-buffer attend needs a full sink; steps start with nothing committed
    schedule = [(0 if steps else w.sink_chunks, 1), (0, nb), (1, 2), ("refresh", None), (1, nb),
                (w.window_chunks + 2, nb), (1, max(1, nb - 2)), (2, nb)]
    for i, (commits, n) in enumerate(schedule):
        if commits == "refresh":
            assert s.rope_refresh(-1, 0) == hist.refresh(None, 0)
            if emu is not None:
                emu.refresh(None, 0)
            continue
        commit(commits)
        q, k, v = _buffer(w, 500 + 10 * i, n)
        lse = torch.empty((w.batch, w.heads, n * w.tokens_per_chunk), dtype=torch.float32, device="cuda")
        out = s.buffer_attend(dev(q, w.dtype), dev(k, w.dtype), dev(v, w.dtype), lse=lse, steps=steps)
        torch.cuda.synchronize()
        check(out, lse, q, k, v, f"step {i}: {commits} commits then a buffer of {n}", steps, n)
        assert s.query()["staged_valid"] == 0
    # an ordinary attend afterwards is unaffected by the buffer slots
    q, k, v = synth.chunk_qkv(w, 900)
    lse = torch.empty((w.batch, w.heads, w.tokens_per_chunk), dtype=torch.float32, device="cuda")
    out = s.chunk_attend(dev(q, w.dtype), dev(k, w.dtype), dev(v, w.dtype), lse=lse)
    torch.cuda.synchronize()
    check(out, lse, q, k, v, "chunk attend after the buffers", False, 1)
    s.close()


@pytest.mark.gpu
@pytest.mark.parametrize("steps", [False, True])
def test_buffer_attend_full_size_sampled(steps):
    """long512p shape (H = 24, Nc = 2048, S = 1, W = 3) with a buffer of 4 chunks: sampled
    rows of two heads against the oracle, after the ring has wrapped."""
    w = synth.WORKLOADS["long512p"]
    nb = 4
    s = cwa.Stream(config_for(w, max_buffer_chunks=nb))
    hist = HistoryOracle(spec_for(w))
    for c in range(w.sink_chunks + w.window_chunks + 2):
        _, k, v = synth.chunk_qkv(w, c)
        s.kv_append(dev(k, w.dtype), dev(v, w.dtype))
        hist.append(k, v)
    q, k, v = _buffer(w, 700, nb)
    lse = torch.empty((w.batch, w.heads, nb * w.tokens_per_chunk), dtype=torch.float32, device="cuda")
    out = s.buffer_attend(dev(q, w.dtype), dev(k, w.dtype), dev(v, w.dtype), lse=lse, steps=steps)
    torch.cuda.synchronize()
    nc = w.tokens_per_chunk
    g = np.random.default_rng(5)
    rows = sorted(set(int(x) for x in g.integers(0, nb * nc, 96)) | {0, nc - 1, nc, nb * nc - 1})
    heads = [0, w.heads - 1]
    want, want_lse = hist.buffer_attend(q, k, v, rows=rows, heads=heads, steps=steps)
    got = host(out)[:, rows][:, :, heads]
    a, r = err(got, want[:, rows][:, :, heads])
    la, _ = err(host(lse)[:, heads][:, :, rows], want_lse[:, heads][:, :, rows])
    say(f"  long512p {'steps' if steps else 'buffer'} of {nb}: sampled max {a:.2e} rel {r:.2e}; lse {la:.2e}")
    assert a <= BF16_ABS and r <= BF16_REL and la <= BF16_ABS
    s.close()


@pytest.mark.gpu
def test_largest_cache_region():
    """A cache region per (b, h) just under the 2^31 bytes the kernels address with 32-bit buffer
    offsets: Nc = 65536 (one 256 x 256 frame), S = 1, W = 123 and two buffer chunks make 127 slots,
    127 * 65536 * 128 * 2 = 2.13e9 bytes of K and as many of V^T per (b, h). The V^T rows of the high
    channels start near the bound for every attend, and the buffer chunks take the last two slots, so
    their K rows sit there too. Sampled rows of a chunk attend and of a two-chunk buffer attend are
    checked against the oracle."""
    w = synth.small_variant(synth.WORKLOADS["wan1.3b"], name="largest_region", batch=1, heads=2, frame_h=256,
                            frame_w=256, frames_per_chunk=1, sink_chunks=1, window_chunks=123)
    nb, nc = 2, w.tokens_per_chunk
    cfg = config_for(w, max_buffer_chunks=nb)
    slots = w.sink_chunks + w.window_chunks + 1 + nb
    assert slots * nc * w.head_dim * 2 < 2 ** 31 <= (slots + 1) * nc * w.head_dim * 2
    say("largest region: Nc", nc, "slots", slots, "workspace GB", cwa.sa_workspace_bytes(cfg) / 1e9)
    s = cwa.Stream(cfg)
    hist = HistoryOracle(spec_for(w))
    for c in range(3):                                # the sink and two window chunks
        _, k, v = synth.chunk_qkv(w, c)
        s.kv_append(dev(k, w.dtype), dev(v, w.dtype))
        hist.append(k, v)
    g = np.random.default_rng(11)
    q, k, v = synth.chunk_qkv(w, 3)
    out = s.chunk_attend(dev(q, w.dtype), dev(k, w.dtype), dev(v, w.dtype))
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([np.arange(4), np.arange(nc - 4, nc), g.choice(nc, 40, replace=False)]))
    want, _ = hist.attend(q, k, v, rows=rows)
    a, r = err(host(out[:, torch.as_tensor(rows, device=out.device)]), want[:, rows])
    say(f"  chunk attend: max {a:.2e} rel {r:.2e}")
    assert a <= BF16_ABS and r <= BF16_REL, (a, r)
    q, k, v = _buffer(w, 40, nb)
    out = s.buffer_attend(dev(q, w.dtype), dev(k, w.dtype), dev(v, w.dtype))
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([np.arange(4), np.arange(nb * nc - 4, nb * nc), [nc - 1, nc],
                                     g.choice(nb * nc, 40, replace=False)]))
    want, _ = hist.buffer_attend(q, k, v, rows=rows)
    a, r = err(host(out[:, torch.as_tensor(rows, device=out.device)]), want[:, rows])
    say(f"  buffer attend (slots {slots - nb}, {slots - 1}): max {a:.2e} rel {r:.2e}")
    assert a <= BF16_ABS and r <= BF16_REL, (a, r)
    s.close()
