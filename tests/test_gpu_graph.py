"""HIP graph capture of the attend of one chunk.

Within a chunk the denoising steps call sa_chunk_attend again at unchanged positions, so a
caller may capture that call once and replay it per step with new q, k, v in the same
buffers. The attend path launches kernels only (RoPE write, attention, and the combine pass
when the key range is split), no memset or copy nodes. The captured call is replayed for
several data sets, with the program's own eager work and synchronisations between replays,
and every replay must equal the eager call bit for bit (the kernels are deterministic); the
eager results are themselves held against the fp64 oracle.
"""
import numpy as np
import pytest
import torch

import causal_windowed_attention_amd as cwa
import synth
from gpu_util import BF16_ABS, BF16_REL, config_for, dev, err, host, say, spec_for
from oracle import HistoryOracle

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("splits", [0, 2])
def test_captured_attend_replays_match_eager(splits):
    w = synth.small_variant(synth.WORKLOADS["wan1.3b"], heads=2, frame_h=6, frame_w=10, frames_per_chunk=3,
                            window_chunks=3)
    say("graph capture: H", w.heads, "Nc", w.tokens_per_chunk, "splits", splits or "auto")
    s = cwa.Stream(config_for(w))
    if splits:
        s.set_option(cwa.SA_OPT_KV_SPLITS, splits)
    hist = HistoryOracle(spec_for(w))
    for c in range(5):                           # sink full, window wrapped
        _, k, v = synth.chunk_qkv(w, c)
        s.kv_append(dev(k, w.dtype), dev(v, w.dtype))
        hist.append(k, v)
    steps = [synth.chunk_qkv(w, 100 + j) for j in range(3)]    # the denoising steps of chunk 5
    nc = w.tokens_per_chunk
    q_s, k_s, v_s = (torch.empty((w.batch, nc, w.heads, w.head_dim), dtype=torch.bfloat16, device="cuda")
                     for _ in range(3))
    out_s = torch.empty_like(q_s)
    lse_s = torch.empty((w.batch, w.heads, nc), dtype=torch.float32, device="cuda")

    def load(j):
        for dst, x in zip((q_s, k_s, v_s), steps[j]):
            dst.copy_(dev(x, w.dtype))

    eager = []
    for j in range(len(steps)):
        load(j)
        o = s.chunk_attend(q_s, k_s, v_s, lse=lse_s)
        torch.cuda.synchronize()
        eager.append((o.clone(), lse_s.clone()))
        want, want_lse = hist.attend(*steps[j])
        a, r = err(host(o), want)
        la, _ = err(host(lse_s), want_lse)
        say(f"  eager step {j}: max {a:.2e} rel {r:.2e}; lse {la:.2e}")
        assert a <= BF16_ABS and r <= BF16_REL and la <= BF16_ABS
    plan = s.query()
    load(0)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        s.chunk_attend(q_s, k_s, v_s, out=out_s, lse=lse_s)
    assert s.query() == plan                      # capturing changed no stream state
    for rep in range(2):
        for j in range(len(steps)):
            load(j)                              # eager work between replays
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            same = torch.equal(out_s, eager[j][0]) and torch.equal(lse_s, eager[j][1])
            say(f"  replay {rep} step {j}: identical to eager: {same}")
            assert same, (rep, j)
    say("  launch plan: q tiles", plan["last_q_tiles"], "key splits", plan["last_kv_splits"])
    if splits:
        assert plan["last_kv_splits"] == splits
    s.close()


def test_captured_gdn_forward_carries_state_like_eager():
    """sa_gdn_forward keeps no host state: a captured call, replayed over consecutive chunks
    with the state carried in place, equals the same calls made eagerly (bit for bit)."""
    B, N, H, D = 1, 150, 2, 128
    say("graph capture: gdn_forward B", B, "N", N, "H", H, "D", D)
    chunks = [synth.gdn_inputs(B, N, H, D, seed=40 + j, state=False) for j in range(3)]
    d16 = lambda x: torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16).cuda()
    d32 = lambda x: torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()
    q_s, k_s, v_s = (torch.empty((B, N, H, D), dtype=torch.bfloat16, device="cuda") for _ in range(3))
    a_s, b_s = (torch.empty((B, H, N), dtype=torch.float32, device="cuda") for _ in range(2))
    out_s = torch.empty_like(q_s)
    state = torch.zeros((B, H, D, D), dtype=torch.float32, device="cuda")
    ws = torch.empty(cwa.sa_gdn_workspace_bytes(B, N, H, D), dtype=torch.uint8, device="cuda")

    def load(j):
        q, k, v, a, b, _ = chunks[j]
        for dst, x in ((q_s, d16(q)), (k_s, d16(k)), (v_s, d16(v)), (a_s, d32(a)), (b_s, d32(b))):
            dst.copy_(x)

    def call():
        cwa.gdn_forward(q_s, k_s, v_s, a_s, b_s, state=state, out=out_s, state_out=state, workspace=ws)

    eager = []
    for j in range(len(chunks)):
        load(j)
        call()
        torch.cuda.synchronize()
        eager.append((out_s.clone(), state.clone()))
    state.zero_()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    load(0)
    torch.cuda.synchronize()
    snapshot = state.clone()
    with torch.cuda.graph(g):
        call()
    state.copy_(snapshot)                        # capture runs nothing; start again from zeros
    for j in range(len(chunks)):
        load(j)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        same = torch.equal(out_s, eager[j][0]) and torch.equal(state, eager[j][1])
        say(f"  replay chunk {j}: identical to eager: {same}")
        assert same, j


def _replay_check(g, load, n_sets, results, eager):
    for rep in range(2):
        for j in range(n_sets):
            load(j)                              # eager work between replays
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            same = all(torch.equal(a, b) for a, b in zip(results(), eager[j]))
            say(f"  replay {rep} set {j}: identical to eager: {same}")
            assert same, (rep, j)


@pytest.mark.parametrize("steps_mode", [False, True])
def test_captured_buffer_attend_replays_match_eager(steps_mode):
    """sa_buffer_attend launches one RoPE kernel for all its chunks and one attention kernel, no
    memset or copy: captured once and replayed with new q, k, v in the same buffers, it equals
    the eager call bit for bit (the eager calls are held against the oracle)."""
    w = synth.small_variant(synth.WORKLOADS["wan1.3b"], heads=2, frame_h=6, frame_w=10, frames_per_chunk=3,
                            window_chunks=3)
    nb, nc = 3, w.tokens_per_chunk
    say("graph capture: buffer attend of", nb, "chunks, steps" if steps_mode else "moving buffer")
    s = cwa.Stream(config_for(w, max_buffer_chunks=nb))
    hist = HistoryOracle(spec_for(w))
    for c in range(4):                           # sink full, window full
        _, k, v = synth.chunk_qkv(w, c)
        s.kv_append(dev(k, w.dtype), dev(v, w.dtype))
        hist.append(k, v)
    sets = []
    for j in range(3):
        parts = [synth.chunk_qkv(w, 200 + 10 * j + i) for i in range(nb)]
        sets.append([np.concatenate([p[t] for p in parts], axis=1) for t in range(3)])
    q_s, k_s, v_s, out_s = (torch.empty((w.batch, nb * nc, w.heads, w.head_dim), dtype=torch.bfloat16,
                                        device="cuda") for _ in range(4))
    lse_s = torch.empty((w.batch, w.heads, nb * nc), dtype=torch.float32, device="cuda")

    def load(j):
        for dst, x in zip((q_s, k_s, v_s), sets[j]):
            dst.copy_(dev(x, w.dtype))

    eager = []
    for j in range(len(sets)):
        load(j)
        s.buffer_attend(q_s, k_s, v_s, out=out_s, lse=lse_s, steps=steps_mode)
        torch.cuda.synchronize()
        eager.append((out_s.clone(), lse_s.clone()))
        want, want_lse = hist.buffer_attend(*sets[j], steps=steps_mode)
        a, r = err(host(out_s), want)
        la, _ = err(host(lse_s), want_lse)
        say(f"  eager set {j}: max {a:.2e} rel {r:.2e}; lse {la:.2e}")
        assert a <= BF16_ABS and r <= BF16_REL and la <= BF16_ABS
    plan = s.query()
    load(0)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        s.buffer_attend(q_s, k_s, v_s, out=out_s, lse=lse_s, steps=steps_mode)
    assert s.query() == plan                      # capturing changed no stream state
    _replay_check(g, load, len(sets), lambda: (out_s, lse_s), eager)
    s.close()


def test_captured_batch_attend_replays_match_eager():
    """sa_batch_attend over two streams at different states (one RoPE launch, one attention
    launch): captured once and replayed with new data, it equals the eager call bit for bit."""
    w = synth.small_variant(synth.WORKLOADS["wan1.3b"], heads=2, frame_h=6, frame_w=10, frames_per_chunk=3,
                            window_chunks=3)
    nc = w.tokens_per_chunk
    say("graph capture: ragged batch of 2 streams, Nc", nc)
    streams, hists = [], []
    for n_commit in (2, 6):                      # one window still filling, one wrapped
        s = cwa.Stream(config_for(w))
        h = HistoryOracle(spec_for(w))
        for c in range(n_commit):
            _, k, v = synth.chunk_qkv(w, 50 * n_commit + c)
            s.kv_append(dev(k, w.dtype), dev(v, w.dtype))
            h.append(k, v)
        streams.append(s)
        hists.append(h)
    sets = [[synth.chunk_qkv(w, 400 + 10 * j + i) for i in range(2)] for j in range(3)]
    shape = (w.batch, nc, w.heads, w.head_dim)
    bufs = [[torch.empty(shape, dtype=torch.bfloat16, device="cuda") for _ in range(4)] for _ in range(2)]
    lses = [torch.empty((w.batch, w.heads, nc), dtype=torch.float32, device="cuda") for _ in range(2)]

    def load(j):
        for i in range(2):
            for dst, x in zip(bufs[i][:3], sets[j][i]):
                dst.copy_(dev(x, w.dtype))

    def call():
        cwa.sa_batch_attend(streams, [b[0] for b in bufs], [b[1] for b in bufs], [b[2] for b in bufs],
                            [b[3] for b in bufs], lses)

    eager = []
    for j in range(len(sets)):
        load(j)
        call()
        torch.cuda.synchronize()
        eager.append(tuple(x.clone() for i in range(2) for x in (bufs[i][3], lses[i])))
        for i in range(2):
            want, want_lse = hists[i].attend(*sets[j][i])
            a, r = err(host(bufs[i][3]), want)
            la, _ = err(host(lses[i]), want_lse)
            say(f"  eager set {j} stream {i}: max {a:.2e} rel {r:.2e}; lse {la:.2e}")
            assert a <= BF16_ABS and r <= BF16_REL and la <= BF16_ABS
    plans = [s.query() for s in streams]
    load(0)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    assert [s.query() for s in streams] == plans
    _replay_check(g, load, len(sets), lambda: tuple(x for i in range(2) for x in (bufs[i][3], lses[i])), eager)
    for s in streams:
        s.close()
