"""Pins for the oracle's stream semantics (CPU only).

* hand-worked visible sets of the tiny stream (tests/golden/tiny_stream_bookkeeping.json);
* brute force: a tiny stream whose outputs are rebuilt from the hand-worked
  visible sets with complex-number rotations and scalar-loop attention;
* the masked full-history formulation equals attention over the explicitly
  concatenated visible keys;
* HistoryOracle (definition) == RingOracle (bounded storage, re-rotation on
  refresh) on seeded random operation sequences;
* refresh invariances: with SHIFT_SINK, or with no sink, outputs are unchanged;
  without it, only the sink logits move;
* storage emulation stores bf16-exact values and stays close to fp64.
"""
import copy
import json
import math
import os

import numpy as np
import pytest

import synth
from oracle import HistoryOracle, RingOracle, SHIFT_SINK, StreamSpec, attend_bruteforce, round_bf16
from oracle.rope import rope3d, token_coords
from oracle.stream import StreamError

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _tiny_spec(**kw):
    base = dict(batch=1, heads=2, head_dim=64, frame_h=8, frame_w=8, frames_per_chunk=2,
                sink_chunks=1, window_chunks=2)
    base.update(kw)
    return StreamSpec(**base)


def _rand_chunk(spec, seed, n_tokens=None):
    n = spec.tokens_per_chunk if n_tokens is None else n_tokens
    g = np.random.default_rng(seed)
    return [g.standard_normal((spec.batch, n, spec.heads, spec.head_dim)) for _ in range(3)]


def test_golden_tiny_bookkeeping():
    g = json.load(open(os.path.join(GOLD, "tiny_stream_bookkeeping.json")))
    w = synth.WORKLOADS["tiny_f32"]
    assert (w.frames_per_chunk, w.sink_chunks, w.window_chunks) == \
        (g["frames_per_chunk"], g["sink_chunks"], g["window_chunks"])
    spec = StreamSpec.from_workload(w)
    for orc in (HistoryOracle(spec), RingOracle(spec)):
        for entry in g["chunks"]:
            c = entry["chunk"]
            if str(c) in g["refresh_before"]:
                delta = orc.refresh(g["refresh_before"][str(c)])
                assert delta == entry["refresh_delta"]
            assert w.refresh_before(c) == (str(c) in g["refresh_before"])
            st = orc.state()
            assert st["t_next"] == entry["t_next"]
            assert [list(x) for x in st["visible"]] == entry["visible"], (type(orc), c)
            q, k, v = synth.chunk_qkv(w, c)
            orc.append(k, v)


def _complex_rope(u, t, y, x, split, theta=10000.0):
    """Independent rotation for the brute-force pin: pairs as complex numbers."""
    u = np.asarray(u, dtype=np.float64)
    z = u[..., 0::2] + 1j * u[..., 1::2]
    angles = []
    for seg, p in zip(split, (t, y, x)):
        for j in range(seg // 2):
            angles.append(p * theta ** (-2.0 * j / seg))
    zr = z * np.exp(1j * np.array(angles))
    out = np.empty_like(u)
    out[..., 0::2], out[..., 1::2] = zr.real, zr.imag
    return out


def test_bruteforce_tiny_stream_from_golden_sets():
    """Rebuild every output of a tiny stream from the hand-worked visible sets."""
    g = json.load(open(os.path.join(GOLD, "tiny_stream_bookkeeping.json")))
    spec = StreamSpec(batch=1, heads=1, head_dim=6, frame_h=1, frame_w=2,
                      frames_per_chunk=g["frames_per_chunk"], sink_chunks=g["sink_chunks"],
                      window_chunks=g["window_chunks"])
    split = (2, 2, 2)
    assert spec.rope == split
    nc = spec.tokens_per_chunk                     # 4 tokens: frames 0,0,1,1; x 0,1,0,1
    frames, xs = [0, 0, 1, 1], [0, 1, 0, 1]
    data = [_rand_chunk(spec, 100 + c) for c in range(len(g["chunks"]))]
    hist, ring = HistoryOracle(spec), RingOracle(spec)
    for entry in g["chunks"]:
        c = entry["chunk"]
        if str(c) in g["refresh_before"]:
            hist.refresh(g["refresh_before"][str(c)])
            ring.refresh(g["refresh_before"][str(c)])
        q, k, v = data[c]
        keys, vals = [], []
        for kind, cid, t0 in entry["visible"]:
            src = data[cid][1] if kind != "self" else k
            vs = data[cid][2] if kind != "self" else v
            for n in range(nc):
                keys.append(_complex_rope(src[0, n, 0], t0 + frames[n], 0, xs[n], split))
                vals.append(vs[0, n, 0])
        qr = np.array([_complex_rope(q[0, n, 0], entry["t_next"] + frames[n], 0, xs[n], split)
                       for n in range(nc)])
        want, want_lse = attend_bruteforce(qr, np.array(keys), np.array(vals), 1 / math.sqrt(6))
        for orc in (hist, ring):
            o, l = orc.attend(q, k, v)
            np.testing.assert_allclose(o[0, :, 0], want, rtol=0, atol=1e-12)
            np.testing.assert_allclose(l[0, 0], want_lse, rtol=0, atol=1e-12)
        hist.append(k, v)
        ring.append(k, v)


def _masked_full_history(orc: HistoryOracle, all_chunks, q, k, v):
    """Logits over EVERY chunk committed so far (+ self), non-visible ones masked to -inf."""
    from oracle.rope import rope3d, token_coords
    spec = orc.spec
    f, y, x = token_coords(spec.tokens_per_chunk, spec.frame_h, spec.frame_w)
    vis = {(cid) for kind, cid, t0 in orc.visible() if kind != "self"}
    t0_of = {cid: t0 for kind, cid, t0 in orc.visible()}
    out = np.zeros((spec.batch, spec.tokens_per_chunk, spec.heads, spec.head_dim))
    for b in range(spec.batch):
        for h in range(spec.heads):
            K, V, mask = [], [], []
            for cid, (kc, vc) in enumerate(all_chunks):
                t0 = t0_of.get(cid, 0)
                K.append(rope3d(kc[b, :, h], t0 + f, y, x, spec.rope))
                V.append(vc[b, :, h])
                mask.append(np.full(len(f), cid in vis))
            K.append(rope3d(k[b, :, h], orc.t_next + f, y, x, spec.rope))
            V.append(v[b, :, h])
            mask.append(np.full(len(f), True))
            K, V, mask = np.concatenate(K), np.concatenate(V), np.concatenate(mask)
            qr = rope3d(q[b, :, h], orc.t_next + f, y, x, spec.rope)
            s = qr @ K.T * spec.softmax_scale
            s[:, ~mask] = -np.inf
            p = np.exp(s - s.max(axis=1, keepdims=True))
            out[b, :, h] = (p / p.sum(axis=1, keepdims=True)) @ V
    return out


def test_masked_full_history_equals_concatenated_visible():
    spec = _tiny_spec(frame_h=2, frame_w=3, heads=2, head_dim=12, window_chunks=2)
    orc = HistoryOracle(spec)
    committed = []
    for c in range(7):
        q, k, v = _rand_chunk(spec, 200 + c)
        if c == 5:
            orc.refresh()
        o, _ = orc.attend(q, k, v)
        np.testing.assert_allclose(o, _masked_full_history(orc, committed, q, k, v), atol=1e-12)
        orc.append(k, v)
        committed.append((k, v))


def _random_ops(seed, n_ops, spec):
    g = np.random.default_rng(seed)
    ops = []
    for _ in range(n_ops):
        r = g.random()
        if r < 0.55:
            ops.append(("append",))
        elif r < 0.75:
            ops.append(("refresh", int(g.choice([-1, 0, 3, 7])), int(g.random() < 0.3)))
        elif r < 0.85 and spec.sink_chunks > 0:
            ops.append(("sink_update",))
        else:
            ops.append(("attend",))
    return ops


@pytest.mark.parametrize("S,W,seed", [(1, 2, 0), (1, 3, 1), (2, 2, 2), (0, 2, 3), (1, 0, 4),
                                      (0, 0, 5), (3, 1, 6)])
def test_history_equals_ring(S, W, seed):
    spec = _tiny_spec(frame_h=2, frame_w=2, heads=2, head_dim=12, sink_chunks=S, window_chunks=W)
    hist, ring = HistoryOracle(spec), RingOracle(spec)
    for i, op in enumerate(_random_ops(seed, 40, spec) + [("attend",)]):
        if op[0] == "append":
            _, k, v = _rand_chunk(spec, 1000 * seed + i)
            hist.append(k, v)
            ring.append(k, v)
        elif op[0] == "refresh":
            base = op[1] if op[1] >= 0 else None
            assert hist.refresh(base, SHIFT_SINK * op[2]) == ring.refresh(base, SHIFT_SINK * op[2])
        elif op[0] == "sink_update":
            _, k, v = _rand_chunk(spec, 1000 * seed + i, n_tokens=S * spec.tokens_per_chunk)
            hist.sink_update(k, v)
            ring.sink_update(k, v)
        else:
            q, k, v = _rand_chunk(spec, 1000 * seed + i)
            oh, lh = hist.attend(q, k, v)
            orr, lr = ring.attend(q, k, v)
            np.testing.assert_allclose(orr, oh, rtol=0, atol=1e-12)
            np.testing.assert_allclose(lr, lh, rtol=0, atol=1e-12)
        assert hist.state() == ring.state()


def test_refresh_with_shift_sink_or_no_sink_is_output_invariant():
    for S, flags in [(1, SHIFT_SINK), (0, 0), (2, SHIFT_SINK)]:
        spec = _tiny_spec(frame_h=2, frame_w=3, heads=1, head_dim=12, sink_chunks=S, window_chunks=2)
        orc = HistoryOracle(spec)
        for c in range(5):
            _, k, v = _rand_chunk(spec, 300 + c)
            orc.append(k, v)
        q, k, v = _rand_chunk(spec, 399)
        before, lb = orc.attend(q, k, v)
        delta = orc.refresh(None, flags)
        assert delta != 0
        after, la = orc.attend(q, k, v)
        np.testing.assert_allclose(after, before, rtol=0, atol=1e-12)
        np.testing.assert_allclose(la, lb, rtol=0, atol=1e-12)


def test_refresh_pinned_sink_moves_only_sink_logits():
    spec = _tiny_spec(frame_h=2, frame_w=3, heads=1, head_dim=12, sink_chunks=1, window_chunks=2)
    orc = RingOracle(spec)
    for c in range(6):
        _, k, v = _rand_chunk(spec, 400 + c)
        orc.append(k, v)
    q, k, v = _rand_chunk(spec, 499)
    qr, ks, _ = orc.staged(q, k, v)
    sink_before = qr[0, 0] @ orc.sink_k[0, 0, 0].T
    win_before = [qr[0, 0] @ orc.stored_k(cid)[0, 0].T for kind, cid, _ in orc.visible()
                  if kind == "window"]
    self_before = qr[0, 0] @ ks[0, 0].T
    assert orc.refresh() == 6                     # oldest window chunk (chunk 4, t0 = 8) moves to base 2
    qr2, ks2, _ = orc.staged(q, k, v)
    win_after = [qr2[0, 0] @ orc.stored_k(cid)[0, 0].T for kind, cid, _ in orc.visible()
                 if kind == "window"]
    np.testing.assert_allclose(win_after, win_before, atol=1e-11)
    np.testing.assert_allclose(qr2[0, 0] @ ks2[0, 0].T, self_before, atol=1e-11)
    assert np.max(np.abs(qr2[0, 0] @ orc.sink_k[0, 0, 0].T - sink_before)) > 1e-2


def test_storage_emulation_bf16():
    w = synth.small_variant(synth.WORKLOADS["wan1.3b"], heads=2, frame_h=4, frame_w=6,
                            window_chunks=2, n_chunks=6)
    spec = StreamSpec.from_workload(w)
    pure, emu = RingOracle(spec), RingOracle(spec, storage="bf16")
    for c in range(6):
        q, k, v = synth.chunk_qkv(w, c)
        if c == 4:
            pure.refresh()
            emu.refresh()
        op, _ = pure.attend(q, k, v)
        oe, _ = emu.attend(q, k, v)
        qr, kr, vr = emu.staged(q, k, v)
        for x in (qr, kr, vr):
            assert np.array_equal(round_bf16(x), x)
        np.testing.assert_array_equal(vr, np.transpose(v, (0, 2, 1, 3)))
        err = np.abs(oe - op)
        assert err.max() < 2e-2 and np.linalg.norm(err) / np.linalg.norm(op) < 1e-2
        assert err.max() > 0                      # rounding is really applied
        pure.append(k, v)
        emu.append(k, v)
    for kind, cid, _ in emu.visible()[:-1]:
        assert np.array_equal(round_bf16(emu.stored_k(cid)), emu.stored_k(cid))


def test_errors():
    spec = _tiny_spec(frame_h=2, frame_w=2, heads=1, head_dim=12, sink_chunks=0, window_chunks=1,
                      max_t=6)
    for orc in (HistoryOracle(spec), RingOracle(spec)):
        q, k, v = _rand_chunk(spec, 1)
        with pytest.raises(StreamError) as e:
            orc.sink_update(k, v)
        assert e.value.kind == "bad_state"
        with pytest.raises(StreamError) as e:
            orc.append(k[:, :3], v)
        assert e.value.kind == "invalid"
        with pytest.raises(StreamError) as e:
            orc.refresh(-5)
        assert e.value.kind == "invalid"
        for _ in range(3):                       # t = 0, 2, 4 fit below max_t = 6
            orc.append(k, v)
        with pytest.raises(StreamError) as e:
            orc.attend(q, k, v)
        assert e.value.kind == "position_range"
        before = orc.state()
        with pytest.raises(StreamError):
            orc.append(k, v)
        assert orc.state() == before             # failed calls leave the state unchanged
        orc.refresh()                            # re-basing cures the range problem
        orc.attend(q, k, v)


def test_synth_inputs():
    w = synth.WORKLOADS["hybrid1280x704"]
    outl = synth.outlier_channels(w)
    assert outl.shape == (16, 6)
    q = synth.draw(w, 0, synth.T_Q, n_tokens=64)
    v = synth.draw(w, 0, synth.T_V, n_tokens=64)
    assert np.array_equal(synth.to_bf16_exact(q), q)
    for h in range(16):
        others = np.setdiff1d(np.arange(128), outl[h])
        assert np.abs(q[0, :, h, outl[h]]).std() > 4 * np.abs(q[0, :, h, others]).std()
    assert abs(v.std() - 1) < 0.05
    q2 = synth.draw(w, 0, synth.T_Q, n_tokens=64)
    assert np.array_equal(q, q2)                 # seeded
    assert not np.array_equal(q, synth.draw(w, 1, synth.T_Q, n_tokens=64))
    t = synth.WORKLOADS["tiny_f32"]
    a = synth.draw(t, 0, synth.T_Q)
    assert a.dtype == np.float32 and not np.array_equal(synth.to_bf16_exact(a), a)
    d = synth.distinct_set_for(synth.WORKLOADS["long512p"], [500])
    assert d == frozenset({0, 497, 498, 499, 500})
    assert synth.source_id(3, d) != 3 and synth.source_id(499, d) == 499


def _explicit_buffer_attend(spec, committed, t_next, q, k, v, steps=False):
    """Buffer attend from an explicit chunk list: committed = [(t0, k, v)] in commit order (the
    first S are the sink); buffer chunk j at t_next + j*F sees the sink, the last W of
    (committed window chunks, buffer chunks 0..j-1) and itself -- or, with steps, the sink,
    the last W committed window chunks and itself. Scalar-loop attention."""
    S, W, F, nc = spec.sink_chunks, spec.window_chunks, spec.frames_per_chunk, spec.tokens_per_chunk
    f, y, x = token_coords(nc, spec.frame_h, spec.frame_w)
    rot = lambda u, t0: rope3d(np.transpose(u, (0, 2, 1, 3)), t0 + f, y, x, spec.rope, spec.theta)
    n = q.shape[1] // nc
    sink, window = committed[:S], committed[S:]
    buf = [(t_next + j * F, k[:, j * nc:(j + 1) * nc], v[:, j * nc:(j + 1) * nc]) for j in range(n)]
    out = np.empty(q.shape)
    scale = 1.0 / np.sqrt(spec.head_dim)
    for j in range(n):
        prior = window if steps else window + buf[:j]
        vis = sink + (prior[max(0, len(prior) - W):] if W else []) + [buf[j]]
        K = np.concatenate([rot(kk, t0) for t0, kk, _ in vis], axis=2)
        V = np.concatenate([np.transpose(vv, (0, 2, 1, 3)) for _, _, vv in vis], axis=2)
        Q = rot(q[:, j * nc:(j + 1) * nc], t_next + j * F)
        for b in range(spec.batch):
            for h in range(spec.heads):
                o, _ = attend_bruteforce(Q[b, h], K[b, h], V[b, h], scale)
                out[b, j * nc:(j + 1) * nc, h] = o
    return out


@pytest.mark.parametrize("S,W,n,commits", [(1, 2, 4, 5), (0, 1, 3, 2), (2, 0, 2, 3), (1, 3, 2, 1),
                                           (1, 3, 3, 3)])
@pytest.mark.parametrize("steps", [False, True])
def test_buffer_attend_matches_explicit_windows(S, W, n, commits, steps):
    """Pin: each buffer chunk's visible set is enumerated directly, not through the oracle's
    ring or history bookkeeping; both formulations must reproduce it."""
    spec = StreamSpec(batch=1, heads=2, head_dim=8, frame_h=2, frame_w=2, frames_per_chunk=1,
                      sink_chunks=S, window_chunks=W)
    hist, ring = HistoryOracle(spec), RingOracle(spec)
    committed = []
    for c in range(commits):
        _, k, v = _rand_chunk(spec, 100 + c)
        hist.append(k, v)
        ring.append(k, v)
        committed.append((c * spec.frames_per_chunk, k, v))
    q, k, v = _rand_chunk(spec, 7, n_tokens=n * spec.tokens_per_chunk)
    want = _explicit_buffer_attend(spec, committed, hist.t_next, q, k, v, steps=steps)
    before = hist.state()
    for orc in (hist, ring):
        got, lse = orc.buffer_attend(q, k, v, steps=steps)
        np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)
        assert np.all(np.isfinite(lse))
    assert hist.state() == before                    # a buffer attend changes nothing


def test_steps_buffer_partial_sink_and_first_chunk():
    """Stream-Batch over denoising steps: chunk 0 of the batch is exactly an attend; a partial
    sink is allowed (the chunks see the committed sink chunks and themselves); the banded
    buffer's chunk 0 agrees with it, later chunks differ once the band admits chunk 0."""
    spec = _tiny_spec(sink_chunks=2, window_chunks=2)
    nc = spec.tokens_per_chunk
    orc = HistoryOracle(spec)
    _, k, v = _rand_chunk(spec, 0)
    orc.append(k, v)                                 # one of two sink chunks
    q, k, v = _rand_chunk(spec, 1, n_tokens=3 * nc)
    o, _ = orc.buffer_attend(q, k, v, steps=True)
    tmp = copy.deepcopy(orc)
    for j in range(3):
        o1, _ = tmp.attend(q[:, j * nc:(j + 1) * nc], k[:, j * nc:(j + 1) * nc], v[:, j * nc:(j + 1) * nc])
        np.testing.assert_allclose(o[:, j * nc:(j + 1) * nc], o1, rtol=0, atol=1e-12)
        tmp.t_next += spec.frames_per_chunk          # same context, next position
    _, k2, v2 = _rand_chunk(spec, 2)
    orc.append(k2, v2)                               # the sink is full now
    ob, _ = orc.buffer_attend(q, k, v)
    os_, _ = orc.buffer_attend(q, k, v, steps=True)
    np.testing.assert_allclose(ob[:, :nc], os_[:, :nc], rtol=0, atol=1e-12)
    assert np.abs(ob[:, nc:] - os_[:, nc:]).max() > 1e-3


def test_buffer_attend_single_chunk_is_attend_and_rows():
    spec = _tiny_spec()
    orc = HistoryOracle(spec)
    for c in range(3):
        _, k, v = _rand_chunk(spec, c)
        orc.append(k, v)
    q, k, v = _rand_chunk(spec, 9)
    o1, l1 = orc.attend(q, k, v)
    o2, l2 = orc.buffer_attend(q, k, v)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)
    nc = spec.tokens_per_chunk
    q, k, v = _rand_chunk(spec, 10, n_tokens=3 * nc)
    full, lfull = orc.buffer_attend(q, k, v)
    rows = [0, nc - 1, nc, 2 * nc + 5]
    part, lpart = orc.buffer_attend(q, k, v, rows=rows)
    np.testing.assert_allclose(part[:, rows], full[:, rows], rtol=0, atol=1e-12)   # BLAS blocking differs
    np.testing.assert_allclose(lpart[:, :, rows], lfull[:, :, rows], rtol=0, atol=1e-12)
    assert np.isnan(part[:, 1]).all()


def test_buffer_attend_errors():
    spec = _tiny_spec(sink_chunks=2)
    orc = HistoryOracle(spec)
    _, k, v = _rand_chunk(spec, 0)
    orc.append(k, v)                                 # sink not full yet
    q, k, v = _rand_chunk(spec, 1, n_tokens=2 * spec.tokens_per_chunk)
    with pytest.raises(StreamError) as e:
        orc.buffer_attend(q, k, v)
    assert e.value.kind == "bad_state"
    orc.append(k[:, :spec.tokens_per_chunk], v[:, :spec.tokens_per_chunk])
    q, k, v = _rand_chunk(spec, 2, n_tokens=spec.tokens_per_chunk + 3)
    with pytest.raises(StreamError) as e:
        orc.buffer_attend(q, k, v)
    assert e.value.kind == "invalid"
    spec = _tiny_spec(max_t=6)                        # F = 2: chunks at t = 0, 2, 4 fit
    orc = HistoryOracle(spec)
    _, k, v = _rand_chunk(spec, 3)
    orc.append(k, v)
    q, k, v = _rand_chunk(spec, 4, n_tokens=2 * spec.tokens_per_chunk)
    orc.buffer_attend(q, k, v)                       # t = 2, 4
    q, k, v = _rand_chunk(spec, 5, n_tokens=3 * spec.tokens_per_chunk)
    with pytest.raises(StreamError) as e:
        orc.buffer_attend(q, k, v)                   # t = 6 is out of range
    assert e.value.kind == "position_range"
