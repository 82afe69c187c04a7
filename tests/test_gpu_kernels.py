"""GPU parity of every kernel through the C ABI, at oracle-sized shapes.

* rope_apply / kv_ring_append / rope_refresh / sink_update: the cache contents
  (rotated K rows, transposed V) and the rotated Q scratch are compared with the
  storage-emulating ring oracle: K and Q within 1 bf16 step (2 after a refresh,
  which rounds stored keys a second time), V bit-exact;
* chunk_attention (+ attn_combine): outputs and LSE against the fp64 oracle,
  over several query tiles and key tiles with ragged tails, forced key-range
  splits, bf16 D = 128 and D = 64, fp32, lockstep batches, S = 0 / W = 0 and a
  one-token chunk;
* zero-copy commits equal explicit commits, repeated attends are bit-identical,
  refresh with SHIFT_SINK leaves outputs unchanged.
"""
import numpy as np
import pytest
import torch

import causal_windowed_attention_amd as cwa
import synth
from gpu_util import (BF16_ABS, BF16_REL, F32_ABS, bf16_ulp_distance, config_for, dev, err, host,
                      say, spec_for)
from oracle import HistoryOracle, RingOracle, SHIFT_SINK

pytestmark = pytest.mark.gpu

SMALL = synth.Workload(name="small_bf16", cfg_id=101, batch=2, heads=3, head_dim=128, frame_h=5,
                       frame_w=7, frames_per_chunk=3, sink_chunks=1, window_chunks=2, n_chunks=8)


def _slot_of(s: cwa.Stream, chunk_id: int) -> int:
    st = s.query()
    for j in range(st["n_slots"]):
        info = s.slot(j)
        if info["kind"] in (cwa.SA_SLOT_SINK, cwa.SA_SLOT_WINDOW) and info["chunk_id"] == chunk_id:
            return j
    raise KeyError(chunk_id)


def _cache_chunk(s: cwa.Stream, slot: int, w):
    nc = w.tokens_per_chunk
    k = s.k_cache_view()[:, slot * nc:(slot + 1) * nc, :]
    vt = s.vt_cache_view()[:, :, slot * nc:(slot + 1) * nc]
    return (k.reshape(w.batch, w.heads, nc, w.head_dim),
            vt.transpose(1, 2).reshape(w.batch, w.heads, nc, w.head_dim))


def _check_storage(s, ring: RingOracle, w, max_ulp):
    for kind, cid, _ in ring.visible()[:-1]:
        slot = _slot_of(s, cid)
        k, v = _cache_chunk(s, slot, w)
        if w.dtype == "bf16":
            assert bf16_ulp_distance(k, ring.stored_k(cid)) <= max_ulp, (kind, cid)
            assert np.array_equal(host(v), ring.stored_v(cid)), (kind, cid)
        else:
            np.testing.assert_allclose(host(k), ring.stored_k(cid), rtol=0, atol=2e-6)
            assert np.array_equal(host(v), ring.stored_v(cid))


def _run_sequence(w, ops, check_storage=True, variant=0):
    """Drive the GPU stream and both oracles through ops; check every attend."""
    say("sequence", w.name, w.dtype, "B", w.batch, "H", w.heads, "D", w.head_dim, "Nc", w.tokens_per_chunk,
        "variant", variant)
    s = cwa.Stream(config_for(w))
    s.set_option(cwa.SA_OPT_ATTN_VARIANT, variant)
    spec = spec_for(w)
    hist = HistoryOracle(spec)
    ring = RingOracle(spec, storage=w.dtype)
    c = 0
    refreshed = False
    worst = (0.0, 0.0)
    for op in ops:
        if op == "attend":
            q, k, v = synth.chunk_qkv(w, c)
            lse = torch.empty((w.batch, w.heads, w.tokens_per_chunk), dtype=torch.float32, device="cuda")
            out = s.chunk_attend(dev(q, w.dtype), dev(k, w.dtype), dev(v, w.dtype), lse=lse)
            torch.cuda.synchronize()
            want, want_lse = hist.attend(q, k, v)
            emu, _ = ring.attend(q, k, v)
            got = host(out)
            a, r = err(got, want)
            ae, re_ = err(got, emu)
            la, _ = err(host(lse), want_lse)
            say(f"  chunk {c}: vs fp64 max {a:.2e} rel {r:.2e}; vs storage max {ae:.2e} rel {re_:.2e}; lse {la:.2e}")
            if w.dtype == "bf16":
                assert a <= BF16_ABS and r <= BF16_REL, (c, a, r)
                assert la <= BF16_ABS, la
            else:
                assert a <= F32_ABS, (c, a)
                assert la <= F32_ABS, la
            worst = (max(worst[0], a), max(worst[1], r))
            if check_storage:
                qr, ks, vs = ring.staged(q, k, v)
                qs = s.q_scratch_view().reshape(w.batch, w.heads, w.tokens_per_chunk, w.head_dim)
                st = s.query()
                kk, vv = _cache_chunk(s, st["staging_slot"], w)
                if w.dtype == "bf16":
                    assert bf16_ulp_distance(qs, qr) <= 1
                    assert bf16_ulp_distance(kk, ks) <= 1
                    assert np.array_equal(host(vv), vs)
                _check_storage(s, ring, w, 2 if refreshed else 1)
            staged = (k, v)
        elif op in ("append", "append0"):
            k, v = staged
            if op == "append0":
                s.kv_append(None, None)          # commit the staged chunk, no device work
            else:
                s.kv_append(dev(k, w.dtype), dev(v, w.dtype))
            hist.append(k, v)
            ring.append(k, v)
            c += 1
        elif op.startswith("refresh"):
            flags = SHIFT_SINK if op == "refresh_shift" else 0
            d = s.rope_refresh(-1, flags)
            assert d == hist.refresh(None, flags) == ring.refresh(None, flags)
            refreshed = True
        elif op == "sink_update":
            sk, sv = synth.sink_kv(w, 0)
            s.sink_update(dev(sk, w.dtype), dev(sv, w.dtype))
            hist.sink_update(sk, sv)
            ring.sink_update(sk, sv)
        st = s.query()
        assert st["t_next"] == hist.t_next and st["n_appends"] == hist.n_appends
    if check_storage:
        torch.cuda.synchronize()
        _check_storage(s, ring, w, 2 if refreshed else 1)
    s.close()
    return worst


OPS = ["attend", "append", "attend", "append0", "attend", "append", "attend", "append0",
       "refresh", "attend", "append", "sink_update", "attend", "append0", "refresh_shift",
       "attend", "append", "attend"]


@pytest.mark.parametrize("variant", [1, 2, 3, 4])
def test_stream_bf16_d128_storage_and_outputs(variant):
    _run_sequence(SMALL, OPS, variant=variant)


@pytest.mark.parametrize("variant", [1, 2, 3])
def test_stream_bf16_d64(variant):
    w = synth.small_variant(SMALL, name="small_d64", head_dim=64, frame_h=4, frame_w=8,
                            frames_per_chunk=2, window_chunks=3)
    _run_sequence(w, OPS, variant=variant)


def test_stream_f32_tiny_config():
    """The tiny fp32 workload end to end: 6 chunks, refresh before chunk 4 (base 2)."""
    w = synth.WORKLOADS["tiny_f32"]
    ops = []
    for c in range(w.n_chunks):
        if w.refresh_before(c):
            ops.append("refresh")
        ops += ["attend", "append"]
    worst = _run_sequence(w, ops)
    assert worst[0] <= F32_ABS


def test_stream_f32_d128_with_sink_update():
    w = synth.small_variant(SMALL, name="small_f32", dtype="f32", batch=1)
    _run_sequence(w, OPS)


@pytest.mark.parametrize("S,W,B,variant", [(0, 2, 1, 1), (1, 0, 2, 2), (0, 0, 1, 3), (2, 1, 2, 3),
                                             (0, 2, 1, 4), (0, 0, 1, 4), (2, 1, 2, 4)])
def test_edge_shapes(S, W, B, variant):
    w = synth.small_variant(SMALL, name=f"edge_S{S}W{W}", sink_chunks=S, window_chunks=W, batch=B,
                            heads=2)
    _run_sequence(w, ["attend", "append", "attend", "append0", "attend", "append", "refresh",
                      "attend", "append", "attend"], variant=variant)


@pytest.mark.parametrize("frame_h,frame_w,head_dim,dtype", [(5, 8, 128, "bf16"), (5, 8, 128, "f32"),
                                                         (2, 96, 128, "bf16"), (3, 203, 64, "f32")])
def test_spatial_table_sizes(frame_h, frame_w, head_dim, dtype):
    """Spatial (cos, sin) tables of every size class: an odd pair count, (5 + 8) x 21 = 273, which
    a block stages in LDS in 16-byte pieces ending past the table; and more pairs than a block
    stages (98 x 21 = 2058, 206 x 10 = 2060), which the rotation reads from global memory."""
    w = synth.small_variant(SMALL, name=f"tables_{frame_h}x{frame_w}_d{head_dim}_{dtype}", frame_h=frame_h,
                            frame_w=frame_w, head_dim=head_dim, frames_per_chunk=1, batch=1, heads=2,
                            dtype=dtype)
    _run_sequence(w, ["attend", "append", "attend", "append", "refresh", "attend", "append", "sink_update",
                      "attend", "append", "attend"])


@pytest.mark.parametrize("variant", [0, 4])
def test_one_token_chunks(variant):
    w = synth.small_variant(SMALL, name="one_token", frame_h=1, frame_w=1, frames_per_chunk=1,
                            window_chunks=3, heads=2)
    _run_sequence(w, ["attend", "append"] * 6 + ["refresh", "attend"], variant=variant)


def _steady_stream(w, n_commit):
    s = cwa.Stream(config_for(w))
    hist = HistoryOracle(spec_for(w))
    for c in range(n_commit):
        q, k, v = synth.chunk_qkv(w, c)
        s.chunk_attend(dev(q, w.dtype), dev(k, w.dtype), dev(v, w.dtype))
        s.kv_append(None, None)
        hist.append(k, v)
    return s, hist


@pytest.mark.parametrize("dtype,variant", [("bf16", 1), ("bf16", 2), ("bf16", 3), ("bf16", 4), ("f32", 0)])
def test_forced_kv_splits_and_repeat(dtype, variant):
    w = synth.small_variant(SMALL, name="splits", dtype=dtype, frame_h=10, frame_w=10,
                            frames_per_chunk=3, batch=1, heads=2, window_chunks=3)
    say("splits", dtype, "Nc", w.tokens_per_chunk, "variant", variant)
    s, hist = _steady_stream(w, 5)
    s.set_option(cwa.SA_OPT_ATTN_VARIANT, variant)
    q, k, v = synth.chunk_qkv(w, 5)
    want, want_lse = hist.attend(q, k, v)
    qd, kd, vd = dev(q, dtype), dev(k, dtype), dev(v, dtype)
    ref = None
    lay = s.layout()
    for splits in sorted({1, 2, 3, lay["max_kv_splits"]}):
        s.set_option(cwa.SA_OPT_KV_SPLITS, splits)
        lse = torch.empty((1, 2, w.tokens_per_chunk), dtype=torch.float32, device="cuda")
        out = s.chunk_attend(qd, kd, vd, lse=lse)
        torch.cuda.synchronize()
        assert s.query()["last_kv_splits"] == splits
        a, r = err(host(out), want)
        la, _ = err(host(lse), want_lse)
        say(f"  splits {splits}: max {a:.2e} rel {r:.2e} lse {la:.2e}")
        tol = BF16_ABS if dtype == "bf16" else F32_ABS
        assert a <= tol and la <= tol
        if dtype == "bf16":
            assert r <= BF16_REL
        again = s.chunk_attend(qd, kd, vd)
        torch.cuda.synchronize()
        assert torch.equal(again, out), "repeated attend must be bit-identical"
        if ref is None:
            ref = out
    s.close()


def test_zero_copy_commit_equals_explicit_commit():
    w = synth.small_variant(SMALL, name="zc", batch=1, heads=2)
    outs = []
    for mode in ("append", "append0"):
        s = cwa.Stream(config_for(w))
        res = []
        for c in range(6):
            q, k, v = synth.chunk_qkv(w, c)
            res.append(s.chunk_attend(dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16")))
            if mode == "append0":
                s.kv_append(None, None)
            else:
                s.kv_append(dev(k, "bf16"), dev(v, "bf16"))
        torch.cuda.synchronize()
        outs.append(res)
        s.close()
    for a, b in zip(*outs):
        assert torch.equal(a, b)


def test_refresh_shift_sink_keeps_outputs():
    w = synth.small_variant(SMALL, name="shift", batch=1, heads=2)
    s, hist = _steady_stream(w, 6)
    q, k, v = synth.chunk_qkv(w, 6)
    qd, kd, vd = dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16")
    before = host(s.chunk_attend(qd, kd, vd))
    assert s.rope_refresh(-1, cwa.SA_REFRESH_SHIFT_SINK) != 0
    after = host(s.chunk_attend(qd, kd, vd))
    a, r = err(after, before)
    say(f"  shift-sink refresh changed outputs by max {a:.2e} rel {r:.2e}")
    assert a <= BF16_ABS and r <= BF16_REL
    s.close()


def test_profiler_counts_launches():
    w = synth.small_variant(SMALL, name="prof", batch=1, heads=2)
    s = cwa.Stream(config_for(w))
    s.set_option(cwa.SA_OPT_PROFILE, 1)
    for c in range(3):
        q, k, v = synth.chunk_qkv(w, c)
        s.chunk_attend(dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16"))
        s.kv_append(dev(k, "bf16"), dev(v, "bf16"))
    ms, n = s.profile_read(cwa.SA_K_CHUNK_ATTENTION)
    assert n == 3 and ms > 0
    ms, n = s.profile_read(cwa.SA_K_KV_APPEND, reset=True)
    assert n == 3
    assert s.profile_read(cwa.SA_K_KV_APPEND) == (0.0, 0)
    s.close()


@pytest.mark.parametrize("D", [128, 64])
def test_stream_k_schedule(D):
    """Stream-K: 256 persistent workgroups share the q-tile x key-tile iterations;
    here every q-tile is cut across several workgroups, so the partial merge runs
    for all of them. Compared with the oracle and with the grid schedule."""
    w = synth.small_variant(SMALL, name=f"streamk{D}", head_dim=D, frame_h=10, frame_w=10,
                            frames_per_chunk=3, batch=2, heads=8, window_chunks=3)
    say("stream-K", D, "Nc", w.tokens_per_chunk)
    s, hist = _steady_stream(w, 5)
    q, k, v = synth.chunk_qkv(w, 5)
    want, want_lse = hist.attend(q, k, v)
    qd, kd, vd = dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16")
    outs = {}
    for sched in (1, 2):
        s.set_option(cwa.SA_OPT_ATTN_VARIANT, 3)
        s.set_option(cwa.SA_OPT_SCHEDULE, sched)
        lse = torch.empty((w.batch, w.heads, w.tokens_per_chunk), dtype=torch.float32, device="cuda")
        out = s.chunk_attend(qd, kd, vd, lse=lse)
        torch.cuda.synchronize()
        st = s.query()
        assert (st["last_sk_groups"] > 0) == (sched == 2), st
        a, r = err(host(out), want)
        la, _ = err(host(lse), want_lse)
        say(f"  schedule {sched}: sk_groups {st['last_sk_groups']} max {a:.2e} rel {r:.2e} lse {la:.2e}")
        assert a <= BF16_ABS and r <= BF16_REL and la <= BF16_ABS
        outs[sched] = host(out)
    a, _ = err(outs[2], outs[1])
    assert a <= 1e-2, a
    s.close()


def _bf16_round(x):
    t = torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.float().double().numpy()


@pytest.mark.gpu
def test_mfma_probe_computes_the_product():
    """The pure-MFMA measurement kernel really accumulates A.B: every lane's output equals
    iters * 8 accumulators * (sum of its 16 entries of A.B), A and B built from the per-lane
    operand formulas and the 32x32x16 operand layout."""
    blocks, iters = 4, 64
    out = torch.full((blocks * 256,), float("nan"), dtype=torch.float32, device="cuda")
    cwa.sa_probe_mfma_bf16(out, blocks, iters)
    torch.cuda.synchronize()
    a = np.zeros((32, 16)); b = np.zeros((16, 32))
    for lane in range(64):
        for e in range(8):
            a[lane % 32, 8 * (lane // 32) + e] = ((lane * 7 + e) % 13) * 0.01
            b[8 * (lane // 32) + e, lane % 32] = ((lane * 5 + e) % 11) * 0.02
    c = _bf16_round(a) @ _bf16_round(b)
    want = np.empty(64)
    for lane in range(64):
        rows = [8 * (j // 4) + 4 * (lane // 32) + j % 4 for j in range(16)]
        want[lane] = 8 * iters * c[rows, lane % 32].sum()
    got = host(out).reshape(blocks * 4, 64)
    assert np.all(np.isfinite(got))
    np.testing.assert_allclose(got, np.broadcast_to(want, got.shape), rtol=1e-4)


@pytest.mark.gpu
def test_mfma_probe_on_data_operands_computes_the_product():
    """The data-operand measurement kernel takes lane l's A operands from runs 0-3 and B
    operands from runs 4-5 of the caller's buffer and MFMA j uses A[j % 4], B[j % 2]: every
    lane's output equals iters * sum over j < 8 of its 16 entries of A[j % 4] B[j % 2]."""
    blocks, iters = 4, 16
    g = np.random.default_rng(5)
    ops = _bf16_round(g.standard_normal((6, 64, 8)))
    dev_ops = torch.from_numpy(ops.astype(np.float32)).to(torch.bfloat16).cuda().reshape(-1)
    out = torch.full((blocks * 256,), float("nan"), dtype=torch.float32, device="cuda")
    cwa.sa_probe_mfma_bf16_data(out, dev_ops, blocks, iters)
    torch.cuda.synchronize()
    def mat_a(i):
        a = np.zeros((32, 16))
        for lane in range(64):
            a[lane % 32, 8 * (lane // 32):8 * (lane // 32) + 8] = ops[i, lane]
        return a
    def mat_b(i):
        b = np.zeros((16, 32))
        for lane in range(64):
            b[8 * (lane // 32):8 * (lane // 32) + 8, lane % 32] = ops[4 + i, lane]
        return b
    want = np.zeros(64)
    for j in range(8):
        c = mat_a(j % 4) @ mat_b(j % 2)
        for lane in range(64):
            rows = [8 * (r // 4) + 4 * (lane // 32) + r % 4 for r in range(16)]
            want[lane] += iters * c[rows, lane % 32].sum()
    got = host(out).reshape(blocks * 4, 64)
    assert np.all(np.isfinite(got))
    scale = iters * 8 * 16 * 16 * np.abs(ops).max() ** 2       # bound on the summed magnitudes
    np.testing.assert_allclose(got, np.broadcast_to(want, got.shape), rtol=0, atol=1e-5 * scale)
