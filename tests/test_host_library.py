"""CPU tests of the C-ABI library (no GPU, no kernel launches).

* libsa.so loads and exports every function include/sa.h declares;
* planning handles (created without a workspace) run the full bookkeeping:
  their visible sets (chunk ids, positions), refresh deltas and positions are
  compared bit-exactly with the oracle's stream semantics on seeded random
  operation sequences; the physical slots seen by an attend must form the
  prefix [0, visible_chunks) that the attention kernel reads;
* error conventions: status codes, state unchanged after an error.
"""
import copy
import ctypes
import os
import re

import numpy as np
import pytest

import causal_windowed_attention_amd as cwa
from causal_windowed_attention_amd import _lib as L
from oracle import HistoryOracle, SHIFT_SINK, StreamSpec
from oracle.stream import StreamError

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_exports_every_declared_symbol():
    hdr = open(os.path.join(ROOT, "include", "sa.h")).read()
    hdr = re.sub(r"/\*.*?\*/", "", hdr, flags=re.S)
    declared = set(re.findall(r"\b(sa_[a-z0-9_]+)\s*\(", hdr))
    assert len(declared) >= 14
    lib = L.load()
    for name in sorted(declared):
        assert hasattr(lib, name), name
    assert declared == set(L.SIGNATURES), declared ^ set(L.SIGNATURES)


def test_struct_sizes_match_header():
    import ctypes
    assert ctypes.sizeof(L.sa_config) == 72
    assert ctypes.sizeof(L.sa_state) == 16 + 14 * 4
    assert ctypes.sizeof(L.sa_slot_info) == 16


def _cfg(**kw):
    base = dict(batch=1, heads=2, head_dim=64, frame_h=2, frame_w=3, frames_per_chunk=2,
                sink_chunks=1, window_chunks=2, dtype="bf16")
    base.update(kw)
    return cwa.make_config(**base)


def _spec(cfg):
    return StreamSpec(batch=cfg.batch, heads=cfg.heads, head_dim=cfg.head_dim,
                      frame_h=cfg.frame_h, frame_w=cfg.frame_w,
                      frames_per_chunk=cfg.frames_per_chunk, sink_chunks=cfg.sink_chunks,
                      window_chunks=cfg.window_chunks, max_t=cfg.max_t)


def _lib_visible(s: cwa.Stream):
    st = s.query()
    seen = []
    for slot in range(st["n_slots"]):
        info = s.slot(slot)
        if slot < st["visible_chunks"]:
            assert info["kind"] != cwa.SA_SLOT_EMPTY, (slot, info)
            kind = {cwa.SA_SLOT_SINK: "sink", cwa.SA_SLOT_WINDOW: "window",
                    cwa.SA_SLOT_STAGING: "self"}[info["kind"]]
            seen.append((kind, info["chunk_id"], info["t0"]))
        else:
            assert info["kind"] == cwa.SA_SLOT_EMPTY, (slot, info)
    assert [k for k, _, _ in seen].count("self") == 1
    assert seen.index([x for x in seen if x[0] == "self"][0]) == st["staging_slot"]
    return st, sorted(seen, key=lambda x: (x[0] != "sink", x[2], x[1]))


def _oracle_visible(orc):
    return sorted(orc.visible(), key=lambda x: (x[0] != "sink", x[2], x[1]))


def _dummy(spec, n_tokens=None):
    n = spec.tokens_per_chunk if n_tokens is None else n_tokens
    return np.zeros((spec.batch, n, spec.heads, spec.head_dim))


@pytest.mark.parametrize("S,W,seed", [(1, 2, 0), (1, 6, 1), (2, 3, 2), (0, 2, 3), (1, 0, 4),
                                      (0, 0, 5), (3, 1, 6), (1, 3, 7), (4, 4, 8)])
def test_planning_bookkeeping_matches_oracle(S, W, seed):
    cfg = _cfg(sink_chunks=S, window_chunks=W)
    s = cwa.Stream(cfg, planning=True)
    spec = _spec(cfg)
    orc = HistoryOracle(spec)
    g = np.random.default_rng(seed)
    z = _dummy(spec)
    for step in range(300):
        st, vis = _lib_visible(s)
        assert vis == _oracle_visible(orc), (step, vis, orc.visible())
        assert st["t_next"] == orc.t_next and st["n_appends"] == orc.n_appends
        assert st["sink_fill"] == orc.sink_fill and st["ring_commits"] == orc.ring_commits
        assert st["visible_keys"] == len(orc.visible()) * (cfg.frames_per_chunk * 6)
        r = g.random()
        if r < 0.5:
            zero_copy = g.random() < 0.5
            if zero_copy:
                s.chunk_attend(None, None, None)
                s.kv_append(None, None)
            else:
                cwa.sa_kv_append(s.handle, 1, 1)       # explicit k, v (ignored by a planning handle)
            orc.append(z, z)
        elif r < 0.7:
            base = int(g.choice([-1, 0, 2, 5, 11]))
            flags = SHIFT_SINK if g.random() < 0.3 else 0
            d_lib = s.rope_refresh(base, flags)
            d_orc = orc.refresh(None if base == -1 else base, flags)
            assert d_lib == d_orc
            assert s.query()["last_delta"] == d_orc
        elif r < 0.8:
            if S > 0:
                cwa.sa_sink_update(s.handle, 1, 1)
                orc.sink_update(_dummy(spec, S * spec.tokens_per_chunk),
                                _dummy(spec, S * spec.tokens_per_chunk))
            else:
                with pytest.raises(cwa.SaError) as e:
                    cwa.sa_sink_update(s.handle, 1, 1)
                assert e.value.status == L.SA_ERR_BAD_STATE
        else:
            s.chunk_attend(None, None, None)
            st = s.query()
            assert st["staged_valid"] == 1
            assert st["last_key_tiles"] == -(-st["visible_keys"] // 64)
    s.close()


def _buffer_slots_expected(s, orc, spec, j, steps):
    """Physical slots buffer chunk j must read: the oracle's visible set after committing
    buffer chunks 0..j-1 (moving buffer) or as it stands (steps), mapped to slots (sink
    slots, window slots by chunk id, buffer slot S + W + 1 + i for buffer chunk i)."""
    tmp = copy.deepcopy(orc)
    z = _dummy(spec)
    for _ in range(0 if steps else j):
        tmp.append(z, z)
    st = s.query()
    by_id = {}
    for slot in range(st["n_slots"]):
        info = s.slot(slot)
        if info["kind"] == cwa.SA_SLOT_WINDOW:
            by_id[info["chunk_id"]] = slot
    buf0 = spec.sink_chunks + spec.window_chunks + 1
    want = {buf0 + j} if steps else set()
    for kind, cid, _ in tmp.visible():
        if kind == "sink" or (steps and kind == "self"):     # steps: self is buffer chunk j
            continue
        want.add(by_id[cid] if cid < orc.n_appends else buf0 + cid - orc.n_appends)
    return want | set(range(orc.sink_fill))


@pytest.mark.parametrize("S,W,NB,seed", [(1, 2, 4, 0), (1, 6, 8, 1), (2, 3, 5, 2), (0, 2, 3, 3),
                                         (1, 0, 2, 4), (0, 0, 1, 5), (3, 1, 8, 6)])
@pytest.mark.parametrize("steps", [False, True])
def test_buffer_plan_matches_oracle(S, W, NB, seed, steps):
    """Bit-exact: the key segments of every buffer chunk cover exactly the slots of the
    chunks the oracle's buffer reading makes visible, as disjoint sorted ranges."""
    cfg = _cfg(sink_chunks=S, window_chunks=W, max_buffer_chunks=NB)
    s = cwa.Stream(cfg, planning=True)
    spec = _spec(cfg)
    nc = spec.tokens_per_chunk
    orc = HistoryOracle(spec)
    g = np.random.default_rng(seed)
    z = _dummy(spec)
    flags = L.SA_BUFFER_STEPS if steps else 0
    for step in range(120):
        n = int(g.integers(1, NB + 1))
        if orc.sink_fill < S and not steps:
            with pytest.raises(cwa.SaError) as e:
                s.buffer_plan(n)
            assert e.value.status == L.SA_ERR_BAD_STATE
        else:
            plan = s.buffer_plan(n, steps=steps)
            for j, segs in enumerate(plan):
                assert 1 <= len(segs) <= L.SA_MAX_KEY_SEGMENTS
                slots = set()
                for a, (lo, hi) in enumerate(segs):
                    assert lo % nc == 0 and hi % nc == 0 and lo < hi
                    if a:
                        assert lo > segs[a - 1][1]               # sorted, disjoint, not adjacent
                    slots |= set(range(lo // nc, hi // nc))
                assert slots == _buffer_slots_expected(s, orc, spec, j, steps), (step, j, segs)
            before = s.query()
            cwa.sa_buffer_attend(s.handle, None, None, None, n, None, flags=flags)
            after = s.query()
            assert after["staged_valid"] == 0
            for key in ("t_next", "n_appends", "sink_fill", "ring_commits", "visible_keys"):
                assert after[key] == before[key]
        r = g.random()
        if r < 0.75:
            cwa.sa_kv_append(s.handle, 1, 1)
            orc.append(z, z)
        elif r < 0.9:
            base = int(g.choice([-1, 0, 3]))
            assert s.rope_refresh(base, 0) == orc.refresh(None if base == -1 else base, 0)
        elif S > 0:
            cwa.sa_sink_update(s.handle, 1, 1)
            orc.sink_update(_dummy(spec, S * nc), _dummy(spec, S * nc))
    s.close()


def test_buffer_attend_errors():
    for kw, code in [(dict(max_buffer_chunks=-1), L.SA_ERR_INVALID_ARGUMENT),
                     (dict(max_buffer_chunks=L.SA_MAX_BUFFER_CHUNKS + 1), L.SA_ERR_INVALID_ARGUMENT)]:
        assert cwa.sa_config_check(_cfg(**kw)) == code
    cfg = _cfg(max_buffer_chunks=2)
    cfg.reserved = 1
    assert cwa.sa_config_check(cfg) == L.SA_ERR_INVALID_ARGUMENT
    s = cwa.Stream(_cfg(max_buffer_chunks=0), planning=True)
    cwa.sa_kv_append(s.handle, 1, 1)                   # sink full
    with pytest.raises(cwa.SaError) as e:
        s.buffer_plan(1)
    assert e.value.status == L.SA_ERR_INVALID_ARGUMENT
    s = cwa.Stream(_cfg(max_buffer_chunks=3, max_t=8), planning=True)   # F = 2
    with pytest.raises(cwa.SaError) as e:
        cwa.sa_buffer_attend(s.handle, None, None, None, 1, None)       # sink not full
    assert e.value.status == L.SA_ERR_BAD_STATE
    cwa.sa_kv_append(s.handle, 1, 1)                   # t_next = 2
    for n, code in [(0, L.SA_ERR_INVALID_ARGUMENT), (4, L.SA_ERR_INVALID_ARGUMENT),
                    (3, L.SA_OK)]:                      # chunks at t = 2, 4, 6 < 8
        if code == L.SA_OK:
            cwa.sa_buffer_attend(s.handle, None, None, None, n, None)
        else:
            with pytest.raises(cwa.SaError) as e:
                cwa.sa_buffer_attend(s.handle, None, None, None, n, None)
            assert e.value.status == code
    cwa.sa_kv_append(s.handle, 1, 1)                   # t_next = 4: t = 8 would be needed
    for flags in (0, L.SA_BUFFER_STEPS):
        with pytest.raises(cwa.SaError) as e:
            cwa.sa_buffer_attend(s.handle, None, None, None, 3, None, flags=flags)
        assert e.value.status == L.SA_ERR_POSITION_RANGE
    for flags in (2, 0x80000000):                       # unknown flags
        with pytest.raises(cwa.SaError) as e:
            cwa.sa_buffer_attend(s.handle, None, None, None, 1, None, flags=flags)
        assert e.value.status == L.SA_ERR_INVALID_ARGUMENT
    s = cwa.Stream(_cfg(sink_chunks=2, max_buffer_chunks=2), planning=True)
    assert s.buffer_plan(2, steps=True) == [[(s.Nc * 5, s.Nc * 6)], [(s.Nc * 6, s.Nc * 7)]]   # nothing committed


def test_zero_copy_commit_rules():
    s = cwa.Stream(_cfg(), planning=True)
    with pytest.raises(cwa.SaError) as e:          # nothing staged yet
        s.kv_append(None, None)
    assert e.value.status == L.SA_ERR_BAD_STATE
    s.chunk_attend(None, None, None)
    assert s.rope_refresh(0, 0) == 0                # Delta = 0 keeps the staged chunk valid
    assert s.query()["staged_valid"] == 1
    s.kv_append(None, None)
    assert s.query()["n_appends"] == 1
    with pytest.raises(cwa.SaError):                # consumed
        s.kv_append(None, None)
    for _ in range(4):
        s.chunk_attend(None, None, None)
        s.kv_append(None, None)
    s.chunk_attend(None, None, None)
    assert s.rope_refresh(-1, 0) != 0               # moving positions invalidates the staged K
    with pytest.raises(cwa.SaError):
        s.kv_append(None, None)
    s.chunk_attend(None, None, None)
    cwa.sa_sink_update(s.handle, 1, 1)              # so does a sink update
    with pytest.raises(cwa.SaError):
        s.kv_append(None, None)


def test_position_range_and_state_unchanged():
    cfg = _cfg(max_t=7, sink_chunks=1, window_chunks=1)
    s = cwa.Stream(cfg, planning=True)
    for _ in range(3):                               # chunks at t = 0, 2, 4 (F = 2)
        s.chunk_attend(None, None, None)
        s.kv_append(None, None)
    before = s.query()
    with pytest.raises(cwa.SaError) as e:            # t = 6..7 would reach max_t
        s.chunk_attend(None, None, None)
    assert e.value.status == L.SA_ERR_POSITION_RANGE
    with pytest.raises(cwa.SaError) as e:
        cwa.sa_kv_append(s.handle, 1, 1)
    assert e.value.status == L.SA_ERR_POSITION_RANGE
    assert s.query() == before
    assert s.rope_refresh(-1, 0) == 2                # oldest window chunk t0 = 4 -> base 2
    s.chunk_attend(None, None, None)                 # now at t = 4..5


def test_error_codes():
    lib = L.load()
    assert cwa.sa_status_string(0) == "SA_OK"
    assert cwa.sa_status_string(5) == "SA_ERR_POSITION_RANGE"
    bad = [
        (dict(batch=0), L.SA_ERR_INVALID_ARGUMENT),
        (dict(head_dim=63), L.SA_ERR_INVALID_ARGUMENT),
        (dict(head_dim=96), L.SA_ERR_UNSUPPORTED),
        (dict(sink_chunks=-1), L.SA_ERR_INVALID_ARGUMENT),
        (dict(rope_dims=(30, 20, 20)), L.SA_ERR_INVALID_ARGUMENT),
        (dict(rope_dims=(25, 20, 19)), L.SA_ERR_INVALID_ARGUMENT),
        (dict(frames_per_chunk=40, head_dim=128), L.SA_ERR_UNSUPPORTED),
        # 9 slots x 2^20 keys x 128 x 2 bytes per (b, h) >= 2^31: past the 32-bit buffer range
        (dict(frame_h=1024, frame_w=1024, frames_per_chunk=1, window_chunks=7, head_dim=128),
         L.SA_ERR_UNSUPPORTED),
        (dict(dtype=7), L.SA_ERR_INVALID_ARGUMENT),
        (dict(rope_theta=0.5), L.SA_ERR_INVALID_ARGUMENT),
        (dict(max_t=1), L.SA_ERR_POSITION_RANGE),
    ]
    for kw, code in bad:
        cfg = _cfg(**kw)
        assert cwa.sa_config_check(cfg) == code, kw
        assert cwa.sa_workspace_bytes(cfg) == 0
        with pytest.raises(cwa.SaError) as e:
            cwa.sa_stream_create(cfg, None)
        assert e.value.status == code
    cfg = _cfg(rope_dims=(24, 20, 20))
    assert cwa.sa_config_check(cfg) == 0
    s = cwa.Stream(cfg, planning=True)
    with pytest.raises(cwa.SaError) as e:
        s.rope_refresh(-5, 0)
    assert e.value.status == L.SA_ERR_INVALID_ARGUMENT
    with pytest.raises(cwa.SaError) as e:
        s.rope_refresh(-1, 4)
    assert e.value.status == L.SA_ERR_INVALID_ARGUMENT
    with pytest.raises(cwa.SaError):
        s.set_option(cwa.SA_OPT_KV_SPLITS, 99)
    with pytest.raises(cwa.SaError):
        s.set_option(cwa.SA_OPT_PROFILE, 1)          # a planning handle has no device work
    with pytest.raises(cwa.SaError):
        s.set_option(42, 0)
    with pytest.raises(cwa.SaError):
        s.slot(-1)
    with pytest.raises(cwa.SaError):
        s.slot(s.query()["n_slots"])
    assert lib.sa_stream_destroy(None) == 0
    assert lib.sa_chunk_attend(None, None, None, None, None, None, None) == L.SA_ERR_INVALID_ARGUMENT


def test_workspace_layout_and_plans():
    import synth
    for name in ["wan1.3b", "wan14b_b4", "hybrid1280x704", "long512p", "tiny_f32"]:
        w = synth.WORKLOADS[name]
        cfg = cwa.make_config(w.batch, w.heads, w.head_dim, w.frame_h, w.frame_w,
                              w.frames_per_chunk, w.sink_chunks, w.window_chunks, dtype=w.dtype)
        s = cwa.Stream(cfg, planning=True)
        lay = s.layout()
        nc, bh, d = w.tokens_per_chunk, w.batch * w.heads, w.head_dim
        slots = w.sink_chunks + w.window_chunks + 1
        elem = 2 if w.dtype == "bf16" else 4
        assert lay["k_bh_stride"] == lay["key_stride"] * d * elem
        assert lay["key_stride"] % 64 == 0 and lay["key_stride"] >= slots * nc
        assert lay["vt_offset"] >= lay["k_offset"] + bh * lay["k_bh_stride"]
        assert lay["q_offset"] >= lay["vt_offset"] + bh * lay["vt_bh_stride"]
        for off in ("k_offset", "vt_offset", "q_offset", "partial_offset", "table_offset"):
            assert lay[off] % 256 == 0
        assert cwa.sa_workspace_bytes(cfg) >= lay["table_offset"] + lay["table_bytes"]
        for c in range(slots + 2):
            s.chunk_attend(None, None, None)
            st = s.query()
            assert st["visible_chunks"] == min(c, slots - 1) + 1
            bm = 256 if w.dtype == "bf16" else 64
            bn = 64 if w.dtype == "bf16" else 32
            assert st["last_q_tiles"] == -(-nc // bm)
            assert st["last_key_tiles"] == -(-st["visible_keys"] // bn)
            assert 1 <= st["last_kv_splits"] <= lay["max_kv_splits"]
            s.kv_append(None, None)
        assert s.query()["visible_keys"] == slots * nc


def test_mfma_probe_argument_errors():
    """The measurement kernel's entry point validates before touching the device."""
    lib = L.load()
    assert lib.sa_probe_mfma_bf16(None, 1, 1, None) == L.SA_ERR_INVALID_ARGUMENT
    fake = ctypes.c_void_p(0x1000)             # never dereferenced: rejected on the host
    assert lib.sa_probe_mfma_bf16(fake, 0, 1, None) == L.SA_ERR_INVALID_ARGUMENT
    assert lib.sa_probe_mfma_bf16(fake, 1, 0, None) == L.SA_ERR_INVALID_ARGUMENT
    assert lib.sa_probe_mfma_bf16(fake, (1 << 20) + 1, 1, None) == L.SA_ERR_INVALID_ARGUMENT
    assert lib.sa_probe_mfma_bf16_data(fake, None, 1, 1, None) == L.SA_ERR_INVALID_ARGUMENT
    assert lib.sa_probe_mfma_bf16_data(None, fake, 1, 1, None) == L.SA_ERR_INVALID_ARGUMENT
    assert lib.sa_probe_mfma_bf16_data(fake, ctypes.c_void_p(fake.value + 8), 1, 1, None) == L.SA_ERR_INVALID_ARGUMENT
    assert lib.sa_probe_mfma_bf16_data(fake, fake, 0, 1, None) == L.SA_ERR_INVALID_ARGUMENT
    assert lib.sa_probe_mfma_bf16_data(fake, fake, 1, 0, None) == L.SA_ERR_INVALID_ARGUMENT


def test_batch_attend_planning_semantics_and_errors():
    """A ragged batch is n chunk attends: each handle stages its chunk (a zero-copy commit
    follows), plans are per handle; every entry is validated before anything changes."""
    cfg = _cfg(window_chunks=3, max_t=40)
    hs = [cwa.Stream(cfg, planning=True) for _ in range(4)]
    for i, s in enumerate(hs):                       # different states: 0, 2, 4 and 6 commits
        for _ in range(2 * i):
            cwa.sa_kv_append(s.handle, 1, 1)
    cwa.sa_batch_attend(hs, None, None, None, None)
    for s in hs:
        st = s.query()
        assert st["staged_valid"] == 1
        assert st["last_key_tiles"] == -(-st["visible_keys"] // 64) and st["last_kv_splits"] == 1
        s.kv_append(None, None)                      # zero-copy commit of the staged chunk
    t_before = [s.query()["t_next"] for s in hs]
    for bad, code in [([], L.SA_ERR_INVALID_ARGUMENT), (hs + hs[:1], L.SA_ERR_INVALID_ARGUMENT),
                      ([hs[0], cwa.Stream(_cfg(window_chunks=2, max_t=40), planning=True)],
                       L.SA_ERR_INVALID_ARGUMENT)]:
        with pytest.raises(cwa.SaError) as e:
            cwa.sa_batch_attend(bad, None, None, None, None)
        assert e.value.status == code
    many = [cwa.Stream(cfg, planning=True) for _ in range(L.SA_MAX_BATCH_STREAMS + 1)]
    with pytest.raises(cwa.SaError) as e:
        cwa.sa_batch_attend(many, None, None, None, None)
    assert e.value.status == L.SA_ERR_INVALID_ARGUMENT
    while hs[3].query()["t_next"] + cfg.frames_per_chunk <= cfg.max_t:   # push one stream to the end
        cwa.sa_kv_append(hs[3].handle, 1, 1)
    staged = [s.query()["staged_valid"] for s in hs]
    with pytest.raises(cwa.SaError) as e:
        cwa.sa_batch_attend(hs, None, None, None, None)
    assert e.value.status == L.SA_ERR_POSITION_RANGE
    assert [s.query()["staged_valid"] for s in hs] == staged      # nothing changed
    assert [s.query()["t_next"] for s in hs[:3]] == t_before[:3]


def test_fp8_config_and_planning():
    """SA_FP8: head_dim 128 only; the cache and Q scratch take one byte per element; the
    attention kernel is always the ping-pong one; planning matches the bf16 tiling."""
    assert cwa.sa_config_check(_cfg(dtype="fp8", head_dim=64)) == L.SA_ERR_UNSUPPORTED
    c8, c16 = _cfg(dtype="fp8", head_dim=128), _cfg(dtype="bf16", head_dim=128)
    assert cwa.sa_config_check(c8) == 0
    assert cwa.sa_workspace_bytes(c8) < cwa.sa_workspace_bytes(c16)
    s8, s16 = cwa.Stream(c8, planning=True), cwa.Stream(c16, planning=True)
    l8, l16 = s8.layout(), s16.layout()
    assert l8["elem_bytes"] == 1 and l16["elem_bytes"] == 2
    assert l8["k_bh_stride"] * 2 == l16["k_bh_stride"] and l8["vt_bh_stride"] * 2 == l16["vt_bh_stride"]
    for v in (1, 2):
        with pytest.raises(cwa.SaError) as e:
            s8.set_option(cwa.SA_OPT_ATTN_VARIANT, v)
        assert e.value.status == L.SA_ERR_INVALID_ARGUMENT
    s8.set_option(cwa.SA_OPT_ATTN_VARIANT, 3)
    for _ in range(5):
        for s in (s8, s16):
            s.chunk_attend(None, None, None)
            s.kv_append()
    a, b = s8.query(), s16.query()
    for key in ("last_q_tiles", "last_key_tiles", "last_kv_splits", "visible_keys", "t_next"):
        assert a[key] == b[key], key
    s8.close()
    s16.close()


def test_gdn_sizes_and_errors():
    """The GDN entry points validate on the host before any device work."""
    need = cwa.sa_gdn_workspace_bytes(1, 3520, 16, 128)
    nb = 55
    floor = 16 * nb * (64 * 4 + 4 * 64 * 128 * 4 + 128 * 128 * 4)
    assert floor <= need <= floor + 6 * 256
    assert cwa.sa_gdn_workspace_bytes(1, 3520, 16, 96) == 0          # D must be 64 or 128
    assert cwa.sa_gdn_workspace_bytes(0, 10, 1, 64) == 0
    assert cwa.sa_gdn_workspace_bytes(1, 0, 1, 64) > 0                # no tokens is valid
    assert cwa.sa_gdn_workspace_bytes(1, (1 << 24) + 1, 1, 64) == 0
    fake = 1 << 20                                                    # never dereferenced
    args = dict(q=fake, k=fake, v=fake, alpha=fake, beta=fake, state_in=None, state_out=fake, out=fake,
                workspace=fake, workspace_bytes=need)
    for kw, code in [(dict(q=None), L.SA_ERR_INVALID_ARGUMENT), (dict(out=fake + 8), L.SA_ERR_INVALID_ARGUMENT),
                     (dict(alpha=fake + 2), L.SA_ERR_INVALID_ARGUMENT),
                     (dict(state_out=fake + 4), L.SA_ERR_INVALID_ARGUMENT),     # states move as float4s
                     (dict(state_in=fake + 8), L.SA_ERR_INVALID_ARGUMENT),
                     (dict(workspace_bytes=need - 1), L.SA_ERR_WORKSPACE_TOO_SMALL)]:
        a = dict(args, **kw)
        with pytest.raises(cwa.SaError) as e:
            cwa.sa_gdn_forward(1, 3520, 16, 128, a["q"], a["k"], a["v"], a["alpha"], a["beta"], a["state_in"],
                               a["state_out"], a["out"], a["workspace"], a["workspace_bytes"])
        assert e.value.status == code, kw
    with pytest.raises(cwa.SaError) as e:
        cwa.sa_gdn_forward(1, 10, 1, 80, fake, fake, fake, fake, fake, None, fake, fake, fake, need)
    assert e.value.status == L.SA_ERR_UNSUPPORTED


def test_c_consumer_builds_and_validates_before_any_device_call():
    """The plain C consumer of the ABI (tests/c_abi/sa_c_demo, built by build()) links
    against libsa.so and rejects bad arguments with status 2 before any HIP call, so
    this runs without a GPU."""
    import subprocess
    from causal_windowed_attention_amd import build as b
    assert os.path.exists(b.C_DEMO), "tests/c_abi/sa_c_demo is missing: run __graft_entry__.build()"
    r = subprocess.run([b.C_DEMO], capture_output=True, text=True, timeout=60)
    assert r.returncode == 2 and "usage" in r.stderr
    # head_dim 96 has no kernel: sa_config_check says so
    r = subprocess.run([b.C_DEMO, "/nonexistent", "1", "2", "96", "4", "4", "2", "1", "2", "3"],
                       capture_output=True, text=True, timeout=60)
    assert r.returncode == 2 and "unsupported" in r.stderr.lower(), r.stderr


def test_binding_rejects_wrong_tensors_before_any_call():
    """The binding checks shape, dtype and contiguity (and the device, on device handles)
    before calling the library; a planning handle shows the shape and dtype checks on the CPU."""
    import torch
    cfg = _cfg()
    s = cwa.Stream(cfg, planning=True)
    B, H, D = cfg.batch, cfg.heads, cfg.head_dim
    nc = cfg.frames_per_chunk * cfg.frame_h * cfg.frame_w
    good = torch.zeros((B, nc, H, D), dtype=torch.bfloat16)
    bad_shape = torch.zeros((B, nc + 1, H, D), dtype=torch.bfloat16)
    bad_dtype = torch.zeros((B, nc, H, D), dtype=torch.float32)
    strided = torch.zeros((B, nc, H, 2 * D), dtype=torch.bfloat16)[..., :D]
    before = s.query()
    for bad in (bad_shape, bad_dtype, strided):
        with pytest.raises(ValueError):
            s.chunk_attend(good, bad, good, out=good)
        with pytest.raises(ValueError):
            s.kv_append(bad, good)
    with pytest.raises(ValueError):
        s.chunk_attend(good, good, good, out=good, lse=torch.zeros((B, H, nc + 1), dtype=torch.float32))
    with pytest.raises(ValueError):
        s.chunk_attend(good, good, good, out=good, lse=torch.zeros((B, H, nc), dtype=torch.float64))
    assert s.query() == before                   # nothing reached the library
    s2 = cwa.Stream(cfg, planning=True)
    with pytest.raises(ValueError):
        cwa.sa_batch_attend([s, s2], [good, good], [good, bad_shape], [good, good], [good, good])
    with pytest.raises(ValueError):
        cwa.sa_batch_attend([s, s2], [good, good], [good, good], [good, good], [good, good],
                            lses=[None, torch.zeros((B, H, 3), dtype=torch.float32)])
    assert s.query() == before and s2.query()["n_appends"] == 0
    # gdn_forward: host tensors are refused before any call
    q = torch.zeros((1, 64, 2, 128), dtype=torch.bfloat16)
    a = torch.ones((1, 2, 64), dtype=torch.float32)
    with pytest.raises(ValueError):
        cwa.gdn_forward(q, q, q, a, a)
    s.close()
    s2.close()
