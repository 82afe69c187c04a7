"""Pins of the E4M3 rounding the storage-emulating oracle uses for the fp8 cache.

The format is fixed by the OCP 8-bit floating point specification (E4M3: bias 7, 3
mantissa bits, no infinities, S.1111.111 is NaN, largest finite 448). The checks:
every finite code decoded from its bit fields (written out here, independently of
oracle/fp8.py) is a fixed point; every midpoint of two neighbouring values goes to the
even code and values beside it to the nearer neighbour; saturation at +-448; agreement
with PyTorch's float8_e4m3fn cast (a library routine) on random in-range values; and
the relative / absolute error bounds the fp8 parity tolerance is derived from.
"""
import math

import numpy as np
import pytest
import torch

from oracle import (HistoryOracle, RingOracle, StreamSpec, fp8_q_scale, is_e4m3_exact, rotate_temporal,
                    round_e4m3)


def _decode(code: int) -> float:
    s, e, m = code >> 7, (code >> 3) & 15, code & 7
    if e == 15 and m == 7:
        return float("nan")
    mag = (m / 8.0) * 2.0 ** -6 if e == 0 else (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return -mag if s else mag


CODES = {c: _decode(c) for c in range(256)}
POS = sorted((v, c) for c, v in CODES.items() if not np.isnan(v) and v >= 0 and c < 128)


def test_codes_are_fixed_points():
    vals = np.array([v for v in CODES.values() if not np.isnan(v)])
    assert len(vals) == 254 and max(vals) == 448.0 and min(vals) == -448.0
    np.testing.assert_array_equal(round_e4m3(vals), vals)
    assert is_e4m3_exact(vals)
    assert POS[1][0] == 2.0 ** -9 and POS[8][0] == 2.0 ** -6     # smallest subnormal, smallest normal


def test_midpoints_ties_to_even_and_neighbours():
    for (a, ca), (b, cb) in zip(POS[:-1], POS[1:]):
        mid = (a + b) / 2
        even = a if ca % 2 == 0 else b
        for sgn in (1.0, -1.0):
            assert round_e4m3(sgn * mid) == sgn * even, (a, b)
            assert round_e4m3(sgn * (mid - (b - a) * 1e-6)) == sgn * a
            assert round_e4m3(sgn * (mid + (b - a) * 1e-6)) == sgn * b
    assert np.signbit(round_e4m3(-2.0 ** -11))                    # rounds to -0


def test_saturation():
    x = np.array([448.0, 449.0, 463.9, 464.0, 479.0, 480.0, 1e6, np.inf])
    np.testing.assert_array_equal(round_e4m3(x), np.full(x.shape, 448.0))
    np.testing.assert_array_equal(round_e4m3(-x), np.full(x.shape, -448.0))
    assert np.isnan(round_e4m3(np.nan))


def test_matches_torch_float8_e4m3fn():
    g = np.random.default_rng(3)
    x = np.concatenate([g.standard_normal(20000), g.standard_normal(20000) * 40.0,
                        g.standard_normal(20000) * 0.01, g.uniform(-448, 448, 20000)])
    want = torch.from_numpy(x).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    np.testing.assert_array_equal(round_e4m3(x), want)


def test_error_bounds():
    g = np.random.default_rng(4)
    x = np.abs(np.concatenate([g.standard_normal(50000) * 50, g.uniform(0, 2.0 ** -6, 50000)]))
    x = x[x <= 448]
    r = round_e4m3(x)
    normal = x >= 2.0 ** -6
    assert np.all(np.abs(r[normal] - x[normal]) <= 2.0 ** -4 * x[normal])      # half of 2^-3 relative
    assert np.all(np.abs(r[~normal] - x[~normal]) <= 2.0 ** -10)               # half the subnormal step
    s = np.sort(g.uniform(-500, 500, 10000))
    assert np.all(np.diff(round_e4m3(s)) >= 0)                                  # monotone


def test_ring_oracle_fp8_storage():
    """The fp8 storage mode rounds exactly what is stored: the rotated K and V of a
    commit, and again the re-rotated K after a refresh."""
    spec = StreamSpec(batch=1, heads=2, head_dim=16, frame_h=2, frame_w=3, frames_per_chunk=2,
                      sink_chunks=1, window_chunks=2)
    g = np.random.default_rng(5)
    shape = (1, spec.tokens_per_chunk, 2, 16)
    pure, emu = RingOracle(spec), RingOracle(spec, storage="fp8")
    for c in range(4):
        k, v = g.standard_normal(shape), g.standard_normal(shape)
        pure.append(k, v)
        emu.append(k, v)
    for cid in (0, 2, 3):
        np.testing.assert_array_equal(emu.stored_k(cid), round_e4m3(pure.stored_k(cid)))
        np.testing.assert_array_equal(emu.stored_v(cid), round_e4m3(pure.stored_v(cid)))
    before = {cid: emu.stored_k(cid).copy() for cid in (2, 3)}
    delta = emu.refresh(None, 0)
    assert delta == 2 == pure.refresh(None, 0)       # oldest window chunk at t = 4, base S*F = 2
    for cid in (2, 3):
        want = round_e4m3(rotate_temporal(before[cid], -delta, spec.rope, spec.theta))
        np.testing.assert_array_equal(emu.stored_k(cid), want)
    q, k, v = (g.standard_normal(shape) for _ in range(3))
    o, _ = emu.attend(q, k, v)
    o_pure, _ = HistoryOracle(spec).attend(q, k, v)
    assert np.all(np.isfinite(o)) and np.abs(o - o_pure).max() > 0


def test_fp8_q_scale_and_stored_queries():
    """The query factor is softmax_scale * log2(e) times the power of two that brings it
    into [1, 2); the stored queries are E4M3 of the scaled values, scaled back."""
    for d, want in ((128, 1.0 / math.sqrt(128) * math.log2(math.e) * 8),
                    (64, 1.0 / 8.0 * math.log2(math.e) * 8)):
        spec = StreamSpec(batch=1, heads=1, head_dim=d, frame_h=2, frame_w=2, frames_per_chunk=1,
                          sink_chunks=1, window_chunks=1)
        kappa = fp8_q_scale(spec)
        assert 1.0 <= kappa < 2.0 and kappa == pytest.approx(want, rel=1e-15)
    assert fp8_q_scale(StreamSpec(batch=1, heads=1, head_dim=128, frame_h=2, frame_w=2,
                                  frames_per_chunk=1, sink_chunks=1, window_chunks=1,
                                  scale=1.0)) == pytest.approx(math.log2(math.e))   # k = 0
    spec = StreamSpec(batch=1, heads=2, head_dim=128, frame_h=2, frame_w=3, frames_per_chunk=2,
                      sink_chunks=1, window_chunks=2)
    g = np.random.default_rng(9)
    q, k, v = (g.standard_normal((1, spec.tokens_per_chunk, 2, 128)) for _ in range(3))
    emu, pure = RingOracle(spec, storage="fp8"), RingOracle(spec)
    qs, ks, vs = emu.staged(q, k, v)
    qp, kp, vp = pure.staged(q, k, v)
    kappa = fp8_q_scale(spec)
    np.testing.assert_array_equal(qs, round_e4m3(qp * kappa) / kappa)
    np.testing.assert_array_equal(ks, round_e4m3(kp))
    assert not np.array_equal(qs, round_e4m3(qp))                     # the factor matters


@pytest.mark.parametrize("steps", [False, True])
def test_buffer_operands_reproduce_buffer_attend(steps):
    """The per-chunk operands of a buffer attend (used to derive fp8 tolerances) give back
    the buffer attend's own outputs when attended."""
    from oracle import attend
    spec = StreamSpec(batch=1, heads=2, head_dim=16, frame_h=2, frame_w=3, frames_per_chunk=2,
                      sink_chunks=1, window_chunks=2)
    g = np.random.default_rng(11)
    nc = spec.tokens_per_chunk
    emu = RingOracle(spec, storage="fp8")
    for _ in range(3):
        emu.append(g.standard_normal((1, nc, 2, 16)), g.standard_normal((1, nc, 2, 16)))
    q, k, v = (g.standard_normal((1, 3 * nc, 2, 16)) for _ in range(3))
    out, lse = emu.buffer_attend(q, k, v, steps=steps)
    ops = emu.buffer_operands(q, k, v, steps=steps)
    assert len(ops) == 3
    for j, (qrot, keys, vals) in enumerate(ops):
        for h in range(2):
            K = np.concatenate([x[0, h] for x in keys])
            V = np.concatenate([x[0, h] for x in vals])
            o, l = attend(qrot[0, h], K, V, spec.softmax_scale)
            np.testing.assert_allclose(o, out[0, j * nc:(j + 1) * nc, h], rtol=0, atol=1e-12)
            np.testing.assert_allclose(l, lse[0, h, j * nc:(j + 1) * nc], rtol=0, atol=1e-12)
    assert len(ops[2][1]) == 4                        # sink, two window chunks, itself
