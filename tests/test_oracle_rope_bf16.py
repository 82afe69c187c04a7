"""Pins for the oracle's RoPE and bfloat16 rounding (CPU only).

Each test checks the oracle against something other than itself: hand-worked
values from the rotation's definition, complex multiplication (NumPy
complex128), group properties of rotations, and torch's float32 -> bfloat16
conversion as a library special case.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import rope3d, rope_split, rotate_temporal, round_bf16, token_coords
from oracle.rope import rope_freqs

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _ev(expr):
    return float(eval(expr, {"cos": math.cos, "sin": math.sin, "__builtins__": {}}))


def test_rope_hand_values():
    g = json.load(open(os.path.join(GOLD, "rope_hand.json")))
    for case in g["cases"]:
        u = np.array(case["u"], dtype=np.float64)[None, :]
        got = rope3d(u, [case["t"]], [case["y"]], [case["x"]], tuple(case["split"]))[0]
        want = np.array([_ev(e) for e in case["expect"]])
        np.testing.assert_allclose(got, want, rtol=0, atol=1e-14)


def test_default_splits_and_coords():
    g = json.load(open(os.path.join(GOLD, "rope_hand.json")))
    for d, s in g["default_splits"].items():
        assert rope_split(int(d)) == tuple(s)
    tc = g["token_coords"]
    f, y, x = token_coords(tc["n_tokens"], tc["frame_h"], tc["frame_w"])
    assert f.tolist() == tc["frame"] and y.tolist() == tc["y"] and x.tolist() == tc["x"]


def test_bad_split_rejected():
    for bad in [(43, 43, 42), (44, 42, 40), (-2, 66, 64)]:
        with pytest.raises(ValueError):
            rope_split(128, bad)


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


@pytest.mark.parametrize("D", [64, 128, 12])
def test_rope_identity_at_zero_and_norm(D):
    split = rope_split(D)
    u = _rand((50, D), 1)
    z = np.zeros(50, dtype=np.int64)
    np.testing.assert_array_equal(rope3d(u, z, z, z, split), u)
    rng = np.random.default_rng(2)
    t, y, x = (rng.integers(-500, 500, 50) for _ in range(3))
    r = rope3d(u, t, y, x, split)
    np.testing.assert_allclose(np.linalg.norm(r, axis=1), np.linalg.norm(u, axis=1), rtol=1e-13)
    # per pair norms are preserved too (each pair is a plane rotation)
    np.testing.assert_allclose(np.hypot(r[:, 0::2], r[:, 1::2]), np.hypot(u[:, 0::2], u[:, 1::2]),
                               rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("D", [64, 128])
def test_rope_equals_complex_multiplication(D):
    split = rope_split(D)
    u = _rand((40, D), 3)
    rng = np.random.default_rng(4)
    t, y, x = (rng.integers(0, 3000, 40) for _ in range(3))
    got = rope3d(u, t, y, x, split)
    z = u[:, 0::2] + 1j * u[:, 1::2]                      # pairs as complex numbers
    # angle of every pair: segment-wise position times frequency
    ang = []
    for seg, pos in zip(split, (t, y, x)):
        j = np.arange(seg // 2)
        ang.append(pos[:, None] * (10000.0 ** (-(2.0 * j) / seg))[None, :])
    ang = np.concatenate(ang, axis=1)
    zr = z * np.exp(1j * ang)
    want = np.empty_like(u)
    want[:, 0::2], want[:, 1::2] = zr.real, zr.imag
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


def test_rope_composition_pins_refresh():
    D = 128
    split = rope_split(D)
    u = _rand((30, D), 5)
    rng = np.random.default_rng(6)
    t, y, x = (rng.integers(0, 4000, 30) for _ in range(3))
    for delta in [1, 7, 64, 1234, -9]:
        a = rotate_temporal(rope3d(u, t, y, x, split), -delta, split)
        b = rope3d(u, t - delta, y, x, split)
        np.testing.assert_allclose(a, b, rtol=0, atol=1e-11)
    # rotate_temporal touches only the temporal segment
    r = rotate_temporal(u, 17, split)
    np.testing.assert_array_equal(r[:, split[0]:], u[:, split[0]:])


@pytest.mark.parametrize("axis", [0, 1, 2])
def test_rope_shift_invariance_of_dot_products(axis):
    """<R(p+delta) q, R(p'+delta) k> = <R(p) q, R(p') k> for a common shift on one axis."""
    D = 128
    split = rope_split(D)
    q, k = _rand((25, D), 7), _rand((25, D), 8)
    rng = np.random.default_rng(9)
    pq = [rng.integers(0, 500, 25) for _ in range(3)]
    pk = [rng.integers(0, 500, 25) for _ in range(3)]
    base = np.sum(rope3d(q, *pq, split) * rope3d(k, *pk, split), axis=1)
    for delta in [3, 250, -40, 10 ** 5]:
        sq = [p + (delta if i == axis else 0) for i, p in enumerate(pq)]
        sk = [p + (delta if i == axis else 0) for i, p in enumerate(pk)]
        shifted = np.sum(rope3d(q, *sq, split) * rope3d(k, *sk, split), axis=1)
        np.testing.assert_allclose(shifted, base, rtol=0, atol=1e-10 * max(1, abs(delta) / 1e3))
    # and a non-common shift does change them (the test would catch a dropped rotation)
    sq = [p + (5 if i == axis else 0) for i, p in enumerate(pq)]
    moved = np.sum(rope3d(q, *sq, split) * rope3d(k, *pk, split), axis=1)
    assert np.max(np.abs(moved - base)) > 1e-3


def test_rope_freqs_values():
    np.testing.assert_allclose(rope_freqs(44, 10000.0)[[0, 1, 21]],
                               [1.0, 10000 ** (-2 / 44), 10000 ** (-42 / 44)], rtol=1e-15)
    np.testing.assert_allclose(rope_freqs(4, 100.0), [1.0, 0.1], rtol=1e-15)


# --- bfloat16 rounding --------------------------------------------------------

def test_bf16_hand_cases():
    h = float.fromhex
    cases = {
        1.0 + 2 ** -8: 1.0,                          # tie -> even (down)
        1.0 + 3 * 2 ** -8: 1.0 + 2 ** -6,            # tie -> even (up)
        1.0 + 2 ** -8 + 2 ** -40: 1.0 + 2 ** -7,     # just above a tie: up (fp32 first would give 1.0)
        -(1.0 + 2 ** -8 + 2 ** -40): -(1.0 + 2 ** -7),
        h("0x1.ffp127"): math.inf,                   # tie between max finite and 2^128 -> inf
        h("0x1.fefp127"): h("0x1.fep127"),
        2.0 ** -133: 2.0 ** -133,                    # smallest subnormal
        3 * 2.0 ** -134: 2.0 ** -132,                # subnormal tie -> even
        2.0 ** -135: 0.0,                            # below half the smallest subnormal
        0.0: 0.0, 3.0: 3.0, 1 / 3: h("0x1.56p-2"),
    }
    for x, want in cases.items():
        assert round_bf16(np.array([x]))[0] == want, (x, want)
    assert math.isnan(round_bf16(np.array([math.nan]))[0])


def test_bf16_matches_torch_on_fp32_values():
    rng = np.random.default_rng(10)
    x = np.concatenate([rng.standard_normal(200000) * 10.0 ** rng.integers(-30, 30, 200000),
                        rng.standard_normal(1000) * 1e-39]).astype(np.float32)
    want = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    got = round_bf16(x.astype(np.float64))
    np.testing.assert_array_equal(got, want)
