"""Pins for the oracle's masked softmax attention (CPU only).

Brute force on tiny inputs, closed forms, probability rows summing to one,
permutation invariance, a log-sum-exp library routine, and fp64 CPU
scaled_dot_product_attention as a library special case (no RoPE, no mask).
"""
import math

import numpy as np
import pytest
import torch
from scipy.special import logsumexp

from oracle import attend, attend_bruteforce, attention_probs


def _r(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


@pytest.mark.parametrize("nq,nk,d", [(1, 1, 1), (3, 5, 4), (4, 16, 8), (7, 13, 6)])
def test_bruteforce(nq, nk, d):
    q, k, v = _r((nq, d), 1), _r((nk, d), 2), _r((nk, d + 1), 3)
    o, l = attend(q, k, v, 0.7)
    ob, lb = attend_bruteforce(q, k, v, 0.7)
    np.testing.assert_allclose(o, ob, rtol=0, atol=1e-13)
    np.testing.assert_allclose(l, lb, rtol=0, atol=1e-13)


def test_rows_sum_to_one_and_lse():
    q, k = _r((20, 64), 4), _r((300, 64), 5) * 3
    p = attention_probs(q, k, 0.125)
    np.testing.assert_allclose(p.sum(axis=1), 1.0, rtol=0, atol=1e-14)
    assert np.all(p >= 0)
    _, l = attend(q, k, _r((300, 64), 6), 0.125)
    np.testing.assert_allclose(l, logsumexp((q @ k.T) * 0.125, axis=1), rtol=1e-14)


@pytest.mark.parametrize("nq,nk,d", [(5, 5, 4), (3, 9, 6), (8, 8, 3), (6, 2, 5)])
def test_attention_probs_are_the_weights(nq, nk, d):
    """attention_probs is the weight matrix of the same definition: with the identity as
    the values, the scalar-loop twin returns exactly the weights (row i of its output is
    p_i.), the weights times any V give attend()'s output, and log p_ij = s_ij - LSE_i.
    Square cases (nq = nk) catch a transposed score product, which has the right shape
    there."""
    q, k = _r((nq, d), 11), _r((nk, d), 12)
    p = attention_probs(q, k, 0.6)
    assert p.shape == (nq, nk)
    pb, lb = attend_bruteforce(q, k, np.eye(nk), 0.6)
    np.testing.assert_allclose(p, pb, rtol=0, atol=1e-14)
    v = _r((nk, 5), 13)
    o, l = attend(q, k, v, 0.6)
    np.testing.assert_allclose(p @ v, o, rtol=0, atol=1e-13)
    s = np.array([[0.6 * sum(float(a) * float(b) for a, b in zip(qi, kj)) for kj in k] for qi in q])
    np.testing.assert_allclose(np.log(p), s - lb[:, None], rtol=0, atol=1e-12)


def test_closed_forms():
    k, v = _r((9, 4), 7), _r((9, 3), 8)
    # q = 0: uniform weights -> mean of the visible values
    o, l = attend(np.zeros((2, 4)), k, v, 1.0)
    np.testing.assert_allclose(o, np.tile(v.mean(axis=0), (2, 1)), atol=1e-15)
    np.testing.assert_allclose(l, math.log(9), atol=1e-15)
    # a single visible key gives its value; lse = its score
    q = _r((3, 4), 9)
    o, l = attend(q, k[:1], v[:1], 0.5)
    np.testing.assert_allclose(o, np.tile(v[0], (3, 1)), atol=1e-15)
    np.testing.assert_allclose(l, 0.5 * (q @ k[0]), atol=1e-14)
    # logits (a, a + ln 2) -> weights (1/3, 2/3)
    a = 0.37
    kk = np.array([[a], [a + math.log(2.0)]])
    vv = np.array([[3.0, 0.0], [0.0, 6.0]])
    o, _ = attend(np.array([[1.0]]), kk, vv, 1.0)
    np.testing.assert_allclose(o, [[1.0, 4.0]], atol=1e-14)
    # a very large scale picks the value of the argmax key
    q = _r((5, 4), 10)
    o, _ = attend(q, k, v, 1e6)
    np.testing.assert_allclose(o, v[np.argmax(q @ k.T, axis=1)], atol=1e-12)


def test_permutation_invariance():
    q, k, v = _r((16, 32), 11), _r((100, 32), 12), _r((100, 32), 13)
    perm = np.random.default_rng(14).permutation(100)
    o1, l1 = attend(q, k, v, 0.2)
    o2, l2 = attend(q, k[perm], v[perm], 0.2)
    np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-13)
    np.testing.assert_allclose(l1, l2, rtol=0, atol=1e-13)
    # a permutation of k alone (a transposed-operand style mistake) must change the result
    o3, _ = attend(q, k[perm], v, 0.2)
    assert np.max(np.abs(o3 - o1)) > 1e-2


def test_blocked_rows_equal_unblocked():
    q, k, v = _r((1000, 16), 15), _r((50, 16), 16), _r((50, 16), 17)
    o1, l1 = attend(q, k, v, 0.3, block_rows=1000)
    o2, l2 = attend(q, k, v, 0.3, block_rows=7)
    np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-14)
    np.testing.assert_allclose(l1, l2, rtol=0, atol=1e-14)


def test_matches_torch_sdpa_fp64():
    q, k, v = _r((2, 3, 40, 64), 18), _r((2, 3, 90, 64), 19), _r((2, 3, 90, 64), 20)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v)).numpy()
    for b in range(2):
        for h in range(3):
            o, _ = attend(q[b, h], k[b, h], v[b, h], 1.0 / 8.0)
            np.testing.assert_allclose(o, ref[b, h], rtol=0, atol=1e-13)


def test_no_keys_is_an_error():
    with pytest.raises(ValueError):
        attend(np.zeros((1, 4)), np.zeros((0, 4)), np.zeros((0, 4)), 1.0)
