"""Pins of the gated delta rule oracle (oracle/gdn.py) against what the recurrence's
definition fixes, independently of the loop it is written as:

* no writing (beta = 0): the state only decays, S_t = (prod alpha) S_0, a closed form;
* delta-rule retrieval: with alpha = beta = 1 and orthonormal keys, writing (k_i, v_i)
  for a full basis replaces the state by [v_1 .. v_d], so querying k_j returns v_j;
* the one-step identity S_t k_t = alpha_t (1 - beta_t) S_{t-1} k_t + beta_t v_t for a
  unit key, checked at every step;
* splitting a sequence and carrying the state gives the same outputs and final state;
* a scalar-loop twin on tiny inputs.
"""
import numpy as np
import pytest

from oracle.gdn import gdn_recurrent


def _unit(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def _inputs(g, B=2, N=7, H=3, Dk=5, Dv=4):
    q = g.standard_normal((B, N, H, Dk))
    k = _unit(g.standard_normal((B, N, H, Dk)))
    v = g.standard_normal((B, N, H, Dv))
    alpha = g.uniform(0.5, 1.0, (B, H, N))
    beta = g.uniform(0.0, 1.0, (B, H, N))
    S0 = g.standard_normal((B, H, Dv, Dk))
    return q, k, v, alpha, beta, S0


def test_no_writing_only_decays():
    g = np.random.default_rng(1)
    q, k, v, alpha, beta, S0 = _inputs(g)
    o, S = gdn_recurrent(q, k, v, alpha, np.zeros_like(beta), S0)
    gam = np.cumprod(alpha, axis=2)                                   # [B, H, N]
    for t in range(q.shape[1]):
        np.testing.assert_allclose(o[:, t], gam[:, :, t, None] * np.einsum("bhvk,bhk->bhv", S0, q[:, t]),
                                   rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(S, gam[:, :, -1, None, None] * S0, rtol=1e-12, atol=1e-12)


def test_delta_rule_retrieval_with_orthonormal_keys():
    g = np.random.default_rng(2)
    d, dv = 6, 4
    basis = np.linalg.qr(g.standard_normal((d, d)))[0]               # orthonormal columns
    k = basis.T[None, :, None, :]                                     # [1, d, 1, d]: key i = column i
    v = g.standard_normal((1, d, 1, dv))
    S0 = g.standard_normal((1, 1, dv, d))
    ones = np.ones((1, 1, d))
    _, S = gdn_recurrent(np.zeros_like(k), k, v, ones, ones, S0)
    for j in range(d):                                                # every association stored
        np.testing.assert_allclose(S[0, 0] @ basis[:, j], v[0, j, 0], rtol=1e-12, atol=1e-12)
    # querying the keys afterwards (no more writing) reads the values back
    o, _ = gdn_recurrent(k, np.zeros_like(k), np.zeros_like(v), ones, np.zeros_like(ones), S)
    np.testing.assert_allclose(o[0, :, 0], v[0, :, 0], rtol=1e-12, atol=1e-12)


def test_one_step_identity_and_carried_state():
    g = np.random.default_rng(3)
    q, k, v, alpha, beta, S0 = _inputs(g, N=9)
    o_full, S_full = gdn_recurrent(q, k, v, alpha, beta, S0)
    S = S0
    for t in range(q.shape[1]):
        sl = slice(t, t + 1)
        o_t, S_new = gdn_recurrent(q[:, sl], k[:, sl], v[:, sl], alpha[:, :, sl], beta[:, :, sl], S)
        lhs = np.einsum("bhvk,bhk->bhv", S_new, k[:, t])
        rhs = (alpha[:, :, t] * (1 - beta[:, :, t]))[..., None] * np.einsum("bhvk,bhk->bhv", S, k[:, t]) \
            + beta[:, :, t, None] * v[:, t]
        np.testing.assert_allclose(lhs, rhs, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(o_t[:, 0], o_full[:, t], rtol=1e-12, atol=1e-12)
        S = S_new
    np.testing.assert_allclose(S, S_full, rtol=1e-12, atol=1e-12)
    # two halves with the state carried between them
    o1, S1 = gdn_recurrent(q[:, :4], k[:, :4], v[:, :4], alpha[:, :, :4], beta[:, :, :4], S0)
    o2, S2 = gdn_recurrent(q[:, 4:], k[:, 4:], v[:, 4:], alpha[:, :, 4:], beta[:, :, 4:], S1)
    np.testing.assert_allclose(np.concatenate([o1, o2], axis=1), o_full, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(S2, S_full, rtol=1e-12, atol=1e-12)


def test_zero_initial_state_default():
    g = np.random.default_rng(4)
    q, k, v, alpha, beta, _ = _inputs(g)
    o1, S1 = gdn_recurrent(q, k, v, alpha, beta)
    o2, S2 = gdn_recurrent(q, k, v, alpha, beta, np.zeros((2, 3, 4, 5)))
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(S1, S2)


def _scalar_twin(q, k, v, alpha, beta, S0):
    """The recurrence with explicit scalar loops: S_t[r][c] = a (S[r][c] - b (sum_e S[r][e]
    k[e]) k[c]) + b v[r] k[c]; o_t[r] = sum_c S_t[r][c] q[c]."""
    N, Dk, Dv = len(k), len(k[0]), len(v[0])
    S = [[float(S0[r][c]) for c in range(Dk)] for r in range(Dv)]
    out = []
    for t in range(N):
        a, b = float(alpha[t]), float(beta[t])
        Sk = [sum(S[r][e] * k[t][e] for e in range(Dk)) for r in range(Dv)]
        S = [[a * (S[r][c] - b * Sk[r] * k[t][c]) + b * v[t][r] * k[t][c] for c in range(Dk)] for r in range(Dv)]
        out.append([sum(S[r][c] * q[t][c] for c in range(Dk)) for r in range(Dv)])
    return np.array(out), np.array(S)


@pytest.mark.parametrize("seed", [5, 6])
def test_scalar_twin(seed):
    g = np.random.default_rng(seed)
    q, k, v, alpha, beta, S0 = _inputs(g, B=1, N=6, H=1, Dk=3, Dv=2)
    o, S = gdn_recurrent(q, k, v, alpha, beta, S0)
    o2, S2 = _scalar_twin(q[0, :, 0], k[0, :, 0], v[0, :, 0], alpha[0, 0], beta[0, 0], S0[0, 0])
    np.testing.assert_allclose(o[0, :, 0], o2, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(S[0, 0], S2, rtol=1e-12, atol=1e-12)


def _chunkwise(q, k, v, alpha, beta, S0, C):
    """The chunkwise rewriting the GPU path computes, for one (b, h): per chunk of C tokens
    with local cumulative gates gam_i = prod_{j<=i} alpha_j,
      pseudo-values U = T (V - diag(gam) K S0^T),  T = (I + diag(beta) A)^-1 diag(beta),
        A_ij = (gam_i / gam_j) k_i.k_j for j < i (else 0);
      outputs O = diag(gam) Q S0^T + ((Q K^T) o M) U,  M_ij = gam_i / gam_j for j <= i;
      next state S0 <- gam_C S0 + U^T diag(gam_C / gam) K.
    (From S_i = alpha_i S_{i-1} + u_i k_i^T with u_i = beta_i (v_i - alpha_i S_{i-1} k_i).)"""
    N = k.shape[0]
    out = np.empty((N, v.shape[1]))
    S = S0.copy()
    for c0 in range(0, N, C):
        K, V, Q = k[c0:c0 + C], v[c0:c0 + C], q[c0:c0 + C]
        n = K.shape[0]
        gam = np.cumprod(alpha[c0:c0 + C])
        ratio = gam[:, None] / gam[None, :]
        A = np.tril(ratio * (K @ K.T), -1)
        T = np.linalg.solve(np.eye(n) + beta[c0:c0 + C, None] * A, np.diag(beta[c0:c0 + C]))
        U = T @ (V - gam[:, None] * (K @ S.T))
        out[c0:c0 + n] = gam[:, None] * (Q @ S.T) + (np.tril(ratio) * (Q @ K.T)) @ U
        S = gam[-1] * S + U.T @ ((gam[-1] / gam)[:, None] * K)
    return out, S


@pytest.mark.parametrize("C", [1, 4, 64])
def test_chunkwise_rewriting_equals_the_recurrence(C):
    """The derivation the GPU kernels follow, checked against the definition (ragged last
    chunk included)."""
    g = np.random.default_rng(7)
    q, k, v, alpha, beta, S0 = _inputs(g, B=1, N=150, H=1, Dk=16, Dv=8)
    o, S = gdn_recurrent(q, k, v, alpha, beta, S0)
    o2, S2 = _chunkwise(q[0, :, 0], k[0, :, 0], v[0, :, 0], alpha[0, 0], beta[0, 0], S0[0, 0], C)
    np.testing.assert_allclose(o2, o[0, :, 0], rtol=1e-9, atol=1e-9)
    np.testing.assert_allclose(S2, S[0, 0], rtol=1e-9, atol=1e-9)
