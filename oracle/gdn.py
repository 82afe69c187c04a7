"""Gated delta rule (the GDN linear-attention block), fp64 -- TEST INFRASTRUCTURE ONLY.

SANA-Streaming ("Transformer a diffusione ibrido") runs most of its blocks as Gated DeltaNet
linear attention: a fixed-size recurrent state per head, updated as the stream advances,
with only the final state kept between chunks. The pages give no equations; this follows
the published gated delta rule (Yang, Kautz and Hatamizadeh, "Gated Delta Networks:
Improving Mamba2 with Delta Rule", ICLR 2025), token by token:

    S_t = alpha_t * S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T        (S: d_v x d_k)
    o_t = S_t q_t

alpha_t in (0, 1] is the decay gate, beta_t in [0, 1] the writing strength. Tokens of a chunk
are taken in (frame, y, x) raster order, and the state after a chunk's last token is the
one carried to the next chunk. q and k arrive as the caller prepared them (GDN normalises
them to unit length; the recurrence is a contraction for unit keys and beta <= 1).

This is the definition, written as the plain loop over tokens: no chunking, no reordering.
"""
import numpy as np


def gdn_recurrent(q, k, v, alpha, beta, state=None):
    """q, k: [B, N, H, Dk]; v: [B, N, H, Dv]; alpha, beta: [B, H, N]; state: [B, H, Dv, Dk]
    (None: zeros). Returns o [B, N, H, Dv] and the final state [B, H, Dv, Dk], fp64."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    alpha = np.asarray(alpha, dtype=np.float64)
    beta = np.asarray(beta, dtype=np.float64)
    B, N, H, Dk = k.shape
    Dv = v.shape[3]
    S = np.zeros((B, H, Dv, Dk)) if state is None else np.array(state, dtype=np.float64)
    o = np.empty((B, N, H, Dv))
    for t in range(N):
        kt, vt, qt = k[:, t], v[:, t], q[:, t]                       # [B, H, D]
        a, b = alpha[:, :, t, None, None], beta[:, :, t, None, None]
        Sk = np.einsum("bhvk,bhk->bhv", S, kt)                       # S_{t-1} k_t
        S = a * (S - b * Sk[..., None] * kt[:, :, None, :]) + b * vt[..., None] * kt[:, :, None, :]
        o[:, t] = np.einsum("bhvk,bhk->bhv", S, qt)
    return o, S
