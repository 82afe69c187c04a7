"""Softmax attention over an explicit visible key set, fp64.

For query rows q_i and visible keys k_j (already position-rotated) the scores
are s_ij = scale * <q_i, k_j>, the weights p_ij = exp(s_ij - max_j s_ij) /
sum_j exp(s_ij - max_j s_ij), the output O_i = sum_j p_ij v_j and the
log-sum-exp LSE_i = max_j s_ij + log sum_j exp(s_ij - max_j s_ij).

This is full (bidirectional) softmax attention over whatever set is passed in;
the stream module decides the set: the sink chunk, the window of recent chunks
and the current chunk itself (SANA-Streaming, "Transformer a diffusione
ibrido": softmax blocks with a sliding local window and a persistent sink
chunk). The rows are processed in blocks only to bound memory; no other
reordering.
"""
import math

import numpy as np


def attend(q, k, v, scale: float, block_rows: int = 512):
    """O [Nq, Dv] and LSE [Nq] (natural log) for q [Nq, D], k [Nk, D], v [Nk, Dv]."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    nq = q.shape[0]
    if k.shape[0] == 0:
        raise ValueError("attention needs at least one visible key")
    out = np.empty((nq, v.shape[1]), dtype=np.float64)
    lse = np.empty((nq,), dtype=np.float64)
    for r0 in range(0, nq, block_rows):
        s = (q[r0:r0 + block_rows] @ k.T) * scale
        m = s.max(axis=1, keepdims=True)
        p = np.exp(s - m)
        denom = p.sum(axis=1, keepdims=True)
        out[r0:r0 + block_rows] = (p @ v) / denom
        lse[r0:r0 + block_rows] = (m + np.log(denom))[:, 0]
    return out, lse


def attention_probs(q, k, scale: float):
    """The full weight matrix p [Nq, Nk] (small inputs only)."""
    s = (np.asarray(q, dtype=np.float64) @ np.asarray(k, dtype=np.float64).T) * scale
    m = s.max(axis=1, keepdims=True)
    p = np.exp(s - m)
    return p / p.sum(axis=1, keepdims=True)


def attend_bruteforce(q, k, v, scale: float):
    """Scalar-loop twin of attend() for tiny inputs (pure Python floats)."""
    q = [[float(a) for a in row] for row in np.asarray(q)]
    k = [[float(a) for a in row] for row in np.asarray(k)]
    v = [[float(a) for a in row] for row in np.asarray(v)]
    out, lses = [], []
    for qi in q:
        scores = []
        for kj in k:
            acc = 0.0
            for a, b in zip(qi, kj):
                acc += a * b
            scores.append(acc * scale)
        m = max(scores)
        w = [math.exp(s - m) for s in scores]
        z = sum(w)
        row = []
        for d in range(len(v[0])):
            acc = 0.0
            for wj, vj in zip(w, v):
                acc += wj * vj[d]
            row.append(acc / z)
        out.append(row)
        lses.append(m + math.log(z))
    return np.array(out, dtype=np.float64), np.array(lses, dtype=np.float64)
