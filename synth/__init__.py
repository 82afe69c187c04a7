"""Seeded synthetic workloads for streaming chunk attention.

This module only describes workload shapes and draws seeded random inputs. It
holds none of the attention, RoPE or cache arithmetic, so both the fp64 oracle
(test infrastructure) and the GPU path may use it without sharing any of the
method's code.

Shapes follow the streaming setting of the pages: a stream of chunks, each of
F latent frames of Hf x Wf tokens (the B x T' x H x W input form of
StreamDiffusionV2, "Sommario tecnico", section 2.A.1), attending to a persistent
sink chunk plus a sliding window of recent chunks (SANA-Streaming, "Transformer a
diffusione ibrido").

Inputs stand in for DiT Q/K/V activations: N(0, 1) draws in float32 from
PCG64 generators keyed by (20261203, config id, stream b, chunk, tensor id,
256-token block), then
rounded to bfloat16 (round to nearest even) for the bf16 workloads. The
outlier workload scales a per-head set of round(0.05 * D) channels of Q and K
by 8 before rounding. No public dataset stands behind these inputs.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import Optional, Tuple

import numpy as np

SEED_ROOT = 20261203

# tensor ids used in the seed key
T_Q, T_K, T_V, T_SINK_K, T_SINK_V = 0, 1, 2, 3, 4

# chunks outside a workload's "distinct" set reuse a pool of this many chunks
POOL_SIZE = 11
POOL_OFFSET = 1_000_000


@dataclass(frozen=True)
class Workload:
    """Shape of one streaming workload (sizes only, no arithmetic)."""

    name: str
    cfg_id: int
    batch: int
    heads: int
    head_dim: int
    frame_h: int
    frame_w: int
    frames_per_chunk: int
    sink_chunks: int
    window_chunks: int
    n_chunks: int
    refresh_every: int = 0          # 0: never; else refresh before chunk c when c % refresh_every == 0
    refresh_base: int = -1          # -1: default base (sink_chunks * frames_per_chunk)
    dtype: str = "bf16"             # "bf16", "f32" or "fp8" (bf16 inputs, E4M3 cache)
    outlier_channels: int = 0
    outlier_scale: float = 1.0

    @property
    def tokens_per_frame(self) -> int:
        return self.frame_h * self.frame_w

    @property
    def tokens_per_chunk(self) -> int:
        return self.frames_per_chunk * self.frame_h * self.frame_w

    def refresh_before(self, c: int) -> bool:
        return self.refresh_every > 0 and c > 0 and c % self.refresh_every == 0

    def visible_chunks_steady(self) -> int:
        return self.sink_chunks + self.window_chunks + 1


WORKLOADS = {
    "tiny_f32": Workload(
        name="tiny_f32", cfg_id=1, batch=1, heads=2, head_dim=64, frame_h=8, frame_w=8,
        frames_per_chunk=2, sink_chunks=1, window_chunks=2, n_chunks=6, refresh_every=4,
        dtype="f32"),
    "wan1.3b": Workload(
        name="wan1.3b", cfg_id=2, batch=1, heads=12, head_dim=128, frame_h=30, frame_w=52,
        frames_per_chunk=3, sink_chunks=1, window_chunks=6, n_chunks=20),
    "wan14b_b1": Workload(
        name="wan14b_b1", cfg_id=3, batch=1, heads=40, head_dim=128, frame_h=30, frame_w=52,
        frames_per_chunk=3, sink_chunks=1, window_chunks=4, n_chunks=20),
    "wan14b_b2": Workload(
        name="wan14b_b2", cfg_id=3, batch=2, heads=40, head_dim=128, frame_h=30, frame_w=52,
        frames_per_chunk=3, sink_chunks=1, window_chunks=4, n_chunks=20),
    "wan14b_b4": Workload(
        name="wan14b_b4", cfg_id=3, batch=4, heads=40, head_dim=128, frame_h=30, frame_w=52,
        frames_per_chunk=3, sink_chunks=1, window_chunks=4, n_chunks=20),
    "hybrid1280x704": Workload(
        name="hybrid1280x704", cfg_id=4, batch=1, heads=16, head_dim=128, frame_h=22, frame_w=40,
        frames_per_chunk=4, sink_chunks=1, window_chunks=3, n_chunks=20,
        outlier_channels=6, outlier_scale=8.0),
    "long512p": Workload(
        name="long512p", cfg_id=5, batch=1, heads=24, head_dim=128, frame_h=32, frame_w=32,
        frames_per_chunk=2, sink_chunks=1, window_chunks=3, n_chunks=1000, refresh_every=64),
}


def small_variant(w: Workload, **kw) -> Workload:
    """A copy of a workload with some sizes changed (for oracle-sized parity runs)."""
    return replace(w, **kw)


def to_bf16_exact(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); returned as float32.

    Input preparation only: the draws are made in float32 and then stored as
    bfloat16, as a bf16 activation tensor would be.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    b = x.view(np.uint32)
    r = ((b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1)))
         & np.uint32(0xFFFF0000)).view(np.float32)
    nan = np.isnan(x)
    if np.any(nan):
        r = r.copy()
        r[nan] = np.float32(np.nan)
    return r


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """uint16 bit patterns of float32 values that are already bfloat16-exact."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    b = x.view(np.uint32)
    if np.any(b & 0xFFFF):
        raise ValueError("values are not bfloat16-exact")
    return (b >> 16).astype(np.uint16)


def _gen(cfg_id: int, b: int, chunk: int, tensor_id: int, block: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(
        [SEED_ROOT, cfg_id, b, chunk, tensor_id, block])))


# tokens per independently seeded block (blocks are drawn in parallel threads)
TOKEN_BLOCK = 256
_POOL = None


def _pool():
    global _POOL
    if _POOL is None:
        import os
        from concurrent.futures import ThreadPoolExecutor
        _POOL = ThreadPoolExecutor(max_workers=min(16, os.cpu_count() or 1))
    return _POOL


def outlier_channels(w: Workload) -> np.ndarray:
    """[H, n_out] channel indices scaled in Q and K (same set in both), or an empty array."""
    if w.outlier_channels <= 0:
        return np.zeros((w.heads, 0), dtype=np.int64)
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence(
        [SEED_ROOT, w.cfg_id, 999_999])))
    return np.stack([np.sort(g.choice(w.head_dim, size=w.outlier_channels, replace=False))
                     for _ in range(w.heads)])


def source_id(c: int, distinct: Optional[frozenset]) -> int:
    """Seed chunk index for stream chunk c: itself when distinct (or no set given), else a pool entry."""
    if distinct is None or c in distinct:
        return c
    return POOL_OFFSET + (c % POOL_SIZE)


def draw(w: Workload, src_chunk: int, tensor_id: int, n_tokens: Optional[int] = None) -> np.ndarray:
    """One seeded tensor [B, n_tokens, H, D] in float32 (bf16-exact for bf16 and fp8 workloads).

    Token blocks of TOKEN_BLOCK tokens of each stream b have their own generator
    keyed by (20261203, config id, b, chunk, tensor id, block), so the result
    does not depend on how the blocks are scheduled.
    """
    n = w.tokens_per_chunk if n_tokens is None else n_tokens
    out = np.empty((w.batch, n, w.heads, w.head_dim), dtype=np.float32)
    outl = outlier_channels(w)
    scale_outliers = outl.shape[1] and tensor_id in (T_Q, T_K, T_SINK_K)

    def fill(b, blk):
        t0, t1 = blk * TOKEN_BLOCK, min(n, (blk + 1) * TOKEN_BLOCK)
        x = _gen(w.cfg_id, b, src_chunk, tensor_id, blk).standard_normal(
            (t1 - t0, w.heads, w.head_dim), dtype=np.float32)
        if scale_outliers:
            for h in range(w.heads):
                x[:, h, outl[h]] *= np.float32(w.outlier_scale)
        if w.dtype in ("bf16", "fp8"):            # bf16 activations (fp8 caches take bf16 inputs)
            x = to_bf16_exact(x)
        out[b, t0:t1] = x

    jobs = [(b, blk) for b in range(w.batch) for blk in range((n + TOKEN_BLOCK - 1) // TOKEN_BLOCK)]
    for f in [_pool().submit(fill, b, blk) for b, blk in jobs]:
        f.result()
    return out


def chunk_qkv(w: Workload, c: int, distinct: Optional[frozenset] = None) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """(q, k, v) of stream chunk c, each [B, Nc, H, D] float32."""
    s = source_id(c, distinct)
    return draw(w, s, T_Q), draw(w, s, T_K), draw(w, s, T_V)


def sink_kv(w: Workload, update_index: int) -> Tuple[np.ndarray, np.ndarray]:
    """(k, v) for the update_index-th sink update, each [B, S*Nc, H, D] float32."""
    n = w.sink_chunks * w.tokens_per_chunk
    return (draw(w, update_index, T_SINK_K, n_tokens=n),
            draw(w, update_index, T_SINK_V, n_tokens=n))


def distinct_set_for(w: Workload, checked) -> frozenset:
    """Chunks that must carry distinct data so that every checked chunk's visible set is distinct."""
    s = set(range(w.sink_chunks))
    for c in checked:
        for j in range(max(0, c - w.window_chunks), c + 1):
            s.add(j)
    return frozenset(s)



# tensor ids of the gated delta rule (GDN) inputs
T_GDN = 16


def gdn_inputs(batch: int, tokens: int, heads: int, head_dim: int, seed: int, state: bool = True):
    """Seeded inputs of the gated delta rule (GDN linear attention) block, as the layer would
    hand them over: q and k drawn N(0, 1), scaled to unit length per token and head (GDN's
    own normalisation, input preparation here) and rounded to bf16; v N(0, 1) in bf16;
    decay gates alpha ~ U[0.9, 1] and write strengths beta ~ U[0, 1] in float32 ([B, H, N]);
    an initial state [B, H, D, D] drawn N(0, 1/D) (or None). Returns float32 arrays (the
    bf16 tensors bf16-exact): q, k, v [B, N, H, D], alpha, beta, state."""
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([SEED_ROOT, T_GDN, seed])))
    shape = (batch, tokens, heads, head_dim)
    q = g.standard_normal(shape, dtype=np.float32)
    k = g.standard_normal(shape, dtype=np.float32)
    q = to_bf16_exact(q / np.maximum(np.linalg.norm(q, axis=-1, keepdims=True), 1e-6))
    k = to_bf16_exact(k / np.maximum(np.linalg.norm(k, axis=-1, keepdims=True), 1e-6))
    v = to_bf16_exact(g.standard_normal(shape, dtype=np.float32))
    alpha = g.uniform(0.9, 1.0, (batch, heads, tokens)).astype(np.float32)
    beta = g.uniform(0.0, 1.0, (batch, heads, tokens)).astype(np.float32)
    s0 = ((g.standard_normal((batch, heads, head_dim, head_dim), dtype=np.float32)
           / np.float32(np.sqrt(head_dim))).astype(np.float32) if state else None)
    return q, k, v, alpha, beta, s0
