"""Stream semantics of chunk attention with a sink chunk, a sliding window and RoPE refresh, fp64.

What the pages fix (in words, not quoted):
* video is processed chunk by chunk, each chunk a few latent frames
  (StreamDiffusionV2, "Sommario tecnico" 2.A.1, the B x T' x H x W form);
* softmax blocks attend to a bounded context: a sliding local window of recent
  chunks plus a persistent sink chunk (SANA-Streaming, "Transformer a
  diffusione ibrido");
* sink tokens are updated during the stream (StreamDiffusionV2, 2.A.2);
* RoPE offsets are reset periodically at chunk boundaries so positions stay
  aligned over long horizons (StreamDiffusionV2, 2.A.2).

Readings where the pages are silent:
* the chunk attends to itself fully (no causal mask inside the chunk);
* W counts previous committed chunks, excluding the current one;
* the first S committed chunks become the sink and do not also enter the
  window; every committed sink chunk is visible;
* a commit stores the chunk at the current position t_next and advances
  t_next by F (one temporal unit per latent frame);
* a sink update replaces all S sink chunks (no blending), placing them at
  t in [0, S*F);
* refresh with base b: Delta = (t0 of the oldest visible window chunk, or t_next
  when no window chunk is visible) - b; every visible window chunk and t_next
  move by -Delta; the sink stays pinned unless SHIFT_SINK is given (then it
  moves by -Delta too, which leaves every logit unchanged).

``HistoryOracle`` is the definition: it keeps every committed chunk's raw k and
v with its integer position and rotates at use time. ``RingOracle`` keeps
rotated keys in S sink slots and W window slots, re-rotates stored keys on
refresh (R(-Delta) composed with R(t0) = R(t0 - Delta)), and can round every
stored value the way a bf16 (or fp32) device cache would.
"""
from __future__ import annotations

import copy
import math
from dataclasses import dataclass
from typing import List, Optional, Tuple

import numpy as np

from .attention import attend
from .bf16 import round_bf16
from .fp8 import round_e4m3
from .rope import rope3d, rope_split, rotate_temporal, token_coords

SHIFT_SINK = 1


class StreamError(Exception):
    """Raised for an invalid call; ``kind`` is one of 'invalid', 'bad_state', 'position_range'."""

    def __init__(self, kind: str, msg: str):
        super().__init__(f"{kind}: {msg}")
        self.kind = kind


@dataclass(frozen=True)
class StreamSpec:
    batch: int
    heads: int
    head_dim: int
    frame_h: int
    frame_w: int
    frames_per_chunk: int
    sink_chunks: int
    window_chunks: int
    split: Tuple[int, int, int] = (0, 0, 0)
    theta: float = 10000.0
    scale: float = 0.0
    max_t: int = 0

    @property
    def tokens_per_chunk(self) -> int:
        return self.frames_per_chunk * self.frame_h * self.frame_w

    @property
    def rope(self) -> Tuple[int, int, int]:
        return rope_split(self.head_dim, self.split)

    @property
    def softmax_scale(self) -> float:
        return self.scale if self.scale > 0 else 1.0 / math.sqrt(self.head_dim)

    @classmethod
    def from_workload(cls, w) -> "StreamSpec":
        return cls(batch=w.batch, heads=w.heads, head_dim=w.head_dim, frame_h=w.frame_h,
                   frame_w=w.frame_w, frames_per_chunk=w.frames_per_chunk,
                   sink_chunks=w.sink_chunks, window_chunks=w.window_chunks)


def _rotate_chunk(spec: StreamSpec, u: np.ndarray, t0: int) -> np.ndarray:
    """RoPE3D of a chunk u [B, Nc, H, D] placed at frames t0.. ; returns [B, H, Nc, D] fp64."""
    f, y, x = token_coords(u.shape[1], spec.frame_h, spec.frame_w)
    uh = np.transpose(np.asarray(u, dtype=np.float64), (0, 2, 1, 3))
    return rope3d(uh, t0 + f, y, x, spec.rope, spec.theta)


def _heads_major(u: np.ndarray) -> np.ndarray:
    return np.transpose(np.asarray(u, dtype=np.float64), (0, 2, 1, 3)).copy()


def _attend_all(spec: StreamSpec, qrot, keys, vals, rows=None, heads=None):
    """Per (b, h) attention of qrot [B,H,Nc,D] over concatenated keys/vals lists of [B,H,n,D].

    Returns O [B, Nc, H, D] and LSE [B, H, Nc] (entries outside rows/heads are NaN).
    """
    B, H, Nc, D = qrot.shape
    out = np.full((B, Nc, H, D), np.nan)
    lse = np.full((B, H, Nc), np.nan)
    hs = range(H) if heads is None else heads
    for b in range(B):
        for h in hs:
            K = np.concatenate([k[b, h] for k in keys], axis=0)
            V = np.concatenate([v[b, h] for v in vals], axis=0)
            r = np.arange(Nc) if rows is None else np.asarray(rows)
            o, l = attend(qrot[b, h, r], K, V, spec.softmax_scale)
            out[b, r, h] = o
            lse[b, h, r] = l
    return out, lse


class _Common:
    """State shared by both formulations: counters and the position clock."""

    def __init__(self, spec: StreamSpec):
        if spec.head_dim % 2 or spec.frames_per_chunk <= 0 or spec.sink_chunks < 0 \
                or spec.window_chunks < 0:
            raise StreamError("invalid", "bad stream spec")
        spec.rope  # validates the split
        self.spec = spec
        self.t_next = 0
        self.n_appends = 0
        self.sink_fill = 0
        self.ring_commits = 0

    def _check_positions(self):
        s = self.spec
        if s.max_t > 0 and self.t_next + s.frames_per_chunk > s.max_t:
            raise StreamError("position_range", f"t_next {self.t_next} + F exceeds max_t {s.max_t}")

    def _check_chunk(self, *arrs, n_tokens=None):
        s = self.spec
        n = s.tokens_per_chunk if n_tokens is None else n_tokens
        for a in arrs:
            if a.shape != (s.batch, n, s.heads, s.head_dim):
                raise StreamError("invalid", f"expected [B, {n}, H, D], got {a.shape}")

    def buffer_attend(self, q, k, v, rows=None, heads=None, steps=False):
        """Several chunks that follow the committed stream, attended in one call; q, k, v hold
        n consecutive chunks [B, n*Nc, H, D] and buffer chunk j sits at t_next + j*F.

        steps=False, the moving buffer (StreamDiT: a buffer of consecutive chunks denoised
        together, with window attention): chunk j attends to what an attend would see once
        buffer chunks 0..j-1 were committed -- the sink, the last W chunks of (committed window,
        buffer 0..j-1), and itself: a block-banded chunk mask. Needs a full sink (else earlier
        buffer chunks would become sink chunks).

        steps=True, Stream-Batch over denoising steps (StreamDiffusionV2: chunks in flight at
        different denoising steps form one batch): no buffer chunk is committed yet, so chunk j
        attends to the committed context an attend would see now (sink and window) and itself.

        State unchanged. rows: global query rows in [0, n*Nc).
        Returns O [B, n*Nc, H, D], LSE [B, H, n*Nc]."""
        s = self.spec
        nc = s.tokens_per_chunk
        n = q.shape[1] // nc if q.ndim == 4 else 0
        B, H, D = s.batch, s.heads, s.head_dim
        out = np.full((B, n * nc, H, D), np.nan)
        lse = np.full((B, H, n * nc), np.nan)
        for j, sl, tmp in self._buffer_states(q, k, v, steps):
            r = None if rows is None else [x - j * nc for x in rows if j * nc <= x < (j + 1) * nc]
            if r is None or r:
                o, lj = tmp.attend(q[:, sl], k[:, sl], v[:, sl], rows=r, heads=heads)
                out[:, sl], lse[:, :, sl] = o, lj
            else:
                tmp._check_positions()
        return out, lse

    def _buffer_states(self, q, k, v, steps):
        """(j, token slice of chunk j, a copy of the stream in the state chunk j is attended
        in), for each buffer chunk in order (see buffer_attend); validates the call first."""
        s = self.spec
        nc = s.tokens_per_chunk
        if q.ndim != 4 or q.shape[1] == 0 or q.shape[1] % nc:
            raise StreamError("invalid", f"buffer of {q.shape[1] if q.ndim == 4 else '?'} tokens is not whole chunks")
        n = q.shape[1] // nc
        self._check_chunk(q, k, v, n_tokens=n * nc)
        if not steps and self.sink_fill < s.sink_chunks:
            raise StreamError("bad_state", "a moving-buffer attend needs a full sink")
        tmp = copy.deepcopy(self)
        for j in range(n):
            sl = slice(j * nc, (j + 1) * nc)
            if steps:                                # same committed context, j chunks further on
                tmp = copy.deepcopy(self)
                tmp.t_next = self.t_next + j * s.frames_per_chunk
            yield j, sl, tmp
            if not steps and j + 1 < n:
                tmp.append(k[:, sl], v[:, sl])

    def _base(self, new_base):
        if new_base is None or new_base == -1:
            return self.spec.sink_chunks * self.spec.frames_per_chunk
        if new_base < 0:
            raise StreamError("invalid", "new_base must be >= 0 (or -1 for the default)")
        return int(new_base)


class HistoryOracle(_Common):
    """The definition: every committed chunk kept raw with its integer position."""

    def __init__(self, spec: StreamSpec):
        super().__init__(spec)
        self.sink: List[Optional[list]] = [None] * spec.sink_chunks   # [chunk_id, t0, k, v]
        self.ring: List[list] = []                                      # [chunk_id, t0, k, v]

    # --- bookkeeping -------------------------------------------------------
    def _window(self) -> List[list]:
        W = self.spec.window_chunks
        return self.ring[max(0, len(self.ring) - W):] if W > 0 else []

    def visible(self) -> List[Tuple[str, int, int]]:
        """(kind, chunk_id, t0) of every chunk the next attend sees, sink first, self last."""
        out = [("sink", e[0], e[1]) for e in self.sink[:self.sink_fill]]
        out += [("window", e[0], e[1]) for e in self._window()]
        out.append(("self", self.n_appends, self.t_next))
        return out

    def state(self) -> dict:
        return dict(t_next=self.t_next, n_appends=self.n_appends, sink_fill=self.sink_fill,
                    ring_commits=self.ring_commits, visible=self.visible())

    # --- operations --------------------------------------------------------
    def attend(self, q, k, v, rows=None, heads=None):
        """O [B, Nc, H, D], LSE [B, H, Nc] of the current chunk (state unchanged)."""
        self._check_chunk(q, k, v)
        self._check_positions()
        s = self.spec
        keys, vals = [], []
        for e in self.sink[:self.sink_fill] + self._window():
            keys.append(_rotate_chunk(s, e[2], e[1]))
            vals.append(_heads_major(e[3]))
        keys.append(_rotate_chunk(s, k, self.t_next))
        vals.append(_heads_major(v))
        qrot = _rotate_chunk(s, q, self.t_next)
        return _attend_all(s, qrot, keys, vals, rows=rows, heads=heads)

    def append(self, k, v):
        self._check_chunk(k, v)
        self._check_positions()
        s = self.spec
        entry = [self.n_appends, self.t_next, np.array(k, dtype=np.float64),
                 np.array(v, dtype=np.float64)]
        if self.sink_fill < s.sink_chunks:
            self.sink[self.sink_fill] = entry
            self.sink_fill += 1
        else:
            self.ring.append(entry)
            self.ring_commits += 1
            # chunks older than the window are never visible again
            if len(self.ring) > s.window_chunks:
                self.ring = self.ring[len(self.ring) - s.window_chunks:]
        self.t_next += s.frames_per_chunk
        self.n_appends += 1

    def refresh(self, new_base=None, flags: int = 0) -> int:
        base = self._base(new_base)
        win = self._window()
        ref = win[0][1] if win else self.t_next
        delta = ref - base
        for e in win:
            e[1] -= delta
        self.t_next -= delta
        if flags & SHIFT_SINK:
            for e in self.sink[:self.sink_fill]:
                e[1] -= delta
        return delta

    def sink_update(self, k, v):
        s = self.spec
        if s.sink_chunks == 0:
            raise StreamError("bad_state", "stream has no sink")
        self._check_chunk(k, v, n_tokens=s.sink_chunks * s.tokens_per_chunk)
        nc = s.tokens_per_chunk
        for j in range(s.sink_chunks):
            self.sink[j] = [-1, j * s.frames_per_chunk,
                            np.array(k[:, j * nc:(j + 1) * nc], dtype=np.float64),
                            np.array(v[:, j * nc:(j + 1) * nc], dtype=np.float64)]
        self.sink_fill = s.sink_chunks


def fp8_q_scale(spec: StreamSpec) -> float:
    """The factor the fp8 variant applies to rotated queries before E4M3 rounding:
    c * 2^k with c = softmax_scale * log2(e) and the integer k that puts it in [1, 2)
    (for D = 128: c = 0.1275, k = 3, factor 1.0202). Scores then come out of the
    product in base-2 units once it multiplies by 2^-k, an exact power of two."""
    c = spec.softmax_scale * math.log2(math.e)
    k = -math.floor(math.log2(c))
    return c * 2.0 ** k


class RingOracle(_Common):
    """Rotated keys in S sink slots + W window slots; refresh re-rotates stored keys.

    storage: None (pure fp64), 'bf16', 'f32' or 'fp8' -- round every stored value
    (rotated Q, rotated K, V, re-rotated K) the way a device cache of that type holds
    it ('fp8': E4M3, saturating). The fp8 variant stores the rotated queries scaled by
    fp8_q_scale(spec) before rounding (the softmax scale in base 2, brought into [1, 2)
    by a power of two that the product takes back exactly); the stored Q here is that
    rounded value divided by the same factor, so the scores keep their usual scale.
    """

    def __init__(self, spec: StreamSpec, storage: Optional[str] = None):
        super().__init__(spec)
        if storage not in (None, "bf16", "f32", "fp8"):
            raise ValueError(storage)
        self.storage = storage
        B, H, Nc, D = spec.batch, spec.heads, spec.tokens_per_chunk, spec.head_dim
        S, W = spec.sink_chunks, spec.window_chunks
        self.sink_k = np.zeros((S, B, H, Nc, D))
        self.sink_v = np.zeros((S, B, H, Nc, D))
        self.sink_meta = [[False, 0, 0] for _ in range(S)]     # valid, chunk_id, t0
        self.ring_k = np.zeros((W, B, H, Nc, D))
        self.ring_v = np.zeros((W, B, H, Nc, D))
        self.ring_meta = [[False, 0, 0] for _ in range(W)]
        self.ring_next = 0

    def _store(self, x: np.ndarray) -> np.ndarray:
        if self.storage == "bf16":
            return round_bf16(x)
        if self.storage == "f32":
            return np.asarray(x, dtype=np.float32).astype(np.float64)
        if self.storage == "fp8":
            return round_e4m3(x)
        return np.array(x, dtype=np.float64)

    def _window_slots(self) -> List[int]:
        """Valid window slots, oldest first."""
        W = self.spec.window_chunks
        if W == 0:
            return []
        order = [(self.ring_next + i) % W for i in range(W)]
        return [j for j in order if self.ring_meta[j][0]]

    def visible(self) -> List[Tuple[str, int, int]]:
        out = [("sink", m[1], m[2]) for m in self.sink_meta if m[0]]
        out += [("window", self.ring_meta[j][1], self.ring_meta[j][2]) for j in self._window_slots()]
        out.append(("self", self.n_appends, self.t_next))
        return out

    def state(self) -> dict:
        return dict(t_next=self.t_next, n_appends=self.n_appends, sink_fill=self.sink_fill,
                    ring_commits=self.ring_commits, visible=self.visible())

    def stored_k(self, chunk_id: int) -> np.ndarray:
        """Stored rotated K [B, H, Nc, D] of a visible committed chunk (sink or window)."""
        for j, m in enumerate(self.sink_meta):
            if m[0] and m[1] == chunk_id:
                return self.sink_k[j]
        for j in self._window_slots():
            if self.ring_meta[j][1] == chunk_id:
                return self.ring_k[j]
        raise KeyError(chunk_id)

    def stored_v(self, chunk_id: int) -> np.ndarray:
        for j, m in enumerate(self.sink_meta):
            if m[0] and m[1] == chunk_id:
                return self.sink_v[j]
        for j in self._window_slots():
            if self.ring_meta[j][1] == chunk_id:
                return self.ring_v[j]
        raise KeyError(chunk_id)

    def _store_q(self, qrot: np.ndarray) -> np.ndarray:
        if self.storage == "fp8":
            kappa = fp8_q_scale(self.spec)
            return round_e4m3(qrot * kappa) / kappa
        return self._store(qrot)

    def staged(self, q, k, v):
        """What the attend call stores before the product: (Qrot, Kself, Vself), each [B,H,Nc,D]."""
        s = self.spec
        return (self._store_q(_rotate_chunk(s, q, self.t_next)),
                self._store(_rotate_chunk(s, k, self.t_next)),
                self._store(_heads_major(v)))

    def operands(self, q, k, v):
        """(Qrot, keys, vals) of the attend call: the stored rotated queries [B,H,Nc,D] and
        the stored visible keys and values, lists of [B,H,Nc,D] in sink, window, self order
        (views of the stored slots: a later commit may overwrite them)."""
        qrot, kself, vself = self.staged(q, k, v)
        keys = [self.sink_k[j] for j, m in enumerate(self.sink_meta) if m[0]]
        vals = [self.sink_v[j] for j, m in enumerate(self.sink_meta) if m[0]]
        for j in self._window_slots():
            keys.append(self.ring_k[j])
            vals.append(self.ring_v[j])
        keys.append(kself)
        vals.append(vself)
        return qrot, keys, vals

    def buffer_operands(self, q, k, v, steps=False):
        """operands() of every chunk of a buffer attend, in order (see buffer_attend)."""
        res = []
        for _, sl, tmp in self._buffer_states(q, k, v, steps):
            tmp._check_positions()
            qrot, keys, vals = tmp.operands(q[:, sl], k[:, sl], v[:, sl])
            # copies: the slot arrays are overwritten by the next chunk's commit
            res.append((qrot.copy(), [x.copy() for x in keys], [x.copy() for x in vals]))
        return res

    def attend(self, q, k, v, rows=None, heads=None):
        self._check_chunk(q, k, v)
        self._check_positions()
        qrot, keys, vals = self.operands(q, k, v)
        return _attend_all(self.spec, qrot, keys, vals, rows=rows, heads=heads)

    def append(self, k, v):
        self._check_chunk(k, v)
        self._check_positions()
        s = self.spec
        kr = self._store(_rotate_chunk(s, k, self.t_next))
        vr = self._store(_heads_major(v))
        if self.sink_fill < s.sink_chunks:
            j = self.sink_fill
            self.sink_k[j], self.sink_v[j] = kr, vr
            self.sink_meta[j] = [True, self.n_appends, self.t_next]
            self.sink_fill += 1
        else:
            if s.window_chunks > 0:
                j = self.ring_next
                self.ring_k[j], self.ring_v[j] = kr, vr
                self.ring_meta[j] = [True, self.n_appends, self.t_next]
                self.ring_next = (self.ring_next + 1) % s.window_chunks
            self.ring_commits += 1
        self.t_next += s.frames_per_chunk
        self.n_appends += 1

    def refresh(self, new_base=None, flags: int = 0) -> int:
        base = self._base(new_base)
        s = self.spec
        slots = self._window_slots()
        ref = self.ring_meta[slots[0]][2] if slots else self.t_next
        delta = ref - base
        for j in slots:
            self.ring_k[j] = self._store(rotate_temporal(self.ring_k[j], -delta, s.rope, s.theta))
            self.ring_meta[j][2] -= delta
        if flags & SHIFT_SINK:
            for j, m in enumerate(self.sink_meta):
                if m[0]:
                    self.sink_k[j] = self._store(
                        rotate_temporal(self.sink_k[j], -delta, s.rope, s.theta))
                    m[2] -= delta
        self.t_next -= delta
        return delta

    def sink_update(self, k, v):
        s = self.spec
        if s.sink_chunks == 0:
            raise StreamError("bad_state", "stream has no sink")
        self._check_chunk(k, v, n_tokens=s.sink_chunks * s.tokens_per_chunk)
        nc = s.tokens_per_chunk
        for j in range(s.sink_chunks):
            kj = k[:, j * nc:(j + 1) * nc]
            self.sink_k[j] = self._store(_rotate_chunk(s, kj, j * s.frames_per_chunk))
            self.sink_v[j] = self._store(_heads_major(v[:, j * nc:(j + 1) * nc]))
            self.sink_meta[j] = [True, -1, j * s.frames_per_chunk]
        self.sink_fill = s.sink_chunks
