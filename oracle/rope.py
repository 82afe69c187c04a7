"""3D rotary position embedding (t, h, w), fp64.

The pages name RoPE offsets and their periodic re-basing at chunk boundaries
(StreamDiffusionV2, "Sommario tecnico" 2.A.2) but print no formula. The
rotation itself is the published one of RoFormer (Su et al., 2021): a pair of
channels (u0, u1) at position p with frequency theta is mapped to
(u0 cos(p theta) - u1 sin(p theta), u0 sin(p theta) + u1 cos(p theta)).

Readings where the pages are silent (each a parameter of the stream config):
* the head dimension D is split into contiguous segments [t | h | w] of even
  lengths (d_t, d_h, d_w); default d_h = d_w = 2*floor(D/6), d_t = D - 2*d_h,
  i.e. (44, 42, 42) for D = 128 and (24, 20, 20) for D = 64;
* inside a segment of length d, pair j (0 <= j < d/2) is channels
  (o + 2j, o + 2j + 1) and has frequency base^(-2j/d), base 10000 per axis;
* coordinates: one temporal unit per latent frame; a chunk's tokens are in
  frame-major raster order, token n -> (frame n // (Hf Wf), row (n // Wf) % Hf,
  column n % Wf), 0-based, no centring.
"""
import numpy as np


def rope_split(head_dim: int, dims=None):
    """(d_t, d_h, d_w): the default split, or the given one after validation."""
    if dims is None or tuple(dims) == (0, 0, 0):
        dh = 2 * (head_dim // 6)
        return (head_dim - 2 * dh, dh, dh)
    dt, dh, dw = (int(d) for d in dims)
    if min(dt, dh, dw) < 0 or dt % 2 or dh % 2 or dw % 2 or dt + dh + dw != head_dim:
        raise ValueError(f"bad RoPE split {dims} for head_dim {head_dim}")
    return (dt, dh, dw)


def token_coords(n_tokens: int, frame_h: int, frame_w: int):
    """(frame, y, x) integer arrays for tokens 0..n_tokens-1 in frame-major raster order."""
    n = np.arange(n_tokens, dtype=np.int64)
    per_frame = frame_h * frame_w
    return n // per_frame, (n // frame_w) % frame_h, n % frame_w


def rope_freqs(seg_len: int, theta: float) -> np.ndarray:
    """Frequencies base^(-2j/d) of the seg_len/2 pairs of one axis segment, fp64."""
    j = np.arange(seg_len // 2, dtype=np.float64)
    return np.power(float(theta), -2.0 * j / seg_len)


def _rotate_segment(u: np.ndarray, offset: int, seg_len: int, pos: np.ndarray,
                    theta: float) -> None:
    """In place: rotate the pairs of segment [offset, offset+seg_len) of u[..., N, D] by pos[N]."""
    if seg_len == 0:
        return
    freqs = rope_freqs(seg_len, theta)                         # [d/2]
    phi = np.asarray(pos, dtype=np.float64)[:, None] * freqs   # [N, d/2]
    c, s = np.cos(phi), np.sin(phi)
    a = u[..., offset:offset + seg_len:2].copy()                # first of each pair
    b = u[..., offset + 1:offset + seg_len:2].copy()            # second of each pair
    u[..., offset:offset + seg_len:2] = a * c - b * s
    u[..., offset + 1:offset + seg_len:2] = a * s + b * c


def rope3d(u, t, y, x, split, theta: float = 10000.0) -> np.ndarray:
    """RoPE3D of u[..., N, D] at per-token coordinates t[N], y[N], x[N]; returns a new fp64 array.

    Axis segments are laid out [t | h | w] along D; each is rotated by its own coordinate.
    """
    out = np.array(u, dtype=np.float64, copy=True)
    dt, dh, dw = split
    if dt + dh + dw != out.shape[-1]:
        raise ValueError("split does not cover head_dim")
    _rotate_segment(out, 0, dt, t, theta)
    _rotate_segment(out, dt, dh, y, theta)
    _rotate_segment(out, dt + dh, dw, x, theta)
    return out


def rotate_temporal(u, delta_t, split, theta: float = 10000.0) -> np.ndarray:
    """Rotate only the temporal segment of u[..., N, D] by a position offset delta_t (scalar or [N]).

    Composition R(a) R(b) = R(a + b) makes this the re-basing step: a key rotated
    at t and then by -delta equals a key rotated at t - delta.
    """
    out = np.array(u, dtype=np.float64, copy=True)
    n = out.shape[-2]
    pos = np.broadcast_to(np.asarray(delta_t, dtype=np.float64), (n,))
    _rotate_segment(out, 0, split[0], pos, theta)
    return out
