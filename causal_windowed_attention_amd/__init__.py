"""Streaming chunk attention for MI355X (gfx950): Python binding of libsa.so.

Each new chunk of latent video tokens gets 3D (t, h, w) RoPE and attends with
full softmax attention to itself, a persistent sink chunk and a sliding window
of recent chunks kept in a KV ring cache; temporal RoPE offsets can be
re-based and the sink replaced (StreamDiffusionV2, "Sommario tecnico" 2.A;
SANA-Streaming, "Transformer a diffusione ibrido").

The functions below carry the C ABI's names (include/sa.h) and only marshal
arguments: tensors become device pointers, the current torch stream becomes
the hipStream_t. Every step of the computation runs in the library's HIP
kernels; PyTorch only provides device memory and streams. ``Stream`` bundles a
handle with its workspace for convenience.
"""
import ctypes
from typing import Optional, Tuple

from . import _lib as L
from ._lib import (SA_BF16, SA_F32, SA_FP8, SA_K_ATTN_COMBINE, SA_K_CHUNK_ATTENTION, SA_K_COUNT,
                   SA_K_KV_APPEND, SA_K_ROPE_APPLY, SA_K_ROPE_REFRESH, SA_K_SINK_UPDATE,
                   SA_BUFFER_STEPS, SA_OK, SA_OPT_ATTN_VARIANT, SA_OPT_KV_SPLITS, SA_OPT_SCHEDULE, SA_OPT_PROFILE, SA_REFRESH_SHIFT_SINK,
                   SA_SLOT_EMPTY, SA_SLOT_SINK, SA_SLOT_STAGING, SA_SLOT_WINDOW, sa_config)

__all__ = [
    "SaError", "make_config", "sa_status_string", "sa_config_check", "sa_workspace_bytes",
    "sa_stream_create", "sa_stream_destroy", "sa_chunk_attend", "sa_kv_append",
    "sa_rope_refresh", "sa_sink_update", "sa_stream_query", "sa_stream_slot",
    "sa_stream_layout", "sa_stream_set_option", "sa_profile_read", "sa_probe_mfma_bf16", "sa_probe_mfma_bf16_data",
    "sa_gdn_workspace_bytes", "sa_gdn_forward", "sa_gdn_forward_noalloc", "gdn_forward",
    "sa_buffer_attend", "sa_buffer_plan", "sa_batch_attend", "Stream",
    "SA_F32", "SA_BF16", "SA_FP8", "SA_REFRESH_SHIFT_SINK", "SA_OPT_KV_SPLITS", "SA_OPT_PROFILE",
    "SA_OPT_ATTN_VARIANT", "SA_OPT_SCHEDULE",
    "SA_K_ROPE_APPLY", "SA_K_CHUNK_ATTENTION", "SA_K_ATTN_COMBINE", "SA_K_KV_APPEND",
    "SA_K_ROPE_REFRESH", "SA_K_SINK_UPDATE", "SA_K_COUNT",
    "SA_SLOT_EMPTY", "SA_SLOT_SINK", "SA_SLOT_WINDOW", "SA_SLOT_STAGING",
]

_STATUS_NAMES = {0: "SA_OK", 1: "SA_ERR_INVALID_ARGUMENT", 2: "SA_ERR_UNSUPPORTED",
                 3: "SA_ERR_BAD_STATE", 4: "SA_ERR_WORKSPACE_TOO_SMALL",
                 5: "SA_ERR_POSITION_RANGE", 6: "SA_ERR_DEVICE"}


class SaError(RuntimeError):
    """A non-SA_OK status returned by the library."""

    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {_STATUS_NAMES.get(status, status)}")


def _check(status: int, where: str) -> None:
    if status != SA_OK:
        raise SaError(status, where)


def make_config(batch, heads, head_dim, frame_h, frame_w, frames_per_chunk, sink_chunks,
                window_chunks, rope_dims=(0, 0, 0), max_t=0, rope_theta=0.0, softmax_scale=0.0,
                dtype=SA_BF16, max_buffer_chunks=0) -> sa_config:
    if isinstance(dtype, str):
        dtype = {"bf16": SA_BF16, "f32": SA_F32, "fp8": SA_FP8}[dtype]
    return sa_config(batch, heads, head_dim, frame_h, frame_w, frames_per_chunk, sink_chunks,
                     window_chunks, rope_dims[0], rope_dims[1], rope_dims[2], max_t,
                     float(rope_theta), float(softmax_scale), dtype, max_buffer_chunks, 0)


def _ptr(x) -> Optional[int]:
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream_ptr(stream) -> Optional[int]:
    if stream is None:
        import torch
        if not torch.cuda.is_available():
            return None
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def sa_status_string(status: int) -> str:
    return L.load().sa_status_string(status).decode()


def sa_config_check(cfg: sa_config) -> int:
    return L.load().sa_config_check(ctypes.byref(cfg))


def sa_workspace_bytes(cfg: sa_config) -> int:
    return L.load().sa_workspace_bytes(ctypes.byref(cfg))


def sa_stream_create(cfg: sa_config, workspace=None, stream=None) -> ctypes.c_void_p:
    """Handle for a stream; workspace None creates a planning handle (no device work)."""
    h = ctypes.c_void_p()
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(L.load().sa_stream_create(ctypes.byref(cfg), _ptr(workspace), nbytes,
                                     _stream_ptr(stream) if workspace is not None else None,
                                     ctypes.byref(h)), "sa_stream_create")
    return h


def sa_stream_destroy(handle) -> None:
    _check(L.load().sa_stream_destroy(handle), "sa_stream_destroy")


def sa_chunk_attend(handle, q, k, v, out, lse=None, stream=None) -> None:
    _check(L.load().sa_chunk_attend(handle, _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse),
                                    _stream_ptr(stream)), "sa_chunk_attend")


def sa_kv_append(handle, k=None, v=None, stream=None) -> None:
    _check(L.load().sa_kv_append(handle, _ptr(k), _ptr(v), _stream_ptr(stream)), "sa_kv_append")


def sa_rope_refresh(handle, new_base_t: int = -1, flags: int = 0, stream=None) -> int:
    delta = ctypes.c_int32()
    _check(L.load().sa_rope_refresh(handle, new_base_t, flags, _stream_ptr(stream),
                                    ctypes.byref(delta)), "sa_rope_refresh")
    return delta.value


def sa_sink_update(handle, k, v, stream=None) -> None:
    _check(L.load().sa_sink_update(handle, _ptr(k), _ptr(v), _stream_ptr(stream)), "sa_sink_update")


def _struct_dict(s) -> dict:
    return {name: getattr(s, name) for name, _ in s._fields_}


def sa_stream_query(handle) -> dict:
    st = L.sa_state()
    _check(L.load().sa_stream_query(handle, ctypes.byref(st)), "sa_stream_query")
    return _struct_dict(st)


def sa_stream_slot(handle, slot: int) -> dict:
    info = L.sa_slot_info()
    _check(L.load().sa_stream_slot(handle, slot, ctypes.byref(info)), "sa_stream_slot")
    return _struct_dict(info)


def sa_stream_layout(handle) -> dict:
    lay = L.sa_layout()
    _check(L.load().sa_stream_layout(handle, ctypes.byref(lay)), "sa_stream_layout")
    return _struct_dict(lay)


def sa_stream_set_option(handle, option: int, value: int) -> None:
    _check(L.load().sa_stream_set_option(handle, option, value), "sa_stream_set_option")


def sa_profile_read(handle, kernel_id: int, reset: bool = False) -> Tuple[float, int]:
    ms, n = ctypes.c_double(), ctypes.c_int64()
    _check(L.load().sa_profile_read(handle, kernel_id, ctypes.byref(ms), ctypes.byref(n),
                                    1 if reset else 0), "sa_profile_read")
    return ms.value, n.value


def sa_buffer_attend(handle, q, k, v, n_chunks: int, out, lse=None, stream=None, flags: int = 0) -> None:
    _check(L.load().sa_buffer_attend(handle, _ptr(q), _ptr(k), _ptr(v), n_chunks, flags, _ptr(out), _ptr(lse),
                                     _stream_ptr(stream)), "sa_buffer_attend")


def sa_buffer_plan(handle, n_chunks: int, flags: int = 0):
    """Per buffer chunk, the [lo, hi) physical key-row ranges a buffer attend would read."""
    m = L.SA_MAX_KEY_SEGMENTS
    n_seg = (ctypes.c_int32 * max(n_chunks, 1))()
    lo = (ctypes.c_int32 * (m * max(n_chunks, 1)))()
    hi = (ctypes.c_int32 * (m * max(n_chunks, 1)))()
    _check(L.load().sa_buffer_plan(handle, n_chunks, flags, n_seg, lo, hi), "sa_buffer_plan")
    return [[(lo[j * m + i], hi[j * m + i]) for i in range(n_seg[j])] for j in range(n_chunks)]


def sa_batch_attend(handles, qs, ks, vs, outs, lses=None, stream=None) -> None:
    """Ragged batch: one attend per handle (each at its own state), one attention launch.
    Entries given as Stream objects have their tensors checked (shape, dtype, device,
    contiguity) before the call; raw handles pass pointers through (planning handles
    ignore them)."""
    n = len(handles)
    for i, hd in enumerate(handles):
        if isinstance(hd, Stream):
            for xs, name in ((qs, "q"), (ks, "k"), (vs, "v"), (outs, "out")):
                hd._check_tensor(None if xs is None else xs[i], hd.Nc, f"{name}[{i}]")
            if lses is not None:
                hd._check_lse(lses[i], hd.Nc, f"lse[{i}]")
    arr = lambda xs: (ctypes.c_void_p * max(n, 1))(*[_ptr(x) for x in xs]) if xs is not None else None
    h = (ctypes.c_void_p * max(n, 1))(*[x.handle if isinstance(x, Stream) else x for x in handles])
    _check(L.load().sa_batch_attend(n, h, arr(qs), arr(ks), arr(vs), arr(outs), arr(lses),
                                    _stream_ptr(stream)), "sa_batch_attend")


def sa_probe_mfma_bf16(out, blocks: int, iters: int, stream=None) -> None:
    """Launch the pure-MFMA measurement kernel (out: float32 device tensor of blocks*256)."""
    _check(L.load().sa_probe_mfma_bf16(_ptr(out), blocks, iters, _stream_ptr(stream)), "sa_probe_mfma_bf16")


def sa_probe_mfma_bf16_data(out, operands, blocks: int, iters: int, stream=None) -> None:
    """The pure-MFMA measurement on data operands (operands: a bf16 device tensor of 6*64*8
    values, runs 0-3 the A operands and 4-5 the B operands of every wave's lanes)."""
    import torch
    if operands.dtype != torch.bfloat16 or operands.numel() != 6 * 64 * 8 or not operands.is_contiguous():
        raise ValueError("operands: a contiguous bf16 tensor of 3072 values")
    if operands.device != out.device:
        raise ValueError("operands and out must be on one device")
    _check(L.load().sa_probe_mfma_bf16_data(_ptr(out), _ptr(operands), blocks, iters, _stream_ptr(stream)),
           "sa_probe_mfma_bf16_data")


def sa_gdn_workspace_bytes(batch: int, tokens: int, heads: int, head_dim: int) -> int:
    return int(L.load().sa_gdn_workspace_bytes(batch, tokens, heads, head_dim))


def sa_gdn_forward(batch, tokens, heads, head_dim, q, k, v, alpha, beta, state_in, state_out, out, workspace,
                   workspace_bytes, stream=None) -> None:
    _check(L.load().sa_gdn_forward(batch, tokens, heads, head_dim, _ptr(q), _ptr(k), _ptr(v), _ptr(alpha),
                                   _ptr(beta), _ptr(state_in), _ptr(state_out), _ptr(out), _ptr(workspace),
                                   workspace_bytes, _stream_ptr(stream)), "sa_gdn_forward")


def sa_gdn_forward_noalloc(batch, tokens, heads, head_dim, q, k, v, alpha, beta, state_in, state_out, out,
                           stream=None) -> None:
    _check(L.load().sa_gdn_forward_noalloc(batch, tokens, heads, head_dim, _ptr(q), _ptr(k), _ptr(v), _ptr(alpha),
                                           _ptr(beta), _ptr(state_in), _ptr(state_out), _ptr(out),
                                           _stream_ptr(stream)), "sa_gdn_forward_noalloc")


def gdn_forward(q, k, v, alpha, beta, state=None, out=None, state_out=None, workspace=None, stream=None):
    """Gated delta rule forward (see sa_gdn_forward): q, k, v [B, N, H, D] bf16 CUDA tensors,
    alpha, beta [B, H, N] float32, state [B, H, D, D] float32 or None. Returns (out, state_out);
    state_out may be the state tensor itself (updated in place)."""
    import torch
    B, N, H, D = q.shape
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        if tuple(t.shape) != (B, N, H, D) or t.dtype != torch.bfloat16 or not t.is_contiguous() or not t.is_cuda:
            raise ValueError(f"{n}: expected contiguous bf16 CUDA [B, N, H, D], got {t.dtype} {tuple(t.shape)}")
    for t, n in ((alpha, "alpha"), (beta, "beta")):
        if tuple(t.shape) != (B, H, N) or t.dtype != torch.float32 or not t.is_contiguous() or not t.is_cuda:
            raise ValueError(f"{n}: expected contiguous float32 CUDA [B, H, N]")
    for t, n in ((state, "state"), (state_out, "state_out")):
        if t is not None and (tuple(t.shape) != (B, H, D, D) or t.dtype != torch.float32 or not t.is_contiguous()
                              or t.device != q.device):
            raise ValueError(f"{n}: expected contiguous float32 [B, H, D, D] on {q.device}")
    if out is not None and (tuple(out.shape) != (B, N, H, D) or out.dtype != torch.bfloat16
                            or not out.is_contiguous() or out.device != q.device):
        raise ValueError(f"out: expected contiguous bf16 [B, N, H, D] on {q.device}")
    for t, n in ((k, "k"), (v, "v"), (alpha, "alpha"), (beta, "beta")):
        if t.device != q.device:
            raise ValueError(f"{n}: expected on {q.device}, got {t.device}")
    if out is None:
        out = torch.empty_like(v)
    if state_out is None:
        state_out = torch.empty((B, H, D, D), dtype=torch.float32, device=q.device)
    need = sa_gdn_workspace_bytes(B, N, H, D)
    if need == 0:
        raise SaError(L.SA_ERR_UNSUPPORTED, "gdn_forward: unsupported sizes")
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    elif workspace.device != q.device or not workspace.is_contiguous():
        raise ValueError(f"workspace: expected contiguous memory on {q.device}")
    sa_gdn_forward(B, N, H, D, q, k, v, alpha, beta, state, state_out, out, workspace, workspace.numel(), stream)
    return out, state_out


class Stream:
    """A stream handle plus its caller-owned workspace (a torch uint8 tensor)."""

    def __init__(self, cfg: sa_config, device="cuda", planning: bool = False, stream=None):
        self.cfg = cfg
        self.nbytes = sa_workspace_bytes(cfg)
        if self.nbytes == 0:
            _check(sa_config_check(cfg) or 1, "sa_workspace_bytes")
        if planning:
            self.workspace = None
        else:
            import torch
            self.workspace = torch.empty(self.nbytes, dtype=torch.uint8, device=device)
        self.handle = sa_stream_create(cfg, self.workspace, stream)
        self.Nc = cfg.frames_per_chunk * cfg.frame_h * cfg.frame_w

    # -- argument checks (shapes and dtypes; the library checks the rest) --------
    def _torch_dtype(self):
        import torch
        return torch.float32 if self.cfg.dtype == SA_F32 else torch.bfloat16

    def _cache_dtype(self):
        import torch
        return {SA_F32: torch.float32, SA_BF16: torch.bfloat16, SA_FP8: torch.float8_e4m3fn}[self.cfg.dtype]

    def _check_tensor(self, t, n_tokens, name):
        """Shape, dtype, contiguity and (for a device handle) the device of an input or output.
        A planning handle accepts None (it ignores data pointers)."""
        if t is None:
            if self.workspace is None:
                return
            raise ValueError(f"{name}: a tensor is required")
        shape = (self.cfg.batch, n_tokens, self.cfg.heads, self.cfg.head_dim)
        where = self.workspace.device if self.workspace is not None else None
        if tuple(t.shape) != shape or t.dtype != self._torch_dtype() or not t.is_contiguous() \
                or (where is not None and t.device != where):
            raise ValueError(f"{name}: expected contiguous {self._torch_dtype()} {shape}"
                             + (f" on {where}" if where is not None else "")
                             + f", got {t.dtype} {tuple(t.shape)} on {t.device}")

    def _check_lse(self, lse, rows, name="lse"):
        if lse is None:
            return
        import torch
        where = self.workspace.device if self.workspace is not None else None
        if tuple(lse.shape) != (self.cfg.batch, self.cfg.heads, rows) or lse.dtype != torch.float32 \
                or not lse.is_contiguous() or (where is not None and lse.device != where):
            raise ValueError(f"{name}: expected contiguous float32 [B, H, {rows}]"
                             + (f" on {where}" if where is not None else ""))

    def new_output(self):
        import torch
        return torch.empty((self.cfg.batch, self.Nc, self.cfg.heads, self.cfg.head_dim),
                           dtype=self._torch_dtype(), device=self.workspace.device)

    def chunk_attend(self, q, k, v, out=None, lse=None, stream=None):
        if self.workspace is not None and out is None:
            out = self.new_output()
        for t, n in ((q, "q"), (k, "k"), (v, "v"), (out, "out")):
            self._check_tensor(t, self.Nc, n)
        self._check_lse(lse, self.Nc)
        sa_chunk_attend(self.handle, q, k, v, out, lse, stream)
        return out

    def buffer_attend(self, q, k, v, out=None, lse=None, stream=None, n_chunks=None, steps=False):
        """Buffer attend: q, k, v hold n consecutive chunks [B, n*Nc, H, D]; steps selects
        Stream-Batch over denoising steps instead of the moving buffer."""
        if n_chunks is None:
            if q is None or q.shape[1] % self.Nc:
                raise ValueError("buffer_attend: q must hold whole chunks (or pass n_chunks)")
            n_chunks = q.shape[1] // self.Nc
        rows = n_chunks * self.Nc
        if self.workspace is not None and out is None:
            import torch
            out = torch.empty((self.cfg.batch, rows, self.cfg.heads, self.cfg.head_dim),
                              dtype=self._torch_dtype(), device=self.workspace.device)
        for t, n in ((q, "q"), (k, "k"), (v, "v"), (out, "out")):
            self._check_tensor(t, rows, n)
        self._check_lse(lse, rows)
        sa_buffer_attend(self.handle, q, k, v, n_chunks, out, lse, stream,
                         L.SA_BUFFER_STEPS if steps else 0)
        return out

    def buffer_plan(self, n_chunks: int, steps=False):
        return sa_buffer_plan(self.handle, n_chunks, L.SA_BUFFER_STEPS if steps else 0)

    def kv_append(self, k=None, v=None, stream=None):
        if k is not None or v is not None:
            self._check_tensor(k, self.Nc, "k")
            self._check_tensor(v, self.Nc, "v")
        sa_kv_append(self.handle, k, v, stream)

    def rope_refresh(self, new_base_t: int = -1, flags: int = 0, stream=None) -> int:
        return sa_rope_refresh(self.handle, new_base_t, flags, stream)

    def sink_update(self, k, v, stream=None):
        n = self.cfg.sink_chunks * self.Nc
        self._check_tensor(k, n, "k")
        self._check_tensor(v, n, "v")
        sa_sink_update(self.handle, k, v, stream)

    def query(self) -> dict:
        return sa_stream_query(self.handle)

    def slot(self, i: int) -> dict:
        return sa_stream_slot(self.handle, i)

    def layout(self) -> dict:
        return sa_stream_layout(self.handle)

    def set_option(self, option: int, value: int) -> None:
        sa_stream_set_option(self.handle, option, value)

    def profile_read(self, kernel_id: int, reset: bool = False):
        return sa_profile_read(self.handle, kernel_id, reset)

    # -- read-only views of the cache inside the workspace (inspection, tests) ---
    def k_cache_view(self):
        """[B*H, key_stride, D] rotated keys (slot s at rows [s*Nc, (s+1)*Nc))."""
        lay = self.layout()
        bh = self.cfg.batch * self.cfg.heads
        n = bh * lay["key_stride"] * self.cfg.head_dim
        raw = self.workspace[lay["k_offset"]:lay["k_offset"] + n * lay["elem_bytes"]]
        return raw.view(self._cache_dtype()).view(bh, lay["key_stride"], self.cfg.head_dim)

    def vt_cache_view(self):
        """[B*H, D, key_stride] transposed values."""
        lay = self.layout()
        bh = self.cfg.batch * self.cfg.heads
        n = bh * self.cfg.head_dim * lay["key_stride"]
        raw = self.workspace[lay["vt_offset"]:lay["vt_offset"] + n * lay["elem_bytes"]]
        return raw.view(self._cache_dtype()).view(bh, self.cfg.head_dim, lay["key_stride"])

    def q_scratch_view(self):
        """[B*H, Nc, D] rotated queries of the last attend."""
        lay = self.layout()
        bh = self.cfg.batch * self.cfg.heads
        n = bh * self.Nc * self.cfg.head_dim
        raw = self.workspace[lay["q_offset"]:lay["q_offset"] + n * lay["elem_bytes"]]
        return raw.view(self._cache_dtype()).view(bh, self.Nc, self.cfg.head_dim)

    def close(self):
        if self.handle is not None:
            sa_stream_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
