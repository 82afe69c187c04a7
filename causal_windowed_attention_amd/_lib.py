"""ctypes declarations of the C ABI in include/sa.h (libsa.so, built in-tree).

Loading fails loudly when the library is missing: there is no fallback path.
"""
import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libsa.so")

# sa_status
SA_OK = 0
SA_ERR_INVALID_ARGUMENT = 1
SA_ERR_UNSUPPORTED = 2
SA_ERR_BAD_STATE = 3
SA_ERR_WORKSPACE_TOO_SMALL = 4
SA_ERR_POSITION_RANGE = 5
SA_ERR_DEVICE = 6
# sa_dtype
SA_F32 = 0
SA_BF16 = 1
SA_FP8 = 2
SA_REFRESH_SHIFT_SINK = 1
SA_MAX_TEMPORAL_PAIRS = 320
SA_MAX_BUFFER_CHUNKS = 8
SA_MAX_KEY_SEGMENTS = 4
SA_MAX_BATCH_STREAMS = 8
SA_BUFFER_STEPS = 1
SA_GDN_SCRATCH_BYTES = 67108864
# sa_slot_kind
SA_SLOT_EMPTY, SA_SLOT_SINK, SA_SLOT_WINDOW, SA_SLOT_STAGING = 0, 1, 2, 3
# sa_kernel_id
SA_K_ROPE_APPLY, SA_K_CHUNK_ATTENTION, SA_K_ATTN_COMBINE = 0, 1, 2
SA_K_KV_APPEND, SA_K_ROPE_REFRESH, SA_K_SINK_UPDATE, SA_K_COUNT = 3, 4, 5, 6
# sa_option
SA_OPT_KV_SPLITS, SA_OPT_PROFILE, SA_OPT_ATTN_VARIANT, SA_OPT_SCHEDULE = 0, 1, 2, 3


class sa_config(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("frame_h", ctypes.c_int32), ("frame_w", ctypes.c_int32),
                ("frames_per_chunk", ctypes.c_int32), ("sink_chunks", ctypes.c_int32),
                ("window_chunks", ctypes.c_int32), ("rope_dim_t", ctypes.c_int32),
                ("rope_dim_h", ctypes.c_int32), ("rope_dim_w", ctypes.c_int32),
                ("max_t", ctypes.c_int32), ("rope_theta", ctypes.c_double),
                ("softmax_scale", ctypes.c_float), ("dtype", ctypes.c_int32),
                ("max_buffer_chunks", ctypes.c_int32), ("reserved", ctypes.c_int32)]


class sa_state(ctypes.Structure):
    _fields_ = [("n_appends", ctypes.c_int64), ("ring_commits", ctypes.c_int64),
                ("t_next", ctypes.c_int32), ("sink_fill", ctypes.c_int32),
                ("window_valid", ctypes.c_int32), ("staging_slot", ctypes.c_int32),
                ("n_slots", ctypes.c_int32), ("visible_chunks", ctypes.c_int32),
                ("visible_keys", ctypes.c_int32), ("staged_valid", ctypes.c_int32),
                ("last_q_tiles", ctypes.c_int32), ("last_kv_splits", ctypes.c_int32),
                ("last_key_tiles", ctypes.c_int32), ("last_delta", ctypes.c_int32),
                ("last_sk_groups", ctypes.c_int32), ("reserved", ctypes.c_int32)]


class sa_slot_info(ctypes.Structure):
    _fields_ = [("chunk_id", ctypes.c_int64), ("t0", ctypes.c_int32), ("kind", ctypes.c_int32)]


class sa_layout(ctypes.Structure):
    _fields_ = [("k_offset", ctypes.c_uint64), ("k_bh_stride", ctypes.c_uint64),
                ("vt_offset", ctypes.c_uint64), ("vt_bh_stride", ctypes.c_uint64),
                ("q_offset", ctypes.c_uint64), ("q_bh_stride", ctypes.c_uint64),
                ("partial_offset", ctypes.c_uint64), ("partial_bytes", ctypes.c_uint64),
                ("table_offset", ctypes.c_uint64), ("table_bytes", ctypes.c_uint64),
                ("key_stride", ctypes.c_int32), ("elem_bytes", ctypes.c_int32),
                ("max_kv_splits", ctypes.c_int32), ("reserved", ctypes.c_int32)]


# every symbol include/sa.h declares, with (restype, argtypes)
_P = ctypes.c_void_p
_I32, _U32, _I64 = ctypes.c_int32, ctypes.c_uint32, ctypes.c_int64
SIGNATURES = {
    "sa_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "sa_config_check": (ctypes.c_int, [ctypes.POINTER(sa_config)]),
    "sa_workspace_bytes": (ctypes.c_size_t, [ctypes.POINTER(sa_config)]),
    "sa_stream_create": (ctypes.c_int, [ctypes.POINTER(sa_config), _P, ctypes.c_size_t, _P,
                                        ctypes.POINTER(_P)]),
    "sa_stream_destroy": (ctypes.c_int, [_P]),
    "sa_chunk_attend": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P]),
    "sa_kv_append": (ctypes.c_int, [_P, _P, _P, _P]),
    "sa_rope_refresh": (ctypes.c_int, [_P, _I32, _U32, _P, ctypes.POINTER(_I32)]),
    "sa_sink_update": (ctypes.c_int, [_P, _P, _P, _P]),
    "sa_stream_query": (ctypes.c_int, [_P, ctypes.POINTER(sa_state)]),
    "sa_stream_slot": (ctypes.c_int, [_P, _I32, ctypes.POINTER(sa_slot_info)]),
    "sa_stream_layout": (ctypes.c_int, [_P, ctypes.POINTER(sa_layout)]),
    "sa_stream_set_option": (ctypes.c_int, [_P, _I32, _I64]),
    "sa_profile_read": (ctypes.c_int, [_P, _I32, ctypes.POINTER(ctypes.c_double),
                                       ctypes.POINTER(_I64), _I32]),
    "sa_probe_mfma_bf16": (ctypes.c_int, [_P, _I32, _I32, _P]),
    "sa_probe_mfma_bf16_data": (ctypes.c_int, [_P, _P, _I32, _I32, _P]),
    "sa_buffer_attend": (ctypes.c_int, [_P, _P, _P, _P, _I32, _U32, _P, _P, _P]),
    "sa_buffer_plan": (ctypes.c_int, [_P, _I32, _U32, ctypes.POINTER(_I32), ctypes.POINTER(_I32),
                                      ctypes.POINTER(_I32)]),
    "sa_batch_attend": (ctypes.c_int, [_I32, ctypes.POINTER(_P), ctypes.POINTER(_P), ctypes.POINTER(_P),
                                       ctypes.POINTER(_P), ctypes.POINTER(_P), ctypes.POINTER(_P), _P]),
    "sa_gdn_workspace_bytes": (ctypes.c_size_t, [_I32, _I32, _I32, _I32]),
    "sa_gdn_forward": (ctypes.c_int, [_I32, _I32, _I32, _I32, _P, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]),
    "sa_gdn_forward_noalloc": (ctypes.c_int, [_I32, _I32, _I32, _I32, _P, _P, _P, _P, _P, _P, _P, _P, _P]),
}

_lib = None


def load() -> ctypes.CDLL:
    """The loaded libsa.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is missing: build it with `python -m causal_windowed_attention_amd.build` "
                "(there is no fallback implementation)")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib
