"""ctypes binding of ``libkvq.so``: one Python function per C entry point,
with the same name and argument order.  Pointers are plain integers (device
addresses from ``tensor.data_ptr()``), streams are ``hipStream_t`` values
(``torch.cuda.Stream.cuda_stream``).  Status codes are returned as-is; the
``QuantizedKVCache`` wrapper turns them into exceptions.
"""
from __future__ import annotations

import ctypes
import os

KVQ_OK = 0
KVQ_ERR_ARG = -1
KVQ_ERR_UNSUPPORTED = -2
KVQ_ERR_WORKSPACE = -3
KVQ_ERR_STATE = -4
KVQ_ERR_CAPACITY = -5
KVQ_ERR_HIP = -6
KVQ_ERR_SCRATCH = -7

KVQ_STATIC_SCRATCH_BYTES = 4 << 20

KVQ_F16 = 0
KVQ_F32 = 1

KVQ_FORMAT_INT = 0
KVQ_FORMAT_FP8_E4M3 = 1

KVQ_KEYS_PER_TOKEN = 1
KVQ_VALUES_PER_CHANNEL = 2

KVQ_METRIC_KEY_ERROR = 0
KVQ_METRIC_SCORE_ERROR = 1
KVQ_METRIC_VALUE_ERROR = 2
KVQ_METRIC_VALUE_OUTPUT_REL_ERROR = 3
KVQ_METRIC_OUTPUT_REL_ERROR = 4
KVQ_METRICS = 5

_HERE = os.path.dirname(os.path.abspath(__file__))


def library_path() -> str:
    return os.path.join(_HERE, "libkvq.so")


class KvqError(RuntimeError):
    def __init__(self, status: int, what: str = ""):
        self.status = status
        super().__init__(f"{what}: {kvq_strerror(status)} ({status})" if what
                         else f"{kvq_strerror(status)} ({status})")


class KvqConfig(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("q_heads", ctypes.c_int32),
        ("kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("max_tokens", ctypes.c_int32),
        ("group", ctypes.c_int32),
        ("key_bits", ctypes.c_int32),
        ("value_bits", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("rope_base", ctypes.c_float),
        ("residual", ctypes.c_int32),
        ("sink", ctypes.c_int32),
        ("geometry", ctypes.c_int32),
        ("format", ctypes.c_int32),
    ]


class KvqLayout(ctypes.Structure):
    _fields_ = [
        ("k_codes", ctypes.c_size_t),
        ("k_meta", ctypes.c_size_t),
        ("v_codes", ctypes.c_size_t),
        ("v_meta", ctypes.c_size_t),
        ("k_tail", ctypes.c_size_t),
        ("v_tail", ctypes.c_size_t),
        ("k_sink", ctypes.c_size_t),
        ("v_sink", ctypes.c_size_t),
        ("rope_group", ctypes.c_size_t),
        ("rope_offset", ctypes.c_size_t),
        ("partials", ctypes.c_size_t),
        ("total_bytes", ctypes.c_size_t),
        ("gcap", ctypes.c_int32),
        ("tcap", ctypes.c_int32),
        ("max_splits", ctypes.c_int32),
        ("tail_slots", ctypes.c_int32),
    ]


_lib = None


def lib() -> ctypes.CDLL:
    """Load libkvq.so.  Raises if it has not been built: there is no
    fallback implementation."""
    global _lib
    if _lib is None:
        path = library_path()
        if not os.path.exists(path):
            raise ImportError(
                f"{path} is missing: build it with "
                "`python -m quantized_decode_attention_keys_amd.build`")
        L = ctypes.CDLL(path)
        P = ctypes.c_void_p
        CP = ctypes.POINTER(KvqConfig)
        L.kvq_workspace_bytes.argtypes = [CP]
        L.kvq_workspace_bytes.restype = ctypes.c_size_t
        L.kvq_create.argtypes = [CP, P, ctypes.c_size_t, ctypes.POINTER(P)]
        L.kvq_create.restype = ctypes.c_int
        L.kvq_quantize_prefill.argtypes = [P, P, P, ctypes.c_int32, P]
        L.kvq_quantize_prefill.restype = ctypes.c_int
        L.kvq_append_token.argtypes = [P, P, P, P]
        L.kvq_append_token.restype = ctypes.c_int
        L.kvq_attend_decode.argtypes = [P, P, P, P]
        L.kvq_attend_decode.restype = ctypes.c_int
        L.kvq_append_attend.argtypes = [P, P, P, P, P, P]
        L.kvq_append_attend.restype = ctypes.c_int
        L.kvq_append_attend_static.argtypes = [P, P, P, P, P, P]
        L.kvq_append_attend_static.restype = ctypes.c_int
        L.kvq_error_metrics.argtypes = [P, P, P, P, P, P]
        L.kvq_error_metrics.restype = ctypes.c_int
        L.kvq_destroy.argtypes = [P]
        L.kvq_destroy.restype = ctypes.c_int
        L.kvq_length.argtypes = [P]
        L.kvq_length.restype = ctypes.c_int32
        L.kvq_get_layout.argtypes = [P, ctypes.POINTER(KvqLayout)]
        L.kvq_get_layout.restype = ctypes.c_int
        L.kvq_layout_for.argtypes = [CP, ctypes.POINTER(KvqLayout)]
        L.kvq_layout_for.restype = ctypes.c_int
        L.kvq_strerror.argtypes = [ctypes.c_int]
        L.kvq_strerror.restype = ctypes.c_char_p
        _lib = L
    return _lib


def _cfg_ptr(cfg):
    return None if cfg is None else ctypes.byref(cfg)


def kvq_workspace_bytes(cfg: KvqConfig) -> int:
    return lib().kvq_workspace_bytes(_cfg_ptr(cfg))


def kvq_layout_for(cfg: KvqConfig):
    """Returns (status, KvqLayout)."""
    out = KvqLayout()
    st = lib().kvq_layout_for(_cfg_ptr(cfg), ctypes.byref(out))
    return st, out


def kvq_create(cfg: KvqConfig, d_ws: int, ws_bytes: int):
    """Returns (status, handle).  handle is an int (opaque host pointer)."""
    h = ctypes.c_void_p()
    st = lib().kvq_create(_cfg_ptr(cfg), d_ws, ws_bytes, ctypes.byref(h))
    return st, h.value


def kvq_quantize_prefill(h: int, d_k: int, d_v: int, n_tokens: int, stream: int) -> int:
    return lib().kvq_quantize_prefill(h, d_k, d_v, n_tokens, stream)


def kvq_append_token(h: int, d_k: int, d_v: int, stream: int) -> int:
    return lib().kvq_append_token(h, d_k, d_v, stream)


def kvq_attend_decode(h: int, d_q: int, d_out: int, stream: int) -> int:
    return lib().kvq_attend_decode(h, d_q, d_out, stream)


def kvq_append_attend(h: int, d_k: int, d_v: int, d_q: int, d_out: int, stream: int) -> int:
    return lib().kvq_append_attend(h, d_k, d_v, d_q, d_out, stream)


def kvq_append_attend_static(h: int, d_k: int, d_v: int, d_q: int, d_out: int,
                             stream: int) -> int:
    return lib().kvq_append_attend_static(h, d_k, d_v, d_q, d_out, stream)


def kvq_error_metrics(h: int, d_k: int, d_v: int, d_q: int, d_metrics: int,
                      stream: int) -> int:
    return lib().kvq_error_metrics(h, d_k, d_v, d_q, d_metrics, stream)


def kvq_destroy(h: int) -> int:
    return lib().kvq_destroy(h)


def kvq_length(h: int) -> int:
    return lib().kvq_length(h)


def kvq_get_layout(h: int):
    """Returns (status, KvqLayout)."""
    out = KvqLayout()
    st = lib().kvq_get_layout(h, ctypes.byref(out))
    return st, out


def kvq_strerror(status: int) -> str:
    return lib().kvq_strerror(status).decode()
