"""KIVI-style asymmetric quantized KV cache and fused decode attention for
MI355X (gfx950).

All computation runs in the HIP kernels of ``libkvq.so`` behind the C ABI in
``include/kvq.h``; this package only marshals arguments (ctypes) and uses
PyTorch for device memory and streams.  There is no CPU fallback: importing
works without a GPU, but every call that enqueues work needs the built
library and a ROCm device.
"""
from ._lib import (  # noqa: F401
    KVQ_OK, KVQ_ERR_ARG, KVQ_ERR_UNSUPPORTED, KVQ_ERR_WORKSPACE, KVQ_ERR_STATE,
    KVQ_ERR_CAPACITY, KVQ_ERR_HIP, KVQ_ERR_SCRATCH, KVQ_STATIC_SCRATCH_BYTES, KVQ_F16, KVQ_F32, KVQ_KEYS_PER_TOKEN,
    KVQ_VALUES_PER_CHANNEL, KVQ_METRICS, KVQ_FORMAT_INT, KVQ_FORMAT_FP8_E4M3,
    KvqConfig, KvqLayout, KvqError, lib, library_path,
    kvq_workspace_bytes, kvq_create, kvq_quantize_prefill, kvq_append_token,
    kvq_attend_decode, kvq_append_attend, kvq_append_attend_static, kvq_error_metrics, kvq_destroy, kvq_length,
    kvq_get_layout, kvq_layout_for, kvq_strerror,
)
from .cache import QuantizedKVCache  # noqa: F401
