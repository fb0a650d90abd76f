"""CPU tests of the C ABI boundary: the library loads, exports every function
include/kvq.h declares, computes layouts, and rejects bad arguments before
any HIP call (so these run without a GPU)."""
import ctypes
import os
import re
import subprocess

import pytest

import quantized_decode_attention_keys_amd as kvq
from quantized_decode_attention_keys_amd import _lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvq.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kvq_[a-z_]+)\s*\(", text)))


def cfg(**kw):
    base = dict(batch=2, q_heads=8, kv_heads=2, head_dim=128, max_tokens=1000, group=32,
                key_bits=2, value_bits=4, dtype=L.KVQ_F16, rope_base=10000.0)
    base.update(kw)
    return L.KvqConfig(**base)


def test_library_exports_every_declared_function():
    names = _declared()
    assert "kvq_attend_decode" in names and len(names) >= 10
    syms = subprocess.check_output(["nm", "-D", "--defined-only", L.library_path()]).decode()
    exported = set(re.findall(r" T (\w+)", syms))
    for n in names:
        assert n in exported, n
        assert hasattr(L.lib(), n)


def test_python_binding_names_match_the_header():
    for n in _declared():
        assert callable(getattr(kvq, n)), n


def test_layout_sizes_alignment_and_order():
    c = cfg()
    st, lay = L.kvq_layout_for(c)
    assert st == L.KVQ_OK
    assert lay.gcap == 32 and lay.tcap == 1024
    offs = [lay.k_codes, lay.k_meta, lay.v_codes, lay.v_meta, lay.k_tail, lay.v_tail,
            lay.k_sink, lay.v_sink, lay.rope_group, lay.rope_offset, lay.partials,
            lay.total_bytes]
    assert offs == sorted(offs)
    assert all(o % 256 == 0 for o in offs)
    nb, h, D = 2, 2, 128
    assert lay.k_meta - lay.k_codes >= nb * h * 32 * D * 2 * 4       # Wk = 2
    assert lay.v_codes - lay.k_meta >= nb * h * 32 * D * 4
    assert lay.v_meta - lay.v_codes >= nb * h * 1024 * 4 * 4 * 4     # D/G = 4, Wv = 4
    assert lay.k_tail - lay.v_meta >= nb * h * 1024 * 4 * 4
    assert lay.v_tail - lay.k_tail >= nb * h * 32 * D * 2
    assert lay.k_sink == lay.v_tail == lay.v_sink == lay.rope_group  # no window planes
    assert lay.tail_slots == 32
    assert L.kvq_workspace_bytes(c) == lay.total_bytes
    assert lay.max_splits >= 1


def test_layout_with_sink_window():
    st, lay = L.kvq_layout_for(cfg(sink=64))
    assert st == L.KVQ_OK
    nb, h, D = 2, 2, 128
    assert lay.v_sink - lay.k_sink >= nb * h * 64 * D * 2
    assert lay.rope_group - lay.v_sink >= nb * h * 64 * D * 2


def test_layout_with_residual_window():
    c = cfg(residual=128)
    st, lay = L.kvq_layout_for(c)
    assert st == L.KVQ_OK and lay.tail_slots == 160
    nb, h, D = 2, 2, 128
    assert lay.v_tail - lay.k_tail >= nb * h * 160 * D * 2
    assert lay.k_sink - lay.v_tail >= nb * h * 160 * D * 2
    _, lay0 = L.kvq_layout_for(cfg())
    assert lay.total_bytes > lay0.total_bytes


@pytest.mark.parametrize("field,value,status", [
    ("batch", 0, L.KVQ_ERR_ARG),
    ("q_heads", 3, L.KVQ_ERR_ARG),           # not a multiple of kv_heads
    ("head_dim", 96, L.KVQ_ERR_UNSUPPORTED),
    ("group", 64, L.KVQ_ERR_UNSUPPORTED),
    ("key_bits", 3, L.KVQ_ERR_UNSUPPORTED),
    ("value_bits", 16, L.KVQ_ERR_UNSUPPORTED),
    ("q_heads", 32, L.KVQ_ERR_UNSUPPORTED),  # 16 query heads per KV head
    ("dtype", 7, L.KVQ_ERR_ARG),
    ("rope_base", 0.5, L.KVQ_ERR_ARG),
    ("max_tokens", 0, L.KVQ_ERR_ARG),
    ("residual", -32, L.KVQ_ERR_ARG),
    ("residual", 48, L.KVQ_ERR_UNSUPPORTED),      # not a multiple of the group
    ("residual", 1056, L.KVQ_ERR_UNSUPPORTED),    # beyond the 1024-token window
    ("sink", -32, L.KVQ_ERR_ARG),
    ("sink", 40, L.KVQ_ERR_UNSUPPORTED),
    ("sink", 2048, L.KVQ_ERR_UNSUPPORTED),
    ("geometry", -1, L.KVQ_ERR_ARG),
    ("geometry", 4, L.KVQ_ERR_ARG),
    ("format", 2, L.KVQ_ERR_ARG),
    ("format", 1, L.KVQ_ERR_UNSUPPORTED),         # FP8 needs key_bits == value_bits == 8
])
def test_bad_configs_rejected_on_host(field, value, status):
    c = cfg(**{field: value})
    assert L.kvq_workspace_bytes(c) == 0
    st, _ = L.kvq_layout_for(c)
    assert st == status
    # create fails the same way before touching the device
    st, h = L.kvq_create(c, 0x10000, 1 << 40)
    assert st == status and h is None


@pytest.mark.parametrize("geometry", [1, 2, 3])
@pytest.mark.parametrize("window", [dict(residual=32), dict(sink=32)])
def test_geometry_ablation_has_no_windows(geometry, window):
    c = cfg(geometry=geometry, **window)
    assert L.kvq_layout_for(c)[0] == L.KVQ_ERR_UNSUPPORTED
    assert L.kvq_workspace_bytes(cfg(geometry=geometry)) > 0


@pytest.mark.parametrize("extra", [dict(residual=32), dict(sink=32), dict(geometry=1),
                                   dict(batch=1100, q_heads=64, kv_heads=8)])
def test_fp8_limits(extra):
    c = cfg(key_bits=8, value_bits=8, format=L.KVQ_FORMAT_FP8_E4M3, **extra)
    assert L.kvq_layout_for(c)[0] == L.KVQ_ERR_UNSUPPORTED
    st, lay = L.kvq_layout_for(cfg(key_bits=8, value_bits=8, format=L.KVQ_FORMAT_FP8_E4M3))
    _, lay8 = L.kvq_layout_for(cfg(key_bits=8, value_bits=8))
    assert st == L.KVQ_OK and lay.total_bytes == lay8.total_bytes


def test_layout_with_values_per_channel():
    """Flipped planes keep their sizes; values grouped per channel get a
    G-slot tail (keys per token leave the key tail unused)."""
    _, lay0 = L.kvq_layout_for(cfg())
    for geometry in (1, 2, 3):
        st, lay = L.kvq_layout_for(cfg(geometry=geometry))
        assert st == L.KVQ_OK and lay.tail_slots == 32
        assert (lay.k_meta - lay.k_codes, lay.v_codes - lay.k_meta, lay.v_meta - lay.v_codes,
                lay.k_tail - lay.v_meta) == (lay0.k_meta - lay0.k_codes,
                                             lay0.v_codes - lay0.k_meta,
                                             lay0.v_meta - lay0.v_codes,
                                             lay0.k_tail - lay0.v_meta)
        if geometry & L.KVQ_VALUES_PER_CHANNEL:
            assert lay.k_sink - lay.v_tail >= 2 * 2 * 32 * 128 * 2
        else:
            assert lay.k_sink == lay.v_tail


def test_create_rejects_bad_workspace_before_any_hip_call():
    c = cfg()
    need = L.kvq_workspace_bytes(c)
    assert L.kvq_create(c, 0, need)[0] == L.KVQ_ERR_ARG
    assert L.kvq_create(c, 0x10000, need - 1)[0] == L.KVQ_ERR_WORKSPACE
    assert L.kvq_create(c, 0x10080, need)[0] == L.KVQ_ERR_WORKSPACE   # not 256-B aligned
    assert L.lib().kvq_create(None, ctypes.c_void_p(0x10000), need, None) == L.KVQ_ERR_ARG


def test_null_handle_calls():
    assert L.kvq_length(None) == -1
    assert L.kvq_destroy(None) == L.KVQ_ERR_ARG
    assert L.kvq_get_layout(None)[0] == L.KVQ_ERR_ARG
    assert L.kvq_quantize_prefill(None, 1, 1, 4, None) == L.KVQ_ERR_ARG
    assert L.kvq_append_token(None, 1, 1, None) == L.KVQ_ERR_ARG
    assert L.kvq_attend_decode(None, 1, 1, None) == L.KVQ_ERR_ARG
    assert L.kvq_append_attend(None, 1, 1, 1, 1, None) == L.KVQ_ERR_ARG
    assert L.kvq_error_metrics(None, 1, 1, 1, 1, None) == L.KVQ_ERR_ARG


def test_strerror_covers_every_status():
    for s in (L.KVQ_OK, L.KVQ_ERR_ARG, L.KVQ_ERR_UNSUPPORTED, L.KVQ_ERR_WORKSPACE,
              L.KVQ_ERR_STATE, L.KVQ_ERR_CAPACITY, L.KVQ_ERR_HIP):
        assert L.kvq_strerror(s) != "unknown status"
    assert L.kvq_strerror(12345) == "unknown status"
