"""kvq_append_attend_static (split partials in the library's static device
scratch, no allocation) against kvq_append_attend (partials in the
workspace) through the C ABI: identically prefilled caches, the same decode
steps, planes compared bit for bit, outputs bit for bit where the kernels sum
in a fixed order (one query head per KV head) and to fp32 rounding where
they do not, and the output against the oracle within the attention
tolerance.
Calls in a row on one GPU share the scratch: a large step (many splits)
followed by smaller ones."""
import os

import numpy as np
import pytest
import torch

import oracle
import synth
from _parity import (_TORCH, assert_attention_close, assert_planes_equal, dev, gpu_planes,
                     make_cache, oracle_planes, to_gpu)
from quantized_decode_attention_keys_amd import QuantizedKVCache
from quantized_decode_attention_keys_amd import _lib as L

pytestmark = pytest.mark.gpu


def _pair(cfg, n0, cap, **kw):
    k = synth.make_keys(cfg, 5, 0, n0 + 2)
    v = synth.make_values(cfg, 5, 0, n0 + 2)
    caches = []
    for _ in range(2):
        c = make_cache(cfg, cap, **kw) if "format" not in kw else QuantizedKVCache(
            cfg.batch, cfg.q_heads, cfg.kv_heads, cfg.head_dim, cap, cfg.key_bits,
            cfg.value_bits, _TORCH[cfg.np_dtype], rope_base=cfg.rope_base, device=dev(),
            format=kw["format"])
        c.prefill(to_gpu(k[:, :, :n0]), to_gpu(v[:, :, :n0]))
        caches.append(c)
    return caches, k, v


def _step_both(cfg, caches, k, v, t, step):
    """One decode step on each cache: kvq_append_attend on the first,
    kvq_append_attend_static on the second; returns both outputs."""
    kt, vt = to_gpu(k[:, :, t]), to_gpu(v[:, :, t])
    q = to_gpu(synth.make_query(cfg, 5, step))
    stream = torch.cuda.current_stream(dev()).cuda_stream
    outs = []
    for c, fn in zip(caches, (L.kvq_append_attend, L.kvq_append_attend_static)):
        out = torch.full((cfg.batch, cfg.q_heads, cfg.head_dim), float("nan"),
                         dtype=torch.float32, device=dev())
        st = fn(c.handle, kt.data_ptr(), vt.data_ptr(), q.data_ptr(), out.data_ptr(), stream)
        assert st == L.KVQ_OK, L.kvq_strerror(st)
        outs.append(out)
    torch.cuda.synchronize()
    return [o.cpu().numpy() for o in outs]


def _run(cfg, n0, cap, fmt=None, **kw):
    extra = dict(kw)
    if fmt is not None:
        extra["format"] = fmt
    caches, k, v = _pair(cfg, n0, cap, **extra)
    # One query head per KV head: both paths sum in the same fixed order, so
    # their outputs agree bit for bit.  With several, waves take groups as
    # they become ready and the order varies between calls: the outputs then
    # agree to fp32 rounding, far inside the attention tolerance.
    exact = cfg.q_heads == cfg.kv_heads or fmt is not None
    for s in range(2):
        a, b = _step_both(cfg, caches, k, v, n0 + s, s)
        assert np.isfinite(a).all()
        if exact:
            assert np.array_equal(a, b), "static-scratch output differs from the workspace path"
        else:
            assert np.abs(a - b).max() <= 1e-5 * np.abs(a).max(), \
                "static-scratch output differs from the workspace path"
    n = n0 + 2
    assert len(caches[0]) == len(caches[1]) == n
    ga, gb = gpu_planes(caches[0]), gpu_planes(caches[1])
    if fmt is None:
        # every slot that holds data equals the oracle's, in both caches
        op = oracle_planes(cfg, k[:, :, :n], v[:, :, :n], cap, **kw)
        assert_planes_equal(ga, op, n, **kw)
        assert_planes_equal(gb, op, n, **kw)
        q = synth.make_query(cfg, 5, 1)
        ref = oracle.attend(op, q, n, cfg.key_bits, cfg.value_bits, cfg.kv_heads, **kw)
        assert_attention_close(b, ref)
    else:
        groups = -(-n // cfg.group)  # groups holding tokens; unopened ones are never read
        for name in ga:
            assert np.array_equal(ga[name][:, :, :groups], gb[name][:, :, :groups]), name
    for c in caches:
        c.close()


def test_static_scratch_matches_workspace_path():
    base = synth.CONFIGS["llama2_7b"]
    # 1) one sequence, 4 heads, 4096 tokens: 64 splits (133 KB of partials)
    _run(synth.scaled(base, batch=1, q_heads=4, kv_heads=4), 4094, 4160)
    # 2) then a smaller step on the same scratch: 8 query heads over 2 KV
    #    heads, 1000 tokens (31 splits)
    _run(synth.scaled(base, batch=1, q_heads=8, kv_heads=2), 998, 1024)
    # 3) a residual window (append, then attention: two launches)
    _run(synth.scaled(base, batch=1, q_heads=2, kv_heads=2), 500, 544, residual=32)
    # 4) an FP8 cache (its own attention kernel, split partials as well)
    _run(synth.scaled(base, batch=1, q_heads=2, kv_heads=2, key_bits=8, value_bits=8),
         300, 320, fmt=L.KVQ_FORMAT_FP8_E4M3)


def test_static_scratch_too_small_is_refused():
    """A step whose partials exceed the static array (forced to 256 splits
    over 32 output rows: 4.26 MB) is refused before anything is enqueued:
    status KVQ_ERR_SCRATCH, length unchanged, output untouched."""
    cfg = synth.scaled(synth.CONFIGS["llama2_7b"], batch=1, q_heads=32, kv_heads=4)
    n0 = 8192
    os.environ["KVQ_ATTEND_SPLITS"] = "256"  # read by kvq_create
    try:
        cache = make_cache(cfg, n0 + 32)
    finally:
        del os.environ["KVQ_ATTEND_SPLITS"]
    assert cfg.batch * cfg.q_heads * 256 * (cfg.head_dim + 2) * 4 > L.KVQ_STATIC_SCRATCH_BYTES
    k = to_gpu(synth.make_keys(cfg, 6, 0, n0 + 1))
    v = to_gpu(synth.make_values(cfg, 6, 0, n0 + 1))
    cache.prefill(k[:, :, :n0].contiguous(), v[:, :, :n0].contiguous())
    q = to_gpu(synth.make_query(cfg, 6))
    out = torch.full((cfg.batch, cfg.q_heads, cfg.head_dim), float("nan"), dtype=torch.float32,
                     device=dev())
    stream = torch.cuda.current_stream(dev()).cuda_stream
    kt, vt = k[:, :, n0].contiguous(), v[:, :, n0].contiguous()
    st = L.kvq_append_attend_static(cache.handle, kt.data_ptr(), vt.data_ptr(), q.data_ptr(),
                                    out.data_ptr(), stream)
    torch.cuda.synchronize()
    assert st == L.KVQ_ERR_SCRATCH
    assert len(cache) == n0
    assert torch.isnan(out).all()
    # the workspace path takes the same step
    assert L.kvq_append_attend(cache.handle, kt.data_ptr(), vt.data_ptr(), q.data_ptr(),
                               out.data_ptr(), stream) == L.KVQ_OK
    torch.cuda.synchronize()
    assert len(cache) == n0 + 1 and torch.isfinite(out).all()
    cache.close()
