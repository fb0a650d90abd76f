"""GPU parity of the quantizer's edge cases through every kernel that writes
the packed planes, bit-exact against the oracle.

The quantizer ("Your KV Cache Doesn't Have a Bit Problem...", section "What
Quantization Error Is Actually Made Of"): zero point = group minimum, step =
range / (2^B - 1), nearest step; readings where the page is silent: binary16
zero and step rounded once, exact ties to the even code, a zero step gives
code 0.  Every quantized group of these caches is an edge-case group
(tests/_edges.py): the hand-worked golden groups, zero-range groups (a
constant channel over 32 tokens, a constant token row), exact half-step ties
and values a few ulps either side of them (the kernels' exact fallback
band), subnormal and zero steps, a binary16 rounding tie of the step itself,
large magnitudes, and fp32 inputs whose minimum is not a binary16 value.

Writers covered: the one-launch prefill codec (keys and values together),
the value codec alone (prompts shorter than a group), the append kernel
across group flushes, the residual-window append across window departures,
the decode-attention kernel's own append (one launch per step), and the
geometry-ablation prefill and append kernels (keys per token, values per
channel).
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from _edges import edge_groups, tile_keys, tile_values
from _parity import (assert_attention_close, assert_geometry_planes_equal, assert_planes_equal,
                     gpu_planes, make_cache, oracle_planes, to_gpu)

pytestmark = pytest.mark.gpu

LAYOUTS = {
    # (dtype, head_dim, query heads per KV head)
    "f16_d128": ("float16", 128, 1),
    "f16_d128_gqa4": ("float16", 128, 4),
    "f32_d64": ("float32", 64, 1),
}
BITS = [(2, 2), (4, 4), (8, 8), (2, 8), (8, 4)]


def _cfg(layout, bits, n):
    dtype, D, qpk = LAYOUTS[layout]
    return synth.scaled(synth.CONFIGS["llama2_7b"], batch=2, kv_heads=2, q_heads=2 * qpk,
                        head_dim=D, n_tokens=n, key_bits=bits[0], value_bits=bits[1],
                        dtype=dtype)


def _inputs(cfg, n, seed=0):
    _, kg = edge_groups(cfg.key_bits, cfg.np_dtype)
    _, vg = edge_groups(cfg.value_bits, cfg.np_dtype)
    k = tile_keys(kg, cfg.batch, cfg.kv_heads, n, cfg.head_dim, seed)
    v = tile_values(vg, cfg.batch, cfg.kv_heads, n, cfg.head_dim, seed)
    return k, v


def _query(cfg, step=0):
    # small queries keep the scores of the +-65504 key groups moderate
    q = synth.make_query(cfg, 7, step).astype(np.float32) * 1e-3
    return np.ascontiguousarray(q.astype(cfg.np_dtype))


def _check_attention(cfg, out, planes_o, planes_g, q, n, residual=0):
    for pl in (planes_o, planes_g):
        ref = oracle.attend(pl, q, n, cfg.key_bits, cfg.value_bits, cfg.kv_heads,
                            residual=residual)
        assert_attention_close(out, ref)


@pytest.mark.parametrize("bits", BITS)
@pytest.mark.parametrize("layout", sorted(LAYOUTS))
def test_prefill_edges(layout, bits):
    """Prefill of 69 tokens: two key groups and 69 value tokens through the
    one-launch codec; 5 keys verbatim in the tail."""
    n, cap = 69, 96
    cfg = _cfg(layout, bits, n)
    k, v = _inputs(cfg, n)
    cache = make_cache(cfg, cap)
    cache.prefill(to_gpu(k), to_gpu(v))
    gp = gpu_planes(cache)
    op = oracle_planes(cfg, k, v, cap)
    assert_planes_equal(gp, op, n)
    q = _query(cfg)
    out = cache.attend(to_gpu(q)).cpu().numpy()
    _check_attention(cfg, out, op, gp, q, n)


@pytest.mark.parametrize("bits", [(2, 2), (4, 4), (8, 8)])
@pytest.mark.parametrize("layout", ["f16_d128", "f32_d64"])
def test_prefill_values_only(layout, bits):
    """A 20-token prompt fills no key group: the value codec runs alone and
    every key stays in the tail."""
    n, cap = 20, 64
    cfg = _cfg(layout, bits, n)
    k, v = _inputs(cfg, n, seed=1)
    cache = make_cache(cfg, cap)
    cache.prefill(to_gpu(k), to_gpu(v))
    assert_planes_equal(gpu_planes(cache), oracle_planes(cfg, k, v, cap), n)


@pytest.mark.parametrize("path", ["append", "append_attend"])
@pytest.mark.parametrize("bits", BITS)
@pytest.mark.parametrize("layout", sorted(LAYOUTS))
def test_append_edges(layout, bits, path):
    """Prefill 30 tokens, then append 39 one at a time (key groups flushed
    from the tail at n = 32 and 64; every value quantized on arrival), either
    through the append kernel or through the attention kernel's own append
    (kvq_append_attend, one launch per step)."""
    n0, n1, cap = 30, 69, 96
    cfg = _cfg(layout, bits, n1)
    k, v = _inputs(cfg, n1, seed=2)
    cache = make_cache(cfg, cap)
    cache.prefill(to_gpu(k[:, :, :n0]), to_gpu(v[:, :, :n0]))
    kg, vg = to_gpu(k), to_gpu(v)
    q = _query(cfg, 1)
    qg = to_gpu(q)
    out = None
    for t in range(n0, n1):
        if path == "append":
            cache.append(kg[:, :, t].contiguous(), vg[:, :, t].contiguous())
        else:
            out = cache.append_attend(kg[:, :, t].contiguous(), vg[:, :, t].contiguous(), qg)
        n = t + 1
        if n in (32, 33, 64, 69):
            gp = gpu_planes(cache)
            op = oracle_planes(cfg, k[:, :, :n], v[:, :, :n], cap)
            assert_planes_equal(gp, op, n)
    if path == "append_attend":
        _check_attention(cfg, out.cpu().numpy(), op, gp, q, n1)


@pytest.mark.parametrize("bits", [(2, 2), (4, 4), (8, 8), (2, 8)])
@pytest.mark.parametrize("layout", ["f16_d128", "f32_d64"])
def test_residual_window_edges(layout, bits):
    """A 32-token residual window: prefill 70 tokens (one block quantized by
    the prefill codec, the rest in the rings), then append 60 (blocks leave
    the window at n = 96 and 128 and are quantized from the rings)."""
    R, n0, n1, cap = 32, 70, 130, 160
    cfg = _cfg(layout, bits, n1)
    k, v = _inputs(cfg, n1, seed=3)
    cache = make_cache(cfg, cap, residual=R)
    cache.prefill(to_gpu(k[:, :, :n0]), to_gpu(v[:, :, :n0]))
    op = oracle_planes(cfg, k[:, :, :n0], v[:, :, :n0], cap, residual=R)
    assert_planes_equal(gpu_planes(cache), op, n0, residual=R)
    kg, vg = to_gpu(k), to_gpu(v)
    for t in range(n0, n1):
        cache.append(kg[:, :, t].contiguous(), vg[:, :, t].contiguous())
        n = t + 1
        if n in (95, 96, 97, 128, 130):
            gp = gpu_planes(cache)
            op = oracle_planes(cfg, k[:, :, :n], v[:, :, :n], cap, residual=R)
            assert_planes_equal(gp, op, n, residual=R)
    q = _query(cfg, 2)
    out = cache.attend(to_gpu(q)).cpu().numpy()
    _check_attention(cfg, out, op, gp, q, n1, residual=R)


@pytest.mark.parametrize("geom", [1, 2, 3])
@pytest.mark.parametrize("bits", [(2, 2), (4, 8), (8, 4)])
def test_geometry_edges(geom, bits):
    """The geometry ablation's writers: keys per token go through the value
    codec, values per channel through the key codec (and a value tail), at
    prefill (69 tokens) and on append (30 more, flushing value groups per
    channel at n = 96)."""
    n0, n1, cap = 69, 99, 128
    cfg = _cfg("f16_d128", bits, n1)
    k, v = _inputs(cfg, n1, seed=4)
    cache = make_cache(cfg, cap, geometry=geom)
    cache.prefill(to_gpu(k[:, :, :n0]), to_gpu(v[:, :, :n0]))
    op = oracle.geometry_planes(k[:, :, :n0], v[:, :, :n0], cfg.key_bits, cfg.value_bits, geom,
                                max_tokens=cap)
    assert_geometry_planes_equal(gpu_planes(cache), op, n0, geom)
    kg, vg = to_gpu(k), to_gpu(v)
    for t in range(n0, n1):
        cache.append(kg[:, :, t].contiguous(), vg[:, :, t].contiguous())
    op = oracle.geometry_planes(k, v, cfg.key_bits, cfg.value_bits, geom, max_tokens=cap)
    assert_geometry_planes_equal(gpu_planes(cache), op, n1, geom)
    torch.cuda.synchronize()
