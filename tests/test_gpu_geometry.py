"""GPU parity of the geometry ablation (keys per token and/or values per
channel) and of the error-where-consumed metrics: prefill and append planes
bit-exact against the oracle, attention within 2e-3 of max|out| (against the
oracle's planes and against the GPU's planes fed to the oracle), the metrics
within 1e-9 relative of the oracle's fp64 metrics."""
import numpy as np
import pytest
import torch

import oracle
import synth
from _parity import (TOL, _TORCH, assert_attention_close, assert_geometry_planes_equal,
                     assert_planes_equal, dev, gpu_planes, oracle_planes, to_gpu)
from quantized_decode_attention_keys_amd import QuantizedKVCache

pytestmark = pytest.mark.gpu

G = 32


def make_cache(cfg, cap, geometry=0, residual=0, sink=0):
    return QuantizedKVCache(cfg.batch, cfg.q_heads, cfg.kv_heads, cfg.head_dim, cap,
                            cfg.key_bits, cfg.value_bits, _TORCH[cfg.np_dtype],
                            rope_base=cfg.rope_base, device=dev(), residual=residual, sink=sink,
                            geometry=geometry)


def check(cfg, cache, k, v, n, geom, cap, q_step=0):
    gp = gpu_planes(cache)
    op = oracle.geometry_planes(k[:, :, :n], v[:, :, :n], cfg.key_bits, cfg.value_bits, geom,
                                max_tokens=cap)
    assert_geometry_planes_equal(gp, op, n, geom)
    q = synth.make_query(cfg, 0, q_step)
    out = cache.attend(to_gpu(q)).cpu().numpy()
    for pl in (op, gp):
        ref = oracle.attend_geometry(pl, q, n, cfg.key_bits, cfg.value_bits, cfg.kv_heads,
                                     geometry=geom)
        assert_attention_close(out, ref)


@pytest.mark.parametrize("geom", [1, 2, 3])
@pytest.mark.parametrize("n", [1, 31, 32, 100, 257])
@pytest.mark.parametrize("qpk", [1, 4])
def test_prefill_d128(geom, n, qpk):
    cfg = synth.scaled(synth.CONFIGS["ablation_7b"], batch=2, kv_heads=2, q_heads=2 * qpk,
                       n_tokens=n)
    cap = 288
    k, v = synth.make_keys(cfg, 0, 0, n), synth.make_values(cfg, 0, 0, n)
    cache = make_cache(cfg, cap, geom)
    cache.prefill(to_gpu(k), to_gpu(v))
    check(cfg, cache, k, v, n, geom, cap)


@pytest.mark.parametrize("bits", [(4, 4), (8, 8), (2, 8), (8, 2), (4, 2)])
@pytest.mark.parametrize("geom", [1, 2, 3])
def test_prefill_bit_widths(bits, geom):
    cfg = synth.scaled(synth.CONFIGS["ablation_7b"], batch=2, kv_heads=2, q_heads=4,
                       key_bits=bits[0], value_bits=bits[1], n_tokens=150)
    n, cap = 150, 160
    k, v = synth.make_keys(cfg, 1, 0, n), synth.make_values(cfg, 1, 0, n)
    cache = make_cache(cfg, cap, geom)
    cache.prefill(to_gpu(k), to_gpu(v))
    check(cfg, cache, k, v, n, geom, cap)


@pytest.mark.parametrize("dtype", ["float16", "float32"])
@pytest.mark.parametrize("geom", [1, 2, 3])
def test_prefill_d64(dtype, geom):
    cfg = synth.scaled(synth.CONFIGS["tiny"], kv_heads=2, q_heads=4, key_bits=4, value_bits=2,
                       dtype=dtype)
    n, cap = 200, 224
    k, v = synth.make_keys(cfg, 0, 0, n), synth.make_values(cfg, 0, 0, n)
    cache = make_cache(cfg, cap, geom)
    cache.prefill(to_gpu(k), to_gpu(v))
    check(cfg, cache, k, v, n, geom, cap)


@pytest.mark.parametrize("geom", [1, 2, 3])
def test_append_through_group_flushes(geom):
    """Prefill 20 tokens, append 130 one at a time: per-token operands are
    quantized on arrival, per-channel ones flush a group every 32 tokens; the
    planes equal the oracle's one-shot planes of all tokens at every check."""
    cfg = synth.scaled(synth.CONFIGS["ablation_7b"], batch=2, kv_heads=2, q_heads=4,
                       n_tokens=150)
    n0, n1, cap = 20, 150, 160
    k, v = synth.make_keys(cfg, 2, 0, n1), synth.make_values(cfg, 2, 0, n1)
    cache = make_cache(cfg, cap, geom)
    cache.prefill(to_gpu(k[:, :, :n0]), to_gpu(v[:, :, :n0]))
    kd, vd = to_gpu(k), to_gpu(v)
    for t in range(n0, n1):
        cache.append(kd[:, :, t].contiguous(), vd[:, :, t].contiguous())
        if t + 1 in (64, 97, 150):
            check(cfg, cache, k, v, t + 1, geom, cap, q_step=t)


@pytest.mark.parametrize("geom", [0, 1, 2, 3])
def test_metrics_match_the_oracle(geom):
    cfg = synth.scaled(synth.CONFIGS["ablation_7b"], batch=2, kv_heads=2, q_heads=4,
                       n_tokens=300)
    n, cap = 300, 320
    k, v = synth.make_keys(cfg, 3, 0, n), synth.make_values(cfg, 3, 0, n)
    q = synth.make_query(cfg, 3)
    cache = make_cache(cfg, cap, geom)
    cache.prefill(to_gpu(k), to_gpu(v))
    got = cache.error_metrics(to_gpu(k), to_gpu(v), to_gpu(q)).cpu().numpy()
    pl = oracle.geometry_planes(k, v, cfg.key_bits, cfg.value_bits, geom, max_tokens=cap)
    want, _ = oracle.error_metrics(pl, k, v, q, n, cfg.key_bits, cfg.value_bits, cfg.kv_heads,
                                   geometry=geom)
    assert np.allclose(got, [want[m] for m in oracle.METRICS], rtol=1e-9, atol=0), (got, want)


@pytest.mark.parametrize("R,S", [(64, 0), (0, 32), (128, 64)])
def test_metrics_with_windows(R, S):
    cfg = synth.scaled(synth.CONFIGS["llama2_7b"], batch=2, kv_heads=2, q_heads=4,
                       n_tokens=260)
    n, cap = 260, 288
    k, v = synth.make_keys(cfg, 4, 0, n), synth.make_values(cfg, 4, 0, n)
    q = synth.make_query(cfg, 4)
    cache = make_cache(cfg, cap, 0, residual=R, sink=S)
    cache.prefill(to_gpu(k), to_gpu(v))
    got = cache.error_metrics(to_gpu(k), to_gpu(v), to_gpu(q)).cpu().numpy()
    pl = oracle_planes(cfg, k, v, cap, residual=R, sink=S)
    assert_planes_equal(gpu_planes(cache), pl, n, residual=R, sink=S)
    want, _ = oracle.error_metrics(pl, k, v, q, n, cfg.key_bits, cfg.value_bits, cfg.kv_heads,
                                   residual=R, sink=S)
    assert np.allclose(got, [want[m] for m in oracle.METRICS], rtol=1e-9, atol=0), (got, want)


def test_full_7b_shape_both_flipped():
    """The ablation workload at its full shape (batch 8, 32 heads, 4095-token
    prompt + 1 append) with both axes flipped, in the launch configuration
    the bench times: planes of sequences 0 and 6 bit-exact, attention of all
    their heads within tolerance."""
    cfg = synth.CONFIGS["ablation_7b"]
    n, cap, geom = 4096, 4128, 3
    k = synth.make_keys(cfg, 0, 0, n)
    v = synth.make_values(cfg, 0, 0, n)
    cache = make_cache(cfg, cap, geom)
    cache.prefill(to_gpu(k[:, :, :n - 1]), to_gpu(v[:, :, :n - 1]))
    cache.append(to_gpu(k[:, :, n - 1]), to_gpu(v[:, :, n - 1]))
    q = synth.make_query(cfg, 0, 0)
    out = cache.attend(to_gpu(q)).cpu().numpy()
    gp = gpu_planes(cache)
    seqs = [0, 6]
    op = oracle.geometry_planes(k[seqs], v[seqs], cfg.key_bits, cfg.value_bits, geom,
                                max_tokens=cap)
    assert_geometry_planes_equal(gp, op, n, geom, seqs=seqs)
    ref = oracle.attend_geometry(op, q[seqs], n, cfg.key_bits, cfg.value_bits, cfg.kv_heads,
                                 geometry=geom)
    assert_attention_close(out[seqs], ref, TOL)


def test_metrics_reject_bad_shapes():
    cfg = synth.scaled(synth.CONFIGS["tiny"], kv_heads=2, q_heads=4)
    cache = make_cache(cfg, 64, 1)
    k = torch.zeros((1, 2, 10, 64), device=dev())
    with pytest.raises(Exception):
        cache.error_metrics(k, k, torch.zeros((1, 4, 64), device=dev()))  # empty cache
    cache.prefill(k, k)
    with pytest.raises(ValueError):
        cache.error_metrics(k[:, :, :9].contiguous(), k, torch.zeros((1, 4, 64), device=dev()))
