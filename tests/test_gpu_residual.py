"""GPU parity with a residual window R (the most recent tokens kept in full
precision, keys and values): prefill planes and rings bit-exact, attention
within 2e-3 of max|out|, appends through many window departures and ring
wrap-arounds equal to the oracle's one-shot cache."""
import numpy as np
import pytest
import torch

import oracle
import synth
from _parity import (assert_attention_close, assert_planes_equal, gpu_planes, make_cache,
                     oracle_planes, to_gpu)

pytestmark = pytest.mark.gpu


def _check(cfg, cache, k, v, n, R, cap, q_seed=0, q_step=0):
    gp = gpu_planes(cache)
    op = oracle_planes(cfg, k[:, :, :n], v[:, :, :n], cap, residual=R)
    assert_planes_equal(gp, op, n, residual=R)
    q = synth.make_query(cfg, q_seed, q_step)
    out = cache.attend(to_gpu(q)).cpu().numpy()
    for pl in (op, gp):
        ref = oracle.attend(pl, q, n, cfg.key_bits, cfg.value_bits, cfg.kv_heads,
                            residual=R)
        assert_attention_close(out, ref)


@pytest.mark.parametrize("R", [32, 128])
@pytest.mark.parametrize("n", [1, 31, 100, 160, 161, 259, 600])
@pytest.mark.parametrize("qpk", [1, 4])
def test_prefill_d128(R, n, qpk):
    cfg = synth.scaled(synth.CONFIGS["llama2_7b"], batch=2, kv_heads=2, q_heads=2 * qpk,
                       n_tokens=n)
    cap = 640
    k = synth.make_keys(cfg, 0, 0, n)
    v = synth.make_values(cfg, 0, 0, n)
    cache = make_cache(cfg, cap, residual=R)
    cache.prefill(to_gpu(k), to_gpu(v))
    _check(cfg, cache, k, v, n, R, cap)


@pytest.mark.parametrize("bits", [(2, 2), (4, 8), (8, 4)])
@pytest.mark.parametrize("dtype", ["float16", "float32"])
def test_prefill_d64_and_widths(bits, dtype):
    cfg = synth.scaled(synth.CONFIGS["tiny"], kv_heads=2, q_heads=4, key_bits=bits[0],
                       value_bits=bits[1], dtype=dtype)
    n, R, cap = 230, 64, 256
    k = synth.make_keys(cfg, 0, 0, n)
    v = synth.make_values(cfg, 0, 0, n)
    cache = make_cache(cfg, cap, residual=R)
    cache.prefill(to_gpu(k), to_gpu(v))
    _check(cfg, cache, k, v, n, R, cap)


@pytest.mark.parametrize("qpk", [1, 2])
def test_append_through_window_departures(qpk):
    """Prefill 70 tokens with R = 64, then append 230 one at a time: blocks
    leave the window at n = 96, 128, ..., 288 and the 96-slot rings wrap
    around twice.  Planes equal the oracle's one-shot cache of all tokens."""
    cfg = synth.scaled(synth.CONFIGS["llama2_7b"], batch=2, kv_heads=3, q_heads=3 * qpk,
                       n_tokens=300)
    R, n0, n1, cap = 64, 70, 300, 320
    k = synth.make_keys(cfg, 0, 0, n1)
    v = synth.make_values(cfg, 0, 0, n1)
    cache = make_cache(cfg, cap, residual=R)
    cache.prefill(to_gpu(k[:, :, :n0].copy()), to_gpu(v[:, :, :n0].copy()))
    kg, vg = to_gpu(k), to_gpu(v)
    checks = {96, 97, 159, 160, 225, 300}
    for t in range(n0, n1):
        cache.append(kg[:, :, t].contiguous(), vg[:, :, t].contiguous())
        if t + 1 in checks:
            _check(cfg, cache, k, v, t + 1, R, cap, q_step=t)
    assert len(cache) == n1


def test_llama2_7b_shape_window_128():
    """The 7B decode shape with a 128-token window: prefill 4000 tokens,
    append 100 (three window departures), sampled rows against the oracle."""
    cfg = synth.CONFIGS["llama2_7b"]
    R, n0, n1 = 128, 4000, 4100
    cap = n1
    k = synth.make_keys(cfg, 0, 0, n1)
    v = synth.make_values(cfg, 0, 0, n1)
    cache = make_cache(cfg, cap, residual=R)
    cache.prefill(to_gpu(k[:, :, :n0].copy()), to_gpu(v[:, :, :n0].copy()))
    kg, vg = to_gpu(k[:, :, n0:].copy()), to_gpu(v[:, :, n0:].copy())
    for s in range(n1 - n0):
        cache.append(kg[:, :, s].contiguous(), vg[:, :, s].contiguous())
    q = synth.make_query(cfg, 0, 3)
    out = cache.attend(to_gpu(q)).cpu().numpy()
    torch.cuda.synchronize()
    b = 5
    one = synth.scaled(cfg, batch=1)
    op = oracle_planes(one, k[b:b + 1], v[b:b + 1], cap, residual=R)
    gp = {name: a[b:b + 1] for name, a in gpu_planes(cache).items()}
    assert_planes_equal(gp, op, n1, residual=R)
    for h in range(0, 32, 5):
        ref = oracle.attend(op, q[b:b + 1], n1, cfg.key_bits, cfg.value_bits, cfg.kv_heads,
                            rows=(h, h + 1), residual=R)
        assert_attention_close(out[b, h][None, :], ref)
