"""GPU parity with a sink window S (the first tokens kept in full precision,
keys and values), alone and with a residual window: prefill planes, rings
and sinks bit-exact, attention within 2e-3 of max|out|, appends across the
sink boundary equal to the oracle's one-shot cache."""
import pytest

import oracle
import synth
from _parity import (assert_attention_close, assert_planes_equal, gpu_planes, make_cache,
                     oracle_planes, to_gpu)

pytestmark = pytest.mark.gpu


def _check(cfg, cache, k, v, n, R, S, cap, q_step=0):
    gp = gpu_planes(cache)
    op = oracle_planes(cfg, k[:, :, :n], v[:, :, :n], cap, residual=R, sink=S)
    assert_planes_equal(gp, op, n, residual=R, sink=S)
    q = synth.make_query(cfg, 0, q_step)
    out = cache.attend(to_gpu(q)).cpu().numpy()
    for pl in (op, gp):
        ref = oracle.attend(pl, q, n, cfg.key_bits, cfg.value_bits, cfg.kv_heads,
                            residual=R, sink=S)
        assert_attention_close(out, ref)


@pytest.mark.parametrize("S,R", [(32, 0), (64, 0), (64, 64), (32, 128)])
@pytest.mark.parametrize("n", [10, 40, 100, 300])
@pytest.mark.parametrize("qpk", [1, 4])
def test_prefill_d128(S, R, n, qpk):
    cfg = synth.scaled(synth.CONFIGS["llama2_7b"], batch=2, kv_heads=2, q_heads=2 * qpk,
                       n_tokens=n)
    cap = 320
    k = synth.make_keys(cfg, 0, 0, n)
    v = synth.make_values(cfg, 0, 0, n)
    cache = make_cache(cfg, cap, residual=R, sink=S)
    cache.prefill(to_gpu(k), to_gpu(v))
    _check(cfg, cache, k, v, n, R, S, cap)


@pytest.mark.parametrize("bits", [(2, 2), (4, 2)])
@pytest.mark.parametrize("dtype", ["float16", "float32"])
def test_prefill_d128_one_head_windows(bits, dtype):
    """One query head per KV head at head_dim 128 with 2-bit keys, or 4-bit
    keys and 2-bit values (the variants whose scores are summed by DPP row
    rotations): sink and window chunks loaded in the rotated token order,
    binary16 and fp32 rows."""
    cfg = synth.scaled(synth.CONFIGS["llama2_7b"], batch=2, kv_heads=2, q_heads=2, n_tokens=300,
                       key_bits=bits[0], value_bits=bits[1], dtype=dtype)
    n, S, R, cap = 300, 32, 64, 320
    k = synth.make_keys(cfg, 0, 0, n)
    v = synth.make_values(cfg, 0, 0, n)
    cache = make_cache(cfg, cap, residual=R, sink=S)
    cache.prefill(to_gpu(k), to_gpu(v))
    _check(cfg, cache, k, v, n, R, S, cap)


@pytest.mark.parametrize("dtype", ["float16", "float32"])
def test_prefill_d64(dtype):
    cfg = synth.scaled(synth.CONFIGS["tiny"], kv_heads=2, q_heads=4, key_bits=4, value_bits=2,
                       dtype=dtype)
    n, S, R, cap = 200, 64, 32, 256
    k = synth.make_keys(cfg, 0, 0, n)
    v = synth.make_values(cfg, 0, 0, n)
    cache = make_cache(cfg, cap, residual=R, sink=S)
    cache.prefill(to_gpu(k), to_gpu(v))
    _check(cfg, cache, k, v, n, R, S, cap)


@pytest.mark.parametrize("R", [0, 64])
def test_append_across_the_sink(R):
    """Prefill 20 tokens (inside a 64-token sink), append 180: the sink fills
    at n = 64, then groups (R = 0) or window departures (R = 64) follow."""
    cfg = synth.scaled(synth.CONFIGS["llama2_7b"], batch=2, kv_heads=2, q_heads=4,
                       n_tokens=200)
    S, n0, n1, cap = 64, 20, 200, 224
    k = synth.make_keys(cfg, 0, 0, n1)
    v = synth.make_values(cfg, 0, 0, n1)
    cache = make_cache(cfg, cap, residual=R, sink=S)
    cache.prefill(to_gpu(k[:, :, :n0].copy()), to_gpu(v[:, :, :n0].copy()))
    kg, vg = to_gpu(k), to_gpu(v)
    checks = {21, 64, 65, 96, 97, 160, 161, 200}
    for t in range(n0, n1):
        cache.append(kg[:, :, t].contiguous(), vg[:, :, t].contiguous())
        if t + 1 in checks:
            _check(cfg, cache, k, v, t + 1, R, S, cap, q_step=t)
