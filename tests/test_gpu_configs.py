"""GPU parity at the full sizes of the larger workloads, in the launch
configuration the bench uses: each decode step is one kvq_append_attend call
(the library picks splits and waves from the shape).  Codes, metadata and
tail bit-exact for sampled sequences; attention within 2e-3 of max|out| for
sampled (sequence, head) rows, computed by the oracle from the same seeded
inputs."""
import numpy as np
import pytest
import torch

import oracle
import synth
from _parity import assert_attention_close, assert_planes_equal, gpu_planes, make_cache, to_gpu

pytestmark = pytest.mark.gpu


def _oracle_seq_planes(cfg, b, n, cap):
    one = synth.scaled(cfg, batch=1)
    k = synth.make_keys(cfg, 0, 0, n, seqs=[b])
    v = synth.make_values(cfg, 0, 0, n, seqs=[b])
    kc, km, kt = oracle.quantize_keys(k, one.key_bits, one.group, max_tokens=cap)
    vc, vm = oracle.quantize_values(v, one.value_bits, one.group, max_tokens=cap)
    return dict(k_codes=kc, k_meta=km, k_tail=kt, v_codes=vc, v_meta=vm)


def _check_rows(cfg, out, q, planes, b, n, heads=None):
    heads = range(cfg.q_heads) if heads is None else heads
    for h in heads:
        r = b * cfg.q_heads + h
        ref = oracle.attend(planes, q[b:b + 1], n, cfg.key_bits, cfg.value_bits, cfg.kv_heads,
                            cfg.group, cfg.rope_base, rows=(h, h + 1))
        assert_attention_close(out[b, h][None, :], ref)


def test_llama2_13b_decode_loop():
    """Prefill 8192 tokens, then 64 decode steps, each appending one token
    and attending in one launch (n = 8193 ... 8256, key groups flushed from
    the tail at steps 32 and 64)."""
    cfg = synth.CONFIGS["llama2_13b"]
    n0, steps = 8192, 64
    cap = n0 + steps
    cache = make_cache(cfg, cap)
    cache.prefill(to_gpu(synth.make_keys(cfg, 0, 0, n0)), to_gpu(synth.make_values(cfg, 0, 0, n0)))
    k_new = to_gpu(synth.make_keys(cfg, 0, n0, cap))
    v_new = to_gpu(synth.make_values(cfg, 0, n0, cap))
    seqs = (3, 12)
    outs = {}
    for s in range(1, steps + 1):
        q = synth.make_query(cfg, 0, s)
        out = cache.append_attend(k_new[:, :, s - 1].contiguous(),
                                  v_new[:, :, s - 1].contiguous(), to_gpu(q))
        if s in (1, 31, 32, 33, 63, 64):
            outs[s] = (q, out.cpu().numpy())
    torch.cuda.synchronize()
    assert len(cache) == cap
    gp = gpu_planes(cache)
    for b in seqs:
        op = _oracle_seq_planes(cfg, b, cap, cap)
        assert_planes_equal(gp, op, cap, seqs=[b])
    # whole sequences (all 40 heads) at steps around both flushes
    for s, (q, out) in outs.items():
        n = n0 + s
        for b in seqs:
            _check_rows(cfg, out, q, _oracle_seq_planes(cfg, b, n, cap), b, n)


def test_llama2_13b_b4_sampled():
    cfg = synth.CONFIGS["llama2_13b_b4"]
    n = cfg.n_tokens
    cache = make_cache(cfg, n)
    cache.prefill(to_gpu(synth.make_keys(cfg, 0, 0, n - 1)),
                  to_gpu(synth.make_values(cfg, 0, 0, n - 1)))
    q = synth.make_query(cfg, 0, 0)
    out = cache.append_attend(to_gpu(synth.make_keys(cfg, 0, n - 1, n)[:, :, 0]),
                              to_gpu(synth.make_values(cfg, 0, n - 1, n)[:, :, 0]),
                              to_gpu(q)).cpu().numpy()
    gp = gpu_planes(cache)
    b = 9
    op = _oracle_seq_planes(cfg, b, n, n)
    assert_planes_equal(gp, op, n, seqs=[b])
    _check_rows(cfg, out, q, op, b, n)


def test_long_context_sampled():
    """131071-token prompt plus one decode step (n = 131072, keys at 4
    bits, values at 2), split over many blocks (the last one appends) and
    merged by the combine kernel; all 32 heads checked."""
    cfg = synth.CONFIGS["long"]
    n = cfg.n_tokens
    cache = make_cache(cfg, n)
    cache.prefill(to_gpu(synth.make_keys(cfg, 0, 0, n - 1)),
                  to_gpu(synth.make_values(cfg, 0, 0, n - 1)))
    last_k = to_gpu(synth.make_keys(cfg, 0, n - 1, n)[:, :, 0])
    last_v = to_gpu(synth.make_values(cfg, 0, n - 1, n)[:, :, 0])
    q = synth.make_query(cfg, 0, 0)
    out = cache.append_attend(last_k, last_v, to_gpu(q)).cpu().numpy()
    gp = gpu_planes(cache)
    op = _oracle_seq_planes(cfg, 0, n, n)
    assert_planes_equal(gp, op, n)
    _check_rows(cfg, out, q, op, 0, n)


def test_long_context_ragged_tail():
    """The long workload with a 31-token tail (n = 131071), attention alone
    (kvq_attend_decode) after the prefill."""
    cfg = synth.scaled(synth.CONFIGS["long"], n_tokens=131071)
    n = cfg.n_tokens
    cache = make_cache(cfg, n)
    cache.prefill(to_gpu(synth.make_keys(cfg, 0, 0, n)), to_gpu(synth.make_values(cfg, 0, 0, n)))
    q = synth.make_query(cfg, 0, 1)
    out = cache.attend(to_gpu(q)).cpu().numpy()
    op = _oracle_seq_planes(cfg, 0, n, n)
    _check_rows(cfg, out, q, op, 0, n, heads=(5,))


def test_gqa_sampled():
    """64 sequences, 32 query heads over 8 KV heads, 16384 tokens: planes and
    all 32 heads of four sequences."""
    cfg = synth.CONFIGS["gqa"]
    n = cfg.n_tokens
    cache = make_cache(cfg, n)
    cache.prefill(to_gpu(synth.make_keys(cfg, 0, 0, n - 1)),
                  to_gpu(synth.make_values(cfg, 0, 0, n - 1)))
    q = synth.make_query(cfg, 0, 0)
    out = cache.append_attend(to_gpu(synth.make_keys(cfg, 0, n - 1, n)[:, :, 0]),
                              to_gpu(synth.make_values(cfg, 0, n - 1, n)[:, :, 0]),
                              to_gpu(q)).cpu().numpy()
    gp = gpu_planes(cache)
    for b in (0, 17, 41, 63):
        op = _oracle_seq_planes(cfg, b, n, n)
        assert_planes_equal(gp, op, n, seqs=[b])
        _check_rows(cfg, out, q, op, b, n)
