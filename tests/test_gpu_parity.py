"""GPU parity: the HIP path through the C ABI against the oracle on the same
seeded inputs.  Codes, metadata and the key tail bit-exact; attention within
2e-3 of max|out|, checked twice: against the oracle on its own planes and
against the oracle fed the GPU's planes (isolating attention error)."""
import numpy as np
import pytest
import torch

import oracle
import synth
from _parity import (assert_attention_close, assert_planes_equal, gpu_planes, make_cache,
                     oracle_planes, run_prefill, to_gpu)

pytestmark = pytest.mark.gpu

TINY = synth.CONFIGS["tiny"]


def _attend_both(cfg, cache, planes_o, planes_g, n, seed=0, step=0):
    q = synth.make_query(cfg, seed, step)
    out = cache.attend(to_gpu(q)).cpu().numpy()
    ref = oracle.attend(planes_o, q, n, cfg.key_bits, cfg.value_bits, cfg.kv_heads)
    assert_attention_close(out, ref)
    ref_g = oracle.attend(planes_g, q, n, cfg.key_bits, cfg.value_bits, cfg.kv_heads)
    assert_attention_close(out, ref_g)


@pytest.mark.parametrize("bits", [(2, 2), (4, 4), (8, 8), (4, 2), (2, 8)])
@pytest.mark.parametrize("n", [1, 31, 32, 256, 257, 287, 288, 300])
def test_tiny_prefill_planes_and_attention(bits, n):
    cfg = synth.scaled(TINY, key_bits=bits[0], value_bits=bits[1])
    cache, k, v = run_prefill(cfg, n, max_tokens=320)
    gp = gpu_planes(cache)
    op = oracle_planes(cfg, k, v, 320)
    assert_planes_equal(gp, op, n)
    _attend_both(cfg, cache, op, gp, n)


@pytest.mark.parametrize("qpk", [1, 2, 4, 8])
@pytest.mark.parametrize("dtype", ["float16", "float32"])
def test_d128_gqa_ragged(qpk, dtype):
    cfg = synth.scaled(synth.CONFIGS["llama2_7b"], batch=2, kv_heads=2, q_heads=2 * qpk,
                       n_tokens=1000, dtype=dtype)
    n = 1000  # 31 full groups + 8 tail tokens, several splits
    cache, k, v = run_prefill(cfg, n, max_tokens=1100)
    gp = gpu_planes(cache)
    op = oracle_planes(cfg, k, v, 1100)
    assert_planes_equal(gp, op, n)
    _attend_both(cfg, cache, op, gp, n)


@pytest.mark.parametrize("bits", [(4, 4), (8, 8), (4, 2), (2, 4), (2, 8), (8, 2)])
@pytest.mark.parametrize("qpk", [1, 2, 4])
def test_d128_bits_ragged(bits, qpk):
    """head_dim 128 at every key/value width pair the value-lane mappings
    depend on (words per token row, words per lane), n = 1000."""
    cfg = synth.scaled(synth.CONFIGS["llama2_7b"], batch=2, kv_heads=2, q_heads=2 * qpk,
                       n_tokens=1000, key_bits=bits[0], value_bits=bits[1])
    n = 1000
    cache, k, v = run_prefill(cfg, n, max_tokens=1024)
    gp = gpu_planes(cache)
    op = oracle_planes(cfg, k, v, 1024)
    assert_planes_equal(gp, op, n)
    _attend_both(cfg, cache, op, gp, n)


@pytest.mark.parametrize("bits", [(2, 2), (4, 4), (8, 8)])
@pytest.mark.parametrize("qpk", [2, 4])
def test_d64_gqa(bits, qpk):
    cfg = synth.scaled(TINY, kv_heads=2, q_heads=2 * qpk, key_bits=bits[0], value_bits=bits[1])
    n = 300
    cache, k, v = run_prefill(cfg, n, max_tokens=320)
    gp = gpu_planes(cache)
    op = oracle_planes(cfg, k, v, 320)
    assert_planes_equal(gp, op, n)
    _attend_both(cfg, cache, op, gp, n)


@pytest.mark.parametrize("bits, qpk", [((2, 2), 1), ((4, 4), 1), ((4, 2), 1), ((2, 2), 4)])
@pytest.mark.parametrize("direction", ["rising", "falling"])
def test_scores_monotone_in_position(bits, qpk, direction):
    """Scores that rise along the sequence (nearly every step raises the
    running maximum and rescales the accumulators) or fall (only the first
    step does).  The keys' energy sits in the last channel, which either
    rotary pairing turns at the lowest frequency (under 0.12 rad over 1000
    tokens), so q.k follows the key's magnitude there.  The shape runs 31
    token splits, merged in chunks of 8: rising scores put the maximum in
    the last chunk, so the sums of the earlier chunks are rescaled."""
    cfg = synth.scaled(synth.CONFIGS["llama2_7b"], batch=2, kv_heads=2, q_heads=2 * qpk,
                       n_tokens=1000, key_bits=bits[0], value_bits=bits[1])
    n, D = 1000, cfg.head_dim
    k = synth.make_keys(cfg, 3, 0, n).astype(np.float32) * 0.01
    ramp = 0.02 * np.arange(n, dtype=np.float32)
    k[..., D - 1] += ramp if direction == "rising" else ramp[::-1]
    k = np.ascontiguousarray(k.astype(cfg.np_dtype))
    v = synth.make_values(cfg, 3, 0, n)
    cache = make_cache(cfg, 1024)
    cache.prefill(to_gpu(k), to_gpu(v))
    gp = gpu_planes(cache)
    op = oracle_planes(cfg, k, v, 1024)
    assert_planes_equal(gp, op, n)
    q = synth.make_query(cfg, 3).astype(np.float32) * 0.01
    q[..., D - 1] = 4.0
    q = np.ascontiguousarray(q.astype(cfg.np_dtype))
    out = cache.attend(to_gpu(q)).cpu().numpy()
    for planes in (op, gp):
        ref = oracle.attend(planes, q, n, cfg.key_bits, cfg.value_bits, cfg.kv_heads)
        assert_attention_close(out, ref)


def test_append_through_tail_and_flushes():
    """Prefill 250 tokens, append 40 one at a time (flushes at n = 256 and
    288); planes equal the oracle's one-shot quantization of all tokens and
    attention is checked at several steps."""
    cfg = synth.scaled(synth.CONFIGS["llama2_7b"], batch=2, kv_heads=3, q_heads=3,
                       n_tokens=290)
    n0, n1 = 250, 290
    k = synth.make_keys(cfg, 0, 0, n1)
    v = synth.make_values(cfg, 0, 0, n1)
    cache = make_cache(cfg, 320)
    cache.prefill(to_gpu(k[:, :, :n0]), to_gpu(v[:, :, :n0]))
    kg, vg = to_gpu(k), to_gpu(v)
    for t in range(n0, n1):
        cache.append(kg[:, :, t].contiguous(), vg[:, :, t].contiguous())
        n = t + 1
        assert len(cache) == n
        if n in (251, 255, 256, 257, 287, 288, 289, 290):
            gp = gpu_planes(cache)
            op = oracle_planes(cfg, k[:, :, :n], v[:, :, :n], 320)
            assert_planes_equal(gp, op, n)
            _attend_both(cfg, cache, op, gp, n, step=n)


def test_append_from_empty():
    cfg = synth.scaled(TINY, batch=2, q_heads=2, kv_heads=2, n_tokens=40)
    k = synth.make_keys(cfg, 0, 0, 40)
    v = synth.make_values(cfg, 0, 0, 40)
    cache = make_cache(cfg, 40)
    cache.prefill(to_gpu(k[:, :, :0]), to_gpu(v[:, :, :0]))
    assert len(cache) == 0
    kg, vg = to_gpu(k), to_gpu(v)
    for t in range(40):
        cache.append(kg[:, :, t].contiguous(), vg[:, :, t].contiguous())
    gp = gpu_planes(cache)
    op = oracle_planes(cfg, k, v, 40)
    assert_planes_equal(gp, op, 40)
    _attend_both(cfg, cache, op, gp, 40)


def test_state_and_capacity_errors_leave_state_unchanged():
    from quantized_decode_attention_keys_amd import KVQ_ERR_CAPACITY, KVQ_ERR_STATE, KvqError
    cfg = synth.scaled(TINY, n_tokens=64)
    cache = make_cache(cfg, 64)
    q = to_gpu(synth.make_query(cfg))
    with pytest.raises(KvqError) as e:
        cache.attend(q)
    assert e.value.status == KVQ_ERR_STATE
    k = to_gpu(synth.make_keys(cfg, 0, 0, 65))
    v = to_gpu(synth.make_values(cfg, 0, 0, 65))
    with pytest.raises(KvqError) as e:
        cache.prefill(k, v)
    assert e.value.status == KVQ_ERR_CAPACITY and len(cache) == 0
    cache.prefill(k[:, :, :64].contiguous(), v[:, :, :64].contiguous())
    with pytest.raises(KvqError) as e:
        cache.prefill(k[:, :, :4].contiguous(), v[:, :, :4].contiguous())
    assert e.value.status == KVQ_ERR_STATE and len(cache) == 64
    with pytest.raises(KvqError) as e:
        cache.append(k[:, :, 64].contiguous(), v[:, :, 64].contiguous())
    assert e.value.status == KVQ_ERR_CAPACITY and len(cache) == 64
    torch.cuda.synchronize()


def test_llama2_7b_full_size():
    """The bench workload at full size (batch 8, 32 heads, 4096 tokens, B=2)
    in the bench's launch configuration (the last token appended and
    attended in one launch): every plane of all 8 sequences bit-exact, and
    attention for all 256 (sequence, head) rows."""
    cfg = synth.CONFIGS["llama2_7b"]
    n = cfg.n_tokens
    cache, k, v = run_prefill(cfg, n - 1, max_tokens=n + 64)
    del k, v
    kg = to_gpu(synth.make_keys(cfg, 0, n - 1, n)[:, :, 0])
    vg = to_gpu(synth.make_values(cfg, 0, n - 1, n)[:, :, 0])
    q = synth.make_query(cfg, 0, 0)
    out = cache.append_attend(kg, vg, to_gpu(q)).cpu().numpy()
    gp = gpu_planes(cache)
    for b in range(cfg.batch):
        kb = synth.make_keys(cfg, 0, 0, n, seqs=[b])
        vb = synth.make_values(cfg, 0, 0, n, seqs=[b])
        op = oracle_planes(synth.scaled(cfg, batch=1), kb, vb, n + 64)
        assert_planes_equal(gp, op, n, seqs=[b])
        ref = oracle.attend(op, q[b:b + 1], n, cfg.key_bits, cfg.value_bits, cfg.kv_heads)
        assert_attention_close(out[b:b + 1], ref)
