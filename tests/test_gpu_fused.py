"""GPU parity of the one-launch decode step (kvq_append_attend): the same
planes, bit for bit, as kvq_append_token followed by kvq_attend_decode, and
attention within the oracle's tolerance, through key-group flushes and from
an empty cache.  The two forms' outputs also agree with each other to
AGREE: the one launch may use more waves, and then the tokens meet other
running maxima, so the order of fp32 additions and the binary16 rounding of
the value weights p * step (relative 2^-11) differ."""
import numpy as np
import pytest
import torch

import oracle
import synth
from _parity import (assert_attention_close, assert_planes_equal, gpu_planes, make_cache,
                     oracle_planes, to_gpu)

pytestmark = pytest.mark.gpu

TINY = synth.CONFIGS["tiny"]
L7B = synth.CONFIGS["llama2_7b"]
AGREE = 1e-3  # max|one - two| / max|two|


def _run(cfg, n0, n1, cap, residual=0, sink=0, checks=()):
    """Prefill n0 tokens into two caches, then step one with append + attend
    and the other with append_attend up to n1 tokens.  Returns the largest
    relative difference of the two outputs over all steps."""
    k = synth.make_keys(cfg, 0, 0, n1)
    v = synth.make_values(cfg, 0, 0, n1)
    two = make_cache(cfg, cap, residual=residual, sink=sink)
    one = make_cache(cfg, cap, residual=residual, sink=sink)
    for c in (two, one):
        c.prefill(to_gpu(k[:, :, :n0]), to_gpu(v[:, :, :n0]))
    kg, vg = to_gpu(k), to_gpu(v)
    worst = 0.0
    for t in range(n0, n1):
        n = t + 1
        q = synth.make_query(cfg, 0, n)
        qg = to_gpu(q)
        kt, vt = kg[:, :, t].contiguous(), vg[:, :, t].contiguous()
        two.append(kt, vt)
        a = two.attend(qg).cpu().numpy()
        b = one.append_attend(kt, vt, qg).cpu().numpy()
        assert len(one) == len(two) == n
        scale = np.abs(a).max()
        worst = max(worst, float(np.abs(a - b).max() / scale))
        if n in checks or n == n1:
            gp1, gp2 = gpu_planes(one), gpu_planes(two)
            op = oracle_planes(cfg, k[:, :, :n], v[:, :, :n], cap, residual=residual, sink=sink)
            assert_planes_equal(gp1, op, n, residual=residual, sink=sink)
            assert_planes_equal(gp2, op, n, residual=residual, sink=sink)
            ref = oracle.attend(op, q, n, cfg.key_bits, cfg.value_bits, cfg.kv_heads,
                                residual=residual, sink=sink)
            assert_attention_close(b, ref)
    for c in (two, one):
        c.close()
    return worst


@pytest.mark.parametrize("qpk", [1, 2, 4])
@pytest.mark.parametrize("bits", [(2, 2), (4, 2), (8, 4)])
def test_d128_steps_through_flushes(qpk, bits):
    cfg = synth.scaled(L7B, batch=2, kv_heads=2, q_heads=2 * qpk, n_tokens=130,
                       key_bits=bits[0], value_bits=bits[1])
    worst = _run(cfg, 60, 130, 160, checks=(63, 64, 65, 96, 128))
    assert worst <= AGREE, worst


@pytest.mark.parametrize("dtype", ["float16", "float32"])
def test_d64_from_empty(dtype):
    cfg = synth.scaled(TINY, batch=2, q_heads=4, kv_heads=4, n_tokens=70, dtype=dtype)
    worst = _run(cfg, 0, 70, 80, checks=(1, 2, 31, 32, 33, 64))
    assert worst <= AGREE, worst


def test_d128_from_short_prompt_single_wave_share():
    """Few groups: the completed group falls in a wave's first step."""
    cfg = synth.scaled(L7B, batch=1, kv_heads=4, q_heads=4, n_tokens=100)
    worst = _run(cfg, 5, 100, 128, checks=(31, 32, 33, 64, 96))
    assert worst <= AGREE, worst


def test_7b_shape_steps():
    """The bench's workload shape: the full 7B cache, 40 fused steps across
    the flush at n = 4128."""
    cfg = L7B
    n0, n1, cap = 4095, 4135, 4160
    k = synth.make_keys(cfg, 0, 0, n1)
    v = synth.make_values(cfg, 0, 0, n1)
    two = make_cache(cfg, cap)
    one = make_cache(cfg, cap)
    for c in (two, one):
        c.prefill(to_gpu(k[:, :, :n0]), to_gpu(v[:, :, :n0]))
    kg, vg = to_gpu(k), to_gpu(v)
    for t in range(n0, n1):
        q = to_gpu(synth.make_query(cfg, 0, t + 1))
        kt, vt = kg[:, :, t].contiguous(), vg[:, :, t].contiguous()
        two.append(kt, vt)
        a = two.attend(q)
        b = one.append_attend(kt, vt, q)
        rel = float((a - b).abs().max() / a.abs().max())
        assert rel <= AGREE, (t + 1, rel)
    torch.cuda.synchronize()
    g1, g2 = gpu_planes(one), gpu_planes(two)
    # the slots that hold data at n1 tokens (the rest of the workspace is
    # never written)
    for name, hi in (("k_codes", n1 // 32), ("k_meta", n1 // 32), ("v_codes", n1),
                     ("v_meta", n1)):
        assert np.array_equal(g1[name][:, :, :hi], g2[name][:, :, :hi]), name
    slots = list(range(n1 - n1 // 32 * 32))
    assert np.array_equal(g1["k_tail"][:, :, slots].view(np.uint8),
                          g2["k_tail"][:, :, slots].view(np.uint8))
    for c in (two, one):
        c.close()


@pytest.mark.parametrize("window", [(32, 0), (0, 32)])
def test_windows_take_the_two_call_path(window):
    residual, sink = window
    cfg = synth.scaled(L7B, batch=2, kv_heads=2, q_heads=2, n_tokens=110)
    worst = _run(cfg, 40, 110, 128, residual=residual, sink=sink, checks=(64, 96))
    assert worst == 0.0, worst


def test_eight_heads_per_kv_head_take_the_two_call_path():
    cfg = synth.scaled(L7B, batch=2, kv_heads=1, q_heads=8, n_tokens=80)
    worst = _run(cfg, 50, 80, 96, checks=(64,))
    assert worst == 0.0, worst


@pytest.mark.parametrize("window", [(0, 0), (32, 0)])
def test_fills_to_a_ragged_capacity(window):
    """max_tokens = 77, not a multiple of G: the cache is stepped through
    the flush at 64 to exactly max_tokens, where the last group (tokens 64
    .. 76) is still partial and its planes' slots run past the capacity.
    With a residual window the step takes the two-call path."""
    residual, sink = window
    cfg = synth.scaled(L7B, batch=2, kv_heads=2, q_heads=4, n_tokens=77)
    worst = _run(cfg, 40, 77, 77, residual=residual, sink=sink, checks=(63, 64, 65))
    assert worst <= (AGREE if residual == 0 else 0.0), worst


def test_capacity_error_leaves_state_unchanged():
    from quantized_decode_attention_keys_amd import KVQ_ERR_CAPACITY, KvqError
    cfg = synth.scaled(TINY, n_tokens=33)
    k = synth.make_keys(cfg, 0, 0, 33)
    v = synth.make_values(cfg, 0, 0, 33)
    c = make_cache(cfg, 32)
    c.prefill(to_gpu(k[:, :, :32]), to_gpu(v[:, :, :32]))
    with pytest.raises(KvqError) as e:
        c.append_attend(to_gpu(k[:, :, 32]), to_gpu(v[:, :, 32]),
                        to_gpu(synth.make_query(cfg)))
    assert e.value.status == KVQ_ERR_CAPACITY
    assert len(c) == 32
    c.close()
