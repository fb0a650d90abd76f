"""GPU parity of the FP8 (OCP E4M3) cache: the encoder bit-exact against the
oracle on every finite binary16 value and on fp32 draws, the hardware decode
exact on every finite code (one-token attention returns the decoded value),
planes of prefill and appends bit-exact, attention within 2e-3 of max|out|."""
import numpy as np
import pytest
import torch

import oracle
import synth
from fp8_layout import to_logical
from _parity import TOL, _TORCH, assert_attention_close, dev, to_gpu
from quantized_decode_attention_keys_amd import (KVQ_FORMAT_FP8_E4M3, KvqError,
                                                 QuantizedKVCache)

pytestmark = pytest.mark.gpu

G = 32


def make_cache(cfg, cap):
    return QuantizedKVCache(cfg.batch, cfg.q_heads, cfg.kv_heads, cfg.head_dim, cap, 8, 8,
                            _TORCH[cfg.np_dtype], rope_base=cfg.rope_base, device=dev(),
                            format=KVQ_FORMAT_FP8_E4M3)


def planes(cache):
    """The cache's FP8 planes in the oracle's [group][channel][token] order."""
    torch.cuda.synchronize()
    return {k: to_logical(t.cpu().numpy()) for k, t in cache.planes().items()}


def assert_bytes_equal(gp, k, v, n, cap, seqs=None):
    """Rows of every group that holds tokens: token bytes and the zero bytes
    past n in the last group."""
    sel = slice(None) if seqs is None else list(seqs)
    ng = -(-n // G)
    for name, x in (("k_fp8", k), ("v_fp8", v)):
        want = oracle.quantize_fp8(x[:, :, :n], G, max_tokens=cap)[:, :, :ng]
        got = gp[name][sel][:, :, :ng]
        if not np.array_equal(got, want):
            bad = np.argwhere(got != want)
            raise AssertionError(f"{name}: {len(bad)} mismatches, first at {bad[0].tolist()}")


def check(cfg, cache, k, v, n, cap, q_step=0):
    gp = planes(cache)
    assert_bytes_equal(gp, k, v, n, cap)
    q = synth.make_query(cfg, 0, q_step)
    out = cache.attend(to_gpu(q)).cpu().numpy()
    for src in ((oracle.quantize_fp8(k[:, :, :n], G, max_tokens=cap),
                 oracle.quantize_fp8(v[:, :, :n], G, max_tokens=cap)),
                (gp["k_fp8"], gp["v_fp8"])):
        ref = oracle.attend_fp8(src[0], src[1], q, n, cfg.kv_heads)
        assert_attention_close(out, ref)


def test_encoder_every_binary16():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    x = bits.view(np.float16)
    x = x[np.isfinite(x)]                      # 63488 = 496 * 128 values
    k = x.reshape(1, 1, 496, 128)
    v = np.ascontiguousarray(k[:, :, ::-1])
    cfg = synth.scaled(synth.CONFIGS["llama2_7b"], batch=1, q_heads=1, kv_heads=1,
                       n_tokens=496)
    cache = make_cache(cfg, 512)
    cache.prefill(to_gpu(k), to_gpu(v))
    assert_bytes_equal(planes(cache), k, v, 496, 512)


def test_encoder_fp32_draws():
    rng = np.random.default_rng(0)
    cfg = synth.scaled(synth.CONFIGS["tiny"], kv_heads=2, q_heads=2)
    scale = np.array([1e-3, 0.05, 1.0, 30.0, 300.0, 1e4])[rng.integers(0, 6, (1, 2, 300, 64))]
    k = (rng.standard_normal((1, 2, 300, 64)) * scale).astype(np.float32)
    v = (rng.standard_normal((1, 2, 300, 64)) * scale[:, ::-1]).astype(np.float32)
    cache = make_cache(cfg, 320)
    cache.prefill(to_gpu(k), to_gpu(v))
    assert_bytes_equal(planes(cache), k, v, 300, 320)


def test_hardware_decode_every_code():
    """One cached token: the weight is exactly 1, so the output is the
    decoded value of each stored byte; values are the 254 finite codes."""
    codes = [b for b in range(256) if b not in (0x7F, 0xFF)] + [0, 0]
    vals = np.array([oracle.fp8_decode(b) for b in codes], dtype=np.float16)  # exact
    cfg = synth.scaled(synth.CONFIGS["llama2_7b"], batch=2, q_heads=2, kv_heads=1, n_tokens=1)
    v = vals.reshape(2, 1, 1, 128)
    k = np.zeros_like(v)
    cache = make_cache(cfg, 32)
    cache.prefill(to_gpu(k), to_gpu(v))
    q = np.ones((2, 2, 128), dtype=np.float16)
    out = cache.attend(to_gpu(q)).cpu().numpy()
    want = np.repeat(vals.astype(np.float32).reshape(2, 1, 128), 2, axis=1)
    assert np.array_equal(out, want)


@pytest.mark.parametrize("n", [1, 31, 32, 33, 100, 257])
@pytest.mark.parametrize("qpk", [1, 4, 8])
def test_prefill_d128(n, qpk):
    cfg = synth.scaled(synth.CONFIGS["llama2_7b"], batch=2, kv_heads=2, q_heads=2 * qpk,
                       key_bits=8, value_bits=8, n_tokens=n)
    cap = 288
    k, v = synth.make_keys(cfg, 0, 0, n), synth.make_values(cfg, 0, 0, n)
    cache = make_cache(cfg, cap)
    cache.prefill(to_gpu(k), to_gpu(v))
    check(cfg, cache, k, v, n, cap)


@pytest.mark.parametrize("dtype", ["float16", "float32"])
@pytest.mark.parametrize("n", [40, 200])
def test_prefill_d64(dtype, n):
    cfg = synth.scaled(synth.CONFIGS["tiny"], kv_heads=2, q_heads=4, key_bits=8, value_bits=8,
                       dtype=dtype)
    k, v = synth.make_keys(cfg, 0, 0, n), synth.make_values(cfg, 0, 0, n)
    cache = make_cache(cfg, 224)
    cache.prefill(to_gpu(k), to_gpu(v))
    check(cfg, cache, k, v, n, 224)


@pytest.mark.parametrize("n0", [0, 20])
def test_append_through_groups(n0):
    """From an empty cache or a 20-token prompt, append up to 150 tokens:
    bytes are written as tokens arrive, opened groups are cleared."""
    cfg = synth.scaled(synth.CONFIGS["llama2_7b"], batch=2, kv_heads=2, q_heads=4,
                       key_bits=8, value_bits=8, n_tokens=150)
    n1, cap = 150, 160
    k, v = synth.make_keys(cfg, 2, 0, n1), synth.make_values(cfg, 2, 0, n1)
    cache = make_cache(cfg, cap)
    if n0:
        cache.prefill(to_gpu(k[:, :, :n0]), to_gpu(v[:, :, :n0]))
    kd, vd = to_gpu(k), to_gpu(v)
    for t in range(n0, n1):
        cache.append(kd[:, :, t].contiguous(), vd[:, :, t].contiguous())
        if t + 1 in (1, 32, 33, 97, 150):
            check(cfg, cache, k, v, t + 1, cap, q_step=t)


def test_full_7b_shape():
    """FP8 keys and values at the Llama-2-7B decode shape (batch 8, 32 heads,
    4095-token prompt + 1 append), in the launch configuration the bench
    times: bytes of sequences 1 and 7 bit-exact, attention of all their
    heads within tolerance."""
    cfg = synth.scaled(synth.CONFIGS["llama2_7b"], key_bits=8, value_bits=8)
    n, cap = 4096, 4128
    k = synth.make_keys(cfg, 0, 0, n)
    v = synth.make_values(cfg, 0, 0, n)
    cache = make_cache(cfg, cap)
    cache.prefill(to_gpu(k[:, :, :n - 1]), to_gpu(v[:, :, :n - 1]))
    cache.append(to_gpu(k[:, :, n - 1]), to_gpu(v[:, :, n - 1]))
    q = synth.make_query(cfg, 0, 0)
    out = cache.attend(to_gpu(q)).cpu().numpy()
    seqs = [1, 7]
    assert_bytes_equal(planes(cache), k[seqs], v[seqs], n, cap, seqs=seqs)
    k8 = oracle.quantize_fp8(k[seqs], G, max_tokens=cap)
    v8 = oracle.quantize_fp8(v[seqs], G, max_tokens=cap)
    ref = oracle.attend_fp8(k8, v8, q[seqs], n, cfg.kv_heads)
    assert_attention_close(out[seqs], ref, TOL)


def test_metrics_not_taken():
    cfg = synth.scaled(synth.CONFIGS["tiny"], kv_heads=2, q_heads=2, key_bits=8, value_bits=8)
    cache = make_cache(cfg, 64)
    k = torch.zeros((1, 2, 8, 64), device=dev())
    cache.prefill(k, k)
    with pytest.raises(KvqError):
        cache.error_metrics(k, k, torch.zeros((1, 2, 64), device=dev()))
