"""The bench's algorithmic byte counts against a hand count of what the
method moves per decode step (CPU only).

Per step and (sequence, KV head): B_k/8 bytes of key codes per quantized key
element plus one 4-byte (step, zero) word per channel of each 32-token key
group; B_v/8 bytes of value codes per quantized value element plus one
4-byte word per 32-channel value group of each token; the unfilled key tail
at full precision; and per query head q in (binary16 or fp32) and the fp32
output.  The figures below are written out from those rules with the
workloads' sizes, independently of bench.py's formula."""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import synth  # noqa: E402


def hand(nb, hkv, hq, D, n, kb, vb, esz=2):
    tq = n // 32 * 32
    per_head = (tq * D * kb // 8            # key codes
                + (tq // 32) * D * 4        # key (step, zero) words
                + (n - tq) * D * esz        # key tail
                + n * D * vb // 8           # value codes
                + n * (D // 32) * 4)        # value (step, zero) words
    return nb * hkv * per_head + nb * hq * D * (esz + 4)


@pytest.mark.parametrize("name, expected", [
    ("llama2_7b", 100_859_904),
    ("llama2_13b", 503_808_000),
    ("llama2_13b_b4", 839_352_320),
    ("long", 536_895_488),
    ("gqa", 806_879_232),
])
def test_attend_bytes_match_the_hand_count(name, expected):
    cfg = synth.CONFIGS[name]
    n = cfg.n_tokens
    assert hand(cfg.batch, cfg.kv_heads, cfg.q_heads, cfg.head_dim, n, cfg.key_bits,
                cfg.value_bits) == expected
    assert bench.attend_bytes(cfg, n) == expected


@pytest.mark.parametrize("n", [4097, 4127, 4128, 4100])
def test_attend_bytes_with_a_key_tail(n):
    cfg = synth.CONFIGS["llama2_7b"]
    assert bench.attend_bytes(cfg, n) == hand(8, 32, 32, 128, n, 2, 2)


def test_gqa_prefill_bytes():
    # 4 GiB of fp16 keys and values read; codes and metadata written
    cfg = synth.CONFIGS["gqa"]
    n = cfg.n_tokens
    read = 2 * 64 * 8 * n * 128 * 2
    written = 64 * 8 * (n * 128 * 2 // 8 + (n // 32) * 128 * 4 + n * 128 * 2 // 8 + n * 4 * 4)
    assert read == 4_294_967_296 and written == 805_306_368
    assert bench.prefill_bytes(cfg, n) == read + written


def test_windows_count_their_full_precision_rows():
    # residual window R = 128 at n = 4100: tokens [3968, 4100) stay fp16 for
    # keys and values; quantized region [0, 3968)
    cfg = synth.CONFIGS["llama2_7b"]
    n, R = 4100, 128
    tq = 3968
    per_head = (tq * 128 * 2 // 8 + (tq // 32) * 128 * 4 + (n - tq) * 128 * 2
                + tq * 128 * 2 // 8 + tq * 4 * 4 + (n - tq) * 128 * 2)
    assert bench.attend_bytes(cfg, n, residual=R) == 8 * 32 * per_head + 8 * 32 * 128 * 6


def test_fp8_bytes():
    cfg = synth.CONFIGS["llama2_7b"]
    assert bench.fp8_bytes(cfg, 4096) == 2 * 8 * 32 * 4096 * 128 + 8 * 32 * 128 * 6
