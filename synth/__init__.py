"""Seeded synthetic KV-cache workloads.

This module only draws random numbers in the shapes and value distributions
of the workloads; it holds none of the quantization or attention arithmetic.
Both the GPU path (through the tests and the bench) and the oracle are fed the
identical host arrays it returns.

Distributions follow what the pages say about real key/value activations:
keys carry a few large-magnitude outlier channels that stay fixed across
tokens ("Your KV Cache Doesn't Have a Bit Problem...", section "Keys: The
Outliers Live in Fixed Channels"); values are flat, here with a small
fraction of larger tokens.  The pages' own measurements come from trained
models (Llama-2-7B/13B) that are not available here; these seeded draws stand
in for them.

The geometry ablation uses a second key recipe ("steady"): the outlier
channels keep a fixed sign and a large magnitude with a small spread across
tokens (factor * (sign + 0.25 * N(0, 1))), the page's picture of channels that
carry very large magnitudes consistently across every token.

Random access: every (sequence, 256-token block) has its own generator,
seeded by ``SeedSequence([seed, stream, sequence, block])``, and tokens are
drawn token-major, so token t of sequence b has the same value whatever range
is requested.  That lets a check regenerate one sequence of a large workload.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

BLOCK = 256
_S_KEYS, _S_VALS, _S_VOUT, _S_QUERY, _S_KOUT, _S_KSIGN = 1, 2, 3, 4, 5, 6


@dataclass(frozen=True)
class Config:
    name: str
    batch: int
    q_heads: int
    kv_heads: int
    head_dim: int
    n_tokens: int
    key_bits: int
    value_bits: int
    dtype: str                 # "float16" | "float32"
    key_recipe: str            # "tiny" | "u20_100" | "x50" | "steady"
    value_outliers: bool       # 1 % of tokens x5
    group: int = 32
    rope_base: float = 10000.0
    description: str = ""
    extra: dict = field(default_factory=dict)

    @property
    def np_dtype(self):
        return np.dtype(self.dtype)

    def kv_elems(self, n=None) -> int:
        n = self.n_tokens if n is None else n
        return self.batch * self.kv_heads * n * self.head_dim


CONFIGS = {
    "tiny": Config(
        "tiny", 1, 4, 4, 64, 256, 2, 2, "float32", "tiny", False,
        description="1 sequence, 4 heads, head_dim 64, 256 tokens, fp32; key "
                    "channels 3 and 17 of every head x50; B=2, G=32; seed 0"),
    "llama2_7b": Config(
        "llama2_7b", 8, 32, 32, 128, 4096, 2, 2, "float16", "u20_100", True,
        description="Llama-2-7B-shaped single-layer decode: batch 8, 32 heads, "
                    "head_dim 128, 4096 tokens, fp16, B=2, G=32"),
    "llama2_13b": Config(
        "llama2_13b", 16, 40, 40, 128, 8192, 2, 2, "float16", "u20_100", True,
        description="Llama-2-13B-shaped: batch 16, 40 heads, head_dim 128, "
                    "8192 tokens, fp16, B=2"),
    "llama2_13b_b4": Config(
        "llama2_13b_b4", 16, 40, 40, 128, 8192, 4, 4, "float16", "u20_100", True,
        description="Llama-2-13B-shaped at B=4"),
    "long": Config(
        "long", 1, 32, 32, 128, 131072, 4, 2, "float16", "x50", False,
        description="long context: batch 1, 32 heads, head_dim 128, 131072 "
                    "tokens, fp16, keys B=4, values B=2"),
    "ablation_7b": Config(
        "ablation_7b", 8, 32, 32, 128, 4096, 2, 2, "float16", "steady", True,
        description="geometry ablation on the Llama-2-7B shape: batch 8, 32 heads, "
                    "head_dim 128, 4096 tokens, fp16, B=2, G=32; outlier key "
                    "channels of steady sign and magnitude"),
    "gqa": Config(
        "gqa", 64, 32, 8, 128, 16384, 2, 2, "float16", "u20_100", True,
        description="Llama-3-8B-shaped GQA: batch 64, 32 query heads over 8 KV "
                    "heads, head_dim 128, 16384 tokens, fp16, B=2"),
}


def _rng(*key) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([int(k) for k in key]))


def key_outliers(cfg: Config, seed: int = 0):
    """Outlier channels and factors per KV head: (channels int[Hkv][m],
    factors float32[Hkv][m]).  Fixed for every sequence and token."""
    H, D = cfg.kv_heads, cfg.head_dim
    if cfg.key_recipe == "tiny":
        ch = np.tile(np.array([3, 17]), (H, 1))
        return ch, np.full(ch.shape, 50.0, dtype=np.float32)
    rng = _rng(seed, _S_KOUT)
    ch = np.stack([np.sort(rng.choice(D, 4, replace=False)) for _ in range(H)])
    if cfg.key_recipe == "x50":
        f = np.full(ch.shape, 50.0, dtype=np.float32)
    else:
        f = rng.uniform(20.0, 100.0, size=ch.shape).astype(np.float32)
    return ch, f


def key_outlier_signs(cfg: Config, seed: int = 0):
    """Signs (+-1, float32[Hkv][m]) of the steady outlier channels."""
    ch, _ = key_outliers(cfg, seed)
    return _rng(seed, _S_KSIGN).choice(np.array([-1.0, 1.0], dtype=np.float32), size=ch.shape)


def _block_tokens(cfg, seed, stream, b, blk):
    rng = _rng(seed, stream, b, blk)
    return rng.standard_normal((BLOCK, cfg.kv_heads, cfg.head_dim), dtype=np.float32)


def _draw(cfg, seed, stream, t0, t1, seqs):
    """float32 [len(seqs)][Hkv][t1-t0][D], token-major draws per block."""
    seqs = range(cfg.batch) if seqs is None else seqs
    seqs = list(seqs)
    out = np.empty((len(seqs), cfg.kv_heads, t1 - t0, cfg.head_dim), dtype=np.float32)
    for si, b in enumerate(seqs):
        for blk in range(t0 // BLOCK, (t1 - 1) // BLOCK + 1 if t1 > t0 else 0):
            a = _block_tokens(cfg, seed, stream, b, blk)
            lo = max(t0, blk * BLOCK)
            hi = min(t1, (blk + 1) * BLOCK)
            out[si, :, lo - t0:hi - t0, :] = a[lo - blk * BLOCK:hi - blk * BLOCK].transpose(1, 0, 2)
    return out


def make_keys(cfg: Config, seed: int = 0, t0: int = 0, t1=None, seqs=None):
    """Pre-RoPE keys for tokens [t0, t1): [len(seqs)][Hkv][t1-t0][D], cfg dtype."""
    t1 = cfg.n_tokens if t1 is None else t1
    k = _draw(cfg, seed, _S_KEYS, t0, t1, seqs)
    ch, f = key_outliers(cfg, seed)
    sg = key_outlier_signs(cfg, seed) if cfg.key_recipe == "steady" else None
    for h in range(cfg.kv_heads):
        for m in range(ch.shape[1]):
            if sg is None:
                k[:, h, :, ch[h, m]] *= f[h, m]
            else:
                k[:, h, :, ch[h, m]] = f[h, m] * (sg[h, m] + 0.25 * k[:, h, :, ch[h, m]])
    return k.astype(cfg.np_dtype)


def make_values(cfg: Config, seed: int = 0, t0: int = 0, t1=None, seqs=None):
    """Values for tokens [t0, t1).  With value outliers on, every token is
    independently (probability 0.01) scaled x5 across all heads."""
    t1 = cfg.n_tokens if t1 is None else t1
    v = _draw(cfg, seed, _S_VALS, t0, t1, seqs)
    if cfg.value_outliers:
        seq_list = list(range(cfg.batch) if seqs is None else seqs)
        for si, b in enumerate(seq_list):
            for blk in range(t0 // BLOCK, (t1 - 1) // BLOCK + 1 if t1 > t0 else 0):
                u = _rng(seed, _S_VOUT, b, blk).random(BLOCK)
                lo = max(t0, blk * BLOCK)
                hi = min(t1, (blk + 1) * BLOCK)
                sel = np.nonzero(u[lo - blk * BLOCK:hi - blk * BLOCK] < 0.01)[0]
                v[si, :, lo - t0 + sel, :] *= 5.0
    return v.astype(cfg.np_dtype)


def make_query(cfg: Config, seed: int = 0, step: int = 0, seqs=None):
    """Pre-RoPE queries [len(seqs)][Hq][D] for decode step `step`."""
    q = _rng(seed, _S_QUERY, step).standard_normal(
        (cfg.batch, cfg.q_heads, cfg.head_dim), dtype=np.float32)
    if seqs is not None:
        q = q[list(seqs)]
    return np.ascontiguousarray(q.astype(cfg.np_dtype))


def scaled(cfg: Config, **changes) -> Config:
    """A copy of cfg with some fields replaced (smaller parity cases)."""
    d = dict(cfg.__dict__)
    d.update(changes)
    return Config(**d)
