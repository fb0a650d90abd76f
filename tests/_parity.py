"""Helpers for the GPU parity tests: run the HIP path through the C ABI on
seeded synthetic inputs and compare it with the oracle on the same bytes."""
import numpy as np
import torch

import oracle
import synth
from quantized_decode_attention_keys_amd import QuantizedKVCache

TOL = 2e-3  # attention: max|out - ref| <= TOL * max|ref| over the output tensor
G = 32

_TORCH = {np.dtype(np.float16): torch.float16, np.dtype(np.float32): torch.float32}


def dev():
    return torch.device("cuda", 0)


def to_gpu(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev())


def make_cache(cfg, max_tokens, residual=0, sink=0, geometry=0):
    return QuantizedKVCache(cfg.batch, cfg.q_heads, cfg.kv_heads, cfg.head_dim, max_tokens,
                            cfg.key_bits, cfg.value_bits, _TORCH[cfg.np_dtype],
                            rope_base=cfg.rope_base, device=dev(), residual=residual, sink=sink,
                            geometry=geometry)


def gpu_planes(cache):
    torch.cuda.synchronize()
    out = {}
    for k, t in cache.planes().items():
        a = t.cpu().numpy()
        out[k] = a.view(np.uint32) if a.dtype == np.int32 else a
    return out


def oracle_planes(cfg, k, v, max_tokens, residual=0, sink=0):
    kp = oracle.quantize_keys(k, cfg.key_bits, cfg.group, max_tokens=max_tokens,
                              residual=residual, sink=sink)
    vals = oracle.quantize_values(v, cfg.value_bits, cfg.group, max_tokens=max_tokens,
                                  residual=residual, sink=sink)
    pl = dict(k_codes=kp[0], k_meta=kp[1], k_tail=kp[2], v_codes=vals[0], v_meta=vals[1])
    if residual > 0:
        pl["v_tail"] = vals[2]
    if sink > 0:
        pl["k_sink"], pl["v_sink"] = kp[3], vals[-1]
    return pl


def assert_planes_equal(gp, op, n, G=32, seqs=None, residual=0, sink=0):
    """Bit-exact comparison of every slot that holds data at length n: codes
    and metadata of the quantized tokens, ring and sink slots of the others."""
    tq = oracle.quantized_tokens(n, G, residual, sink)
    vq = tq if residual > 0 else n
    ns = min(n, sink)
    ring = residual + G
    # seqs selects GPU sequences; op holds the oracle planes of just those
    sel = slice(None) if seqs is None else list(seqs)
    g = {k: a[sel] for k, a in gp.items()}
    o = op
    for name, lo, hi in (("k_codes", sink // G, tq // G), ("k_meta", sink // G, tq // G),
                         ("v_codes", ns, vq), ("v_meta", ns, vq)):
        a, b = g[name][:, :, lo:hi], o[name][:, :, lo:hi]
        if not np.array_equal(a, b):
            bad = np.argwhere(a != b)
            raise AssertionError(f"{name}: {len(bad)} mismatches, first at {bad[0].tolist()}: "
                                 f"gpu {a[tuple(bad[0])]:#x} oracle {b[tuple(bad[0])]:#x}")
    slots = [t % ring for t in range(tq, n)]
    tails = ("k_tail", "v_tail") if residual > 0 else ("k_tail",)
    for name in tails:
        at, bt = g[name][:, :, slots], o[name][:, :, slots]
        assert np.array_equal(at.view(np.uint8), bt.view(np.uint8)), f"{name} differs"
    for name in (("k_sink", "v_sink") if sink > 0 else ()):
        at, bt = g[name][:, :, :ns], o[name][:, :, :ns]
        assert np.array_equal(at.view(np.uint8), bt.view(np.uint8)), f"{name} differs"


def assert_geometry_planes_equal(gp, op, n, geom, seqs=None):
    sel = slice(None) if seqs is None else list(seqs)
    tq = n // G * G
    for op_name, per_token in (("k", bool(geom & 1)), ("v", not geom & 2)):
        for part in ("codes", "meta"):
            name = f"{op_name}_{part}"
            hi = n if per_token else tq // G
            a, b = gp[name][sel][:, :, :hi], op[name][:, :, :hi]
            if not np.array_equal(a, b):
                bad = np.argwhere(a != b)
                raise AssertionError(f"geometry {geom} {name}: {len(bad)} mismatches, first "
                                     f"at {bad[0].tolist()}")
        if not per_token:
            slots = [t % G for t in range(tq, n)]
            a = gp[f"{op_name}_tail"][sel][:, :, slots]
            b = op[f"{op_name}_tail"][:, :, slots]
            assert np.array_equal(a.view(np.uint8), b.view(np.uint8)), f"{op_name}_tail"


def assert_attention_close(out, ref, tol=TOL):
    err = np.abs(out - ref).max()
    scale = np.abs(ref).max()
    assert err <= tol * scale, f"attention max err {err:.3e} > {tol} * {scale:.3e}"
    return err / scale


def run_prefill(cfg, n, max_tokens=None, seed=0):
    """Prefill n tokens on the GPU; return (cache, k, v) with host inputs."""
    max_tokens = max(n, 1) if max_tokens is None else max_tokens
    k = synth.make_keys(cfg, seed, 0, n)
    v = synth.make_values(cfg, seed, 0, n)
    cache = make_cache(cfg, max_tokens)
    cache.prefill(to_gpu(k), to_gpu(v))
    return cache, k, v
