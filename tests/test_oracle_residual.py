"""Pins for the oracle's residual window (KIVI keeps the most recent tokens
in full precision: "Your KV Cache Doesn't Have a Bit Problem...", section
"The Systems Tax, and Why It Is Not a Detail").

Reading: with a window R (a multiple of G), keys and values of tokens
[Tq, n) stay unquantized, Tq = G * floor(max(0, n - R) / G); the rest is the
R = 0 cache of the first Tq tokens.  The unquantized tokens live in rings of
R + G slots (token t in slot t mod (R + G)).

Each check is against something other than the oracle's own window code: the
R = 0 planes of a truncated prompt, the input tensors themselves, and the
plain dense attention formula on numpy-assembled tensors."""
import numpy as np
import pytest

D = 64
G = 32


def _tq(n, R):
    return max(0, n - R) // G * G


@pytest.mark.parametrize("n,R", [(10, 32), (32, 32), (63, 32), (64, 32), (65, 32), (95, 32),
                                 (96, 32), (200, 64), (130, 128), (300, 128)])
def test_split_point_and_rings(orc, n, R):
    rng = np.random.default_rng(n + R)
    nb, h = 2, 3
    k = rng.standard_normal((nb, h, n, D)).astype(np.float16)
    v = rng.standard_normal((nb, h, n, D)).astype(np.float16)
    tq = _tq(n, R)
    assert orc.quantized_tokens(n, G, R) == tq
    # at least R (at most R + G - 1) recent tokens stay in full precision
    assert min(n, R) <= n - tq <= R + G - 1
    cap = 320
    kc, km, kt = orc.quantize_keys(k, 2, G, max_tokens=cap, residual=R)
    vc, vm, vt = orc.quantize_values(v, 4, G, max_tokens=cap, residual=R)
    ring = R + G
    assert kt.shape[2] == ring and vt.shape[2] == ring
    # the quantized region is the R = 0 cache of the first tq tokens
    kc0, km0, _ = orc.quantize_keys(k[:, :, :tq], 2, G, max_tokens=cap)
    vc0, vm0 = orc.quantize_values(v[:, :, :tq], 4, G, max_tokens=cap)
    assert np.array_equal(kc, kc0) and np.array_equal(km, km0)
    assert np.array_equal(vc, vc0) and np.array_equal(vm, vm0)
    # rings hold the remaining tokens verbatim, token t in slot t mod ring
    for t in range(tq, n):
        assert np.array_equal(kt[:, :, t % ring], k[:, :, t])
        assert np.array_equal(vt[:, :, t % ring], v[:, :, t])


def test_zero_window_is_the_plain_cache(orc):
    rng = np.random.default_rng(5)
    k = rng.standard_normal((1, 2, 70, D)).astype(np.float16)
    v = rng.standard_normal((1, 2, 70, D)).astype(np.float16)
    a = orc.quantize_keys(k, 2, G, max_tokens=96)
    b = orc.quantize_keys(k, 2, G, max_tokens=96, residual=0)
    assert all(np.array_equal(x, y) for x, y in zip(a, b))
    assert len(orc.quantize_values(v, 2, G, max_tokens=96, residual=0)) == 2


@pytest.mark.parametrize("n", [1, 31, 64])
def test_window_covering_everything_is_full_precision_attention(orc, n):
    """R >= n: nothing is quantized, so the result is plain attention on the
    inputs (the dense formula, a separate code path)."""
    rng = np.random.default_rng(n)
    nb, hkv, hq, R = 2, 2, 4, 64
    k = rng.standard_normal((nb, hkv, n, D)).astype(np.float32)
    k[..., 5] *= 30
    v = rng.standard_normal((nb, hkv, n, D)).astype(np.float32)
    q = rng.standard_normal((nb, hq, D)).astype(np.float32)
    kc, km, kt = orc.quantize_keys(k, 2, G, max_tokens=96, residual=R)
    vc, vm, vt = orc.quantize_values(v, 2, G, max_tokens=96, residual=R)
    pl = dict(k_codes=kc, k_meta=km, k_tail=kt, v_codes=vc, v_meta=vm, v_tail=vt)
    out = orc.attend(pl, q, n, 2, 2, hkv=hkv, residual=R)
    dense = orc.attend_dense(k, v, q)
    assert np.allclose(out, dense, rtol=0, atol=1e-12)


def _dequant(words, meta, n, bits):
    import oracle
    c = oracle.unpack(words, n, bits).astype(np.float64)
    s = np.uint16(meta & 0xFFFF).view(np.float16).astype(np.float64)
    z = np.uint16(meta >> 16).view(np.float16).astype(np.float64)
    return z + s * c


@pytest.mark.parametrize("n,R", [(95, 32), (96, 32), (200, 64), (300, 128)])
def test_mixed_cache_equals_dense_on_assembled_tensors(orc, n, R):
    """Quantized tokens below Tq, raw tokens above: the window read equals
    the dense formula on tensors assembled with numpy (dequantized prefix
    from the planes, the raw recent tokens from the inputs)."""
    rng = np.random.default_rng(n * 7 + R)
    nb, hkv, hq, kb, vb = 1, 2, 4, 2, 4
    k = rng.standard_normal((nb, hkv, n, D)).astype(np.float16)
    k[..., 3] *= 50
    v = rng.standard_normal((nb, hkv, n, D)).astype(np.float16)
    q = rng.standard_normal((nb, hq, D)).astype(np.float16)
    tq = _tq(n, R)
    kc, km, kt = orc.quantize_keys(k, kb, G, max_tokens=320, residual=R)
    vc, vm, vt = orc.quantize_values(v, vb, G, max_tokens=320, residual=R)
    pl = dict(k_codes=kc, k_meta=km, k_tail=kt, v_codes=vc, v_meta=vm, v_tail=vt)
    out = orc.attend(pl, q, n, kb, vb, hkv=hkv, residual=R)
    kh = k.astype(np.float64)
    vh = v.astype(np.float64)
    for b in range(nb):
        for hh in range(hkv):
            for g in range(tq // G):
                for c in range(D):
                    kh[b, hh, g * G:(g + 1) * G, c] = _dequant(kc[b, hh, g, c], km[b, hh, g, c],
                                                               G, kb)
            for t in range(tq):
                for cg in range(D // G):
                    vh[b, hh, t, cg * G:(cg + 1) * G] = _dequant(vc[b, hh, t, cg],
                                                                 vm[b, hh, t, cg], G, vb)
    assert np.array_equal(kh.astype(np.float32).astype(np.float64), kh)
    assert np.array_equal(vh.astype(np.float32).astype(np.float64), vh)
    dense = orc.attend_dense(kh.astype(np.float32), vh.astype(np.float32),
                             q.astype(np.float32))
    assert np.allclose(out, dense, rtol=0, atol=1e-12)
    # the window changes the result: the R = 0 cache of the same tokens differs
    kc0, km0, kt0 = orc.quantize_keys(k, kb, G, max_tokens=320)
    vc0, vm0 = orc.quantize_values(v, vb, G, max_tokens=320)
    pl0 = dict(k_codes=kc0, k_meta=km0, k_tail=kt0, v_codes=vc0, v_meta=vm0)
    assert not np.allclose(orc.attend(pl0, q, n, kb, vb, hkv=hkv), out, rtol=0, atol=1e-9)


def test_window_moves_error_towards_full_precision(orc):
    """With more recent tokens in full precision the output error against
    unquantized attention cannot grow on average (here: it shrinks)."""
    rng = np.random.default_rng(11)
    nb, hkv, n = 2, 4, 256
    k = rng.standard_normal((nb, hkv, n, D)).astype(np.float32)
    k[..., 7] *= 40
    v = rng.standard_normal((nb, hkv, n, D)).astype(np.float32)
    q = rng.standard_normal((nb, hkv, D)).astype(np.float32) * 2
    ref = orc.attend_dense(k, v, q)
    errs = []
    for R in (0, 64, 128, 192):
        kc, km, kt = orc.quantize_keys(k, 2, G, max_tokens=n, residual=R)
        vals = orc.quantize_values(v, 2, G, max_tokens=n, residual=R)
        pl = dict(k_codes=kc, k_meta=km, k_tail=kt, v_codes=vals[0], v_meta=vals[1])
        if R > 0:
            pl["v_tail"] = vals[2]
        out = orc.attend(pl, q, n, 2, 2, hkv=hkv, residual=R)
        errs.append(np.abs(out - ref).mean())
    assert all(a > b for a, b in zip(errs, errs[1:])), errs
