"""Pins for the oracle's sink window (InnerQ keeps high-precision windows
for the recent tokens and for the attention-sink tokens: "Your KV Cache
Doesn't Have a Bit Problem...", section "Where the Work Is Headed").

Reading: with a sink S (a multiple of G), keys and values of tokens
[0, min(n, S)) stay unquantized for good; quantization starts at token S, so
key groups keep their alignment to token 0; Tq = max(min(n, S),
G * floor(max(0, n - R) / G)), and the tail ring holds [Tq, n) as before.

Checked against the inputs, the plain (S = 0) planes of the same prompt and
the dense attention formula on numpy-assembled tensors."""
import numpy as np
import pytest

D = 64
G = 32


def _tq(n, R, S):
    q = max(0, n - R) // G * G
    return max(min(n, S), q)


@pytest.mark.parametrize("n,R,S", [(10, 0, 32), (40, 0, 32), (100, 0, 64), (100, 64, 64),
                                   (200, 32, 64), (300, 128, 32), (64, 0, 64)])
def test_segments_and_planes(orc, n, R, S):
    rng = np.random.default_rng(n + R + S)
    nb, h, cap = 2, 2, 320
    k = rng.standard_normal((nb, h, n, D)).astype(np.float16)
    v = rng.standard_normal((nb, h, n, D)).astype(np.float16)
    tq = _tq(n, R, S)
    assert orc.quantized_tokens(n, G, R, S) == tq
    kc, km, kt, ks = orc.quantize_keys(k, 2, G, max_tokens=cap, residual=R, sink=S)
    vals = orc.quantize_values(v, 4, G, max_tokens=cap, residual=R, sink=S)
    vc, vm, vs = vals[0], vals[1], vals[-1]
    ns = min(n, S)
    assert np.array_equal(ks[:, :, :ns], k[:, :, :ns])
    assert np.array_equal(vs[:, :, :ns], v[:, :, :ns])
    # quantized region: the same groups / tokens as the plain cache of the prompt
    kc0, km0, _ = orc.quantize_keys(k, 2, G, max_tokens=cap)
    vc0, vm0 = orc.quantize_values(v, 4, G, max_tokens=cap)
    g0, g1 = S // G, tq // G
    assert np.array_equal(kc[:, :, g0:g1], kc0[:, :, g0:g1])
    assert np.array_equal(km[:, :, g0:g1], km0[:, :, g0:g1])
    assert not kc[:, :, :g0].any() and not km[:, :, :g0].any()
    vq = tq if R > 0 else n
    assert np.array_equal(vc[:, :, S:vq], vc0[:, :, S:vq])
    assert np.array_equal(vm[:, :, S:vq], vm0[:, :, S:vq])
    assert not vm[:, :, :min(S, vq)].any()
    ring = R + G
    for t in range(max(tq, ns), n):
        assert np.array_equal(kt[:, :, t % ring], k[:, :, t])
        if R > 0:
            assert np.array_equal(vals[2][:, :, t % ring], v[:, :, t])


def _planes(orc, k, v, kb, vb, cap, R, S):
    kpl = orc.quantize_keys(k, kb, G, max_tokens=cap, residual=R, sink=S)
    vals = orc.quantize_values(v, vb, G, max_tokens=cap, residual=R, sink=S)
    pl = dict(k_codes=kpl[0], k_meta=kpl[1], k_tail=kpl[2], v_codes=vals[0], v_meta=vals[1])
    if S > 0:
        pl["k_sink"], pl["v_sink"] = kpl[3], vals[-1]
    if R > 0:
        pl["v_tail"] = vals[2]
    return pl


@pytest.mark.parametrize("n", [1, 20, 64])
def test_sink_covering_everything_is_full_precision_attention(orc, n):
    rng = np.random.default_rng(n)
    nb, hkv, hq, S = 2, 2, 4, 64
    k = rng.standard_normal((nb, hkv, n, D)).astype(np.float32)
    k[..., 9] *= 30
    v = rng.standard_normal((nb, hkv, n, D)).astype(np.float32)
    q = rng.standard_normal((nb, hq, D)).astype(np.float32)
    pl = _planes(orc, k, v, 2, 2, 96, 0, S)
    out = orc.attend(pl, q, n, 2, 2, hkv=hkv, sink=S)
    assert np.allclose(out, orc.attend_dense(k, v, q), rtol=0, atol=1e-12)


def _dequant(words, meta, n, bits):
    import oracle
    c = oracle.unpack(words, n, bits).astype(np.float64)
    s = np.uint16(meta & 0xFFFF).view(np.float16).astype(np.float64)
    z = np.uint16(meta >> 16).view(np.float16).astype(np.float64)
    return z + s * c


@pytest.mark.parametrize("n,R,S", [(150, 0, 32), (200, 64, 64), (300, 32, 96)])
def test_segments_equal_dense_on_assembled_tensors(orc, n, R, S):
    rng = np.random.default_rng(n * 3 + R + S)
    nb, hkv, hq, kb, vb = 1, 2, 4, 2, 4
    k = rng.standard_normal((nb, hkv, n, D)).astype(np.float16)
    k[..., 3] *= 50
    v = rng.standard_normal((nb, hkv, n, D)).astype(np.float16)
    q = rng.standard_normal((nb, hq, D)).astype(np.float16)
    pl = _planes(orc, k, v, kb, vb, 320, R, S)
    out = orc.attend(pl, q, n, kb, vb, hkv=hkv, residual=R, sink=S)
    tq = _tq(n, R, S)
    vq = tq if R > 0 else n
    kh = k.astype(np.float64)
    vh = v.astype(np.float64)
    for b in range(nb):
        for hh in range(hkv):
            for g in range(S // G, tq // G):
                for c in range(D):
                    kh[b, hh, g * G:(g + 1) * G, c] = _dequant(pl["k_codes"][b, hh, g, c],
                                                               pl["k_meta"][b, hh, g, c], G, kb)
            for t in range(S, vq):
                for cg in range(D // G):
                    vh[b, hh, t, cg * G:(cg + 1) * G] = _dequant(pl["v_codes"][b, hh, t, cg],
                                                                 pl["v_meta"][b, hh, t, cg], G, vb)
    assert np.array_equal(kh.astype(np.float32).astype(np.float64), kh)
    assert np.array_equal(vh.astype(np.float32).astype(np.float64), vh)
    dense = orc.attend_dense(kh.astype(np.float32), vh.astype(np.float32), q.astype(np.float32))
    assert np.allclose(out, dense, rtol=0, atol=1e-12)
    # the sink changes the result
    pl0 = _planes(orc, k, v, kb, vb, 320, R, 0)
    assert not np.allclose(orc.attend(pl0, q, n, kb, vb, hkv=hkv, residual=R), out,
                           rtol=0, atol=1e-9)
