"""Pins for the oracle's rotary embedding and decode attention.

Pages: keys are stored before the rotary embedding and rotated after
dequantization ("Your KV Cache Doesn't Have a Bit Problem...", section
"Rotary Embeddings Complicate the Keys"; "Why KV Cache Geometry Matters...",
section "What Data Scientists Should Do Next"); the attention output is the
softmax-weighted sum of value vectors ("...Bit Problem...", section "Values:
Where the Intuition Breaks").  Readings: neighbouring channels (2i, 2i+1)
pair up, theta_i = base^(-2i/D), query at position n-1, scale 1/sqrt(D).
Checks use textbook identities and closed forms."""
import numpy as np
import pytest

import synth

D = 64
BASE = 10000.0


def test_rope_identity_norm_and_pair_closed_form(orc):
    rng = np.random.default_rng(0)
    u = rng.standard_normal(D)
    assert np.array_equal(orc.rope(u, 0.0), u)
    for p in (1, 77, 4095, 131071):
        r = orc.rope(u, p)
        assert abs(np.linalg.norm(r) - np.linalg.norm(u)) < 1e-12 * np.linalg.norm(u)
    # One pair at a time: q'.k' = Re[Q conj(K) e^{i (p - t) theta_i}] with
    # Q = q_{2i} + i q_{2i+1}, K likewise (complex-number form of a 2-D rotation).
    q = rng.standard_normal(D)
    k = rng.standard_normal(D)
    p, t = 300, 41
    for i in (0, 1, 5, 31):
        qi = np.zeros(D); qi[2 * i:2 * i + 2] = q[2 * i:2 * i + 2]
        ki = np.zeros(D); ki[2 * i:2 * i + 2] = k[2 * i:2 * i + 2]
        got = orc.rope(qi, p) @ orc.rope(ki, t)
        th = BASE ** (-2.0 * i / D)
        Q = q[2 * i] + 1j * q[2 * i + 1]
        K = k[2 * i] + 1j * k[2 * i + 1]
        want = (Q * np.conj(K) * np.exp(1j * (p - t) * th)).real
        assert abs(got - want) < 1e-12


def test_rope_relative_position(orc):
    rng = np.random.default_rng(1)
    q, k = rng.standard_normal(D), rng.standard_normal(D)
    s0 = orc.rope(q, 100) @ orc.rope(k, 20)
    for shift in (1, 1000, 100000):
        s1 = orc.rope(q, 100 + shift) @ orc.rope(k, 20 + shift)
        assert abs(s1 - s0) < 1e-9 * (1 + abs(s0))


def _planes(orc, k, v, kb, vb, cap=None):
    kc, km, kt = orc.quantize_keys(k, kb, 32, max_tokens=cap)
    vc, vm = orc.quantize_values(v, vb, 32, max_tokens=cap)
    return dict(k_codes=kc, k_meta=km, k_tail=kt, v_codes=vc, v_meta=vm)


def _dequant(words, meta, n, bits):
    import oracle
    c = oracle.unpack(words, n, bits).astype(np.float64)
    s = np.uint16(meta & 0xFFFF).view(np.float16).astype(np.float64)
    z = np.uint16(meta >> 16).view(np.float16).astype(np.float64)
    return z + s * c


def _vhat(orc, pl, nb, h, n, vb):
    vh = np.zeros((nb, h, n, D))
    for b in range(nb):
        for hh in range(h):
            for t in range(n):
                for cg in range(D // 32):
                    vh[b, hh, t, cg * 32:(cg + 1) * 32] = _dequant(
                        pl["v_codes"][b, hh, t, cg], pl["v_meta"][b, hh, t, cg], 32, vb)
    return vh


def _khat(orc, pl, nb, h, n, kb):
    tq = n // 32 * 32
    kh = np.zeros((nb, h, n, D))
    for b in range(nb):
        for hh in range(h):
            for g in range(tq // 32):
                for c in range(D):
                    kh[b, hh, g * 32:(g + 1) * 32, c] = _dequant(
                        pl["k_codes"][b, hh, g, c], pl["k_meta"][b, hh, g, c], 32, kb)
            kh[b, hh, tq:n] = pl["k_tail"][b, hh, :n - tq].astype(np.float64)
    return kh


def test_zero_query_gives_mean_of_dequantized_values(orc):
    rng = np.random.default_rng(2)
    nb, h, n = 1, 2, 70
    k = rng.standard_normal((nb, h, n, D)).astype(np.float16)
    v = rng.standard_normal((nb, h, n, D)).astype(np.float16)
    pl = _planes(orc, k, v, 2, 2)
    q = np.zeros((nb, h, D), dtype=np.float16)
    out = orc.attend(pl, q, n, 2, 2, hkv=h)
    vh = _vhat(orc, pl, nb, h, n, 2)
    assert np.allclose(out, vh.mean(axis=2), rtol=0, atol=1e-13)


def test_single_token_and_zero_keys(orc):
    rng = np.random.default_rng(3)
    nb, h = 1, 2
    k = rng.standard_normal((nb, h, 40, D)).astype(np.float16)
    v = rng.standard_normal((nb, h, 40, D)).astype(np.float16)
    pl = _planes(orc, k, v, 4, 4)
    q = rng.standard_normal((nb, h, D)).astype(np.float16)
    out1 = orc.attend(pl, q, 1, 4, 4, hkv=h)
    vh = _vhat(orc, pl, nb, h, 1, 4)
    assert np.allclose(out1, vh[:, :, 0], rtol=0, atol=1e-14)
    # zero keys everywhere except the newest token: weights are closed-form;
    # the newest key sits at the query's own position, so it is not rotated
    # relative to the query: score = q.k / sqrt(D).
    n = 40
    k0 = np.zeros_like(k)
    k0[:, :, n - 1] = k[:, :, n - 1]
    pl0 = _planes(orc, k0, v, 4, 4)
    out = orc.attend(pl0, q, n, 4, 4, hkv=h)
    vh = _vhat(orc, pl0, nb, h, n, 4)
    for hh in range(h):
        s = float(q[0, hh].astype(np.float64) @ k[0, hh, n - 1].astype(np.float64)) / np.sqrt(D)
        w_last = np.exp(s) / (np.exp(s) + (n - 1))
        w_rest = 1.0 / (np.exp(s) + (n - 1))
        want = w_last * vh[0, hh, n - 1] + w_rest * vh[0, hh, :n - 1].sum(axis=0)
        assert np.allclose(out[0, hh], want, rtol=0, atol=1e-12)


@pytest.mark.parametrize("n", [32, 63, 64, 95])
def test_planes_attention_equals_dense_on_dequantized(orc, n):
    """Reading the planes (unpack, dequantize, tail, GQA head map) equals the
    plain attention formula applied to the dequantized tensors, computed here
    with numpy from the planes."""
    rng = np.random.default_rng(n)
    nb, hkv, hq = 2, 2, 4
    k = rng.standard_normal((nb, hkv, n, D)).astype(np.float16)
    k[..., 3] *= 50
    v = rng.standard_normal((nb, hkv, n, D)).astype(np.float16)
    pl = _planes(orc, k, v, 2, 4, cap=128)
    q = rng.standard_normal((nb, hq, D)).astype(np.float16)
    out = orc.attend(pl, q, n, 2, 4, hkv=hkv)
    kh, vh = _khat(orc, pl, nb, hkv, n, 2), _vhat(orc, pl, nb, hkv, n, 4)
    # float32 holds every dequantized value here exactly, so the dense
    # attention over float32 copies sees the same numbers.
    assert np.array_equal(kh.astype(np.float32).astype(np.float64), kh)
    assert np.array_equal(vh.astype(np.float32).astype(np.float64), vh)
    dense = orc.attend_dense(kh.astype(np.float32), vh.astype(np.float32),
                             q.astype(np.float32))
    assert np.allclose(out, dense, rtol=0, atol=1e-12)
    # and the head map: query heads 2g and 2g+1 read KV head g
    assert not np.allclose(out[:, 0], out[:, 2])


def test_converges_to_full_precision_as_bits_grow(orc):
    """Tiny workload: error against unquantized attention shrinks as B goes
    2 -> 4 -> 8, and obeys |dout| <= max|vhat - v| + (e^{2 delta} - 1) max|v|
    with delta = max_t |ds_t| <= |q'| max_t |khat_t - k_t| / sqrt(D)."""
    cfg = synth.CONFIGS["tiny"]
    k = synth.make_keys(cfg)
    v = synth.make_values(cfg)
    q = synth.make_query(cfg)
    n, h = cfg.n_tokens, cfg.kv_heads
    dense = orc.attend_dense(k, v, q)
    errs = []
    for bits in (2, 4, 8):
        pl = _planes(orc, k, v, bits, bits)
        out = orc.attend(pl, q, n, bits, bits, hkv=h)
        err = np.abs(out - dense).max()
        errs.append(err)
        kh = _khat(orc, pl, 1, h, n, bits)
        vh = _vhat(orc, pl, 1, h, n, bits)
        for hh in range(h):
            dk = np.linalg.norm(kh[0, hh] - k[0, hh].astype(np.float64), axis=1).max()
            delta = np.linalg.norm(q[0, hh].astype(np.float64)) * dk / np.sqrt(D)
            dv = np.abs(vh[0, hh] - v[0, hh]).max()
            bound = dv + (np.exp(2 * delta) - 1) * np.abs(v[0, hh]).max()
            assert np.abs(out[0, hh] - dense[0, hh]).max() <= bound + 1e-12
    assert errs[0] > errs[1] > errs[2]
    assert errs[2] < 0.05 * np.abs(dense).max()


def test_per_channel_keys_beat_per_token_keys_on_outlier_data(orc):
    """Direction of the pages' key result ("...Bit Problem...", section
    "Keys: The Outliers Live in Fixed Channels"): with fixed outlier
    channels, grouping keys per channel gives lower attention-score error
    than grouping them per token.  Per-token grouping is emulated by
    transposing the key tensor so the oracle's per-channel groups run along
    channels."""
    cfg = synth.CONFIGS["tiny"]
    k = synth.make_keys(cfg)[0, 0].astype(np.float64)       # [256][64]
    q = synth.make_query(cfg)[0, 0].astype(np.float64)
    def score_err(khat):
        return np.abs((khat - k) @ q).mean()
    pc = np.zeros_like(k)
    pt = np.zeros_like(k)
    for g in range(8):
        for c in range(D):
            codes, s, z = orc.quant_group(k[g * 32:(g + 1) * 32, c], 2)
            pc[g * 32:(g + 1) * 32, c] = _h(z) + _h(s) * codes
    for t in range(256):
        for cg in range(2):
            codes, s, z = orc.quant_group(k[t, cg * 32:(cg + 1) * 32], 2)
            pt[t, cg * 32:(cg + 1) * 32] = _h(z) + _h(s) * codes
    assert score_err(pc) < score_err(pt)
    # the mechanism the page gives: with per-token groups the ordinary
    # channels share the outliers' step and pay for it
    ordinary = [c for c in range(D) if c not in (3, 17)]
    e_pc = np.abs(pc - k)[:, ordinary].mean()
    e_pt = np.abs(pt - k)[:, ordinary].mean()
    assert e_pc < 0.25 * e_pt


def _h(bits):
    return float(np.uint16(bits).view(np.float16))
