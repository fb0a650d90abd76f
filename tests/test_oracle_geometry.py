"""Pins for the oracle's geometry ablation and its error-where-consumed
metrics ("Your KV Cache Doesn't Have a Bit Problem...", lede and sections
"Keys: The Outliers Live in Fixed Channels", "Values: Where the Intuition
Breaks").

Each check stands on something other than the oracle's own geometry code:
the planes are decoded here with numpy bit operations and compared with the
quantizer's definition applied along the declared axis; attention is checked
against the dense formula on numpy-assembled tensors; the metrics against a
numpy transcription of their definitions (vectorized RoPE and softmax, not
the oracle's loops), against exact zeros where one geometry represents the
data exactly and the other does not, against the n = 1 closed form, and
against the direction the page reports on data with its structure."""
import numpy as np
import pytest

import synth

D = 64
G = 32
GEOMS = (0, 1, 2, 3)


def _decode(words, bits, n):
    """codes[..., n] from u32 words[..., W] (LSB first), numpy only."""
    w = words.astype(np.uint64)
    j = np.arange(n)
    word = w[..., (j * bits) // 32]
    return ((word >> ((j * bits) % 32).astype(np.uint64)) & ((1 << bits) - 1)).astype(np.int64)


def _meta(m):
    s = (m & 0xFFFF).astype(np.uint16).view(np.float16).astype(np.float64)
    z = (m >> 16).astype(np.uint16).view(np.float16).astype(np.float64)
    return s, z


def _dequant_token_major(codes, meta, bits, n):
    """[nb][h][tcap][D/G][W] planes -> [nb][h][n][D]."""
    c = _decode(codes[:, :, :n], bits, G)            # nb h n ncg G
    s, z = _meta(meta[:, :, :n].astype(np.uint32))   # nb h n ncg
    x = z[..., None] + s[..., None] * c
    return x.reshape(x.shape[0], x.shape[1], n, -1)


def _dequant_channel_major(codes, meta, bits, n, tail):
    """[nb][h][gcap][D][W] planes + G-slot tail -> [nb][h][n][D]."""
    ng = n // G
    nb, h = codes.shape[:2]
    out = np.zeros((nb, h, n, codes.shape[3]))
    if ng:
        c = _decode(codes[:, :, :ng], bits, G)          # nb h ng D G
        s, z = _meta(meta[:, :, :ng].astype(np.uint32))
        x = z[..., None] + s[..., None] * c              # nb h ng D G
        out[:, :, :ng * G] = x.transpose(0, 1, 2, 4, 3).reshape(nb, h, ng * G, -1)
    for t in range(ng * G, n):
        out[:, :, t] = tail[:, :, t % G].astype(np.float64)
    return out


def _stored(pl, n, kb, vb, geom):
    if geom & 1:
        kh = _dequant_token_major(pl["k_codes"], pl["k_meta"], kb, n)
    else:
        kh = _dequant_channel_major(pl["k_codes"], pl["k_meta"], kb, n, pl["k_tail"])
    if geom & 2:
        vh = _dequant_channel_major(pl["v_codes"], pl["v_meta"], vb, n, pl["v_tail"])
    else:
        vh = _dequant_token_major(pl["v_codes"], pl["v_meta"], vb, n)
    return kh, vh


def _data(n, seed, nb=1, h=2, hq=4, dtype=np.float16):
    rng = np.random.default_rng(seed)
    k = rng.standard_normal((nb, h, n, D)).astype(np.float32)
    k[..., 5] = 30 + rng.standard_normal((nb, h, n))
    v = rng.standard_normal((nb, h, n, D)).astype(np.float32)
    q = rng.standard_normal((nb, hq, D)).astype(np.float32)
    return k.astype(dtype), v.astype(dtype), q.astype(dtype)


@pytest.mark.parametrize("geom", GEOMS)
@pytest.mark.parametrize("bits", [2, 4, 8])
def test_planes_follow_the_definition_along_the_declared_axis(orc, geom, bits):
    """Zero = group minimum, step = range/(2^B-1) (each rounded to binary16),
    code = nearest level (ties to even) -- with the group running along
    tokens for per-channel operands and along channels for per-token ones.
    fp16 data keeps the numpy quotient exact enough to decide every code."""
    n = 77
    k, v, _ = _data(n, bits * 10 + geom)
    pl = orc.geometry_planes(k, v, bits, bits, geom, max_tokens=96)
    levels = (1 << bits) - 1

    def check(x, codes, meta, per_token):
        x = x.astype(np.float64)
        if per_token:     # groups: [t][cg][j] = x[t, cg*G + j]
            grp = x.reshape(x.shape[0], x.shape[1], n, D // G, G)
            c = _decode(codes[:, :, :n], bits, G)
            s, z = _meta(meta[:, :, :n].astype(np.uint32))
        else:             # groups: [g][c][j] = x[g*G + j, c]
            ng = n // G
            grp = x[:, :, :ng * G].reshape(x.shape[0], x.shape[1], ng, G, D).transpose(
                0, 1, 2, 4, 3)
            c = _decode(codes[:, :, :ng], bits, G)
            s, z = _meta(meta[:, :, :ng].astype(np.uint32))
        mn, mx = grp.min(-1), grp.max(-1)
        assert np.array_equal(z, mn.astype(np.float16).astype(np.float64))
        assert np.array_equal(s, ((mx - mn) / levels).astype(np.float16).astype(np.float64))
        with np.errstate(divide="ignore", invalid="ignore"):
            want = np.where(s[..., None] > 0,
                            np.clip(np.rint((grp - z[..., None]) / s[..., None]), 0, levels), 0)
        assert np.array_equal(c, want.astype(np.int64))

    check(k, pl["k_codes"], pl["k_meta"], per_token=bool(geom & 1))
    check(v, pl["v_codes"], pl["v_meta"], per_token=not geom & 2)
    # the unfilled group of a per-channel operand waits verbatim in its tail
    for name, x, per_ch in (("k_tail", k, not geom & 1), ("v_tail", v, bool(geom & 2))):
        if per_ch:
            for t in range(n // G * G, n):
                assert np.array_equal(pl[name][:, :, t % G], x[:, :, t])


@pytest.mark.parametrize("n", [1, 31, 32, 95, 130])
def test_geometry_zero_is_the_plain_cache(orc, n):
    k, v, q = _data(n, n)
    pl = orc.geometry_planes(k, v, 2, 4, 0, max_tokens=160)
    a = orc.attend_geometry(pl, q, n, 2, 4, hkv=2, geometry=0)
    b = orc.attend(pl, q, n, 2, 4, hkv=2)
    assert np.array_equal(a, b)


@pytest.mark.parametrize("geom", GEOMS)
@pytest.mark.parametrize("n", [1, 40, 96, 131])
def test_attention_equals_dense_on_assembled_tensors(orc, geom, n):
    k, v, q = _data(n, 3 * n + geom)
    kb, vb = 2, 4
    pl = orc.geometry_planes(k, v, kb, vb, geom, max_tokens=160)
    out = orc.attend_geometry(pl, q, n, kb, vb, hkv=2, geometry=geom)
    kh, vh = _stored(pl, n, kb, vb, geom)
    assert np.array_equal(kh.astype(np.float32).astype(np.float64), kh)
    dense = orc.attend_dense(kh.astype(np.float32), vh.astype(np.float32), q.astype(np.float32))
    assert np.allclose(out, dense, rtol=0, atol=1e-12)


def _rope_np(x, pos, base=10000.0):
    """x[..., D] rotated to positions pos[...] (numpy, vectorized)."""
    i = np.arange(D // 2)
    ang = pos[..., None] * base ** (-2.0 * i / D)
    c, s = np.cos(ang), np.sin(ang)
    x0, x1 = x[..., 0::2], x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = x0 * c - x1 * s
    out[..., 1::2] = x0 * s + x1 * c
    return out


def _softmax(s):
    e = np.exp(s - s.max(-1, keepdims=True))
    return e / e.sum(-1, keepdims=True)


@pytest.mark.parametrize("geom", GEOMS)
@pytest.mark.parametrize("n", [5, 64, 100])
def test_metrics_follow_their_definitions(orc, geom, n):
    k, v, q = _data(n, 7 * n + geom)
    kb, vb = 2, 2
    pl = orc.geometry_planes(k, v, kb, vb, geom, max_tokens=128)
    summary, rows = orc.error_metrics(pl, k, v, q, n, kb, vb, hkv=2, geometry=geom)
    kh, vh = _stored(pl, n, kb, vb, geom)
    kx, vx, qx = k.astype(np.float64), v.astype(np.float64), q.astype(np.float64)
    hq, hkv = q.shape[1], k.shape[1]
    want = np.zeros((hq, 6))
    for h in range(hq):
        kvh = h // (hq // hkv)
        qr = _rope_np(qx[0, h], np.array(n - 1.0))
        pos = np.arange(n, dtype=np.float64)
        a = _softmax(_rope_np(kx[0, kvh], pos) @ qr / np.sqrt(D))
        ah = _softmax(_rope_np(kh[0, kvh], pos) @ qr / np.sqrt(D))
        ref = a @ vx[0, kvh]
        want[h] = [((ah - a) ** 2).sum(), ((a @ vh[0, kvh] - ref) ** 2).sum(), (ref ** 2).sum(),
                   ((ah @ vh[0, kvh] - ref) ** 2).sum(), ((kh[0, kvh] - kx[0, kvh]) ** 2).sum(),
                   ((vh[0, kvh] - vx[0, kvh]) ** 2).sum()]
    assert np.allclose(rows, want, rtol=1e-9, atol=1e-15)
    assert summary["key_error"] == pytest.approx(np.sqrt(want[:, 4]).mean(), rel=1e-12)
    assert summary["score_error"] == pytest.approx(np.sqrt(want[:, 0]).mean(), rel=1e-12)
    assert summary["value_output_rel_error"] == pytest.approx(
        np.sqrt(want[:, 1] / want[:, 2]).mean(), rel=1e-12)


def test_exact_axis_gives_exact_zeros(orc):
    """Keys constant along tokens and values constant along each token's
    channel groups: the page's geometry stores both exactly (every group has
    zero range), so every error is exactly 0; flipping an axis makes that
    operand's errors non-zero."""
    rng = np.random.default_rng(2)
    nb, h, n = 1, 2, 96
    a = rng.standard_normal((nb, h, 1, D)).astype(np.float16)
    k = np.ascontiguousarray(np.broadcast_to(a, (nb, h, n, D)))
    b = rng.standard_normal((nb, h, n, D // G, 1)).astype(np.float16)
    v = np.ascontiguousarray(np.broadcast_to(b, (nb, h, n, D // G, G)).reshape(nb, h, n, D))
    q = rng.standard_normal((nb, 4, D)).astype(np.float16)
    res = {}
    for geom in GEOMS:
        pl = orc.geometry_planes(k, v, 2, 2, geom, max_tokens=n)
        res[geom], _ = orc.error_metrics(pl, k, v, q, n, 2, 2, hkv=h, geometry=geom)
    assert all(x == 0.0 for x in res[0].values())
    assert res[1]["key_error"] > 0 and res[1]["value_error"] == 0
    assert res[2]["key_error"] == 0 and res[2]["score_error"] == 0
    assert res[2]["value_error"] > 0 and res[2]["value_output_rel_error"] > 0


@pytest.mark.parametrize("geom", GEOMS)
def test_single_token_closed_form(orc, geom):
    """n = 1: both weight vectors are [1], so the score error is 0 and both
    output errors are |vhat_0 - v_0| / |v_0|."""
    k, v, q = _data(1, 40 + geom)
    pl = orc.geometry_planes(k, v, 2, 2, geom, max_tokens=32)
    s, rows = orc.error_metrics(pl, k, v, q, 1, 2, 2, hkv=2, geometry=geom)
    _, vh = _stored(pl, 1, 2, 2, geom)
    v0 = v.astype(np.float64)[0, :, 0]
    rel = np.linalg.norm(vh[0, :, 0] - v0, axis=-1) / np.linalg.norm(v0, axis=-1)
    assert s["score_error"] == 0.0
    assert s["value_output_rel_error"] == pytest.approx(rel.mean(), rel=1e-12)
    assert s["output_rel_error"] == pytest.approx(rel.mean(), rel=1e-12)


def test_direction_of_the_pages_claim(orc):
    """On keys with steady outlier channels and flat values with a few large
    tokens (the pages' structure, synthetic), at B = 2, G = 32: per-channel
    keys beat per-token keys on reconstruction and on attention scores, and
    per-token values beat per-channel values on the attention output; the
    page's geometry has the smallest end-to-end output error and the
    doubly flipped one the largest.  (The page's value-reconstruction
    reversal comes from real value statistics and is not asserted.)"""
    cfg = synth.scaled(synth.CONFIGS["ablation_7b"], batch=1, kv_heads=8, q_heads=8,
                       n_tokens=512)
    k, v, q = synth.make_keys(cfg), synth.make_values(cfg), synth.make_query(cfg)
    res = {}
    for geom in GEOMS:
        pl = orc.geometry_planes(k, v, 2, 2, geom)
        res[geom], _ = orc.error_metrics(pl, k, v, q, cfg.n_tokens, 2, 2, hkv=8, geometry=geom)
    assert res[0]["key_error"] * 2 < res[1]["key_error"]
    assert res[0]["score_error"] * 1.5 < res[1]["score_error"]
    assert res[0]["value_output_rel_error"] * 1.2 < res[2]["value_output_rel_error"]
    e2e = [res[g]["output_rel_error"] for g in GEOMS]
    assert min(e2e) == e2e[0] and max(e2e) == e2e[3]
