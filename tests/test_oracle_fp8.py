"""Pins for the oracle's FP8 (OCP E4M3) cache ("Rotate, Then Round: The
Geometry of KV-Cache Compression", key takeaways: FP8 as the production
default).  Readings: round to nearest, ties to even, saturation at +-448,
no scale factor, the oracle's planes in the logical order (group, channel,
token in group); the GPU library's 16-byte piece order is a permutation of
it that the tests undo (tests/fp8_layout.py).

The format is checked against its definition (closed-form values of named
codes, symmetry, ordering), the encoder by brute force over every finite
binary16 value and 100,000 fp32 draws (nearest of the 127 finite
non-negative values, ties to the even code), the planes by re-deriving each
byte with that brute-force encoder, attention against the dense formula on
the decoded tensors."""
import numpy as np
import pytest

from fp8_layout import piece_offset, to_logical

D = 64
G = 32


def _table(orc):
    """Finite non-negative E4M3 values by code 0x00..0x7E (brute force)."""
    return np.array([orc.fp8_decode(b) for b in range(0x7F)])


def _brute_encode(x, table):
    """Nearest code, ties to the even code, |x| >= 448 saturates."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    d = np.abs(a[:, None] - table[None, :])
    best = d.min(axis=1, keepdims=True)
    cand = d == best
    # ties: two adjacent codes; take the even one
    codes = np.where(cand.sum(1) > 1, np.argmax(cand & (np.arange(0x7F) % 2 == 0), 1),
                     np.argmax(cand, 1))
    codes = np.where(a >= 448.0, 0x7E, codes)
    return (codes | np.where(np.signbit(x), 0x80, 0)).astype(np.uint8)


def test_named_codes(orc):
    assert orc.fp8_decode(0x38) == 1.0
    assert orc.fp8_decode(0x7E) == 448.0           # largest finite: 1.75 * 2^8
    assert orc.fp8_decode(0x08) == 2.0 ** -6       # smallest normal
    assert orc.fp8_decode(0x01) == 2.0 ** -9       # smallest subnormal
    assert orc.fp8_decode(0x07) == 7 * 2.0 ** -9   # largest subnormal
    assert orc.fp8_decode(0x40) == 2.0 and orc.fp8_decode(0x3C) == 1.5
    assert np.isnan(orc.fp8_decode(0x7F)) and np.isnan(orc.fp8_decode(0xFF))
    assert orc.fp8_decode(0x00) == 0.0 and np.signbit(orc.fp8_decode(0x80))


def test_sign_symmetry_and_order(orc):
    t = _table(orc)
    assert np.all(np.diff(t) > 0)                  # strictly increasing by code
    for b in range(0x7F):
        assert orc.fp8_decode(b | 0x80) == -orc.fp8_decode(b)
    # binade structure: 8 values per binade, step 2^(e-10) for biased e >= 1
    for e in range(1, 16):
        vals = t[e * 8:min(e * 8 + 8, 0x7F)]
        assert np.allclose(np.diff(vals), 2.0 ** (e - 10), rtol=0, atol=0)


def test_encoder_exhaustive_over_binary16(orc):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    x = bits.view(np.float16).astype(np.float64)
    x = x[np.isfinite(x)]
    want = _brute_encode(x, _table(orc))
    got = np.array([orc.fp8_encode(v) for v in x], dtype=np.uint8)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, f"{bad.size} mismatches, first x={x[bad[0]]!r}"


def test_encoder_on_fp32_draws(orc):
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(20000) * s for s in (1e-3, 0.05, 1, 30, 300)])
    x = x.astype(np.float32).astype(np.float64)
    want = _brute_encode(x, _table(orc))
    got = np.array([orc.fp8_encode(v) for v in x], dtype=np.uint8)
    assert np.array_equal(got, want)


def test_round_trip_error_bound(orc):
    """Half a step: 2^-4 relative on normal values, 2^-10 absolute below 2^-6."""
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.uniform(-448, 448, 20000), rng.uniform(-2 ** -6, 2 ** -6, 5000)])
    xr = np.array([orc.fp8_decode(orc.fp8_encode(v)) for v in x])
    normal = np.abs(x) >= 2 ** -6
    assert np.all(np.abs(xr - x)[normal] <= 2 ** -4 * np.abs(x)[normal])
    assert np.all(np.abs(xr - x)[~normal] <= 2 ** -10)


@pytest.mark.parametrize("T", [1, 31, 32, 77])
def test_planes_layout(orc, T):
    """Byte of token t = 32g + j, channel c at offset 32 c + j of group block
    g (the logical order), checked on the flat bytes; bytes past T are 0."""
    rng = np.random.default_rng(T)
    x = (rng.standard_normal((2, 3, T, D)) * 20).astype(np.float16)
    pl = orc.quantize_fp8(x, max_tokens=96)
    assert pl.shape == (2, 3, 3, D, G)
    flat = pl.reshape(2, 3, 3, D * G)
    table = _table(orc)
    c = np.arange(D)
    for t in range(-(-T // G) * G):
        got = flat[:, :, t // G][:, :, 32 * c + t % G]
        if t < T:
            want = _brute_encode(x[:, :, t].astype(np.float64).ravel(), table).reshape(2, 3, D)
            assert np.array_equal(got, want)
        else:
            assert not got.any()


def test_gpu_piece_permutation():
    """The tests' map from the GPU library's piece order to the logical one
    moves the byte at the documented piece offset of (c, j) to [c][j]."""
    rng = np.random.default_rng(5)
    pieces = rng.integers(0, 256, (2, 3, 2, 2, 2, D // 2, 16), dtype=np.uint8)
    flat = pieces.reshape(2, 3, 2, D * G)
    logical = to_logical(pieces)
    assert logical.shape == (2, 3, 2, D, G)
    offs = [piece_offset(D, c, j) for c in range(D) for j in range(G)]
    assert sorted(offs) == list(range(D * G))      # a permutation of the block
    for c in range(D):
        for j in range(G):
            assert np.array_equal(logical[:, :, :, c, j], flat[:, :, :, piece_offset(D, c, j)])


@pytest.mark.parametrize("n", [1, 33, 100])
def test_attention_equals_dense_on_decoded(orc, n):
    rng = np.random.default_rng(n)
    k = (rng.standard_normal((1, 2, n, D)) * 3).astype(np.float16)
    k[..., 5] *= 40
    v = rng.standard_normal((1, 2, n, D)).astype(np.float16)
    q = rng.standard_normal((1, 4, D)).astype(np.float16)
    k8, v8 = orc.quantize_fp8(k, max_tokens=128), orc.quantize_fp8(v, max_tokens=128)
    out = orc.attend_fp8(k8, v8, q, n, hkv=2)
    dec = np.vectorize(orc.fp8_decode)
    kd = np.stack([dec(k8[:, :, t // G, :, t % G]) for t in range(n)], axis=2)
    vd = np.stack([dec(v8[:, :, t // G, :, t % G]) for t in range(n)], axis=2)
    dense = orc.attend_dense(kd.astype(np.float32), vd.astype(np.float32), q.astype(np.float32))
    assert np.allclose(out, dense, rtol=0, atol=1e-12)
