"""ctypes shim over the plain C fp64 oracle (``oracle/oracle.c``).

TEST INFRASTRUCTURE ONLY: imported by the tests, the package smoke check and
the bench's CPU-baseline leg, never by the product path.  It shares no code
with the GPU library and imports nothing from it.

The functions take and return numpy arrays.  Element types: ``numpy.float16``
or ``numpy.float32`` inputs (passed to the C code as raw bits with a dtype
code); planes are ``uint32`` arrays in the packed layout documented in
``oracle.c``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

F16 = 0
F32 = 1


def build() -> str:
    """Compile oracle.c with gcc into liboracle.so (always recompiles)."""
    tmp = _LIB + ".tmp"
    subprocess.check_call(
        ["gcc", "-O2", "-std=c99", "-Wall", "-Wextra", "-fPIC", "-shared",
         "-o", tmp, _SRC, "-lm"])
    os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        L = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        i = ctypes.c_int
        d = ctypes.c_double
        L.orc_half_to_double.argtypes = [ctypes.c_uint16]
        L.orc_half_to_double.restype = d
        L.orc_double_to_half.argtypes = [d]
        L.orc_double_to_half.restype = ctypes.c_uint16
        L.orc_quant_group.argtypes = [P, i, i, P, P, P]
        L.orc_quant_group.restype = i
        L.orc_pack.argtypes = [P, i, i, P]
        L.orc_pack.restype = None
        L.orc_unpack.argtypes = [P, i, i, P]
        L.orc_unpack.restype = None
        L.orc_code_at.argtypes = [P, i, i]
        L.orc_code_at.restype = i
        L.orc_quantized_tokens.argtypes = [i, i, i]
        L.orc_quantized_tokens.restype = i
        L.orc_quantized_end.argtypes = [i, i, i, i]
        L.orc_quantized_end.restype = i
        L.orc_quantize_keys.argtypes = [P, i, i, i, i, i, i, i, i, i, i, P, P, P, P]
        L.orc_quantize_keys.restype = i
        L.orc_quantize_values.argtypes = [P, i, i, i, i, i, i, i, i, i, i, P, P, P, P]
        L.orc_quantize_values.restype = i
        L.orc_rope.argtypes = [P, i, d, d]
        L.orc_rope.restype = None
        L.orc_attend.argtypes = [i, i, i, i, i, i, i, i, i, i, i, d, P, P, P, P, P,
                                 P, P, P, i, P, i, i, i, P]
        L.orc_attend.restype = i
        L.orc_attend_dense.argtypes = [i, i, i, i, d, P, P, i, P, i, i, i, P]
        L.orc_attend_dense.restype = i
        L.orc_attend_geometry.argtypes = [i, i, i, i, i, i, i, i, i, i, i, i, d, P, P, P,
                                          P, P, P, P, P, i, P, i, i, i, P]
        L.orc_attend_geometry.restype = i
        L.orc_error_metrics.argtypes = [i, i, i, i, i, i, i, i, i, i, i, i, d, P, P, P,
                                        P, P, P, P, P, i, P, P, P, i, i, i, P]
        L.orc_error_metrics.restype = i
        L.orc_fp8_decode.argtypes = [ctypes.c_uint8]
        L.orc_fp8_decode.restype = d
        L.orc_fp8_encode.argtypes = [d]
        L.orc_fp8_encode.restype = ctypes.c_uint8
        L.orc_quantize_fp8.argtypes = [P, i, i, i, i, i, i, i, P]
        L.orc_quantize_fp8.restype = i
        L.orc_attend_fp8.argtypes = [i, i, i, i, i, i, d, P, P, i, P, i, i, i, P]
        L.orc_attend_fp8.restype = i
        _lib = L
    return _lib


def _ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


def _dtype_code(a: np.ndarray) -> int:
    if a.dtype == np.float16:
        return F16
    if a.dtype == np.float32:
        return F32
    raise TypeError(f"oracle inputs are float16 or float32, got {a.dtype}")


# ------------------------------------------------------------------ binary16

def half_to_double(bits: int) -> float:
    return lib().orc_half_to_double(bits)


def double_to_half(x: float) -> int:
    return lib().orc_double_to_half(float(x))


# ----------------------------------------------------------------- quantizer

def quant_group(x, bits: int):
    """Quantize one group. Returns (codes uint8[n], s16 bits, z16 bits)."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    codes = np.zeros(x.size, dtype=np.uint8)
    s = np.zeros(1, dtype=np.uint16)
    z = np.zeros(1, dtype=np.uint16)
    rc = lib().orc_quant_group(_ptr(x), x.size, bits, _ptr(codes), _ptr(s), _ptr(z))
    if rc != 0:
        raise ValueError("orc_quant_group failed")
    return codes, int(s[0]), int(z[0])


def pack(codes, bits: int) -> np.ndarray:
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    words = np.zeros(codes.size * bits // 32, dtype=np.uint32)
    lib().orc_pack(_ptr(codes), codes.size, bits, _ptr(words))
    return words


def unpack(words, n: int, bits: int) -> np.ndarray:
    words = np.ascontiguousarray(words, dtype=np.uint32)
    codes = np.zeros(n, dtype=np.uint8)
    lib().orc_unpack(_ptr(words), n, bits, _ptr(codes))
    return codes


def quantized_tokens(n: int, G: int = 32, residual: int = 0, sink: int = 0) -> int:
    """Tq: tokens [min(n, sink), Tq) are quantized, the sink tokens and
    [Tq, n) held in full precision."""
    return lib().orc_quantized_end(n, G, residual, sink)


def plane_shapes(nb, hkv, D, G, kbits, vbits, max_tokens, residual=0, sink=0):
    """Shapes of the packed planes for a cache of capacity max_tokens.  The
    key tail (and with residual > 0 the value tail) is a ring of
    residual + G token slots."""
    gcap = -(-max_tokens // G)
    tcap = gcap * G
    ring = residual + G
    return {
        "k_codes": (nb, hkv, gcap, D, G * kbits // 32),
        "k_meta": (nb, hkv, gcap, D),
        "v_codes": (nb, hkv, tcap, D // G, G * vbits // 32),
        "v_meta": (nb, hkv, tcap, D // G),
        "k_tail": (nb, hkv, ring, D),
        "v_tail": (nb, hkv, ring if residual > 0 else 0, D),
        "k_sink": (nb, hkv, sink, D),
        "v_sink": (nb, hkv, sink, D),
    }


def quantize_keys(k: np.ndarray, bits: int, G: int = 32, max_tokens=None, residual=0,
                  sink=0):
    """Key planes for k[nb][Hkv][T][D]: (k_codes, k_meta, k_tail), and the
    key sink fourth when sink > 0."""
    k = np.ascontiguousarray(k)
    nb, hkv, T, D = k.shape
    cap = T if max_tokens is None else max_tokens
    sh = plane_shapes(nb, hkv, D, G, bits, bits, max(cap, 1), residual, sink)
    kc = np.zeros(sh["k_codes"], dtype=np.uint32)
    km = np.zeros(sh["k_meta"], dtype=np.uint32)
    kt = np.zeros(sh["k_tail"], dtype=k.dtype)
    ks = np.zeros(sh["k_sink"], dtype=k.dtype)
    rc = lib().orc_quantize_keys(_ptr(k), _dtype_code(k), nb, hkv, T, D, G,
                                 bits, residual, sink, sh["k_meta"][2], _ptr(kc), _ptr(km),
                                 _ptr(kt), _ptr(ks) if sink > 0 else None)
    if rc != 0:
        raise ValueError("orc_quantize_keys failed")
    return (kc, km, kt, ks) if sink > 0 else (kc, km, kt)


def quantize_values(v: np.ndarray, bits: int, G: int = 32, max_tokens=None, residual=0,
                    sink=0):
    """Value planes for v[nb][Hkv][T][D]: (v_codes, v_meta), then the value
    tail ring when residual > 0, then the value sink when sink > 0."""
    v = np.ascontiguousarray(v)
    nb, hkv, T, D = v.shape
    cap = T if max_tokens is None else max_tokens
    sh = plane_shapes(nb, hkv, D, G, bits, bits, max(cap, 1), residual, sink)
    vc = np.zeros(sh["v_codes"], dtype=np.uint32)
    vm = np.zeros(sh["v_meta"], dtype=np.uint32)
    vt = np.zeros(sh["v_tail"], dtype=v.dtype)
    vs = np.zeros(sh["v_sink"], dtype=v.dtype)
    rc = lib().orc_quantize_values(_ptr(v), _dtype_code(v), nb, hkv, T, D, G,
                                   bits, residual, sink, sh["v_meta"][2], _ptr(vc), _ptr(vm),
                                   _ptr(vt) if residual > 0 else None,
                                   _ptr(vs) if sink > 0 else None)
    if rc != 0:
        raise ValueError("orc_quantize_values failed")
    out = (vc, vm)
    if residual > 0:
        out += (vt,)
    if sink > 0:
        out += (vs,)
    return out


# ---------------------------------------------------------------- attention

def rope(u, p: float, base: float = 10000.0) -> np.ndarray:
    u = np.array(u, dtype=np.float64)
    lib().orc_rope(_ptr(u), u.size, float(p), float(base))
    return u


def attend(planes: dict, q: np.ndarray, n: int, kbits: int, vbits: int,
           hkv: int, G: int = 32, base: float = 10000.0, rows=None,
           residual: int = 0, sink: int = 0) -> np.ndarray:
    """Decode attention over quantized planes for queries q[nb][Hq][D].

    ``planes`` holds k_codes, k_meta, k_tail, v_codes, v_meta (numpy), v_tail
    when residual > 0, k_sink and v_sink when sink > 0.  The tails' element type is q's.  ``rows`` =
    (begin, end) over b*Hq + hq.  Returns float64 [rows, D] (all rows:
    reshaped to [nb, Hq, D])."""
    q = np.ascontiguousarray(q)
    nb, hq, D = q.shape
    kc = np.ascontiguousarray(planes["k_codes"], dtype=np.uint32)
    km = np.ascontiguousarray(planes["k_meta"], dtype=np.uint32)
    kt = np.ascontiguousarray(planes["k_tail"]).astype(q.dtype, copy=False)
    kt = np.ascontiguousarray(kt)
    vc = np.ascontiguousarray(planes["v_codes"], dtype=np.uint32)
    vm = np.ascontiguousarray(planes["v_meta"], dtype=np.uint32)
    def opt(name, on):
        if not on:
            return None
        return np.ascontiguousarray(np.ascontiguousarray(planes[name]).astype(q.dtype,
                                                                            copy=False))
    vt = opt("v_tail", residual > 0)
    ks, vs = opt("k_sink", sink > 0), opt("v_sink", sink > 0)
    gcap = km.shape[2]
    tcap = vm.shape[2]
    r0, r1 = (0, nb * hq) if rows is None else rows
    out = np.zeros((r1 - r0, D), dtype=np.float64)
    P = lambda a: _ptr(a) if a is not None else None  # noqa: E731
    rc = lib().orc_attend(nb, hq, hkv, D, G, kbits, vbits, residual, sink, gcap, tcap,
                          float(base), _ptr(kc), _ptr(km), _ptr(kt), P(ks), _ptr(vc), _ptr(vm),
                          P(vt), P(vs), _dtype_code(q), _ptr(q), n, r0, r1, _ptr(out))
    if rc != 0:
        raise ValueError("orc_attend failed")
    if rows is None:
        return out.reshape(nb, hq, D)
    return out


def attend_dense(k: np.ndarray, v: np.ndarray, q: np.ndarray,
                 base: float = 10000.0, rows=None) -> np.ndarray:
    """Full-precision attention over unquantized k, v [nb][Hkv][n][D]."""
    k = np.ascontiguousarray(k)
    v = np.ascontiguousarray(v, dtype=k.dtype)
    q = np.ascontiguousarray(q, dtype=k.dtype)
    nb, hkv, n, D = k.shape
    hq = q.shape[1]
    r0, r1 = (0, nb * hq) if rows is None else rows
    out = np.zeros((r1 - r0, D), dtype=np.float64)
    rc = lib().orc_attend_dense(nb, hq, hkv, D, float(base), _ptr(k), _ptr(v),
                                _dtype_code(k), _ptr(q), n, r0, r1, _ptr(out))
    if rc != 0:
        raise ValueError("orc_attend_dense failed")
    if rows is None:
        return out.reshape(nb, hq, D)
    return out


# -------------------------------------------------------- geometry ablation

KEYS_PER_TOKEN = 1
VALUES_PER_CHANNEL = 2
GEOMETRIES = {"kivi": 0, "keys_per_token": KEYS_PER_TOKEN,
              "values_per_channel": VALUES_PER_CHANNEL,
              "both_flipped": KEYS_PER_TOKEN | VALUES_PER_CHANNEL}


def geometry_planes(k: np.ndarray, v: np.ndarray, kbits: int, vbits: int, geometry: int,
                    G: int = 32, max_tokens=None) -> dict:
    """Planes of a cache in any geometry (no windows).  A flipped operand
    takes the other operand's layout: keys per token are grouped like values
    (``k_codes`` [nb][Hkv][Tcap][D/G][Wk], ``k_meta`` [nb][Hkv][Tcap][D/G], no
    key tail); values per channel are grouped like keys (``v_codes``
    [nb][Hkv][Gcap][D][Wv], ``v_meta`` [nb][Hkv][Gcap][D], ``v_tail`` of G
    slots for the unfilled group)."""
    pl = {}
    if geometry & KEYS_PER_TOKEN:
        pl["k_codes"], pl["k_meta"] = quantize_values(k, kbits, G, max_tokens)
        nb, hkv, _, D = k.shape
        pl["k_tail"] = np.zeros((nb, hkv, G, D), dtype=k.dtype)
    else:
        pl["k_codes"], pl["k_meta"], pl["k_tail"] = quantize_keys(k, kbits, G, max_tokens)
    if geometry & VALUES_PER_CHANNEL:
        pl["v_codes"], pl["v_meta"], pl["v_tail"] = quantize_keys(v, vbits, G, max_tokens)
    else:
        pl["v_codes"], pl["v_meta"] = quantize_values(v, vbits, G, max_tokens)
    return pl


def _plane_args(planes, dtype, residual, sink, geometry):
    def u32(name):
        return np.ascontiguousarray(planes[name], dtype=np.uint32)

    def opt(name, on):
        if not on:
            return None
        return np.ascontiguousarray(np.ascontiguousarray(planes[name]).astype(dtype,
                                                                            copy=False))
    kc, km, vc, vm = u32("k_codes"), u32("k_meta"), u32("v_codes"), u32("v_meta")
    kt = opt("k_tail", True)
    vt = opt("v_tail", residual > 0 or bool(geometry & VALUES_PER_CHANNEL))
    ks, vs = opt("k_sink", sink > 0), opt("v_sink", sink > 0)
    # capacities from whichever plane is grouped per channel / per token
    if geometry & KEYS_PER_TOKEN:
        tcap = km.shape[2]
        gcap = vm.shape[2] if geometry & VALUES_PER_CHANNEL else tcap // 32
    else:
        gcap = km.shape[2]
        tcap = gcap * 32 if geometry & VALUES_PER_CHANNEL else vm.shape[2]
    return (kc, km, kt, ks, vc, vm, vt, vs), gcap, tcap


def attend_geometry(planes: dict, q: np.ndarray, n: int, kbits: int, vbits: int, hkv: int,
                    geometry: int, G: int = 32, base: float = 10000.0, rows=None,
                    residual: int = 0, sink: int = 0) -> np.ndarray:
    """Decode attention over a cache in any geometry (``geometry_planes``);
    geometry 0 also takes the residual and sink windows of ``attend``."""
    q = np.ascontiguousarray(q)
    nb, hq, D = q.shape
    arrs, gcap, tcap = _plane_args(planes, q.dtype, residual, sink, geometry)
    r0, r1 = (0, nb * hq) if rows is None else rows
    out = np.zeros((r1 - r0, D), dtype=np.float64)
    P = lambda a: _ptr(a) if a is not None else None  # noqa: E731
    rc = lib().orc_attend_geometry(nb, hq, hkv, D, G, kbits, vbits, geometry, residual, sink,
                                   gcap, tcap, float(base), *[P(a) for a in arrs],
                                   _dtype_code(q), _ptr(q), n, r0, r1, _ptr(out))
    if rc != 0:
        raise ValueError("orc_attend_geometry failed")
    return out.reshape(nb, hq, D) if rows is None else out


METRICS = ("key_error", "score_error", "value_error", "value_output_rel_error",
           "output_rel_error")


def summarize_metrics(rows: np.ndarray) -> dict:
    """Row sums (see ``error_metrics``) -> the five metrics, each a mean over
    output rows: key and value reconstruction error (Frobenius norm over the
    row's KV head), attention-score error (L2 norm of the weight
    difference), relative output error of the value side and end to end."""
    rows = np.asarray(rows, dtype=np.float64)
    return {
        "key_error": float(np.mean(np.sqrt(rows[:, 4]))),
        "score_error": float(np.mean(np.sqrt(rows[:, 0]))),
        "value_error": float(np.mean(np.sqrt(rows[:, 5]))),
        "value_output_rel_error": float(np.mean(np.sqrt(rows[:, 1] / rows[:, 2]))),
        "output_rel_error": float(np.mean(np.sqrt(rows[:, 3] / rows[:, 2]))),
    }


def error_metrics(planes: dict, k: np.ndarray, v: np.ndarray, q: np.ndarray, n: int,
                  kbits: int, vbits: int, hkv: int, geometry: int = 0, G: int = 32,
                  base: float = 10000.0, rows=None, residual: int = 0, sink: int = 0):
    """Error where it is consumed for the cache holding the unquantized
    k, v [nb][Hkv][n][D] (q's dtype).  Returns (summary dict, per-row sums
    [rows][6]): sum (ahat - a)^2, |A vhat - A v|^2, |A v|^2,
    |Ahat vhat - A v|^2, sum (khat - k)^2 and sum (vhat - v)^2."""
    q = np.ascontiguousarray(q)
    k = np.ascontiguousarray(k, dtype=q.dtype)
    v = np.ascontiguousarray(v, dtype=q.dtype)
    nb, hq, D = q.shape
    arrs, gcap, tcap = _plane_args(planes, q.dtype, residual, sink, geometry)
    r0, r1 = (0, nb * hq) if rows is None else rows
    out = np.zeros((r1 - r0, 6), dtype=np.float64)
    P = lambda a: _ptr(a) if a is not None else None  # noqa: E731
    rc = lib().orc_error_metrics(nb, hq, hkv, D, G, kbits, vbits, geometry, residual, sink,
                                 gcap, tcap, float(base), *[P(a) for a in arrs],
                                 _dtype_code(q), _ptr(k), _ptr(v), _ptr(q), n, r0, r1,
                                 _ptr(out))
    if rc != 0:
        raise ValueError("orc_error_metrics failed")
    return summarize_metrics(out), out


# ------------------------------------------------------------ FP8 E4M3 cache

def fp8_decode(b: int) -> float:
    return lib().orc_fp8_decode(int(b))


def fp8_encode(x: float) -> int:
    return lib().orc_fp8_encode(float(x))


def quantize_fp8(x: np.ndarray, G: int = 32, max_tokens=None) -> np.ndarray:
    """FP8 E4M3 planes uint8[nb][Hkv][Gcap][D][32] of x[nb][Hkv][T][D]:
    channel c, token j of group g at [g][c][j] (bytes of a group past T are
    0)."""
    x = np.ascontiguousarray(x)
    nb, hkv, T, D = x.shape
    cap = T if max_tokens is None else max_tokens
    gcap = -(-max(cap, 1) // G)
    out = np.zeros((nb, hkv, gcap, D, G), dtype=np.uint8)
    if lib().orc_quantize_fp8(_ptr(x), _dtype_code(x), nb, hkv, T, D, G, gcap, _ptr(out)) != 0:
        raise ValueError("orc_quantize_fp8 failed")
    return out


def attend_fp8(k8: np.ndarray, v8: np.ndarray, q: np.ndarray, n: int, hkv: int, G: int = 32,
               base: float = 10000.0, rows=None) -> np.ndarray:
    """Decode attention over FP8 planes (``quantize_fp8``) for q[nb][Hq][D]."""
    q = np.ascontiguousarray(q)
    nb, hq, D = q.shape
    k8 = np.ascontiguousarray(k8, dtype=np.uint8)
    v8 = np.ascontiguousarray(v8, dtype=np.uint8)
    r0, r1 = (0, nb * hq) if rows is None else rows
    out = np.zeros((r1 - r0, D), dtype=np.float64)
    rc = lib().orc_attend_fp8(nb, hq, hkv, D, G, k8.shape[2], float(base), _ptr(k8), _ptr(v8),
                              _dtype_code(q), _ptr(q), n, r0, r1, _ptr(out))
    if rc != 0:
        raise ValueError("orc_attend_fp8 failed")
    return out.reshape(nb, hq, D) if rows is None else out
