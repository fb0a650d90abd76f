"""``QuantizedKVCache``: a thin object over the C ABI.  PyTorch supplies the
device workspace, the input/output tensors and the stream; every step of the
computation runs in the library's HIP kernels."""
from __future__ import annotations

import torch

from . import _lib as L

_DTYPES = {torch.float16: L.KVQ_F16, torch.float32: L.KVQ_F32}


def _check(status: int, what: str):
    if status != L.KVQ_OK:
        raise L.KvqError(status, what)


class QuantizedKVCache:
    """One layer's quantized KV cache for `batch` sequences.

    k/v inputs are [batch][kv_heads][T][head_dim] (prefill) or
    [batch][kv_heads][head_dim] (append), q is [batch][q_heads][head_dim], all
    contiguous tensors of `dtype` on the cache's device; keys and queries are
    before the rotary embedding.  `residual` keeps the most recent tokens
    (at least `residual`, fewer than `residual` + group) in full precision,
    `sink` the first `sink` tokens.  `geometry` (ablation, no windows) flips
    the grouping axis: KVQ_KEYS_PER_TOKEN and/or KVQ_VALUES_PER_CHANNEL.
    `format` KVQ_FORMAT_FP8_E4M3 stores E4M3 bytes instead (key_bits and
    value_bits 8).
    Calls enqueue on the current torch stream (or `stream`) and return at
    once."""

    def __init__(self, batch, q_heads, kv_heads, head_dim, max_tokens, key_bits=2,
                 value_bits=2, dtype=torch.float16, rope_base=10000.0, group=32,
                 device=None, residual=0, sink=0, geometry=0, format=L.KVQ_FORMAT_INT):
        if dtype not in _DTYPES:
            raise TypeError("dtype must be torch.float16 or torch.float32")
        self.cfg = L.KvqConfig(batch, q_heads, kv_heads, head_dim, max_tokens, group,
                               key_bits, value_bits, _DTYPES[dtype], rope_base, residual,
                               sink, geometry, format)
        self.dtype = dtype
        self.device = torch.device("cuda", torch.cuda.current_device()) if device is None \
            else torch.device(device)
        st, self.layout = L.kvq_layout_for(self.cfg)
        _check(st, "kvq_layout_for")
        nbytes = self.layout.total_bytes
        # torch's caching allocator returns 512-byte aligned blocks
        self.workspace = torch.empty(nbytes, dtype=torch.uint8, device=self.device)
        st, self.handle = L.kvq_create(self.cfg, self.workspace.data_ptr(), nbytes)
        _check(st, "kvq_create")

    # ------------------------------------------------------------ helpers
    def _stream(self, stream):
        s = torch.cuda.current_stream(self.device) if stream is None else stream
        return s.cuda_stream

    def _arg(self, t, shape, name):
        if not isinstance(t, torch.Tensor) or t.dtype != self.dtype or t.device != self.device \
                or not t.is_contiguous() or tuple(t.shape) != tuple(shape):
            raise ValueError(f"{name}: expected a contiguous {self.dtype} tensor of shape "
                             f"{tuple(shape)} on {self.device}, got "
                             f"{getattr(t, 'dtype', None)} {tuple(getattr(t, 'shape', ()))}")
        return t.data_ptr()

    # --------------------------------------------------------------- API
    def __len__(self):
        return L.kvq_length(self.handle)

    def prefill(self, k, v, stream=None):
        c = self.cfg
        n = k.shape[2] if k.dim() == 4 else -1
        shape = (c.batch, c.kv_heads, n, c.head_dim)
        pk = self._arg(k, shape, "k")
        pv = self._arg(v, shape, "v")
        _check(L.kvq_quantize_prefill(self.handle, pk, pv, n, self._stream(stream)),
               "kvq_quantize_prefill")

    def append(self, k, v, stream=None):
        c = self.cfg
        shape = (c.batch, c.kv_heads, c.head_dim)
        pk = self._arg(k, shape, "k")
        pv = self._arg(v, shape, "v")
        _check(L.kvq_append_token(self.handle, pk, pv, self._stream(stream)),
               "kvq_append_token")

    def attend(self, q, out=None, stream=None):
        c = self.cfg
        pq = self._arg(q, (c.batch, c.q_heads, c.head_dim), "q")
        if out is None:
            out = torch.empty((c.batch, c.q_heads, c.head_dim), dtype=torch.float32,
                              device=self.device)
        elif out.dtype != torch.float32 or not out.is_contiguous() or \
                tuple(out.shape) != (c.batch, c.q_heads, c.head_dim):
            raise ValueError("out must be a contiguous float32 [batch][q_heads][head_dim] tensor")
        _check(L.kvq_attend_decode(self.handle, pq, out.data_ptr(), self._stream(stream)),
               "kvq_attend_decode")
        return out

    def append_attend(self, k, v, q, out=None, stream=None):
        """append(k, v) then attend(q) as one decode step (one kernel launch
        for a plain cache); returns the attention output."""
        c = self.cfg
        shape = (c.batch, c.kv_heads, c.head_dim)
        pk = self._arg(k, shape, "k")
        pv = self._arg(v, shape, "v")
        pq = self._arg(q, (c.batch, c.q_heads, c.head_dim), "q")
        if out is None:
            out = torch.empty((c.batch, c.q_heads, c.head_dim), dtype=torch.float32,
                              device=self.device)
        elif out.dtype != torch.float32 or not out.is_contiguous() or \
                tuple(out.shape) != (c.batch, c.q_heads, c.head_dim):
            raise ValueError("out must be a contiguous float32 [batch][q_heads][head_dim] tensor")
        _check(L.kvq_append_attend(self.handle, pk, pv, pq, out.data_ptr(), self._stream(stream)),
               "kvq_append_attend")
        return out

    def error_metrics(self, k, v, q, stream=None):
        """Error where it is consumed for the current cache: k, v are the
        unquantized keys and values of all cached tokens
        ([batch][kv_heads][n][head_dim]), q as for `attend`.  Returns a float64
        tensor of KVQ_METRICS entries on the device (key, score, value,
        value-output and output error; see kvq.h)."""
        c = self.cfg
        n = len(self)
        shape = (c.batch, c.kv_heads, n, c.head_dim)
        pk = self._arg(k, shape, "k")
        pv = self._arg(v, shape, "v")
        pq = self._arg(q, (c.batch, c.q_heads, c.head_dim), "q")
        out = torch.empty(L.KVQ_METRICS, dtype=torch.float64, device=self.device)
        _check(L.kvq_error_metrics(self.handle, pk, pv, pq, out.data_ptr(),
                                   self._stream(stream)), "kvq_error_metrics")
        return out

    def planes(self):
        """Views of the packed planes inside the workspace (no copy)."""
        c, lay = self.cfg, self.layout
        G = c.group
        nb, h, D = c.batch, c.kv_heads, c.head_dim
        wk, wv = G * c.key_bits // 32, G * c.value_bits // 32
        ws = self.workspace

        def view(off, shape, dt):
            n = 1
            for s in shape:
                n *= s
            esz = torch.tensor([], dtype=dt).element_size()
            return ws[off:off + n * esz].view(dt).view(shape)

        by_token = lambda w: (nb, h, lay.tcap, D // G, w)  # noqa: E731
        by_channel = lambda w: (nb, h, lay.gcap, D, w)  # noqa: E731
        kpt = bool(c.geometry & L.KVQ_KEYS_PER_TOKEN)
        vpc = bool(c.geometry & L.KVQ_VALUES_PER_CHANNEL)
        if c.format == L.KVQ_FORMAT_FP8_E4M3:
            # E4M3 bytes of group g, channel c, token j at
            # [g][c % 2][j // 16][c // 2][j % 16] in both code planes
            shape = (nb, h, lay.gcap, 2, 2, D // 2, 16)
            return {"k_fp8": view(lay.k_codes, shape, torch.uint8),
                    "v_fp8": view(lay.v_codes, shape, torch.uint8)}
        ks = by_token(wk) if kpt else by_channel(wk)
        vs = by_channel(wv) if vpc else by_token(wv)
        return {
            "k_codes": view(lay.k_codes, ks, torch.int32),
            "k_meta": view(lay.k_meta, ks[:-1], torch.int32),
            "v_codes": view(lay.v_codes, vs, torch.int32),
            "v_meta": view(lay.v_meta, vs[:-1], torch.int32),
            "k_tail": view(lay.k_tail, (nb, h, lay.tail_slots, D), self.dtype),
            "v_tail": view(lay.v_tail, (nb, h, lay.tail_slots if c.residual > 0 or vpc else 0,
                                        D), self.dtype),
            "k_sink": view(lay.k_sink, (nb, h, c.sink, D), self.dtype),
            "v_sink": view(lay.v_sink, (nb, h, c.sink, D), self.dtype),
        }

    def close(self):
        if getattr(self, "handle", None):
            L.kvq_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
