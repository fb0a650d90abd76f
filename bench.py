#!/usr/bin/env python3
"""Decode-attention throughput of the quantized KV cache on one MI355X.

One step = one decode step for the whole batch of one layer: append the new
token (key into the full-precision tail, flushed into a quantized group when
G keys have accumulated; value quantized at once), then decode attention of
one query per head over every cached token (unpack, dequantize, rotary
embedding, q.k, online softmax, weighted sum of values).  By default a step
is one kvq_append_attend call where that is one kernel launch (a plain cache
with at most 4 query heads per KV head), else kvq_append_token then
kvq_attend_decode; --two-call always makes the two calls.

The timed steps rotate over R independent caches (R chosen so that R caches
exceed twice the 256 MB Infinity Cache), so a cache is never still resident
in that cache when its step starts: the bytes come from HBM.

Prints one JSON line.  value = decode-attention algorithmic bytes moved per
second over the timed steps (wall clock, launches included); the roofline
object reports the attention kernel alone against the HBM roofline, timed
with HIP events on the stream it runs on, over as many further steps (events
in the timed steps would add their own queue packets to the wall clock),
with the VALU view beside it.  A third set of event-timed steps writes a
1 GiB scratch buffer before each step (flushing the Infinity Cache), so each
line also shows whether cache residency inflates the rotating-cache figure.

The prefill figure times the caches' prompt prefills enqueued back to back
(the first, after an idle GPU, reported apart).

--decode-loop K (with --config llama2_13b or llama2_13b_b4): prefill the
prompt once, then time K consecutive decode steps on that one cache end to
end (appends included, no flush inside the loop); prints tokens/s = batch *
K / loop time instead.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0       # MI355X HBM3E, vendor figure
FP32_UNPACKED_PEAK_TFLOPS = 256 * 64 * 2 * 2.4e9 / 1e12  # 78.6: one FMA per lane per cycle
INFINITY_CACHE = 256 << 20  # bytes
FLUSH_BYTES = 1 << 30       # scratch written before each flushed step
SIMDS = 256 * 4             # compute units x SIMDs per CU
NOMINAL_CLOCK_HZ = 2.4e9    # MI355X peak engine clock
KERNEL_SOURCES = ["quantized_decode_attention_keys_amd/csrc/kvq_attend_kernel.h",
                  "quantized_decode_attention_keys_amd/csrc/kvq_append.h",
                  "quantized_decode_attention_keys_amd/csrc/kvq_codec.h",
                  "quantized_decode_attention_keys_amd/csrc/kvq_internal.h"]
TRAFFIC_FILE = "profiles/decode_attention_traffic.json"


def kernel_source_hash() -> str:
    import hashlib
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_counters(config_name: str):
    """The committed rocprofv3 counter record of the attention kernel for
    this workload (HBM bytes per launch from FETCH_SIZE/WRITE_SIZE, VALU
    instructions per launch from SQ_INSTS_VALU), or {} when there is none or
    the kernel source changed since it was taken."""
    path = os.path.join(ROOT, TRAFFIC_FILE)
    if not os.path.exists(path):
        return {}
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_sha256") != kernel_source_hash() or rec.get("config") != config_name:
        return {}
    return rec


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def calibrate_copy():
    """A plain device-to-device copy of 1 GiB, three times: the reference
    whose FETCH_SIZE / WRITE_SIZE readings scale the counters to bytes."""
    import torch
    x = torch.ones(256 * 1024 * 1024, dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)
    for _ in range(3):
        y.copy_(x)
    torch.cuda.synchronize()
    print(json.dumps({"calibration_copy_bytes": x.numel() * 4, "copies": 3}))


def quantized_tokens(n: int, G: int, residual: int, sink: int = 0) -> int:
    """Tokens [min(n, sink), Tq) are quantized; with a residual window R the
    last tokens (at least R) stay in full precision, with a sink the first
    `sink` tokens."""
    a = n - residual
    q = a // G * G if a > 0 else 0
    return max(q, min(n, sink))


GEOMETRIES = {"kivi": 0, "keys_per_token": 1, "values_per_channel": 2, "both_flipped": 3}


def cache_bytes(cfg, n: int, residual: int = 0, sink: int = 0, geometry: int = 0) -> int:
    """Bytes a cache of n tokens holds for the attention to read: per
    operand, packed codes and binary16 (step, zero) pairs of the quantized
    tokens and the unquantized rows of the others.  Keys grouped per channel
    (the default) have one meta word per (group of G tokens, channel), keys
    grouped per token one per (token, group of G channels); the same for
    values.  Windows: tokens [min(n, S), Tq) are quantized (values [S, n)
    without a residual window); a flipped geometry has no windows, an
    operand grouped per token is fully quantized and one grouped per channel
    up to G * floor(n / G)."""
    G, D = cfg.group, cfg.head_dim
    nbh = cfg.batch * cfg.kv_heads
    esz = 2 if cfg.dtype == "float16" else 4
    ns = min(n, sink)
    tq = quantized_tokens(n, G, residual, sink)
    key_tok, val_tok = bool(geometry & 1), not geometry & 2
    kq = n if key_tok else tq - ns
    vq = (tq if residual > 0 else n) - ns if val_tok else tq

    def operand(bits, nq, per_token):
        meta = nq * (D // G) if per_token else (nq // G) * D
        return nbh * (nq * D * bits // 8 + meta * 4 + (n - nq) * D * esz)

    return operand(cfg.key_bits, kq, key_tok) + operand(cfg.value_bits, vq, val_tok)


def attend_bytes(cfg, n: int, residual: int = 0, sink: int = 0, geometry: int = 0) -> int:
    """Algorithmic bytes of one decode-attention call at length n: the
    cache's planes and unquantized rows, q and out."""
    return (cache_bytes(cfg, n, residual, sink, geometry)
            + cfg.batch * cfg.q_heads * cfg.head_dim * ((2 if cfg.dtype == "float16" else 4) + 4))


def attend_flops(cfg, n: int) -> int:
    """The method's fp32 arithmetic per decode call: per cached (key, value)
    element pair, key dequantize (2) + rotary rotation (3: a pair turns with
    4 multiplies and 2 adds) + value dequantize (2), and per query head
    sharing the KV head q.k (2) + p*v (2)."""
    qpk = cfg.q_heads // cfg.kv_heads
    return cfg.batch * cfg.kv_heads * n * cfg.head_dim * (7 + 4 * qpk)


def fp8_bytes(cfg, n: int, with_q: bool = True) -> int:
    """One E4M3 byte per cached key and value element (+ q and out); the
    prefill moves 2 input bytes in and 1 out per element (3x the cache at
    fp16 inputs, reported as 3 * fp8_bytes without q)."""
    esz = 2 if cfg.dtype == "float16" else 4
    kv = 2 * cfg.batch * cfg.kv_heads * n * cfg.head_dim
    return kv + (cfg.batch * cfg.q_heads * cfg.head_dim * (esz + 4) if with_q else 0)


def prefill_bytes(cfg, n: int, residual: int = 0, sink: int = 0, geometry: int = 0) -> int:
    """Quantize-and-pack of n tokens: K and V read once, planes written."""
    esz = 2 if cfg.dtype == "float16" else 4
    return (2 * cfg.batch * cfg.kv_heads * n * cfg.head_dim * esz
            + cache_bytes(cfg, n, residual, sink, geometry))


class HipEvents:
    """hipEventCreateWithFlags/Record/ElapsedTime through ctypes: recording
    costs a few microseconds of host time, so the timed loop stays ahead of
    the GPU.  The events are timing-only (hipEventDisableSystemFence): no
    system-scope cache writeback/invalidate when they complete."""

    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self, count: int):
        import ctypes
        self.ct = ctypes
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float),
                                                 ctypes.c_void_p, ctypes.c_void_p]
        self.ev = []
        for _ in range(count):
            e = ctypes.c_void_p()
            if self.hip.hipEventCreateWithFlags(ctypes.byref(e),
                                                ctypes.c_uint(self.DISABLE_SYSTEM_FENCE)) != 0:
                raise RuntimeError("hipEventCreateWithFlags failed")
            self.ev.append(e.value)

    def record(self, i: int, stream: int):
        return self.hip.hipEventRecord(self.ev[i], stream)

    def elapsed_ms(self, i: int, j: int) -> float:
        ms = self.ct.c_float()
        if self.hip.hipEventElapsedTime(self.ct.byref(ms), self.ev[i], self.ev[j]) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def close(self):
        for e in self.ev:
            self.hip.hipEventDestroy(self.ct.c_void_p(e))
        self.ev = []


def cpu_baseline(cfg, n: int, budget_s: float = 12.0, residual: int = 0, sink: int = 0,
                 geometry: int = 0, fp8: bool = False):
    """The oracle (plain single-threaded fp64 C) on a bounded sample of the
    same workload: decode attention for whole sequences, rows timed until
    about budget_s seconds of CPU work."""
    import numpy as np

    import oracle
    import synth
    try:
        os.sched_setaffinity(0, {sorted(os.sched_getaffinity(0))[0]})
    except (AttributeError, OSError):
        pass
    q = synth.make_query(cfg, 0, 0)
    rows_done, t_total, bytes_done = 0, 0.0, 0
    one = synth.scaled(cfg, batch=1)
    per_row = (fp8_bytes(one, n) if fp8 else attend_bytes(one, n, residual, sink, geometry)) \
        / cfg.q_heads
    for b in range(cfg.batch):
        k = synth.make_keys(cfg, 0, 0, n, seqs=[b])
        v = synth.make_values(cfg, 0, 0, n, seqs=[b])
        if fp8:
            pl = (oracle.quantize_fp8(k, cfg.group), oracle.quantize_fp8(v, cfg.group))
        elif geometry:
            pl = oracle.geometry_planes(k, v, cfg.key_bits, cfg.value_bits, geometry, cfg.group)
        else:
            kp = oracle.quantize_keys(k, cfg.key_bits, cfg.group, residual=residual, sink=sink)
            vals = oracle.quantize_values(v, cfg.value_bits, cfg.group, residual=residual,
                                          sink=sink)
            pl = dict(k_codes=kp[0], k_meta=kp[1], k_tail=kp[2], v_codes=vals[0],
                      v_meta=vals[1])
            if residual > 0:
                pl["v_tail"] = vals[2]
            if sink > 0:
                pl["k_sink"], pl["v_sink"] = kp[3], vals[-1]
        for r in range(cfg.q_heads):
            t0 = time.perf_counter()
            if fp8:
                oracle.attend_fp8(pl[0], pl[1], q[b:b + 1], n, cfg.kv_heads, cfg.group,
                                  cfg.rope_base, rows=(r, r + 1))
            elif geometry:
                oracle.attend_geometry(pl, q[b:b + 1], n, cfg.key_bits, cfg.value_bits,
                                       cfg.kv_heads, geometry, cfg.group, cfg.rope_base,
                                       rows=(r, r + 1))
            else:
                oracle.attend(pl, q[b:b + 1], n, cfg.key_bits, cfg.value_bits, cfg.kv_heads,
                              cfg.group, cfg.rope_base, rows=(r, r + 1), residual=residual,
                              sink=sink)
            t_total += time.perf_counter() - t0
            rows_done += 1
            bytes_done += per_row
            if t_total >= budget_s:
                break
        if t_total >= budget_s:
            break
    return {
        "value": round(bytes_done / t_total / 1e9, 4),
        "unit": "GB/s",
        "cores": 1,
        "kind": "oracle",
        "sample": f"decode attention of {rows_done} of {cfg.batch * cfg.q_heads} (sequence, head) "
                  f"rows at n={n}, {t_total:.1f} s on one host core "
                  f"(host has {os.cpu_count()} cores); same algorithmic bytes per row as the GPU",
        "cpu_model": cpu_model(),
        "tokens_per_s": round(rows_done / cfg.q_heads / t_total, 4),
    }


def decode_loop(cfg, steps: int, dev):
    """K consecutive decode steps on one cache, timed end to end: prefill
    the n-token prompt, then per step append the next token and attend with
    that step's query (one kvq_append_attend call), no flush inside the loop.
    The code objects are loaded first on a one-group cache of the same
    shape, so the loop's first step does not pay for it."""
    import numpy as np
    import torch

    import synth
    from quantized_decode_attention_keys_amd import QuantizedKVCache
    from quantized_decode_attention_keys_amd import _lib as L

    n0 = cfg.n_tokens
    tdt = torch.float16 if cfg.dtype == "float16" else torch.float32
    cap = n0 + steps
    k_new = torch.from_numpy(synth.make_keys(cfg, 0, n0, cap)).to(dev)
    v_new = torch.from_numpy(synth.make_values(cfg, 0, n0, cap)).to(dev)
    k_new = [k_new[:, :, i].contiguous() for i in range(steps)]
    v_new = [v_new[:, :, i].contiguous() for i in range(steps)]
    qs = [torch.from_numpy(synth.make_query(cfg, 0, s + 1)).to(dev) for s in range(steps)]
    out = torch.empty((cfg.batch, cfg.q_heads, cfg.head_dim), dtype=torch.float32, device=dev)

    def new_cache(cap_tokens):
        return QuantizedKVCache(cfg.batch, cfg.q_heads, cfg.kv_heads, cfg.head_dim, cap_tokens,
                                cfg.key_bits, cfg.value_bits, tdt, cfg.rope_base, device=dev)

    warm = new_cache(2 * cfg.group)
    k = torch.from_numpy(synth.make_keys(cfg, 0, 0, cfg.group)).to(dev)
    v = torch.from_numpy(synth.make_values(cfg, 0, 0, cfg.group)).to(dev)
    warm.prefill(k, v)
    for i in range(3):
        warm.append_attend(k_new[i], v_new[i], qs[i], out)
    torch.cuda.synchronize()
    warm.close()

    loops = []
    lib = L.lib()
    stream = torch.cuda.current_stream(dev).cuda_stream
    for rep in range(2):  # two loops, each on a freshly prefilled cache
        cache = new_cache(cap)
        k = torch.from_numpy(synth.make_keys(cfg, 0, 0, n0)).to(dev)
        v = torch.from_numpy(synth.make_values(cfg, 0, 0, n0)).to(dev)
        cache.prefill(k, v)
        del k, v
        torch.cuda.synchronize()
        h = cache.handle
        args = [(k_new[i].data_ptr(), v_new[i].data_ptr(), qs[i].data_ptr()) for i in range(steps)]
        op = out.data_ptr()
        status = 0
        t0 = time.perf_counter()
        for kp, vp, qp in args:
            status |= lib.kvq_append_attend(h, kp, vp, qp, op, stream)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        if status != 0 or len(cache) != cap:
            raise RuntimeError("a library call failed during the decode loop")
        loops.append(t1 - t0)
        cache.close()
        print(f"decode loop {rep}: {steps} steps in {(t1 - t0) * 1e3:.3f} ms", file=sys.stderr,
              flush=True)
    best = min(loops)
    total_bytes = sum(attend_bytes(cfg, n0 + s + 1) for s in range(steps))
    res = {
        "metric": f"{cfg.name} {steps}-step decode loop tokens/s",
        "value": round(cfg.batch * steps / best, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "loop_ms": [round(t * 1e3, 4) for t in loops],
        "ms_per_step": round(best / steps * 1e3, 5),
        "higher_is_better": True,
        "effective_GB_per_s": round(total_bytes / best / 1e9, 2),
        "pct_hbm_peak": round(100.0 * total_bytes / best / 1e9 / HBM_PEAK_GBS, 2),
        "dtype": "f32 (value weights p*step in binary16)",
        "data": "synthetic",
        "config": {"workload": f"{cfg.name}: {cfg.description}", "batch": cfg.batch,
                   "q_heads": cfg.q_heads, "kv_heads": cfg.kv_heads,
                   "head_dim": cfg.head_dim, "prompt": n0, "key_bits": cfg.key_bits,
                   "value_bits": cfg.value_bits, "step_calls": "kvq_append_attend",
                   "context_during_steps": [n0 + 1, n0 + steps]},
    }
    print(json.dumps(res), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", default="llama2_7b")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--caches", type=int, default=0, help="rotating caches (0 = auto)")
    ap.add_argument("--residual", type=int, default=0,
                    help="recent tokens kept in full precision (a multiple of 32)")
    ap.add_argument("--sink", type=int, default=0,
                    help="first tokens kept in full precision (a multiple of 32)")
    ap.add_argument("--geometry", default="kivi", choices=sorted(GEOMETRIES),
                    help="grouping axes (the ablation flips keys and/or values; no windows)")
    ap.add_argument("--format", default="int", choices=["int", "fp8"],
                    help="fp8: E4M3 bytes for keys and values (8 bits each, no windows)")
    ap.add_argument("--two-call", action="store_true",
                    help="step = kvq_append_token then kvq_attend_decode (default: "
                         "kvq_append_attend where it is one launch, i.e. a plain cache with "
                         "at most 4 query heads per KV head; the two calls otherwise)")
    ap.add_argument("--no-metrics", action="store_true",
                    help="skip the error-where-consumed metrics of the prompt cache")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a 1 GiB device copy (reference for the traffic counters)")
    ap.add_argument("--flush-mode", default="read", choices=["read", "write", "rw"],
                    help="how the flushed steps clear the Infinity Cache: read, write, or read "
                         "and write a 1 GiB scratch buffer before each step")
    ap.add_argument("--decode-loop", type=int, default=0, metavar="K",
                    help="time K consecutive decode steps on one cache end to end "
                         "(tokens/s = batch * K / loop time) instead of the rotating-cache steps")
    args = ap.parse_args()
    if args.calibrate_copy:
        calibrate_copy()
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the library has no multi-GPU component)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import synth
    from quantized_decode_attention_keys_amd import QuantizedKVCache

    if not torch.cuda.is_available():
        print("bench.py needs a ROCm GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    cfg = synth.CONFIGS[args.config]
    if args.decode_loop > 0:
        decode_loop(cfg, args.decode_loop, dev)
        return
    fp8 = args.format == "fp8"
    if fp8:
        cfg = synth.scaled(cfg, key_bits=8, value_bits=8,
                           description=cfg.description + "; FP8 E4M3 keys and values")
    n = cfg.n_tokens
    tdt = torch.float16 if cfg.dtype == "float16" else torch.float32
    # warm-up, the timed steps, then as many again with HIP events around
    # each launch (the per-launch figures): events add queue packets and
    # host calls, so the timed steps carry none; then as many again with a
    # 1 GiB scratch write before each (Infinity Cache flushed)
    total_steps = args.warmup + 3 * args.steps

    Rw, Sw = args.residual, args.sink
    geom = GEOMETRIES[args.geometry]
    one_cache = fp8_bytes(cfg, n) if fp8 else attend_bytes(cfg, n, Rw, Sw, geom)
    R = args.caches or max(2, math.ceil(2 * INFINITY_CACHE / one_cache) + 1)
    visits = math.ceil(total_steps / R)
    max_tokens = n + visits

    # inputs: a prompt of n-1 tokens, then one new token per visit
    k = torch.from_numpy(synth.make_keys(cfg, 0, 0, n - 1)).to(dev)
    v = torch.from_numpy(synth.make_values(cfg, 0, 0, n - 1)).to(dev)
    k_new = torch.from_numpy(synth.make_keys(cfg, 0, n - 1, n - 1 + visits)).to(dev)
    v_new = torch.from_numpy(synth.make_values(cfg, 0, n - 1, n - 1 + visits)).to(dev)
    k_new = [k_new[:, :, i].contiguous() for i in range(visits)]
    v_new = [v_new[:, :, i].contiguous() for i in range(visits)]
    q = torch.from_numpy(synth.make_query(cfg, 0, 0)).to(dev)
    out = torch.empty((cfg.batch, cfg.q_heads, cfg.head_dim), dtype=torch.float32, device=dev)

    caches = [QuantizedKVCache(cfg.batch, cfg.q_heads, cfg.kv_heads, cfg.head_dim, max_tokens,
                               cfg.key_bits, cfg.value_bits, tdt, cfg.rope_base, device=dev,
                               residual=Rw, sink=Sw, geometry=geom, format=int(fp8))
              for _ in range(R)]
    # prefill (quantize-and-pack of the whole prompt) of every cache, after
    # one untimed prefill of a one-group cache (first launches load the code).
    # The caches' prefills are enqueued back to back with an event after
    # each: while one runs the host enqueues the next, so the time between
    # consecutive events is the GPU's.  The first follows an idle GPU and
    # also holds the host's enqueue; it is reported apart and, with two or
    # more caches, left out of the median.
    warm = QuantizedKVCache(cfg.batch, cfg.q_heads, cfg.kv_heads, cfg.head_dim, cfg.group,
                            cfg.key_bits, cfg.value_bits, tdt, cfg.rope_base, device=dev)
    warm.prefill(k[:, :, :cfg.group].contiguous(), v[:, :, :cfg.group].contiguous())
    torch.cuda.synchronize()
    warm.close()
    pf_ev = [torch.cuda.Event(enable_timing=True) for _ in range(len(caches) + 1)]
    pf_ev[0].record()
    for i, c in enumerate(caches):
        c.prefill(k, v)
        pf_ev[i + 1].record()
    torch.cuda.synchronize()
    pf_all = [pf_ev[i].elapsed_time(pf_ev[i + 1]) for i in range(len(caches))]
    pf_ms = pf_all[1:] if len(pf_all) > 1 else pf_all
    # error where it is consumed, on the first cache's prompt (before the
    # appends): the unquantized prompt keys and values are still at hand
    metrics = None
    if not args.no_metrics and not fp8:
        q_prompt = torch.from_numpy(synth.make_query(cfg, 0, 0)).to(dev)
        mv = caches[0].error_metrics(k, v, q_prompt).cpu().numpy()
        metrics = {name: float(x) for name, x in zip(
            ("key_error", "score_error", "value_error", "value_output_rel_error",
             "output_rel_error"), mv)}
        metrics["tokens"] = n - 1
        del q_prompt
    del k, v
    torch.cuda.synchronize()

    # The timed loop calls the C ABI directly with precomputed device
    # pointers so that host overhead stays below GPU time per step and the
    # GPU queue never runs dry (then the events time the kernels themselves).
    from quantized_decode_attention_keys_amd import _lib as L
    lib = L.lib()
    stream = torch.cuda.current_stream(dev).cuda_stream
    handles = [c.handle for c in caches]
    kp = [t.data_ptr() for t in k_new]
    vp = [t.data_ptr() for t in v_new]
    qp, op = q.data_ptr(), out.data_ptr()
    append, attend = lib.kvq_append_token, lib.kvq_attend_decode
    append_attend = lib.kvq_append_attend

    hev = HipEvents(4 * args.steps)
    scratch = torch.zeros(FLUSH_BYTES // 4, dtype=torch.float32, device=dev)
    flush_sink = torch.empty((), dtype=torch.float32, device=dev)

    def flush():
        if args.flush_mode == "read":  # clean lines only: nothing to write back later
            torch.sum(scratch, dim=0, out=flush_sink)
        elif args.flush_mode == "write":
            scratch.fill_(0.0)
        else:
            scratch.add_(1.0)
    record = hev.hip.hipEventRecord
    evp = hev.ev

    # kvq_append_attend runs as one launch only for a plain cache with at
    # most 4 query heads per KV head; otherwise it makes the two calls, and
    # the bench then makes them itself so that the events time the
    # attention launch alone
    one_launch = (Rw == 0 and Sw == 0 and geom == 0 and not fp8
                  and cfg.q_heads // cfg.kv_heads <= 4)
    two_call = args.two_call or not one_launch

    def step(s, j=None):
        h = handles[s % R]
        i = s // R
        if two_call:
            st = append(h, kp[i], vp[i], stream)
            if j is not None:
                st |= record(evp[2 * j], stream)
            st |= attend(h, qp, op, stream)
        else:
            st = record(evp[2 * j], stream) if j is not None else 0
            st |= append_attend(h, kp[i], vp[i], qp, op, stream)
        if j is not None:
            st |= record(evp[2 * j + 1], stream)
        return st

    status = 0
    for s in range(args.warmup):
        status |= step(s)
    torch.cuda.synchronize()

    def step_bytes(L):
        return fp8_bytes(cfg, L) if fp8 else attend_bytes(cfg, L, Rw, Sw, geom)

    lengths = [n - 1 + (args.warmup + j) // R + 1 for j in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for j in range(args.steps):
        status |= step(args.warmup + j)
    t_enq = time.perf_counter()  # host time to enqueue the timed steps
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ev_base = args.warmup + args.steps
    ev_lengths = [n - 1 + (ev_base + j) // R + 1 for j in range(args.steps)]
    for j in range(args.steps):
        status |= step(ev_base + j, j)
    torch.cuda.synchronize()
    fl_base = ev_base + args.steps
    fl_lengths = [n - 1 + (fl_base + j) // R + 1 for j in range(args.steps)]
    for j in range(args.steps):
        flush()  # 1 GiB through the caches on the same stream: the step starts cold
        status |= step(fl_base + j, args.steps + j)
    torch.cuda.synchronize()
    if status != 0:
        raise RuntimeError(f"a library call failed during the timed steps (status bits {status})")
    if [len(c) for c in caches] != [n - 1 + len(range(r, total_steps, R)) for r in range(R)]:
        raise RuntimeError("cache lengths do not match the steps issued")

    wall = t1 - t0
    total_bytes = sum(step_bytes(L) for L in lengths)
    value = total_bytes / wall / 1e9
    attend_ms = np.array([hev.elapsed_ms(2 * j, 2 * j + 1) for j in range(args.steps)])
    flushed_ms = np.array([hev.elapsed_ms(2 * j, 2 * j + 1)
                           for j in range(args.steps, 2 * args.steps)])
    hev.close()
    del scratch
    att_avg_s = float(attend_ms.mean()) / 1e3
    bytes_per_launch = sum(step_bytes(L) for L in ev_lengths) / len(ev_lengths)
    achieved = bytes_per_launch / att_avg_s / 1e9
    flops_per_launch = sum(attend_flops(cfg, L) for L in ev_lengths) / len(ev_lengths)
    achieved_tflops = flops_per_launch / att_avg_s / 1e12
    fl_avg_s = float(flushed_ms.mean()) / 1e3
    fl_bytes = sum(step_bytes(L) for L in fl_lengths) / len(fl_lengths)
    counters = (measured_counters(cfg.name) if Rw == 0 and Sw == 0 and geom == 0 and not fp8
                else {})
    valu_insts = counters.get("sq_insts_valu_per_launch")

    res = {
        "metric": "quantized decode-attention effective KV GB/s (% of HBM peak); tokens/s",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 5),
        # host time per step spent enqueueing the timed steps (the library
        # call and its kernel launch): when it reaches ms_per_step the GPU
        # waited on the host
        "host_ms_per_step": round((t_enq - t0) / args.steps * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        # scores, softmax and accumulators in fp32; the value side multiplies
        # each code by its weight p*step rounded to binary16 (integer cache)
        "dtype": "f32" if fp8 or geom else "f32 (value weights p*step in binary16)",
        "data": "synthetic",
        "config": {
            "workload": f"{cfg.name}: {cfg.description}",
            "batch": cfg.batch, "q_heads": cfg.q_heads, "kv_heads": cfg.kv_heads,
            "head_dim": cfg.head_dim, "context": n, "key_bits": cfg.key_bits,
            "value_bits": cfg.value_bits, "group": cfg.group, "kv_dtype": cfg.dtype,
            "residual": Rw,
            "sink": Sw,
            "geometry": args.geometry,
            "format": "fp8_e4m3" if fp8 else "int",
            "step_calls": ("kvq_append_token + kvq_attend_decode" if two_call
                           else "kvq_append_attend"),
            "context_during_steps": [min(lengths), max(ev_lengths)],
            "rotating_caches": R,
            "parallelism": "single GPU",
        },
        "pct_hbm_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
        "tokens_per_s": round(cfg.batch * args.steps / wall, 1),
        "roofline": {
            # the attention kernel against the HBM roofline: algorithmic
            # bytes per launch / mean event-timed launch duration
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": counters.get("bytes_per_launch"),
            "kernel": ("attend_fp8_kernel (FP8 E4M3 decode attention)" if fp8 else
                       "attend_kernel (decode attention)" if geom == 0 else
                       "attend_geometry_kernel (geometry ablation attention)")
                      + ("; HIP events around each kvq_attend_decode call, over as many steps"
                         " after the timed ones"
                         if two_call else
                         "; HIP events around each kvq_append_attend call (append and attention"
                         " in one launch for a plain cache), over as many steps after the"
                         " timed ones"),
            "bytes_per_launch": int(bytes_per_launch),
            "avg_launch_us": round(att_avg_s * 1e6, 3),
            "p10_p90_us": [round(float(np.percentile(attend_ms, 10)) * 1e3, 3),
                           round(float(np.percentile(attend_ms, 90)) * 1e3, 3)],
            # the same launches with the Infinity Cache flushed before each
            "flushed": {"mode": args.flush_mode,
                        "avg_launch_us": round(fl_avg_s * 1e6, 3),
                        "achieved": round(fl_bytes / fl_avg_s / 1e9, 2),
                        "frac": round(fl_bytes / fl_avg_s / 1e9 / HBM_PEAK_GBS, 4)},
            # the VALU view: the method's fp32 arithmetic against the one-FMA-
            # per-lane rate (the library is built without packed fp32), and
            # the VALU instruction issue the counters measured
            "valu": {
                "flops_per_launch": int(flops_per_launch),
                "achieved": round(achieved_tflops, 3),
                "peak": round(FP32_UNPACKED_PEAK_TFLOPS, 1),
                "unit": "TFLOP/s",
                "frac": round(achieved_tflops / FP32_UNPACKED_PEAK_TFLOPS, 4),
                "insts_per_launch": valu_insts,
                "issue_frac_at_2.4GHz": (round(valu_insts * 4 / SIMDS / NOMINAL_CLOCK_HZ
                                               / att_avg_s, 4) if valu_insts else None),
            },
        },
        "prefill": {
            "tokens": n - 1,
            "median_ms": round(float(np.median(pf_ms)), 4),
            "samples": len(pf_ms),
            "first_call_ms": round(pf_all[0], 4),
            "GB_per_s": round((3 * fp8_bytes(cfg, n - 1, with_q=False) if fp8 else
                               prefill_bytes(cfg, n - 1, Rw, Sw, geom))
                              / (np.median(pf_ms) / 1e3) / 1e9, 2),
            "tokens_per_s": round(cfg.batch * (n - 1) / (np.median(pf_ms) / 1e3), 1),
        },
    }
    if metrics is not None:
        res["error_metrics"] = metrics
    for c in caches:
        c.close()
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(cfg, n, residual=Rw, sink=Sw, geometry=geom, fp8=fp8)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
