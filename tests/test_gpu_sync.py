"""The debug-sync mode (KVQ_SYNC=1 when a handle is created): every call
drains its stream and checks the runtime's error state before returning.
It must leave results unchanged: a cache made in that mode gives the same
attention output and error metrics, bit for bit, as one made without it,
and both caches' planes equal the oracle's in every used slot, through
prefill, appends across a key-group flush, the one-launch step and the
plain attention; each call reports KVQ_OK."""
import os

import numpy as np
import pytest
import torch

import synth
from _parity import assert_planes_equal, gpu_planes, make_cache, oracle_planes, to_gpu

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name,residual", [("tiny", 0), ("llama2_7b", 0), ("tiny", 32)])
def test_sync_mode_matches(name, residual, monkeypatch):
    cfg = synth.scaled(synth.CONFIGS[name], batch=2, n_tokens=70) if name != "tiny" else \
        synth.CONFIGS[name]
    n0, n1, cap = 30, 70, 96
    k = synth.make_keys(cfg, 0, 0, n1)
    v = synth.make_values(cfg, 0, 0, n1)
    monkeypatch.delenv("KVQ_SYNC", raising=False)
    plain = make_cache(cfg, cap, residual=residual)
    monkeypatch.setenv("KVQ_SYNC", "1")
    synced = make_cache(cfg, cap, residual=residual)
    monkeypatch.delenv("KVQ_SYNC")
    kg, vg = to_gpu(k), to_gpu(v)
    outs = []
    for c in (plain, synced):
        c.prefill(kg[:, :, :n0].contiguous(), vg[:, :, :n0].contiguous())
        res = []
        for t in range(n0, n1):
            kt, vt = kg[:, :, t].contiguous(), vg[:, :, t].contiguous()
            q = to_gpu(synth.make_query(cfg, 0, t + 1))
            if t % 2:
                res.append(c.append_attend(kt, vt, q).cpu().numpy())
            else:
                c.append(kt, vt)
                res.append(c.attend(q).cpu().numpy())
        if residual == 0:
            m = c.error_metrics(kg, vg, to_gpu(synth.make_query(cfg, 0, 0))).cpu().numpy()
            res.append(np.asarray(m))
        outs.append((res, gpu_planes(c)))
    (ra, pa), (rb, pb) = outs
    for a, b in zip(ra, rb):
        np.testing.assert_array_equal(a, b)
    op = oracle_planes(cfg, k, v, cap, residual=residual)
    for pl in (pa, pb):  # unused slots of the workspace hold whatever was there
        assert_planes_equal(pl, op, n1, residual=residual)
    for c in (plain, synced):
        c.close()
    torch.cuda.synchronize()
