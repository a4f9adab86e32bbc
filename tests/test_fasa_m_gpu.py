"""FASA-M: the K and V caches in pinned host memory, the sidecar on the GPU
(gist.science/pt, "Resumo Tecnico" section 2, "Variantes de Implementacao").

The kernels are the same ones, reading and writing the caches over the host
link, so the caches, the indices and (with one launch shape) the outputs must
be bit-identical to the device-resident run, and the decode step must pass the
oracle's checks as before.  One launch shape differs on purpose: with K and V
on the host, the filtered select + FAC takes one workgroup per row where the
device run splits a row's columns over 4 workgroups when rows are few, so
that each selected row crosses the link once.  The two shapes sum the same
products in a different order, so there the outputs agree to fp32 rounding.
"""

import numpy as np
import pytest
import torch

import workloads as W
from fasa_harness import GpuSetup, check_index_set, check_out, oracle_setup, run_decode, to_dev

pytestmark = pytest.mark.gpu

CASES = {
    "c2s": W.shrink(W.get("c2"), context=5003, steps=3),
    "c3s": W.shrink(W.get("c3"), batch=3, context=3001, context_min=1500, steps=2),
    "c5s": W.shrink(W.get("c5"), context=9000, budget=300, steps=2),
}


def _decode_all(gpu, w, x, kv_on_host):
    g = GpuSetup(gpu, w, x, kv_on_host=kv_on_host)
    if kv_on_host:
        assert g.k.device.type == "cpu" and g.k.is_pinned() and g.v.is_pinned()
        assert gpu.pointer_kind(g.k) == gpu.PTR_HOST_MAPPED
        assert gpu.pointer_kind(g.v) == gpu.PTR_HOST_MAPPED
    assert gpu.pointer_kind(g.side) == gpu.PTR_DEVICE
    outs, idxs = [], []
    for t in range(w.steps):
        out, idx = run_decode(g, t, w.budget)
        outs.append(out.cpu().numpy())
        idxs.append(idx.cpu().numpy())
    torch.cuda.synchronize()
    assert g.ctx.check(g.ws) == 0
    return g, outs, idxs


@pytest.mark.parametrize("name", list(CASES))
def test_host_kv_matches_device_kv_and_oracle(gpu, name):
    w = CASES[name]
    x = W.generate(w)
    gd, out_d, idx_d = _decode_all(gpu, w, x, False)
    gh, out_h, idx_h = _decode_all(gpu, w, x, True)
    assert torch.equal(gd.k.cpu(), gh.k), "K caches differ"
    assert torch.equal(gd.v.cpu(), gh.v), "V caches differ"
    assert torch.equal(gd.side, gh.side), "sidecars differ"
    msl = int(x["ctx"].max()) + w.steps - 1  # as run_decode passes it
    filtered = gpu.decode_layout(msl, w.budget)[0] == "group_filter"
    vmax = float(gd.v.float().abs().max())
    split = w.batch * w.n_q_heads * 4 <= torch.cuda.get_device_properties(0).multi_processor_count
    for t in range(w.steps):
        assert np.array_equal(idx_d[t], idx_h[t]), f"step {t}: indices differ"
        if filtered and split:
            # An output is sum(p v) / sum(p) over at most B rows, each sum in
            # fp32 in some order: either order is within B * 2^-24 of the
            # exact sums relative to sum(p |v|) and sum(p), so two orders
            # differ by at most about 4 B 2^-24 max|v|.
            bound = 4 * w.budget * 2.0 ** -24 * vmax
            assert np.all(np.abs(out_d[t] - out_h[t]) <= bound), f"step {t}: outputs differ"
        else:
            assert np.array_equal(out_d[t], out_h[t]), f"step {t}: outputs differ"
    assert np.array_equal(gh.seq_lens.cpu().numpy(), (x["ctx"] - 1 + w.steps).astype(np.int32))

    o = oracle_setup(w, x)
    heads = range(0, w.n_q_heads, 3)
    for t in range(w.steps):
        res = o.step(x["q"][t], x["k_new"][t], x["v_new"][t], w.budget, heads=heads)
        for b in range(w.batch):
            n = int(o.lens[b])
            qr = o.query_rot(b, x["q"][t][b])
            for h in heads:
                where = f"step {t} b{b} h{h}"
                check_index_set(idx_h[t][b, h], res["scores"][(b, h)], w.budget, n, where)
                want = o.attend(b, h, qr[h], idx_h[t][b, h])
                check_out(out_h[t][b, h], want, w.dtype, where)


def test_dense_from_host_cache_matches_device(gpu):
    w = CASES["c2s"]
    x = W.generate(w)
    gd = GpuSetup(gpu, w, x)
    gh = GpuSetup(gpu, w, x, kv_on_host=True)
    n = int(x["ctx"].max()) - 1
    q = to_dev(x["q"][0], gd.td)
    a = torch.empty(w.batch, w.n_q_heads, w.head_dim, device="cuda")
    b = torch.empty_like(a)
    gd.ctx.dense_attn(gd.k, gd.v, q, gd.seq_lens, n, a, gd.ws)
    gh.ctx.dense_attn(gh.k, gh.v, q, gh.seq_lens, n, b, gh.ws)
    assert torch.equal(a, b)


def test_pageable_cache_is_refused(gpu):
    """Pageable host memory is not mapped into the device: the binding refuses
    it before any kernel runs."""
    w = W.shrink(W.get("c2"), context=300)
    x = W.generate(w)
    g = GpuSetup(gpu, w, x)
    pageable = torch.zeros(g.k.shape, dtype=g.k.dtype)
    assert gpu.pointer_kind(pageable) == gpu.PTR_UNUSABLE
    kp = torch.zeros(w.batch, w.n_kv_heads, 2, w.head_dim, dtype=g.k.dtype, device="cuda")
    start = torch.zeros(w.batch, dtype=torch.int32, device="cuda")
    with pytest.raises(ValueError):
        g.ctx.append_kv(pageable, g.v, g.side, kp, kp, start, g.ws)
    q = to_dev(x["q"][0], g.td)
    kn = to_dev(x["k_new"][0], g.td)
    out = torch.empty(w.batch, w.n_q_heads, w.head_dim, device="cuda")
    with pytest.raises(ValueError):
        g.ctx.decode_step(pageable, g.v, g.side, q, kn, kn, g.seq_lens, n_max(x), w.budget,
                          out, g.ws)


def n_max(x):
    return int(x["ctx"].max())
