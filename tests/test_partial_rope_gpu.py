"""Partial RoPE through the C ABI (fasa_create_partial_rope).

The pages claim the functional sparsity holds under Partial-RoPE too
(gist.science/pt, "Resumo Tecnico", "Contribuicoes").  Reading: the first r
dims of a head rotate (rotate-half within them, theta^(-2c/r)); the rest pass
through and pair into zero-frequency FCs.  Every stage is checked against the
oracle under that reading: append (K, V, sidecar), TIP, whole decode steps,
dense decode, and r = d against the full-RoPE context.
"""

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from fasa_harness import (GpuSetup, check_index_set, check_out, oracle_setup, run_decode,
                          tip_bound, to_dev, ulp_diff_bf16)

pytestmark = pytest.mark.gpu

CASES = {
    # bf16, d = 128, G = 4, r = 64 (32 rotated FCs, 32 pass-through pairs)
    "c6s": W.shrink(W.get("c6"), context=5003, steps=2),
    # fp32, d = 64, G = 2, r = 16
    "c1p": W.shrink(W.get("c1"), rotary_dim=16, context=700, steps=2),
    # ragged batch, r = 32
    "c6r": W.shrink(W.get("c6"), batch=3, context=3001, context_min=1500, rotary_dim=32),
}


def _setup(gpu, name):
    w = CASES[name]
    x = W.generate(w)
    return w, x, GpuSetup(gpu, w, x), oracle_setup(w, x)


@pytest.mark.parametrize("name", list(CASES))
def test_partial_append(gpu, name):
    w, x, g, o = _setup(gpu, name)
    K = g.k.float().cpu().numpy()
    V = g.v.float().cpu().numpy()
    side = g.side.float().cpu().numpy()
    off, fcs = g.ctx.sidecar_layout()
    lo, hi = oracle.rope.fc_pairs(w.head_dim, w.rotary_dim)
    r = w.rotary_dim
    for b in range(w.batch):
        n0 = int(x["ctx"][b]) - 1
        want = o.K[b, :, :n0]
        got = K[b, :, :n0].astype(np.float64)
        if w.dtype == "bf16":
            ulps = ulp_diff_bf16(got.astype(np.float32), want.astype(np.float32))
            assert ulps.max() <= 1 and (ulps == 0).mean() >= 0.999
        else:
            R = r // 2
            partner = np.concatenate([want[..., R:r], want[..., :R]], -1)
            bound = 4 * 2.0 ** -24 * (np.abs(partner) + np.abs(want[..., :r]))
            assert np.all(np.abs(got[..., :r] - want[..., :r]) <= bound)
        # Pass-through dims are the inputs, bit for bit.
        assert np.array_equal(K[b, :, :n0, r:], x["k_prefill"][b][:, :n0, r:])
        assert np.array_equal(V[b, :, :n0], x["v_prefill"][b][:, :n0])
        for g_ in range(w.n_kv_heads):
            for p in range(off[g_], off[g_ + 1]):
                c = fcs[p]
                assert np.array_equal(side[b, p, :n0, 0], K[b, g_, :n0, lo[c]])
                assert np.array_equal(side[b, p, :n0, 1], K[b, g_, :n0, hi[c]])


@pytest.mark.parametrize("name", list(CASES))
def test_partial_tip_scores(gpu, name):
    w, x, g, o = _setup(gpu, name)
    n = torch.from_numpy((x["ctx"] - 1).astype(np.int32)).cuda()
    scores = torch.full((w.batch, w.n_q_heads, g.cap), np.nan, dtype=torch.float32,
                        device="cuda")
    g.ctx.tip_scores(g.side, to_dev(x["q"][0], g.td), n, int(x["ctx"].max()), scores, g.ws)
    s = scores.cpu().numpy().astype(np.float64)
    assert g.ctx.check(g.ws) == 0
    for b in range(w.batch):
        nb = int(x["ctx"][b]) - 1
        qr = oracle.rope.rope_rotate_partial(x["q"][0][b], nb - 1, w.rope_theta, w.rotary_dim)
        for h in range(w.n_q_heads):
            ks = o.K[b, h // w.group, :nb]
            want = oracle.tip.tip_scores(qr[h], ks, x["dom"][h], o.pairs)
            lim = 1e-5 * tip_bound(qr[h], ks, x["dom"][h], o.pairs) + 1e-30
            assert np.all(np.abs(s[b, h, :nb] - want) <= lim), (b, h)
            assert np.all(np.isnan(s[b, h, nb:]))


def _decode_parity(gpu, w, x, heads=None):
    g = GpuSetup(gpu, w, x)
    o = oracle_setup(w, x)
    for t in range(w.steps):
        out, idx = run_decode(g, t, w.budget)
        got_out, got_idx = out.cpu().numpy(), idx.cpu().numpy()
        res = o.step(x["q"][t], x["k_new"][t], x["v_new"][t], w.budget, heads=heads)
        for b in range(w.batch):
            n = int(o.lens[b])
            qr = o.query_rot(b, x["q"][t][b])
            for h in (range(w.n_q_heads) if heads is None else heads):
                where = f"step {t} b{b} h{h}"
                check_index_set(got_idx[b, h], res["scores"][(b, h)], w.budget, n, where)
                check_out(got_out[b, h], o.attend(b, h, qr[h], got_idx[b, h]), w.dtype, where)
    assert g.ctx.check(g.ws) == 0
    return g


@pytest.mark.parametrize("name", list(CASES))
def test_partial_decode_step(gpu, name):
    w = CASES[name]
    _decode_parity(gpu, w, W.generate(w))


def test_partial_decode_step_c6_full(gpu):
    """The 32k partial-RoPE layer at full size, in the launch configuration the
    benchmark times, on sampled heads."""
    w = W.get("c6")
    _decode_parity(gpu, w, W.generate(w), heads=[0, 7, 13, 31])


def test_partial_dense_matches_oracle(gpu):
    w, x, g, o = _setup(gpu, "c6s")
    n = torch.from_numpy((x["ctx"] - 1).astype(np.int32)).cuda()
    out = torch.empty(w.batch, w.n_q_heads, w.head_dim, dtype=torch.float32, device="cuda")
    g.ctx.dense_attn(g.k, g.v, to_dev(x["q"][0], g.td), n, int(x["ctx"].max()), out, g.ws)
    got = out.cpu().numpy()
    assert g.ctx.check(g.ws) == 0
    nb = int(x["ctx"][0]) - 1
    o.lens[0] = nb
    qr = o.query_rot(0, x["q"][0][0])
    for h in range(0, w.n_q_heads, 3):
        check_out(got[0, h], o.attend(0, h, qr[h], np.arange(nb)), w.dtype, f"h{h}")


def test_rotary_dim_equal_to_head_dim_is_full_rope(gpu):
    w = W.shrink(W.get("c2"), context=3000)
    x = W.generate(w)
    a = GpuSetup(gpu, w, x)
    wb = W.shrink(w, rotary_dim=w.head_dim)
    b = GpuSetup(gpu, wb, x)
    assert torch.equal(a.k, b.k) and torch.equal(a.side, b.side)
    oa, ia = run_decode(a, 0, w.budget)
    ob, ib = run_decode(b, 0, w.budget)
    assert torch.equal(oa, ob) and torch.equal(ia, ib)
