"""Budgets per query head (and per layer) through the C ABI.

The pages note that FASA composes with allocating the budget across layers
(gist.science/pt, "Resumo Tecnico", "Variantes de Implementacao").  A
per-layer budget is each layer's own `budget` argument; fasa_topk_per_head and
fasa_decode_step_per_head also let the query heads of one layer differ.  Every
select layout is covered: rows held whole (4, 8, 16 or 32 scores per thread),
chunks then candidates, and the one-workgroup-per-row path.
"""

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from fasa_harness import (GpuSetup, check_out, oracle_setup, run_decode, to_dev)

pytestmark = pytest.mark.gpu

HB_CASES = [
    # (kind, rows, n, budget, ragged, budget kind)
    ("normal", 8, 1800, 256, True, "edges"),       # whole row, 4 per thread
    ("ties", 8, 3000, 100, False, "edges"),        # whole row, 8 per thread
    ("normal", 8, 5003, 256, False, "uniform"),    # whole row, 16 per thread
    ("wide", 8, 12345, 1000, True, "edges"),       # whole row, 32 per thread
    ("planted", 8, 32768, 256, False, "edges"),    # chunks then candidates
    ("normal", 8, 4096 * 3 + 256, 256, True, "uniform"),
    ("ties", 4, 20000, 1024, False, "edges"),
    ("planted", 2, 24000, 8000, False, "edges"),  # whole row, 1024 threads x 32
    ("ties", 4, 36000, 3000, True, "edges"),       # whole row, 1024 threads x 40
    ("normal", 4, 131072, 1024, False, "uniform"),
    ("normal", 2, 100000, 3000, False, "edges"),   # one workgroup per row
]


def _ctx(gpu, rows, cap, budget):
    return gpu.Context(1, rows, 1 if rows in (1, 2, 4, 8) else rows, 64, cap, 1e4, "f32",
                       np.zeros((rows, 1), np.int32), budget)


@pytest.mark.parametrize("case", HB_CASES, ids=lambda c: f"{c[0]}-{c[2]}-B{c[3]}-{c[5]}")
def test_topk_per_head_exact(gpu, case):
    """Index work: bit-exact against the oracle on the same fp32 scores."""
    kind, rows, n, budget, ragged, hkind = case
    sc = W.random_scores(9, rows, n, kind)
    hb = W.head_budgets(5, rows, budget, hkind)
    cap = (n + 63) // 64 * 64
    ctx = _ctx(gpu, rows, cap, budget)
    buf = torch.zeros(1, rows, cap, dtype=torch.float32, device="cuda")
    buf[0, :, :n] = torch.from_numpy(sc).cuda()
    ws = ctx.new_workspace()
    seq = n - (37 if ragged else 0)
    lens = torch.tensor([seq], dtype=torch.int32, device="cuda")
    hb_d = torch.from_numpy(hb).cuda()
    for rep in range(2):  # the second pass checks the workspace was left clean
        idx = torch.full((1, rows, budget), -7, dtype=torch.int32, device="cuda")
        ctx.topk(buf, lens, n, budget, idx, ws, head_budgets=hb_d)
        got = idx.cpu().numpy()[0]
        assert ctx.check(ws) == 0
        for r in range(rows):
            want = oracle.select.select_topb_width(sc[r, :seq].astype(np.float64),
                                                   int(hb[r]), budget)
            assert np.array_equal(got[r], want), (r, int(hb[r]), rep)


def test_topk_per_head_all_equal_is_uniform(gpu):
    rows, n, budget = 8, 9000, 700
    sc = W.random_scores(10, rows, n, "ties")
    ctx = _ctx(gpu, rows, 9024, budget)
    buf = torch.zeros(1, rows, 9024, dtype=torch.float32, device="cuda")
    buf[0, :, :n] = torch.from_numpy(sc).cuda()
    ws = ctx.new_workspace()
    lens = torch.tensor([n], dtype=torch.int32, device="cuda")
    a = torch.empty(1, rows, budget, dtype=torch.int32, device="cuda")
    b = torch.empty_like(a)
    ctx.topk(buf, lens, n, budget, a, ws)
    ctx.topk(buf, lens, n, budget, b, ws,
             head_budgets=torch.full((rows,), budget, dtype=torch.int32, device="cuda"))
    assert torch.equal(a, b)


def test_head_budget_out_of_range_is_clamped_and_flagged(gpu):
    rows, n, budget = 4, 3000, 64
    sc = W.random_scores(11, rows, n, "normal")
    ctx = _ctx(gpu, rows, 3008, budget)
    buf = torch.zeros(1, rows, 3008, dtype=torch.float32, device="cuda")
    buf[0, :, :n] = torch.from_numpy(sc).cuda()
    ws = ctx.new_workspace()
    lens = torch.tensor([n], dtype=torch.int32, device="cuda")
    idx = torch.empty(1, rows, budget, dtype=torch.int32, device="cuda")
    hb = torch.tensor([-3, budget + 5, 10, budget], dtype=torch.int32, device="cuda")
    ctx.topk(buf, lens, n, budget, idx, ws, head_budgets=hb)
    assert ctx.check(ws) & gpu.DEVFLAG_BUDGET
    got = idx.cpu().numpy()[0]
    for r, b_eff in enumerate([0, budget, 10, budget]):
        want = oracle.select.select_topb_width(sc[r].astype(np.float64), b_eff, budget)
        assert np.array_equal(got[r], want), r
    assert ctx.check(ws) == 0  # the flag was cleared by the first check


DECODE_CASES = {
    # fused select + FAC, rows held whole
    "c2s": (W.shrink(W.get("c2"), context=5003, budget=512, steps=2), "edges"),
    # ragged batch
    "c3s": (W.shrink(W.get("c3"), batch=3, context=3001, context_min=1500, steps=1), "uniform"),
    # chunks then candidates, fused FAC
    "c5s": (W.shrink(W.get("c5"), context=20000, budget=1024, steps=1), "edges"),
    # chunks then candidates, split-K FAC (B > 1024)
    "c4s": (W.shrink(W.get("c4"), batch=2, context=9000, budget=2000, steps=2), "edges"),
    # one workgroup per row for the select, split-K FAC
    "c4l": (W.shrink(W.get("c4"), batch=1, context=100000, budget=3000, steps=1), "uniform"),
}


@pytest.mark.parametrize("name", list(DECODE_CASES))
def test_decode_step_per_head(gpu, name):
    w, hkind = DECODE_CASES[name]
    x = W.generate(w)
    hb = W.head_budgets(6, w.n_q_heads, w.budget, hkind)
    g = GpuSetup(gpu, w, x)
    o = oracle_setup(w, x)
    hb_d = torch.from_numpy(hb).cuda()
    heads = list(range(w.n_q_heads)) if w.context <= 10000 else [0, 1, 2, 3, 9, 31]
    for t in range(w.steps):
        out = torch.empty(w.batch, w.n_q_heads, w.head_dim, dtype=torch.float32, device="cuda")
        idx = torch.empty(w.batch, w.n_q_heads, w.budget, dtype=torch.int32, device="cuda")
        g.ctx.decode_step(g.k, g.v, g.side, to_dev(x["q"][t], g.td), to_dev(x["k_new"][t], g.td),
                          to_dev(x["v_new"][t], g.td), g.seq_lens,
                          int(x["ctx"].max()) + w.steps - 1, w.budget, out, g.ws, idx_out=idx,
                          advance=True, head_budgets=hb_d)
        got_out, got_idx = out.cpu().numpy(), idx.cpu().numpy()
        res = o.step(x["q"][t], x["k_new"][t], x["v_new"][t], w.budget, heads=heads,
                     head_budgets=hb)
        for b in range(w.batch):
            n = int(o.lens[b])
            qr = o.query_rot(b, x["q"][t][b])
            for h in heads:
                where = f"step {t} b{b} h{h} B_h={hb[h]}"
                bh = int(hb[h])
                row = got_idx[b, h]
                take = min(bh, n)
                assert np.all(row[take:] == -1), where
                sel = row[:take]
                assert np.all(np.diff(sel) > 0) and np.all((sel >= 0) & (sel < n)), where
                if bh:
                    want = res["idx"][b, h][:take]
                    diff = np.setxor1d(sel, want)
                    s = res["scores"][(b, h)]
                    tau = res["tau"][b, h]
                    assert np.all(np.abs(s[diff] - tau) <= 1e-3 * abs(tau)), where
                check_out(got_out[b, h], o.attend(b, h, qr[h], row), w.dtype, where)
    assert g.ctx.check(g.ws) == 0


def test_decode_step_per_head_all_equal_is_uniform(gpu):
    w = W.shrink(W.get("c2"), context=5003)
    x = W.generate(w)
    ga = GpuSetup(gpu, w, x)
    gb = GpuSetup(gpu, w, x)
    oa, ia = run_decode(ga, 0, w.budget)
    q = to_dev(x["q"][0], gb.td)
    kn, vn = to_dev(x["k_new"][0], gb.td), to_dev(x["v_new"][0], gb.td)
    ob = torch.empty_like(oa)
    ib = torch.empty_like(ia)
    hb = torch.full((w.n_q_heads,), w.budget, dtype=torch.int32, device="cuda")
    gb.ctx.decode_step(gb.k, gb.v, gb.side, q, kn, vn, gb.seq_lens, int(x["ctx"].max()),
                       w.budget, ob, gb.ws, idx_out=ib, advance=True, head_budgets=hb)
    assert torch.equal(ia, ib) and torch.equal(oa, ob)


def test_per_layer_budgets_in_one_graph(gpu):
    """Layer-wise allocation: L layers, each with its own budget and per-head
    budgets, captured in one HIP graph; every replay matches eager, and each
    layer's eager step meets the oracle's step with its budgets."""
    w = W.shrink(W.get("c2"), context=3000, budget=512)
    x = W.generate(w)
    L = 4
    layer_budget = [512, 256, 128, 64]
    setups = [GpuSetup(gpu, w, x) for _ in range(L)]
    hbs = [torch.from_numpy(W.head_budgets(20 + i, w.n_q_heads, layer_budget[i], "uniform")).cuda()
           for i in range(L)]
    q = to_dev(x["q"][0], setups[0].td)
    kn, vn = to_dev(x["k_new"][0], setups[0].td), to_dev(x["v_new"][0], setups[0].td)
    outs = [torch.empty(w.batch, w.n_q_heads, w.head_dim, device="cuda") for _ in range(L)]
    idxs = [torch.empty(w.batch, w.n_q_heads, layer_budget[i], dtype=torch.int32, device="cuda")
            for i in range(L)]
    msl = int(x["ctx"].max())

    def run_all():
        for i, g in enumerate(setups):
            g.ctx.decode_step(g.k, g.v, g.side, q, kn, vn, g.seq_lens, msl, layer_budget[i],
                              outs[i], g.ws, idx_out=idxs[i], head_budgets=hbs[i])

    run_all()
    torch.cuda.synchronize()
    eager = [(o.clone(), i.clone()) for o, i in zip(outs, idxs)]
    for g in setups:
        assert g.ctx.check(g.ws) == 0
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run_all()
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run_all()
    for rep in range(3):
        for o in outs:
            o.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for i in range(L):
            assert torch.equal(outs[i], eager[i][0]) and torch.equal(idxs[i], eager[i][1]), (rep, i)
    # Each layer's eager step against the oracle's step with that layer's
    # budgets: the per-head index sets (tau band) and the outputs recomputed
    # on the GPU's sets.
    for i in range(L):
        hb = hbs[i].cpu().numpy()
        got_idx, got_out = eager[i][1].cpu().numpy(), eager[i][0].cpu().numpy()
        o = oracle_setup(w, x)
        res = o.step(x["q"][0], x["k_new"][0], x["v_new"][0], layer_budget[i], head_budgets=hb)
        n = int(o.lens[0])
        qr = o.query_rot(0, x["q"][0][0])
        for h in range(w.n_q_heads):
            where = f"layer {i} h{h} B_h={hb[h]}"
            bh = int(hb[h])
            row = got_idx[0, h]
            take = min(bh, n)
            assert np.all(row[take:] == -1), where
            sel = row[:take]
            assert np.all(np.diff(sel) > 0) and np.all((sel >= 0) & (sel < n)), where
            if bh:
                diff = np.setxor1d(sel, res["idx"][0, h][:take])
                s, tau = res["scores"][(0, h)], res["tau"][0, h]
                assert np.all(np.abs(s[diff] - tau) <= 1e-3 * abs(tau)), where
            check_out(got_out[0, h], o.attend(0, h, qr[h], row), w.dtype, where)
