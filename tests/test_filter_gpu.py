"""The filtered decode step through the C ABI: T_t selected through TIP's
group maxima (gist.science/pt, "Resumo Tecnico" section 2, FAC first
bullet: the critical subset is chosen from the TIP scores).

On long rows with a fused budget, the TIP launch also writes the largest
score of every 16 consecutive tokens, and one launch selects T_t and attends.
The selection takes one of two routes, decided on the device per row:
  "filter"  a histogram of the group maxima gives the bin of the B-th largest;
            groups from that bin up are read again, their tokens at or above
            the smallest surviving maximum are listed, and a second histogram
            of those (plus a rank of its pivot bin) gives T_t exactly;
  "stream"  when those would not fit (at most B groups, every score equal,
            too many survivors or listed tokens, a crowded pivot bin):
            streaming passes over the row's scores.
Rows of at most B tokens ("whole") keep every position.  Each case names the
routes it is meant to reach, and the test checks that with a host copy of the
route decision on the GPU's own scores.

Checks per (sequence, query head):
* index work, bit-exact: the step's T_t equals the oracle's selection rule
  applied to the GPU's own fp32 TIP scores of that step (read back with
  fasa_tip_scores, the same kernel and arithmetic);
* the project's acceptance rules against the oracle's own fp64 scores (the
  tau band) and its output recomputed on the GPU's set.
"""

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from fasa_harness import GpuSetup, check_index_set, check_out, oracle_setup, run_decode, to_dev

pytestmark = pytest.mark.gpu

GROUP = 16
THREADS, WAVES = 512, 8
WAVE_PLAY_CAP = 512  # in-play tokens a wave lists
PIVOT_CAP = 64       # pivot-bin elements one wave ranks


def small(name, **kw):
    return W.shrink(W.get(name), **kw)


def _keys(s):
    """Order-preserving keys of fp32 scores as the kernels form them (-0 folded
    onto +0; a key of 0, from NaN only, taken as 1)."""
    u = np.asarray(s, np.float32).view(np.uint32).astype(np.uint64)
    u = np.where((u << 1) & 0xFFFFFFFF == 0, 0, u)
    k = np.where(u & 0x80000000, (~u) & 0xFFFFFFFF, u | 0x80000000)
    return np.where(k == 0, 1, k).astype(np.uint64)


def _key_value(k):
    k = np.asarray(k, np.uint64)
    bits = np.where(k & 0x80000000, k & 0x7FFFFFFF, (~k) & 0xFFFFFFFF)
    return bits.astype(np.uint32).view(np.float32)


def _pick(bins, nbins, budget):
    """(bin, count above it, its count) of the budget-th largest, from the top."""
    counts = np.bincount(bins, minlength=nbins)[::-1]
    cum = counts.cumsum()
    r = int(np.searchsorted(cum, budget))
    return nbins - 1 - r, int(cum[r] - counts[r]), int(counts[r])


def route(scores, budget):
    """The device's route for one row of fp32 scores at budget B (the
    decision described in the module docstring, in fp32 like the kernel):
    "whole", "filter" or "stream"."""
    s = np.asarray(scores, np.float32)
    n = s.size
    if n <= budget:
        return "whole"
    ng = -(-n // GROUP)
    if ng <= budget:
        return "stream"
    cap_w = 64 if budget <= 320 else 160  # surviving groups a wave holds
    k = np.zeros(ng * GROUP, np.uint64)
    k[:n] = _keys(s)
    gk = k.reshape(ng, GROUP).max(axis=1)
    vmin, vmax = _key_value(gk.min()), _key_value(gk.max())
    span = np.float32(vmax - vmin)
    if not (np.isfinite(vmin) and np.isfinite(vmax) and np.isfinite(span) and span > 0):
        return "stream"
    scale = np.float32(1024) / span
    if not np.isfinite(scale):
        return "stream"
    bins = np.minimum(1023, ((_key_value(gk) - vmin) * scale).astype(np.int64))
    pbin, above, count = _pick(bins, 1024, budget)
    surv = bins >= pbin
    if above + count > WAVES * cap_w:
        return "stream"
    # Group g belongs to thread g % 512, so to wave (g % 512) // 64.
    wave = (np.arange(ng) % THREADS) // (THREADS // WAVES)
    if np.bincount(wave[surv], minlength=WAVES).max() > cap_w:
        return "stream"
    kp = gk[surv].min()
    tok = k.reshape(ng, GROUP)
    in_play = (tok >= kp) & surv[:, None]
    if np.bincount(wave, weights=in_play.sum(axis=1), minlength=WAVES).max() > WAVE_PLAY_CAP:
        return "stream"
    play = tok[in_play]
    span2 = int(gk.max() - kp)
    sh2 = 0 if span2 < 1024 else span2.bit_length() - 10
    b2 = ((play - kp) >> np.uint64(sh2)).astype(np.int64)
    _, above2, count2 = _pick(b2, 1024, budget)
    need = budget - above2
    return "filter" if count2 == need or count2 <= PIVOT_CAP else "stream"


CASES = {
    # 32k-layer shapes at 9k-20k tokens.
    "c2_20k": (small("c2", context=20000), {"filter"}),
    "c2_9k_b100": (small("c2", context=9000, budget=100), {"filter"}),
    # Clustered planting (64-token spans), and rows past 2048 groups (20
    # group maxima per thread), with B past 320 (the larger survivor slots).
    "c5_40k": (small("c5", context=40000, budget=512, steps=2), {"filter"}),
    "c5_70k": (small("c5", n_q_heads=8, n_kv_heads=2, context=70000), {"filter"}),
    # Ragged batch with short rows (at most B groups: streamed).
    "ragged": (small("c3", batch=4, context=16000, context_min=900, budget=200),
               {"filter", "stream"}),
    # Ragged rows at B = 1000, all of at most B groups: streamed.
    "ragged_b1000": (small("c3", batch=3, context=16000, context_min=2500, budget=1000),
                     {"filter", "stream"}),
    # One query head per KV head, and eight.
    "g1": (small("c3", batch=2, n_q_heads=8, n_kv_heads=8, context=12000, budget=150),
           {"filter"}),
    "g8": (small("c3", batch=2, n_q_heads=16, n_kv_heads=2, context=12000, budget=150),
           {"filter"}),
    # bf16 at d = 64 and fp32 at d = 128.
    "d64": (small("c2", head_dim=64, context=20000, budget=256), {"filter"}),
    "f32": (small("c2", dtype="f32", context=10000, budget=128), {"filter"}),
    # A 1024-token span of planted keys: about 64 surviving groups fall to
    # one or two waves, past their slots, so the row is streamed.
    "wave_crowd": (small("c5", n_q_heads=8, n_kv_heads=2, context=30000, budget=256,
                         spans=(1, 1024), planted_count=1000), {"stream"}),
    # One 12288-token span of planted keys holding all of T_t.
    "one_span": (small("c5", n_q_heads=8, n_kv_heads=2, context=30000, budget=400,
                       spans=(1, 12288), planted_count=11000), {"filter"}),
}


def _scores_after(g, step, n_max):
    """The step's fp32 TIP scores, recomputed by the query-mode TIP launch on
    the cache the step appended to (seq_lens already advanced)."""
    w, x = g.w, g.x
    q = to_dev(x["q"][step], g.td)
    sc = torch.zeros(w.batch, w.n_q_heads, g.cap, dtype=torch.float32, device="cuda")
    g.ctx.tip_scores(g.side, q, g.seq_lens, n_max, sc, g.ws)
    return sc.cpu().numpy()


def _filter_parity(gpu, w, x, regimes=None, head_budgets=None):
    g = GpuSetup(gpu, w, x)
    o = oracle_setup(w, x)
    n_max = int(x["ctx"].max()) + w.steps - 1
    assert gpu.decode_layout(n_max, w.budget)[0] == "group_filter"
    hb_d = None if head_budgets is None else torch.from_numpy(head_budgets).cuda()
    seen = set()
    for t in range(w.steps):
        q = to_dev(x["q"][t], g.td)
        kn, vn = to_dev(x["k_new"][t], g.td), to_dev(x["v_new"][t], g.td)
        out = torch.empty(w.batch, w.n_q_heads, w.head_dim, dtype=torch.float32, device="cuda")
        idx = torch.full((w.batch, w.n_q_heads, w.budget), -7, dtype=torch.int32, device="cuda")
        g.ctx.decode_step(g.k, g.v, g.side, q, kn, vn, g.seq_lens, n_max, w.budget, out, g.ws,
                          idx_out=idx, advance=True, head_budgets=hb_d)
        assert g.ctx.check(g.ws) == 0
        got_idx, got_out = idx.cpu().numpy(), out.cpu().numpy()
        sc = _scores_after(g, t, n_max)
        res = o.step(x["q"][t], x["k_new"][t], x["v_new"][t], w.budget)
        for b in range(w.batch):
            n = int(o.lens[b])
            qr = o.query_rot(b, x["q"][t][b])
            for h in range(w.n_q_heads):
                where = f"step {t} b{b} h{h}"
                bh = w.budget if head_budgets is None else int(head_budgets[h])
                row = sc[b, h, :n].astype(np.float64)
                want = oracle.select.select_topb_width(row, min(bh, w.budget), w.budget)
                assert np.array_equal(got_idx[b, h], want), (
                    f"{where}: index set differs from the selection on the GPU's scores")
                seen.add(route(row, bh) if bh else "none")
                if head_budgets is None:
                    check_index_set(got_idx[b, h], res["scores"][(b, h)], w.budget, n, where)
                want_out = o.attend(b, h, qr[h], got_idx[b, h])
                check_out(got_out[b, h], want_out, w.dtype, where)
    if regimes is not None:
        assert seen & regimes, f"the case took routes {seen}, meant for {regimes}"
    return seen


@pytest.mark.parametrize("name", sorted(CASES))
def test_filtered_decode(gpu, name):
    w, regimes = CASES[name]
    _filter_parity(gpu, w, W.generate(w), regimes)


def test_filtered_per_head_budgets(gpu):
    """Budgets per query head (0, 1, B, B - 1 and others) on the filtered path."""
    w = small("c2", context=20000, budget=256)
    hb = W.head_budgets(3, w.n_q_heads, w.budget, "edges")
    _filter_parity(gpu, w, W.generate(w), head_budgets=hb)


@pytest.mark.parametrize("budget", [256, 700])
def test_filtered_zero_query_all_ties(gpu, budget):
    """q = 0: every score is 0, so T_t is the B lowest positions; every group
    maximum is equal, so the row is streamed."""
    w = small("c2", context=20000, budget=budget)
    x = W.generate(w)
    x["q"][:] = 0.0
    assert route(np.zeros(20000), budget) == "stream"
    g = GpuSetup(gpu, w, x)
    out, idx = run_decode(g, 0, budget)
    assert g.ctx.check(g.ws) == 0
    assert np.all(idx.cpu().numpy() == np.arange(budget))
    o = oracle_setup(w, x)
    res = o.step(x["q"][0], x["k_new"][0], x["v_new"][0], budget, heads=[0, 17, 31])
    for h in (0, 17, 31):
        check_out(out.cpu().numpy()[0, h], res["out"][0, h], "bf16", f"h{h}")


def test_filtered_repeat_and_graph_replay(gpu):
    """Bit-identical repeats, and a captured step replayed several times with
    eager work in between equals the eager result every time."""
    w = small("c5", context=40000, budget=512)
    x = W.generate(w)
    g = GpuSetup(gpu, w, x)
    a_out, a_idx = run_decode(g, 0, w.budget, advance=False)
    b_out, b_idx = run_decode(g, 0, w.budget, advance=False)
    assert torch.equal(a_idx, b_idx) and torch.equal(a_out, b_out)
    q, kn, vn = (to_dev(x[k][0], g.td) for k in ("q", "k_new", "v_new"))
    out, idx = torch.zeros_like(a_out), torch.zeros_like(a_idx)
    msl = int(x["ctx"].max())
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        g.ctx.decode_step(g.k, g.v, g.side, q, kn, vn, g.seq_lens, msl, w.budget, out, g.ws,
                          idx_out=idx)
    torch.cuda.current_stream().wait_stream(s)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        g.ctx.decode_step(g.k, g.v, g.side, q, kn, vn, g.seq_lens, msl, w.budget, out, g.ws,
                          idx_out=idx)
    for rep in range(4):
        out.zero_()
        idx.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(idx, a_idx), rep
        assert torch.equal(out, a_out), rep
        _ = run_decode(g, 0, w.budget, advance=False)


@pytest.mark.parametrize("kv_on_host", [False, True])
def test_filtered_step_captured_before_any_eager_call(gpu, kv_on_host):
    """A context's first decode step captured in a HIP graph (the step asks
    the runtime once whether K lives in host memory, here inside the capture)
    replays to exactly what the same step gives eagerly afterwards."""
    w = small("c5", context=12000, budget=512)
    x = W.generate(w)
    g = GpuSetup(gpu, w, x, kv_on_host=kv_on_host)
    q, kn, vn = (to_dev(x[k][0], g.td) for k in ("q", "k_new", "v_new"))
    msl = int(x["ctx"].max())
    out = torch.zeros(w.batch, w.n_q_heads, w.head_dim, dtype=torch.float32, device="cuda")
    idx = torch.zeros(w.batch, w.n_q_heads, w.budget, dtype=torch.int32, device="cuda")
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        g.ctx.decode_step(g.k, g.v, g.side, q, kn, vn, g.seq_lens, msl, w.budget, out, g.ws,
                          idx_out=idx)
    graph.replay()
    torch.cuda.synchronize()
    assert g.ctx.check(g.ws) == 0
    e_out, e_idx = run_decode(g, 0, w.budget, advance=False, max_seq_len=msl)
    assert torch.equal(idx, e_idx)
    assert torch.equal(out, e_out)
