"""HIP path against the oracle, element by element, through the C ABI.

Each call of include/fasa.h is checked on seeded inputs at sizes the oracle
finishes in seconds (several tiles and a ragged tail), then the whole decode
step on all five workloads.  Acceptance rules: tests/fasa_harness.py.
"""

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from fasa_harness import (GpuSetup, oracle_setup, check_index_set, check_out, tip_bound,
                          ulp_diff_bf16, run_decode, to_dev)

pytestmark = pytest.mark.gpu


def small(name, **kw):
    return W.shrink(W.get(name), **kw)


# Shrunk workloads: same heads/dims/dtypes as the named ones, contexts the
# oracle handles in seconds, with ragged tails (not multiples of any tile).
SMALL = {
    "c1": W.get("c1"),
    "c2s": small("c2", context=5003),
    "c3s": small("c3", batch=3, context=3001, context_min=1500),
    "c4s": small("c4", batch=2, context=2500, budget=473, steps=3),
    "c5s": small("c5", context=9000, budget=300, steps=2),
    # Query heads per KV head 1, 2 and 8 with budgets of several FAC splits
    # (256 rows each), ragged batches and a batch that is not a multiple of 8.
    "g1s": small("c3", batch=3, n_q_heads=8, n_kv_heads=8, context=3001, context_min=1500,
                 budget=700),
    "g2s": small("c2", n_q_heads=8, n_kv_heads=4, context=5003, budget=1300),
    "g8s": small("c3", batch=3, n_q_heads=16, n_kv_heads=2, context=3001, context_min=1500,
                 budget=700),
    # The other two (dtype, head_dim) builds: bf16 at d = 64 and fp32 at d = 128.
    "h64s": small("c3", batch=2, head_dim=64, context=4003, context_min=2500, budget=300),
    "f128s": small("c2", dtype="f32", context=3001, budget=1100),
    "f128f": small("c2", dtype="f32", context=3001),  # fused select + FAC
    # Fused FAC split over column parts with budgets of several attend
    # rounds per part (256 rows a round): bf16 at d = 128 and d = 64, fp32
    # at d = 128.
    "c2m": small("c2", context=5003, budget=700),
    "h64m": small("c2", head_dim=64, context=4003, budget=600),
    "f128m": small("c2", dtype="f32", context=3001, budget=512),
    # B past the fused limit on rows chunks would barely cut: each row held
    # whole in 1024 threads (32 per thread), then the split FAC.
    "c4w": small("c4", batch=1, context=20000, budget=5000, steps=2),
    # TIP's per-head kernel at its edges: one dominant FC per head (3 of a
    # wave's 4 plane slots empty), and 8 query heads per KV head with 13
    # dominant FCs (16 slots, 3 empty).  (Partial RoPE: its own test file.)
    "t1": small("c2", n_dom=1, context=3001),
    "t8": small("c3", batch=2, n_q_heads=16, n_kv_heads=2, context=3001, context_min=2000,
                n_dom=13),
    # Dense grids past two workgroups per CU, so each workgroup walks several
    # 256-token chunks: 1, 2, 4 (ragged) and 8 query heads per KV head.
    "dm1": small("c3", batch=4, n_q_heads=8, n_kv_heads=8, context=6001, context_min=3000),
    "dm2": small("c2", n_q_heads=16, n_kv_heads=8, context=20000),
    "dm4": small("c3", batch=6, context=8192, context_min=4096),
    "dm8": small("c3", batch=3, n_q_heads=16, n_kv_heads=2, context=30001, context_min=15000),
}


def _prefilled(gpu, name):
    w = SMALL[name]
    x = W.generate(w)
    return w, x, GpuSetup(gpu, w, x), oracle_setup(w, x)


# ------------------------------------------------------------- append ----

@pytest.mark.parametrize("name", ["c1", "c2s", "c3s", "h64s", "f128s"])
def test_append_rope_and_sidecar(gpu, name):
    w, x, g, o = _prefilled(gpu, name)
    K = g.k.float().cpu().numpy()
    V = g.v.float().cpu().numpy()
    side = g.side.float().cpu().numpy()
    off, fcs = g.ctx.sidecar_layout()
    half = w.head_dim // 2
    for b in range(w.batch):
        n0 = int(x["ctx"][b]) - 1
        want = o.K[b, :, :n0]
        got = K[b, :, :n0].astype(np.float64)
        if w.dtype == "bf16":
            ulps = ulp_diff_bf16(got.astype(np.float32), want.astype(np.float32))
            assert ulps.max() <= 1, f"K off by {ulps.max()} ulp"
            assert (ulps == 0).mean() >= 0.999
        else:
            bound = 4 * 2.0 ** -24 * (np.abs(np.concatenate([want[..., half:], want[..., :half]], -1))
                                      + np.abs(want))
            assert np.all(np.abs(got - want) <= bound)
        assert np.array_equal(V[b, :, :n0], x["v_prefill"][b][:, :n0])
        # Sidecar is bit-identical to its K columns.
        for g_ in range(w.n_kv_heads):
            for p in range(off[g_], off[g_ + 1]):
                c = fcs[p]
                assert np.array_equal(side[b, p, :n0, 0], K[b, g_, :n0, c])
                assert np.array_equal(side[b, p, :n0, 1], K[b, g_, :n0, c + half])


def test_append_past_capacity_raises_flag(gpu):
    w = small("c1", context=65)
    x = W.generate(w)
    g = GpuSetup(gpu, w, x, capacity=64)
    assert g.ctx.check(g.ws) == 0
    kn = to_dev(x["k_new"][0][:, :, None, :], g.td)
    start = torch.full((1,), 64, dtype=torch.int32, device="cuda")
    g.ctx.append_kv(g.k, g.v, g.side, kn, kn, start, g.ws)
    assert g.ctx.check(g.ws) & gpu.DEVFLAG_APPEND
    assert g.ctx.check(g.ws) == 0  # cleared by the read


# ---------------------------------------------------------------- TIP ----

@pytest.mark.parametrize("name", ["c1", "c2s", "c3s", "h64s", "f128s", "g1s", "g2s", "g8s",
                                  "t1", "t8"])
def test_tip_scores(gpu, name):
    w, x, g, o = _prefilled(gpu, name)
    # Score the prefilled tokens with the step-0 query at position n0 - 1.
    n = torch.from_numpy((x["ctx"] - 1).astype(np.int32)).cuda()
    scores = torch.full((w.batch, w.n_q_heads, g.cap), np.nan, dtype=torch.float32, device="cuda")
    q = to_dev(x["q"][0], g.td)
    g.ctx.tip_scores(g.side, q, n, int(x["ctx"].max()), scores, g.ws)
    s = scores.cpu().numpy().astype(np.float64)
    assert g.ctx.check(g.ws) == 0
    for b in range(w.batch):
        nb = int(x["ctx"][b]) - 1
        qr = oracle.rope.rope_rotate(x["q"][0][b], nb - 1, w.rope_theta)
        for h in range(w.n_q_heads):
            ks = o.K[b, h // w.group, :nb]
            want = oracle.tip.tip_scores(qr[h], ks, x["dom"][h])
            lim = 1e-5 * tip_bound(qr[h], ks, x["dom"][h]) + 1e-30
            assert np.all(np.abs(s[b, h, :nb] - want) <= lim), (b, h)
            assert np.all(np.isnan(s[b, h, nb:])), "wrote past n_b"


# ---------------------------------------------------------------- top-B --

TOPK_CASES = [
    # (kind, rows, n, budget, ragged)
    ("normal", 4, 5003, 256, False),
    ("planted", 3, 32768, 256, False),
    ("ties", 4, 9000, 700, False),
    ("zeros", 2, 4100, 64, False),
    ("wide", 3, 12345, 1000, True),
    ("sorted_up", 2, 8193, 4097, False),
    ("normal", 2, 300, 256, True),      # some rows n <= B
    ("normal", 2, 256, 256, False),     # n == B
    ("normal", 2, 131072, 1024, False),
    ("normal", 1, 32831, 6193, False),
    ("normal", 2, 4097, 1, False),
    # Two-stage path (chunks of 4096): ties across chunk edges, a last chunk
    # shorter than B, one exactly B long, and the largest candidate count.
    ("ties", 2, 20000, 1024, False),
    ("normal", 2, 4096 * 2 + 5, 256, False),
    ("planted", 2, 4096 * 3 + 256, 256, False),
    ("normal", 2, 32768, 256, True),
    ("wide", 1, 8 * 4096, 1024, False),
    # Row held whole at 8 per thread; 16384-position chunks with the largest
    # candidate set; a row held whole at 32 per thread (no chunk reduces B).
    ("normal", 2, 3000, 100, False),
    ("planted", 1, 24000, 8000, False),
    ("ties", 1, 16000, 8500, True),
    # B past the fused limit on rows of 16k-40k that chunks would not cut by
    # three quarters: held whole in 1024 threads at 32 per thread (up to
    # 32768) or 40 (up to 40960).  The shortest such row, a 32k row, ties
    # with a ragged length, the longest; then one that chunks do cut, and the
    # first length past the whole-row limit.
    ("normal", 2, 16385, 1025, False),
    ("sorted_up", 1, 32768, 15000, False),
    ("ties", 2, 36000, 3000, True),
    ("planted", 1, 40960, 12000, False),
    ("ties", 2, 32768, 2000, True),
    ("normal", 1, 40961, 6193, False),
]


@pytest.mark.parametrize("case", TOPK_CASES, ids=lambda c: f"{c[0]}-{c[2]}-B{c[3]}")
def test_topk_exact(gpu, case):
    """Selection is index work: bit-exact against the oracle on the same fp32
    scores (both sides rank the identical fp32 values)."""
    kind, rows, n, budget, ragged = case
    sc = W.random_scores(7, rows, n, kind)
    cap = (n + 63) // 64 * 64
    lens = np.full(1, n, dtype=np.int32)
    ctx = gpu.Context(1, rows, 1 if rows in (1, 2, 4, 8) else rows, 64, cap, 1e4, "f32",
                      np.zeros((rows, 1), np.int32), max(budget, 1))
    buf = torch.zeros(1, rows, cap, dtype=torch.float32, device="cuda")
    buf[0, :, :n] = torch.from_numpy(sc).cuda()
    ws = ctx.new_workspace()
    for rep in range(2):  # second pass checks the workspace was left clean
        seq = n - (37 if ragged else 0)
        lens[0] = seq
        idx = torch.full((1, rows, budget), -7, dtype=torch.int32, device="cuda")
        ctx.topk(buf, torch.from_numpy(lens).cuda(), n, budget, idx, ws)
        got = idx.cpu().numpy()[0]
        assert ctx.check(ws) == 0
        for r in range(rows):
            want = oracle.select.select_topb(sc[r, :seq].astype(np.float64), budget)
            assert np.array_equal(got[r], want), (r, rep)


def _random_topk_cases(per_layout=4, seed=0x70B):
    """Seeded shapes, per_layout of them in each select layout: rows held whole
    (n <= 8192), chunks then candidates (B <= 1024), rows held whole in 1024
    threads at 32 and at 40 per thread (B > 1024, at least a third of n), and
    the one-workgroup-per-row path (rows past 40960 with B of 9000 and more);
    kinds, row counts and ragged lengths drawn at random."""
    r = np.random.Generator(np.random.PCG64(seed))
    kinds = ["normal", "ties", "wide", "planted", "zeros"]
    ranges = [  # (n range, B range as a function of n)
        ((1, 8192), lambda n: (1, n)),
        ((8193, 70000), lambda n: (1, 1024)),
        ((16385, 32768), lambda n: (max(1025, n // 3), n)),
        ((32769, 40960), lambda n: (max(1025, n // 3), n)),
        ((40961, 70000), lambda n: (9000, 20000)),
    ]
    cases = []
    for (n_lo, n_hi), b_of in ranges:
        for _ in range(per_layout):
            n = int(r.integers(n_lo, n_hi + 1))
            b_lo, b_hi = b_of(n)
            budget = int(r.integers(b_lo, b_hi + 1))
            cases.append((kinds[len(cases) % len(kinds)], int(r.integers(1, 4)), n, budget,
                          bool(r.integers(0, 2)) and n > 40))
    return cases


@pytest.mark.parametrize("case", _random_topk_cases(), ids=lambda c: f"{c[0]}-{c[2]}-B{c[3]}")
def test_topk_random_shapes(gpu, case):
    """Bit-exact top-B on seeded random shapes, two passes over one workspace."""
    test_topk_exact(gpu, case)


def test_topk_length_beyond_max_seq_len_flags(gpu):
    ctx = gpu.Context(1, 1, 1, 64, 128, 1e4, "f32", np.zeros((1, 1), np.int32), 8)
    ws = ctx.new_workspace()
    sc = torch.zeros(1, 1, 128, dtype=torch.float32, device="cuda")
    idx = torch.zeros(1, 1, 8, dtype=torch.int32, device="cuda")
    ctx.topk(sc, torch.tensor([100], dtype=torch.int32, device="cuda"), 64, 8, idx, ws)
    assert ctx.check(ws) & gpu.DEVFLAG_SEQ_LEN
    assert np.all(idx.cpu().numpy() == -1)


# ---------------------------------------------------------------- FAC ----

@pytest.mark.parametrize("name", ["c1", "c2s", "c3s", "g1s", "g2s", "g8s", "h64s", "f128s"])
def test_sparse_attn(gpu, name):
    w, x, g, o = _prefilled(gpu, name)
    budget = w.budget
    rng = np.random.default_rng(3)
    idx = np.full((w.batch, w.n_q_heads, budget), -1, dtype=np.int32)
    for b in range(w.batch):
        nb = int(x["ctx"][b]) - 1
        for h in range(w.n_q_heads):
            k = min(budget, nb) - (h % 3)  # some heads leave -1 holes at the end
            idx[b, h, :k] = np.sort(rng.choice(nb, size=k, replace=False))
    out = torch.empty(w.batch, w.n_q_heads, w.head_dim, dtype=torch.float32, device="cuda")
    n = torch.from_numpy((x["ctx"] - 1).astype(np.int32)).cuda()
    g.ctx.sparse_attn(g.k, g.v, to_dev(x["q"][0], g.td), n, to_dev(idx, torch.int32), budget,
                      out, g.ws)
    got = out.cpu().numpy()
    assert g.ctx.check(g.ws) == 0
    for b in range(w.batch):
        nb = int(x["ctx"][b]) - 1
        o.lens[b] = nb
        qr = oracle.rope.rope_rotate(x["q"][0][b], nb - 1, w.rope_theta)
        for h in range(w.n_q_heads):
            want = o.attend(b, h, qr[h], idx[b, h])
            check_out(got[b, h], want, w.dtype, f"b{b} h{h}")


def test_sparse_attn_bad_index_flags(gpu):
    w, x, g, o = _prefilled(gpu, "c1")
    idx = np.full((1, 2, w.budget), -1, dtype=np.int32)
    idx[0, 0, 0] = 5
    idx[0, 1, 0] = 10_000  # beyond n_b
    out = torch.empty(1, 2, w.head_dim, dtype=torch.float32, device="cuda")
    n = torch.from_numpy((x["ctx"] - 1).astype(np.int32)).cuda()
    g.ctx.sparse_attn(g.k, g.v, to_dev(x["q"][0], g.td), n, to_dev(idx, torch.int32), w.budget,
                      out, g.ws)
    assert g.ctx.check(g.ws) & gpu.DEVFLAG_INDEX
    got = out.cpu().numpy()
    assert np.array_equal(got[0, 1], np.zeros(w.head_dim, np.float32))
    assert np.allclose(got[0, 0], x["v_prefill"][0, 0, 5], rtol=0, atol=1e-6)


# -------------------------------------------------------------- dense ----

@pytest.mark.parametrize("name", ["c1", "c2s", "c3s", "h64s", "f128s", "g1s", "g8s",
                                  "dm1", "dm2", "dm4", "dm8"])
def test_dense_attn(gpu, name):
    w, x, g, o = _prefilled(gpu, name)
    n = torch.from_numpy((x["ctx"] - 1).astype(np.int32)).cuda()
    out = torch.empty(w.batch, w.n_q_heads, w.head_dim, dtype=torch.float32, device="cuda")
    g.ctx.dense_attn(g.k, g.v, to_dev(x["q"][0], g.td), n, int(x["ctx"].max()), out, g.ws)
    got = out.cpu().numpy()
    assert g.ctx.check(g.ws) == 0
    for b in range(w.batch):
        nb = int(x["ctx"][b]) - 1
        o.lens[b] = nb
        qr = oracle.rope.rope_rotate(x["q"][0][b], nb - 1, w.rope_theta)
        for h in range(w.n_q_heads):
            want = o.attend(b, h, qr[h], np.arange(nb))
            check_out(got[b, h], want, w.dtype, f"b{b} h{h}")


def test_dense_empty_and_invalid_rows_in_chunk_walking_grid(gpu):
    """A grid whose workgroups walk several chunks (every split then writes a
    state and the merge reads no lengths): an empty sequence gives zeros
    without a flag, a length past max_seq_len gives zeros and the flag, and
    the other rows still match the oracle."""
    w, x, g, o = _prefilled(gpu, "dm4")
    lens = (x["ctx"] - 1).astype(np.int32)
    msl = int(lens.max())
    lens[0] = 0
    lens[1] = msl + 5
    n = torch.from_numpy(lens).cuda()
    out = torch.full((w.batch, w.n_q_heads, w.head_dim), np.nan, dtype=torch.float32,
                     device="cuda")
    g.ctx.dense_attn(g.k, g.v, to_dev(x["q"][0], g.td), n, msl, out, g.ws)
    got = out.cpu().numpy()
    assert g.ctx.check(g.ws) & gpu.DEVFLAG_SEQ_LEN
    assert np.all(got[0] == 0) and np.all(got[1] == 0)
    for b in range(2, w.batch):
        nb = int(lens[b])
        o.lens[b] = nb
        qr = oracle.rope.rope_rotate(x["q"][0][b], nb - 1, w.rope_theta)
        for h in range(0, w.n_q_heads, 5):
            check_out(got[b, h], o.attend(b, h, qr[h], np.arange(nb)), w.dtype, f"b{b} h{h}")


# -------------------------------------------------------- decode step ----

def _decode_parity(gpu, w, x, steps=None, heads=None, check_steps=None):
    g = GpuSetup(gpu, w, x)
    o = oracle_setup(w, x)
    steps = w.steps if steps is None else steps
    diffs = 0
    for t in range(steps):
        out, idx = run_decode(g, t, w.budget)
        want_steps = check_steps is None or t in check_steps
        if not want_steps:
            for b in range(w.batch):
                o.append(b, x["k_new"][t][b][:, None, :], x["v_new"][t][b][:, None, :])
            continue
        got_out, got_idx = out.cpu().numpy(), idx.cpu().numpy()
        res = o.step(x["q"][t], x["k_new"][t], x["v_new"][t], w.budget, heads=heads)
        for b in range(w.batch):
            n = int(o.lens[b])
            qr = o.query_rot(b, x["q"][t][b])
            for h in (range(w.n_q_heads) if heads is None else heads):
                where = f"step {t} b{b} h{h}"
                diffs += check_index_set(got_idx[b, h], res["scores"][(b, h)], w.budget, n, where)
                want = o.attend(b, h, qr[h], got_idx[b, h])
                check_out(got_out[b, h], want, w.dtype, where)
    assert g.ctx.check(g.ws) == 0
    # seq_lens advanced on the device by one per step
    assert np.array_equal(g.seq_lens.cpu().numpy(), (x["ctx"] - 1 + steps).astype(np.int32))
    return diffs


@pytest.mark.parametrize("name", ["c1", "c2s", "c3s", "c4s", "c5s", "g1s", "g2s", "g8s", "h64s", "f128s",
                                  "f128f", "c2m", "h64m", "f128m", "c4w"])
def test_decode_step_small(gpu, name):
    w = SMALL[name]
    _decode_parity(gpu, w, W.generate(w))


def _random_decode_workloads(count=6, seed=0xDEC):
    """Seeded small workloads: head groupings, head sizes, dtypes, partial
    RoPE, dominant-FC counts, budgets (B >= n included), ragged contexts and
    step counts drawn at random."""
    r = np.random.Generator(np.random.PCG64(seed))
    groups = [(8, 8), (8, 4), (16, 4), (16, 2), (32, 8)]
    out = []
    for i in range(count):
        hq, hkv = groups[int(r.integers(0, len(groups)))]
        d = int(r.choice([64, 128]))
        ctx = int(r.integers(600, 6001))
        ragged = bool(r.integers(0, 2))
        steps = int(r.integers(1, 3))
        budget = int(r.choice([r.integers(1, 300), r.integers(300, 1025), r.integers(1025, 3000)]))
        cap = (ctx + steps - 1 + 63) // 64 * 64  # the context's capacity bounds max_budget
        out.append(W.shrink(
            W.get("c3"), name=f"rand{i}", batch=int(r.integers(1, 4)), n_q_heads=hq,
            n_kv_heads=hkv, head_dim=d, dtype=str(r.choice(["bf16", "f32"])), context=ctx,
            context_min=ctx // 2 if ragged else None, budget=min(budget, cap),
            n_dom=int(r.integers(2, 17)), steps=steps,
            rotary_dim=(d // 2 if r.integers(0, 3) == 0 else None)))
    return out


@pytest.mark.parametrize("w", _random_decode_workloads(), ids=lambda w: w.name)
def test_decode_step_random_workloads(gpu, w):
    _decode_parity(gpu, w, W.generate(w))


def test_decode_step_c1_full(gpu):
    w = W.get("c1")
    _decode_parity(gpu, w, W.generate(w))


def test_decode_step_c2_full(gpu):
    """32k context, B = 256: every head of the single step."""
    w = W.get("c2")
    _decode_parity(gpu, w, W.generate(w))


def _full_parity(gpu, w, x, check_steps=None, threads=16):
    """Every (sequence, query head) row of the checked steps against the
    oracle, at the workload's full size, through the launch configuration
    bench.py times.  The GPU runs every step; the oracle appends every
    step's token and checks the chosen steps' rows in a thread pool (NumPy
    releases the GIL in its heavy calls)."""
    from concurrent.futures import ThreadPoolExecutor
    g = GpuSetup(gpu, w, x)
    o = oracle_setup(w, x)
    check = set(range(w.steps)) if check_steps is None else set(check_steps)
    rows = [(b, h) for b in range(w.batch) for h in range(w.n_q_heads)]
    diffs, worst = 0, 0.0
    with ThreadPoolExecutor(threads) as pool:
        for t in range(w.steps):
            out, idx = run_decode(g, t, w.budget)
            o.step(x["q"][t], x["k_new"][t], x["v_new"][t], w.budget, heads=[])  # append only
            if t not in check:
                continue
            got_idx, got_out = idx.cpu().numpy(), out.cpu().numpy()
            qrs = [o.query_rot(b, x["q"][t][b]) for b in range(w.batch)]

            def one(bh):
                b, h = bh
                n = int(o.lens[b])
                where = f"step {t} b{b} h{h}"
                s = o.head_scores(b, h, qrs[b][h])
                d = check_index_set(got_idx[b, h], s, w.budget, n, where)
                want = o.attend(b, h, qrs[b][h], got_idx[b, h])
                return d, check_out(got_out[b, h], want, w.dtype, where)

            for d, r in pool.map(one, rows):
                diffs += d
                worst = max(worst, r)
    assert g.ctx.check(g.ws) == 0
    assert np.array_equal(g.seq_lens.cpu().numpy(), (x["ctx"] - 1 + w.steps).astype(np.int32))
    return diffs, worst


@pytest.mark.timeout(600)
def test_decode_step_c3_full(gpu):
    """16 ragged sequences of 4k-8k tokens: every head of every sequence."""
    w = W.get("c3")
    _full_parity(gpu, w, W.generate(w))


@pytest.mark.timeout(900)
def test_decode_step_c4_full(gpu):
    """64 steps with append at 4 x 32k tokens, B = 6193: every head of every
    sequence at every step."""
    w = W.get("c4")
    _full_parity(gpu, w, W.generate(w))


@pytest.mark.timeout(900)
def test_decode_step_c5_full(gpu):
    """32 steps with append at 128k tokens, B = 1024: every head at every
    step."""
    w = W.get("c5")
    _full_parity(gpu, w, W.generate(w))


# -------------------------------------------------------- edge cases ----

def test_budget_at_least_context_is_dense(gpu):
    """B >= n: the step attends over everything and equals dense attention."""
    w = small("c2", context=200, budget=256)
    x = W.generate(w)
    g = GpuSetup(gpu, w, x)
    out, idx = run_decode(g, 0, 256)
    got_idx = idx.cpu().numpy()
    assert np.all(got_idx[:, :, :200] == np.arange(200)) and np.all(got_idx[:, :, 200:] == -1)
    # Against the oracle: its step with B >= n selects every token, and its
    # output is then dense attention over the whole context.
    o = oracle_setup(w, x)
    res = o.step(x["q"][0], x["k_new"][0], x["v_new"][0], 256)
    assert np.all(res["idx"][:, :, :200] == np.arange(200))
    for h in range(w.n_q_heads):
        check_out(out.cpu().numpy()[0, h], res["out"][0, h], w.dtype, f"h{h}")
    # The in-build dense kernel on the same cache meets the same oracle.
    dense = torch.empty_like(out)
    n = torch.full((1,), 200, dtype=torch.int32, device="cuda")
    g.ctx.dense_attn(g.k, g.v, to_dev(x["q"][0], g.td), n, 200, dense, g.ws)
    for h in range(w.n_q_heads):
        check_out(dense.cpu().numpy()[0, h], res["out"][0, h], w.dtype, f"dense h{h}")


def test_single_token_context(gpu):
    w = small("c1", context=1)
    x = W.generate(w)
    g = GpuSetup(gpu, w, x)
    out, idx = run_decode(g, 0, w.budget)
    assert np.all(idx.cpu().numpy()[:, :, 0] == 0)
    assert np.all(idx.cpu().numpy()[:, :, 1:] == -1)
    vn = x["v_new"][0][0, 0]
    assert np.allclose(out.cpu().numpy()[0, 0], vn, rtol=0, atol=1e-6)


def test_zero_query_selects_lowest_positions(gpu):
    """q = 0: every score is 0, ties go to the lower position, FAC averages."""
    w = small("c2", context=3000)
    x = W.generate(w)
    x["q"][:] = 0.0
    g = GpuSetup(gpu, w, x)
    out, idx = run_decode(g, 0, w.budget)
    assert np.all(idx.cpu().numpy() == np.arange(w.budget))
    o = oracle_setup(w, x)
    res = o.step(x["q"][0], x["k_new"][0], x["v_new"][0], w.budget, heads=[0, 31])
    check_out(out.cpu().numpy()[0, 0], res["out"][0, 0], "bf16")
    check_out(out.cpu().numpy()[0, 31], res["out"][0, 31], "bf16")


def test_budget_one(gpu):
    w = small("c2", context=4500, budget=1)
    x = W.generate(w)
    _decode_parity(gpu, w, x)


def test_seq_len_beyond_max_flags_and_zeroes(gpu):
    w = small("c1", context=300)
    x = W.generate(w)
    g = GpuSetup(gpu, w, x)
    out, idx = run_decode(g, 0, w.budget, max_seq_len=100)  # n_b = 300 > 100
    assert g.ctx.check(g.ws) & gpu.DEVFLAG_SEQ_LEN
    assert np.all(out.cpu().numpy() == 0) and np.all(idx.cpu().numpy() == -1)
    assert g.seq_lens.cpu().numpy()[0] == 299  # not advanced


@pytest.mark.parametrize("name", ["c2s", "g2s", "c4w"])
def test_repeat_is_bit_identical(gpu, name):
    w = SMALL[name]
    x = W.generate(w)
    g = GpuSetup(gpu, w, x)
    a_out, a_idx = run_decode(g, 0, w.budget, advance=False)
    b_out, b_idx = run_decode(g, 0, w.budget, advance=False)
    assert torch.equal(a_idx, b_idx)
    assert torch.equal(a_out, b_out)


@pytest.mark.parametrize("name", ["c2s", "g2s", "c4w"])
def test_graph_replay_matches_eager(gpu, name):
    """The decode step captured in a HIP graph, replayed several times with
    eager work in between, gives the eager result every time: the fused
    select + FAC path (c2s) and the separate select, FAC splits and merge
    path (g2s, B = 1300)."""
    w = SMALL[name]
    x = W.generate(w)
    g = GpuSetup(gpu, w, x)
    eager_out, eager_idx = run_decode(g, 0, w.budget, advance=False)
    q = to_dev(x["q"][0], g.td)
    kn = to_dev(x["k_new"][0], g.td)
    vn = to_dev(x["v_new"][0], g.td)
    out = torch.zeros_like(eager_out)
    idx = torch.zeros_like(eager_idx)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        g.ctx.decode_step(g.k, g.v, g.side, q, kn, vn, g.seq_lens, int(x["ctx"].max()),
                          w.budget, out, g.ws, idx_out=idx)
    torch.cuda.current_stream().wait_stream(s)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        g.ctx.decode_step(g.k, g.v, g.side, q, kn, vn, g.seq_lens, int(x["ctx"].max()),
                          w.budget, out, g.ws, idx_out=idx)
    for rep in range(4):
        out.zero_()
        idx.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(idx, eager_idx), rep
        assert torch.equal(out, eager_out), rep
        _ = run_decode(g, 0, w.budget, advance=False)  # eager work between replays
