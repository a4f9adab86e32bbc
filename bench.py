"""Benchmark of the FASA decode step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config c2] [--layers L]

Workload (default): a Llama-3-8B-shaped attention layer, one decode step at
32768 tokens of context with B = 256 and 16 dominant FCs per query head
(32 query heads on 8 KV heads, d = 128, bf16 caches, RoPE theta 5e5).  Inputs
are seeded synthetic data (workloads/); they stand in for the LongBench-V1
setting the pages quote at 256 retained tokens.

A step is one fasa_decode_step (append + query rotation, TIP, top-B, FAC) on
one layer's cache.  Steps rotate over L distinct layer caches (16 by default,
about 2.9 GB) so that the 256 MB Infinity Cache cannot serve a repeated
layer, as in a real multi-layer decode.  The timed steps are replayed from a
HIP graph of L steps; inputs are resident in HBM before timing starts.

Printed: one JSON line with the metric (context tokens scanned per second),
the fraction of HBM peak on the algorithmic bytes, the dominant kernel's
roofline figure (TIP: sidecar bytes read / its average duration from HIP
events over back-to-back launches), the in-build dense
decode comparator, the step with K/V caches in pinned host memory (FASA-M),
the measured copy bandwidth of the GPU, and the CPU oracle baseline on a
bounded sample (one core, and all cores up to 16).
"""

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = "context tokens scanned/s per decode step + % HBM peak (32k ctx, B=256)"


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=480)
    p.add_argument("--warmup", type=int, default=32)
    p.add_argument("--config", default="c2")
    p.add_argument("--layers", type=int, default=16)
    p.add_argument("--cpu-seconds", type=float, default=15.0,
                   help="CPU oracle sample budget (0 disables)")
    p.add_argument("--no-dense", action="store_true")
    p.add_argument("--eager", action="store_true", help="time eager launches, no graph")
    p.add_argument("--no-calibration", action="store_true",
                   help="skip timing fasa_calibrate (offline I_dom calibration)")
    p.add_argument("--step-only", action="store_true",
                   help="time only the step, its TIP kernel and the dense comparator: no "
                        "calibration, per-head, partial-RoPE or FASA-M fields (for profiling "
                        "the step's own kernels)")
    p.add_argument("--no-partial-rope", action="store_true",
                   help="skip timing the partial-RoPE layer")
    p.add_argument("--no-per-head", action="store_true",
                   help="skip timing the step with a budget per query head")
    p.add_argument("--no-fasa-m", action="store_true",
                   help="skip timing the step with K/V caches in pinned host memory")
    p.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                   help="only run 4 plain device-to-device copies of MIB MiB (the "
                        "reference kernel for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE)")
    return p.parse_args()


def copy_probe(mib):
    import torch
    n = mib << 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(4):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": n, "copies": 4}), flush=True)


def source_code_hash(paths):
    """sha256 of C/C++ sources with comments and blank space removed, so that
    only a change of the code itself changes it."""
    import re
    h = hashlib.sha256()
    for p in paths:
        with open(p) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        for line in text.splitlines():
            line = " ".join(line.split())
            if line:
                h.update(line.encode() + b"\n")
    return h.hexdigest()


def tip_kernel_name(w):
    """The TIP kernel the library launches for this shape: one wave per query
    head when a KV head serves 4 or 8 of them and each has at most 16
    dominant FCs, else the union kernel."""
    g = w.n_q_heads // w.n_kv_heads
    return "tip_head_kernel" if g in (4, 8) and w.n_dom <= 16 else "tip_kernel"


def traffic_from_profile():
    """HBM bytes per TIP launch from the committed rocprofv3 --pmc summary, if
    it was taken on the current kernel code (comments aside); else None."""
    path = os.path.join(ROOT, "profiles", "tip_c2_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        prof = json.load(f)
    srcs = [os.path.join(ROOT, rel) for rel in prof.get("sources", [])]
    if not srcs or not all(os.path.exists(p) for p in srcs):
        return None
    if prof.get("source_code_sha256") != source_code_hash(srcs):
        return None
    return prof.get("hbm_bytes_per_launch")


def calibration_timing(ctx, k_cache, q, seq_full, msl, w, reps, topk=256):
    """fasa_calibrate on one layer of the workload (each sequence one
    calibration sample): HIP events around `reps` back-to-back calls."""
    import torch
    ws = ctx.new_calibration_workspace(topk)
    ca = torch.zeros(w.batch, w.n_q_heads, w.head_dim // 2, dtype=torch.float32,
                     device=q.device)
    for _ in range(2):
        ctx.calibrate(k_cache, q, seq_full, msl, topk, ca, ws)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = max(4, min(reps, 32))
    e0.record()
    for _ in range(reps):
        ctx.calibrate(k_cache, q, seq_full, msl, topk, ca, ws)
    e1.record()
    torch.cuda.synchronize()
    assert ctx.check(ws) == 0
    ms = e0.elapsed_time(e1) / reps
    n = int(seq_full.sum().item())
    C = w.head_dim // 2
    es = 2 if w.dtype == "bf16" else 4
    # K rows read once per KV head, every FC score row written once.
    score_bytes = n * w.n_q_heads * (C + 1) * 4
    k_bytes = n * w.n_kv_heads * w.head_dim * es
    return {"topk": topk, "ms_per_call": ms, "samples_per_call": w.batch,
            "score_rows_per_sample": w.n_q_heads * (C + 1),
            "k_plus_score_bytes": k_bytes + score_bytes,
            "gbps_on_those_bytes": (k_bytes + score_bytes) / (ms * 1e-3) / 1e9}


def fasa_m_timing(ctx, w, x, q, kn, vn, seq, seq_full, msl, reps, with_dense):
    """FASA-M: one layer with its K and V caches in pinned host memory (the
    device reaches them over the host link), the sidecar in HBM.  HIP events
    around `reps` back-to-back decode steps, and around dense decode over the
    same host-resident caches for comparison."""
    import torch
    dev = q.device
    k, v, side = ctx.new_cache(kv_on_host=True)
    ws = ctx.new_workspace()
    td = k.dtype
    zero = torch.zeros(w.batch, dtype=torch.int32, device=dev)
    ctx.append_kv(k, v, side, torch.from_numpy(x["k_prefill"]).to(dev, td),
                  torch.from_numpy(x["v_prefill"]).to(dev, td), zero, ws)
    out = torch.empty(w.batch, w.n_q_heads, w.head_dim, dtype=torch.float32, device=dev)
    idx = torch.empty(w.batch, w.n_q_heads, w.budget, dtype=torch.int32, device=dev)

    def run(fn, n):
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    ms = run(lambda: ctx.decode_step(k, v, side, q, kn, vn, seq, msl, w.budget, out, ws,
                                     idx_out=idx), max(8, min(reps, 64)))
    assert ctx.check(ws) == 0
    es = k.element_size()
    n_b = x["ctx"].astype(np.int64)
    # Host-link bytes of a step: the B selected K and V rows per query head
    # (FAC) and the appended K and V rows.
    link = int(sum(min(w.budget, n) for n in n_b)) * 2 * w.head_dim * es * w.n_q_heads \
        + w.batch * w.n_kv_heads * 2 * w.head_dim * es
    kv_bytes = 2 * k.numel() * es
    res = {"ms_per_step": ms, "value": float(n_b.sum()) / (ms * 1e-3),
           "unit": "context tokens/s", "host_link_bytes_per_step": link,
           "host_link_gbps": link / (ms * 1e-3) / 1e9,
           "device_bytes_per_layer": ctx.sidecar_bytes,
           "device_bytes_per_layer_fasa_c": ctx.sidecar_bytes + kv_bytes,
           "device_kv_compression": (ctx.sidecar_bytes + kv_bytes) / ctx.sidecar_bytes,
           "host_bytes_per_layer": kv_bytes}
    # The link's yardstick: one streaming read pass over the host-resident K
    # cache (large contiguous reads), next to the step's gather of scattered
    # rows over the same link.
    import sparse_kv_cache_rope_amd as fasa_lib
    sink = torch.zeros(1, device=dev)
    probe_ms = run(lambda: fasa_lib.read_probe(k, sink), 4)
    k_bytes = k.numel() * es
    res["host_link_read_probe_gbps"] = k_bytes / (probe_ms * 1e-3) / 1e9
    res["host_link_read_probe_bytes"] = k_bytes
    res["host_link_gather_frac_of_read_probe"] = (res["host_link_gbps"]
                                                  / res["host_link_read_probe_gbps"])
    if with_dense:
        dense_out = torch.empty_like(out)
        res["dense_from_host_ms"] = run(
            lambda: ctx.dense_attn(k, v, q, seq_full, msl, dense_out, ws), 4)
        res["sparse_speedup_from_host"] = res["dense_from_host_ms"] / ms
    del k, v
    return res


def per_head_timing(fasa, w, x, layers, q, kn, vn, seq, msl, dev, reps):
    """Budgets per query head: a linear allocation over the heads (head h gets
    round(2B (h + 0.5) / Hq), mean B, at most 2B) on the same rotated layers,
    replayed from a HIP graph like the uniform step."""
    import torch
    import workloads as W
    top = 2 * w.budget
    ctx2 = fasa.Context(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.capacity,
                        w.rope_theta, w.dtype, x["dom"], top, device=dev)
    ws2 = ctx2.new_workspace()
    hb = W.head_budgets(0, w.n_q_heads, top, "ramp")
    hb_d = torch.from_numpy(hb).to(dev)
    out = torch.empty(w.batch, w.n_q_heads, w.head_dim, dtype=torch.float32, device=dev)
    idx = torch.empty(w.batch, w.n_q_heads, top, dtype=torch.int32, device=dev)
    L = len(layers)

    def one(i):
        k, v, sd = layers[i % L]
        ctx2.decode_step(k, v, sd, q, kn, vn, seq, msl, top, out, ws2, idx_out=idx,
                         head_budgets=hb_d)

    for i in range(L):
        one(i)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for i in range(L):
            one(i)
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(L):
            one(i)
    g.replay()
    torch.cuda.synchronize()
    n_rep = max(1, reps // L)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(n_rep):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    assert ctx2.check(ws2) == 0
    got = (idx.cpu().numpy() >= 0).sum(axis=2)
    assert np.array_equal(got, np.minimum(hb[None, :], x["ctx"][:, None]))
    ms = e0.elapsed_time(e1) / (n_rep * L)
    return {"allocation": "linear over heads, round(2B (h + 0.5) / Hq)", "mean_budget":
            float(hb.mean()), "min_budget": int(hb.min()), "max_budget": int(hb.max()),
            "ms_per_step": ms, "value": float(x["ctx"].sum()) / (ms * 1e-3),
            "unit": "context tokens/s"}


def partial_rope_timing(fasa, dev, L, reps):
    """The 32k partial-RoPE layer (rotary_dim 64 of 128): the same decode step
    over L rotated layer caches, replayed from a HIP graph, and its TIP kernel
    back-to-back."""
    import torch
    import workloads as W
    w = W.get("c6")
    x = W.generate(w)
    td = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    to = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev, td)
    ctx = fasa.Context(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.capacity,
                       w.rope_theta, w.dtype, x["dom"], w.budget, device=dev,
                       rotary_dim=w.rotary_dim)
    ws = ctx.new_workspace()
    layers = [ctx.new_cache() for _ in range(L)]
    kp, vp = to(x["k_prefill"]), to(x["v_prefill"])
    zero = torch.zeros(w.batch, dtype=torch.int32, device=dev)
    for (k, v, sd) in layers:
        ctx.append_kv(k, v, sd, kp, vp, zero, ws)
    del kp, vp
    seq = torch.from_numpy((x["ctx"] - 1).astype(np.int32)).to(dev)
    msl = int(x["ctx"].max())
    q, kn, vn = to(x["q"][0]), to(x["k_new"][0]), to(x["v_new"][0])
    out = torch.empty(w.batch, w.n_q_heads, w.head_dim, dtype=torch.float32, device=dev)
    idx = torch.empty(w.batch, w.n_q_heads, w.budget, dtype=torch.int32, device=dev)
    scores = torch.empty(w.batch, w.n_q_heads, w.capacity, dtype=torch.float32, device=dev)
    seq_full = seq + 1

    def one(i):
        k, v, sd = layers[i % L]
        ctx.decode_step(k, v, sd, q, kn, vn, seq, msl, w.budget, out, ws, idx_out=idx)

    for i in range(L):
        one(i)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for i in range(L):
            one(i)
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(L):
            one(i)
    g.replay()
    torch.cuda.synchronize()
    n_rep = max(1, reps // L)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(n_rep):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / (n_rep * L)
    e0.record()
    for i in range(n_rep * L):
        ctx.tip_scores(layers[i % L][2], q, seq_full, msl, scores, ws)
    e1.record()
    torch.cuda.synchronize()
    tip_ms = e0.elapsed_time(e1) / (n_rep * L)
    assert ctx.check(ws) == 0
    es = 2 if w.dtype == "bf16" else 4
    off, _ = ctx.sidecar_layout()
    n = int(x["ctx"].sum())
    tip_bytes = int(off[-1]) * 2 * es * n  # sidecar pairs read
    del layers
    return {"workload": w.name, "rotary_dim": w.rotary_dim, "ms_per_step": ms,
            "value": n / (ms * 1e-3), "unit": "context tokens/s", "tip_kernel_avg_ms": tip_ms,
            "tip_gbps": tip_bytes / (tip_ms * 1e-3) / 1e9}


def cpu_baseline(w, x, budget_s):
    """The oracle (fp64 NumPy, one thread) on consecutive decode steps of the
    same workload until ~budget_s seconds of step time are spent."""
    import oracle
    from threadpoolctl import threadpool_limits

    with threadpool_limits(limits=1):
        st = oracle.OracleState(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.rope_theta,
                                w.dtype, x["dom"], w.capacity + 4096)
        for b in range(w.batch):
            n0 = int(x["ctx"][b]) - 1
            st.append(b, x["k_prefill"][b][:, :n0], x["v_prefill"][b][:, :n0])
        spent, steps, tokens = 0.0, 0, 0
        while spent < budget_s and steps < 4096:
            t = steps % w.steps
            t0 = time.perf_counter()
            st.step(x["q"][t], x["k_new"][t], x["v_new"][t], w.budget)
            spent += time.perf_counter() - t0
            tokens += int(st.lens.sum())
            steps += 1
    return {"value": tokens / spent, "unit": "context tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"{steps} consecutive decode steps of the same workload (all "
                      f"{w.n_q_heads} query heads, append + TIP + top-B + FAC), fp64 NumPy "
                      f"on one host thread, {spent:.1f} s of step time, prefill excluded"}


# Oracle state shared with forked workers (set before the fork).
_POOL_STATE = {}


def _oracle_worker(heads):
    """Runs the oracle's decode steps for `heads` only (a forked copy of the
    prefilled state); returns (steps, seconds)."""
    from threadpoolctl import threadpool_limits
    st, x, w, n_steps = (_POOL_STATE[k] for k in ("st", "x", "w", "steps"))
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        for s in range(n_steps):
            t = s % w.steps
            st.step(x["q"][t], x["k_new"][t], x["v_new"][t], w.budget, heads=heads)
        return n_steps, time.perf_counter() - t0


def cpu_baseline_all_cores(w, x, budget_s):
    """The oracle on all host cores this process may use (at most 16): one
    forked worker per share of the query heads, each running the same
    consecutive decode steps over its heads.  Must run before the GPU is
    touched (the workers are forked)."""
    import multiprocessing as mp
    import oracle
    cores = max(1, min(16, len(os.sched_getaffinity(0)), w.n_q_heads))
    st = oracle.OracleState(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.rope_theta,
                            w.dtype, x["dom"], w.capacity + 4096)
    for b in range(w.batch):
        n0 = int(x["ctx"][b]) - 1
        st.append(b, x["k_prefill"][b][:, :n0], x["v_prefill"][b][:, :n0])
    tokens_per_step = int(x["ctx"].sum())
    # Size the run from one step of one worker's share.
    share = [list(range(i, w.n_q_heads, cores)) for i in range(cores)]
    _POOL_STATE.update(st=st, x=x, w=w, steps=1)
    _, t1 = _oracle_worker(share[0])
    steps = max(1, int(budget_s / max(t1, 1e-6)))
    _POOL_STATE["steps"] = steps
    with mp.get_context("fork").Pool(cores) as pool:
        res = pool.map(_oracle_worker, share)
    slowest = max(t for _, t in res)
    return {"value": steps * tokens_per_step / slowest, "unit": "context tokens/s",
            "cores": cores, "kind": "oracle",
            "sample": f"{steps} consecutive decode steps of the same workload, the "
                      f"{w.n_q_heads} query heads split over {cores} forked processes (one "
                      f"thread each, append + TIP + top-B + FAC per process), rate from the "
                      f"slowest process, prefill excluded"}


def bw_probe(dev, mib=1024, reps=10):
    """Measured copy bandwidth of this GPU: a plain device-to-device copy of
    `mib` MiB, read + write bytes over HIP events."""
    import torch
    n = mib << 20
    src = torch.ones(n, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del src, dst
    return 2 * n / (ms * 1e-3) / 1e9


def read_probe_at(fasa, dev, nbytes, layers=16, reps=160):
    """GB/s of a plain streaming read (fasa_read_probe) of `nbytes`, back to
    back over `layers` rotating buffers (more bytes than the Infinity Cache
    holds), over HIP events: what HBM gives a kernel that only streams that
    many bytes, the yardstick next to TIP's launch of the same size."""
    import torch
    n = (int(nbytes) + 15) // 16 * 16
    bufs = [torch.zeros(n, dtype=torch.uint8, device=dev) for _ in range(layers)]
    sink = torch.zeros(1, dtype=torch.float32, device=dev)
    for i in range(layers):
        fasa.read_probe(bufs[i], sink)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(reps):
        fasa.read_probe(bufs[i % layers], sink)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del bufs
    return n / (ms * 1e-3) / 1e9, ms


def main():
    args = parse()
    if args.step_only:
        args.no_calibration = args.no_per_head = args.no_partial_rope = args.no_fasa_m = True
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: the library has no multi-GPU path "
              "(the decode step shards by sequence / KV head with no exchange).",
              file=sys.stderr)
        sys.exit(2)

    if args.copy_probe > 0:
        copy_probe(args.copy_probe)
        return

    import workloads as W

    w = W.get(args.config)
    x = W.generate(w)
    # The CPU legs run first: the all-cores one forks, before any GPU use.
    cpu = cpu_all = None
    if args.cpu_seconds > 0:
        cpu = cpu_baseline(w, x, args.cpu_seconds)
        cpu_all = cpu_baseline_all_cores(w, x, args.cpu_seconds)

    import torch
    import sparse_kv_cache_rope_amd as fasa

    torch.cuda.set_device(0)
    dev = torch.device("cuda", 0)
    L = max(1, args.layers)
    td = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    to = lambda a, dt=td: torch.from_numpy(np.ascontiguousarray(a)).to(dev, dt)

    ctx = fasa.Context(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.capacity,
                       w.rope_theta, w.dtype, x["dom"], w.budget, device=dev)
    ws = ctx.new_workspace()
    layers = [ctx.new_cache() for _ in range(L)]
    kp, vp = to(x["k_prefill"]), to(x["v_prefill"])
    zero = torch.zeros(w.batch, dtype=torch.int32, device=dev)
    for (k, v, s) in layers:
        ctx.append_kv(k, v, s, kp, vp, zero, ws)
    del kp, vp
    seq = torch.from_numpy((x["ctx"] - 1).astype(np.int32)).to(dev)
    n_b = x["ctx"].astype(np.int64)  # tokens attended by the timed step
    msl = int(n_b.max())
    q, kn, vn = to(x["q"][0]), to(x["k_new"][0]), to(x["v_new"][0])
    out = torch.empty(w.batch, w.n_q_heads, w.head_dim, dtype=torch.float32, device=dev)
    idx = torch.empty(w.batch, w.n_q_heads, w.budget, dtype=torch.int32, device=dev)
    dense_out = torch.empty_like(out)
    seq_full = seq + 1

    def step(i):
        k, v, s = layers[i % L]
        ctx.decode_step(k, v, s, q, kn, vn, seq, msl, w.budget, out, ws, idx_out=idx)

    def dense(i):
        k, v, _ = layers[i % L]
        ctx.dense_attn(k, v, q, seq_full, msl, dense_out, ws)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    assert ctx.check(ws) == 0

    # Exactly --steps timed steps, layer i % L for step i: `reps` replays of
    # a graph over all L layers, then one graph over the first K % L.
    K = max(1, args.steps)
    reps, rem = divmod(K, L)

    def capture(fn, count):
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for i in range(count):
                fn(i)
        torch.cuda.current_stream().wait_stream(side)
        with torch.cuda.graph(g):
            for i in range(count):
                fn(i)
        g.replay()
        torch.cuda.synchronize()
        return g

    def timed(fn, use_graph):
        if use_graph:
            g = capture(fn, L) if reps else None
            g_rem = capture(fn, rem) if rem else None
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        if use_graph:
            for _ in range(reps):
                g.replay()
            if g_rem is not None:
                g_rem.replay()
        else:
            for i in range(K):
                fn(i)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / K

    use_graph = not args.eager
    ms_step = timed(step, use_graph)
    ms_step_eager = timed(step, False) if use_graph else ms_step
    # Warm figure, labelled as such: one layer's cache stepped over and over,
    # so much of it may stay in the 256 MB Infinity Cache.
    e0w, e1w = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0w.record()
    for _ in range(K):
        step(0)
    e1w.record()
    torch.cuda.synchronize()
    ms_step_warm = e0w.elapsed_time(e1w) / K
    assert ctx.check(ws) == 0
    ms_dense = None if args.no_dense else timed(dense, use_graph)

    # Dominant kernel (TIP): HIP events on the launch stream around R rounds of
    # back-to-back launches over the rotated layers, so the average holds no
    # event or dispatch gaps.  These are query-mode launches of the same kernel
    # (same grid, same sidecar and score bytes as in the step, without the
    # step's one-token append).
    scores_buf = torch.empty(w.batch, w.n_q_heads, w.capacity, dtype=torch.float32, device=dev)

    def tip_only(i):
        ctx.tip_scores(layers[i % L][2], q, seq_full, msl, scores_buf, ws)

    for i in range(L):
        tip_only(i)
    torch.cuda.synchronize()
    tip_n = max(K, 8 * L)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(tip_n):
        tip_only(i)
    e1.record()
    torch.cuda.synchronize()
    tip_ms = e0.elapsed_time(e1) / tip_n
    assert ctx.check(ws) == 0

    # Per-kernel breakdown of the step: HIP events around every launch, eager,
    # same rotation (each figure includes one event + dispatch gap).
    ctx.timing_enable(True)
    fams = {}

    def add(part):
        for f, (ms, n) in part.items():
            a = fams.get(f, (0.0, 0))
            fams[f] = (a[0] + ms, a[1] + n)

    for i in range(K):
        step(i)
        if (i + 1) % 256 == 0:
            add(ctx.timing_collect())
    add(ctx.timing_collect())
    ctx.timing_enable(False)
    kernel_ms = {f: ms / n for f, (ms, n) in fams.items() if n}

    # Algorithmic bytes of a step: the sidecar pairs TIP reads (P planes x 2
    # elements per token), the B selected K and V rows FAC reads per query
    # head (B * 2 * d elements), and the step's appended K, V and sidecar
    # entries.  Score, candidate and index traffic between the step's kernels
    # is overhead, reported on its own.
    es = 2 if w.dtype == "bf16" else 4
    off, _ = ctx.sidecar_layout()
    P = int(off[-1])
    sidecar_bytes = int(sum(P * 2 * es * n for n in n_b))
    fac_bytes = int(sum(min(w.budget, n) * 2 * w.head_dim * es * w.n_q_heads for n in n_b))
    append_bytes = w.batch * (w.n_kv_heads * 2 * w.head_dim * es + P * 2 * es)
    algo_bytes = sidecar_bytes + fac_bytes + append_bytes
    overhead_bytes = int(sum(w.n_q_heads * 4 * n for n in n_b)) \
        + w.batch * w.n_q_heads * w.budget * 4
    dense_bytes = int(sum(2 * n * w.head_dim * es * w.n_kv_heads for n in n_b))
    t_step = ms_step * 1e-3
    tokens = int(n_b.sum())
    tip_s = tip_ms * 1e-3
    achieved = sidecar_bytes / tip_s / 1e9
    traffic = traffic_from_profile() if args.config == "c2" else None
    copy_peak = bw_probe(dev)
    read_gbps, read_ms = read_probe_at(fasa, dev, sidecar_bytes)

    res = {
        "metric": METRIC,
        "value": tokens / t_step,
        "unit": "context tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded N(0,1) q/k/v with planted salient keys; stands in for LongBench-V1 at B=256)",
        "config": {"workload": w.name, "batch": w.batch, "n_q_heads": w.n_q_heads,
                   "n_kv_heads": w.n_kv_heads, "head_dim": w.head_dim,
                   "context": int(n_b.max()), "budget": w.budget, "n_dom": w.n_dom,
                   "rope_theta": w.rope_theta, "layers_rotated": L,
                   "launch": "hipgraph" if use_graph else "eager"},
        "hbm_peak_frac": algo_bytes / t_step / (HBM_PEAK_GBS * 1e9),
        "algorithmic_bytes_per_step": algo_bytes,
        "algorithmic_bytes_parts": {"sidecar": sidecar_bytes, "fac_rows": fac_bytes,
                                    "append": append_bytes},
        "overhead_bytes_per_step": overhead_bytes,
        "overhead_bytes_what": "fp32 TIP scores written (one per query head and token) "
                               "and the int32 index rows written; not algorithmic",
        "decode_steps_per_s": 1.0 / t_step,
        "head_tokens_per_s": tokens * w.n_q_heads / t_step,
        "achieved_gbps_algorithmic": algo_bytes / t_step / 1e9,
        "measured_copy_peak_gbps": copy_peak,
        "hbm_measured_peak_frac": algo_bytes / t_step / (copy_peak * 1e9),
        "ms_per_step_warm_single_cache_eager": ms_step_warm,
        "ms_per_step_eager": ms_step_eager,
        "kernel_avg_ms_with_event_gaps": kernel_ms,
        "roofline": {"bound": "hbm", "kernel": tip_kernel_name(w), "kernel_avg_ms": tip_ms,
                     "kernel_launches_timed": tip_n,
                     "achieved": achieved,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                     "traffic": traffic, "algorithmic_bytes_per_launch": sidecar_bytes,
                     "algorithmic_bytes_what": "sidecar pairs read; the launch also writes "
                                               "the fp32 scores (overhead)",
                     "frac_of_measured_copy_peak": achieved / copy_peak,
                     "plain_read_same_bytes_ms": read_ms,
                     "plain_read_same_bytes_gbps": read_gbps,
                     "frac_of_plain_read_same_bytes": achieved / read_gbps},
    }
    if not args.no_calibration:
        res["calibration"] = calibration_timing(ctx, layers[0][0], q, seq_full, msl, w, K)
    if not args.no_per_head and 2 * w.budget <= w.capacity:
        res["per_head_budgets"] = per_head_timing(fasa, w, x, layers, q, kn, vn, seq, msl, dev,
                                                  K)
    if not args.no_partial_rope:
        res["partial_rope"] = partial_rope_timing(fasa, dev, L, K)
    if not args.no_fasa_m:
        res["fasa_m"] = fasa_m_timing(ctx, w, x, q, kn, vn, seq, seq_full, msl, K,
                                      not args.no_dense)
    if ms_dense is not None:
        res["dense"] = {"ms_per_step": ms_dense, "bytes_per_step": dense_bytes,
                        "hbm_gbps": dense_bytes / (ms_dense * 1e-3) / 1e9,
                        "sparse_speedup": ms_dense / ms_step}
    if cpu is not None:
        res["cpu_baseline"] = cpu
        res["cpu_baseline_all_cores"] = cpu_all
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
