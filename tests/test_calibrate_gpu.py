"""fasa_calibrate (per-FC scores, top-k, agreement) against the oracle.

Agreement counts must match the oracle's exactly, except where a top-k set
may legitimately differ: the oracle's k-th and (k+1)-th scores of that FC (or
of the full head) lie within 1e-4 of the row's largest magnitude, which fp32
summation on the GPU cannot order reliably.
"""

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from fasa_harness import GpuSetup, oracle_setup, to_dev

pytestmark = pytest.mark.gpu

CASES = {
    "c1": (W.get("c1"), 64),
    "c2s": (W.shrink(W.get("c2"), context=5003), 256),
    "c3s": (W.shrink(W.get("c3"), batch=3, context=3001, context_min=1500), 100),
    # partial RoPE: 32 rotated FCs and 32 pass-through pairs
    "c6s": (W.shrink(W.get("c6"), context=4001), 128),
}


def near_tie(s, k, rel=1e-4):
    s = np.sort(np.asarray(s, np.float64))[::-1]
    if k >= s.size:
        return False
    return s[k - 1] - s[k] <= rel * np.max(np.abs(s))


@pytest.mark.parametrize("name", list(CASES))
def test_calibrate_matches_oracle(gpu, name):
    w, topk = CASES[name]
    x = W.generate(w)
    g = GpuSetup(gpu, w, x)
    o = oracle_setup(w, x)
    q = to_dev(x["q"][0], g.td)
    ws = g.ctx.new_calibration_workspace(topk)
    C = w.head_dim // 2
    ca = torch.full((w.batch, w.n_q_heads, C), -1.0, device="cuda")
    msl = int(x["ctx"].max()) - 1
    for rep in range(2):  # the second call reuses the workspace
        g.ctx.calibrate(g.k, q, g.seq_lens, msl, topk, ca, ws)
        assert g.ctx.check(ws) == 0
    got = ca.cpu().numpy().astype(np.float64)
    want = np.zeros_like(got)
    # The oracle's agreement as the GPU reports it: count / take in fp32.
    want32 = np.zeros(got.shape, dtype=np.float32)
    mismatches = 0
    for b in range(w.batch):
        n = int(o.lens[b])
        take = min(topk, n)
        qr = o.query_rot(b, x["q"][0][b])
        for h in range(w.n_q_heads):
            K = o.K[b, h // w.group, :n]
            want[b, h] = oracle.calibrate.contextual_agreement(qr[h], K, topk, o.pairs)
            cg = np.rint(got[b, h] * take).astype(np.int64)
            cw = np.rint(want[b, h] * take).astype(np.int64)
            want32[b, h] = cw.astype(np.float32) / np.float32(take)
            bad = np.nonzero(cg != cw)[0]
            if bad.size:
                s_c = oracle.calibrate.fc_scores(qr[h], K, o.pairs)
                full_tie = near_tie(s_c.sum(axis=0), take)
                for c in bad:
                    assert full_tie or near_tie(s_c[c], take), (b, h, int(c), cg[c], cw[c])
                mismatches += bad.size
    if mismatches == 0:
        # Agreements are fractions, so equal means are common: compare the
        # choice of I_dom on the very values the GPU reported.
        assert np.array_equal(got.astype(np.float32), want32)
        assert np.array_equal(gpu.select_dominant(want32, w.n_dom),
                              oracle.calibrate.dominant_from_ca(want32.astype(np.float64),
                                                                w.n_dom))


def test_calibrate_recovers_loud_fcs(gpu):
    """Keys whose FCs 5 and 9 are ten times louder than the rest, and queries
    with a fixed large pair on those FCs, make the two FCs carry every head's
    ranking: calibration must pick them for every head."""
    # No planted keys: they would favour the workload's own dominant FCs.
    w = W.shrink(W.get("c2"), context=3000, batch=2, planted_frac=0.0)
    x = W.generate(w)
    half = w.head_dim // 2
    for c in (5, 9):
        x["k_prefill"][..., c] *= 10.0
        x["k_prefill"][..., c + half] *= 10.0
        x["q"][..., c] = 2.0
        x["q"][..., c + half] = 1.0
    x["k_prefill"] = W.round_bf16(x["k_prefill"])
    g = GpuSetup(gpu, w, x)
    topk = 64
    ws = g.ctx.new_calibration_workspace(topk)
    ca = torch.zeros(w.batch, w.n_q_heads, half, device="cuda")
    g.ctx.calibrate(g.k, to_dev(x["q"][0], g.td), g.seq_lens, int(x["ctx"].max()) - 1, topk,
                    ca, ws)
    assert g.ctx.check(ws) == 0
    dom = gpu.select_dominant(ca.cpu().numpy(), 2)
    assert np.all(dom == np.array([5, 9])), dom
