"""Shared set-up and acceptance rules for the GPU parity tests.

Acceptance rules (the project's stated bar):
* index sets: |S| = min(B, n), no duplicates, every entry in [0, n), listed
  ascending and padded with -1; every position where the GPU's set and the
  oracle's set differ has an oracle score within 1e-3 * |tau| of tau, the
  oracle's B-th largest score;
* attention outputs, recomputed by the oracle on the GPU's own set:
  |delta| <= 1e-3 + 2e-3 |o| for bf16 inputs, <= 1e-5 + 1e-5 |o| for fp32;
* TIP scores: |delta| <= 1e-5 * sum_c |terms| (fp32 summation of at most
  2 * n_dom products, each rounded once, has error below 2n * 2^-24 of that
  sum; 1e-5 leaves margin).
"""

import numpy as np
import torch

import oracle
import workloads as W

OUT_TOL = {"bf16": (1e-3, 2e-3), "f32": (1e-5, 1e-5)}


def torch_dtype(w):
    return torch.bfloat16 if w.dtype == "bf16" else torch.float32


def to_dev(a, dtype, device="cuda"):
    return torch.from_numpy(np.ascontiguousarray(a)).to(device=device, dtype=dtype)


class GpuSetup:
    """Context, caches and workspace for workload ``w`` with inputs ``x``,
    prefilled with ctx[b] - 1 tokens per sequence."""

    def __init__(self, fasa, w, x, max_budget=None, capacity=None, kv_on_host=False):
        self.w, self.x = w, x
        self.cap = capacity or w.capacity
        self.ctx = fasa.Context(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, self.cap,
                                w.rope_theta, w.dtype, x["dom"], max_budget or w.budget,
                                rotary_dim=w.rotary_dim)
        self.k, self.v, self.side = self.ctx.new_cache(kv_on_host=kv_on_host)
        self.ws = self.ctx.new_workspace()
        self.td = torch_dtype(w)
        L = x["k_prefill"].shape[2]
        if L > 0:
            kp = to_dev(x["k_prefill"], self.td)
            vp = to_dev(x["v_prefill"], self.td)
            start = torch.zeros(w.batch, dtype=torch.int32, device="cuda")
            self.ctx.append_kv(self.k, self.v, self.side, kp, vp, start, self.ws)
        self.seq_lens = torch.from_numpy((x["ctx"] - 1).astype(np.int32)).cuda()

    def k_as_f64(self):
        return self.k.float().double().cpu().numpy()

    def v_as_f64(self):
        return self.v.float().double().cpu().numpy()


def oracle_setup(w, x, capacity=None):
    st = oracle.OracleState(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.rope_theta,
                            w.dtype, x["dom"], capacity or w.capacity, rotary_dim=w.rotary_dim)
    for b in range(w.batch):
        n0 = int(x["ctx"][b]) - 1
        st.append(b, x["k_prefill"][b][:, :n0], x["v_prefill"][b][:, :n0])
    return st


def check_index_set(idx_row, scores_oracle, budget, n, where=""):
    """Applies the index-set rule to one (b, h) row; raises AssertionError."""
    idx_row = np.asarray(idx_row)
    take = min(budget, n)
    got = idx_row[:take]
    assert np.all(idx_row[take:] == -1), f"{where}: padding is not -1"
    assert np.all(got >= 0) and np.all(got < n), f"{where}: index out of range"
    assert np.all(np.diff(got) > 0), f"{where}: not strictly ascending"
    want = oracle.select.select_topb(scores_oracle, budget)[:take]
    diff = np.setxor1d(got, want)
    if diff.size:
        tau = oracle.select.threshold(scores_oracle, budget)
        bad = diff[np.abs(scores_oracle[diff] - tau) > 1e-3 * abs(tau)]
        assert bad.size == 0, (f"{where}: {bad.size} disagreeing positions outside the "
                               f"tau band (tau={tau}), e.g. {bad[:5]}")
    return diff.size


def check_out(got, want, dtype, where=""):
    atol, rtol = OUT_TOL[dtype]
    err = np.abs(np.asarray(got, np.float64) - want)
    lim = atol + rtol * np.abs(want)
    bad = err > lim
    assert not bad.any(), (f"{where}: {bad.sum()} outputs out of tolerance, worst "
                           f"{float((err - lim).max()):.3e} over")
    return float((err / lim).max()) if err.size else 0.0


def tip_bound(q_rot, k_rot, dom, pairs=None):
    half = q_rot.shape[-1] // 2
    dom = np.asarray(dom)
    if pairs is None:
        cols = np.concatenate([dom, dom + half])
    else:
        cols = np.concatenate([pairs[0][dom], pairs[1][dom]])
    return np.abs(k_rot[:, cols]) @ np.abs(q_rot[cols])


def ulp_diff_bf16(a, b):
    """Per-element distance in bf16 units of the last place (a, b exactly bf16)."""
    ia = (np.asarray(a, np.float32).view(np.int32) >> 16).astype(np.int64)
    ib = (np.asarray(b, np.float32).view(np.int32) >> 16).astype(np.int64)
    ia = np.where(ia < 0, -(ia & 0x7FFF), ia)
    ib = np.where(ib < 0, -(ib & 0x7FFF), ib)
    return np.abs(ia - ib)


def run_decode(setup, step, budget, idx=True, advance=True, max_seq_len=None):
    w, x = setup.w, setup.x
    q = to_dev(x["q"][step], setup.td)
    kn = to_dev(x["k_new"][step], setup.td)
    vn = to_dev(x["v_new"][step], setup.td)
    out = torch.empty(w.batch, w.n_q_heads, w.head_dim, dtype=torch.float32, device="cuda")
    ix = torch.empty(w.batch, w.n_q_heads, budget, dtype=torch.int32, device="cuda") if idx else None
    msl = max_seq_len or int(x["ctx"].max()) + w.steps - 1
    setup.ctx.decode_step(setup.k, setup.v, setup.side, q, kn, vn, setup.seq_lens, msl, budget,
                          out, setup.ws, idx_out=ix, advance=advance)
    return out, ix
