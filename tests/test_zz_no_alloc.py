"""fasa_decode_step_static, the decode step that allocates nothing (its
workspace is the library's own per-GPU array), against fasa_decode_step with
a caller workspace: two calls in a row on different contexts, the second
with a smaller input, each bit-identical to the workspace call on the same
caches, with its device flags delivered; and a context too large for the
array refused before anything runs."""

import numpy as np
import pytest
import torch

import workloads as W
from fasa_harness import GpuSetup, to_dev

pytestmark = pytest.mark.gpu


def _compare(gpu, w):
    x = W.generate(w)
    g = GpuSetup(gpu, w, x)
    assert g.ctx.workspace_bytes <= gpu.STATIC_SCRATCH_BYTES
    q, kn, vn = (to_dev(x[k][0], g.td) for k in ("q", "k_new", "v_new"))
    msl = int(x["ctx"].max())
    shape = (w.batch, w.n_q_heads, w.head_dim)
    out_ws = torch.full(shape, 7.0, dtype=torch.float32, device="cuda")
    idx_ws = torch.full((w.batch, w.n_q_heads, w.budget), -7, dtype=torch.int32, device="cuda")
    g.ctx.decode_step(g.k, g.v, g.side, q, kn, vn, g.seq_lens, msl, w.budget, out_ws, g.ws,
                      idx_out=idx_ws)
    assert g.ctx.check(g.ws) == 0
    out_st = torch.full(shape, -7.0, dtype=torch.float32, device="cuda")
    idx_st = torch.full_like(idx_ws, -9)
    flags = torch.full((1,), 123, dtype=torch.int32, device="cuda")
    g.ctx.decode_step_static(g.k, g.v, g.side, q, kn, vn, g.seq_lens, msl, w.budget, out_st,
                             idx_out=idx_st, dev_flags=flags)
    torch.cuda.synchronize()
    assert int(flags.item()) == 0
    assert torch.equal(idx_st, idx_ws)
    assert torch.equal(out_st, out_ws)
    # The static call advances seq_lens like the workspace call when asked.
    before = g.seq_lens.clone()
    g.ctx.decode_step_static(g.k, g.v, g.side, q, kn, vn, g.seq_lens, msl, w.budget, out_st,
                             idx_out=idx_st, advance=True)
    torch.cuda.synchronize()
    assert torch.equal(g.seq_lens, before + 1)
    assert torch.equal(idx_st, idx_ws) and torch.equal(out_st, out_ws)


def test_static_matches_workspace_call_twice_second_smaller(gpu):
    """First the 20k-token filtered path (TIP group maxima, one select + FAC
    launch), then a smaller ragged batch on the whole-row path."""
    _compare(gpu, W.shrink(W.get("c2"), context=20000))
    _compare(gpu, W.shrink(W.get("c3"), batch=2, context=3001, context_min=1500))


def test_static_flags_reach_the_caller(gpu):
    """A length beyond max_seq_len raises the SEQ_LEN flag into dev_flags, and
    the next good call clears it."""
    w = W.shrink(W.get("c1"), context=300)
    x = W.generate(w)
    g = GpuSetup(gpu, w, x)
    q, kn, vn = (to_dev(x[k][0], g.td) for k in ("q", "k_new", "v_new"))
    out = torch.empty(w.batch, w.n_q_heads, w.head_dim, dtype=torch.float32, device="cuda")
    flags = torch.zeros(1, dtype=torch.int32, device="cuda")
    g.ctx.decode_step_static(g.k, g.v, g.side, q, kn, vn, g.seq_lens, 100, w.budget, out,
                             dev_flags=flags)
    torch.cuda.synchronize()
    assert int(flags.item()) & gpu.DEVFLAG_SEQ_LEN
    g.ctx.decode_step_static(g.k, g.v, g.side, q, kn, vn, g.seq_lens, 300, w.budget, out,
                             dev_flags=flags)
    torch.cuda.synchronize()
    assert int(flags.item()) == 0


def test_static_refuses_a_workspace_past_the_array(gpu):
    """A context whose workspace exceeds the array is refused on the host,
    before any pointer is looked at or anything is enqueued."""
    w = W.shrink(W.get("c4"), batch=4, context=200000, steps=1)
    x = W.generate(w, with_prefill=False)
    ctx = gpu.Context(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.capacity, w.rope_theta,
                      w.dtype, x["dom"], 1024)
    assert ctx.workspace_bytes > gpu.STATIC_SCRATCH_BYTES
    st = gpu._lib.fasa_decode_step_static(ctx._h, None, None, None, None, None, None, None,
                                          1000, 1024, None, None, None, 0, None)
    assert st == -2  # FASA_ERR_CAPACITY
    assert "static scratch" in gpu._lib.fasa_last_error().decode()
