"""Seeded generators: determinism, shapes and the planted structure (CPU)."""

import numpy as np
import pytest

import oracle
import workloads as W


def test_deterministic_and_seed_sensitive():
    w = W.shrink(W.get("c2"), context=512)
    a, b = W.generate(w), W.generate(w)
    for key in ("dom", "ctx", "q", "k_new", "v_new", "k_prefill", "v_prefill"):
        assert np.array_equal(a[key], b[key]), key
    c = W.generate(w, seed=1)
    assert not np.array_equal(a["q"], c["q"])


@pytest.mark.parametrize("name", ["c1", "c2", "c3", "c4", "c5"])
def test_shapes_and_counts(name):
    w = W.get(name)
    x = W.generate(w, with_prefill=False)
    assert x["dom"].shape == (w.n_q_heads, w.n_dom)
    for row in x["dom"]:
        assert len(set(row.tolist())) == w.n_dom and row.min() >= 0 and row.max() < w.n_fc
        assert np.all(np.diff(row) > 0)
    assert x["q"].shape == (w.steps, w.batch, w.n_q_heads, w.head_dim)
    assert x["k_new"].shape == (w.steps, w.batch, w.n_kv_heads, w.head_dim)
    for i, pos in enumerate(x["planted"]):
        ctx = int(x["ctx"][i])
        assert len(pos) == w.planted_for(ctx)
        assert len(set(pos.tolist())) == len(pos)
        assert pos.min() >= 0 and pos.max() < ctx - 1
    if w.context_min is not None:
        assert x["ctx"].min() >= w.context_min and x["ctx"].max() <= w.context
        assert len(set(x["ctx"].tolist())) > 1
    assert w.capacity >= w.context + w.steps - 1 and w.capacity % 64 == 0


def test_planted_counts_match_the_configs():
    assert W.get("c1").planted_for(512) == 8
    assert W.get("c2").planted_for(32768) == 328
    assert W.get("c4").planted_for(32768) == 655
    assert W.get("c5").planted_for(131072) == 655


def test_c5_spans():
    w = W.get("c5")
    x = W.generate(w, with_prefill=False)
    pos = np.sort(x["planted"][0])
    assert len(pos) == 655
    # Greedy cover by 64-token intervals is minimal; it must need <= 16.
    count, end = 0, -1
    for p in pos:
        if p > end:
            count, end = count + 1, p + 63
    assert count <= 16


def test_values_are_dtype_representable():
    w = W.shrink(W.get("c2"), context=256)
    x = W.generate(w)
    for key in ("q", "k_prefill", "v_prefill", "k_new"):
        v = x[key].astype(np.float64)
        assert np.array_equal(oracle.rope.round_to_dtype(v, "bf16"), v), key


def test_planted_positions_rank_high():
    """Statistical sanity (not a parity pin): with B >= #planted, head 0's
    selection (whose FCs are all planted for it) contains every planted token."""
    w = W.shrink(W.get("c2"), context=2048)
    x = W.generate(w)
    st = oracle.OracleState(1, w.n_q_heads, w.n_kv_heads, w.head_dim, w.rope_theta,
                            w.dtype, x["dom"], w.capacity)
    st.append(0, x["k_prefill"][0], x["v_prefill"][0])
    r = st.step(x["q"][0], x["k_new"][0], x["v_new"][0], w.budget, heads=[0])
    pl = set(x["planted"][0].tolist())
    sel = set(r["idx"][0, 0][r["idx"][0, 0] >= 0].tolist())
    assert pl <= sel


@pytest.mark.parametrize("head_dim,rotary_dim,theta", [(128, 128, 5e5), (64, 64, 1e4),
                                                       (128, 64, 1e4), (64, 16, 1e4)])
def test_planting_ladder_matches_the_oracle(head_dim, rotary_dim, theta):
    """The planting's own frequency and FC-pair tables (workloads keep none
    of the method's arithmetic for the kernels; planting needs these to align
    keys with the query) equal the oracle's."""
    from workloads.generate import plant_ladder
    w = W.shrink(W.get("c2"), head_dim=head_dim, rotary_dim=rotary_dim, rope_theta=theta)
    omega, lo, hi = plant_ladder(w)
    R = rotary_dim // 2
    want_w = np.zeros(head_dim // 2)
    want_w[:R] = oracle.rope.inv_freq(rotary_dim, theta)
    np.testing.assert_array_equal(omega, want_w)
    olo, ohi = oracle.rope.fc_pairs(head_dim, rotary_dim)
    np.testing.assert_array_equal(lo, olo)
    np.testing.assert_array_equal(hi, ohi)
