"""Pins: checks that tie the oracle to something other than itself.

Each ``pin_*`` function raises AssertionError when the oracle disagrees with a
closed form, a brute-force enumeration, a library routine or a hand-built
example.  They look the oracle's functions up through the module attributes at
call time, so ``test_oracle_mutations.py`` can plant a mistake in the oracle
and check that some pin catches it.

Passages ("FASA: Frequency-aware Sparse Attention"): gist.science/pt,
"Resumo Tecnico" section 2 -- "A Descoberta" (RoPE's 2-D frequency chunks),
TIP "Previsao Online" (sum of dominant-FC contributions), FAC bullets (select
T_t, full attention over it, absolute positions kept); the decode setting is
section 1.  Among the pins: with every FC dominant TIP equals the full q.k;
with B >= n, FAC equals dense attention; TIP is the sum of per-FC rotated 2-D
dot products; brute force on tiny contexts.
"""

import cmath
import itertools
import json
import math
import os

import numpy as np
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


# ----------------------------------------------------------------- RoPE ----

def pin_rope_identity_at_zero():
    x = _rng(1).standard_normal((3, 64))
    y = oracle.rope.rope_rotate(x, 0, 1e4)
    assert np.array_equal(y, x), "RoPE at position 0 must be the identity"


def pin_rope_norm_per_fc():
    x = _rng(2).standard_normal((5, 128))
    y = oracle.rope.rope_rotate(x, np.array([0, 1, 77, 4096, 131071]), 5e5)
    nx = x[:, :64] ** 2 + x[:, 64:] ** 2
    ny = y[:, :64] ** 2 + y[:, 64:] ** 2
    assert np.allclose(nx, ny, rtol=1e-12, atol=1e-12), "FC norms must be kept"


def pin_rope_relative_shift():
    r = _rng(3)
    q, k = r.standard_normal(64), r.standard_normal(64)
    for (m, n, s) in [(5, 2, 100), (300, 17, 4096), (1, 0, 99999)]:
        a = oracle.rope.rope_rotate(q, m, 1e4) @ oracle.rope.rope_rotate(k, n, 1e4)
        b = oracle.rope.rope_rotate(q, m + s, 1e4) @ oracle.rope.rope_rotate(k, n + s, 1e4)
        assert abs(a - b) <= 1e-9 * (1 + abs(a)), "q.k must depend on m - n only"


def pin_rope_literal_angles():
    """Hand-built case: angles are powers of ten by construction."""
    with open(os.path.join(GOLDEN, "rope_d8_theta1e4.json")) as f:
        g = json.load(f)
    d, half = g["head_dim"], g["head_dim"] // 2
    ang = g["angles_rad"]
    for c in range(half):
        e = np.zeros(d)
        e[c] = 1.0
        y = oracle.rope.rope_rotate(e, g["position"], g["theta"])
        want = np.zeros(d)
        want[c], want[c + half] = math.cos(ang[c]), math.sin(ang[c])
        assert np.allclose(y, want, rtol=0, atol=1e-13), f"e_{c} rotated wrongly"
        e = np.zeros(d)
        e[c + half] = 1.0
        y = oracle.rope.rope_rotate(e, g["position"], g["theta"])
        want = np.zeros(d)
        want[c], want[c + half] = -math.sin(ang[c]), math.cos(ang[c])
        assert np.allclose(y, want, rtol=0, atol=1e-13), f"e_{c+half} rotated wrongly"


def pin_rope_complex_form():
    """(x_c + i x_{c+C}) * exp(i m theta^(-2c/d)), scalar complex arithmetic."""
    x = _rng(4).standard_normal(64)
    m, theta = 123, 1e4
    y = oracle.rope.rope_rotate(x, m, theta)
    for c in range(32):
        z = complex(x[c], x[c + 32]) * cmath.exp(1j * m * math.pow(theta, -2 * c / 64))
        assert abs(z.real - y[c]) < 1e-12 and abs(z.imag - y[c + 32]) < 1e-12


def pin_rope_partial_with_full_rotary_dim_is_full():
    x = _rng(40).standard_normal((3, 64))
    pos = np.array([0, 7, 123456])
    got = oracle.rope.rope_rotate_partial(x, pos, 1e4, 64)
    assert np.allclose(got, oracle.rope.rope_rotate(x, pos, 1e4), rtol=0, atol=1e-12)


def pin_rope_partial_complex_form():
    """r = 24 of d = 64: (x_c + i x_{c+12}) exp(i m theta^(-2c/24)) on the
    rotated dims, the other 40 dims unchanged bit for bit."""
    r = _rng(41)
    x = r.standard_normal(64)
    for m in (0, 1, 999, 65535):
        got = oracle.rope.rope_rotate_partial(x, m, 5e5, 24)
        z = (x[:12] + 1j * x[12:24]) * np.exp(1j * m * 5e5 ** (-np.arange(12) / 12.0))
        assert np.allclose(got[:12], z.real, rtol=0, atol=1e-12)
        assert np.allclose(got[12:24], z.imag, rtol=0, atol=1e-12)
        assert np.array_equal(got[24:], x[24:])


def pin_fc_pairs_partial_layout():
    """FC pairs partition the dims; full layout is (c, c + d/2); with r = 16 of
    d = 64 the rotated FCs are (c, c + 8) and the pass-through pairs are
    (16 + i, 16 + i + 24)."""
    lo, hi = oracle.rope.fc_pairs(64, 64)
    assert lo.tolist() == list(range(32)) and hi.tolist() == list(range(32, 64))
    lo, hi = oracle.rope.fc_pairs(64, 16)
    assert sorted(lo.tolist() + hi.tolist()) == list(range(64))
    assert lo[:8].tolist() == list(range(8)) and hi[:8].tolist() == list(range(8, 16))
    assert lo[8:].tolist() == list(range(16, 40)) and hi[8:].tolist() == list(range(40, 64))


def pin_tip_partial_all_fcs_is_full_dot_and_relative():
    """Partial RoPE: with every FC dominant TIP is the full dot product, and
    the score depends on the two positions only through their difference."""
    r = _rng(42)
    d, rd, theta = 64, 16, 1e4
    pairs = oracle.rope.fc_pairs(d, rd)
    q, k = r.standard_normal(d), r.standard_normal((5, d))
    dom = np.arange(d // 2)
    for (m, n, t) in ((10, 3, 100), (4000, 17, 12345)):
        qa = oracle.rope.rope_rotate_partial(q, m, theta, rd)
        ka = oracle.rope.rope_rotate_partial(k, n, theta, rd)
        qb = oracle.rope.rope_rotate_partial(q, m + t, theta, rd)
        kb = oracle.rope.rope_rotate_partial(k, n + t, theta, rd)
        sa = oracle.tip.tip_scores(qa, ka, dom, pairs)
        assert np.allclose(sa, ka @ qa, rtol=1e-12, atol=1e-12)
        assert np.allclose(sa, oracle.tip.tip_scores(qb, kb, dom, pairs), rtol=1e-9, atol=1e-9)
    # A pass-through FC alone does not depend on the positions at all.
    c = 20
    s1 = oracle.tip.tip_scores(oracle.rope.rope_rotate_partial(q, 5, theta, rd),
                               oracle.rope.rope_rotate_partial(k, 2, theta, rd), [c], pairs)
    lo, hi = pairs[0][c], pairs[1][c]
    assert np.allclose(s1, k[:, lo] * q[lo] + k[:, hi] * q[hi], rtol=0, atol=1e-12)


def pin_round_to_dtype():
    rd = oracle.rope.round_to_dtype
    # bf16: 8 significant bits.  Representable values stay put.
    exact = np.array([1.0, -1.5, 2.0 ** -126, 2.0 ** -133, 0.0, 1.0 + 2 ** -7,
                      2.0 ** 127, -(2 - 2 ** -7) * 2.0 ** 127])
    assert np.array_equal(rd(exact, "bf16"), exact)
    # Midpoints go to the even neighbour; just above a midpoint goes up.
    cases = [(1 + 2 ** -8, 1.0), (1 + 3 * 2 ** -8, 1 + 2 ** -6),
             (1 + 2 ** -8 + 2 ** -30, 1 + 2 ** -7), (-(1 + 2 ** -8), -1.0),
             (2.0 ** -134, 0.0), (3 * 2.0 ** -134, 2.0 ** -132),
             (255.5, 256.0), (254.5, 254.0)]
    for x, want in cases:
        assert rd(np.array([x]), "bf16")[0] == want, (x, want)
    # Against torch's fp32 -> bf16 conversion on fp32 inputs (no double rounding).
    x = (_rng(5).standard_normal(20000) * 10.0 ** _rng(6).uniform(-30, 30, 20000))
    x = x.astype(np.float32)
    t = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(rd(x.astype(np.float64), "bf16"), t)
    # fp32: ties to even at 24 bits.
    assert rd(np.array([1 + 2 ** -24]), "f32")[0] == 1.0
    assert rd(np.array([1 + 3 * 2 ** -24]), "f32")[0] == 1 + 2 ** -22


# ------------------------------------------------------------------ TIP ----

def pin_tip_all_fcs_is_full_dot():
    r = _rng(7)
    q, k = r.standard_normal(128), r.standard_normal((50, 128))
    qr = oracle.rope.rope_rotate(q, 49, 5e5)
    kr = oracle.rope.rope_rotate(k, np.arange(50), 5e5)
    s = oracle.tip.tip_scores(qr, kr, np.arange(64))
    full = np.array([float(np.dot(qr, kr[j])) for j in range(50)])
    assert np.allclose(s, full, rtol=1e-12, atol=1e-12), "all-FC TIP must equal q.k"


def pin_tip_relative_complex():
    """TIP from pre-RoPE values: sum_c Re[z_q conj(z_k) exp(i (m_q - m_k) w_c)]."""
    r = _rng(8)
    d, half, theta = 64, 32, 1e4
    q, k = r.standard_normal(d), r.standard_normal((20, d))
    dom = np.array([0, 3, 17, 31])
    mq = 40
    qr = oracle.rope.rope_rotate(q, mq, theta)
    kr = oracle.rope.rope_rotate(k, np.arange(20), theta)
    s = oracle.tip.tip_scores(qr, kr, dom)
    for j in range(20):
        want = 0.0
        for c in dom:
            zq, zk = complex(q[c], q[c + half]), complex(k[j, c], k[j, c + half])
            w = math.pow(theta, -2 * c / d)
            want += (zq * zk.conjugate() * cmath.exp(1j * (mq - j) * w)).real
        assert abs(s[j] - want) < 1e-10, (j, s[j], want)


def pin_tip_single_fc():
    r = _rng(9)
    q, k = r.standard_normal(128), r.standard_normal((7, 128))
    for c in (0, 5, 63):
        s = oracle.tip.tip_scores(q, k, np.array([c]))
        want = q[c] * k[:, c] + q[c + 64] * k[:, c + 64]
        assert np.allclose(s, want, rtol=1e-14, atol=1e-14)


def pin_tip_linear_in_q():
    r = _rng(10)
    q1, q2, k = r.standard_normal(64), r.standard_normal(64), r.standard_normal((9, 64))
    dom = np.array([1, 2, 30])
    lhs = oracle.tip.tip_scores(2.5 * q1 - 0.75 * q2, k, dom)
    rhs = 2.5 * oracle.tip.tip_scores(q1, k, dom) - 0.75 * oracle.tip.tip_scores(q2, k, dom)
    assert np.allclose(lhs, rhs, rtol=1e-12, atol=1e-12)


# ------------------------------------------------------------ selection ----

def _brute_force_topb(s, budget):
    """Max-sum subset of size min(B, n); among equal sums the lexicographically
    smallest ascending tuple (= ties to the lower position)."""
    n = len(s)
    take = min(budget, n)
    best, best_key = None, None
    for comb in itertools.combinations(range(n), take):
        key = (-sum(s[j] for j in comb), comb)
        if best_key is None or key < best_key:
            best, best_key = comb, key
    return list(best) + [-1] * (budget - take)


def pin_select_brute_force():
    r = _rng(11)
    for trial in range(60):
        n = int(r.integers(1, 11))
        budget = int(r.integers(1, 5))
        # Small integer scores force many ties.
        s = r.integers(-3, 4, size=n).astype(np.float64)
        got = oracle.select.select_topb(s, budget).tolist()
        assert got == _brute_force_topb(s.tolist(), budget), (s, budget, got)


def pin_select_vs_stable_argsort():
    r = _rng(12)
    s = np.round(r.standard_normal(3000), 2)  # many ties
    for budget in (1, 17, 256, 2999, 3000):
        got = oracle.select.select_topb(s, budget)
        want = np.sort(np.argsort(-s, kind="stable")[:budget])
        assert np.array_equal(got, want)


def pin_select_hand_example():
    with open(os.path.join(GOLDEN, "select_ties.json")) as f:
        g = json.load(f)
    # Worked by hand from the ranking 0, 2, 4, 3, 1, 5 (see the fixture).
    expect = {1: [0], 2: [0, 2], 3: [0, 2, 4], 4: [0, 2, 3, 4],
              8: [0, 1, 2, 3, 4, 5, -1, -1]}
    for budget in g["budgets"]:
        got = oracle.select.select_topb(np.array(g["scores"]), budget).tolist()
        assert got == expect[budget], (budget, got)


def pin_select_budget_ge_n():
    s = _rng(13).standard_normal(10)
    got = oracle.select.select_topb(s, 16)
    assert got.tolist() == list(range(10)) + [-1] * 6


def pin_select_per_head_budget_brute_force():
    """A head of budget B_h in a row of width W: the brute-force top-B_h set
    (B_h = 0 keeps nothing), padded with -1 to W."""
    r = _rng(14)
    for trial in range(60):
        n = int(r.integers(1, 10))
        width = int(r.integers(1, 6))
        bh = int(r.integers(0, width + 1))
        s = r.integers(-2, 3, size=n).astype(np.float64)
        got = oracle.select.select_topb_width(s, bh, width).tolist()
        want = _brute_force_topb(s.tolist(), bh) + [-1] * (width - bh)
        assert got == want, (s, bh, width, got)


def pin_select_sets_nest_with_budget():
    """Raising the budget only adds tokens: T(B) is a subset of T(B + 1), and
    the token added is the best one outside T(B) (ties to the lower position)."""
    r = _rng(15)
    s = np.round(r.standard_normal(40), 1)
    prev = set()
    for b in range(0, 41):
        cur = set(oracle.select.select_topb_width(s, b, 40)[:b].tolist())
        assert prev <= cur and len(cur) == b
        if b:
            (new,) = cur - prev
            rest = [j for j in range(40) if j not in prev]
            assert new == min(rest, key=lambda j: (-s[j], j))
        prev = cur


def pin_threshold_brute_force():
    """tau is the smallest score of the brute-force best subset of size
    min(B, n) (T_t's own definition), on tiny integer rows with many ties."""
    r = _rng(16)
    for trial in range(80):
        n = int(r.integers(1, 10))
        budget = int(r.integers(1, 6))
        s = r.integers(-3, 4, size=n).astype(np.float64)
        best = [j for j in _brute_force_topb(s.tolist(), budget) if j >= 0]
        want = min(s[j] for j in best)
        got = oracle.select.threshold(s, budget)
        assert got == want, (s, budget, got, want)


def pin_threshold_hand_example():
    """The hand-ranked fixture: ranking 0 (3), 2 (3), 4 (3), 3 (2), 1 (1),
    5 (0), so tau is 3, 3, 3, 2 for B = 1..4, and 0 (the smallest score)
    for B = 8 > n."""
    with open(os.path.join(GOLDEN, "select_ties.json")) as f:
        g = json.load(f)
    expect = {1: 3.0, 2: 3.0, 3: 3.0, 4: 2.0, 8: 0.0}
    for budget in g["budgets"]:
        got = oracle.select.threshold(np.array(g["scores"]), budget)
        assert got == expect[budget], (budget, got)


def pin_threshold_vs_partition():
    """tau equals the B-th largest score from numpy's introselect
    (np.partition), a routine the oracle does not call."""
    r = _rng(17)
    s = np.round(r.standard_normal(5000), 2)
    for budget in (1, 2, 255, 256, 4999, 5000, 7000):
        k = min(budget, s.size)
        want = float(np.partition(s, s.size - k)[s.size - k])
        assert oracle.select.threshold(s, budget) == want, budget


def pin_threshold_rejects_empty_selection():
    """B = 0 keeps nothing, so there is no threshold: the oracle must refuse
    rather than return some score."""
    for budget, row in ((0, [1.0, 2.0]), (-1, [1.0]), (3, [])):
        try:
            oracle.select.threshold(np.array(row), budget)
        except ValueError:
            continue
        raise AssertionError(f"threshold accepted budget {budget} on {row}")


# ------------------------------------------------------------------ FAC ----

def _sdpa(q, k, v):
    out = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None, None, None, :],
        torch.from_numpy(k)[None, None], torch.from_numpy(v)[None, None])
    return out[0, 0, 0].numpy()


def pin_fac_dense_when_budget_covers_all():
    r = _rng(14)
    q, k, v = r.standard_normal(128), r.standard_normal((40, 128)), r.standard_normal((40, 128))
    got = oracle.fac.attend_subset(q, k, v, np.arange(40))
    assert np.allclose(got, _sdpa(q, k, v), rtol=1e-12, atol=1e-12)


def pin_fac_single_token():
    r = _rng(15)
    q, k, v = r.standard_normal(64), r.standard_normal((12, 64)), r.standard_normal((12, 64))
    got = oracle.fac.attend_subset(q, k, v, np.array([7, -1, -1]))
    assert np.allclose(got, v[7], rtol=0, atol=1e-15)


def pin_fac_constant_values():
    r = _rng(16)
    q, k = r.standard_normal(64), r.standard_normal((12, 64))
    v = np.tile(r.standard_normal(64), (12, 1))
    got = oracle.fac.attend_subset(q, k, v, np.array([1, 4, 9]))
    assert np.allclose(got, v[0], rtol=1e-14, atol=1e-14)


def pin_fac_zero_query_is_mean():
    r = _rng(17)
    k, v = r.standard_normal((12, 64)), r.standard_normal((12, 64))
    sub = np.array([0, 3, 5, 11])
    got = oracle.fac.attend_subset(np.zeros(64), k, v, sub)
    assert np.allclose(got, v[sub].mean(axis=0), rtol=1e-13, atol=1e-13)


def pin_fac_permutation_invariant():
    r = _rng(18)
    q, k, v = r.standard_normal(64), r.standard_normal((30, 64)), r.standard_normal((30, 64))
    sub = np.array([2, 8, 9, 20, 29])
    a = oracle.fac.attend_subset(q, k, v, sub)
    b = oracle.fac.attend_subset(q, k, v, sub[::-1].copy())
    assert np.allclose(a, b, rtol=1e-14, atol=1e-14)


def pin_fac_scale_closed_form():
    """q.k_A = sqrt(d) ln 3, q.k_B = 0  =>  weights 3/4 and 1/4."""
    d = 64
    q = np.zeros(d)
    q[0] = 1.0
    k = np.zeros((2, d))
    k[0, 0] = math.sqrt(d) * math.log(3.0)
    v = np.zeros((2, d))
    v[0, 0], v[1, 1] = 1.0, 1.0
    got = oracle.fac.attend_subset(q, k, v, np.array([0, 1]))
    assert abs(got[0] - 0.75) < 1e-14 and abs(got[1] - 0.25) < 1e-14, got[:2]


def pin_fac_ignores_unselected():
    r = _rng(19)
    q, k, v = r.standard_normal(64), r.standard_normal((10, 64)), r.standard_normal((10, 64))
    sub = np.array([1, 6])
    a = oracle.fac.attend_subset(q, k, v, sub)
    k2, v2 = k.copy(), v.copy()
    k2[[0, 2, 3]] *= 50.0
    v2[[0, 2, 3]] += 7.0
    b = oracle.fac.attend_subset(q, k2, v2, sub)
    assert np.allclose(a, b, rtol=0, atol=0)


# --------------------------------------------------------------- decode ----

def _state(n_q, n_kv, d, theta, dtype, dom, cap, batch=1):
    return oracle.decode.OracleState(batch, n_q, n_kv, d, theta, dtype, dom, cap)


def pin_decode_dense_equivalence():
    """All FCs dominant and B >= n: the step is dense attention with RoPE."""
    r = _rng(20)
    d, n, theta = 64, 33, 1e4
    dom = np.tile(np.arange(32), (2, 1))
    st = _state(2, 1, d, theta, "f32", dom, 64)
    k = r.standard_normal((1, n - 1, d)).astype(np.float32).astype(np.float64)
    v = r.standard_normal((1, n - 1, d))
    st.append(0, k, v)
    q = r.standard_normal((1, 2, d))
    kn, vn = r.standard_normal((1, 1, d)), r.standard_normal((1, 1, d))
    res = st.step(q, kn, vn, budget=64)
    kall = np.concatenate([k[0], kn[0]], axis=0)
    vall = np.concatenate([v[0], vn[0]], axis=0)
    # Independent rotation: complex phasors, query at the last position n-1.
    def rot(x, m):
        z = x[:32] + 1j * x[32:]
        z = z * np.exp(1j * m * theta ** (-2.0 * np.arange(32) / d))
        return np.concatenate([z.real, z.imag])
    kr = np.stack([rot(kall[j], j) for j in range(n)])
    for h in range(2):
        want = _sdpa(rot(q[0, h], n - 1), kr, vall)
        # The oracle rounds K to fp32 once; allow for that rounding only.
        assert np.allclose(res["out"][0, h], want, rtol=1e-6, atol=1e-6), h
        assert res["idx"][0, h].tolist()[:n] == list(range(n))


def pin_decode_per_head_budgets():
    """Budgets per head: a head with B_h >= n is dense attention (closed form
    with complex rotations), a head with B_h = 0 outputs zeros and selects
    nothing, and a head with B_h = 1 outputs the V row of its best-scoring
    token."""
    r = _rng(23)
    d, n, theta, width = 64, 24, 1e4, 32
    dom = np.tile(np.arange(32), (3, 1))
    st = _state(3, 1, d, theta, "f32", dom, 32)
    k = r.standard_normal((1, n - 1, d)).astype(np.float32).astype(np.float64)
    v = r.standard_normal((1, n - 1, d))
    st.append(0, k, v)
    q = r.standard_normal((1, 3, d))
    kn, vn = r.standard_normal((1, 1, d)), r.standard_normal((1, 1, d))
    res = st.step(q, kn, vn, budget=width, head_budgets=[width, 0, 1])
    kall = np.concatenate([k[0], kn[0]], axis=0)
    vall = np.concatenate([v[0], vn[0]], axis=0)

    def rot(x, m):
        z = x[:32] + 1j * x[32:]
        z = z * np.exp(1j * m * theta ** (-2.0 * np.arange(32) / d))
        return np.concatenate([z.real, z.imag])
    kr = np.stack([rot(kall[j], j) for j in range(n)])
    want0 = _sdpa(rot(q[0, 0], n - 1), kr, vall)
    assert np.allclose(res["out"][0, 0], want0, rtol=1e-6, atol=1e-6)
    assert res["idx"][0, 0].tolist() == list(range(n)) + [-1] * (width - n)
    assert np.all(res["out"][0, 1] == 0) and np.all(res["idx"][0, 1] == -1)
    best = int(np.argmax(kr @ rot(q[0, 2], n - 1)))
    assert res["idx"][0, 2].tolist() == [best] + [-1] * (width - 1)
    assert np.allclose(res["out"][0, 2], vall[best], rtol=0, atol=1e-12)


def pin_decode_partial_rope_dense_equivalence():
    """Partial RoPE (r = 32 of d = 64), all FCs dominant, B >= n: the step is
    dense attention with the first 32 dims rotated (complex phasors) and the
    rest as given."""
    r = _rng(24)
    d, rd, n, theta = 64, 32, 29, 1e4
    dom = np.tile(np.arange(32), (2, 1))
    st = oracle.decode.OracleState(1, 2, 1, d, theta, "f32", dom, 64, rotary_dim=rd)
    k = r.standard_normal((1, n - 1, d)).astype(np.float32).astype(np.float64)
    v = r.standard_normal((1, n - 1, d))
    st.append(0, k, v)
    q = r.standard_normal((1, 2, d))
    kn = r.standard_normal((1, 1, d)).astype(np.float32).astype(np.float64)
    vn = r.standard_normal((1, 1, d))
    res = st.step(q, kn, vn, budget=64)
    kall = np.concatenate([k[0], kn[0]], axis=0)
    vall = np.concatenate([v[0], vn[0]], axis=0)

    def rot(x, m):
        z = (x[:16] + 1j * x[16:32]) * np.exp(1j * m * theta ** (-2.0 * np.arange(16) / rd))
        return np.concatenate([z.real, z.imag, x[32:]])
    kr = np.stack([rot(kall[j], j) for j in range(n)])
    for h in range(2):
        want = _sdpa(rot(q[0, h], n - 1), kr, vall)
        assert np.allclose(res["out"][0, h], want, rtol=1e-6, atol=1e-6), h
        assert res["idx"][0, h].tolist()[:n] == list(range(n))
    # Pass-through dims of the cache are the inputs, unrotated.
    assert np.array_equal(st.K[0, 0, :n, 32:], kall[:, 32:])


def pin_decode_query_position():
    """Equal pre-RoPE q and k rows at every position: the score of the token at
    the query's own position is exactly |k|^2, the Cauchy-Schwarz maximum."""
    r = _rng(21)
    d, n, theta = 64, 20, 1e4
    x = r.standard_normal(d)
    dom = np.arange(32)[None, :]
    st = _state(1, 1, d, theta, "f32", dom, 32)
    st.append(0, np.tile(x, (1, n - 1, 1)), np.zeros((1, n - 1, d)))
    st.append(0, x[None, None, :], np.zeros((1, 1, d)))
    qr = st.query_rot(0, x[None, :])
    s = st.head_scores(0, 0, qr[0])
    assert abs(s[n - 1] - float(x @ x)) < 1e-5 * float(x @ x)
    assert np.argmax(s) == n - 1


def pin_decode_append_consistency():
    """Bulk append and one-row appends give the same cache, and each row is
    its own position's rotation rounded to the dtype."""
    r = _rng(22)
    d, n = 128, 40
    dom = np.tile(np.arange(8), (4, 1))
    k, v = r.standard_normal((2, n, d)), r.standard_normal((2, n, d))
    a = _state(4, 2, d, 5e5, "bf16", dom, 64)
    a.append(0, k, v)
    b = _state(4, 2, d, 5e5, "bf16", dom, 64)
    for j in range(n):
        b.append(0, k[:, j:j + 1], v[:, j:j + 1])
    assert np.array_equal(a.K, b.K) and np.array_equal(a.V, b.V)
    j = 31
    want = oracle.rope.round_to_dtype(oracle.rope.rope_rotate(k[1, j], j, 5e5), "bf16")
    assert np.array_equal(a.K[0, 1, j], want)


def pin_loops_agree():
    """NumPy steps against the scalar-loop restatements."""
    r = _rng(23)
    d, n = 32, 25
    q, k, v = r.standard_normal(d), r.standard_normal((n, d)), r.standard_normal((n, d))
    kr = oracle.rope.rope_rotate(k, np.arange(n), 1e4)
    for j in (0, 9, 24):
        assert np.allclose(kr[j], oracle.loops.rope_loop(list(k[j]), j, 1e4), atol=1e-13)
    dom = [2, 5, 11]
    s = oracle.tip.tip_scores(q, kr, np.array(dom))
    assert np.allclose(s, oracle.loops.tip_loop(list(q), kr.tolist(), dom), atol=1e-12)
    for budget in (1, 4, 25, 30):
        assert oracle.select.select_topb(s, budget).tolist() == \
            oracle.loops.topb_loop(list(s), budget)
    sub = oracle.select.select_topb(s, 6)
    assert np.allclose(oracle.fac.attend_subset(q, kr, v, sub),
                       oracle.loops.attend_loop(list(q), kr.tolist(), v.tolist(), list(sub)),
                       atol=1e-13)


# ---------------------------------------------------------- calibration ----
# gist.science/pt, "Resumo Tecnico" section 2, TIP "Calibracao Offline": the
# agreement of one FC's scores with the full head's picks I_dom.

def _topk_by_sort(s, k):
    """Top-k positions by Python's own sort on (-score, position)."""
    return sorted(range(len(s)), key=lambda j: (-s[j], j))[:k]


def pin_calib_fc_scores_complex():
    # FC c's score is Re[(q_c + i q_{c+C}) conj(k_c + i k_{c+C})].
    r = _rng(40)
    d, half = 16, 8
    q = r.standard_normal(d)
    k = r.standard_normal((5, d))
    got = oracle.calibrate.fc_scores(q, k)
    assert got.shape == (half, 5)
    for c in range(half):
        zq = complex(q[c], q[c + half])
        for j in range(5):
            zk = complex(k[j, c], k[j, c + half])
            assert abs(got[c, j] - (zq * zk.conjugate()).real) < 1e-12


def pin_calib_fc_scores_sum_to_full_dot():
    r = _rng(41)
    q = r.standard_normal(64)
    k = r.standard_normal((30, 64))
    assert np.allclose(oracle.calibrate.fc_scores(q, k).sum(axis=0), k @ q, atol=1e-12)


def pin_calib_single_signal_fc():
    # A query carrying FC 3 alone: the head's scores are FC 3's, so CA(3) = 1.
    # An FC whose key columns are zero scores every token 0, so its top-k is
    # the k lowest positions.
    r = _rng(42)
    d, half, n, k = 16, 8, 40, 6
    q = np.zeros(d)
    q[3], q[3 + half] = r.standard_normal(2)
    keys = r.standard_normal((n, d))
    keys[:, 5] = 0.0
    keys[:, 5 + half] = 0.0
    ca = oracle.calibrate.contextual_agreement(q, keys, k)
    assert ca[3] == 1.0
    full = _topk_by_sort((keys @ q).tolist(), k)
    assert ca[5] == len(set(full) & set(range(k))) / k


def pin_calib_topk_covering_all_agrees():
    r = _rng(43)
    q = r.standard_normal(32)
    keys = r.standard_normal((7, 32))
    assert np.all(oracle.calibrate.contextual_agreement(q, keys, 7) == 1.0)
    assert np.all(oracle.calibrate.contextual_agreement(q, keys, 50) == 1.0)


def pin_calib_brute_force():
    r = _rng(44)
    for _ in range(40):
        n = int(r.integers(2, 10))
        k = int(r.integers(1, 5))
        d = 8
        # Small integers force many ties in both the FC and the full scores.
        q = r.integers(-2, 3, size=d).astype(np.float64)
        keys = r.integers(-2, 3, size=(n, d)).astype(np.float64)
        got = oracle.calibrate.contextual_agreement(q, keys, k)
        kk = min(k, n)
        full = _topk_by_sort([float(np.dot(keys[j], q)) for j in range(n)], kk)
        for c in range(d // 2):
            s = [q[c] * keys[j, c] + q[c + 4] * keys[j, c + 4] for j in range(n)]
            want = len(set(_topk_by_sort(s, kk)) & set(full)) / kk
            assert got[c] == want, (c, got[c], want)


def pin_calib_dominant_hand_example():
    # [samples, heads, C]; means per head: [0.5, 0.4, 0.8, 0.1] and
    # [0.1, 0.3, 0.2, 0.3] (worked by hand).
    ca = np.array([[[0.5, 0.5, 0.9, 0.1], [0.2, 0.2, 0.2, 0.2]],
                   [[0.5, 0.3, 0.7, 0.1], [0.0, 0.4, 0.2, 0.4]]])
    assert oracle.calibrate.dominant_from_ca(ca, 2).tolist() == [[0, 2], [1, 3]]
    assert oracle.calibrate.dominant_from_ca(ca, 1).tolist() == [[2], [1]]
    assert oracle.calibrate.dominant_from_ca(ca[0], 3).tolist() == [[0, 1, 2], [0, 1, 2]]


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
