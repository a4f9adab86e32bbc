"""Plant plausible mistakes in the oracle (on the CPU) and check that the pins
catch every one of them.

A pin set that lets a dropped term, a flipped sign, a wrong index or a swapped
operand through would not be worth trusting; this file is the evidence that it
does not.
"""

import numpy as np
import pytest

import oracle
import pins

_rope_rotate = oracle.rope.rope_rotate
_round = oracle.rope.round_to_dtype
_tip = oracle.tip.tip_scores
_select = oracle.select.select_topb
_select_width = oracle.select.select_topb_width
_step = oracle.decode.OracleState.step
_attend = oracle.fac.attend_subset
_query_rot = oracle.decode.OracleState.query_rot
_append = oracle.decode.OracleState.append
_fc_scores = oracle.calibrate.fc_scores
_rope_partial = oracle.rope.rope_rotate_partial
_fc_pairs = oracle.rope.fc_pairs
_ca = oracle.calibrate.contextual_agreement
_dominant = oracle.calibrate.dominant_from_ca


def rope_interleaved(x, pos, theta):
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    w = oracle.rope.inv_freq(d, theta)
    phi = np.asarray(pos, dtype=np.float64)[..., None] * w
    a, b = x[..., 0::2], x[..., 1::2]
    y = np.empty_like(x)
    y[..., 0::2] = a * np.cos(phi) - b * np.sin(phi)
    y[..., 1::2] = b * np.cos(phi) + a * np.sin(phi)
    return y


def rope_backwards(x, pos, theta):
    return _rope_rotate(x, -np.asarray(pos), theta)


def rope_wrong_ladder(x, pos, theta):
    x = np.asarray(x, dtype=np.float64)
    d, half = x.shape[-1], x.shape[-1] // 2
    w = np.power(float(theta), -np.arange(half) / d)  # exponent -c/d
    phi = np.asarray(pos, dtype=np.float64)[..., None] * w
    lo, hi = x[..., :half], x[..., half:]
    return np.concatenate([lo * np.cos(phi) - hi * np.sin(phi),
                           hi * np.cos(phi) + lo * np.sin(phi)], axis=-1)


def rope_off_by_one(x, pos, theta):
    return _rope_rotate(x, np.asarray(pos) + 1, theta)


def round_truncate(x, dtype):
    x = np.asarray(x, dtype=np.float64)
    if dtype != "bf16":
        return _round(x, dtype)
    _, e = np.frexp(x)
    sp = np.ldexp(1.0, np.maximum(e - 8, -133))
    return np.trunc(x / sp) * sp


def tip_drop_second_half(q, k, dom, pairs=None):
    q, k = np.asarray(q, np.float64), np.asarray(k, np.float64)
    return k[:, np.asarray(dom)] @ q[np.asarray(dom)]


def tip_adjacent_pairs(q, k, dom, pairs=None):
    q, k = np.asarray(q, np.float64), np.asarray(k, np.float64)
    dom = np.asarray(dom)
    cols = np.concatenate([2 * dom, 2 * dom + 1])
    return k[:, cols] @ q[cols]


def tip_wrong_partner(q, k, dom, pairs=None):
    q, k = np.asarray(q, np.float64), np.asarray(k, np.float64)
    half = q.shape[-1] // 2
    dom = np.asarray(dom)
    return k[:, dom] @ q[dom + half] + k[:, dom + half] @ q[dom]


def select_ties_high(scores, budget):
    s = np.asarray(scores, np.float64)
    n = s.shape[0]
    order = np.lexsort((-np.arange(n), -s))
    take = min(budget, n)
    out = np.full(budget, -1, dtype=np.int64)
    out[:take] = np.sort(order[:take])
    return out


def select_lowest(scores, budget):
    return _select(-np.asarray(scores, np.float64), budget)


def select_one_short(scores, budget):
    out = _select(scores, budget)
    take = int((out >= 0).sum())
    if take > 1:
        out[take - 1] = -1
    return out


def threshold_next_rank(scores, budget):
    st = np.sort(np.asarray(scores, np.float64))[::-1]
    return float(st[min(budget, st.shape[0] - 1)])


def threshold_ascending(scores, budget):
    st = np.sort(np.asarray(scores, np.float64))
    return float(st[min(budget, st.shape[0]) - 1])


def threshold_budget_zero_wraps(scores, budget):
    st = np.sort(np.asarray(scores, np.float64))[::-1]
    return float(st[min(budget, st.shape[0]) - 1])


def attend_no_scale(q, k, v, subset):
    return _attend(np.asarray(q) * np.sqrt(np.asarray(q).shape[-1]), k, v, subset)


def attend_all_rows(q, k, v, subset):
    return _attend(q, k, v, np.arange(np.asarray(k).shape[0]))


def attend_k_for_v(q, k, v, subset):
    return _attend(q, k, k, subset)


def query_at_n(self, b, q):
    return oracle.rope.rope_rotate(q, int(self.lens[b]), self.theta)


def append_rotates_v(self, b, k_new, v_new):
    p0 = int(self.lens[b])
    pos = np.arange(p0, p0 + np.asarray(k_new).shape[1])
    _append(self, b, k_new, oracle.rope.rope_rotate(v_new, pos[None, :], self.theta))


def fc_scores_swapped_partner(q, k, pairs=None):
    q, k = np.asarray(q, np.float64), np.asarray(k, np.float64)
    half = q.shape[-1] // 2
    return (k[:, :half] * q[None, half:]).T + (k[:, half:] * q[None, :half]).T


def ca_unnormalised(q, k, topk, pairs=None):
    return _ca(q, k, topk, pairs) * min(topk, np.asarray(k).shape[0])


def ca_against_first_fc(q, k, topk, pairs=None):
    s_c = oracle.calibrate.fc_scores(q, k, pairs)
    kk = min(topk, s_c.shape[1])
    ref = set(oracle.select.select_topb(s_c[0], kk).tolist())
    return np.array([len(ref & set(oracle.select.select_topb(s, kk).tolist())) / kk for s in s_c])


def dominant_lowest(ca, n_dom):
    return _dominant(-np.asarray(ca, np.float64), n_dom)


def dominant_ties_high(ca, n_dom):
    a = np.asarray(ca, np.float64)
    a = a.mean(axis=0) if a.ndim == 3 else a
    picks = [np.sort(np.lexsort((-np.arange(a.shape[1]), -row))[:n_dom]) for row in a]
    return np.array(picks, dtype=np.int32)


def width_ignores_budget(scores, budget, width):
    return _select_width(scores, width, width)


def width_zero_keeps_one(scores, budget, width):
    return _select_width(scores, max(budget, 1), width)


def step_budgets_reversed(self, q, k_new, v_new, budget, heads=None, head_budgets=None):
    hb = None if head_budgets is None else list(head_budgets)[::-1]
    return _step(self, q, k_new, v_new, budget, heads=heads, head_budgets=hb)


def partial_freq_over_d(x, pos, theta, rotary_dim):
    # frequencies spaced over the head dim instead of the rotary dim
    x = np.asarray(x, np.float64)
    d, R = x.shape[-1], rotary_dim // 2
    w = np.power(float(theta), -2.0 * np.arange(R) / d)
    phi = np.asarray(pos, np.float64)[..., None] * w
    out = x.copy()
    a, b = x[..., :R], x[..., R:rotary_dim]
    out[..., :R] = a * np.cos(phi) - b * np.sin(phi)
    out[..., R:rotary_dim] = b * np.cos(phi) + a * np.sin(phi)
    return out


def partial_rotates_all(x, pos, theta, rotary_dim):
    return _rope_rotate(x, pos, theta)


def pairs_full_layout(head_dim, rotary_dim=None):
    return _fc_pairs(head_dim, None)


MUTATIONS = {
    "rope_interleaved_pairs": (oracle.rope, "rope_rotate", rope_interleaved),
    "rope_backwards": (oracle.rope, "rope_rotate", rope_backwards),
    "rope_frequency_ladder": (oracle.rope, "rope_rotate", rope_wrong_ladder),
    "rope_position_plus_one": (oracle.rope, "rope_rotate", rope_off_by_one),
    "bf16_truncation": (oracle.rope, "round_to_dtype", round_truncate),
    "tip_drops_cos_partner": (oracle.tip, "tip_scores", tip_drop_second_half),
    "tip_adjacent_pairs": (oracle.tip, "tip_scores", tip_adjacent_pairs),
    "tip_swapped_partner": (oracle.tip, "tip_scores", tip_wrong_partner),
    "select_ties_to_higher": (oracle.select, "select_topb", select_ties_high),
    "select_lowest_scores": (oracle.select, "select_topb", select_lowest),
    "select_one_short": (oracle.select, "select_topb", select_one_short),
    "select_width_ignores_budget": (oracle.select, "select_topb_width", width_ignores_budget),
    "select_width_zero_keeps_one": (oracle.select, "select_topb_width", width_zero_keeps_one),
    "threshold_next_rank": (oracle.select, "threshold", threshold_next_rank),
    "threshold_ascending_sort": (oracle.select, "threshold", threshold_ascending),
    "threshold_budget_zero_wraps": (oracle.select, "threshold", threshold_budget_zero_wraps),
    "decode_head_budgets_reversed": (oracle.decode.OracleState, "step", step_budgets_reversed),
    "fac_missing_scale": (oracle.fac, "attend_subset", attend_no_scale),
    "fac_ignores_subset": (oracle.fac, "attend_subset", attend_all_rows),
    "fac_keys_as_values": (oracle.fac, "attend_subset", attend_k_for_v),
    "decode_query_at_n": (oracle.decode.OracleState, "query_rot", query_at_n),
    "partial_freq_over_head_dim": (oracle.rope, "rope_rotate_partial", partial_freq_over_d),
    "partial_rotates_pass_through": (oracle.rope, "rope_rotate_partial", partial_rotates_all),
    "partial_pairs_full_layout": (oracle.rope, "fc_pairs", pairs_full_layout),
    "decode_rotates_values": (oracle.decode.OracleState, "append", append_rotates_v),
    "calib_swapped_partner": (oracle.calibrate, "fc_scores", fc_scores_swapped_partner),
    "calib_ca_unnormalised": (oracle.calibrate, "contextual_agreement", ca_unnormalised),
    "calib_ca_wrong_reference": (oracle.calibrate, "contextual_agreement", ca_against_first_fc),
    "calib_dominant_lowest": (oracle.calibrate, "dominant_from_ca", dominant_lowest),
    "calib_dominant_ties_high": (oracle.calibrate, "dominant_from_ca", dominant_ties_high),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_mutation(name, monkeypatch):
    owner, attr, fn = MUTATIONS[name]
    monkeypatch.setattr(owner, attr, fn)
    caught = []
    for pin in pins.ALL_PINS:
        try:
            pin()
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, f"no pin caught the planted mistake {name}"


def test_unmutated_oracle_passes_all_pins():
    for pin in pins.ALL_PINS:
        pin()
