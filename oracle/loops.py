"""Every oracle step again, as pure-Python loops (test infrastructure only).

Meant for small inputs (n up to a few hundred, d up to 128).  They follow the
same passages and readings as ``rope.py``, ``tip.py``, ``select.py`` and
``fac.py`` ("FASA: Frequency-aware Sparse Attention", gist.science/pt,
"Resumo Tecnico" section 2) but use scalar ``math`` only, so a vectorisation
slip in the NumPy versions (a wrong axis, a broadcast) shows up as a mismatch.
"""

import math


def rope_loop(x, pos, theta):
    d = len(x)
    half = d // 2
    y = [0.0] * d
    for c in range(half):
        w = math.pow(theta, -2.0 * c / d)
        a = pos * w
        co, si = math.cos(a), math.sin(a)
        y[c] = x[c] * co - x[c + half] * si
        y[c + half] = x[c + half] * co + x[c] * si
    return y


def tip_loop(q_rot, k_rows, dom):
    half = len(q_rot) // 2
    out = []
    for k in k_rows:
        s = 0.0
        for c in dom:
            s += q_rot[c] * k[c] + q_rot[c + half] * k[c + half]
        out.append(s)
    return out


def topb_loop(scores, budget):
    n = len(scores)
    ranked = sorted(range(n), key=lambda j: (-scores[j], j))
    chosen = sorted(ranked[:min(budget, n)])
    return chosen + [-1] * (budget - len(chosen))


def attend_loop(q_rot, k_rows, v_rows, subset):
    d = len(q_rot)
    sel = [j for j in subset if j >= 0]
    if not sel:
        return [0.0] * d
    z = {}
    for j in sel:
        z[j] = sum(q_rot[i] * k_rows[j][i] for i in range(d)) / math.sqrt(d)
    m = max(z.values())
    e = {j: math.exp(z[j] - m) for j in sel}
    tot = sum(e.values())
    out = [0.0] * d
    for j in sel:
        for i in range(d):
            out[i] += e[j] / tot * v_rows[j][i]
    return out
