"""Offline calibration of the dominant FCs, fp64 (test infrastructure only).

Source: "FASA: Frequency-aware Sparse Attention", gist.science/pt, "Resumo
Tecnico" section 2, TIP, "Calibracao Offline": once, before decoding, the
indices of the dominant FCs (I_dom) of every attention head are found from a
"Contextual Agreement" (CA) between the attention scores of a single FC and
those of the full head, on a small calibration set.  Same page, section 4,
"Robustez": the result is insensitive to the calibration window and set.

The pages give no formula for CA.  Reading (the plainest one the rest
supports, since the scores only ever serve to pick a top-B set):
  * FC c's score of token j is its 2-D dot product,
        s_c[j] = q~_c k~_{j,c} + q~_{c+C} k~_{j,c+C},
    and the full head's is s[j] = sum_c s_c[j] = q~ . k~_j;
  * CA(c) = |top_k(s_c) intersect top_k(s)| / k for one calibration query,
    with top_k the selection rule of select.py (ties to the lower position),
    averaged over the calibration queries;
  * I_dom(h) = the n_dom FCs of highest mean CA, equal CA to the lower FC,
    listed ascending.
"""

import numpy as np

from . import select


def fc_scores(q_rot, k_rot, pairs=None) -> np.ndarray:
    """Per-FC scores of one query head: fp64 [C, n], s_c[j] as above.

    q_rot: [d] rotated query; k_rot: [n, d] rotated keys; pairs: (lo, hi)
    dimensions of every FC (rope.fc_pairs), None for the full layout.
    """
    q = np.asarray(q_rot, dtype=np.float64)
    k = np.asarray(k_rot, dtype=np.float64)
    half = q.shape[-1] // 2
    if pairs is None:
        return (k[:, :half] * q[None, :half]).T + (k[:, half:] * q[None, half:]).T
    lo, hi = np.asarray(pairs[0]), np.asarray(pairs[1])
    return (k[:, lo] * q[None, lo]).T + (k[:, hi] * q[None, hi]).T


def contextual_agreement(q_rot, k_rot, topk: int, pairs=None) -> np.ndarray:
    """CA of every FC for one calibration query: fp64 [C] in [0, 1]."""
    s_c = fc_scores(q_rot, k_rot, pairs)
    n = s_c.shape[1]
    k = min(topk, n)
    full = set(select.select_topb(s_c.sum(axis=0), k).tolist())
    out = np.empty(s_c.shape[0], dtype=np.float64)
    for c in range(s_c.shape[0]):
        mine = select.select_topb(s_c[c], k)
        out[c] = len(full.intersection(mine.tolist())) / k
    return out


def dominant_from_ca(ca, n_dom: int) -> np.ndarray:
    """I_dom per head from CA values [samples, heads, C] (or [heads, C]).

    Mean over samples, then the n_dom highest per head, equal means to the
    lower FC; returned ascending, int32 [heads, n_dom].
    """
    a = np.asarray(ca, dtype=np.float64)
    if a.ndim == 3:
        a = a.mean(axis=0)
    heads, C = a.shape
    out = np.empty((heads, n_dom), dtype=np.int32)
    for h in range(heads):
        order = np.lexsort((np.arange(C), -a[h]))
        out[h] = np.sort(order[:n_dom])
    return out
