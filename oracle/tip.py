"""Token Importance Prediction (TIP), fp64 (test infrastructure only).

Source: "FASA: Frequency-aware Sparse Attention", gist.science/pt, "Resumo
Tecnico" section 2, TIP, "Previsao Online": during decoding, instead of the
full attention score, FASA adds up only the contributions of the pre-calibrated
dominant FCs (I_dom, found offline per head) to estimate each cached token's
importance.  The English abstract (chatpaper.ai) calls this proxy
computationally free.

Reading: the contribution of FC c is the 2-D dot product of the rotated query
pair with the rotated key pair,
    s_j = sum_{c in I_dom(h)} (q~_c k~_{j,c} + q~_{c+C} k~_{j,c+C}),
a raw sum with no 1/sqrt(d) and no per-FC softmax (neither changes the
ranking that selection uses).  Under partial RoPE an FC's two dimensions are
those rope.py names (pass-through pairs at frequency 0).
"""

import numpy as np


def tip_scores(q_rot, k_rot, dom, pairs=None) -> np.ndarray:
    """TIP scores of one query head against cached keys.

    q_rot: [d] rotated query (fp64).
    k_rot: [n, d] rotated cached keys.
    dom:   dominant FC indices of this head (values in 0 .. d/2 - 1).
    pairs: (lo, hi) dimension pair of every FC (rope.fc_pairs); None is the
           full-RoPE layout (c, c + d/2).
    Returns fp64 [n].
    """
    q = np.asarray(q_rot, dtype=np.float64)
    k = np.asarray(k_rot, dtype=np.float64)
    half = q.shape[-1] // 2
    dom = np.asarray(dom, dtype=np.int64)
    if pairs is None:
        cols = np.concatenate([dom, dom + half])
    else:
        cols = np.concatenate([np.asarray(pairs[0])[dom], np.asarray(pairs[1])[dom]])
    return k[:, cols] @ q[cols]
