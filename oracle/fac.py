"""Focused Attention Computation (FAC), fp64 (test infrastructure only).

Source: "FASA: Frequency-aware Sparse Attention", gist.science/pt, "Resumo
Tecnico" section 2, FAC, second and third bullets: full, high-fidelity
attention is executed over the reduced token subset only, and the tokens'
original absolute positions are kept, so the cached (already rotated) keys are
used as they are.

Reading: standard scaled dot-product attention restricted to T_t,
    z_j = q~ . k~_j / sqrt(d),  w = softmax over j in T_t,  o = sum_j w_j v_j,
with the softmax normalised over T_t only.
"""

import numpy as np


def attend_subset(q_rot, k_rot, v, subset) -> np.ndarray:
    """Attention of one query over the rows ``subset`` of the cache.

    q_rot: [d]; k_rot: [n, d] rotated keys; v: [n, d] values;
    subset: positions (entries < 0 are padding and ignored).
    Returns fp64 [d].
    """
    q = np.asarray(q_rot, dtype=np.float64)
    idx = np.asarray(subset, dtype=np.int64)
    idx = idx[idx >= 0]
    if idx.size == 0:
        return np.zeros(q.shape[-1], dtype=np.float64)
    k = np.asarray(k_rot, dtype=np.float64)[idx]
    vv = np.asarray(v, dtype=np.float64)[idx]
    z = (k @ q) / np.sqrt(q.shape[-1])
    w = np.exp(z - z.max())
    w /= w.sum()
    return w @ vv
