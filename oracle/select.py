"""Selection of the critical token set T_t (test infrastructure only).

Source: "FASA: Frequency-aware Sparse Attention", gist.science/pt, "Resumo
Tecnico" section 2, FAC, first bullet: from the TIP scores the system picks a
critical subset of tokens T_t.  The English abstract's headline setting keeps
256 tokens; the lay pages (gist.science/pt "Etapa 1", gist.science/ja step 1)
describe keeping the 256 most important tokens.

Readings: T_t holds the min(B, n) highest-scoring tokens; equal scores go to
the lower position; no token is forced in (no sink, no recent window).  It is
reported in ascending position order and padded with -1 up to B.
"""

import numpy as np


def select_topb(scores, budget: int) -> np.ndarray:
    """Top-``budget`` positions of ``scores`` [n] by (score desc, position asc).

    Returns int64 [budget]: the chosen positions ascending, then -1 padding.
    """
    s = np.asarray(scores, dtype=np.float64)
    n = s.shape[0]
    take = min(budget, n)
    # Sort by (-score, position): lexsort's last key is the primary one.
    order = np.lexsort((np.arange(n), -s))
    chosen = np.sort(order[:take].astype(np.int64))
    out = np.full(budget, -1, dtype=np.int64)
    out[:take] = chosen
    return out


def threshold(scores, budget: int) -> float:
    """tau: the score of the budget-th ranked token, i.e. the smallest score
    T_t keeps (with budget >= n every token is kept, so the smallest score of
    the row).  Raises ValueError for budget < 1 or an empty row, where T_t
    keeps nothing and no such score exists."""
    if budget < 1:
        raise ValueError(f"budget {budget} < 1: T_t is empty and has no threshold")
    s = np.sort(np.asarray(scores, dtype=np.float64))[::-1]
    if s.shape[0] == 0:
        raise ValueError("empty row: T_t is empty and has no threshold")
    return float(s[min(budget, s.shape[0]) - 1])


def select_topb_width(scores, budget: int, width: int) -> np.ndarray:
    """T_t of a head whose budget is ``budget`` (0 <= budget <= width), in a
    row ``width`` wide: the set ascending, then -1 padding.  int64 [width]."""
    if not 0 <= budget <= width:
        raise ValueError(f"budget {budget} not in [0, {width}]")
    out = np.full(width, -1, dtype=np.int64)
    out[:budget] = select_topb(scores, budget)
    return out
