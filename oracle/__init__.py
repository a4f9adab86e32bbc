"""Oracle: a plain, slow, fp64 CPU statement of FASA's decode step.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this package.  Only the test suite, the smoke check and the CPU
baseline leg of the benchmark use it, as the yardstick the HIP path is checked
against.  It shares no code, table or helper with the HIP library and imports
nothing from it.

What it computes follows "FASA: Frequency-aware Sparse Attention":

* RoPE splits a head vector into 2-D orthogonal frequency chunks (FCs), each
  with its own angular frequency (gist.science/pt, "Resumo Tecnico" section 2,
  "A Descoberta").  ``rope.py``.
* TIP predicts each cached token's importance from the contributions of the
  per-head dominant FCs only (same section, TIP, "Previsao Online").
  ``tip.py``.
* A critical token subset T_t is chosen from those scores (same section, FAC,
  first bullet).  ``select.py``.
* Full attention runs on T_t only, with the tokens' original absolute
  positions kept (same section, FAC, second and third bullets).  ``fac.py``.
* ``decode.py`` strings these together into a decode step over a KV cache that
  grows by one row per generated token (same page, section 1, "O Problema").
* ``loops.py`` restates every step as pure-Python loops for small inputs.
* ``calibrate.py`` finds each head's dominant FCs offline from the agreement
  of single-FC scores with the full head's (same section, TIP, "Calibracao
  Offline").
* Partial RoPE (same page, "Contribuicoes": the sparsity holds under
  Partial-RoPE): ``rope.rope_rotate_partial`` and the FC pair map
  ``rope.fc_pairs``, used by TIP, calibration and the decode state.
* Budgets per head (same page, "Variantes de Implementacao": FASA composes
  with budget allocation across layers): ``select.select_topb_width`` and the
  ``head_budgets`` argument of ``OracleState.step``.

Readings where the pages are silent (rotate-half pairing, frequencies
theta^(-2c/d), the query's position, tie order, the softmax scale) are stated
in each function's docstring.

Pins: every function here is checked against closed forms, brute force or a
library routine in ``tests/test_oracle_pins.py``.  The method's end quality
against full attention on a trained model is parity unpinned (it needs
weights and data that are not part of this project).
"""

from . import rope, tip, select, fac, decode, loops, calibrate  # noqa: F401
from .rope import inv_freq, rope_rotate, rope_rotate_partial, fc_pairs, round_to_dtype  # noqa: F401
from .tip import tip_scores  # noqa: F401
from .select import select_topb, select_topb_width  # noqa: F401
from .fac import attend_subset  # noqa: F401
from .decode import OracleState  # noqa: F401
