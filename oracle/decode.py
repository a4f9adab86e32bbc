"""One FASA decode step over a growing KV cache, fp64 (test infrastructure only).

Source: "FASA: Frequency-aware Sparse Attention", gist.science/pt, "Resumo
Tecnico" section 1 (every generated token reads the whole KV cache, which grows
with the sequence) and section 2 (TIP scores the cached tokens with the
dominant FCs, T_t is selected, FAC attends over T_t keeping absolute
positions); FASA-C (same section, "Variantes de Implementacao") keeps the
whole cache on the GPU and only reads a sparse subset, so nothing is evicted
for good.

Readings:
* cache slot j holds the token at absolute position j; keys are stored after
  RoPE at that position, rounded once to the cache dtype; values as given;
* a decode step first appends the new token's K/V at position n_b - 1 and then
  attends over all n_b cached tokens, the query sitting at position n_b - 1;
* grouped-query attention: query head h reads KV head h // (Hq / Hkv), and
  selection is done per query head;
* I_dom is per query head and fixed across sequences and steps.
"""

import numpy as np

from . import rope, tip, select, fac


class OracleState:
    """fp64 copy of the cache: K~ (rotated, dtype-rounded) and V per sequence."""

    def __init__(self, batch, n_q_heads, n_kv_heads, head_dim, rope_theta,
                 dtype, dom, capacity, rotary_dim=None):
        if n_q_heads % n_kv_heads:
            raise ValueError("n_q_heads must be a multiple of n_kv_heads")
        self.batch, self.hq, self.hkv = batch, n_q_heads, n_kv_heads
        self.group = n_q_heads // n_kv_heads
        self.d, self.theta, self.dtype = head_dim, float(rope_theta), dtype
        self.dom = np.asarray(dom, dtype=np.int64)
        self.K = np.zeros((batch, n_kv_heads, capacity, head_dim), np.float64)
        self.V = np.zeros((batch, n_kv_heads, capacity, head_dim), np.float64)
        self.lens = np.zeros(batch, dtype=np.int64)
        # Partial RoPE (rope.py): rotary_dim < head_dim rotates the first
        # rotary_dim dims only; None or head_dim is full RoPE.
        self.rotary_dim = None if rotary_dim in (None, head_dim) else int(rotary_dim)
        self.pairs = None if self.rotary_dim is None else rope.fc_pairs(head_dim, self.rotary_dim)

    def _rotate(self, x, pos):
        if self.rotary_dim is None:
            return rope.rope_rotate(x, pos, self.theta)
        return rope.rope_rotate_partial(x, pos, self.theta, self.rotary_dim)

    def append(self, b, k_new, v_new):
        """Append rows at positions lens[b] ..; k_new, v_new: [Hkv, n_new, d]."""
        k_new = np.asarray(k_new, dtype=np.float64)
        n_new = k_new.shape[1]
        p0 = int(self.lens[b])
        pos = np.arange(p0, p0 + n_new)
        self.K[b, :, p0:p0 + n_new] = rope.round_to_dtype(
            self._rotate(k_new, pos[None, :]), self.dtype)
        self.V[b, :, p0:p0 + n_new] = np.asarray(v_new, dtype=np.float64)
        self.lens[b] = p0 + n_new

    def query_rot(self, b, q):
        """Rotated queries [Hq, d] at position lens[b] - 1 (not re-rounded)."""
        return self._rotate(q, int(self.lens[b]) - 1)

    def kv_head(self, h):
        return h // self.group

    def head_scores(self, b, h, q_rot_h):
        n = int(self.lens[b])
        return tip.tip_scores(q_rot_h, self.K[b, self.kv_head(h), :n], self.dom[h],
                              self.pairs)

    def attend(self, b, h, q_rot_h, subset):
        n = int(self.lens[b])
        g = self.kv_head(h)
        return fac.attend_subset(q_rot_h, self.K[b, g, :n], self.V[b, g, :n], subset)

    def step(self, q, k_new, v_new, budget, heads=None, head_budgets=None):
        """One decode step for every sequence.

        q: [b, Hq, d] pre-RoPE queries; k_new, v_new: [b, Hkv, d] pre-RoPE.
        ``heads`` limits the query heads computed (the rest stay zero / -1).
        ``head_budgets`` ([Hq], each in [0, budget]) gives query head h the
        budget head_budgets[h] (select.py, budgets per head); idx rows stay
        ``budget`` wide.
        Returns dict with idx [b, Hq, budget], out [b, Hq, d], tau [b, Hq]
        (NaN for a head of budget 0) and the per-(b, h) score vectors in
        ``scores``.
        """
        heads = range(self.hq) if heads is None else heads
        bh = [budget] * self.hq if head_budgets is None else [int(x) for x in head_budgets]
        idx = np.full((self.batch, self.hq, budget), -1, dtype=np.int64)
        out = np.zeros((self.batch, self.hq, self.d), dtype=np.float64)
        tau = np.zeros((self.batch, self.hq), dtype=np.float64)
        scores = {}
        for b in range(self.batch):
            self.append(b, np.asarray(k_new)[b][:, None, :],
                        np.asarray(v_new)[b][:, None, :])
            qr = self.query_rot(b, np.asarray(q)[b])
            for h in heads:
                s = self.head_scores(b, h, qr[h])
                sel = select.select_topb_width(s, bh[h], budget)
                idx[b, h] = sel
                tau[b, h] = select.threshold(s, bh[h]) if bh[h] > 0 else np.nan
                out[b, h] = self.attend(b, h, qr[h], sel)
                scores[(b, h)] = s
        return {"idx": idx, "out": out, "tau": tau, "scores": scores}
