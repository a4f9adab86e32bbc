"""The five FASA decode workloads, with their sizes.

They stand in for the settings the pages report on ("FASA: Frequency-aware
Sparse Attention"): the 256-token budget of the LongBench-V1 result (English
abstract, chatpaper.ai; gist.science/pt "Resumo Tecnico" section 4) and the
18.9% cache fraction of the AIME24 speed figure (same places).  No benchmark
item is used; every input is seeded and synthetic.

A workload's ``context`` is the number of tokens the first decode step attends
to: ``context - 1`` tokens are prefilled and the step appends the last one.
Each further step appends one more token.
"""

from dataclasses import dataclass, replace
from typing import Optional, Tuple


@dataclass(frozen=True)
class Workload:
    name: str
    config_id: int
    batch: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    context: int                 # tokens attended at step 0 (max when ragged)
    rope_theta: float
    dtype: str                   # 'f32' or 'bf16'
    budget: int
    n_dom: int                   # dominant FCs per query head
    plant_mult: float
    steps: int = 1
    context_min: Optional[int] = None   # ragged: contexts ~ U{context_min..context}
    planted_count: Optional[int] = None  # fixed count, else round(frac * context)
    planted_frac: Optional[float] = None
    spans: Optional[Tuple[int, int]] = None  # (count, length) clusters for planting
    rotary_dim: Optional[int] = None    # partial RoPE: dims rotated (None = all)

    @property
    def n_fc(self) -> int:
        return self.head_dim // 2

    @property
    def rotated(self) -> int:
        return self.head_dim if self.rotary_dim is None else self.rotary_dim

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @property
    def capacity(self) -> int:
        """Cache rows needed for all steps, rounded up to a multiple of 64."""
        need = self.context + self.steps - 1
        return (need + 63) // 64 * 64

    def planted_for(self, ctx: int) -> int:
        if self.planted_count is not None:
            return self.planted_count
        return int(round(self.planted_frac * ctx))


CONFIGS = {
    # Tiny fp32 single step: parity-focused.
    "c1": Workload("tiny_fp32_ctx512", 1, batch=1, n_q_heads=2, n_kv_heads=1,
                   head_dim=64, context=512, rope_theta=1e4, dtype="f32",
                   budget=64, n_dom=4, plant_mult=4.0, planted_count=8),
    # Llama-3-8B-shaped layer, one decode step at 32k context, B = 256.
    "c2": Workload("llama3_8b_layer_ctx32k_b256", 2, batch=1, n_q_heads=32,
                   n_kv_heads=8, head_dim=128, context=32768, rope_theta=5e5,
                   dtype="bf16", budget=256, n_dom=16, plant_mult=3.0,
                   planted_frac=0.01),
    # Batched ragged decode, contexts U{4096..8192}.
    "c3": Workload("batched16_ragged_4k_8k_b256", 3, batch=16, n_q_heads=32,
                   n_kv_heads=8, head_dim=128, context=8192, context_min=4096,
                   rope_theta=5e5, dtype="bf16", budget=256, n_dom=16,
                   plant_mult=3.0, planted_frac=0.01),
    # Long reasoning-style decode: B = 18.9% of 32k, 64 steps with append.
    "c4": Workload("reasoning_b4_ctx32k_b6193_64steps", 4, batch=4,
                   n_q_heads=32, n_kv_heads=8, head_dim=128, context=32768,
                   rope_theta=5e5, dtype="bf16", budget=6193, n_dom=12,
                   plant_mult=3.0, planted_frac=0.02, steps=64),
    # Very long context: 128k, B = 1024, planting clustered in 16 x 64 spans.
    "c5": Workload("long_ctx128k_b1024_32steps", 5, batch=1, n_q_heads=32,
                   n_kv_heads=8, head_dim=128, context=131072, rope_theta=5e5,
                   dtype="bf16", budget=1024, n_dom=8, plant_mult=3.0,
                   planted_frac=0.005, steps=32, spans=(16, 64)),
    # Partial RoPE: the 32k Llama-3-shaped layer with only the first half of
    # each head rotated (rotary_dim 64 of 128, theta 1e4); the pages name no
    # model for it, so the shape is the 32k layer's.
    "c6": Workload("partial_rope_r64_ctx32k_b256", 6, batch=1, n_q_heads=32,
                   n_kv_heads=8, head_dim=128, context=32768, rope_theta=1e4,
                   dtype="bf16", budget=256, n_dom=16, plant_mult=3.0,
                   planted_frac=0.01, rotary_dim=64),
}


def get(name: str) -> Workload:
    return CONFIGS[name]


def shrink(w: Workload, **kw) -> Workload:
    """A smaller copy (for parity at sizes the oracle finishes in seconds)."""
    return replace(w, **kw)
