"""Seeded input generation for the FASA decode workloads.

Recipe (every choice is a reading; the pages fix none of it):

* seeds: ``numpy.random.SeedSequence([seed, config_id, stream])`` with one
  PCG64 stream per kind of tensor, so changing one size does not reshuffle
  the others;
* dominant FCs: per query head, ``n_dom`` FC indices drawn uniformly without
  replacement from the d/2 FCs, sorted;
* pre-RoPE q, k, v ~ N(0, 1), rounded to the cache dtype (bf16: round to
  nearest even from fp32);
* contexts: fixed, or per sequence ~ U{context_min .. context} (ragged);
* planted salient positions: ``planted_for(context)`` positions per sequence,
  drawn without replacement from the prefilled range [0, context - 1) (or
  from ``spans`` non-overlapping clusters of equal length); at each one, for
  every KV head and for every dominant FC of that head's query heads (query
  heads visited in ascending order, first one wins for a shared FC), the key
  pair is turned so that, once both are rotated to their positions, it points
  along step 0's query pair, with its own length times ``plant_mult``;
* steps after the first get fresh N(0, 1) queries; appended rows are plain
  N(0, 1).

Planting needs the relative angle between the query's and the key's
positions, (t_q - t_k) * omega_c, omega_c = theta^(-2c/r) for the r rotated
dims (r = d unless the workload has a rotary_dim; pass-through pairs have
omega 0), and each FC's dimension pair; both are formed here, with a complex
phasor, purely to shape the inputs.  Nothing downstream reads it, and a
mistake in it would only make planted tokens less salient.
"""

import numpy as np

from .configs import Workload

S_DOM, S_CTX, S_Q, S_K, S_V, S_PLANT, S_KNEW, S_VNEW, S_SPAN = range(9)


def _rng(seed: int, cfg: int, stream: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(
        np.random.SeedSequence([seed, cfg, stream])))


def round_bf16(x) -> np.ndarray:
    """fp32 -> nearest-even bf16 value, returned as fp32."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).copy()
    u += np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    u &= np.uint32(0xFFFF0000)
    return u.view(np.float32)


def to_bf16_bits(x) -> np.ndarray:
    """bf16-representable fp32 values -> their uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    return (u >> np.uint32(16)).astype(np.uint16)


def _normal(rng, shape, dtype):
    x = rng.standard_normal(size=shape, dtype=np.float32)
    return round_bf16(x) if dtype == "bf16" else x


def _cast(x, dtype):
    x = np.asarray(x, dtype=np.float32)
    return round_bf16(x) if dtype == "bf16" else x


def _plant_positions(w: Workload, rng_plant, rng_span, ctx: int):
    count = w.planted_for(ctx)
    avail = ctx - 1  # prefilled positions 0 .. ctx-2
    if w.spans is None:
        count = min(count, avail)
        return np.sort(rng_plant.choice(avail, size=count, replace=False))
    n_span, length = w.spans
    free = avail - n_span * (length - 1)
    if free < n_span:
        raise ValueError("spans do not fit in the context")
    x = np.sort(rng_span.choice(free, size=n_span, replace=False))
    starts = x + np.arange(n_span) * (length - 1)
    slots = (starts[:, None] + np.arange(length)[None, :]).reshape(-1)
    count = min(count, slots.size)
    return np.sort(rng_plant.choice(slots, size=count, replace=False))


def plant_ladder(w):
    """The frequency of every FC and its dimension pair (lo, hi), as the
    planting aligns keys with the query: frequencies theta^(-2c/r) for the r
    rotated dims' FCs and 0 for pass-through FCs; pairs (c, c + R) for
    c < R = r/2, else the pass-through dims paired in order.  Only the
    planting uses it; tests hold it against the oracle's own tables."""
    d, r_dim = w.head_dim, w.rotated
    half, R = d // 2, r_dim // 2
    ci = np.arange(half)
    omega = np.where(ci < R, np.power(float(w.rope_theta), -2.0 * np.minimum(ci, R) / r_dim), 0.0)
    lo_d = np.where(ci < R, ci, r_dim + ci - R)
    hi_d = np.where(ci < R, ci + R, r_dim + ci - R + (d - r_dim) // 2)
    return omega, lo_d, hi_d


def generate(w: Workload, seed: int = 0xFA5A, with_prefill: bool = True):
    """Draw every input of workload ``w``.

    Returns a dict of NumPy arrays (values exactly representable in w.dtype):
      dom        int32  [Hq, n_dom]
      ctx        int64  [b]             tokens attended at step 0
      q          fp32   [steps, b, Hq, d]
      k_prefill  fp32   [b, Hkv, max(ctx) - 1, d]  (rows >= ctx[b]-1 unused)
      v_prefill  fp32   same
      k_new      fp32   [steps, b, Hkv, d]  row appended at each step
      v_new      fp32   same
      planted    list of int64 arrays, one per sequence
    """
    b, hq, hkv, d = w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim
    half, grp = d // 2, w.group
    cid = w.config_id

    r = _rng(seed, cid, S_DOM)
    dom = np.stack([np.sort(r.choice(half, size=w.n_dom, replace=False))
                    for _ in range(hq)]).astype(np.int32)

    if w.context_min is None:
        ctx = np.full(b, w.context, dtype=np.int64)
    else:
        ctx = _rng(seed, cid, S_CTX).integers(
            w.context_min, w.context + 1, size=b).astype(np.int64)

    q = _normal(_rng(seed, cid, S_Q), (w.steps, b, hq, d), w.dtype)
    k_new = _normal(_rng(seed, cid, S_KNEW), (w.steps, b, hkv, d), w.dtype)
    v_new = _normal(_rng(seed, cid, S_VNEW), (w.steps, b, hkv, d), w.dtype)
    out = {"dom": dom, "ctx": ctx, "q": q, "k_new": k_new, "v_new": v_new,
           "planted": []}

    rp, rs = _rng(seed, cid, S_PLANT), _rng(seed, cid, S_SPAN)
    planted = [_plant_positions(w, rp, rs, int(ctx[i])) for i in range(b)]
    out["planted"] = planted
    if not with_prefill:
        return out

    L = int(ctx.max()) - 1
    k = _normal(_rng(seed, cid, S_K), (b, hkv, L, d), w.dtype)
    v = _normal(_rng(seed, cid, S_V), (b, hkv, L, d), w.dtype)

    # Planting (see module docstring).
    omega, lo_d, hi_d = plant_ladder(w)
    for i in range(b):
        pos = planted[i]
        if pos.size == 0:
            continue
        t_q = int(ctx[i]) - 1
        for g in range(hkv):
            owner = np.full(half, -1, dtype=np.int64)
            for h in range(g * grp, (g + 1) * grp):
                for c in dom[h]:
                    if owner[c] < 0:
                        owner[c] = h
            cs = np.nonzero(owner >= 0)[0]
            hs = owner[cs]
            lo, hi = lo_d[cs], hi_d[cs]
            zq = q[0, i, hs, lo].astype(np.float64) + 1j * q[0, i, hs, hi]
            zk = (k[i, g][np.ix_(pos, lo)].astype(np.float64)
                  + 1j * k[i, g][np.ix_(pos, hi)])
            phase = np.exp(1j * np.outer(t_q - pos, omega[cs]))
            nz = np.where(np.abs(zq) > 0, zq / np.maximum(np.abs(zq), 1e-300), 1.0)
            znew = w.plant_mult * np.abs(zk) * nz[None, :] * phase
            k[i, g][np.ix_(pos, lo)] = _cast(znew.real, w.dtype)
            k[i, g][np.ix_(pos, hi)] = _cast(znew.imag, w.dtype)

    out["k_prefill"], out["v_prefill"] = k, v
    return out


def random_scores(seed: int, rows: int, n: int, kind: str) -> np.ndarray:
    """Seeded fp32 score rows [rows, n] for selection tests.

    kinds: 'normal' (N(0,1)), 'ties' (few distinct values), 'zeros' (all +0
    and -0), 'wide' (magnitudes across 1e-30..1e30, both signs), 'sorted_up'
    (strictly increasing), 'planted' (N(0,1) with a 1% block of large values).
    """
    r = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 0xC0DE, rows, n])))
    if kind == "normal":
        x = r.standard_normal((rows, n))
    elif kind == "ties":
        x = r.integers(-3, 4, size=(rows, n)).astype(np.float64) * 0.5
    elif kind == "zeros":
        x = np.where(r.random((rows, n)) < 0.5, 0.0, -0.0)
    elif kind == "wide":
        x = r.standard_normal((rows, n)) * 10.0 ** r.uniform(-30, 30, (rows, n))
    elif kind == "sorted_up":
        x = np.tile(np.arange(n, dtype=np.float64), (rows, 1))
    elif kind == "planted":
        x = r.standard_normal((rows, n))
        k = max(1, n // 100)
        for i in range(rows):
            x[i, r.choice(n, size=k, replace=False)] += 6.0
    else:
        raise ValueError(kind)
    return np.ascontiguousarray(x.astype(np.float32))


def head_budgets(seed: int, n_heads: int, budget: int, kind: str) -> np.ndarray:
    """Seeded per-query-head budgets int32 [n_heads], each in [0, budget].

    kinds: 'edges' (0, 1, budget, budget - 1, then uniform draws), 'uniform'
    (uniform draws in [0, budget]), 'ramp' (round(budget (h + 0.5) / n_heads):
    a linear allocation whose mean is budget / 2).
    """
    r = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 0xB0D6, n_heads, budget])))
    if kind == "ramp":
        x = np.round(budget * (np.arange(n_heads) + 0.5) / n_heads)
    elif kind == "uniform":
        x = r.integers(0, budget + 1, size=n_heads)
    elif kind == "edges":
        x = r.integers(0, budget + 1, size=n_heads)
        head = [0, 1, budget, max(budget - 1, 0)]
        x[:min(4, n_heads)] = head[:min(4, n_heads)]
    else:
        raise ValueError(kind)
    return np.clip(x, 0, budget).astype(np.int32)
