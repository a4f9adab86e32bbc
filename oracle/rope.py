"""RoPE and its frequency chunks, in fp64 (test infrastructure only).

Source: "FASA: Frequency-aware Sparse Attention", gist.science/pt, "Resumo
Tecnico" section 2, "A Descoberta": RoPE splits the attention vectors into
2-D orthogonal subspaces, the frequency chunks (FCs), each tied to one angular
frequency.  The page gives no formula; the readings used here are:

* pairing: rotate-half, FC c is the dimension pair (c, c + d/2), c = 0..d/2-1;
* frequency of FC c: omega_c = theta ** (-2c/d);
* the angle at absolute position m is m * omega_c, taken in fp64;
* rotation direction: (x_c + i x_{c+C}) is multiplied by exp(+i m omega_c).

Rounding to the cache dtype happens once, round-to-nearest-even, on the fp64
rotated value (``round_to_dtype``).

Partial RoPE.  The same page's "Contribuicoes" claim that the functional
sparsity also holds under Partial-RoPE; it gives no layout.  Reading: only the
first r (even) dimensions of a head are rotated, rotate-half within them, with
frequencies theta ** (-2c/r), c < R = r/2; dimensions r .. d-1 pass through.
The FCs are then:
* c < R: the pair (c, c + R) at omega_c = theta ** (-2c/r);
* c >= R: the pass-through dimensions paired the same way,
  (r + i, r + i + (d - r)/2) with i = c - R, at frequency 0 (no rotation).
With r = d this is the full layout above.
"""

import numpy as np


def inv_freq(head_dim: int, theta: float) -> np.ndarray:
    """omega_c = theta ** (-2c/d) for c = 0 .. d/2 - 1, fp64."""
    if head_dim % 2:
        raise ValueError("head_dim must be even")
    c = np.arange(head_dim // 2, dtype=np.float64)
    return np.power(np.float64(theta), -2.0 * c / head_dim)


def rope_rotate(x, pos, theta: float) -> np.ndarray:
    """Rotate each FC of ``x`` by its angle at absolute position ``pos``.

    x:   array [..., d]; any float dtype, computed in fp64.
    pos: integer array broadcastable to x.shape[:-1] (or a scalar).
    Returns fp64 [..., d]:
        y_c     = x_c cos(phi_c) - x_{c+C} sin(phi_c)
        y_{c+C} = x_{c+C} cos(phi_c) + x_c sin(phi_c),  phi_c = pos * omega_c.
    """
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    half = d // 2
    w = inv_freq(d, theta)
    p = np.asarray(pos, dtype=np.float64)[..., None]
    phi = p * w
    cos, sin = np.cos(phi), np.sin(phi)
    lo, hi = x[..., :half], x[..., half:]
    return np.concatenate([lo * cos - hi * sin, hi * cos + lo * sin], axis=-1)


def rope_rotate_partial(x, pos, theta: float, rotary_dim: int) -> np.ndarray:
    """Partial RoPE: rotate-half over the first ``rotary_dim`` dims of ``x``
    at absolute position ``pos`` with frequencies theta ** (-2c/rotary_dim);
    the remaining dims are returned unchanged.  fp64 [..., d]."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    r = int(rotary_dim)
    if r % 2 or not 2 <= r <= d:
        raise ValueError(f"rotary_dim {r} must be even and in [2, {d}]")
    R = r // 2
    w = np.power(np.float64(theta), -2.0 * np.arange(R, dtype=np.float64) / r)
    phi = np.asarray(pos, dtype=np.float64)[..., None] * w
    cos, sin = np.cos(phi), np.sin(phi)
    a, b = x[..., :R], x[..., R:r]
    out = x.copy()
    out[..., :R] = a * cos - b * sin
    out[..., R:r] = b * cos + a * sin
    return out


def fc_pairs(head_dim: int, rotary_dim: int = None):
    """Dimension pair (lo[c], hi[c]) of every FC c = 0 .. d/2 - 1 (module
    docstring: full and partial RoPE).  int64 arrays [d/2]."""
    d = int(head_dim)
    r = d if rotary_dim is None else int(rotary_dim)
    R, P = r // 2, (d - r) // 2
    c = np.arange(d // 2, dtype=np.int64)
    i = c - R
    lo = np.where(c < R, c, r + i)
    hi = np.where(c < R, c + R, r + i + P)
    return lo, hi


def round_to_dtype(x, dtype: str) -> np.ndarray:
    """Round fp64 values once to ``dtype`` ('f32' or 'bf16'), nearest-even.

    Returns fp64 holding exactly representable values.  bf16 has fp32's
    exponent range and 8 significant bits, so the grid spacing for |x| in
    [2^k, 2^(k+1)) is 2^(k-7), and 2^-133 below the normal range.
    """
    x = np.asarray(x, dtype=np.float64)
    if dtype == "f32":
        return x.astype(np.float32).astype(np.float64)
    if dtype != "bf16":
        raise ValueError(f"unknown dtype {dtype!r}")
    _, e = np.frexp(x)  # x = f * 2^e, 0.5 <= |f| < 1, so |x| in [2^(e-1), 2^e)
    spacing = np.ldexp(1.0, np.maximum(e - 8, -133))
    out = np.rint(x / spacing) * spacing  # rint: ties to even
    out[x == 0] = x[x == 0]
    if np.any(np.abs(out) > 3.3895313892515355e38):
        raise OverflowError("value outside the bf16 range")
    return out
