"""Plain CPU oracle of the step just upstream of the attention read: rotary
encoding with YaRN-scaled and LeRoPE-multiplied frequencies, the per-head
query scaling, and the cache append.

TEST INFRASTRUCTURE ONLY (same rule as the rest of this package): only the
tests, the smoke check and the benchmark's CPU leg may call it.

Sources ("Mistral Large 4" concept page, sections "Positions" and "Query
scaling", and its executable example's YaRN wavelength function):
  * pair i < 32 of the 64-value rotary part rotates at omega_i = 10000^(-2i/64);
  * YaRN, original window 512, factor 2,048: pairs that complete at least 32
    turns within the window keep omega_i, pairs that complete less than one
    get omega_i / 2,048, and the pairs in between blend linearly in the pair
    index, between the rounded-down index where a pair completes 32 turns
    and the rounded-up index where it completes one (as the page's example
    computes it);
  * LeRoPE multiplies frequency i by a learned e^{alpha_i};
  * query scaling: each head multiplies its query by a learned function of
    position.  The formula was lost in extraction.  Reading taken here (parity
    unpinned): m_h(t) = s_h * ln(t + 1) + b_h at 0-based position t, i.e. a
    learned affine function of the log of the number of visible positions,
    after the Scalable-Softmax idea the section describes (logits times
    c ln n).
Readings for what the pages leave open: dimension pair i is (2i, 2i+1) of
the rotary part; a position rotates by the angle t * omega''_i; the scaling
multiplies the whole attention query (latent-space and rotary parts).  All
arithmetic in float64.
"""
from __future__ import annotations

import math

import numpy as np

ROPE_DIMS = 64
THETA = 10000.0
WINDOW = 512
FACTOR = 2048.0
BETA_FAST = 32.0
BETA_SLOW = 1.0


def base_frequencies() -> np.ndarray:
    """omega_i = 10000^(-2i/64), i < 32 (radians per position)."""
    i = np.arange(ROPE_DIMS // 2, dtype=np.float64)
    return THETA ** (-2.0 * i / ROPE_DIMS)


def _pair_completing(turns: float) -> float:
    """Fractional pair index whose rotation completes `turns` turns within
    the original window: solve WINDOW * omega_i = turns * 2 pi for i."""
    return ROPE_DIMS * math.log(WINDOW / (turns * 2.0 * math.pi)) / (2.0 * math.log(THETA))


def yarn_frequencies() -> np.ndarray:
    """YaRN-blended frequencies (concept page, "Positions")."""
    w = base_frequencies()
    lo = math.floor(_pair_completing(BETA_FAST))
    hi = math.ceil(_pair_completing(BETA_SLOW))
    out = np.empty_like(w)
    for i in range(w.shape[0]):
        keep = 1.0 - min(max((i - lo) / (hi - lo), 0.0), 1.0)
        out[i] = w[i] * keep + (w[i] / FACTOR) * (1.0 - keep)
    return out


def rope_frequencies(alpha=None) -> np.ndarray:
    """LeRoPE: YaRN frequency i times e^{alpha_i} (alpha None: all zero)."""
    f = yarn_frequencies()
    if alpha is not None:
        f = f * np.exp(np.asarray(alpha, np.float64))
    return f


def rotate(x, t: int, freq) -> np.ndarray:
    """Rotate the 64-value rotary vector x (float) by position t: pair i =
    (x[2i], x[2i+1]) turns by t * freq[i]."""
    x = np.asarray(x, np.float64)
    out = np.empty(ROPE_DIMS, np.float64)
    for i in range(ROPE_DIMS // 2):
        a = t * float(freq[i])
        c, s = math.cos(a), math.sin(a)
        u, v = x[2 * i], x[2 * i + 1]
        out[2 * i] = u * c - v * s
        out[2 * i + 1] = u * s + v * c
    return out


def query_scale(t: int, s, b) -> np.ndarray:
    """Per-head query multiplier m_h(t) = s_h ln(t + 1) + b_h (reading above)."""
    return np.asarray(s, np.float64) * math.log(t + 1) + np.asarray(b, np.float64)


def append_row(latent, rope_key, t: int, freq) -> np.ndarray:
    """Cache row of the token at position t: the 512-value latent, then (if
    rope_key is not None) its rotary key rotated by t."""
    lat = np.asarray(latent, np.float64)
    if rope_key is None:
        return lat.copy()
    return np.concatenate([lat, rotate(rope_key, t, freq)])


def prepare_query(q, t: int, freq, s=None, b=None) -> np.ndarray:
    """Attention query of one token, [64][512 + R]: each head scaled by
    m_h(t) (if s and b are given), the last 64 values (R = 64) rotated by t."""
    q = np.asarray(q, np.float64)
    out = q.copy()
    heads, width = q.shape
    m = query_scale(t, s, b) if s is not None else np.ones(heads)
    for h in range(heads):
        row = q[h] * m[h]
        if width > 512:
            row = np.concatenate([row[:512], rotate(row[512:], t, freq)])
        out[h] = row
    return out
