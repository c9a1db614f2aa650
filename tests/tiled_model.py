"""Float64 model of tiled attention built on one combine operation (test helper, not the oracle).

The oracle evaluates the plain definition. This module reaches the same result the way a
tiled kernel does, with the keys taken a tile or a chunk at a time, so agreement between
the two (to float64 rounding) pins the oracle against an independent formulation, and the
intermediate states can be compared with the ones the pages print.

Everything here is a fold of one operation on partial results. The partial result of a
query row over a set of keys is the triple (m, l, o): m the largest visible score, l the sum
of exp(s - m) over the visible keys and o the same weights applied to the value rows. Two
partials over disjoint key sets combine into the partial over their union by bringing both
to the larger of the two maxima (factors exp(m_a - m) and exp(m_b - m)); a partial with no
visible key (m = -inf, l = 0, o = 0) is the neutral element and takes factor 0, so -inf - -inf
is never formed. The pages' two forms are both this combine:
- the running update by a new tile, where the new tile's partial is taken against its own
  max and combined into the running state ("FlashAttention: Attention Is Limited by Memory,
  Not Math", section "How tiling and online softmax stay exact"; "Explain FlashAttention
  ...", section "Keep only the state needed for the final weighted average"; a fully masked
  tile is neutral, which is the empty-state policy of section "Executable recurrence, with
  an empty-state policy");
- the merge of chunk states computed against their own maxima ("Flash Attention
  Optimization", section "The fix: tile the computation, never materialize the full
  matrix"; "Handwritten Notes on Flash Attention", section "Merging two blocks").
The result is o / l and LSE = m + ln l; a row that saw no key gives (0, -inf).

All functions work on every query row of one head at once (arrays over rows).
"""
from __future__ import annotations

import math
from typing import NamedTuple

import numpy as np

NEG_INF = -math.inf


class Partial(NamedTuple):
    m: np.ndarray      # [rows] largest visible score, -inf if none
    l: np.ndarray      # [rows] sum of exp(s - m)
    o: np.ndarray      # [rows, dv] sum of exp(s - m) * v


def empty(rows: int, dv: int) -> Partial:
    return Partial(np.full(rows, NEG_INF), np.zeros(rows), np.zeros((rows, dv)))


def _finite_or_zero(x: np.ndarray) -> np.ndarray:
    return np.where(np.isfinite(x), x, 0.0)


def of_keys(s: np.ndarray, v: np.ndarray) -> Partial:
    """Partial over a block of keys: scores s [rows, n] (-inf = hidden), values v [n, dv],
    taken against the block's own row maxima."""
    rows, n = s.shape
    if n == 0:
        return empty(rows, v.shape[1])
    m = s.max(axis=1)
    w = np.exp(s - _finite_or_zero(m)[:, None])   # hidden scores give exactly 0
    return Partial(m, w.sum(axis=1), w @ v)


def factors(a: Partial, b: Partial):
    """The two factors that bring a and b to their common max (0 for an empty side)."""
    m = np.maximum(a.m, b.m)
    base = _finite_or_zero(m)
    fa = np.where(np.isfinite(a.m), np.exp(_finite_or_zero(a.m) - base), 0.0)
    fb = np.where(np.isfinite(b.m), np.exp(_finite_or_zero(b.m) - base), 0.0)
    return m, fa, fb


def combine(a: Partial, b: Partial) -> Partial:
    """Partial over the union of the two disjoint key sets of a and b."""
    m, fa, fb = factors(a, b)
    return Partial(m, fa * a.l + fb * b.l, fa[:, None] * a.o + fb[:, None] * b.o)


def finish(p: Partial):
    """(output rows, log-sum-exp per row); rows that saw no key give (0, -inf)."""
    seen = p.l > 0
    l_safe = np.where(seen, p.l, 1.0)
    o = np.where(seen[:, None], p.o / l_safe[:, None], 0.0)
    lse = np.where(seen, p.m + np.log(l_safe), NEG_INF)
    return o, lse


def scores(q: np.ndarray, k: np.ndarray, scale: float, causal: bool) -> np.ndarray:
    """Scaled scores [Nq, Nk] of one head with -inf at masked positions.

    Causal masking uses absolute positions with the query block aligned to the
    end of the key sequence: query i may see key j iff j <= i + (Nk - Nq).
    """
    nq, nk = q.shape[0], k.shape[0]
    s = (q @ k.T) * scale
    if causal:
        i = np.arange(nq)[:, None]
        j = np.arange(nk)[None, :]
        s = np.where(j <= i + (nk - nq), s, NEG_INF)
    return s


def bounds(nk: int, size: int):
    """[lo, hi) of consecutive key blocks of ``size`` (the last may be short)."""
    return [(lo, min(nk, lo + size)) for lo in range(0, nk, size)]


def tiled_head(q, k, v, scale, causal, tile):
    """Attention for one head, key tiles of ``tile`` folded left to right into a running
    partial."""
    s = scores(q, k, scale, causal)
    acc = empty(s.shape[0], v.shape[1])
    for lo, hi in bounds(s.shape[1], tile):
        acc = combine(acc, of_keys(s[:, lo:hi], v[lo:hi]))
    return finish(acc)


def split_merge_head(q, k, v, scale, causal, num_splits):
    """Attention for one head with the keys split into num_splits chunks of ceil(Nk/S)
    (trailing chunks may be short or empty), one partial per chunk, merged afterwards by a
    balanced tree of combines (a different association than the running fold)."""
    s = scores(q, k, scale, causal)
    nk = s.shape[1]
    chunk = -(-nk // num_splits)
    parts = [of_keys(s[:, c * chunk:min(nk, (c + 1) * chunk)], v[c * chunk:min(nk, (c + 1) * chunk)])
             for c in range(num_splits)]
    while len(parts) > 1:
        parts = [combine(parts[i], parts[i + 1]) if i + 1 < len(parts) else parts[i]
                 for i in range(0, len(parts), 2)]
    return finish(parts[0])
