"""Float64 model of the tiled online-softmax recurrence (test helper, not the oracle).

The oracle evaluates the plain definition. This module evaluates the same
result the way the kernels do: keys arrive in tiles, and each query row keeps
a running state (m, l, o) that is rescaled whenever the running max rises.
Agreement between the two (to float64 rounding) pins the oracle against an
independent formulation, and the per-block states are compared with the
intermediates the pages print.

- One-sided update of the running state by a new tile (running max m, running
  sum of exponentials l, unnormalised weighted sum o, rescale factor
  alpha = exp(m_old - m_new), divide by l after the last tile):
  "FlashAttention: Attention Is Limited by Memory, Not Math", section "How
  tiling and online softmax stay exact"; "Explain FlashAttention ...",
  section "Keep only the state needed for the final weighted average".
- Tiles whose scores are all masked are skipped, so the first real update
  never evaluates -inf - (-inf); a row that saw no key returns zeros:
  "Explain FlashAttention ...", section "Executable recurrence, with an
  empty-state policy".
- Two-sided merge of partial states computed against their own local maxima
  (scale_old = exp(m_old - m_new), scale_new = exp(m_block - m_new)), which
  returns a state of the same shape and therefore chains:
  "Flash Attention Optimization", section "The fix: tile the computation,
  never materialize the full matrix"; "Handwritten Notes on Flash
  Attention", section "Merging two blocks".
"""
from __future__ import annotations

import math

import numpy as np

NEG_INF = -math.inf


class State:
    """Running (m, l, o) of one query row; o has the value dimension."""

    def __init__(self, dv: int):
        self.m = NEG_INF
        self.l = 0.0
        self.o = np.zeros(dv, np.float64)

    def copy(self):
        s = State(self.o.size)
        s.m, s.l, s.o = self.m, self.l, self.o.copy()
        return s


def update(state: State, s_tile: np.ndarray, v_tile: np.ndarray) -> State:
    """Fold one tile of scores (-inf = masked) and its value rows into the state."""
    tile_max = float(np.max(s_tile)) if s_tile.size else NEG_INF
    if tile_max == NEG_INF:          # nothing visible in this tile: skip it
        return state
    m_new = max(state.m, tile_max)
    alpha = 0.0 if state.m == NEG_INF else math.exp(state.m - m_new)
    w = np.exp(s_tile - m_new)       # masked entries give exactly 0
    state.l = alpha * state.l + float(w.sum())
    state.o = alpha * state.o + w @ v_tile
    state.m = m_new
    return state


def local_state(s_tile: np.ndarray, v_tile: np.ndarray, dv: int) -> State:
    """A block's own state, relative to the block's own max (as in a split chunk)."""
    return update(State(dv), s_tile, v_tile)


def merge(a: State, b: State) -> State:
    """Two-sided merge of two partial states; an empty state (m=-inf) is skipped."""
    if b.m == NEG_INF:
        return a.copy()
    if a.m == NEG_INF:
        return b.copy()
    out = State(a.o.size)
    out.m = max(a.m, b.m)
    scale_old = math.exp(a.m - out.m)
    scale_new = math.exp(b.m - out.m)
    out.l = a.l * scale_old + b.l * scale_new
    out.o = a.o * scale_old + b.o * scale_new
    return out


def finish(state: State):
    """(output row, log-sum-exp) of a finished state; empty row -> (0, -inf)."""
    if state.l == 0.0:
        return np.zeros_like(state.o), NEG_INF
    return state.o / state.l, state.m + math.log(state.l)


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


def tiled_head(q, k, v, scale, causal, tile):
    """Attention for one head by the one-sided recurrence over key tiles of size ``tile``."""
    s = scores(q, k, scale, causal)
    nq, nk = s.shape
    o = np.zeros((nq, v.shape[1]))
    lse = np.zeros(nq)
    for i in range(nq):
        st = State(v.shape[1])
        for j0 in range(0, nk, tile):
            update(st, s[i, j0:j0 + tile], v[j0:j0 + tile])
        o[i], lse[i] = finish(st)
    return o, lse


def split_merge_head(q, k, v, scale, causal, num_splits):
    """Attention for one head by splitting keys into chunks of ceil(Nk/S) and merging."""
    s = scores(q, k, scale, causal)
    nq, nk = s.shape
    chunk = -(-nk // num_splits)
    o = np.zeros((nq, v.shape[1]))
    lse = np.zeros(nq)
    for i in range(nq):
        parts = []
        for c in range(num_splits):
            lo, hi = c * chunk, min(nk, (c + 1) * chunk)
            parts.append(local_state(s[i, lo:hi], v[lo:hi], v.shape[1]))
        acc = State(v.shape[1])
        for p in parts:
            acc = merge(acc, p)
        o[i], lse[i] = finish(acc)
    return o, lse
