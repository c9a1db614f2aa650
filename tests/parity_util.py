"""Shared helpers of the GPU parity tests: run the HIP path, run the oracle on the same
bytes, compare at the tolerances the tests state."""
from __future__ import annotations

import math
import sys

import numpy as np
import torch

import oracle

# bfloat16 inputs: absolute bounds on O (max and mean over the compared elements) and on LSE
BF16_O_MAX, BF16_O_MEAN, BF16_LSE_MAX = 1e-2, 2e-3, 1e-3
# float32 inputs: bounds relative to the largest reference magnitude
F32_REL = 1e-5
# Derived bounds (tests/tolerance_model.py reproduces the model figures they rest on):
# backward, bfloat16 inputs: max and mean error of each gradient relative to its own max and
# mean magnitude
BWD_BF16_MAX_REL, BWD_BF16_MEAN_REL = 1e-2, 5e-3
# backward, float32 inputs, the same form
BWD_F32_MAX_REL, BWD_F32_MEAN_REL = 2e-5, 1e-5
# forward on E4M3 inputs with values drawn N(0,1) (times a factor for Q and K): absolute max
# and mean error of O, absolute LSE error
FP8_O_MAX, FP8_O_MEAN, FP8_LSE_MAX = 0.12, 6e-3, 1e-3


def say(msg: str):
    """Name the case before each GPU step, flushed, so a failing run shows what ran."""
    print(msg, flush=True)
    sys.stdout.flush()


def compare(o, lse, o_ref, lse_ref, dtype, what=""):
    """o, lse: GPU results (numpy float32/float64) on the compared rows; *_ref: oracle rows.
    Returns a dict of error statistics; raises AssertionError outside the tolerance."""
    o = np.asarray(o, np.float64).reshape(o_ref.shape)
    lse = np.asarray(lse, np.float64).reshape(lse_ref.shape)
    assert np.all(np.isfinite(o)), f"{what}: non-finite O"
    empty = np.isneginf(lse_ref)
    assert np.array_equal(np.isneginf(lse), empty), f"{what}: -inf LSE rows differ"
    assert not np.any(np.isnan(lse)), f"{what}: NaN LSE"
    assert np.all(o[empty] == 0.0), f"{what}: empty rows must be zero"
    err = np.abs(o - o_ref)
    lerr = np.abs(lse[~empty] - lse_ref[~empty]) if np.any(~empty) else np.zeros(1)
    stats = dict(o_max=float(err.max(initial=0.0)), o_mean=float(err.mean()) if err.size else 0.0,
                 lse_max=float(lerr.max(initial=0.0)))
    if dtype == torch.float32:
        o_tol = F32_REL * max(1e-30, float(np.abs(o_ref).max(initial=0.0)))
        l_tol = F32_REL * max(1e-30, float(np.abs(lse_ref[~empty]).max(initial=0.0)))
        assert stats["o_max"] <= o_tol, f"{what}: O max err {stats['o_max']:.3e} > {o_tol:.3e}"
        assert stats["lse_max"] <= l_tol, f"{what}: LSE max err {stats['lse_max']:.3e} > {l_tol:.3e}"
    else:
        assert stats["o_max"] <= BF16_O_MAX, f"{what}: O max err {stats['o_max']:.3e}"
        assert stats["o_mean"] <= BF16_O_MEAN, f"{what}: O mean err {stats['o_mean']:.3e}"
        assert stats["lse_max"] <= BF16_LSE_MAX, f"{what}: LSE max err {stats['lse_max']:.3e}"
    return stats


def rows_of(t: torch.Tensor, rows, d=None):
    """Select flat rows (b*H + h)*N + i of a [B, H, N(, d)] GPU tensor, to host float64."""
    idx = torch.as_tensor(np.asarray(rows, np.int64), device=t.device)
    flat = t.reshape(-1, d) if d is not None else t.reshape(-1)
    return flat.index_select(0, idx).double().cpu().numpy()


def seeded(shape, seed, dtype, device="cuda", mult=1.0):
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return (torch.randn(shape, generator=g, device=device, dtype=torch.float32) * mult).to(dtype)


def finite_scale(d):
    return float(torch.tensor(1.0 / math.sqrt(d), dtype=torch.float32).item())


def oracle_rows(q, k, v, scale, causal, rows=None):
    return oracle.attention(q.cpu(), k.cpu(), v.cpu(), scale, causal, rows=rows)
