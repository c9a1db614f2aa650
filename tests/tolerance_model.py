"""Float32 models of the kernels' arithmetic, used to derive the tolerances of the parity
tests where the stated bounds do not apply (gradients, 8-bit inputs) and to check that the
stated bounds are met with margin by the forward's own rounding. Test infrastructure only.

Each model performs the same roundings as the HIP kernels, in the same places, with every
other operation in float32 (torch on the CPU; a matrix product stands for a float32 MFMA
accumulation, whose summation order differs but whose error has the same size):

- forward, bfloat16 inputs: scores in float32 from exact products; the online softmax of
  "FlashAttention: Attention Is Limited by Memory, Not Math", section "How tiling and online
  softmax stay exact", over key tiles, with the exact running max as the offset of every
  exponent; the probabilities rounded to bfloat16 (nearest even) for the PV product; the
  normaliser summed over the float32 probabilities; O divided once at the end;
- backward, bfloat16 inputs: the chain-rule gradients ("Explain FlashAttention ...",
  section "Exact attention, finite precision and backward") with P recomputed from the
  float32 LSE of the forward model, P and dS rounded to bfloat16 as operands of the dV, dK
  and dQ products, the row terms dO.O from the forward model's float32 O;
- backward, float32 inputs: the same without any rounding below float32;
- forward, E4M3 inputs: scores in float32 from the exactly dequantised values, weights
  entering the PV product as E4M3(256 * 2^(s - m)) with m the row max, the normaliser
  summed over the float32 weights.

The reference is the float64 oracle on the same inputs.
"""
from __future__ import annotations

import math

import numpy as np
import torch

import oracle

LOG2E = 1.4426950408889634
LN2 = 0.6931471805599453


def _f32(x: float) -> float:
    return float(np.float32(x))


def _bf16(x: torch.Tensor) -> torch.Tensor:
    return x.to(torch.bfloat16).float()


def _mask(nq: int, nk: int, causal: int) -> torch.Tensor | None:
    """True where key j is hidden from query i (absolute positions; 1 bottom-right, 2 top-left)."""
    if not causal:
        return None
    off = nk - nq if int(causal) == 1 else 0
    i = torch.arange(nq)[:, None]
    j = torch.arange(nk)[None, :]
    return j > i + off


def fwd_bf16(q, k, v, scale: float, causal: int = 0, tile: int = 96, round_p: bool = True):
    """Online-softmax forward over key tiles of `tile` keys; float32 throughout except P,
    rounded to bfloat16 for the PV product when round_p. Returns (O, LSE) float32, LSE in
    natural-log units; rows that see no key get O = 0 and LSE = -inf."""
    qf, kf, vf = q.float(), k.float(), v.float()
    *lead, nq, d = qf.shape
    nk = kf.shape[-2]
    c = _f32(_f32(scale) * _f32(LOG2E))
    hidden = _mask(nq, nk, causal)
    m = torch.full((*lead, nq, 1), -math.inf)
    l = torch.zeros((*lead, nq, 1))
    acc = torch.zeros((*lead, nq, d))
    for t0 in range(0, nk, tile):
        s = qf @ kf[..., t0:t0 + tile, :].transpose(-1, -2)
        if hidden is not None:
            s = s.masked_fill(hidden[:, t0:t0 + tile], -math.inf)
        mt = s.amax(-1, keepdim=True) * c
        m_new = torch.maximum(m, mt)
        alpha = torch.where(m_new > m, torch.exp2(m - m_new), torch.ones_like(m))
        off = torch.where(torch.isinf(m_new), torch.zeros_like(m_new), m_new)
        p = torch.exp2(s * c - off)
        l = l * alpha + p.sum(-1, keepdim=True)
        pv = _bf16(p) if round_p else p
        acc = acc * alpha + pv @ vf[..., t0:t0 + tile, :]
        m = m_new
    o = torch.where(l > 0, acc / torch.where(l > 0, l, torch.ones_like(l)), torch.zeros_like(acc))
    lse = torch.where(l[..., 0] > 0, (m[..., 0] + torch.log2(l[..., 0])) * _f32(LN2),
                      torch.full_like(l[..., 0], -math.inf))
    return o, lse


def bwd(q, k, v, o, lse, do, scale: float, causal: int = 0, round_ops: bool = True):
    """Gradients (dQ, dK, dV) from the forward's O and LSE, float32, with P and dS rounded to
    bfloat16 as product operands when round_ops."""
    qf, kf, vf, dof = q.float(), k.float(), v.float(), do.float()
    nq, nk = qf.shape[-2], kf.shape[-2]
    c = _f32(_f32(scale) * _f32(LOG2E))
    lse2 = lse * _f32(LOG2E)
    lse2 = torch.where(torch.isinf(lse2), torch.full_like(lse2, math.inf), lse2)  # P = 0 rows
    s = qf @ kf.transpose(-1, -2)
    p = torch.exp2(s * c - lse2[..., None])
    hidden = _mask(nq, nk, causal)
    if hidden is not None:
        p = p.masked_fill(hidden, 0.0)
    dp = dof @ vf.transpose(-1, -2)
    dsum = (dof * o).sum(-1, keepdim=True)
    ds = p * (dp - dsum)
    rnd = _bf16 if round_ops else (lambda x: x)
    dv = rnd(p).transpose(-1, -2) @ dof
    dk = _f32(scale) * (rnd(ds).transpose(-1, -2) @ qf)
    dq = _f32(scale) * (rnd(ds) @ kf)
    return dq, dk, dv


def fwd_e4m3(q8, k8, v8, qd: float, kd: float, vd: float, scale: float, causal: int = 0):
    """Forward on E4M3 inputs with per-tensor descales. Returns O float32."""
    qf, kf, vf = q8.float(), k8.float(), v8.float()
    nq, nk = qf.shape[-2], kf.shape[-2]
    c = _f32(_f32(scale) * _f32(qd) * _f32(kd) * _f32(LOG2E))
    s = (qf @ kf.transpose(-1, -2)) * c
    hidden = _mask(nq, nk, causal)
    if hidden is not None:
        s = s.masked_fill(hidden, -math.inf)
    m = s.amax(-1, keepdim=True)
    m = torch.where(torch.isinf(m), torch.zeros_like(m), m)
    e = torch.exp2(s - (m - 8.0))                 # the row's largest weight is 256
    pt = e.to(torch.float8_e4m3fn).float()
    l = e.sum(-1, keepdim=True)
    o = (pt @ vf) * _f32(vd) / torch.where(l > 0, l, torch.ones_like(l))
    return torch.where(l > 0, o, torch.zeros_like(o))


def draw(shape, gen, mult=1.0, dtype=torch.bfloat16):
    return (torch.randn(shape, generator=gen) * mult).to(dtype)


def bwd_case(B, H, nq, nk, d, causal, mult, seed, dtype=torch.bfloat16):
    """Model and oracle gradients on one seeded case: {name: (max err / max|g*|,
    mean err / mean|g*|)} for the gradients that are not identically zero."""
    g = torch.Generator().manual_seed(seed)
    q = draw((B, H, nq, d), g, mult, dtype)
    k = draw((B, H, nk, d), g, mult, dtype)
    v = draw((B, H, nk, d), g, 1.0, dtype)
    do = draw((B, H, nq, d), g, 1.0, dtype)
    scale = _f32(1.0 / math.sqrt(d))
    low = dtype == torch.bfloat16
    o, lse = fwd_bf16(q, k, v, scale, causal, round_p=low)
    got = bwd(q, k, v, o, lse, do, scale, causal, round_ops=low)
    ref = oracle.attention_bwd(q, k, v, do, scale, causal)
    out = {}
    for name, gm, r in zip(("dq", "dk", "dv"), got, ref):
        gm = gm.double().numpy().reshape(r.shape)
        e = np.abs(gm - r)
        out[name] = (float(e.max() / np.abs(r).max()), float(e.mean() / np.abs(r).mean()))
    return out


def fwd_case(B, H, n, d, causal, mult, seed, tile=96):
    """Forward model against the oracle: (max|O - O*|, mean|O - O*|, max|LSE - LSE*|) with O
    kept in float32, and max|O - O*| with O rounded to bfloat16 on output."""
    g = torch.Generator().manual_seed(seed)
    q = draw((B, H, n, d), g, mult)
    k = draw((B, H, n, d), g, mult)
    v = draw((B, H, n, d), g, 1.0)
    scale = _f32(1.0 / math.sqrt(d))
    o, lse = fwd_bf16(q, k, v, scale, causal, tile=tile)
    o_ref, l_ref = oracle.attention(q, k, v, scale, causal)
    e = np.abs(o.double().numpy().reshape(o_ref.shape) - o_ref)
    ob = o.to(torch.bfloat16).double().numpy().reshape(o_ref.shape)
    le = np.abs(lse.double().numpy().reshape(-1) - l_ref)
    return float(e.max()), float(e.mean()), float(le.max()), float(np.abs(ob - o_ref).max())


def e4m3_case(B, H, n, d, causal, mult, seed):
    """E4M3 model against the oracle on the dequantised inputs: (max, mean) of |O - O*|."""
    g = torch.Generator().manual_seed(seed)
    xs = [torch.randn((B, H, n, d), generator=g) * m for m in (mult, mult, 1.0)]
    quant = []
    for x in xs:
        amax = float(x.abs().max())
        ds = _f32(amax / 448.0)
        quant.append(((x / ds).to(torch.float8_e4m3fn), ds))
    (q8, qd), (k8, kd), (v8, vd) = quant
    scale = _f32(1.0 / math.sqrt(d))
    o = fwd_e4m3(q8, k8, v8, qd, kd, vd, scale, causal)
    o_ref, _ = oracle.attention(q8.double() * qd, k8.double() * kd, v8.double() * vd, scale, causal)
    e = np.abs(o.double().numpy().reshape(o_ref.shape) - o_ref)
    return float(e.max()), float(e.mean())
