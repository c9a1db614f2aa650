"""Seeded synthetic attention workloads: shapes, seeds and value distributions.

This module only draws random numbers and names shapes. It holds none of the
attention arithmetic, so both the float64 oracle and the HIP path may take
their inputs from it.

Recipe (the same for every workload): per tensor, a ``torch.Generator`` on the
target device is seeded with ``10*c + t`` (c = workload number 1..5, t = 0 for
Q, 1 for K, 2 for V); then, for b = 0..B-1 in order, one ``torch.randn`` call
draws the [H, N, d] float32 slice, which is multiplied by the workload's scale
factor and rounded to the storage dtype (bfloat16 rounding is
round-to-nearest-even). The backward pass takes a fourth tensor, dO, drawn the same way
with t = 3 and factor 1. The oracle always consumes the rounded bytes, so input
quantisation is never counted as kernel error. Different devices give
different (equally valid) draws for one seed; a test always reads back the
bytes the kernel received.
"""
from __future__ import annotations

import dataclasses
import math

import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    number: int
    name: str
    B: int
    H: int
    Nq: int
    Nk: int
    d: int
    dtype: torch.dtype
    causal: bool
    qk_mult: float = 1.0   # Q and K are drawn N(0,1) and multiplied by this
    num_splits: int = 0    # > 0: the split-KV decode path with this many chunks

    @property
    def scale(self) -> float:
        """Softmax scale 1/sqrt(d), rounded to float32 as the kernel receives it."""
        return float(torch.tensor(1.0 / math.sqrt(self.d), dtype=torch.float32).item())

    @property
    def flops(self) -> float:
        """Algorithmic FLOPs of the two contractions: 4*B*H*Nq*Nk*d, halved if causal."""
        f = 4.0 * self.B * self.H * self.Nq * self.Nk * self.d
        return f / 2 if self.causal else f

    @property
    def bwd_flops(self) -> float:
        """Algorithmic FLOPs of the backward pass: the five contractions S = QK^T, dV = P^T dO,
        dP = dO V^T, dQ = dS K and dK = dS^T Q, 2*Nq*Nk*d each per head, halved if causal."""
        f = 10.0 * self.B * self.H * self.Nq * self.Nk * self.d
        return f / 2 if self.causal else f

    @property
    def elem_bytes(self) -> int:
        return torch.tensor([], dtype=self.dtype).element_size()

    @property
    def io_bytes(self) -> int:
        """Compulsory HBM bytes: read Q, K, V once; write O (fp32) and LSE (fp32) once."""
        e = self.elem_bytes
        q = self.B * self.H * self.Nq * self.d * e
        kv = 2 * self.B * self.H * self.Nk * self.d * e
        o = self.B * self.H * self.Nq * self.d * 4
        lse = self.B * self.H * self.Nq * 4
        return q + kv + o + lse


WORKLOADS = {
    1: Workload(1, "f32 single head N=256 d=64", 1, 1, 256, 256, 64, torch.float32, False),
    2: Workload(2, "bf16 B=4 H=16 N=2048 d=64", 4, 16, 2048, 2048, 64, torch.bfloat16, False),
    3: Workload(3, "bf16 causal B=2 H=16 N=8192 d=128, Q,K x3", 2, 16, 8192, 8192, 128,
                torch.bfloat16, True, qk_mult=3.0),
    4: Workload(4, "bf16 causal B=1 H=32 N=30000 d=128", 1, 32, 30000, 30000, 128,
                torch.bfloat16, True),
    5: Workload(5, "bf16 decode B=16 H=32 Nk=32768 d=128, 64 splits", 16, 32, 1, 32768, 128,
                torch.bfloat16, False, num_splits=64),
}


def draw(shape, seed: int, mult: float = 1.0, dtype=torch.bfloat16, device="cpu") -> torch.Tensor:
    """Draw a [B, ...] tensor slice by slice along dim 0 (see the module recipe)."""
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    out = torch.empty(shape, dtype=dtype, device=device)
    for b in range(shape[0]):
        x = torch.randn(tuple(shape[1:]), generator=g, dtype=torch.float32, device=device)
        if mult != 1.0:
            x.mul_(mult)
        out[b].copy_(x)  # float32 -> storage dtype, round-to-nearest-even
        del x
    return out


def make_inputs(w: Workload, device="cpu"):
    """(q, k, v) for workload ``w`` on ``device``, following the module recipe."""
    c = w.number
    q = draw((w.B, w.H, w.Nq, w.d), 10 * c + 0, w.qk_mult, w.dtype, device)
    k = draw((w.B, w.H, w.Nk, w.d), 10 * c + 1, w.qk_mult, w.dtype, device)
    v = draw((w.B, w.H, w.Nk, w.d), 10 * c + 2, 1.0, w.dtype, device)
    return q, k, v


def quantize_e4m3(x: torch.Tensor):
    """Per-tensor E4M3 quantisation: descale = max|x| / 448 (the largest finite E4M3 value),
    x8 = E4M3(x / descale) rounded to nearest even. Returns (x8, descale); the value the
    kernel and the oracle both use is x8 * descale. Data preparation only."""
    amax = float(x.abs().max())
    descale = amax / 448.0 if amax > 0 else 1.0
    descale = float(torch.tensor(descale, dtype=torch.float32))  # the kernel takes float32
    x8 = (x.float() / descale).to(torch.float8_e4m3fn)
    return x8, descale


def make_inputs_fp8(w: Workload, device="cpu"):
    """E4M3 versions of workload w's Q, K, V: the recipe's float32 draws (same seeds and
    factors) quantised per tensor with quantize_e4m3. Returns ((q8, qd), (k8, kd), (v8, vd))."""
    c = w.number
    out = []
    for t, (n, mult) in enumerate(((w.Nq, w.qk_mult), (w.Nk, w.qk_mult), (w.Nk, 1.0))):
        x = draw((w.B, w.H, n, w.d), 10 * c + t, mult, torch.float32, device)
        out.append(quantize_e4m3(x))
        del x
    return tuple(out)


def make_bias(w: Workload, device="cpu", mult: float = 2.0):
    """The additive bias of the biased prefill on workload w: a full [B, H, Nq, Nk] tensor of
    w's dtype, N(0,1) * mult drawn as in `draw` with seed 10c + 4 (one value per (b, h, query,
    key): the general case, nothing shared or broadcast)."""
    return draw((w.B, w.H, w.Nq, w.Nk), 10 * w.number + 4, mult, w.dtype, device)


def make_grad(w: Workload, device="cpu"):
    """dO, the gradient fed to the backward pass: N(0,1) of q's shape and dtype, seed 10c + 3."""
    return draw((w.B, w.H, w.Nq, w.d), 10 * w.number + 3, 1.0, w.dtype, device)


VARLEN_SEQS, VARLEN_H, VARLEN_D = 16, 16, 128


def varlen_lengths(seed: int = 60, n: int = VARLEN_SEQS, lo: int = 256, hi: int = 8192):
    """Sequence lengths of the packed variable-length prefill: n lengths drawn uniformly
    from [lo, hi] with a seeded CPU generator (a mix of short and long sequences)."""
    g = torch.Generator().manual_seed(int(seed))
    return [int(x) for x in torch.randint(lo, hi + 1, (n,), generator=g)]


def make_varlen(device="cpu", seed: int = 60):
    """(q, k, v, cu_seqlens, lengths) of the packed variable-length prefill: bfloat16
    N(0,1) [total, H, d] tensors, seeds seed+1, seed+2, seed+3, drawn as in `draw` with
    the packed tensor as one slice; cu_seqlens int32 [n+1] (queries and keys alike)."""
    lens = varlen_lengths(seed)
    total = sum(lens)
    shape = (1, total, VARLEN_H, VARLEN_D)
    q, k, v = (draw(shape, seed + 1 + t, 1.0, torch.bfloat16, device)[0] for t in range(3))
    cu = torch.tensor([0] + list(torch.tensor(lens).cumsum(0)), dtype=torch.int32, device=device)
    return q, k, v, cu, lens


def make_varlen_grad(device="cpu", seed: int = 60):
    """dO of the packed variable-length batch: bfloat16 N(0,1) [total, H, d], seed seed+4."""
    total = sum(varlen_lengths(seed))
    return draw((1, total, VARLEN_H, VARLEN_D), seed + 4, 1.0, torch.bfloat16, device)[0]


def varlen_flops(lens, H: int = VARLEN_H, d: int = VARLEN_D, causal: bool = True) -> float:
    """Algorithmic FLOPs of the packed prefill: 4*H*n*n*d per sequence, halved if causal."""
    f = sum(4.0 * H * n * n * d for n in lens)
    return f / 2 if causal else f


def to_paged(k: torch.Tensor, page_size: int, seed: int):
    """Lay a contiguous [B, H, N, d] cache out as pages: returns (cache [B*P, page_size, H, d],
    block_table int32 [B, P]) with P = ceil(N / page_size) and the B*P pages placed in the
    pool in a seeded random order (positions past N in the last page are zero). Data
    movement only: the logical rows of sequence b are those of k[b]."""
    B, H, N, d = k.shape
    P = -(-N // page_size)
    g = torch.Generator().manual_seed(int(seed))
    order = torch.randperm(B * P, generator=g)
    cache = torch.zeros((B * P, page_size, H, d), dtype=k.dtype, device=k.device)
    for b in range(B):
        for j in range(P):
            n = min(page_size, N - j * page_size)
            cache[order[b * P + j], :n] = k[b, :, j * page_size:j * page_size + n].transpose(0, 1)
    table = order.view(B, P).to(torch.int32).to(k.device)
    return cache, table


def sample_rows(w: Workload, per_head: int = 64, seed: int = 12345):
    """Flat row ids (b*H + h)*Nq + i for a sampled parity check on a large workload.

    Per (b, h): fixed rows that straddle every power-of-two tile edge from 16
    to 256 and the ragged tail, plus seeded random rows, ``per_head`` in total.
    """
    N = w.Nq
    fixed = [0, 1, 15, 16, 17, 31, 32, 33, 63, 64, 65, 127, 128, 129, 255, 256, 257,
             N // 2, N - 129, N - 65, N - 49, N - 48, N - 47, N - 17, N - 2, N - 1]
    fixed = sorted({i for i in fixed if 0 <= i < N})
    g = torch.Generator().manual_seed(seed)
    rows = []
    for bh in range(w.B * w.H):
        chosen = list(fixed)
        extra = max(0, min(per_head, N) - len(chosen))
        if extra:
            pool = torch.randperm(N, generator=g).tolist()
            have = set(chosen)
            for i in pool:
                if len(chosen) >= len(fixed) + extra:
                    break
                if i not in have:
                    chosen.append(i)
                    have.add(i)
        rows.extend(bh * N + i for i in sorted(chosen))
    return rows
