"""Pins of the variable-length backward oracle (CPU only).

oracle.attention_varlen_bwd returns the gradients of sum(O * dO) for the packed-batch
attention of oracle.attention_varlen. Pinned against things other than its own code:
- central finite differences, in float64, of the variable-length forward oracle's loss, on
  ragged batches with query and key counts that differ inside a sequence, an empty
  sequence and a sequence with no keys, under all three mask settings;
- torch.autograd in float64 through one explicit softmax over the whole packed batch with a
  block-diagonal (same-sequence) mask;
- equal lengths packed by explicit loops reproduce oracle.attention_bwd on the dense tensors;
- no cross-talk: changing one sequence's inputs leaves every other sequence's gradients
  bit-identical;
- three plausible slips planted in a copy of the function each fail a pin.
"""
import inspect
import math

import numpy as np
import pytest
import torch

import oracle

NQS, NKS = [3, 0, 5, 2, 4, 1], [3, 2, 7, 0, 6, 4]


def _ragged(seed, nqs=NQS, nks=NKS, H=2, d=4):
    g = torch.Generator().manual_seed(seed)
    cq = np.concatenate([[0], np.cumsum(nqs)]).astype(int)
    ck = np.concatenate([[0], np.cumsum(nks)]).astype(int)
    mk = lambda n: torch.randn((n, H, d), generator=g, dtype=torch.float64)
    return mk(cq[-1]), mk(ck[-1]), mk(ck[-1]), mk(cq[-1]), cq, ck


def _loss(q, k, v, do, cq, ck, scale, causal):
    o, _ = oracle.attention_varlen(q, k, v, cq, ck, scale, causal)
    return float((o * do.numpy()).sum())


@pytest.mark.parametrize("causal", [0, 1, 2])
def test_finite_differences(causal, fn=None):
    fn = fn or oracle.attention_varlen_bwd
    q, k, v, do, cq, ck = _ragged(3)
    scale = 0.6
    grads = dict(zip("qkv", fn(q, k, v, do, cq, ck, scale, causal)))
    h = 1e-6
    rng = np.random.default_rng(5)
    for name, t in (("q", q), ("k", k), ("v", v)):
        flat = t.view(-1)
        for e in rng.choice(flat.numel(), size=14, replace=False):
            orig = float(flat[e])
            flat[e] = orig + h
            lp = _loss(q, k, v, do, cq, ck, scale, causal)
            flat[e] = orig - h
            lm = _loss(q, k, v, do, cq, ck, scale, causal)
            flat[e] = orig
            fd = (lp - lm) / (2 * h)
            assert abs(fd - grads[name].reshape(-1)[e]) <= 1e-7 * max(1.0, abs(fd)), (name, e)


def _autograd(q, k, v, do, cq, ck, scale, causal):
    """One softmax over all packed keys with a mask that keeps each query to its own
    sequence's keys (and the in-sequence causal rule); rows with no key give 0."""
    q, k, v = (t.clone().requires_grad_(True) for t in (q, k, v))
    tq, tk = q.shape[0], k.shape[0]
    seq_q = np.searchsorted(cq, np.arange(tq), side="right") - 1
    seq_k = np.searchsorted(ck, np.arange(tk), side="right") - 1
    i = np.arange(tq) - cq[seq_q]
    j = np.arange(tk) - ck[seq_k]
    nq = (cq[seq_q + 1] - cq[seq_q])[:, None]
    nk = (ck[seq_q + 1] - ck[seq_q])[:, None]
    vis = seq_q[:, None] == seq_k[None, :]
    if causal == 1:
        vis &= j[None, :] <= i[:, None] + nk - nq
    elif causal == 2:
        vis &= j[None, :] <= i[:, None]
    s = scale * torch.einsum("qhd,khd->hqk", q, k)
    s = s.masked_fill(torch.from_numpy(~vis)[None], float("-inf"))
    p = torch.softmax(s, dim=-1).nan_to_num(0.0)
    o = torch.einsum("hqk,khd->qhd", p, v)
    (o * do).sum().backward()
    return q.grad, k.grad, v.grad


@pytest.mark.parametrize("causal", [0, 1, 2])
def test_matches_autograd_over_the_whole_batch(causal, fn=None):
    fn = fn or oracle.attention_varlen_bwd
    q, k, v, do, cq, ck = _ragged(7, H=3, d=8)
    got = fn(q, k, v, do, cq, ck, 0.4, causal)
    ref = _autograd(q, k, v, do, cq, ck, 0.4, causal)
    for g, r in zip(got, ref):
        assert np.abs(g - r.numpy()).max() <= 1e-12 * max(1.0, float(r.abs().max()))


def _pack(x):
    """[B, H, N, d] -> [B*N, H, d] by loops."""
    B, H, N, d = x.shape
    out = torch.empty((B * N, H, d), dtype=x.dtype)
    for b in range(B):
        for n in range(N):
            for h in range(H):
                out[b * N + n, h] = x[b, h, n]
    return out


@pytest.mark.parametrize("causal", [0, 1])
def test_equal_lengths_match_dense(causal, fn=None):
    fn = fn or oracle.attention_varlen_bwd
    g = torch.Generator().manual_seed(9)
    B, H, N, d = 3, 2, 11, 8
    q, k, v, do = (torch.randn((B, H, N, d), generator=g) for _ in range(4))
    cu = [0, N, 2 * N, 3 * N]
    got = fn(_pack(q), _pack(k), _pack(v), _pack(do), cu, cu, 0.3, causal)
    ref = oracle.attention_bwd(q, k, v, do, 0.3, causal)
    for gt, rt in zip(got, ref):
        rt = rt.reshape(B, H, N, d)
        for b in range(B):
            for n in range(N):
                for h in range(H):
                    assert np.array_equal(gt[b * N + n, h], rt[b, h, n])


def test_no_cross_talk_and_empty_sequences(fn=None):
    fn = fn or oracle.attention_varlen_bwd
    q, k, v, do, cq, ck = _ragged(13)
    a = fn(q, k, v, do, cq, ck, 0.5, 1)
    q2, k2, v2, do2 = (t.clone() for t in (q, k, v, do))
    q2[cq[2]:cq[3]] += 1.0
    k2[ck[2]:ck[3]] *= -1.0
    v2[ck[2]:ck[3]] += 2.0
    do2[cq[2]:cq[3]] *= 3.0
    b = fn(q2, k2, v2, do2, cq, ck, 0.5, 1)
    for x, y in zip(a, b):
        keep = np.ones(x.shape[0], bool)
        lo, hi = (cq[2], cq[3]) if x.shape[0] == q.shape[0] else (ck[2], ck[3])
        keep[lo:hi] = False
        assert np.array_equal(x[keep], y[keep])
    # sequence 1 has no query rows (its keys get no gradient); sequence 3 has no keys
    assert np.all(a[1][ck[1]:ck[2]] == 0) and np.all(a[2][ck[1]:ck[2]] == 0)
    assert np.all(a[0][cq[3]:cq[4]] == 0)


MUTANTS = {
    "key gradients written at the query offsets": ("dk[ck[b]:ck[b + 1]]", "dk[cq[b]:cq[b] + nk]"),
    "head and row axes swapped on the way back": (
        "dq[cq[b]:cq[b + 1]] = gq.reshape(H, nq, d).transpose(1, 0, 2)",
        "dq[cq[b]:cq[b + 1]] = gq.reshape(nq, H, d)"),
    "mask dropped": ("scale, causal, threads=threads)", "scale, 0, threads=threads)"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name):
    src = inspect.getsource(oracle.attention_varlen_bwd)
    old, new = MUTANTS[name]
    assert src.count(old) == 1, name
    ns = dict(vars(oracle))
    exec(compile(src.replace(old, new), "<mutant>", "exec"), ns)
    bad = ns["attention_varlen_bwd"]
    pins = [lambda: test_finite_differences(1, fn=bad), lambda: test_finite_differences(2, fn=bad),
            lambda: test_matches_autograd_over_the_whole_batch(2, fn=bad),
            lambda: test_no_cross_talk_and_empty_sequences(fn=bad)]
    failed = 0
    for pin in pins:
        try:
            pin()
        except (AssertionError, ValueError, RuntimeError, IndexError):
            failed += 1
    assert failed > 0, f"no pin caught the mutant: {name}"
