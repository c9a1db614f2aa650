"""Pins of the variable-length oracle (CPU only).

oracle.attention_varlen applies the attention definition to each sequence of a packed
batch ([total, H, d] with cumulative sequence offsets). Pinned against:
- a packed batch of equal lengths built here by explicit loops from dense [B, H, N, d]
  tensors: must equal oracle.attention on the dense tensors;
- brute force in pure Python (math.fsum, no max subtraction) on tiny ragged batches, both
  mask settings, query and key counts that differ inside a sequence;
- no cross-talk: changing one sequence's keys and values leaves every other sequence's
  outputs bit-identical;
- sequences with no query rows, and query rows with no key (O = 0, LSE = -inf).
"""
import math

import numpy as np
import pytest
import torch

import oracle


def _pack(x):
    """[B, H, N, d] -> [B*N, H, d] by loops."""
    B, H, N, d = x.shape
    out = torch.empty((B * N, H, d), dtype=x.dtype)
    for b in range(B):
        for n in range(N):
            for h in range(H):
                out[b * N + n, h] = x[b, h, n]
    return out


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_equal_lengths_match_dense(causal, dtype):
    g = torch.Generator().manual_seed(7)
    B, H, N, d = 3, 2, 19, 8
    q, k, v = ((torch.randn((B, H, N, d), generator=g) * 2).to(dtype) for _ in range(3))
    cu = [0, N, 2 * N, 3 * N]
    o, l = oracle.attention_varlen(_pack(q), _pack(k), _pack(v), cu, cu, 0.3, causal)
    wo, wl = oracle.attention(q, k, v, 0.3, causal)
    wo = wo.reshape(B, H, N, d)
    wl = wl.reshape(B, H, N)
    for b in range(B):
        for n in range(N):
            for h in range(H):
                assert np.max(np.abs(o[b * N + n, h] - wo[b, h, n])) <= 1e-14
                assert abs(l[h, b * N + n] - wl[b, h, n]) <= 1e-14


def _brute(qi, kk, vv, scale, last):
    w = [math.exp(scale * math.fsum(float(a) * float(b) for a, b in zip(qi, kk[j]))) for j in range(last + 1)]
    if not w:
        return [0.0] * len(qi), -math.inf
    tot = math.fsum(w)
    return [math.fsum(w[j] * float(vv[j][t]) for j in range(len(w))) / tot for t in range(len(qi))], math.log(tot)


@pytest.mark.parametrize("causal", [False, True])
def test_ragged_batch_brute_force(causal):
    rng = np.random.default_rng(11)
    H, d, scale = 2, 4, 0.45
    nqs, nks = [3, 0, 5, 1, 4], [3, 2, 7, 4, 0]
    cq, ck = np.concatenate([[0], np.cumsum(nqs)]), np.concatenate([[0], np.cumsum(nks)])
    q = torch.tensor(rng.standard_normal((cq[-1], H, d)), dtype=torch.float32)
    k = torch.tensor(rng.standard_normal((ck[-1], H, d)), dtype=torch.float32)
    v = torch.tensor(rng.standard_normal((ck[-1], H, d)), dtype=torch.float32)
    o, l = oracle.attention_varlen(q, k, v, cq, ck, scale, causal)
    for b, (nq, nk) in enumerate(zip(nqs, nks)):
        for i in range(nq):
            for h in range(H):
                last = min(nk - 1, i + nk - nq) if causal else nk - 1
                kk = [k[ck[b] + j, h] for j in range(nk)]
                vv = [v[ck[b] + j, h] for j in range(nk)]
                want, wl = _brute(q[cq[b] + i, h], kk, vv, scale, last)
                assert np.max(np.abs(o[cq[b] + i, h] - np.array(want))) <= 1e-13
                if wl == -math.inf:
                    assert l[h, cq[b] + i] == -math.inf and np.all(o[cq[b] + i, h] == 0)
                else:
                    assert abs(l[h, cq[b] + i] - wl) <= 1e-13


def test_no_cross_talk_between_sequences():
    g = torch.Generator().manual_seed(8)
    H, d = 3, 8
    cq, ck = [0, 10, 30, 31], [0, 12, 12, 40]
    q = torch.randn((31, H, d), generator=g)
    k = torch.randn((40, H, d), generator=g)
    v = torch.randn((40, H, d), generator=g)
    o1, l1 = oracle.attention_varlen(q, k, v, cq, ck, 0.2, True)
    k2, v2 = k.clone(), v.clone()
    k2[12:] += 5.0
    v2[12:] *= -3.0
    o2, l2 = oracle.attention_varlen(q, k2, v2, cq, ck, 0.2, True)
    assert np.array_equal(o1[:30], o2[:30]) and np.array_equal(l1[:, :30], l2[:, :30])
    assert not np.array_equal(o1[30:], o2[30:])
    # sequence 1 has 20 queries and no key: zero output, -inf LSE
    assert np.all(o1[10:30] == 0) and np.all(np.isneginf(l1[:, 10:30]))


def test_rejects_bad_offsets():
    x = torch.zeros((4, 1, 2))
    with pytest.raises(ValueError):
        oracle.attention_varlen(x, x, x, [0, 3], [0, 4], 1.0)
    with pytest.raises(ValueError):
        oracle.attention_varlen(x, x, x, [0, 3, 2, 4], [0, 1, 2, 4], 1.0)
