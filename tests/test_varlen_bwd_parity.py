"""GPU parity of the packed variable-length backward (fa_bwd_varlen) against the float64
oracle (oracle.attention_varlen_bwd), with O and LSE from fa_fwd_varlen as in training, at
the bounds of the bfloat16 backward (test_bwd_parity.py: each gradient's max and mean error
within 1e-2 and 5e-3 of its own max and mean size)."""
import numpy as np
import pytest
import torch

import exact_tiled_attention_08_amd as fa
import oracle
from parity_util import finite_scale, say, seeded
from test_bwd_parity import compare_grads

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fa.library()


def _cu(lens):
    return torch.tensor([0] + list(np.cumsum(lens)), dtype=torch.int32)


def _run(q, k, v, do, cq, ck, scale, causal, outs=None):
    mq, mk = int((cq[1:] - cq[:-1]).max()), int((ck[1:] - ck[:-1]).max())
    o, lse = fa.fwd_varlen(q, k, v, cq.to(DEV), ck.to(DEV), max(1, mq), scale=scale, causal=causal)
    kw = {} if outs is None else dict(dq=outs[0], dk=outs[1], dv=outs[2])
    g = fa.bwd_varlen(q, k, v, o, lse, do, cq.to(DEV), ck.to(DEV), max(1, mq), max(1, mk),
                      scale=scale, causal=causal, **kw)
    torch.cuda.synchronize()
    return g


def _unattended(nqs, nks, causal):
    """Packed query rows that see no key and key rows that no query sees."""
    qz, kz = [], []
    for nq, nk in zip(nqs, nks):
        for i in range(nq):
            last = nk - 1 if causal == 0 else min(nk - 1, i + nk - nq if causal == 1 else i)
            qz.append(last < 0)
        for j in range(nk):
            first = 0 if causal == 0 else (max(0, j - nk + nq) if causal == 1 else j)
            kz.append(first >= nq)
    return np.array(qz, bool), np.array(kz, bool)


BATCHES = [
    ([1, 255, 256, 257, 100], [1, 255, 256, 257, 100]),
    ([300, 0, 17, 512], [200, 40, 0, 700]),
    ([1000, 1, 96, 97, 129], [1000, 2000, 95, 1, 127]),
]


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [0, 1, 2], ids=["full", "bottom_right", "top_left"])
def test_bwd_varlen_ragged_batches(d, causal):
    """Lengths 0, 1 and around every tile edge; query and key counts differing inside a
    sequence; sequences with keys but no queries and the reverse. Outputs start as NaN and
    every row must be written (zero where a row attends to nothing or is attended by
    nothing)."""
    scale = finite_scale(d)
    H = 3
    for i, (nqs, nks) in enumerate(BATCHES):
        cq, ck = _cu(nqs), _cu(nks)
        say(f"bwd varlen d={d} causal={causal} nq={nqs} nk={nks}")
        tq, tk = int(cq[-1]), int(ck[-1])
        q = seeded((tq, H, d), 7700 + i, torch.bfloat16, mult=2.0)
        k = seeded((tk, H, d), 7710 + i, torch.bfloat16, mult=2.0)
        v = seeded((tk, H, d), 7720 + i, torch.bfloat16)
        do = seeded((tq, H, d), 7730 + i, torch.bfloat16)
        outs = [torch.full(s, float("nan"), device=DEV) for s in ((tq, H, d), (tk, H, d), (tk, H, d))]
        dq, dk, dv = _run(q, k, v, do, cq, ck, scale, causal, outs)
        assert not any(torch.isnan(t).any() for t in (dq, dk, dv))
        rq, rk, rv = oracle.attention_varlen_bwd(q.cpu(), k.cpu(), v.cpu(), do.cpu(), cq.tolist(),
                                                 ck.tolist(), scale, causal)
        got = {"dq": dq.cpu().numpy().reshape(-1, d), "dk": dk.cpu().numpy().reshape(-1, d),
               "dv": dv.cpu().numpy().reshape(-1, d)}
        ref = {"dq": rq.reshape(-1, d), "dk": rk.reshape(-1, d), "dv": rv.reshape(-1, d)}
        # a query row that sees no key, and a key that no query sees, get exactly zero
        qz, kz = _unattended(nqs, nks, causal)
        assert np.all(dq.cpu().numpy()[qz] == 0.0), "query rows that see no key are not zero"
        assert np.all(dk.cpu().numpy()[kz] == 0.0) and np.all(dv.cpu().numpy()[kz] == 0.0), \
            "keys that no query sees are not zero"
        st = compare_grads(got, ref, f"batch {i}")
        say(f"  {st}")


def test_bwd_varlen_equal_lengths_match_dense_bitwise():
    """Equal lengths: the packed path runs the arithmetic of the dense backward on the same
    rows, so the gradients agree bit for bit (each path fed its own forward's O and LSE,
    which agree bit for bit too)."""
    B, H, N, d = 3, 4, 700, 128
    q = seeded((B, H, N, d), 7801, torch.bfloat16, mult=2.0)
    k = seeded((B, H, N, d), 7802, torch.bfloat16, mult=2.0)
    v = seeded((B, H, N, d), 7803, torch.bfloat16)
    do = seeded((B, H, N, d), 7804, torch.bfloat16)
    pack = lambda x: x.permute(0, 2, 1, 3).reshape(B * N, H, d).contiguous()
    cu = _cu([N] * B)
    for causal in (0, 1, 2):
        say(f"bwd varlen vs dense causal={causal}")
        g1 = _run(pack(q), pack(k), pack(v), pack(do), cu, cu, finite_scale(d), causal)
        o, lse = fa.fwd(q, k, v, causal=causal)
        g2 = fa.bwd(q, k, v, o, lse, do, causal=causal)
        torch.cuda.synchronize()
        for a, b in zip(g1, g2):
            assert torch.equal(a, pack(b))


def test_bwd_varlen_deterministic():
    nqs, nks = [300, 0, 17, 512], [200, 40, 0, 700]
    cq, ck = _cu(nqs), _cu(nks)
    H, d = 2, 128
    q = seeded((int(cq[-1]), H, d), 7901, torch.bfloat16, mult=2.0)
    k = seeded((int(ck[-1]), H, d), 7902, torch.bfloat16, mult=2.0)
    v = seeded((int(ck[-1]), H, d), 7903, torch.bfloat16)
    do = seeded((int(cq[-1]), H, d), 7904, torch.bfloat16)
    say("bwd varlen determinism")
    a = _run(q, k, v, do, cq, ck, 0.1, 1)
    b = _run(q, k, v, do, cq, ck, 0.1, 1)
    assert all(torch.equal(x, y) for x, y in zip(a, b))


def test_bwd_varlen_malformed_offsets_stay_inside_tensors():
    """Offsets past the packed lengths are clamped on the device: NaN guard bands around
    every output stay NaN, and the gradients are those of the clamped offsets."""
    H, d = 2, 128
    tq, tk = 300, 250
    q = seeded((tq, H, d), 7951, torch.bfloat16)
    k = seeded((tk, H, d), 7952, torch.bfloat16)
    v = seeded((tk, H, d), 7953, torch.bfloat16)
    do = seeded((tq, H, d), 7954, torch.bfloat16)
    good_q, good_k = _cu([100, 200]), _cu([200, 50])
    o, lse = fa.fwd_varlen(q, k, v, good_q.to(DEV), good_k.to(DEV), 200, scale=0.1, causal=True)
    bands = []
    views = []
    for n in (tq, tk, tk):
        numel = n * H * d
        buf = torch.full((numel + 8192,), float("nan"), device=DEV)
        bands.append((buf, numel))
        views.append(buf[4096:4096 + numel].view(n, H, d))
    cq = torch.tensor([0, 100, 300], dtype=torch.int32, device=DEV)
    ck = torch.tensor([0, 200, 99999], dtype=torch.int32, device=DEV)   # clamped to 250
    say("bwd varlen malformed offsets")
    fa.bwd_varlen(q, k, v, o, lse, do, cq, ck, 200, 200, scale=0.1, causal=True,
                  dq=views[0], dk=views[1], dv=views[2])
    torch.cuda.synchronize()
    for buf, numel in bands:
        assert torch.isnan(buf[:4096]).all() and torch.isnan(buf[4096 + numel:]).all()
    rq, rk, rv = oracle.attention_varlen_bwd(q.cpu(), k.cpu(), v.cpu(), do.cpu(), [0, 100, 300],
                                             [0, 200, 250], 0.1, True)
    got = {n: t.cpu().numpy().reshape(-1, d) for n, t in zip(("dq", "dk", "dv"), views)}
    compare_grads(got, {"dq": rq.reshape(-1, d), "dk": rk.reshape(-1, d), "dv": rv.reshape(-1, d)},
                  "clamped")


def test_bwd_varlen_rejects_on_gpu():
    q = seeded((10, 1, 128), 7990, torch.bfloat16)
    o, lse = torch.zeros((10, 1, 128), device=DEV), torch.zeros((1, 10), device=DEV)
    cu = _cu([10]).to(DEV)
    with pytest.raises(NotImplementedError):   # float32 inputs are not offered here
        fa.bwd_varlen(q.float(), q.float(), q.float(), o, lse, q.float(), cu, cu, 10, 10)
    with pytest.raises(ValueError):            # lse of the wrong layout
        fa.bwd_varlen(q, q, q, o, lse.t().contiguous(), q, cu, cu, 10, 10)
