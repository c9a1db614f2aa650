"""GPU parity of the packed variable-length prefill (fa_fwd_varlen) against the float64
oracle (oracle.attention_varlen), at the bfloat16 bounds of the prefill (parity_util):
max|O-O*| <= 1e-2, mean|O-O*| <= 2e-3, max|LSE-LSE*| <= 1e-3."""
import numpy as np
import pytest
import torch

import exact_tiled_attention_08_amd as fa
import oracle
import workloads as W
from parity_util import compare, finite_scale, say, seeded

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fa.library()


def _cu(lens):
    return torch.tensor([0] + list(np.cumsum(lens)), dtype=torch.int32)


def _check(q, k, v, cq, ck, max_q, scale, causal, what, rows=None):
    o, lse = fa.fwd_varlen(q, k, v, cq.to(DEV), ck.to(DEV), max_q, scale=scale, causal=causal)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.attention_varlen(q.cpu(), k.cpu(), v.cpu(), cq.tolist(), ck.tolist(),
                                           scale, causal)
    H, d = q.shape[1], q.shape[2]
    got_o = o.cpu().numpy()
    got_l = lse.cpu().numpy()
    if rows is not None:
        got_o, o_ref = got_o[rows], o_ref[rows]
        got_l, l_ref = got_l[:, rows], l_ref[:, rows]
    # compare per (row, head): O [rows*H, d], LSE in the same (row, head) order
    return compare(got_o.reshape(-1, d), got_l.T.reshape(-1), o_ref.reshape(-1, d),
                   l_ref.T.reshape(-1), torch.bfloat16, what)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
def test_varlen_ragged_batches(d, causal):
    """Lengths 0, 1 and around every tile edge; query and key counts differing inside a
    sequence (bottom-right causal alignment); sequences with keys but no queries and the
    reverse."""
    scale = finite_scale(d)
    for i, (nqs, nks) in enumerate([
            ([1, 255, 256, 257, 100], [1, 255, 256, 257, 100]),
            ([300, 0, 17, 512], [200, 40, 0, 700]),
            ([1000, 1, 96, 97], [1000, 2000, 95, 1])]):
        H = 3
        cq, ck = _cu(nqs), _cu(nks)
        say(f"varlen d={d} causal={causal} nq={nqs} nk={nks}")
        q = seeded((int(cq[-1]), H, d), 700 + i, torch.bfloat16, mult=2.0)
        k = seeded((int(ck[-1]), H, d), 710 + i, torch.bfloat16, mult=2.0)
        v = seeded((int(ck[-1]), H, d), 720 + i, torch.bfloat16)
        st = _check(q, k, v, cq, ck, max(nqs), scale, causal, f"varlen {i}")
        say(f"  {st}")


def test_varlen_equal_lengths_match_dense_bitwise():
    """Equal lengths: the packed layout holds the same rows as a dense [B, H, N, d] tensor,
    and the two entry points run the same arithmetic, so they agree bit for bit."""
    B, H, N, d = 3, 4, 700, 128
    q = seeded((B, H, N, d), 81, torch.bfloat16, mult=2.0)
    k = seeded((B, H, N, d), 82, torch.bfloat16, mult=2.0)
    v = seeded((B, H, N, d), 83, torch.bfloat16)
    pack = lambda x: x.permute(0, 2, 1, 3).reshape(B * N, H, d).contiguous()
    cu = _cu([N] * B).to(DEV)
    for causal in (False, True):
        say(f"varlen vs dense causal={causal}")
        o1, l1 = fa.fwd_varlen(pack(q), pack(k), pack(v), cu, cu, N, causal=causal)
        o2, l2 = fa.fwd(q, k, v, causal=causal)
        torch.cuda.synchronize()
        assert torch.equal(o1, pack(o2))
        assert torch.equal(l1, l2.permute(1, 0, 2).reshape(H, B * N))


def test_varlen_malformed_offsets_stay_inside_tensors():
    """Offsets past the packed lengths are clamped on the device: no access outside the
    tensors (NaN guard bands around every buffer stay NaN) and the result is that of the
    clamped offsets."""
    H, d = 2, 128
    tq, tk = 300, 250
    bufs = []
    for n, seed in ((tq, 91), (tk, 92), (tk, 93)):
        numel = n * H * d
        buf = torch.full((numel + 8192,), float("nan"), dtype=torch.bfloat16, device=DEV)
        buf[4096:4096 + numel] = seeded((numel,), seed, torch.bfloat16)
        bufs.append(buf[4096:4096 + numel].view(n, H, d))
    q, k, v = bufs
    ob = torch.full((tq * H * d + 8192,), float("nan"), device=DEV)
    o = ob[4096:4096 + tq * H * d].view(tq, H, d)
    lb = torch.full((H * tq + 8192,), float("nan"), device=DEV)
    lse = lb[4096:4096 + H * tq].view(H, tq)
    cq = torch.tensor([0, 100, 300], dtype=torch.int32)
    ck = torch.tensor([0, 200, 99999], dtype=torch.int32)   # past total_k: clamped to 250
    say("varlen malformed offsets")
    fa.fwd_varlen(q, k, v, cq.to(DEV), ck.to(DEV), 200, scale=0.1, causal=True, out=o, lse=lse)
    torch.cuda.synchronize()
    assert torch.isnan(ob[:4096]).all() and torch.isnan(ob[4096 + tq * H * d:]).all()
    assert torch.isnan(lb[:4096]).all() and torch.isnan(lb[4096 + H * tq:]).all()
    o_ref, l_ref = oracle.attention_varlen(q.cpu(), k.cpu(), v.cpu(), [0, 100, 300], [0, 200, 250], 0.1, True)
    compare(o.cpu().numpy().reshape(-1, d), lse.cpu().numpy().T.reshape(-1), o_ref.reshape(-1, d),
            l_ref.T.reshape(-1), torch.bfloat16, "clamped")


def test_varlen_workload_sampled():
    """The packed prefill the benchmark times (16 causal sequences of seeded lengths in
    [256, 8192], H = 16, d = 128): sampled rows of every sequence, each over all its keys."""
    q, k, v, cu, lens = W.make_varlen(DEV)
    say(f"varlen workload: {len(lens)} sequences, {sum(lens)} tokens")
    rng = np.random.default_rng(3)
    rows = []
    for b, n in enumerate(lens):
        s = int(cu[b])
        pick = {0, 1, n // 2, n - 2, n - 1, *rng.choice(n, size=8, replace=False).tolist()}
        rows.extend(s + i for i in sorted(pick) if 0 <= i < n)
    # the oracle evaluates whole sequences: restrict it to the sampled rows' sequences by
    # running it on each sequence separately
    o, lse = fa.fwd_varlen(q, k, v, cu, cu, max(lens), causal=True)
    torch.cuda.synchronize()
    scale = finite_scale(128)
    got_o, got_l, ref_o, ref_l = [], [], [], []
    for b, n in enumerate(lens):
        s = int(cu[b])
        rb = [r - s for r in rows if s <= r < s + n]
        qb = q[s:s + n].permute(1, 0, 2)[None].cpu()
        kb = k[s:s + n].permute(1, 0, 2)[None].cpu()
        vb = v[s:s + n].permute(1, 0, 2)[None].cpu()
        H = qb.shape[1]
        flat = [h * n + i for h in range(H) for i in rb]
        ob, lb = oracle.attention(qb.contiguous(), kb.contiguous(), vb.contiguous(), scale, True, rows=flat)
        ref_o.append(ob)
        ref_l.append(lb)
        idx = torch.tensor([s + i for i in rb], device=DEV)
        got_o.append(o[idx].permute(1, 0, 2).reshape(-1, 128).double().cpu().numpy())
        got_l.append(lse[:, idx].reshape(-1).double().cpu().numpy())
    st = compare(np.concatenate(got_o), np.concatenate(got_l), np.concatenate(ref_o),
                 np.concatenate(ref_l), torch.bfloat16, "varlen workload")
    say(f"  {len(rows)} rows x 16 heads: {st}")
