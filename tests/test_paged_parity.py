"""GPU parity of the paged-cache decode (fa_decode_paged) against the float64 oracle.

Tolerances are those of the contiguous decode (parity_util): bfloat16 max|O-O*| <= 1e-2,
mean <= 2e-3, max|LSE-LSE*| <= 1e-3; float32 1e-5 relative. The oracle gathers each
sequence's rows through the block table (oracle.paged_attention) from CPU copies of the
exact bytes the kernel read.
"""
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


def _case(B, H, d, ps, lens, S, dtype, seed, extra_pages=3, bad_ids=False):
    P = max(1, max(-(-n // ps) for n in lens))
    num_pages = B * P + extra_pages
    kc = seeded((num_pages, ps, H, d), seed, dtype, mult=2.0)
    vc = seeded((num_pages, ps, H, d), seed + 1, dtype)
    q = seeded((B, H, 1, d), seed + 2, dtype, mult=2.0)
    g = torch.Generator().manual_seed(seed)
    table = torch.randperm(num_pages, generator=g)[:B * P].view(B, P).to(torch.int32)
    if bad_ids:
        table[0, 0] = num_pages          # outside the pool
        table[B - 1, P - 1] = -5
    lens_t = torch.tensor(lens, dtype=torch.int32)
    scale = finite_scale(d)
    say(f"paged {dtype} d={d} B={B} H={H} ps={ps} lens={lens[:6]}{'...' if len(lens) > 6 else ''} "
        f"S={S} bad_ids={bad_ids}")
    o, lse = fa.decode_paged(q, kc, vc, table.to(DEV), lens_t.to(DEV), num_splits=S, scale=scale)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.paged_attention(q.cpu(), kc.cpu(), vc.cpu(), table, lens, ps, scale)
    return compare(o.cpu().numpy().reshape(-1, d), lse.cpu().numpy().reshape(-1), o_ref, l_ref,
                   dtype, f"paged ps={ps}")


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
@pytest.mark.parametrize("d", [64, 128])
def test_paged_lengths_and_page_sizes(dtype, d):
    """Page sizes 1 to 256; lengths 0, 1, around page edges and several thousand; chunk
    counts from 1 to more chunks than keys."""
    for i, (ps, lens, S) in enumerate([
            (16, [1, 15, 16, 17], 1), (16, [0, 33, 300, 1000], 7), (1, [1, 5, 64], 64),
            (64, [63, 64, 65, 4000], 64), (256, [255, 257, 3000], 3), (4, [9, 100], 1024),
            (128, [5000, 1, 0, 129], 64)]):
        st = _case(len(lens), 3, d, ps, lens, S, dtype, 500 + 10 * i)
        say(f"  {st}")


def test_paged_pages_outside_pool_are_skipped():
    st = _case(3, 2, 128, 16, [100, 40, 64], 8, torch.bfloat16, 900, bad_ids=True)
    say(f"  {st}")


def test_paged_matches_contiguous_decode_bitwise():
    """Pages in order with full lengths hold the same rows in the same order as the
    contiguous cache: the two entry points run the same arithmetic and agree bit for bit."""
    B, H, N, d, ps, S = 3, 4, 1000, 128, 64, 16
    q = seeded((B, H, 1, d), 61, torch.bfloat16, mult=2.0)
    k = seeded((B, H, N, d), 62, torch.bfloat16, mult=2.0)
    v = seeded((B, H, N, d), 63, torch.bfloat16)
    say("paged vs contiguous, identity placement")
    P = -(-N // ps)
    kc = torch.zeros((B * P, ps, H, d), dtype=torch.bfloat16, device=DEV)
    vc = torch.zeros_like(kc)
    for b in range(B):
        for j in range(P):
            n = min(ps, N - j * ps)
            kc[b * P + j, :n] = k[b, :, j * ps:j * ps + n].transpose(0, 1)
            vc[b * P + j, :n] = v[b, :, j * ps:j * ps + n].transpose(0, 1)
    table = torch.arange(B * P, dtype=torch.int32, device=DEV).view(B, P)
    lens = torch.full((B,), N, dtype=torch.int32, device=DEV)
    o1, l1 = fa.decode_paged(q, kc, vc, table, lens, num_splits=S)
    o2, l2 = fa.decode(q, k, v, num_splits=S)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_paged_decode_workload_shape_sampled():
    """The decode workload (B=16, H=32, Nk=32768, d=128, 64 splits) laid out in 64-key pages
    placed in a seeded random order across the pool, as the benchmark times it; the oracle
    checks a sample of (b, h) pairs over all their keys."""
    w = W.WORKLOADS[5]
    say("paged decode workload shape, page size 64, shuffled pages")
    q, k, v = W.make_inputs(w, DEV)
    kc, table = W.to_paged(k, 64, 55)
    del k
    vc, _ = W.to_paged(v, 64, 55)
    del v
    torch.cuda.empty_cache()
    lens = torch.full((w.B,), w.Nk, dtype=torch.int32, device=DEV)
    o, lse = fa.decode_paged(q, kc, vc, table, lens, num_splits=w.num_splits, scale=w.scale)
    torch.cuda.synchronize()
    bs = [0, 7, 15]
    tab = table.cpu()
    qs = q[bs].cpu()
    kcs, vcs = kc.cpu(), vc.cpu()
    o_ref, l_ref = oracle.paged_attention(qs, kcs, vcs, tab[bs], [w.Nk] * len(bs), 64, w.scale)
    got_o = o[bs].reshape(-1, w.d).double().cpu().numpy()
    got_l = lse[bs].reshape(-1).double().cpu().numpy()
    st = compare(got_o, got_l, o_ref, l_ref, w.dtype, "paged workload")
    say(f"  {len(bs)} sequences x {w.H} heads: {st}")


def test_paged_python_layer_rejects_on_gpu():
    q = torch.zeros((2, 2, 1, 64), dtype=torch.bfloat16, device=DEV)
    kc = torch.zeros((4, 16, 2, 64), dtype=torch.bfloat16, device=DEV)
    tab = torch.zeros((2, 2), dtype=torch.int32, device=DEV)
    lens = torch.ones((2,), dtype=torch.int32, device=DEV)
    with pytest.raises(ValueError):
        fa.decode_paged(q, kc, kc, tab.long(), lens)       # table must be int32
    with pytest.raises(NotImplementedError):
        kc3 = torch.zeros((4, 12, 2, 64), dtype=torch.bfloat16, device=DEV)
        fa.decode_paged(q, kc3, kc3, tab, lens)            # page size not a power of two
