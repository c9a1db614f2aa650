"""GPU parity of the HIP prefill and decode paths against the float64 oracle.

Tolerances (written out in parity_util): bfloat16 inputs max|O-O*| <= 1e-2,
mean|O-O*| <= 2e-3, max|LSE-LSE*| <= 1e-3; float32 inputs max|O-O*| <= 1e-5*max|O*|
and the same for LSE. The five named workloads run at their full sizes in the launch
configuration the benchmark times; the large ones are compared on sampled rows (every
row the oracle computes is compared element by element).
"""
import math

import numpy as np
import pytest
import torch

import exact_tiled_attention_08_amd as fa
import workloads as W
from parity_util import compare, finite_scale, oracle_rows, rows_of, say, seeded

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fa.library()


def _run_fwd(q, k, v, scale, causal):
    o, lse = fa.fwd(q, k, v, scale=scale, causal=causal)
    torch.cuda.synchronize()
    return o, lse


# ------------------------------------------------------------------ named workloads

@pytest.mark.parametrize("num", [1, 2])
def test_workload_full(num):
    w = W.WORKLOADS[num]
    say(f"workload {num}: {w.name} (all rows)")
    q, k, v = W.make_inputs(w, DEV)
    o, lse = _run_fwd(q, k, v, w.scale, w.causal)
    o_ref, l_ref = oracle_rows(q, k, v, w.scale, w.causal)
    st = compare(o.cpu().numpy().reshape(-1, w.d), lse.cpu().numpy().reshape(-1), o_ref, l_ref,
                 w.dtype, w.name)
    say(f"  {st}")


@pytest.mark.parametrize("num,per_head", [(3, 64), (4, 64)])
def test_workload_sampled(num, per_head):
    w = W.WORKLOADS[num]
    say(f"workload {num}: {w.name} (sampled rows, {per_head} per head)")
    q, k, v = W.make_inputs(w, DEV)
    # outputs start as NaN: every element of the full-size output must be written
    o = torch.full((w.B, w.H, w.Nq, w.d), float("nan"), device=DEV)
    lse = torch.full((w.B, w.H, w.Nq), float("nan"), device=DEV)
    fa.fwd(q, k, v, scale=w.scale, causal=w.causal, out=o, lse=lse)
    torch.cuda.synchronize()
    assert not torch.isnan(o).any() and not torch.isnan(lse).any()
    rows = W.sample_rows(w, per_head)
    o_ref, l_ref = oracle_rows(q, k, v, w.scale, w.causal, rows)
    st = compare(rows_of(o, rows, w.d), rows_of(lse, rows), o_ref, l_ref, w.dtype, w.name)
    say(f"  {st}")


def test_workload_decode_full_size():
    """Decode workload at full size (K and V are 4 GiB each); the oracle checks a sample of
    (b, h) pairs, each over all 32768 keys."""
    w = W.WORKLOADS[5]
    say(f"workload 5: {w.name}")
    q, k, v = W.make_inputs(w, DEV)
    o = torch.full((w.B, w.H, 1, w.d), float("nan"), device=DEV)
    lse = torch.full((w.B, w.H, 1), float("nan"), device=DEV)
    fa.decode(q, k, v, num_splits=w.num_splits, scale=w.scale, out=o, lse=lse)
    torch.cuda.synchronize()
    assert not torch.isnan(o).any() and not torch.isnan(lse).any()  # every (b, h) written
    BH = w.B * w.H
    pick = torch.tensor(sorted({0, 1, 31, 32, 255, 256, BH - 2, BH - 1, *range(7, BH, 37)}))
    qs = q.reshape(BH, 1, 1, w.d)[pick.to(DEV)].reshape(1, -1, 1, w.d)
    ks = k.reshape(BH, w.Nk, w.d)[pick.to(DEV)].reshape(1, -1, w.Nk, w.d)
    vs = v.reshape(BH, w.Nk, w.d)[pick.to(DEV)].reshape(1, -1, w.Nk, w.d)
    o_ref, l_ref = oracle_rows(qs, ks, vs, w.scale, False)
    got_o = o.reshape(BH, w.d)[pick.to(DEV)].double().cpu().numpy()
    got_l = lse.reshape(BH)[pick.to(DEV)].double().cpu().numpy()
    st = compare(got_o, got_l, o_ref, l_ref, w.dtype, w.name)
    say(f"  {len(pick)} heads: {st}")
    # the prefill entry point with one query row must agree as well
    o2, l2 = _run_fwd(qs, ks, vs, w.scale, False)
    compare(o2.cpu().numpy().reshape(-1, w.d), l2.cpu().numpy().reshape(-1), o_ref, l_ref,
            w.dtype, "fa_fwd with Nq=1")


# ------------------------------------------------------------------ edge grid

EDGE_N = [1, 2, 15, 16, 17, 47, 48, 63, 64, 65, 127, 128, 129, 255, 257, 1000]
PAIRS = [(n, n) for n in EDGE_N] + [
    (1, 1000), (1, 129), (17, 1000), (64, 65), (65, 64), (128, 300), (300, 128), (129, 257),
    (257, 129), (1000, 17), (48, 1000), (1000, 255), (2, 63), (63, 2), (255, 256), (16, 15)]


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
def test_edge_grid(dtype, d, causal):
    """Ragged query and key counts around every tile edge, Nq != Nk both ways (bottom-right
    causal alignment; rows that see no key are zero with LSE -inf)."""
    scale = finite_scale(d)
    worst = {}
    for idx, (nq, nk) in enumerate(PAIRS):
        B, H = (1, 3) if nq * nk > 100000 else (2, 3)
        say(f"edge {dtype} d={d} causal={causal} Nq={nq} Nk={nk}")
        q = seeded((B, H, nq, d), 1000 + idx, dtype, mult=2.0)
        k = seeded((B, H, nk, d), 2000 + idx, dtype, mult=2.0)
        v = seeded((B, H, nk, d), 3000 + idx, dtype)
        o, lse = _run_fwd(q, k, v, scale, causal)
        o_ref, l_ref = oracle_rows(q, k, v, scale, causal)
        st = compare(o.cpu().numpy().reshape(-1, d), lse.cpu().numpy().reshape(-1), o_ref, l_ref,
                     dtype, f"Nq={nq} Nk={nk}")
        for key, val in st.items():
            worst[key] = max(worst.get(key, 0.0), val)
    say(f"  worst: {worst}")


@pytest.mark.parametrize("d", [64, 128])
def test_many_heads_grid_mapping(d):
    """B*H divisible by 8 and not: every (b, h, query tile) is computed exactly once."""
    for B, H, n in [(8, 16, 200), (3, 7, 130), (1, 8, 1000), (5, 13, 33)]:
        for causal in (False, True):
            say(f"grid B={B} H={H} N={n} d={d} causal={causal}")
            q = seeded((B, H, n, d), 11, torch.bfloat16, mult=2.0)
            k = seeded((B, H, n, d), 12, torch.bfloat16, mult=2.0)
            v = seeded((B, H, n, d), 13, torch.bfloat16)
            o, lse = _run_fwd(q, k, v, finite_scale(d), causal)
            o_ref, l_ref = oracle_rows(q, k, v, finite_scale(d), causal)
            compare(o.cpu().numpy().reshape(-1, d), lse.cpu().numpy().reshape(-1), o_ref, l_ref,
                    torch.bfloat16, f"B={B} H={H}")


def _tile_edge_rows(BH: int, n: int, tile: int):
    """Flat rows (b*H + h)*n + i: the first and last row of every `tile`-row tile of every
    (b, h), so that every (b, h, tile) of the grid is checked."""
    rows = []
    for bh in range(BH):
        for t0 in range(0, n, tile):
            rows += [bh * n + t0, bh * n + min(n, t0 + tile) - 1]
    return rows


@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
def test_long_heads_grid_mapping(causal):
    """Heads of more than 64 query tiles, two per XCD (B*H = 16): the block -> tile map then
    gives each head its own XCD group. Outputs start as NaN (every element must be written)
    and the first and last row of each of the 65 query tiles of every head match the
    oracle."""
    B, H, n, d = 2, 8, 16640, 64
    say(f"long heads B={B} H={H} N={n} d={d} causal={causal}")
    q = seeded((B, H, n, d), 41, torch.bfloat16, mult=2.0)
    k = seeded((B, H, n, d), 42, torch.bfloat16, mult=2.0)
    v = seeded((B, H, n, d), 43, torch.bfloat16)
    o = torch.full((B, H, n, d), float("nan"), device=DEV)
    lse = torch.full((B, H, n), float("nan"), device=DEV)
    fa.fwd(q, k, v, scale=finite_scale(d), causal=causal, out=o, lse=lse)
    torch.cuda.synchronize()
    assert not torch.isnan(o).any() and not torch.isnan(lse).any()
    rows = _tile_edge_rows(B * H, n, 256)
    o_ref, l_ref = oracle_rows(q, k, v, finite_scale(d), causal, rows)
    st = compare(rows_of(o, rows, d), rows_of(lse, rows), o_ref, l_ref, torch.bfloat16,
                 "long heads")
    say(f"  {st}")


# Causal bfloat16 launches whose B*H is a multiple of 8, with at least 64 query tiles per
# XCD run, hand the lightest tiles of every run out through a ticket counter (one slot of a
# ring of 4096 per call, put back to zero by the last ticket of the launch); the tests
# below use such shapes.

@pytest.mark.parametrize("d,causal,nq,nk", [(128, 1, 4096, 4000), (128, 2, 4000, 4096), (64, 1, 2048, 2048)],
                         ids=["d128-bottom-right", "d128-top-left", "d64"])
def test_dynamic_tail_oracle(d, causal, nq, nk):
    """Outputs start as NaN (every element must be written) and the first and last row of
    every query tile of every head match the oracle."""
    B, H = (2, 16) if d == 128 else (4, 16)
    say(f"dynamic tail B={B} H={H} Nq={nq} Nk={nk} d={d} causal={causal}")
    q = seeded((B, H, nq, d), 51, torch.bfloat16, mult=2.0)
    k = seeded((B, H, nk, d), 52, torch.bfloat16, mult=2.0)
    v = seeded((B, H, nk, d), 53, torch.bfloat16)
    o = torch.full((B, H, nq, d), float("nan"), device=DEV)
    lse = torch.full((B, H, nq), float("nan"), device=DEV)
    fa.fwd(q, k, v, scale=finite_scale(d), causal=causal, out=o, lse=lse)
    torch.cuda.synchronize()
    assert not torch.isnan(o).any() and not torch.isnan(lse).any()
    rows = _tile_edge_rows(B * H, nq, 256)
    o_ref, l_ref = oracle_rows(q, k, v, finite_scale(d), causal, rows)
    st = compare(rows_of(o, rows, d), rows_of(lse, rows), o_ref, l_ref, torch.bfloat16,
                 "dynamic tail")
    say(f"  {st}")


def _count_mismatches(o, lse, o_ref, l_ref, bad):
    # NaN compares unequal, so an element left unwritten counts as a mismatch
    bad += ((o != o_ref).any() | (lse != l_ref).any()).to(torch.int32)


def test_dynamic_tail_counter_reuse():
    """4100 launches in a row, more than the 4096 counter slots, so every slot is used again
    after the launch before put it back to zero: each launch writes every element of its
    NaN-filled outputs and matches the first launch bitwise."""
    B, H, n, d = 64, 8, 256, 128  # 512 one-tile heads: 64 items per XCD run
    say(f"dynamic tail counter reuse B={B} H={H} N={n} d={d}, 4100 launches")
    q = seeded((B, H, n, d), 61, torch.bfloat16, mult=2.0)
    k = seeded((B, H, n, d), 62, torch.bfloat16, mult=2.0)
    v = seeded((B, H, n, d), 63, torch.bfloat16)
    o_ref, l_ref = fa.fwd(q, k, v, scale=finite_scale(d), causal=True)
    o = torch.empty_like(o_ref)
    lse = torch.empty_like(l_ref)
    bad = torch.zeros((), dtype=torch.int32, device=DEV)
    for _ in range(4100):
        o.fill_(float("nan"))
        lse.fill_(float("nan"))
        fa.fwd(q, k, v, scale=finite_scale(d), causal=True, out=o, lse=lse)
        _count_mismatches(o, lse, o_ref, l_ref, bad)
    torch.cuda.synchronize()
    assert not torch.isnan(o_ref).any()
    assert int(bad) == 0, f"{int(bad)} of 4100 launches differ from the first"


def test_dynamic_tail_two_streams():
    """Calls on two streams at once take different counter slots: interleaved launches on
    two streams, each into its own NaN-filled outputs, all match a lone launch bitwise."""
    B, H, n, d = 2, 16, 4096, 128
    say(f"dynamic tail on two streams B={B} H={H} N={n} d={d}")
    q = seeded((B, H, n, d), 71, torch.bfloat16, mult=2.0)
    k = seeded((B, H, n, d), 72, torch.bfloat16, mult=2.0)
    v = seeded((B, H, n, d), 73, torch.bfloat16)
    o_ref, l_ref = fa.fwd(q, k, v, scale=finite_scale(d), causal=True)
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    bufs = [(torch.empty_like(o_ref), torch.empty_like(l_ref)) for _ in streams]
    bads = [torch.zeros((), dtype=torch.int32, device=DEV) for _ in streams]
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())
    for _ in range(20):
        for s, (o, lse), bad in zip(streams, bufs, bads):
            with torch.cuda.stream(s):
                o.fill_(float("nan"))
                lse.fill_(float("nan"))
                fa.fwd(q, k, v, scale=finite_scale(d), causal=True, out=o, lse=lse)
                _count_mismatches(o, lse, o_ref, l_ref, bad)
    torch.cuda.synchronize()
    assert [int(b) for b in bads] == [0, 0]


# ------------------------------------------------------------------ closed forms on the GPU

@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
def test_zero_query_gives_mean_of_visible_values(dtype):
    d, B, H, n = 128, 2, 4, 300
    v = seeded((B, H, n, d), 5, dtype)
    k = seeded((B, H, n, d), 6, dtype)
    q = torch.zeros((B, H, n, d), dtype=dtype, device=DEV)
    for causal in (False, True):
        say(f"q=0 {dtype} causal={causal}")
        o, lse = _run_fwd(q, k, v, 0.1, causal)
        vd = v.double().cpu()
        cnt = torch.arange(1, n + 1, dtype=torch.float64)
        want = vd.cumsum(2) / cnt[None, None, :, None] if causal else vd.mean(2, keepdim=True).expand_as(vd)
        assert torch.max(torch.abs(o.double().cpu() - want)).item() <= 2e-6
        wl = torch.log(cnt) if causal else torch.full((n,), math.log(n), dtype=torch.float64)
        assert torch.max(torch.abs(lse.double().cpu() - wl)).item() <= 2e-6


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
def test_constant_values_and_causal_first_row(dtype):
    d, B, H, n = 64, 2, 2, 257
    q = seeded((B, H, n, d), 7, dtype, mult=3.0)
    k = seeded((B, H, n, d), 8, dtype, mult=3.0)
    ones = torch.ones((B, H, n, d), dtype=dtype, device=DEV)
    say(f"V=1 {dtype}")
    o, _ = _run_fwd(q, k, ones, 0.125, False)
    # float32: numerator and denominator are two float32 sums of n positive terms in different
    # orders, each within (n-1)u of exact (u = 2^-24), so their ratio is within 2(n-1)u of 1.
    # bfloat16: the numerator sums bf16-rounded weights (relative error <= 2^-9 each).
    tol = 4e-3 if dtype == torch.bfloat16 else 2 * (n - 1) * 2.0 ** -24
    assert torch.max(torch.abs(o - 1.0)).item() <= tol
    v = seeded((B, H, n, d), 9, dtype)
    o, lse = _run_fwd(q, k, v, 0.125, True)
    # row 0 sees only key 0: its weight is exp(s - m) with m = s, i.e. 1 up to the rounding of s*c
    v0 = v[:, :, 0].double().cpu()
    assert torch.max(torch.abs(o[:, :, 0].double().cpu() - v0)).item() <= 1e-6 * v0.abs().max().item()
    s00 = (q[:, :, 0].double() * k[:, :, 0].double()).sum(-1) * 0.125
    assert torch.max(torch.abs(lse[:, :, 0].double() - s00)).item() <= 1e-4


# ------------------------------------------------------------------ memory behaviour

def test_outputs_fully_overwritten_and_no_reads_past_tensors():
    """Inputs sit between NaN guard bands and outputs start as NaN: every output element is
    written, and no kernel reads outside its tensors (a NaN read would surface in O)."""
    d = 128
    for (B, H, nq, nk, causal) in [(1, 2, 100, 77, False), (2, 1, 77, 100, True), (1, 1, 1, 1000, False)]:
        say(f"guard bands B={B} H={H} Nq={nq} Nk={nk} causal={causal}")
        bufs = []
        for (n, seed) in ((nq, 21), (nk, 22), (nk, 23)):
            numel = B * H * n * d
            guard = 4096
            buf = torch.full((numel + 2 * guard,), float("nan"), dtype=torch.bfloat16, device=DEV)
            buf[guard:guard + numel] = seeded((numel,), seed, torch.bfloat16)
            bufs.append(buf[guard:guard + numel].view(B, H, n, d))
        q, k, v = bufs
        o = torch.full((B, H, nq, d), float("nan"), device=DEV)
        lse = torch.full((B, H, nq), float("nan"), device=DEV)
        fa.fwd(q, k, v, scale=0.09, causal=causal, out=o, lse=lse)
        torch.cuda.synchronize()
        assert not torch.isnan(o).any() and not torch.isnan(lse).any()
        o_ref, l_ref = oracle_rows(q, k, v, 0.09, causal)
        compare(o.cpu().numpy().reshape(-1, d), lse.cpu().numpy().reshape(-1), o_ref, l_ref,
                torch.bfloat16, "guard")
    # decode: same guard bands, splits that leave empty chunks
    B, H, nk = 2, 3, 50
    numel = B * H * nk * d
    kv = []
    for seed in (31, 32):
        buf = torch.full((numel + 8192,), float("nan"), dtype=torch.bfloat16, device=DEV)
        buf[4096:4096 + numel] = seeded((numel,), seed, torch.bfloat16)
        kv.append(buf[4096:4096 + numel].view(B, H, nk, d))
    q = seeded((B, H, 1, d), 33, torch.bfloat16)
    o = torch.full((B, H, 1, d), float("nan"), device=DEV)
    lse = torch.full((B, H, 1), float("nan"), device=DEV)
    say("guard bands decode")
    fa.decode(q, kv[0], kv[1], num_splits=64, scale=0.09, out=o, lse=lse)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle_rows(q, kv[0], kv[1], 0.09, False)
    compare(o.cpu().numpy().reshape(-1, d), lse.cpu().numpy().reshape(-1), o_ref, l_ref,
            torch.bfloat16, "guard decode")


def test_bitwise_deterministic():
    w = W.WORKLOADS[3]
    say("determinism on the causal N=8192 workload shape (one batch)")
    q, k, v = (t[:1].contiguous() for t in W.make_inputs(w, DEV))
    o1, l1 = _run_fwd(q, k, v, w.scale, True)
    o2, l2 = _run_fwd(q, k, v, w.scale, True)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    q = seeded((4, 8, 1, 128), 41, torch.bfloat16)
    k = seeded((4, 8, 5000, 128), 42, torch.bfloat16)
    v = seeded((4, 8, 5000, 128), 43, torch.bfloat16)
    a = fa.decode(q, k, v, num_splits=37)
    b = fa.decode(q, k, v, num_splits=37)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


# ------------------------------------------------------------------ decode cases

@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
@pytest.mark.parametrize("d", [64, 128])
def test_decode_splits(dtype, d):
    """Chunk count from 1 to more chunks than keys (empty chunks), ragged Nk."""
    for (B, H, nk, S) in [(2, 3, 1, 1), (2, 3, 1, 64), (1, 4, 7, 3), (2, 2, 100, 7), (1, 2, 129, 64),
                          (3, 2, 1000, 1), (2, 2, 4097, 64), (1, 3, 513, 1024), (1, 1, 33000, 64)]:
        say(f"decode {dtype} d={d} B={B} H={H} Nk={nk} S={S}")
        q = seeded((B, H, 1, d), 51 + nk, dtype, mult=2.0)
        k = seeded((B, H, nk, d), 52 + nk, dtype, mult=2.0)
        v = seeded((B, H, nk, d), 53 + nk, dtype)
        o, lse = fa.decode(q, k, v, num_splits=S, scale=finite_scale(d))
        torch.cuda.synchronize()
        o_ref, l_ref = oracle_rows(q, k, v, finite_scale(d), False)
        compare(o.cpu().numpy().reshape(-1, d), lse.cpu().numpy().reshape(-1), o_ref, l_ref, dtype,
                f"decode Nk={nk} S={S}")


def test_python_layer_rejects_on_gpu():
    q = torch.zeros((1, 1, 4, 96), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(NotImplementedError):
        fa.fwd(q, q, q)
    q = torch.zeros((1, 1, 4, 64), dtype=torch.float16, device=DEV)
    with pytest.raises(NotImplementedError):
        fa.fwd(q, q, q)
    q = torch.zeros((1, 1, 2, 64), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(ValueError):
        fa.decode(q, q, q)
