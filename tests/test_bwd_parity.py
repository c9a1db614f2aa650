"""GPU parity of the HIP backward pass (fa_bwd) against the float64 oracle.

The forward O and LSE fed to fa_bwd come from fa_fwd, as in training. The oracle
(oracle.attention_bwd) recomputes everything from q, k, v and dO in float64.

Tolerance (the forward's bounds do not cover gradients, so it is derived from the
kernels' arithmetic): P and dS enter the MFMAs as bfloat16 (relative rounding error up to
2^-9 per operand); S, dP, the row statistics and every accumulation are float32. A float32
model of exactly that arithmetic (tests/tolerance_model.py, checked by
tests/test_tolerance_model.py), fed the O and LSE of a model of the forward with its own
bfloat16 rounding of P, stays within 3.0e-3 * max|g*| (max error) and 1.8e-3 * mean|g*|
(mean error) on shapes from N = 128 to 2048, d = 64 and 128, every mask setting and the
sharp (x3) Q, K of the N = 8192 workload. The bounds are about three times that, for each
of dQ, dK and dV over the compared elements:
    max|g - g*| <= 1e-2 * max|g*|        mean|g - g*| <= 5e-3 * mean|g*|
A gradient that is zero in exact arithmetic (dQ and dK when no query row sees more than
one key) is float32 rounding residue; only for such a gradient are max|g*| and mean|g*|
replaced by 1e-2 of the largest gradient of the case.
"""
import math

import numpy as np
import pytest
import torch

import exact_tiled_attention_08_amd as fa
import oracle
import workloads as W
from parity_util import BWD_BF16_MAX_REL, BWD_BF16_MEAN_REL, finite_scale, rows_of, say, seeded

pytestmark = pytest.mark.gpu

DEV = "cuda"
GRAD_MAX_REL, GRAD_MEAN_REL = BWD_BF16_MAX_REL, BWD_BF16_MEAN_REL


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fa.library()


def _fwd_bwd(q, k, v, do, scale, causal):
    """Forward, then backward into NaN-filled gradients, every element of which must be
    written (zero where a row or key takes part in nothing)."""
    o, lse = fa.fwd(q, k, v, scale=scale, causal=causal)
    dq = torch.full(q.shape, float("nan"), device=q.device)
    dk = torch.full(k.shape, float("nan"), device=q.device)
    dv = torch.full(v.shape, float("nan"), device=q.device)
    fa.bwd(q, k, v, o, lse, do, scale=scale, causal=causal, dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    assert not any(torch.isnan(t).any() for t in (dq, dk, dv)), "gradient elements left unwritten"
    return dq, dk, dv


def exact_zero_grads(nq: int, nk: int, causal) -> set:
    """Gradients that are identically zero in exact arithmetic for this shape and mask: when no
    query row sees more than one key, every probability is 0 or 1, dS = P (dP - dO.O) = 0, and
    so dQ = dK = 0. A row sees at most Nk keys; with the top-left causal mask (2) row i sees
    min(Nk, i + 1), so a single query row sees one key."""
    c = int(causal)
    most = min(nk, nq) if c == 2 else nk
    return {"dq", "dk"} if most <= 1 else set()


def compare_grads(got: dict, ref: dict, what: str, max_rel: float = GRAD_MAX_REL,
                  mean_rel: float = GRAD_MEAN_REL, floor_frac: float = 1e-2, zero=frozenset()):
    """got/ref: name -> [rows, d] arrays of the compared rows. Raises outside the bounds
    max_rel * max|ref| and mean_rel * mean|ref| of each gradient (the bfloat16 path's by
    default).

    `zero` names the gradients that are identically zero in exact arithmetic for the case
    (exact_zero_grads): what the kernels return for them is float32 rounding residue, so their
    bounds are taken relative to floor_frac times the largest gradient of the case instead of
    their own (zero) size. Every other gradient is judged against its own size only."""
    stats = {}
    floor = floor_frac * max(float(np.abs(r).max(initial=0.0)) for r in ref.values())
    for name in ("dq", "dk", "dv"):
        if name not in ref or ref[name].size == 0:
            continue
        g = np.asarray(got[name], np.float64).reshape(ref[name].shape)
        r = ref[name]
        assert np.all(np.isfinite(g)), f"{what}: non-finite {name}"
        err = np.abs(g - r)
        if name in zero:
            assert float(np.abs(r).max()) <= 1e-12 * max(floor, 1e-300), \
                f"{what}: {name} was declared zero but the oracle's is not"
            amax = amean = floor
        else:
            amax, amean = float(np.abs(r).max()), float(np.abs(r).mean())
        emax, emean = float(err.max()), float(err.mean())
        stats[name] = (emax / max(amax, 1e-30), emean / max(amean, 1e-30))
        assert emax <= max_rel * amax, f"{what}: {name} max err {emax:.3e} vs max|ref| {amax:.3e}"
        assert emean <= mean_rel * amean, \
            f"{what}: {name} mean err {emean:.3e} vs mean|ref| {amean:.3e}"
    return {k: f"{a:.2e}/{b:.2e}" for k, (a, b) in stats.items()}


def _all_rows(q, k, v, do, scale, causal, dq, dk, dv, what, **bounds):
    d = q.shape[-1]
    rq, rk, rv = oracle.attention_bwd(q.cpu(), k.cpu(), v.cpu(), do.cpu(), scale, causal)
    got = {"dq": dq.cpu().numpy().reshape(-1, d), "dk": dk.cpu().numpy().reshape(-1, d),
           "dv": dv.cpu().numpy().reshape(-1, d)}
    zero = exact_zero_grads(q.shape[2], k.shape[2], causal)
    return compare_grads(got, {"dq": rq, "dk": rk, "dv": rv}, what, zero=zero, **bounds)


# ------------------------------------------------------------------ edge grid

BWD_PAIRS = [(1, 1), (2, 2), (17, 17), (31, 33), (63, 64), (64, 64), (65, 65), (127, 129),
             (128, 128), (129, 127), (200, 200), (257, 255), (1, 300), (300, 1), (17, 200),
             (200, 17), (64, 300), (300, 64), (500, 500)]


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
def test_bwd_edge_grid(d, causal):
    """Ragged sizes around every tile edge (64-row LDS tiles, 128-row workgroups), Nq != Nk
    both ways; rows that see no key (causal, Nq > Nk) contribute nothing."""
    scale = finite_scale(d)
    for idx, (nq, nk) in enumerate(BWD_PAIRS):
        B, H = (1, 2) if nq * nk > 50000 else (2, 3)
        say(f"bwd edge d={d} causal={causal} Nq={nq} Nk={nk}")
        q = seeded((B, H, nq, d), 100 + idx, torch.bfloat16, mult=2.0)
        k = seeded((B, H, nk, d), 200 + idx, torch.bfloat16, mult=2.0)
        v = seeded((B, H, nk, d), 300 + idx, torch.bfloat16)
        do = seeded((B, H, nq, d), 400 + idx, torch.bfloat16)
        dq, dk, dv = _fwd_bwd(q, k, v, do, scale, causal)
        st = _all_rows(q, k, v, do, scale, causal, dq, dk, dv, f"Nq={nq} Nk={nk}")
        say(f"  {st}")


@pytest.mark.parametrize("d", [64, 128])
def test_bwd_many_heads_grid_mapping(d):
    """B*H divisible by 8 and not, several key and query tiles per head."""
    for B, H, n in [(8, 2, 260), (3, 5, 130), (1, 8, 700)]:
        for causal in (False, True):
            say(f"bwd grid B={B} H={H} N={n} d={d} causal={causal}")
            q = seeded((B, H, n, d), 11, torch.bfloat16, mult=2.0)
            k = seeded((B, H, n, d), 12, torch.bfloat16, mult=2.0)
            v = seeded((B, H, n, d), 13, torch.bfloat16)
            do = seeded((B, H, n, d), 14, torch.bfloat16)
            dq, dk, dv = _fwd_bwd(q, k, v, do, finite_scale(d), causal)
            _all_rows(q, k, v, do, finite_scale(d), causal, dq, dk, dv, f"B={B} H={H}")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [1, 2], ids=["bottom_right", "top_left"])
def test_bwd_diagonal_loop_boundaries(d, causal):
    """The dK/dV kernel runs the query tiles that cross the causal diagonal in a loop of their
    own before the unmasked ones; these shapes put the switch at even and odd tile counts,
    at the first tile (keys offset far behind the queries) and past the last one (keys far
    ahead), with several 128-key workgroups per head."""
    for nq, nk in [(1000, 1000), (1000, 1064), (1064, 1000), (640, 2000), (2000, 640),
                   (130, 1500), (1500, 130)]:
        say(f"bwd diagonal loops d={d} causal={causal} Nq={nq} Nk={nk}")
        q = seeded((1, 2, nq, d), 31, torch.bfloat16, mult=2.0)
        k = seeded((1, 2, nk, d), 32, torch.bfloat16, mult=2.0)
        v = seeded((1, 2, nk, d), 33, torch.bfloat16)
        do = seeded((1, 2, nq, d), 34, torch.bfloat16)
        dq, dk, dv = _fwd_bwd(q, k, v, do, finite_scale(d), causal)
        st = _all_rows(q, k, v, do, finite_scale(d), causal, dq, dk, dv, f"Nq={nq} Nk={nk}")
        say(f"  {st}")


# ------------------------------------------------------------------ named workloads

def _sampled_workload(num, heads_kv, per_head_q, per_head_k):
    w = W.WORKLOADS[num]
    q, k, v = W.make_inputs(w, DEV)
    do = W.make_grad(w, DEV)
    dq, dk, dv = _fwd_bwd(q, k, v, do, w.scale, w.causal)
    BH = w.B * w.H
    qrows = W.sample_rows(w, per_head_q)
    # dK/dV rows need the statistics of every query row of their head: a few heads only
    kw = W.Workload(w.number, w.name, w.B, w.H, w.Nk, w.Nk, w.d, w.dtype, w.causal)
    all_k = np.asarray(W.sample_rows(kw, per_head_k), np.int64)
    pick = sorted({0, BH - 1, *range(5, BH, max(1, BH // max(1, heads_kv - 2)))})[:heads_kv]
    krows = [int(r) for r in all_k if (r // w.Nk) in set(pick)]
    say(f"  oracle: {len(qrows)} dQ rows, {len(krows)} dK/dV rows in heads {pick}")
    rq, rk, rv = oracle.attention_bwd(q.cpu(), k.cpu(), v.cpu(), do.cpu(), w.scale, w.causal,
                                      qrows=qrows, krows=krows)
    got = {"dq": rows_of(dq, qrows, w.d), "dk": rows_of(dk, krows, w.d), "dv": rows_of(dv, krows, w.d)}
    return compare_grads(got, {"dq": rq, "dk": rk, "dv": rv}, w.name), (w, do, dk, dv)


def test_bwd_workload2_sampled():
    say("bwd workload 2: bf16 B=4 H=16 N=2048 d=64 (sampled rows)")
    st, _ = _sampled_workload(2, heads_kv=4, per_head_q=32, per_head_k=48)
    say(f"  {st}")


def test_bwd_workload3_sampled():
    say("bwd workload 3: bf16 causal B=2 H=16 N=8192 d=128, Q,K x3 (sampled rows)")
    st, _ = _sampled_workload(3, heads_kv=2, per_head_q=32, per_head_k=48)
    say(f"  {st}")


def test_bwd_workload4_properties():
    """N = 30000 causal at full size: the sums that hold exactly for any input.
    sum_j dV_j = sum_i dO_i (rows of P sum to 1; every query row sees key 0) and
    sum_j dK_j = 0 (each row of dS sums to 0), each per (b, h) and dimension."""
    w = W.WORKLOADS[4]
    say(f"bwd workload 4: {w.name} (column sums)")
    q, k, v = W.make_inputs(w, DEV)
    do = W.make_grad(w, DEV)
    dq, dk, dv = _fwd_bwd(q, k, v, do, w.scale, w.causal)
    sv = dv.double().sum(2)
    so = do.double().sum(2)
    # each dV_j is float32 with relative error ~1e-3 of its size; the sums compare to the
    # scale of the summed magnitudes
    mag_v = dv.double().abs().sum(2)
    assert torch.all((sv - so).abs() <= 5e-3 * mag_v + 1e-3), float(((sv - so).abs() / mag_v).max())
    sk = dk.double().sum(2)
    mag_k = dk.double().abs().sum(2)
    assert torch.all(sk.abs() <= 5e-3 * mag_k), float((sk.abs() / mag_k).max())
    assert torch.isfinite(dq).all()


@pytest.mark.timeout(900)
def test_bwd_workload4_oracle():
    """N = 30000 causal at full size against the oracle: dQ on 64 sampled rows of every head;
    dK and dV on every key row of head (0, 0) (all 235 of its 128-key workgroups, in the
    mapping that gives each head its own XCD group, which only heads of more than 64 key
    tiles use) and on 64 sampled key rows of the last head."""
    w = W.WORKLOADS[4]
    say(f"bwd workload 4: {w.name} (oracle: sampled dQ rows, one full head of dK/dV)")
    q, k, v = W.make_inputs(w, DEV)
    do = W.make_grad(w, DEV)
    dq, dk, dv = _fwd_bwd(q, k, v, do, w.scale, w.causal)
    BH = w.B * w.H
    qrows = W.sample_rows(w, 64)
    kw = W.Workload(w.number, w.name, w.B, w.H, w.Nk, w.Nk, w.d, w.dtype, w.causal)
    last = [int(r) for r in W.sample_rows(kw, 64) if r // w.Nk == BH - 1]
    krows = list(range(w.Nk)) + last
    say(f"  oracle: {len(qrows)} dQ rows, {len(krows)} dK/dV rows (head 0 whole, head {BH - 1} "
        f"sampled)")
    rq, rk, rv = oracle.attention_bwd(q.cpu(), k.cpu(), v.cpu(), do.cpu(), w.scale, w.causal,
                                      qrows=qrows, krows=krows)
    got = {"dq": rows_of(dq, qrows, w.d), "dk": rows_of(dk, krows, w.d),
           "dv": rows_of(dv, krows, w.d)}
    st = compare_grads(got, {"dq": rq, "dk": rk, "dv": rv}, w.name)
    say(f"  {st}")


@pytest.mark.timeout(600)
@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
def test_bwd_long_heads_grid_mapping(causal):
    """Heads of more than 64 key and query tiles of 128, two per XCD (B*H = 16): both main
    kernels then give each head its own XCD group. Gradients start as NaN (every element
    must be written); dQ on the first and last row of every 128-row query tile and dK, dV on
    the first and last row of every 128-key tile of every head match the oracle."""
    B, H, n, d = 2, 8, 8320, 64
    say(f"bwd long heads B={B} H={H} N={n} d={d} causal={causal}")
    q = seeded((B, H, n, d), 71, torch.bfloat16, mult=2.0)
    k = seeded((B, H, n, d), 72, torch.bfloat16, mult=2.0)
    v = seeded((B, H, n, d), 73, torch.bfloat16)
    do = seeded((B, H, n, d), 74, torch.bfloat16)
    scale = finite_scale(d)
    o, lse = fa.fwd(q, k, v, scale=scale, causal=causal)
    g = [torch.full((B, H, n, d), float("nan"), device=DEV) for _ in range(3)]
    fa.bwd(q, k, v, o, lse, do, scale=scale, causal=causal, dq=g[0], dk=g[1], dv=g[2])
    torch.cuda.synchronize()
    assert not any(torch.isnan(t).any() for t in g)
    rows = []
    for bh in range(B * H):
        for t0 in range(0, n, 128):
            rows += [bh * n + t0, bh * n + min(n, t0 + 128) - 1]
    say(f"  oracle: {len(rows)} rows of dQ and of dK/dV")
    rq, rk, rv = oracle.attention_bwd(q.cpu(), k.cpu(), v.cpu(), do.cpu(), scale, causal,
                                      qrows=rows, krows=rows)
    got = {"dq": rows_of(g[0], rows, d), "dk": rows_of(g[1], rows, d), "dv": rows_of(g[2], rows, d)}
    st = compare_grads(got, {"dq": rq, "dk": rk, "dv": rv}, "long heads")
    say(f"  {st}")


# ------------------------------------------------------------------ closed forms and behaviour

def test_bwd_zero_grad_and_single_key():
    """dO = 0 gives exactly zero gradients. With one key, P = 1, so dV_0 = sum_i dO_i and
    dS = dP - dO.O = 0 up to float32 rounding (O = v_0 to ~1e-7 relative, dP and dO.O of
    size ~10): dQ and dK stay below 1e-3, against gradients of order 1 to 10."""
    d, B, H, n = 128, 1, 2, 200
    q = seeded((B, H, n, d), 61, torch.bfloat16, mult=2.0)
    k = seeded((B, H, n, d), 62, torch.bfloat16, mult=2.0)
    v = seeded((B, H, n, d), 63, torch.bfloat16)
    zero = torch.zeros_like(q)
    for causal in (False, True):
        say(f"bwd dO=0 causal={causal}")
        dq, dk, dv = _fwd_bwd(q, k, v, zero, 0.1, causal)
        assert not dq.any() and not dk.any() and not dv.any()
    k1, v1 = k[:, :, :1].contiguous(), v[:, :, :1].contiguous()
    do = seeded((B, H, n, d), 64, torch.bfloat16)
    say("bwd Nk=1")
    dq, dk, dv = _fwd_bwd(q, k1, v1, do, 0.1, False)
    want = do.double().sum(2)
    assert torch.allclose(dv[:, :, 0].double(), want, rtol=0, atol=1e-4 * float(want.abs().max()))
    assert float(dq.abs().max()) <= 1e-3 and float(dk.abs().max()) <= 1e-3


def test_bwd_outputs_fully_overwritten_and_deterministic():
    """Outputs start as NaN and every element is written; two calls agree bit for bit."""
    d = 128
    for (B, H, nq, nk, causal) in [(1, 2, 100, 77, False), (2, 1, 77, 300, True), (1, 1, 300, 77, True)]:
        say(f"bwd guard B={B} H={H} Nq={nq} Nk={nk} causal={causal}")
        q = seeded((B, H, nq, d), 71, torch.bfloat16, mult=2.0)
        k = seeded((B, H, nk, d), 72, torch.bfloat16, mult=2.0)
        v = seeded((B, H, nk, d), 73, torch.bfloat16)
        do = seeded((B, H, nq, d), 74, torch.bfloat16)
        o, lse = fa.fwd(q, k, v, scale=0.09, causal=causal)
        outs = []
        for _ in range(2):
            dq = torch.full((B, H, nq, d), float("nan"), device=DEV)
            dk = torch.full((B, H, nk, d), float("nan"), device=DEV)
            dv = torch.full((B, H, nk, d), float("nan"), device=DEV)
            ws = torch.full((fa.bwd_workspace_bytes(B, H, nq) // 4,), float("nan"), device=DEV)
            fa.bwd(q, k, v, o, lse, do, scale=0.09, causal=causal, dq=dq, dk=dk, dv=dv, workspace=ws)
            torch.cuda.synchronize()
            assert not (torch.isnan(dq).any() or torch.isnan(dk).any() or torch.isnan(dv).any())
            outs.append((dq, dk, dv))
        assert all(torch.equal(a, b) for a, b in zip(*outs))
        _all_rows(q, k, v, do, 0.09, causal, *outs[0], "guard")


def test_bwd_python_layer_rejects_on_gpu():
    q = torch.zeros((1, 1, 4, 64), dtype=torch.float32, device=DEV)
    o = torch.zeros((1, 1, 4, 64), dtype=torch.float32, device=DEV)
    lse = torch.zeros((1, 1, 4), dtype=torch.float32, device=DEV)
    q96 = torch.zeros((1, 1, 4, 96), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(NotImplementedError):       # head size 96 is not provided
        fa.bwd(q96, q96, q96, torch.zeros((1, 1, 4, 96), device=DEV), lse, q96)
    qb = q.to(torch.bfloat16)
    with pytest.raises(ValueError):
        fa.bwd(qb, qb, qb, o, lse, q)              # dO dtype differs from q
    with pytest.raises(ValueError):
        fa.bwd(qb, qb, qb, o.to(torch.bfloat16), lse, qb)   # o must be float32
