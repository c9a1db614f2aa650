"""GPU parity at the largest sizes the library accepts: one head whose keys fill the 32-bit
in-head offset range (Nk * d = 2^30 elements, 2 GiB of bfloat16 per tensor), through the
prefill (both dtypes), the split-KV decode and the backward pass. The kernels address a
head's rows with 32-bit byte offsets from a 64-bit head base, so the last key rows sit just
below 2^31 bytes; the oracle checks sampled rows that include them. One size past the limit
is rejected before any launch.
"""
import numpy as np
import pytest
import torch

import exact_tiled_attention_08_amd as fa
import oracle
from parity_util import F32_REL, compare, finite_scale, rows_of, say, seeded
from test_bwd_parity import compare_grads

pytestmark = pytest.mark.gpu

DEV = "cuda"
LIMIT = 1 << 30  # Nk * d elements per head


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fa.library()


def _sample(nq):
    return sorted({0, 1, nq // 2, nq - 2, nq - 1} | set(range(3, nq, max(1, nq // 11))))


@pytest.mark.parametrize("d,causal", [(128, 0), (128, 1), (64, 2)])
def test_prefill_bf16_at_offset_limit(d, causal):
    """300 queries against Nk = 2^30 / d keys (bottom-right causal: every query sees almost
    every key; top-left: the first few keys only, the rest masked)."""
    nk, nq = LIMIT // d, 300
    say(f"max-size prefill bf16 d={d} causal={causal} Nq={nq} Nk={nk}")
    q = seeded((1, 1, nq, d), 9001, torch.bfloat16, mult=2.0)
    k = seeded((1, 1, nk, d), 9002, torch.bfloat16)
    v = seeded((1, 1, nk, d), 9003, torch.bfloat16)
    o, lse = fa.fwd(q, k, v, causal=causal)
    torch.cuda.synchronize()
    rows = _sample(nq)
    say(f"  oracle on {len(rows)} rows")
    ro, rl = oracle.attention(q.cpu(), k.cpu(), v.cpu(), finite_scale(d), causal, rows=rows)
    st = compare(rows_of(o, rows, d), rows_of(lse, rows), ro, rl, torch.bfloat16, "max-size prefill")
    say(f"  {st}")


def test_prefill_f32_at_offset_limit():
    """The float32 prefill (4 GiB per tensor) with 40 queries against Nk = 2^23 keys.

    The float32 bound is 1e-5 relative; with 8.4M values of random sign each output is ~1e-3
    of the values it averages, so the bound is taken relative to the largest sum_j P_ij |v_j|
    (the attention of |V|, which the oracle computes) rather than to max|O*|: the rounding of
    a float32 sum scales with its summands, not with its result (at N = 256 the two differ
    by a small factor; here by ~400x)."""
    d, nq = 128, 40
    nk = LIMIT // d
    say(f"max-size prefill f32 Nq={nq} Nk={nk}")
    q = seeded((1, 1, nq, d), 9011, torch.float32)
    k = seeded((1, 1, nk, d), 9012, torch.float32)
    v = seeded((1, 1, nk, d), 9013, torch.float32)
    o, lse = fa.fwd(q, k, v, causal=1)
    torch.cuda.synchronize()
    rows = _sample(nq)
    qc, kc, vc = q.cpu(), k.cpu(), v.cpu()
    ro, rl = oracle.attention(qc, kc, vc, finite_scale(d), 1, rows=rows)
    ra, _ = oracle.attention(qc, kc, vc.abs(), finite_scale(d), 1, rows=rows)
    go, gl = rows_of(o, rows, d), rows_of(lse, rows)
    o_err = float(np.abs(go - ro).max())
    l_err = float(np.abs(gl - rl).max())
    say(f"  O max err {o_err:.3e} (summand scale {ra.max():.3f}), LSE max err {l_err:.3e}")
    assert np.all(np.isfinite(go))
    assert o_err <= F32_REL * float(ra.max())
    assert l_err <= F32_REL * float(np.abs(rl).max())


def test_decode_at_offset_limit():
    """Split-KV decode of two heads, each with Nk = 2^23 keys (64 chunks of 131072 keys)."""
    d, nk = 128, LIMIT // 128
    say(f"max-size decode H=2 Nk={nk}")
    q = seeded((1, 2, 1, d), 9021, torch.bfloat16)
    k = seeded((1, 2, nk, d), 9022, torch.bfloat16)
    v = seeded((1, 2, nk, d), 9023, torch.bfloat16)
    o, lse = fa.decode(q, k, v, num_splits=64)
    torch.cuda.synchronize()
    ro, rl = oracle.attention(q.cpu(), k.cpu(), v.cpu(), finite_scale(d), 0)
    st = compare(o.cpu().numpy().reshape(-1, d), lse.cpu().numpy().reshape(-1), ro, rl,
                 torch.bfloat16, "max-size decode")
    say(f"  {st}")


def test_backward_at_offset_limit():
    """The backward pass with 64 queries against Nk = 2^23 keys (non-causal): dQ on sampled
    rows, dK and dV on sampled key rows that include the last ones."""
    d, nq = 128, 64
    nk = LIMIT // d
    say(f"max-size backward Nq={nq} Nk={nk}")
    q = seeded((1, 1, nq, d), 9031, torch.bfloat16, mult=2.0)
    k = seeded((1, 1, nk, d), 9032, torch.bfloat16, mult=2.0)
    v = seeded((1, 1, nk, d), 9033, torch.bfloat16)
    do = seeded((1, 1, nq, d), 9034, torch.bfloat16)
    o, lse = fa.fwd(q, k, v)
    dq, dk, dv = fa.bwd(q, k, v, o, lse, do)
    torch.cuda.synchronize()
    qrows = [0, 1, 31, 32, 62, 63]
    krows = [0, 1, 127, 128, nk // 2, nk - 129, nk - 128, nk - 2, nk - 1]
    krows += [int(x) for x in np.random.default_rng(9035).choice(nk, 23, replace=False)]
    krows = sorted(set(krows))
    say(f"  oracle: {len(qrows)} dQ rows, {len(krows)} dK/dV rows")
    rq, rk, rv = oracle.attention_bwd(q.cpu(), k.cpu(), v.cpu(), do.cpu(), finite_scale(d), 0,
                                      qrows=qrows, krows=krows)
    got = {"dq": rows_of(dq, qrows, d), "dk": rows_of(dk, krows, d), "dv": rows_of(dv, krows, d)}
    st = compare_grads(got, {"dq": rq, "dk": rk, "dv": rv}, "max-size backward")
    say(f"  {st}")


def test_one_key_past_the_limit_is_rejected():
    """Nk * d = 2^30 + d: fa_fwd returns FA_ERR_UNSUPPORTED before any launch (the inputs
    are never read, so small stand-ins of the right dtype serve)."""
    d = 128
    nk = LIMIT // d + 1
    lib = fa.library()
    q = torch.zeros((1, 1, 1, d), dtype=torch.bfloat16, device=DEV)
    o = torch.empty((1, 1, 1, d), device=DEV)
    st = lib.fa_fwd(q.data_ptr(), q.data_ptr(), q.data_ptr(), o.data_ptr(), None, 1, 1, 1, nk, d,
                    0.1, 0, 0, fa._stream_ptr(q.device))
    assert st == fa.FA_ERR_UNSUPPORTED
