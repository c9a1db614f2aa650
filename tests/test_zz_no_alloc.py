"""The allocation-free decode entry point (fa_decode_splitkv_noalloc), called through the C
ABI, against the entry point it varies (fa_decode_splitkv with a caller's workspace) and the
float64 oracle, on two calls in a row, the second with a smaller input: the fixed scratch
then still holds the first call's partial states, which the second must not read.

Bar: bit-identical to fa_decode_splitkv (same kernels, same inputs); against the oracle the
bounds of the other parity tests (bfloat16: max|O-O*| <= 1e-2, mean <= 2e-3, max|LSE-LSE*|
<= 1e-3; float32: 1e-5 of the largest reference magnitude).
"""
import numpy as np
import pytest
import torch

import exact_tiled_attention_08_amd as fa
from parity_util import compare, finite_scale, oracle_rows, say, seeded

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fa.library()


def _noalloc_c(q, k, v, S, scale, stream):
    """Direct C-ABI call; q, k, v, o and lse are the caller's (torch-owned) buffers."""
    B, H, _, d = q.shape
    o = torch.full((B, H, 1, d), float("nan"), dtype=torch.float32, device=DEV)
    lse = torch.full((B, H, 1), float("nan"), dtype=torch.float32, device=DEV)
    st = fa.library().fa_decode_splitkv_noalloc(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), B, H,
        k.shape[2], d, scale, S, fa.FA_BF16 if q.dtype == torch.bfloat16 else fa.FA_F32,
        stream.cuda_stream)
    assert st == fa.FA_OK, fa.status_str(st)
    return o, lse


def _case(B, H, Nk, d, S, dtype, seed, stream):
    q = seeded((B, H, 1, d), seed, dtype)
    k = seeded((B, H, Nk, d), seed + 1, dtype)
    v = seeded((B, H, Nk, d), seed + 2, dtype)
    scale = finite_scale(d)
    with torch.cuda.stream(stream):
        o, lse = _noalloc_c(q, k, v, S, scale, stream)
        o_ref_gpu, l_ref_gpu = fa.decode(q, k, v, num_splits=S, scale=scale)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref_gpu) and torch.equal(lse, l_ref_gpu), \
        "differs from fa_decode_splitkv on the same inputs"
    o_ref, l_ref = oracle_rows(q, k, v, scale, False)
    return compare(o.cpu().numpy().reshape(-1, d), lse.cpu().numpy().reshape(-1), o_ref, l_ref,
                   dtype, f"noalloc B={B} H={H} Nk={Nk} d={d} S={S}")


def test_noalloc_decode_two_calls_second_smaller():
    big = (8, 16, 3000, 128, 64, torch.bfloat16)     # 8*16*64 partial states, 4.3 MB
    small = (2, 3, 700, 64, 16, torch.bfloat16)       # 2*3*16 partial states, inside the first
    say(f"noalloc decode, first call {big}")
    st = _case(*big, 1200, torch.cuda.current_stream())
    say(f"  {st}")
    say(f"noalloc decode, second call {small} (scratch still holds the first call's states)")
    st = _case(*small, 1300, torch.cuda.current_stream())
    say(f"  {st}")


def test_noalloc_decode_on_a_side_stream_and_float32():
    side = torch.cuda.Stream()  # default priority
    say("noalloc decode on a side stream, float32, then bfloat16 with more splits than keys")
    st = _case(3, 5, 1500, 128, 32, torch.float32, 1400, side)
    say(f"  {st}")
    st = _case(2, 2, 40, 128, 64, torch.bfloat16, 1500, side)   # empty chunks
    say(f"  {st}")


def test_noalloc_binding_and_limit():
    q = seeded((2, 2, 1, 128), 1600, torch.bfloat16)
    k = seeded((2, 2, 900, 128), 1601, torch.bfloat16)
    v = seeded((2, 2, 900, 128), 1602, torch.bfloat16)
    say("noalloc binding vs decode")
    a = fa.decode_noalloc(q, k, v, num_splits=8)
    b = fa.decode(q, k, v, num_splits=8)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    # a decode whose partial states exceed the fixed scratch is refused before any launch
    S = 1024
    need = fa.decode_workspace_bytes(64, 1, 128, S)
    assert need > fa.NOALLOC_SCRATCH_BYTES
    qb = seeded((64, 1, 1, 128), 1603, torch.bfloat16)
    kb = seeded((64, 1, 8, 128), 1604, torch.bfloat16)
    with pytest.raises(ValueError):
        fa.decode_noalloc(qb, kb, kb, num_splits=S)
