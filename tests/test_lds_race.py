"""Race check of the bfloat16 prefill's LDS pipeline ("Explain FlashAttention ...", section
"Executable recurrence, with an empty-state policy", names race checks among the tests a
GPU implementation needs).

libfa_ldscheck.so is the product library built with FA_LDS_POISON: before each direct
load into an LDS slot (K, V and bias tiles), the issuing lane writes NaN into the slot and
waits for that write. A wave that reads a slot after its refill was issued (a stale tile)
or before the new tile landed reads NaN. With correct barriers and load waits nothing of
the kind happens, so the poisoned build must return bitwise the product library's results
(and those match the oracle); any early or late read shows up as NaN or as a difference.
The shapes put the key tail, the causal diagonal and the first and last tiles of a
workgroup at every tile position, with both head sizes, every mask setting, Nq != Nk both
ways, the packed variable-length path and the additive bias.
"""
import ctypes
import math

import numpy as np
import pytest
import torch

import exact_tiled_attention_08_amd as fa
from exact_tiled_attention_08_amd import build as fabuild
import workloads as W
from parity_util import compare, finite_scale, oracle_rows, say, seeded

pytestmark = pytest.mark.gpu

DEV = "cuda"
_check = None


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fa.library()
    global _check
    lib = ctypes.CDLL(fabuild.CHECK_LIB)
    for name in ("fa_fwd", "fa_fwd_varlen", "fa_fwd_bias"):
        res, args = fa._SIGS[name]
        fn = getattr(lib, name)
        fn.restype, fn.argtypes = res, args
    _check = lib


def _stream():
    return torch.cuda.current_stream().cuda_stream


def _fwd_check(q, k, v, scale, causal):
    B, H, Nq, d = q.shape
    o = torch.full((B, H, Nq, d), float("nan"), dtype=torch.float32, device=DEV)
    lse = torch.full((B, H, Nq), float("nan"), dtype=torch.float32, device=DEV)
    st = _check.fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                       B, H, Nq, k.shape[2], d, scale, int(causal), fa.FA_BF16, _stream())
    assert st == fa.FA_OK, fa.status_str(st)
    return o, lse


def _same(a, b, what):
    assert not torch.isnan(a[0]).any(), f"{what}: NaN in O (a read of a poisoned LDS slot)"
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1]), \
        f"{what}: differs from the product library"


PAIRS = [(1, 1), (31, 33), (95, 97), (96, 96), (97, 95), (200, 200), (255, 257), (256, 256),
         (257, 255), (300, 64), (64, 300), (513, 700), (700, 513), (1000, 1000)]


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [0, 1, 2], ids=["full", "bottom_right", "top_left"])
def test_poisoned_prefill_edge_grid(d, causal):
    scale = finite_scale(d)
    for idx, (nq, nk) in enumerate(PAIRS):
        say(f"poisoned prefill d={d} causal={causal} Nq={nq} Nk={nk}")
        B, H = (1, 2) if nq * nk > 200000 else (2, 3)
        q = seeded((B, H, nq, d), 4000 + idx, torch.bfloat16, mult=2.0)
        k = seeded((B, H, nk, d), 4100 + idx, torch.bfloat16, mult=2.0)
        v = seeded((B, H, nk, d), 4200 + idx, torch.bfloat16)
        got = _fwd_check(q, k, v, scale, causal)
        ref = fa.fwd(q, k, v, scale=scale, causal=causal)
        torch.cuda.synchronize()
        _same(got, ref, f"d={d} causal={causal} Nq={nq} Nk={nk}")
        if nq * nk <= 300000:
            o_ref, l_ref = oracle_rows(q, k, v, scale, causal)
            compare(got[0].cpu().numpy().reshape(-1, d), got[1].cpu().numpy().reshape(-1),
                    o_ref, l_ref, torch.bfloat16, f"poisoned Nq={nq} Nk={nk}")


def test_poisoned_prefill_long_workload():
    """The causal N = 8192 workload at full size (many tiles per workgroup, both buffers of
    every tensor refilled dozens of times), bitwise against the product library."""
    w = W.WORKLOADS[3]
    say(f"poisoned prefill: {w.name}")
    q, k, v = W.make_inputs(w, DEV)
    got = _fwd_check(q, k, v, w.scale, 1)
    ref = fa.fwd(q, k, v, scale=w.scale, causal=True)
    torch.cuda.synchronize()
    _same(got, ref, w.name)


def test_poisoned_varlen_and_bias():
    d, H = 128, 3
    lens_q, lens_k = [300, 1, 97, 700, 0, 256], [300, 5, 96, 700, 10, 257]
    cu_q = torch.tensor(np.concatenate([[0], np.cumsum(lens_q)]), dtype=torch.int32, device=DEV)
    cu_k = torch.tensor(np.concatenate([[0], np.cumsum(lens_k)]), dtype=torch.int32, device=DEV)
    q = seeded((sum(lens_q), H, d), 4300, torch.bfloat16, mult=2.0)
    k = seeded((sum(lens_k), H, d), 4301, torch.bfloat16, mult=2.0)
    v = seeded((sum(lens_k), H, d), 4302, torch.bfloat16)
    scale = finite_scale(d)
    for causal in (0, 1, 2):
        say(f"poisoned varlen causal={causal}")
        o = torch.full((sum(lens_q), H, d), float("nan"), device=DEV)
        lse = torch.full((H, sum(lens_q)), float("nan"), device=DEV)
        st = _check.fa_fwd_varlen(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                  lse.data_ptr(), cu_q.data_ptr(), cu_k.data_ptr(), len(lens_q),
                                  H, sum(lens_q), sum(lens_k), max(lens_q), d, scale, causal,
                                  fa.FA_BF16, _stream())
        assert st == fa.FA_OK
        ref = fa.fwd_varlen(q, k, v, cu_q, cu_k, max(lens_q), scale=scale, causal=causal)
        torch.cuda.synchronize()
        _same((o, lse), ref, f"varlen causal={causal}")
    B, Hb, nq, nk = 2, 2, 333, 517
    qb = seeded((B, Hb, nq, d), 4310, torch.bfloat16, mult=2.0)
    kb = seeded((B, Hb, nk, d), 4311, torch.bfloat16, mult=2.0)
    vb = seeded((B, Hb, nk, d), 4312, torch.bfloat16)
    bias = fa.pad_bias(seeded((B, Hb, nq, nk), 4313, torch.bfloat16, mult=2.0))
    be, sb, sh, sq = fa._bias_strides(bias, qb, B, Hb, nq, nk)
    for causal in (0, 1):
        say(f"poisoned bias causal={causal}")
        o = torch.full((B, Hb, nq, d), float("nan"), device=DEV)
        lse = torch.full((B, Hb, nq), float("nan"), device=DEV)
        st = _check.fa_fwd_bias(qb.data_ptr(), kb.data_ptr(), vb.data_ptr(), be.data_ptr(), sb, sh,
                                sq, o.data_ptr(), lse.data_ptr(), B, Hb, nq, nk, d, scale, causal,
                                fa.FA_BF16, _stream())
        assert st == fa.FA_OK
        ref = fa.fwd_bias(qb, kb, vb, bias, scale=scale, causal=causal)
        torch.cuda.synchronize()
        _same((o, lse), ref, f"bias causal={causal}")
