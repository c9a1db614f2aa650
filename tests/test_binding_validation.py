"""The binding refuses caller-supplied outputs and workspaces that the kernels would write
through wrongly (a host tensor, another shape or dtype, a non-contiguous view, a short
workspace), with ValueError and before any call into libfa.so that could launch a kernel.

The C ABI takes bare device pointers and cannot check the size of what they point to, so
these checks are the only guard against a write past the end of a caller's buffer.
"""
import math

import pytest
import torch

import exact_tiled_attention_08_amd as fa
import workloads as W
from parity_util import say, seeded

pytestmark = pytest.mark.gpu

DEV = "cuda"
# entry points of libfa.so that only compute sizes or strings (never launch anything)
_SIZE_ONLY = {"fa_decode_workspace_bytes", "fa_bwd_workspace_bytes", "fa_status_str",
              "fa_last_hip_error", "fa_last_hip_error_str"}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fa.library()


class _NoLaunch:
    """Stands in for the loaded library: size queries pass through, any other entry point
    fails the test (it would launch a kernel)."""

    def __init__(self, real):
        self._real = real

    def __getattr__(self, name):
        if name in _SIZE_ONLY:
            return getattr(self._real, name)
        raise AssertionError(f"{name} was called although an argument was invalid")


@pytest.fixture
def no_launch(monkeypatch):
    spy = _NoLaunch(fa.library())
    monkeypatch.setattr(fa, "library", lambda: spy)
    return spy


def _bad_outputs(shape):
    """(label, tensor) pairs that must be refused as a float32 output of `shape`."""
    n = math.prod(shape)
    return [
        ("host tensor", torch.empty(shape, dtype=torch.float32)),
        ("one element short", torch.empty(n - 1, dtype=torch.float32, device=DEV)),
        ("wrong shape, same size", torch.empty((n,), dtype=torch.float32, device=DEV)),
        ("bfloat16", torch.empty(shape, dtype=torch.bfloat16, device=DEV)),
        ("not contiguous", torch.empty((*shape[:-1], 2 * shape[-1]), dtype=torch.float32,
                                       device=DEV)[..., ::2]),
    ]


def _qkv(B=1, H=2, Nq=70, Nk=90, d=128, dtype=torch.bfloat16):
    return (seeded((B, H, Nq, d), 900, dtype), seeded((B, H, Nk, d), 901, dtype),
            seeded((B, H, Nk, d), 902, dtype))


def test_fwd_outputs(no_launch):
    q, k, v = _qkv()
    for label, t in _bad_outputs((1, 2, 70, 128)):
        say(f"fwd out: {label}")
        with pytest.raises(ValueError):
            fa.fwd(q, k, v, out=t)
    for label, t in _bad_outputs((1, 2, 70)):
        say(f"fwd lse: {label}")
        with pytest.raises(ValueError):
            fa.fwd(q, k, v, lse=t)


def test_fwd_bias_outputs(no_launch):
    q, k, v = _qkv()
    bias = fa.pad_bias(seeded((1, 1, 1, 90), 903, torch.bfloat16))
    for label, t in _bad_outputs((1, 2, 70, 128)):
        say(f"fwd_bias out: {label}")
        with pytest.raises(ValueError):
            fa.fwd_bias(q, k, v, bias, out=t)
    for label, t in _bad_outputs((1, 2, 70)):
        say(f"fwd_bias lse: {label}")
        with pytest.raises(ValueError):
            fa.fwd_bias(q, k, v, bias, lse=t)


def test_fwd_fp8_outputs(no_launch):
    q, k, v = (x.to(torch.float8_e4m3fn) for x in _qkv())
    for label, t in _bad_outputs((1, 2, 70, 128)):
        say(f"fwd_fp8 out: {label}")
        with pytest.raises(ValueError):
            fa.fwd_fp8(q, k, v, 1.0, 1.0, 1.0, out=t)
    for label, t in _bad_outputs((1, 2, 70)):
        say(f"fwd_fp8 lse: {label}")
        with pytest.raises(ValueError):
            fa.fwd_fp8(q, k, v, 1.0, 1.0, 1.0, lse=t)


def test_fwd_varlen_outputs(no_launch):
    lens = [40, 30]
    cu = torch.tensor([0, 40, 70], dtype=torch.int32, device=DEV)
    q, k, v = (seeded((sum(lens), 2, 128), 910 + i, torch.bfloat16) for i in range(3))
    for label, t in _bad_outputs((70, 2, 128)):
        say(f"fwd_varlen out: {label}")
        with pytest.raises(ValueError):
            fa.fwd_varlen(q, k, v, cu, cu, 40, out=t)
    for label, t in _bad_outputs((2, 70)):
        say(f"fwd_varlen lse: {label}")
        with pytest.raises(ValueError):
            fa.fwd_varlen(q, k, v, cu, cu, 40, lse=t)


def test_decode_outputs_and_workspace(no_launch):
    q = seeded((2, 3, 1, 128), 920, torch.bfloat16)
    k, v = (seeded((2, 3, 500, 128), 921 + i, torch.bfloat16) for i in range(2))
    for label, t in _bad_outputs((2, 3, 1, 128)):
        say(f"decode out: {label}")
        with pytest.raises(ValueError):
            fa.decode(q, k, v, num_splits=8, out=t)
    for label, t in _bad_outputs((2, 3, 1)):
        say(f"decode lse: {label}")
        with pytest.raises(ValueError):
            fa.decode(q, k, v, num_splits=8, lse=t)
    need = fa.decode_workspace_bytes(2, 3, 128, 8)
    for label, ws in (("short", torch.empty(need - 1, dtype=torch.uint8, device=DEV)),
                      ("host", torch.empty(need, dtype=torch.uint8))):
        say(f"decode workspace: {label}")
        with pytest.raises(ValueError):
            fa.decode(q, k, v, num_splits=8, workspace=ws)


def test_decode_paged_outputs_and_workspace(no_launch):
    q = seeded((2, 3, 1, 128), 930, torch.bfloat16)
    k, v = (seeded((2, 3, 256, 128), 931 + i, torch.bfloat16) for i in range(2))
    kc, table = W.to_paged(k, 64, 5)
    vc, _ = W.to_paged(v, 64, 5)
    lens = torch.full((2,), 256, dtype=torch.int32, device=DEV)
    for label, t in _bad_outputs((2, 3, 1, 128)):
        say(f"decode_paged out: {label}")
        with pytest.raises(ValueError):
            fa.decode_paged(q, kc, vc, table, lens, num_splits=4, out=t)
    for label, t in _bad_outputs((2, 3, 1)):
        say(f"decode_paged lse: {label}")
        with pytest.raises(ValueError):
            fa.decode_paged(q, kc, vc, table, lens, num_splits=4, lse=t)
    need = fa.decode_workspace_bytes(2, 3, 128, 4)
    say("decode_paged workspace: short")
    with pytest.raises(ValueError):
        fa.decode_paged(q, kc, vc, table, lens, num_splits=4,
                        workspace=torch.empty(need - 1, dtype=torch.uint8, device=DEV))


def test_bwd_outputs_and_workspace(no_launch):
    q, k, v = _qkv()
    o = torch.zeros((1, 2, 70, 128), dtype=torch.float32, device=DEV)
    lse = torch.zeros((1, 2, 70), dtype=torch.float32, device=DEV)
    do = seeded((1, 2, 70, 128), 940, torch.bfloat16)
    for name, shape in (("dq", (1, 2, 70, 128)), ("dk", (1, 2, 90, 128)), ("dv", (1, 2, 90, 128))):
        for label, t in _bad_outputs(shape):
            say(f"bwd {name}: {label}")
            with pytest.raises(ValueError):
                fa.bwd(q, k, v, o, lse, do, **{name: t})
    need = fa.bwd_workspace_bytes(1, 2, 70)
    say("bwd workspace: short")
    with pytest.raises(ValueError):
        fa.bwd(q, k, v, o, lse, do, workspace=torch.empty(need - 1, dtype=torch.uint8, device=DEV))


def test_valid_outputs_still_accepted():
    """The checks refuse only what they must: exact-size caller buffers work as before."""
    q, k, v = _qkv()
    out = torch.full((1, 2, 70, 128), float("nan"), dtype=torch.float32, device=DEV)
    lse = torch.full((1, 2, 70), float("nan"), dtype=torch.float32, device=DEV)
    say("fwd with caller buffers")
    o2, l2 = fa.fwd(q, k, v, out=out, lse=lse)
    o1, l1 = fa.fwd(q, k, v)
    torch.cuda.synchronize()
    assert o2 is out and l2 is lse
    assert torch.equal(o1, out) and torch.equal(l1, lse)
