"""C-ABI checks that need no GPU: the library loads, exports every declared symbol, and
rejects bad arguments with the documented status before making any HIP call."""
import ctypes
import os
import re

import pytest

import exact_tiled_attention_08_amd as fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")

# a fake, 16-byte aligned, never dereferenced "device" address: validation must reject the
# call before anything touches it
P = 0x10000


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_[a-z_0-9]+)\s*\(", text)))


def test_header_declarations_match_binding():
    assert _declared_functions() == sorted(fa.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = fa.library()
    for name in _declared_functions():
        assert hasattr(lib, name), name
    # and from the dynamic symbol table directly, as a C caller would see it
    raw = ctypes.CDLL(fa.LIB_PATH)
    for name in _declared_functions():
        assert ctypes.cast(getattr(raw, name), ctypes.c_void_p).value


def test_status_strings():
    for st in range(-7, 1):
        s = fa.status_str(st)
        assert s and s != "unknown status"
    assert fa.status_str(-99) == "unknown status"


def test_workspace_bytes():
    assert fa.decode_workspace_bytes(16, 32, 128, 64) == 16 * 32 * 64 * 130 * 4 == 17039360
    assert fa.decode_workspace_bytes(1, 1, 64, 1) == 66 * 4
    for bad in [(0, 1, 64, 1), (1, 0, 64, 1), (1, 1, 0, 1), (1, 1, 64, 0), (-1, 1, 64, 1)]:
        assert fa.decode_workspace_bytes(*bad) == 0


def _fwd(**kw):
    a = dict(q=P, k=P, v=P, o=P, lse=P, B=1, H=1, Nq=16, Nk=16, d=64, scale=0.125, causal=0,
             dtype=fa.FA_BF16, stream=None)
    a.update(kw)
    return fa.library().fa_fwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["Nq"],
                               a["Nk"], a["d"], a["scale"], a["causal"], a["dtype"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), fa.FA_ERR_NULL), (dict(k=None), fa.FA_ERR_NULL),
    (dict(v=None), fa.FA_ERR_NULL), (dict(o=None), fa.FA_ERR_NULL),
    (dict(B=0), fa.FA_ERR_SHAPE), (dict(H=0), fa.FA_ERR_SHAPE), (dict(Nq=0), fa.FA_ERR_SHAPE),
    (dict(Nk=0), fa.FA_ERR_SHAPE), (dict(d=0), fa.FA_ERR_SHAPE), (dict(Nq=-5), fa.FA_ERR_SHAPE),
    (dict(B=1 << 20, H=1 << 12), fa.FA_ERR_SHAPE),
    (dict(d=96), fa.FA_ERR_UNSUPPORTED), (dict(d=256), fa.FA_ERR_UNSUPPORTED),
    (dict(dtype=7), fa.FA_ERR_UNSUPPORTED), (dict(Nk=1 << 25, d=128), fa.FA_ERR_UNSUPPORTED),
    (dict(scale=0.0), fa.FA_ERR_VALUE), (dict(scale=-1.0), fa.FA_ERR_VALUE),
    (dict(scale=float("inf")), fa.FA_ERR_VALUE), (dict(scale=float("nan")), fa.FA_ERR_VALUE),
    (dict(causal=3), fa.FA_ERR_VALUE), (dict(causal=-1), fa.FA_ERR_VALUE),
    (dict(q=P + 8), fa.FA_ERR_ALIGN), (dict(k=P + 2), fa.FA_ERR_ALIGN),
    (dict(v=P + 4), fa.FA_ERR_ALIGN), (dict(o=P + 12), fa.FA_ERR_ALIGN),
])
def test_fwd_rejects(kw, status):
    assert _fwd(**kw) == status


def _dec(**kw):
    a = dict(q=P, k=P, v=P, o=P, lse=P, B=2, H=2, Nk=100, d=128, scale=0.1, S=4, ws=P,
             wsb=fa.decode_workspace_bytes(2, 2, 128, 4), dtype=fa.FA_BF16, stream=None)
    a.update(kw)
    return fa.library().fa_decode_splitkv(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"],
                                          a["Nk"], a["d"], a["scale"], a["S"], a["ws"], a["wsb"],
                                          a["dtype"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), fa.FA_ERR_NULL), (dict(o=None), fa.FA_ERR_NULL),
    (dict(B=0), fa.FA_ERR_SHAPE), (dict(Nk=0), fa.FA_ERR_SHAPE), (dict(S=0), fa.FA_ERR_SHAPE),
    (dict(d=32), fa.FA_ERR_UNSUPPORTED), (dict(S=1025, wsb=1 << 30), fa.FA_ERR_UNSUPPORTED),
    (dict(dtype=3), fa.FA_ERR_UNSUPPORTED),
    (dict(scale=0.0), fa.FA_ERR_VALUE), (dict(scale=float("nan")), fa.FA_ERR_VALUE),
    (dict(ws=None), fa.FA_ERR_WORKSPACE), (dict(wsb=100), fa.FA_ERR_WORKSPACE),
    (dict(wsb=fa.decode_workspace_bytes(2, 2, 128, 4) - 1), fa.FA_ERR_WORKSPACE),
    (dict(ws=P + 4), fa.FA_ERR_ALIGN), (dict(q=P + 2), fa.FA_ERR_ALIGN),
])
def test_decode_rejects(kw, status):
    assert _dec(**kw) == status


def test_python_layer_maps_errors_without_gpu():
    import torch
    x = torch.zeros(1, 1, 4, 64)
    with pytest.raises(ValueError):
        fa.fwd(x, x, x)              # CPU tensors are refused before the library is called
    with pytest.raises(ValueError):
        fa._raise(fa.FA_ERR_SHAPE, "t")
    with pytest.raises(NotImplementedError):
        fa._raise(fa.FA_ERR_UNSUPPORTED, "t")
    with pytest.raises(fa.FaError):
        fa._raise(fa.FA_ERR_HIP, "t")


def test_single_hip_runtime_in_process():
    """libfa.so must bind to the HIP runtime torch already loaded, not load a second copy
    (a second runtime has its own device context and reports no device)."""
    fa.library()
    maps = open("/proc/self/maps").read()
    runtimes = {ln.split()[-1] for ln in maps.splitlines() if "libamdhip64" in ln}
    assert len(runtimes) == 1, runtimes


def test_bwd_workspace_bytes():
    assert fa.bwd_workspace_bytes(2, 16, 8192) == 2 * 16 * 8192 * 8
    assert fa.bwd_workspace_bytes(1, 32, 30000) == 32 * 30080 * 8   # rows padded to 128
    assert fa.bwd_workspace_bytes(1, 1, 1) == 128 * 8
    for bad in [(0, 1, 1), (1, 0, 1), (1, 1, 0), (-3, 1, 1)]:
        assert fa.bwd_workspace_bytes(*bad) == 0


def _bwd(**kw):
    a = dict(q=P, k=P, v=P, o=P, lse=P, do=P, dq=P, dk=P, dv=P, B=1, H=2, Nq=100, Nk=70, d=128,
             scale=0.1, causal=1, ws=P, wsb=fa.bwd_workspace_bytes(1, 2, 100), dtype=fa.FA_BF16,
             stream=None)
    a.update(kw)
    return fa.library().fa_bwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["do"], a["dq"], a["dk"],
                               a["dv"], a["B"], a["H"], a["Nq"], a["Nk"], a["d"], a["scale"],
                               a["causal"], a["ws"], a["wsb"], a["dtype"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), fa.FA_ERR_NULL), (dict(o=None), fa.FA_ERR_NULL), (dict(lse=None), fa.FA_ERR_NULL),
    (dict(do=None), fa.FA_ERR_NULL), (dict(dq=None), fa.FA_ERR_NULL), (dict(dk=None), fa.FA_ERR_NULL),
    (dict(dv=None), fa.FA_ERR_NULL),
    (dict(B=0), fa.FA_ERR_SHAPE), (dict(Nq=0), fa.FA_ERR_SHAPE), (dict(Nk=-1), fa.FA_ERR_SHAPE),
    (dict(dtype=7), fa.FA_ERR_UNSUPPORTED), (dict(d=96), fa.FA_ERR_UNSUPPORTED),
    (dict(Nk=1 << 24, d=128), fa.FA_ERR_UNSUPPORTED),
    (dict(scale=0.0), fa.FA_ERR_VALUE), (dict(scale=float("inf")), fa.FA_ERR_VALUE),
    (dict(causal=-1), fa.FA_ERR_VALUE),
    (dict(ws=None), fa.FA_ERR_WORKSPACE), (dict(wsb=fa.bwd_workspace_bytes(1, 2, 100) - 1),
                                           fa.FA_ERR_WORKSPACE),
    (dict(q=P + 8), fa.FA_ERR_ALIGN), (dict(do=P + 4), fa.FA_ERR_ALIGN), (dict(dk=P + 8), fa.FA_ERR_ALIGN),
    (dict(ws=P + 4), fa.FA_ERR_ALIGN), (dict(lse=P + 2), fa.FA_ERR_ALIGN),
])
def test_bwd_rejects(kw, status):
    assert _bwd(**kw) == status


def test_bwd_lse_needs_only_word_alignment():
    # a 4-byte aligned lse passes validation up to the workspace check (which then fails)
    assert _bwd(lse=P + 4, ws=None) == fa.FA_ERR_WORKSPACE


def _paged(**kw):
    a = dict(q=P, kc=P, vc=P, tab=P, lens=P, o=P, lse=P, B=2, H=2, d=128, ps=16, num_pages=10,
             max_pages=4, scale=0.1, S=4, ws=P, wsb=fa.decode_workspace_bytes(2, 2, 128, 4),
             dtype=fa.FA_BF16, stream=None)
    a.update(kw)
    return fa.library().fa_decode_paged(a["q"], a["kc"], a["vc"], a["tab"], a["lens"], a["o"], a["lse"],
                                        a["B"], a["H"], a["d"], a["ps"], a["num_pages"], a["max_pages"],
                                        a["scale"], a["S"], a["ws"], a["wsb"], a["dtype"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), fa.FA_ERR_NULL), (dict(kc=None), fa.FA_ERR_NULL), (dict(tab=None), fa.FA_ERR_NULL),
    (dict(lens=None), fa.FA_ERR_NULL), (dict(o=None), fa.FA_ERR_NULL),
    (dict(B=0), fa.FA_ERR_SHAPE), (dict(ps=0), fa.FA_ERR_SHAPE), (dict(num_pages=0), fa.FA_ERR_SHAPE),
    (dict(max_pages=0), fa.FA_ERR_SHAPE), (dict(S=0), fa.FA_ERR_SHAPE),
    (dict(max_pages=1 << 20, ps=1 << 12), fa.FA_ERR_SHAPE),
    (dict(ps=12), fa.FA_ERR_UNSUPPORTED), (dict(d=96), fa.FA_ERR_UNSUPPORTED),
    (dict(S=2000, wsb=1 << 30), fa.FA_ERR_UNSUPPORTED), (dict(dtype=5), fa.FA_ERR_UNSUPPORTED),
    (dict(scale=-1.0), fa.FA_ERR_VALUE),
    (dict(ws=None), fa.FA_ERR_WORKSPACE), (dict(wsb=64), fa.FA_ERR_WORKSPACE),
    (dict(kc=P + 8), fa.FA_ERR_ALIGN), (dict(tab=P + 2), fa.FA_ERR_ALIGN), (dict(lens=P + 1), fa.FA_ERR_ALIGN),
])
def test_paged_rejects(kw, status):
    assert _paged(**kw) == status


def test_paged_lse_may_be_null_and_tables_need_word_alignment():
    assert _paged(lse=None, ws=None) == fa.FA_ERR_WORKSPACE   # passes up to the workspace check
    assert _paged(tab=P + 4, lens=P + 12, ws=None) == fa.FA_ERR_WORKSPACE


def _varlen(**kw):
    a = dict(q=P, k=P, v=P, o=P, lse=P, cq=P, ck=P, B=2, H=4, tq=100, tk=120, maxq=60, d=128,
             scale=0.1, causal=1, dtype=fa.FA_BF16, stream=None)
    a.update(kw)
    return fa.library().fa_fwd_varlen(a["q"], a["k"], a["v"], a["o"], a["lse"], a["cq"], a["ck"],
                                      a["B"], a["H"], a["tq"], a["tk"], a["maxq"], a["d"], a["scale"],
                                      a["causal"], a["dtype"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), fa.FA_ERR_NULL), (dict(o=None), fa.FA_ERR_NULL), (dict(cq=None), fa.FA_ERR_NULL),
    (dict(ck=None), fa.FA_ERR_NULL),
    (dict(B=0), fa.FA_ERR_SHAPE), (dict(tq=0), fa.FA_ERR_SHAPE), (dict(tk=0), fa.FA_ERR_SHAPE),
    (dict(maxq=0), fa.FA_ERR_SHAPE),
    (dict(dtype=fa.FA_F32), fa.FA_ERR_UNSUPPORTED), (dict(d=32), fa.FA_ERR_UNSUPPORTED),
    (dict(H=1 << 16), fa.FA_ERR_UNSUPPORTED),
    (dict(scale=0.0), fa.FA_ERR_VALUE), (dict(causal=3), fa.FA_ERR_VALUE),
    (dict(q=P + 8), fa.FA_ERR_ALIGN), (dict(cq=P + 2), fa.FA_ERR_ALIGN),
])
def test_varlen_rejects(kw, status):
    assert _varlen(**kw) == status


def _bwd_varlen(**kw):
    a = dict(q=P, k=P, v=P, o=P, lse=P, do=P, dq=P, dk=P, dv=P, cq=P, ck=P, B=2, H=4, tq=100,
             tk=120, maxq=60, maxk=70, d=128, scale=0.1, causal=1, ws=P,
             wsb=fa.bwd_workspace_bytes(2, 4, 60), dtype=fa.FA_BF16, stream=None)
    a.update(kw)
    return fa.library().fa_bwd_varlen(
        a["q"], a["k"], a["v"], a["o"], a["lse"], a["do"], a["dq"], a["dk"], a["dv"], a["cq"],
        a["ck"], a["B"], a["H"], a["tq"], a["tk"], a["maxq"], a["maxk"], a["d"], a["scale"],
        a["causal"], a["ws"], a["wsb"], a["dtype"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), fa.FA_ERR_NULL), (dict(lse=None), fa.FA_ERR_NULL), (dict(do=None), fa.FA_ERR_NULL),
    (dict(dk=None), fa.FA_ERR_NULL), (dict(cq=None), fa.FA_ERR_NULL), (dict(ck=None), fa.FA_ERR_NULL),
    (dict(B=0), fa.FA_ERR_SHAPE), (dict(tq=0), fa.FA_ERR_SHAPE), (dict(tk=0), fa.FA_ERR_SHAPE),
    (dict(maxq=0), fa.FA_ERR_SHAPE), (dict(maxk=0), fa.FA_ERR_SHAPE),
    (dict(dtype=fa.FA_F32), fa.FA_ERR_UNSUPPORTED), (dict(d=32), fa.FA_ERR_UNSUPPORTED),
    (dict(H=1 << 16), fa.FA_ERR_UNSUPPORTED),
    (dict(scale=0.0), fa.FA_ERR_VALUE), (dict(causal=3), fa.FA_ERR_VALUE),
    (dict(ws=None), fa.FA_ERR_WORKSPACE), (dict(wsb=fa.bwd_workspace_bytes(2, 4, 60) - 1),
                                           fa.FA_ERR_WORKSPACE),
    (dict(maxq=129), fa.FA_ERR_WORKSPACE),  # 256 padded rows per pair against 128
    (dict(q=P + 8), fa.FA_ERR_ALIGN), (dict(dv=P + 8), fa.FA_ERR_ALIGN), (dict(lse=P + 2), fa.FA_ERR_ALIGN),
    (dict(ck=P + 2), fa.FA_ERR_ALIGN), (dict(ws=P + 4), fa.FA_ERR_ALIGN),
])
def test_bwd_varlen_rejects(kw, status):
    assert _bwd_varlen(**kw) == status


def _fp8(**kw):
    a = dict(q=P, k=P, v=P, o=P, lse=P, B=1, H=2, Nq=100, Nk=90, d=128, scale=0.1, qd=0.01, kd=0.02,
             vd=0.03, causal=1, stream=None)
    a.update(kw)
    return fa.library().fa_fwd_fp8(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["Nq"],
                                   a["Nk"], a["d"], a["scale"], a["qd"], a["kd"], a["vd"], a["causal"],
                                   a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), fa.FA_ERR_NULL), (dict(o=None), fa.FA_ERR_NULL),
    (dict(B=0), fa.FA_ERR_SHAPE), (dict(Nk=0), fa.FA_ERR_SHAPE),
    (dict(d=64), fa.FA_ERR_UNSUPPORTED), (dict(Nk=1 << 24), fa.FA_ERR_UNSUPPORTED),
    (dict(scale=0.0), fa.FA_ERR_VALUE), (dict(qd=0.0), fa.FA_ERR_VALUE), (dict(kd=-1.0), fa.FA_ERR_VALUE),
    (dict(vd=float("inf")), fa.FA_ERR_VALUE), (dict(causal=5), fa.FA_ERR_VALUE),
    (dict(q=P + 4), fa.FA_ERR_ALIGN), (dict(v=P + 8), fa.FA_ERR_ALIGN),
])
def test_fp8_rejects(kw, status):
    assert _fp8(**kw) == status


def _bias(**kw):
    a = dict(q=P, k=P, v=P, bias=P, sb=0, sh=0, sq=64, o=P, lse=P, B=1, H=1, Nq=16, Nk=16, d=64,
             scale=0.125, causal=0, dtype=fa.FA_BF16, stream=None)
    a.update(kw)
    return fa.library().fa_fwd_bias(a["q"], a["k"], a["v"], a["bias"], a["sb"], a["sh"], a["sq"],
                                    a["o"], a["lse"], a["B"], a["H"], a["Nq"], a["Nk"], a["d"],
                                    a["scale"], a["causal"], a["dtype"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(bias=None), fa.FA_ERR_NULL),
    (dict(q=None), fa.FA_ERR_NULL),
    (dict(Nk=0), fa.FA_ERR_SHAPE),
    (dict(sq=-8), fa.FA_ERR_SHAPE),
    (dict(sb=-1), fa.FA_ERR_SHAPE),
    (dict(sh=1 << 62), fa.FA_ERR_SHAPE),
    (dict(d=96), fa.FA_ERR_UNSUPPORTED),
    (dict(dtype=7), fa.FA_ERR_UNSUPPORTED),
    (dict(sq=1 << 25), fa.FA_ERR_UNSUPPORTED),   # 32 rows of it exceed 32-bit byte offsets
    (dict(causal=3), fa.FA_ERR_VALUE),
    (dict(scale=0.0), fa.FA_ERR_VALUE),
    (dict(bias=P + 8), fa.FA_ERR_ALIGN),          # bfloat16 bias rows are read 16 bytes at a time
    (dict(sq=20), fa.FA_ERR_ALIGN),
    (dict(sh=4), fa.FA_ERR_ALIGN),
    (dict(dtype=fa.FA_F32, bias=P + 2), fa.FA_ERR_ALIGN),
])
def test_bias_rejects(kw, status):
    assert _bias(**kw) == status


def test_bias_python_layer_checks_without_gpu():
    """The binding refuses CPU tensors before it calls the library."""
    import torch
    x = torch.zeros((1, 1, 8, 64), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        fa.fwd_bias(x, x, x, torch.zeros((8, 8), dtype=torch.bfloat16))


@pytest.mark.parametrize("args,status", [
    ((None, 1 << 20, 4, 10), fa.FA_ERR_NULL),
    ((P, 1 << 20, 0, 10), fa.FA_ERR_SHAPE),
    ((P, 1 << 20, 4, 0), fa.FA_ERR_SHAPE),
    ((P, 4 * 1024 - 1, 4, 10), fa.FA_ERR_WORKSPACE),
    ((P + 2, 1 << 20, 4, 10), fa.FA_ERR_ALIGN),
])
def test_probe_mfma_rejects(args, status):
    assert fa.library().fa_probe_mfma(*args, None) == status


def _noalloc(**kw):
    a = dict(q=P, k=P, v=P, o=P, lse=P, B=2, H=3, Nk=100, d=128, scale=0.1, S=8,
             dtype=fa.FA_BF16, stream=None)
    a.update(kw)
    return fa.library().fa_decode_splitkv_noalloc(a["q"], a["k"], a["v"], a["o"], a["lse"],
                                                  a["B"], a["H"], a["Nk"], a["d"], a["scale"],
                                                  a["S"], a["dtype"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), fa.FA_ERR_NULL), (dict(o=None), fa.FA_ERR_NULL),
    (dict(B=0), fa.FA_ERR_SHAPE), (dict(Nk=0), fa.FA_ERR_SHAPE), (dict(S=0), fa.FA_ERR_SHAPE),
    # partial states beyond the fixed scratch: (d + 2) * 4 bytes per (b, h, split)
    (dict(B=64, H=64, S=16, d=128), fa.FA_ERR_WORKSPACE),
    (dict(B=1, H=1, S=1, d=(32 << 20) // 4), fa.FA_ERR_WORKSPACE),
])
def test_decode_noalloc_rejects_before_any_hip_call(kw, status):
    assert _noalloc(**kw) == status


def test_decode_noalloc_limit_matches_header():
    text = open(HEADER).read()
    assert "#define FA_NOALLOC_SCRATCH_BYTES (32u << 20)" in text
    assert fa.NOALLOC_SCRATCH_BYTES == 32 << 20
    # the largest decode that fits at d = 128 (the header's example)
    assert fa.decode_workspace_bytes(1, 1, 128, 64527) <= fa.NOALLOC_SCRATCH_BYTES
    assert fa.decode_workspace_bytes(1, 1, 128, 64528) > fa.NOALLOC_SCRATCH_BYTES
