"""Python binding of libfa.so: exact tiled attention on MI355X (gfx950).

Argument marshalling only. Every step of the computation runs in the HIP kernels
of libfa.so; torch tensors are used for device memory and the current stream.
There is no CPU or PyTorch fallback: if the library is missing, or a tensor is
not on the GPU, the call raises.

    o, lse = fwd(q, k, v, scale=None, causal=False)        # prefill
    o, lse = fwd_bias(q, k, v, bias, scale=None, causal=False)   # plus an additive bias
    o, lse = fwd_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q)  # packed batch
    o, lse = fwd_fp8(q8, k8, v8, q_descale, k_descale, v_descale)   # E4M3 inputs
    o, lse = decode(q, k, v, num_splits=64, scale=None)     # one query per (b, h)
    o, lse = decode_noalloc(q, k, v, num_splits=64)         # the same, no device allocation
    o, lse = decode_paged(q, k_cache, v_cache, block_table, seq_lens)  # paged cache
    dq, dk, dv = bwd(q, k, v, o, lse, do, scale=None, causal=False)   # gradients
    dq, dk, dv[, dbias] = bwd_bias(q, k, v, bias, o, lse, do)         # ... of fwd_bias

Shapes are [B, H, N, d] (d innermost, contiguous); o is float32 [B, H, Nq, d],
lse float32 [B, H, Nq]. The C header include/fa.h states the full contract.
"""
from __future__ import annotations

import ctypes
import math
import os

__all__ = ["fwd", "fwd_bias", "pad_bias", "fwd_fp8", "fwd_varlen", "decode", "decode_noalloc", "decode_paged", "decode_workspace_bytes", "bwd", "bwd_bias", "bwd_workspace_bytes", "status_str", "NOALLOC_SCRATCH_BYTES",
           "library", "FaError", "FA_OK", "FA_ERR_NULL", "FA_ERR_SHAPE", "FA_ERR_UNSUPPORTED", "FA_ERR_WORKSPACE",
           "FA_ERR_HIP", "FA_ERR_VALUE", "FA_ERR_ALIGN", "FA_BF16", "FA_F32", "EXPORTS"]

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libfa.so")

FA_OK, FA_ERR_NULL, FA_ERR_SHAPE, FA_ERR_UNSUPPORTED = 0, -1, -2, -3
FA_ERR_WORKSPACE, FA_ERR_HIP, FA_ERR_VALUE, FA_ERR_ALIGN = -4, -5, -6, -7
FA_BF16, FA_F32 = 0, 1
# FA_NOALLOC_SCRATCH_BYTES of include/fa.h: the fixed per-GPU scratch of fa_decode_splitkv_noalloc
NOALLOC_SCRATCH_BYTES = 32 << 20

# every symbol include/fa.h declares
EXPORTS = ("fa_fwd", "fa_fwd_bias", "fa_fwd_fp8", "fa_fwd_varlen", "fa_decode_workspace_bytes", "fa_decode_splitkv",
           "fa_decode_splitkv_noalloc", "fa_decode_paged",
           "fa_bwd_workspace_bytes", "fa_bwd", "fa_bwd_varlen", "fa_bwd_bias", "fa_probe_mfma", "fa_status_str", "fa_last_hip_error",
           "fa_last_hip_error_str")

_vp, _i, _f, _sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
_SIGS = {
    "fa_fwd": (_i, [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _f, _i, _i, _vp]),
    "fa_fwd_bias": (_i, [_vp, _vp, _vp, _vp, ctypes.c_longlong, ctypes.c_longlong, ctypes.c_longlong,
                         _vp, _vp, _i, _i, _i, _i, _i, _f, _i, _i, _vp]),
    "fa_fwd_fp8": (_i, [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _f, _f, _f, _f, _i, _vp]),
    "fa_fwd_varlen": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _f, _i, _i,
                           _vp]),
    "fa_decode_workspace_bytes": (_sz, [_i, _i, _i, _i]),
    "fa_decode_splitkv": (_i, [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _f, _i, _vp, _sz, _i, _vp]),
    "fa_decode_splitkv_noalloc": (_i, [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _f, _i, _i, _vp]),
    "fa_decode_paged": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _f, _i, _vp,
                             _sz, _i, _vp]),
    "fa_bwd_workspace_bytes": (_sz, [_i, _i, _i]),
    "fa_bwd": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _f, _i, _vp,
                    _sz, _i, _vp]),
    "fa_bwd_varlen": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i,
                           _i, _i, _i, _f, _i, _vp, _sz, _i, _vp]),
    "fa_bwd_bias": (_i, [_vp, _vp, _vp, _vp, ctypes.c_longlong, ctypes.c_longlong, ctypes.c_longlong,
                         _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _f, _i, _vp, _sz,
                         _i, _vp]),
    "fa_probe_mfma": (_i, [_vp, _sz, _i, _i, _vp]),
    "fa_status_str": (ctypes.c_char_p, [_i]),
    "fa_last_hip_error": (_i, []),
    "fa_last_hip_error_str": (ctypes.c_char_p, []),
}

_lib = None


class FaError(RuntimeError):
    """A status other than FA_OK from libfa.so."""

    def __init__(self, status: int, what: str):
        lib = library()
        self.hip_error = int(lib.fa_last_hip_error())
        hip = lib.fa_last_hip_error_str().decode()
        super().__init__(f"{what}: {status_str(status)} (status {status}; HIP error "
                         f"{self.hip_error}: {hip})")
        self.status = status


def library():
    """The loaded libfa.so (ctypes.CDLL). Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it first (python -m exact_tiled_attention_08_amd.build "
                "or __graft_entry__.build()); there is no fallback path")
        # Load torch's HIP runtime first: libfa.so then binds to that same runtime (one
        # libamdhip64 per process) instead of pulling in a second copy that would not share
        # torch's device context, memory or streams.
        import torch  # noqa: F401
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def status_str(status: int) -> str:
    return library().fa_status_str(int(status)).decode()


def probe_mfma(blocks: int = 2048, iters: int = 2000, reps: int = 3) -> float:
    """Practical dense bf16 MFMA rate of the current GPU in TFLOP/s: times fa_probe_mfma
    (back-to-back 32x32x16 MFMAs on register operands, no memory traffic) with events on
    the current stream and returns the best of `reps` launches. Measurement aid only."""
    import torch
    sink = torch.empty((blocks * 256,), dtype=torch.float32, device="cuda")
    st = _stream_ptr(sink.device)
    lib = library()
    _raise(lib.fa_probe_mfma(sink.data_ptr(), sink.numel() * 4, blocks, 1, st), "fa_probe_mfma")
    best = 0.0
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        _raise(lib.fa_probe_mfma(sink.data_ptr(), sink.numel() * 4, blocks, iters, st), "fa_probe_mfma")
        e1.record()
        torch.cuda.synchronize()
        flops = blocks * 4 * iters * 4 * 32768.0
        best = max(best, flops / (e0.elapsed_time(e1) * 1e-3) / 1e12)
    return best


def decode_workspace_bytes(B: int, H: int, d: int, num_splits: int) -> int:
    return int(library().fa_decode_workspace_bytes(B, H, d, num_splits))


def bwd_workspace_bytes(B: int, H: int, Nq: int) -> int:
    return int(library().fa_bwd_workspace_bytes(B, H, Nq))


def _raise(status: int, what: str):
    if status == FA_OK:
        return
    msg = f"{what}: {status_str(status)} (status {status})"
    if status == FA_ERR_UNSUPPORTED:
        raise NotImplementedError(msg)
    if status in (FA_ERR_NULL, FA_ERR_SHAPE, FA_ERR_VALUE, FA_ERR_ALIGN, FA_ERR_WORKSPACE):
        raise ValueError(msg)
    raise FaError(status, what)


def _dtype_code(t):
    import torch
    if t.dtype == torch.bfloat16:
        return FA_BF16
    if t.dtype == torch.float32:
        return FA_F32
    raise NotImplementedError(f"unsupported dtype {t.dtype}: q, k, v must be bfloat16 or float32")


def _check_inputs(q, k, v):
    import torch
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not isinstance(t, torch.Tensor) or not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor")
        if t.dim() != 4:
            raise ValueError(f"{name} must be [B, H, N, d]")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if not (q.dtype == k.dtype == v.dtype):
        raise ValueError("q, k and v must share one dtype")
    if not (q.device == k.device == v.device):
        raise ValueError("q, k and v must be on one device")
    B, H, _, d = q.shape
    if k.shape[0] != B or k.shape[1] != H or k.shape[3] != d or v.shape != k.shape:
        raise ValueError("k and v must be [B, H, Nk, d] with q's B, H and d")


def _out_arg(t, shape, device, name: str, dtype=None):
    """A caller's output tensor checked against what the kernels write (a new one if t is
    None): a contiguous tensor of exactly `shape` and `dtype` (float32 by default) on
    `device`. The C ABI takes bare device pointers and cannot size them, so a host tensor, a
    short buffer or one on another GPU must be refused here, before any launch."""
    import torch
    dtype = torch.float32 if dtype is None else dtype
    shape = tuple(int(x) for x in shape)
    if t is None:
        return torch.empty(shape, dtype=dtype, device=device)
    if not isinstance(t, torch.Tensor) or not t.is_cuda or t.device != device:
        raise ValueError(f"{name} must be a GPU tensor on {device}")
    if tuple(t.shape) != shape or t.dtype != dtype or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous {dtype} tensor of shape {list(shape)}, "
                         f"got {t.dtype} {list(t.shape)}"
                         f"{'' if t.is_contiguous() else ' (not contiguous)'}")
    return t


def _workspace_arg(t, need: int, device):
    """A caller's workspace checked for device and size in bytes (a new one if t is None)."""
    import torch
    if t is None:
        return torch.empty((max(int(need), 16),), dtype=torch.uint8, device=device)
    if not isinstance(t, torch.Tensor) or not t.is_cuda or t.device != device:
        raise ValueError(f"workspace must be a GPU tensor on {device}")
    if not t.is_contiguous():
        raise ValueError("workspace must be contiguous")
    have = t.numel() * t.element_size()
    if have < need:
        raise ValueError(f"workspace holds {have} bytes, {need} needed")
    return t


def _causal_arg(causal) -> int:
    """False/0: no mask; True/1: causal, queries at the end of the key sequence (bottom-right);
    2: causal, queries at its start (top-left)."""
    c = int(causal)
    if c not in (0, 1, 2):
        raise ValueError("causal must be False/0, True/1 (bottom-right) or 2 (top-left)")
    return c


def _stream_ptr(device):
    import torch
    return torch.cuda.current_stream(device).cuda_stream


def fwd(q, k, v, scale: float | None = None, causal: bool = False, out=None, lse=None,
        return_lse: bool = True):
    """Attention forward on the GPU. Returns (o, lse) (lse None if return_lse is False)."""
    import torch
    _check_inputs(q, k, v)
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out = _out_arg(out, (B, H, Nq, d), q.device, "out")
    if return_lse or lse is not None:
        lse = _out_arg(lse, (B, H, Nq), q.device, "lse")
    st = library().fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                          lse.data_ptr() if lse is not None else None,
                          B, H, Nq, Nk, d, float(scale), _causal_arg(causal), _dtype_code(q),
                          _stream_ptr(q.device))
    _raise(st, "fa_fwd")
    return out, lse


def pad_bias(bias):
    """A view of `bias` (any shape, keys last) whose key dimension sits in rows padded to a
    multiple of 8 elements, as fwd_bias needs for bfloat16; a copy into a new buffer."""
    import torch
    nk = bias.shape[-1]
    buf = torch.zeros((*bias.shape[:-1], -(-nk // 8) * 8), dtype=bias.dtype, device=bias.device)
    buf[..., :nk].copy_(bias)
    return buf[..., :nk]


def _bias_strides(bias, q, B: int, H: int, Nq: int, Nk: int):
    """Element strides (b, h, q) of a bias broadcast to [B, H, Nq, Nk], after checking what
    the kernels read: keys contiguous, and for bfloat16 each row readable up to its first Nk
    elements rounded up to a multiple of 8."""
    import torch
    if not isinstance(bias, torch.Tensor) or not bias.is_cuda or bias.device != q.device:
        raise ValueError("bias must be a GPU tensor on q's device")
    if bias.dtype != q.dtype:
        raise ValueError(f"bias must have q's dtype {q.dtype}, got {bias.dtype}")
    if bias.dim() > 4:
        raise ValueError("bias must broadcast to [B, H, Nq, Nk]")
    bt = bias.reshape((1,) * (4 - bias.dim()) + tuple(bias.shape)) if bias.dim() < 4 else bias
    if bt.shape[3] != Nk or (Nk > 1 and bt.stride(3) != 1):
        raise ValueError("the bias key dimension must have size Nk and stride 1")
    try:
        be = bt.expand(B, H, Nq, Nk)
    except RuntimeError as e:
        raise ValueError(f"bias of shape {tuple(bias.shape)} does not broadcast to "
                         f"[{B}, {H}, {Nq}, {Nk}]") from e
    sb, sh, sq = (int(x) for x in be.stride()[:3])
    if q.dtype == torch.bfloat16:
        last = bt.storage_offset() + (B - 1) * sb + (H - 1) * sh + (Nq - 1) * sq + -(-Nk // 8) * 8
        if (sb | sh | sq) % 8 or be.data_ptr() % 16 or last * 2 > bt.untyped_storage().nbytes():
            raise ValueError("a bfloat16 bias needs 16-byte aligned rows whose key dimension is "
                             "padded to a multiple of 8 elements: pass pad_bias(bias)")
    return be, sb, sh, sq


def fwd_bias(q, k, v, bias, scale: float | None = None, causal: bool = False, out=None, lse=None,
             return_lse: bool = True):
    """Attention forward with an additive bias on the scaled scores (q's dtype, broadcastable
    to [B, H, Nq, Nk], keys contiguous; -inf hides a key). Returns (o, lse)."""
    import torch
    _check_inputs(q, k, v)
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    be, sb, sh, sq = _bias_strides(bias, q, B, H, Nq, Nk)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out = _out_arg(out, (B, H, Nq, d), q.device, "out")
    if return_lse or lse is not None:
        lse = _out_arg(lse, (B, H, Nq), q.device, "lse")
    st = library().fa_fwd_bias(q.data_ptr(), k.data_ptr(), v.data_ptr(), be.data_ptr(), sb, sh, sq,
                               out.data_ptr(), lse.data_ptr() if lse is not None else None,
                               B, H, Nq, Nk, d, float(scale), _causal_arg(causal), _dtype_code(q),
                               _stream_ptr(q.device))
    _raise(st, "fa_fwd_bias")
    return out, lse


def fwd_fp8(q, k, v, q_descale: float, k_descale: float, v_descale: float,
            scale: float | None = None, causal=False, out=None, lse=None):
    """Attention forward on E4M3 inputs (torch.float8_e4m3fn [B, H, N, 128] GPU tensors); the
    real inputs are q * q_descale etc. Returns (o float32 [B, H, Nq, d], lse [B, H, Nq])."""
    import torch
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not isinstance(t, torch.Tensor) or not t.is_cuda or not t.is_contiguous() or t.dim() != 4:
            raise ValueError(f"{name} must be a contiguous [B, H, N, d] GPU tensor")
        if t.dtype != torch.float8_e4m3fn:
            raise ValueError(f"{name} must be torch.float8_e4m3fn")
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    if k.shape[0] != B or k.shape[1] != H or k.shape[3] != d or v.shape != k.shape:
        raise ValueError("k and v must be [B, H, Nk, d] with q's B, H and d")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if not (q.device == k.device == v.device):
        raise ValueError("q, k and v must be on one device")
    out = _out_arg(out, (B, H, Nq, d), q.device, "out")
    lse = _out_arg(lse, (B, H, Nq), q.device, "lse")
    st = library().fa_fwd_fp8(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                              B, H, Nq, Nk, d, float(scale), float(q_descale), float(k_descale),
                              float(v_descale), _causal_arg(causal), _stream_ptr(q.device))
    _raise(st, "fa_fwd_fp8")
    return out, lse


def fwd_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q: int, scale: float | None = None,
               causal: bool = False, out=None, lse=None):
    """Attention forward over a packed batch of variable-length sequences: q [total_q, H, d],
    k, v [total_k, H, d] (bfloat16), cu_seqlens_* int32 [B+1] on the GPU. Returns
    (o [total_q, H, d] float32, lse [H, total_q] float32)."""
    import torch
    for name, t in (("q", q), ("k", k), ("v", v), ("cu_seqlens_q", cu_seqlens_q),
                    ("cu_seqlens_k", cu_seqlens_k)):
        if not isinstance(t, torch.Tensor) or not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous GPU tensor")
    if q.dim() != 3 or k.dim() != 3 or v.shape != k.shape or k.shape[1:] != q.shape[1:]:
        raise ValueError("q must be [total_q, H, d] and k, v [total_k, H, d]")
    if not (q.dtype == k.dtype == v.dtype):
        raise ValueError("q, k and v must share one dtype")
    if cu_seqlens_q.dtype != torch.int32 or cu_seqlens_k.dtype != torch.int32 \
            or cu_seqlens_q.dim() != 1 or cu_seqlens_k.shape != cu_seqlens_q.shape:
        raise ValueError("cu_seqlens_q and cu_seqlens_k must be int32 [B + 1]")
    total_q, H, d = q.shape
    total_k = k.shape[0]
    B = cu_seqlens_q.numel() - 1
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if len({t.device for t in (q, k, v, cu_seqlens_q, cu_seqlens_k)}) != 1:
        raise ValueError("q, k, v and the sequence offsets must be on one device")
    out = _out_arg(out, (total_q, H, d), q.device, "out")
    lse = _out_arg(lse, (H, total_q), q.device, "lse")
    st = library().fa_fwd_varlen(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
        cu_seqlens_q.data_ptr(), cu_seqlens_k.data_ptr(), B, H, total_q, total_k,
        int(max_seqlen_q), d, float(scale), _causal_arg(causal), _dtype_code(q),
        _stream_ptr(q.device))
    _raise(st, "fa_fwd_varlen")
    return out, lse


def decode(q, k, v, num_splits: int = 64, scale: float | None = None, out=None, lse=None,
           workspace=None):
    """Split-KV decode: q [B, H, 1, d] against k, v [B, H, Nk, d]. Returns (o, lse)."""
    import torch
    _check_inputs(q, k, v)
    B, H, Nq, d = q.shape
    if Nq != 1:
        raise ValueError("decode takes exactly one query per (b, h): q must be [B, H, 1, d]")
    Nk = k.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if int(num_splits) < 1:
        raise ValueError("num_splits must be at least 1")
    workspace = _workspace_arg(workspace, decode_workspace_bytes(B, H, d, num_splits), q.device)
    out = _out_arg(out, (B, H, 1, d), q.device, "out")
    lse = _out_arg(lse, (B, H, 1), q.device, "lse")
    st = library().fa_decode_splitkv(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
        B, H, Nk, d, float(scale), int(num_splits), workspace.data_ptr(),
        workspace.numel() * workspace.element_size(), _dtype_code(q), _stream_ptr(q.device))
    _raise(st, "fa_decode_splitkv")
    return out, lse


def decode_noalloc(q, k, v, num_splits: int = 64, scale: float | None = None, out=None,
                   lse=None):
    """decode() through fa_decode_splitkv_noalloc: the partial states live in the library's
    fixed per-GPU scratch (NOALLOC_SCRATCH_BYTES), so the C call allocates nothing. Pass
    out and lse to allocate nothing here either (torch allocates them if they are None).
    Calls that overlap in time on one GPU share that scratch and must not be issued."""
    _check_inputs(q, k, v)
    B, H, Nq, d = q.shape
    if Nq != 1:
        raise ValueError("decode takes exactly one query per (b, h): q must be [B, H, 1, d]")
    if int(num_splits) < 1:
        raise ValueError("num_splits must be at least 1")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out = _out_arg(out, (B, H, 1, d), q.device, "out")
    lse = _out_arg(lse, (B, H, 1), q.device, "lse")
    st = library().fa_decode_splitkv_noalloc(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(), B, H,
        k.shape[2], d, float(scale), int(num_splits), _dtype_code(q), _stream_ptr(q.device))
    _raise(st, "fa_decode_splitkv_noalloc")
    return out, lse


def decode_paged(q, k_cache, v_cache, block_table, seq_lens, num_splits: int = 64,
                 scale: float | None = None, out=None, lse=None, workspace=None):
    """Split-KV decode over a paged cache: q [B, H, 1, d]; k_cache, v_cache
    [num_pages, page_size, H, d]; block_table int32 [B, max_pages]; seq_lens int32 [B] (all
    on the GPU). Returns (o, lse)."""
    import torch
    for name, t in (("q", q), ("k_cache", k_cache), ("v_cache", v_cache),
                    ("block_table", block_table), ("seq_lens", seq_lens)):
        if not isinstance(t, torch.Tensor) or not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous GPU tensor")
    if q.dim() != 4 or q.shape[2] != 1:
        raise ValueError("q must be [B, H, 1, d]")
    B, H, _, d = q.shape
    if k_cache.dim() != 4 or k_cache.shape[2] != H or k_cache.shape[3] != d \
            or v_cache.shape != k_cache.shape:
        raise ValueError("k_cache and v_cache must be [num_pages, page_size, H, d] with q's H and d")
    if not (q.dtype == k_cache.dtype == v_cache.dtype):
        raise ValueError("q, k_cache and v_cache must share one dtype")
    if block_table.dtype != torch.int32 or block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError("block_table must be int32 [B, max_pages]")
    if seq_lens.dtype != torch.int32 or seq_lens.shape != (B,):
        raise ValueError("seq_lens must be int32 [B]")
    if len({t.device for t in (q, k_cache, v_cache, block_table, seq_lens)}) != 1:
        raise ValueError("q, the caches, block_table and seq_lens must be on one device")
    num_pages, page_size = k_cache.shape[0], k_cache.shape[1]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if int(num_splits) < 1:
        raise ValueError("num_splits must be at least 1")
    workspace = _workspace_arg(workspace, decode_workspace_bytes(B, H, d, num_splits), q.device)
    out = _out_arg(out, (B, H, 1, d), q.device, "out")
    lse = _out_arg(lse, (B, H, 1), q.device, "lse")
    st = library().fa_decode_paged(
        q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), block_table.data_ptr(),
        seq_lens.data_ptr(), out.data_ptr(), lse.data_ptr(), B, H, d, page_size, num_pages,
        block_table.shape[1], float(scale), int(num_splits), workspace.data_ptr(),
        workspace.numel() * workspace.element_size(), _dtype_code(q), _stream_ptr(q.device))
    _raise(st, "fa_decode_paged")
    return out, lse


def bwd(q, k, v, o, lse, do, scale: float | None = None, causal: bool = False, dq=None, dk=None,
        dv=None, workspace=None):
    """Attention backward on the GPU: gradients (dq, dk, dv), float32, of a loss with respect
    to q, k, v given do = dL/dO and the (o, lse) that fwd returned for the same inputs."""
    import torch
    _check_inputs(q, k, v)
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    if not isinstance(do, torch.Tensor) or do.shape != q.shape or do.dtype != q.dtype \
            or not do.is_contiguous() or do.device != q.device:
        raise ValueError("do must be a contiguous tensor of q's shape, dtype and device")
    if not isinstance(o, torch.Tensor) or o.shape != (B, H, Nq, d) or o.dtype != torch.float32 \
            or not o.is_contiguous() or o.device != q.device:
        raise ValueError("o must be the contiguous float32 [B, H, Nq, d] output of fwd")
    if not isinstance(lse, torch.Tensor) or lse.shape != (B, H, Nq) or lse.dtype != torch.float32 \
            or not lse.is_contiguous() or lse.device != q.device:
        raise ValueError("lse must be the contiguous float32 [B, H, Nq] output of fwd")
    if scale is None:
        scale = 1.0 / math.sqrt(d)

    dq = _out_arg(dq, (B, H, Nq, d), q.device, "dq")
    dk = _out_arg(dk, (B, H, Nk, d), q.device, "dk")
    dv = _out_arg(dv, (B, H, Nk, d), q.device, "dv")
    workspace = _workspace_arg(workspace, bwd_workspace_bytes(B, H, Nq), q.device)
    st = library().fa_bwd(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), do.data_ptr(),
        dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, H, Nq, Nk, d, float(scale),
        _causal_arg(causal), workspace.data_ptr(), workspace.numel() * workspace.element_size(),
        _dtype_code(q), _stream_ptr(q.device))
    _raise(st, "fa_bwd")
    return dq, dk, dv


def bwd_varlen(q, k, v, o, lse, do, cu_seqlens_q, cu_seqlens_k, max_seqlen_q: int,
               max_seqlen_k: int, scale: float | None = None, causal: bool = False, dq=None,
               dk=None, dv=None, workspace=None):
    """Backward of fwd_varlen: (dq [total_q, H, d], dk, dv [total_k, H, d]) float32, given the
    (o, lse) that fwd_varlen returned for the same packed inputs and offsets."""
    import torch
    for name, t in (("q", q), ("k", k), ("v", v), ("do", do), ("cu_seqlens_q", cu_seqlens_q),
                    ("cu_seqlens_k", cu_seqlens_k)):
        if not isinstance(t, torch.Tensor) or not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous GPU tensor")
    if q.dim() != 3 or k.dim() != 3 or v.shape != k.shape or k.shape[1:] != q.shape[1:] \
            or do.shape != q.shape:
        raise ValueError("q, do must be [total_q, H, d] and k, v [total_k, H, d]")
    if not (q.dtype == k.dtype == v.dtype == do.dtype):
        raise ValueError("q, k, v and do must share one dtype")
    if cu_seqlens_q.dtype != torch.int32 or cu_seqlens_k.dtype != torch.int32 \
            or cu_seqlens_q.dim() != 1 or cu_seqlens_k.shape != cu_seqlens_q.shape:
        raise ValueError("cu_seqlens_q and cu_seqlens_k must be int32 [B + 1]")
    total_q, H, d = q.shape
    total_k = k.shape[0]
    B = cu_seqlens_q.numel() - 1
    if len({t.device for t in (q, k, v, do, cu_seqlens_q, cu_seqlens_k)}) != 1:
        raise ValueError("q, k, v, do and the sequence offsets must be on one device")
    if not isinstance(o, torch.Tensor) or o.shape != q.shape or o.dtype != torch.float32 \
            or not o.is_contiguous() or o.device != q.device:
        raise ValueError("o must be the contiguous float32 [total_q, H, d] output of fwd_varlen")
    if not isinstance(lse, torch.Tensor) or lse.shape != (H, total_q) or lse.dtype != torch.float32 \
            or not lse.is_contiguous() or lse.device != q.device:
        raise ValueError("lse must be the contiguous float32 [H, total_q] output of fwd_varlen")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dq = _out_arg(dq, (total_q, H, d), q.device, "dq")
    dk = _out_arg(dk, (total_k, H, d), q.device, "dk")
    dv = _out_arg(dv, (total_k, H, d), q.device, "dv")
    workspace = _workspace_arg(workspace, bwd_workspace_bytes(B, H, max(1, int(max_seqlen_q))),
                               q.device)
    st = library().fa_bwd_varlen(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), do.data_ptr(),
        dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), cu_seqlens_q.data_ptr(),
        cu_seqlens_k.data_ptr(), B, H, total_q, total_k, int(max_seqlen_q), int(max_seqlen_k), d,
        float(scale), _causal_arg(causal), workspace.data_ptr(),
        workspace.numel() * workspace.element_size(), _dtype_code(q), _stream_ptr(q.device))
    _raise(st, "fa_bwd_varlen")
    return dq, dk, dv


def bwd_bias(q, k, v, bias, o, lse, do, scale: float | None = None, causal=False, dq=None,
             dk=None, dv=None, want_dbias: bool = False, dbias=None, workspace=None):
    """Backward of fwd_bias: (dq, dk, dv) float32, plus dbias (float32 [B, H, Nq, Nk], the
    gradient of a full bias: dS) when want_dbias or a dbias tensor is given. bias as for
    fwd_bias (bfloat16, rows padded with pad_bias); o and lse are fwd_bias's outputs. For a
    bias shared along some dimensions, its gradient is dbias summed over them."""
    import torch
    _check_inputs(q, k, v)
    if q.dtype != torch.bfloat16:
        raise NotImplementedError("bwd_bias takes bfloat16 q, k, v")
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    be, sb, sh, sq = _bias_strides(bias, q, B, H, Nq, Nk)
    if not isinstance(do, torch.Tensor) or do.shape != q.shape or do.dtype != q.dtype \
            or not do.is_contiguous() or do.device != q.device:
        raise ValueError("do must be a contiguous tensor of q's shape, dtype and device")
    if not isinstance(o, torch.Tensor) or o.shape != (B, H, Nq, d) or o.dtype != torch.float32 \
            or not o.is_contiguous() or o.device != q.device:
        raise ValueError("o must be the contiguous float32 [B, H, Nq, d] output of fwd_bias")
    if not isinstance(lse, torch.Tensor) or lse.shape != (B, H, Nq) or lse.dtype != torch.float32 \
            or not lse.is_contiguous() or lse.device != q.device:
        raise ValueError("lse must be the contiguous float32 [B, H, Nq] output of fwd_bias")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dq = _out_arg(dq, (B, H, Nq, d), q.device, "dq")
    dk = _out_arg(dk, (B, H, Nk, d), q.device, "dk")
    dv = _out_arg(dv, (B, H, Nk, d), q.device, "dv")
    if want_dbias or dbias is not None:
        dbias = _out_arg(dbias, (B, H, Nq, Nk), q.device, "dbias")
    workspace = _workspace_arg(workspace, bwd_workspace_bytes(B, H, Nq), q.device)
    st = library().fa_bwd_bias(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), be.data_ptr(), sb, sh, sq, o.data_ptr(),
        lse.data_ptr(), do.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
        dbias.data_ptr() if dbias is not None else None, B, H, Nq, Nk, d, float(scale),
        _causal_arg(causal), workspace.data_ptr(), workspace.numel() * workspace.element_size(),
        _dtype_code(q), _stream_ptr(q.device))
    _raise(st, "fa_bwd_bias")
    return (dq, dk, dv, dbias) if dbias is not None else (dq, dk, dv)
